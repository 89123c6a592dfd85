// generic.hip -- fp32-accumulating VALU kernels of both scans for every
// supported (dtype, head dim) pair.  They carry the fp32 token path (whose
// outputs must track the fp64 reference to ~1e-5) and the bf16 head dims that
// have no MFMA specialisation.  Straightforward LDS-tiled loops: a workgroup
// owns one (frame, token chunk) and each thread owns fixed entries of the
// D x D result.
#include "device_common.h"
#include "kernels.h"

namespace linscan {

namespace {

constexpr int GT = 32;  // tokens per LDS tile

// dS = sum v phi(k)^T, dz = sum phi(k) over one token chunk (RELU), or
// G = c2 sum k k^T, U = c sum v k^T (GDN; with per-token gates `gate`
// [B*H*F][N], each token's terms times its gate).  Output row of `partial`.
// Entries of the D x D result per thread; larger results are split over
// gridDim.y workgroups that share the token chunk.
template <int D>
struct SummarySplit {
  static constexpr int kEPT = (D * D + 255) / 256 < 16 ? (D * D + 255) / 256 : 16;
  static constexpr int kParts = (D * D + 256 * kEPT - 1) / (256 * kEPT);
};

template <typename T, int D, bool RELU>
__global__ __launch_bounds__(256) void gen_summary(const T* __restrict__ k, const T* __restrict__ v,
                                                   float* __restrict__ partial, float c, float c2,
                                                   const float* S0, const float* z0, float* init,
                                                   const float* gate, int F, int N, int nc, int chunk,
                                                   TokLayout L, Prologue P) {
  constexpr int EPT = SummarySplit<D>::kEPT;
  __shared__ float ks[GT][D + 1];
  __shared__ float vs[GT][D + 1];
  __shared__ float bs[GT];  // token gates (GDN)
  __shared__ double sc[GT], sc2[GT];  // per-token prologue factors (RMSNorm, L2)
  // RELU with the rotary embedding: the unrotated features, for the normaliser
  __shared__ float kd[RELU ? GT : 1][RELU ? D + 1 : 1];
  const int tid = threadIdx.x;
  const int e0 = blockIdx.y * 256 * EPT;  // first entry owned by this workgroup
  const long wg = blockIdx.x;
  const long bhf = wg / nc;
  const int n0 = (int)(wg % nc) * chunk;
  const int n1 = min(N, n0 + chunk);
  const T* kf = k + L.base(bhf);
  const T* vf = v + L.base(bhf);

  float a1[EPT], a2[EPT];
#pragma unroll
  for (int x = 0; x < EPT; ++x) a1[x] = a2[x] = 0.0f;
  float az = 0.0f;

  for (int t0 = n0; t0 < n1; t0 += GT) {
    for (int e = tid; e < GT * D; e += 256) {
      const int tok = e / D, d = e % D;
      const int n = t0 + tok;
      float kk = 0.0f, vv = 0.0f;
      if (n < n1) {
        kk = Elem<T>::load(kf, (size_t)n * L.sn + d);
        vv = Elem<T>::load(vf, (size_t)n * L.sn + d);
      }
      ks[tok][d] = RELU && !P.on_k() ? relu_f32(kk) : kk;
      vs[tok][d] = vv;
    }
    if (P.on_k()) {  // the prologue on the staged keys (fp64, one rounding), then the feature map
      const float* wk = P.wk ? P.wk + (size_t)((bhf / L.F) % L.H) * D : nullptr;
      __syncthreads();
      if (tid < GT) {  // the token's RMSNorm and L2 factors
        double s1 = 1.0, s2 = 1.0;
        if (wk) {
          double ss = 0.0;
          for (int d = 0; d < D; ++d) ss = fma((double)ks[tid][d], (double)ks[tid][d], ss);
          s1 = rsqrt_f64(fma(ss, 1.0 / D, (double)P.eps));
        }
        if (P.l2) {
          double ss = 0.0;
          for (int d = 0; d < D; ++d) {
            const double y = prologue_chan(ks[tid][d], wk ? wk[d] : 1.0f, s1, P.relu, 1.0);
            ss = fma(y, y, ss);
          }
          s2 = ss > 0.0 ? rsqrt_f64(ss) : 0.0;
        }
        sc[tid] = s1;
        sc2[tid] = s2;
      }
      __syncthreads();
      // one channel pair per thread: the rotary embedding mixes the two
      for (int e = tid; e < GT * D / 2; e += 256) {
        const int tok = e / (D / 2), d = 2 * (e % (D / 2));
        // RELU with the rotary embedding: the feature map comes before the rotation
        const int fm = P.relu || (RELU && P.rope());
        double y0 = prologue_chan(ks[tok][d], wk ? wk[d] : 1.0f, sc[tok], fm, sc2[tok]);
        double y1 = prologue_chan(ks[tok][d + 1], wk ? wk[d + 1] : 1.0f, sc[tok], fm, sc2[tok]);
        if (RELU && P.rope()) {
          kd[tok][d] = (float)y0;
          kd[tok][d + 1] = (float)y1;
        }
        if (P.rope()) {
          const float* cs = P.rope1(bhf % L.F, t0 + tok < n1 ? t0 + tok : n0, d / 2, D);
          const double c = cs[0], s = cs[1], x0 = y0;
          y0 = x0 * c - y1 * s;
          y1 = x0 * s + y1 * c;
        }
        const float x0 = Elem<T>::round(y0), x1 = Elem<T>::round(y1);
        ks[tok][d] = RELU && !P.rope() ? relu_f32(x0) : x0;
        ks[tok][d + 1] = RELU && !P.rope() ? relu_f32(x1) : x1;
      }
    }
    if (!RELU && tid < GT) {
      const int n = t0 + tid;
      bs[tid] = gate ? (n < n1 ? gate[(size_t)bhf * N + n] : 0.0f) : 1.0f;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = e0 + tid + 256 * x;
      if (e < D * D) {
        const int i = e / D, j = e % D;
        for (int tok = 0; tok < GT; ++tok) {
          const float kj = RELU ? ks[tok][j] : bs[tok] * ks[tok][j];
          a1[x] = fmaf(vs[tok][i], kj, a1[x]);
          if (!RELU) a2[x] = fmaf(ks[tok][i], kj, a2[x]);
        }
      }
    }
    if (RELU && blockIdx.y == 0 && tid < D)
      for (int tok = 0; tok < GT; ++tok) az += P.rope() ? kd[tok][tid] : ks[tok][tid];
    __syncthreads();
  }

  if (RELU) {
    float* dst = partial + (size_t)wg * (D * D + D);
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = e0 + tid + 256 * x;
      if (e < D * D) dst[e] = a1[x];
    }
    if (blockIdx.y == 0 && tid < D) dst[D * D + tid] = az;
    if (blockIdx.y == 0) relu_copy_init<D>(S0, z0, init, wg, F, nc);
  } else {
    float* Gd = partial + (size_t)wg * 2 * D * D;
    float* Ud = Gd + D * D;
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = e0 + tid + 256 * x;
      if (e < D * D) {
        Gd[e] = c2 * a2[x];
        Ud[e] = c * a1[x];
      }
    }
  }
}

// o = S_f phi(q) / (z_f . phi(q) + eps) (RELU) or o = S_f q, one token per
// group of D threads.  RELU forms (S_f, z_f) from the initial state and the
// summary partials (and writes the call's final state from the last frame);
// otherwise S_f (fp32) is read from `states`.
template <typename T, int D, bool RELU>
__global__ __launch_bounds__(256) void gen_output(const T* __restrict__ q, T* __restrict__ o,
                                                  const float* __restrict__ states,
                                                  const float* __restrict__ init, float* S_out,
                                                  float* z_out, float eps, int F, int N, int nc,
                                                  int bfr, int nco, int chunk, TokLayout L, Prologue P) {
  constexpr int SLOTS = 256 / D;
  __shared__ float Ss[D][D + 1];
  __shared__ float zs[D];
  __shared__ float qs[SLOTS][D];
  __shared__ float qd[RELU ? SLOTS : 1][RELU ? D : 1];  // RELU with the rotary embedding: unrotated features
  const int tid = threadIdx.x;
  const long wg = blockIdx.x;
  const long bhf = wg / nco;
  const int n0 = (int)(wg % nco) * chunk;
  const int n1 = min(N, n0 + chunk);
  if (RELU) {
    const long bh = bhf / F;
    const int f = (int)(bhf % F);
    relu_frame_state<D>(states, init, bh, f, F, nc, bfr, &Ss[0][0], D + 1, zs);
    __syncthreads();
    if (f == F - 1 && wg % nco == 0) {
      for (int e = tid; e < D * D; e += 256)
        if (S_out) S_out[(size_t)bh * D * D + e] = Ss[e / D][e % D];
      if (z_out && tid < D) z_out[(size_t)bh * D + tid] = zs[tid];
    }
  } else {
    const float* Sf = states + (size_t)bhf * D * D;
    for (int e = tid; e < D * D; e += 256) Ss[e / D][e % D] = Sf[e];
  }
  const int slot = tid / D, i = tid % D;
  const T* qf = q + L.base(bhf);
  T* of = o + L.base(bhf);
  for (int t0 = n0; t0 < n1; t0 += SLOTS) {
    __syncthreads();
    if (slot < SLOTS) {
      const int n = t0 + slot;
      float x = (n < n1) ? Elem<T>::load(qf, (size_t)n * L.sn + i) : 0.0f;
      qs[slot][i] = RELU && !P.on_q() ? relu_f32(x) : x;
    }
    __syncthreads();
    if (P.on_q()) {  // the prologue on the staged queries (every thread sums its token), then the feature map
      float y = 0.0f;
      if (slot < SLOTS) {
        double s1 = 1.0;
        float wv = 1.0f;
        if (P.wq) {
          double ss = 0.0;
          for (int j = 0; j < D; ++j) ss = fma((double)qs[slot][j], (double)qs[slot][j], ss);
          s1 = rsqrt_f64(fma(ss, 1.0 / D, (double)P.eps));
          wv = P.wq[(size_t)((bhf / L.F) % L.H) * D + i];
        }
        const int fm = P.relu || (RELU && P.rope());  // RELU: the feature map comes before the rotation
        double yd = prologue_chan(qs[slot][i], wv, s1, fm, 1.0);
        if (RELU && P.rope()) qd[slot][i] = (float)yd;
        if (P.rope()) {  // the pair partner's value, then the rotation of the pair
          const float wp = P.wq ? P.wq[(size_t)((bhf / L.F) % L.H) * D + (i ^ 1)] : 1.0f;
          const double yp = prologue_chan(qs[slot][i ^ 1], wp, s1, fm, 1.0);
          const float* cs = P.rope1(bhf % L.F, t0 + slot < n1 ? t0 + slot : n0, i / 2, D);
          const double c = cs[0], sn = cs[1];
          yd = (i & 1) ? yp * sn + yd * c : yd * c - yp * sn;
        }
        y = Elem<T>::round(yd);
        if (RELU && !P.rope()) y = relu_f32(y);
      }
      __syncthreads();
      if (slot < SLOTS) qs[slot][i] = y;
      __syncthreads();
    }
    if (slot < SLOTS && t0 + slot < n1) {
      float num = 0.0f, den = 0.0f;
      for (int j = 0; j < D; ++j) {
        const float qj = qs[slot][j];
        num = fmaf(Ss[i][j], qj, num);
        if (RELU) den = fmaf(zs[j], P.rope() ? qd[slot][j] : qj, den);
      }
      const float out = RELU ? num / (den + eps) : num;
      Elem<T>::store(of, (size_t)(t0 + slot) * L.sn + i, out);
    }
  }
}

template <typename T, int D>
hipError_t summary_launch(const GenArgs& a, hipStream_t st) {
  dim3 grid((unsigned)(a.bhf * a.nc), SummarySplit<D>::kParts), block(256);
  if (a.relu)
    hipLaunchKernelGGL((gen_summary<T, D, true>), grid, block, 0, st, (const T*)a.k, (const T*)a.v,
                       a.partial, a.c, a.c2, a.S0, a.z0, a.init, a.gate, a.F, a.N, a.nc, a.chunk, a.L, a.P);
  else
    hipLaunchKernelGGL((gen_summary<T, D, false>), grid, block, 0, st, (const T*)a.k, (const T*)a.v,
                       a.partial, a.c, a.c2, a.S0, a.z0, a.init, a.gate, a.F, a.N, a.nc, a.chunk, a.L, a.P);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t output_launch(const GenArgs& a, hipStream_t st) {
  dim3 grid((unsigned)(a.bhf * a.nco)), block(256);
  if (a.relu)
    hipLaunchKernelGGL((gen_output<T, D, true>), grid, block, 0, st, (const T*)a.q, (T*)a.o,
                       a.partial, a.init, a.S_out, a.z_out, a.eps, a.F, a.N, a.nc, a.bfr, a.nco, a.chunko, a.L,
                       a.P);
  else
    hipLaunchKernelGGL((gen_output<T, D, false>), grid, block, 0, st, (const T*)a.q, (T*)a.o,
                       (const float*)a.states, nullptr, nullptr, nullptr, 0.0f, a.F, a.N, 1, 1, a.nco, a.chunko,
                       a.L, a.P);
  return hipGetLastError();
}

#define LINSCAN_FOR_EACH_D(X) X(16) X(32) X(48) X(64) X(80) X(96) X(112) X(128)

template <typename T>
hipError_t summary_dispatch(const GenArgs& a, hipStream_t st) {
  switch (a.D) {
#define CASE(d) \
  case d: return summary_launch<T, d>(a, st);
    LINSCAN_FOR_EACH_D(CASE)
#undef CASE
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t output_dispatch(const GenArgs& a, hipStream_t st) {
  switch (a.D) {
#define CASE(d) \
  case d: return output_launch<T, d>(a, st);
    LINSCAN_FOR_EACH_D(CASE)
#undef CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_summary_generic(const GenArgs& a, hipStream_t st) {
  return a.dtype == DT_F32 ? summary_dispatch<float>(a, st) : summary_dispatch<uint16_t>(a, st);
}

hipError_t launch_output_generic(const GenArgs& a, hipStream_t st) {
  return a.dtype == DT_F32 ? output_dispatch<float>(a, st) : output_dispatch<uint16_t>(a, st);
}

}  // namespace linscan
