// scan.hip -- the generic GDN frame scan, the state carry, and the dispatch
// between MFMA and generic kernels.
//
// GDN scan: S_f = alpha_f S_{f-1} (I - beta_f G_f) + beta_f U_f.  Rows of S
// evolve independently given G_f (row r of S_f needs only row r of S_{f-1}),
// so each workgroup owns 16 rows of one head's state and walks all frames.
// The generic kernel here runs the D x D product S_rows G_f in fp32 on the
// VALU against G_f staged in LDS (the fp32-token path); the bf16 head-dim-128
// path uses the MFMA scan next to its gram kernel.
#include "device_common.h"
#include "kernels.h"

#include <map>
#include <cmath>
#include <mutex>
#include <utility>

namespace linscan {

hipError_t launch_gdn_gram_mfma(int D, const void* k, const void* v, const float* gates, bool tg, void* rec,
                                float c, float c2, long bhf, int N, int nc, int chunk, const TokLayout& L,
                                const Prologue& P, hipStream_t st);
hipError_t launch_gdn_scan_mfma(int D, const void* rec, const float* alpha, const float* S0,
                                void* states, float* S_out, long bh, int F, int nc, int rchunk, hipStream_t st);
hipError_t launch_gdn_output_mfma(int D, const void* q, void* o, const void* states, long bhf,
                                  int N, int nco, int chunk, const TokLayout& L, const Prologue& P, hipStream_t st);

namespace {

// One workgroup per (batch*head, 16-row block).  State rows live in LDS; G_f
// is summed over token chunks into LDS each frame; every thread owns EPT
// (row, col) entries.  Each frame's state goes to `states` in fp32.
// rchunk > 0: the reversed scan in chunks of rchunk frames (step l works on
// frame phys(l), with decay 0 at the first step of each chunk, which drops the
// previous chunk's state).
template <int D>
__global__ __launch_bounds__(256) void gdn_scan_kernel(const float* __restrict__ partial,
                                                       const float* __restrict__ alpha,
                                                       const float* __restrict__ beta,
                                                       const float* S0, void* __restrict__ states,
                                                       float* S_out, int F, int nc, int rchunk) {
  constexpr int RB = 16;                       // rows per workgroup
  constexpr int EPT = (RB * D + 255) / 256;    // entries per thread
  constexpr int R = D / RB;                    // row blocks per head
  __shared__ float Gs[D][D + 1];
  __shared__ float Ss[RB][D + 1];
  const int tid = threadIdx.x;
  const long bh = blockIdx.x / R;
  const int r0 = (int)(blockIdx.x % R) * RB;

  float s[EPT];
#pragma unroll
  for (int x = 0; x < EPT; ++x) {
    const int e = tid + 256 * x;
    s[x] = 0.0f;
    if (e < RB * D) {
      const int r = e / D, j = e % D;
      if (S0) s[x] = S0[(size_t)bh * D * D + (size_t)(r0 + r) * D + j];
      Ss[r][j] = s[x];
    }
  }

  for (int l = 0; l < F; ++l) {
    int f = l;
    if (rchunk > 0) {
      const int c0 = l / rchunk * rchunk;
      f = c0 + min(rchunk, F - c0) - 1 - (l - c0);
    }
    const size_t bhf = (size_t)bh * F + f;
    const float a = rchunk > 0 && l % rchunk == 0 ? 0.0f : alpha[bhf];
    const float b = beta ? beta[bhf] : 1.0f;  // per-token gates are inside G and U
    const float* P = partial + bhf * nc * 2 * D * D;
    for (int e = tid; e < D * D; e += 256) {
      float gsum = P[e];
      for (int c = 1; c < nc; ++c) gsum += P[(size_t)c * 2 * D * D + e];
      Gs[e / D][e % D] = gsum;
    }
    float u[EPT];
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = tid + 256 * x;
      u[x] = 0.0f;
      if (e < RB * D) {
        const size_t off = (size_t)D * D + (size_t)(r0 + e / D) * D + e % D;
        for (int c = 0; c < nc; ++c) u[x] += P[(size_t)c * 2 * D * D + off];
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = tid + 256 * x;
      if (e < RB * D) {
        const int r = e / D, j = e % D;
        float t = 0.0f;
        for (int l = 0; l < D; ++l) t = fmaf(Ss[r][l], Gs[l][j], t);
        s[x] = a * (s[x] - b * t) + b * u[x];
      }
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = tid + 256 * x;
      if (e < RB * D) {
        const int r = e / D, j = e % D;
        Ss[r][j] = s[x];
        reinterpret_cast<float*>(states)[bhf * D * D + (size_t)(r0 + r) * D + j] = s[x];
      }
    }
  }
  if (S_out) {
#pragma unroll
    for (int x = 0; x < EPT; ++x) {
      const int e = tid + 256 * x;
      if (e < RB * D) S_out[(size_t)bh * D * D + (size_t)(r0 + e / D) * D + e % D] = s[x];
    }
  }
}

template <int D>
hipError_t scan_launch(const float* partial, const float* alpha, const float* beta, const float* S0,
                       void* states, float* S_out, long bh, int F, int nc, int rchunk, hipStream_t st) {
  dim3 grid((unsigned)(bh * (D / 16))), block(256);
  hipLaunchKernelGGL(gdn_scan_kernel<D>, grid, block, 0, st, partial, alpha, beta, S0, states, S_out, F, nc, rchunk);
  return hipGetLastError();
}

// Copies (or zeroes) two ranges in one launch: the state and the normaliser.
__global__ __launch_bounds__(256) void carry_kernel(const float* __restrict__ src0, float* __restrict__ dst0,
                                                    size_t n0, const float* __restrict__ src1,
                                                    float* __restrict__ dst1, size_t n1, int reset) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n0 + n1; i += stride) {
    if (i < n0)
      dst0[i] = reset ? 0.0f : src0[i];
    else
      dst1[i - n0] = reset ? 0.0f : src1[i - n0];
  }
}

}  // namespace

int device_slots(const void* kernel) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 512;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find({kernel, dev});
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  int slots = 512;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && per_cu > 0 &&
      cus > 0)
    slots = per_cu * cus;
  cache[{kernel, dev}] = slots;
  return slots;
}

int fused_lag(long slots, long items_per_step, int min_lag, int F, double rounds) {
  long lag = items_per_step > 0 ? (long)std::ceil(rounds * (double)slots / (double)items_per_step) + 1 : 1;
  if (lag < min_lag) lag = min_lag;
  if (lag > F) lag = F;
  return lag < 1 ? 1 : (int)lag;
}

// bf16 MFMA head dims always run the single-launch kernels
hipError_t launch_relu_summary(const ScanArgs& a, hipStream_t st) {
  if (a.mfma) return hipErrorInvalidValue;
  return launch_summary_generic(a, st);
}

hipError_t launch_relu_output(const ScanArgs& a, hipStream_t st) {
  if (a.mfma) return hipErrorInvalidValue;
  return launch_output_generic(a, st);
}

hipError_t launch_gdn_gram(const ScanArgs& a, hipStream_t st) {
  if (a.mfma)
    return launch_gdn_gram_mfma(a.D, a.k, a.v, a.tg ? a.gate : a.beta, a.tg, a.partial, a.c, a.c2, a.bhf, a.N, a.nc,
                                a.chunk, a.L, a.P, st);
  return launch_summary_generic(a, st);
}

hipError_t launch_gdn_scan(const ScanArgs& a, hipStream_t st) {
  if (a.mfma)
    return launch_gdn_scan_mfma(a.D, a.partial, a.alpha, a.S0, a.states, a.S_out, a.bh, a.F, a.nc, a.rchunk, st);
  switch (a.D) {
#define CASE(d) \
  case d: return scan_launch<d>(a.partial, a.alpha, a.beta, a.S0, a.states, a.S_out, a.bh, a.F, a.nc, a.rchunk, st);
    CASE(16) CASE(32) CASE(48) CASE(64) CASE(80) CASE(96) CASE(112) CASE(128)
#undef CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gdn_output(const ScanArgs& a, hipStream_t st) {
  if (a.mfma) return launch_gdn_output_mfma(a.D, a.q, a.o, a.states, a.bhf, a.N, a.nco, a.chunko, a.L, a.P, st);
  return launch_output_generic(a, st);
}

hipError_t launch_carry(const float* src0, float* dst0, size_t n0, const float* src1, float* dst1,
                        size_t n1, int reset, hipStream_t st) {
  if (n0 + n1 == 0) return hipSuccess;
  size_t blocks = (n0 + n1 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(carry_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src0, dst0, n0, src1,
                     dst1, n1, reset);
  return hipGetLastError();
}

}  // namespace linscan
