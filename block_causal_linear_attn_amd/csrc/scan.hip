// scan.hip -- the sequential-over-frames parts of both scans, the state carry,
// and the dispatch between MFMA and generic kernels.
//
// ReLU prefix: the ReLU state is a plain running sum, so frame f's state is
// the initial state plus the contributions of every frame in blocks up to and
// including f's block (a block reads the state after all of its own frames;
// SANA-Video practical guide, section on core mechanisms).
//
// GDN scan: S_f = alpha_f S_{f-1} (I - beta_f G_f) + beta_f U_f.  Rows of S
// evolve independently given G_f (row r of S_f needs only row r of S_{f-1}),
// so each workgroup owns 16 rows of one head's state and walks all frames;
// the D x D product S_rows G_f runs in fp32 on the VALU against G_f staged in
// LDS.
#include "device_common.h"
#include "kernels.h"

namespace linscan {

hipError_t launch_relu_summary_mfma(int D, const void* k, const void* v, float* partial, long bhf,
                                    int N, int nc, int chunk, hipStream_t st);
hipError_t launch_relu_output_mfma(int D, const void* q, void* o, const float* prefix, float eps,
                                   long bhf, int N, int nco, int chunk, hipStream_t st);
hipError_t launch_gdn_gram_mfma(int D, const void* k, const void* v, float* partial, float c,
                                float c2, long bhf, int N, int nc, int chunk, hipStream_t st);
hipError_t launch_gdn_output_mfma(int D, const void* q, void* o, const void* states, long bhf,
                                  int N, int nco, int chunk, hipStream_t st);
hipError_t launch_summary_generic(int D, int dtype, bool relu, const void* k, const void* v,
                                  float* partial, float c, float c2, long bhf, int N, int nc, int chunk,
                                  hipStream_t st);
hipError_t launch_output_generic(int D, int dtype, bool relu, const void* q, void* o,
                                 const float* states, size_t stride, float eps, long bhf, int N,
                                 int nco, int chunk, hipStream_t st);

namespace {

__global__ __launch_bounds__(256) void relu_prefix_kernel(const float* __restrict__ partial,
                                                          const float* S0, const float* z0,
                                                          float* __restrict__ prefix, float* S_out,
                                                          float* z_out, int D, int F, int nc,
                                                          int block_frames) {
  const int OUT = D * D + D;
  const long bh = blockIdx.x;
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e >= OUT) return;
  float acc = 0.0f;
  if (e < D * D) {
    if (S0) acc = S0[(size_t)bh * D * D + e];
  } else if (z0) {
    acc = z0[(size_t)bh * D + (e - D * D)];
  }
  for (int f0 = 0; f0 < F; f0 += block_frames) {
    const int f1 = min(F, f0 + block_frames);
    for (int f = f0; f < f1; ++f)
      for (int c = 0; c < nc; ++c) acc += partial[(((size_t)bh * F + f) * nc + c) * OUT + e];
    for (int f = f0; f < f1; ++f) prefix[((size_t)bh * F + f) * OUT + e] = acc;
  }
  if (e < D * D) {
    if (S_out) S_out[(size_t)bh * D * D + e] = acc;
  } else if (z_out) {
    z_out[(size_t)bh * D + (e - D * D)] = acc;
  }
}

// One workgroup per (batch*head, 16-row block).  State rows live in LDS; G_f
// is summed over token chunks into LDS each frame; every thread owns EPT
// (row, col) entries.  HILO stores each frame's state as bf16 hi/lo planes.
template <int D, bool HILO>
__global__ __launch_bounds__(256) void gdn_scan_kernel(const float* __restrict__ partial,
                                                       const float* __restrict__ alpha,
                                                       const float* __restrict__ beta,
                                                       const float* S0, void* __restrict__ states,
                                                       float* S_out, int F, int nc) {
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

  for (int f = 0; f < F; ++f) {
    const size_t bhf = (size_t)bh * F + f;
    const float a = alpha[bhf], b = beta[bhf];
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
        const size_t idx = (size_t)(r0 + r) * D + j;
        if (HILO) {
          uint16_t h, lo;
          split_bf16(s[x], h, lo);
          uint16_t* dst = reinterpret_cast<uint16_t*>(states) + bhf * 2 * D * D;
          dst[idx] = h;
          dst[(size_t)D * D + idx] = lo;
        } else {
          reinterpret_cast<float*>(states)[bhf * D * D + idx] = s[x];
        }
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
hipError_t scan_launch(bool hilo, const float* partial, const float* alpha, const float* beta,
                       const float* S0, void* states, float* S_out, long bh, int F, int nc,
                       hipStream_t st) {
  dim3 grid((unsigned)(bh * (D / 16))), block(256);
  if (hilo)
    hipLaunchKernelGGL((gdn_scan_kernel<D, true>), grid, block, 0, st, partial, alpha, beta, S0,
                       states, S_out, F, nc);
  else
    hipLaunchKernelGGL((gdn_scan_kernel<D, false>), grid, block, 0, st, partial, alpha, beta, S0,
                       states, S_out, F, nc);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void carry_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                    size_t n, int reset) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    dst[i] = reset ? 0.0f : src[i];
}

}  // namespace

hipError_t launch_relu_summary(int D, bool mfma, int dtype, const void* k, const void* v,
                               float* partial, long bhf, int N, int nc, int chunk, hipStream_t st) {
  if (mfma) return launch_relu_summary_mfma(D, k, v, partial, bhf, N, nc, chunk, st);
  return launch_summary_generic(D, dtype, true, k, v, partial, 1.0f, 1.0f, bhf, N, nc, chunk, st);
}

hipError_t launch_relu_prefix(int D, const float* partial, const float* S0, const float* z0,
                              float* prefix, float* S_out, float* z_out, long bh, int F, int nc,
                              int block_frames, hipStream_t st) {
  dim3 grid((unsigned)bh, (unsigned)((D * D + D + 255) / 256)), block(256);
  hipLaunchKernelGGL(relu_prefix_kernel, grid, block, 0, st, partial, S0, z0, prefix, S_out, z_out,
                     D, F, nc, block_frames);
  return hipGetLastError();
}

hipError_t launch_relu_output(int D, bool mfma, int dtype, const void* q, void* o,
                              const float* prefix, float eps, long bhf, int N, int nco, int chunk,
                              hipStream_t st) {
  if (mfma) return launch_relu_output_mfma(D, q, o, prefix, eps, bhf, N, nco, chunk, st);
  return launch_output_generic(D, dtype, true, q, o, prefix, (size_t)D * D + D, eps, bhf, N, nco,
                               chunk, st);
}

hipError_t launch_gdn_gram(int D, bool mfma, int dtype, const void* k, const void* v,
                           float* partial, float c, float c2, long bhf, int N, int nc, int chunk,
                           hipStream_t st) {
  if (mfma) return launch_gdn_gram_mfma(D, k, v, partial, c, c2, bhf, N, nc, chunk, st);
  return launch_summary_generic(D, dtype, false, k, v, partial, c, c2, bhf, N, nc, chunk, st);
}

hipError_t launch_gdn_scan(int D, bool hilo, const float* partial, const float* alpha,
                           const float* beta, const float* S0, void* states, float* S_out,
                           long bh, int F, int nc, hipStream_t st) {
  switch (D) {
#define CASE(d) \
  case d: return scan_launch<d>(hilo, partial, alpha, beta, S0, states, S_out, bh, F, nc, st);
    CASE(16) CASE(32) CASE(48) CASE(64) CASE(80) CASE(96) CASE(112) CASE(128)
#undef CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gdn_output(int D, bool mfma, int dtype, const void* q, void* o,
                             const void* states, long bhf, int N, int nco, int chunk,
                             hipStream_t st) {
  if (mfma) return launch_gdn_output_mfma(D, q, o, states, bhf, N, nco, chunk, st);
  return launch_output_generic(D, dtype, false, q, o, (const float*)states, (size_t)D * D, 0.0f,
                               bhf, N, nco, chunk, st);
}

hipError_t launch_carry(const float* src, float* dst, size_t n, int reset, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(carry_kernel, dim3((unsigned)blocks), dim3(256), 0, st, src, dst, n, reset);
  return hipGetLastError();
}

}  // namespace linscan
