// gdn_mfma.hip -- bf16 MFMA kernels of the frame-wise Gated DeltaNet scan for
// head dim 128 (SANA-WM's frame-wise GDN: one state update per latent frame
// from all of its spatial tokens, keys scaled by 1/sqrt(D*N)).
//
// Gram pass: per frame, G = c^2 K^T K and U = c V^T K (each 128 x 128) are 16
// blocks of 32 x 32 apiece.  Wave w owns block row w of both, so every wave
// needs all four key fragments and one value fragment per 16-token k-step.
// The workgroup stages 64-token K and V tiles in LDS (double buffered, next
// tile's HBM loads in flight while the current one is contracted) and each
// lane gathers 8 tokens of one dimension per operand.  Inputs are exact bf16
// products accumulated in fp32; c and c^2 are applied once at the end.
//
// Output pass: o = S_f q.  Wave w computes output dims [32w, 32w + 32) from
// S_f's rows held in registers as bf16 hi + lo terms (written by the scan),
// against 64-token query tiles staged once per workgroup in LDS.
#include "device_common.h"
#include "kernels.h"

namespace linscan {

namespace {

constexpr int GD = 128;

__global__ __launch_bounds__(256, 2) void gdn_gram_mfma128(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, float* __restrict__ partial,
    float c, float c2, int N, int nc, int chunk) {
  constexpr int D = GD;
  constexpr int TILE = 64;
  constexpr int ROW = D + 4;  // 264-byte pitch: the two lane groups' gathers land 16 banks apart
  constexpr int LPT = TILE * (D / 8) / 256;  // 16-byte loads per thread per tensor per tile (4)
  __shared__ __align__(16) uint16_t lds[2][2][TILE * ROW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const long wg = blockIdx.x;
  const long bhf = wg / nc;
  const int n0 = (int)(wg % nc) * chunk;
  const int n1 = min(N, n0 + chunk);
  const uint16_t* kf = k + (size_t)bhf * N * D;
  const uint16_t* vf = v + (size_t)bhf * N * D;

  floatx16 accG[4], accU[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    accG[j] = floatx16{};
    accU[j] = floatx16{};
  }

  u32x4 kr[LPT], vr[LPT];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const int n = t0 + tok;
      if (n < n1) {
        kr[r] = ld16(kf + (size_t)n * D + cb * 8);
        vr[r] = ld16(vf + (size_t)n * D + cb * 8);
      } else {
        kr[r] = u32x4{0u, 0u, 0u, 0u};
        vr[r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      uint2* kd = reinterpret_cast<uint2*>(&lds[buf][0][tok * ROW + cb * 8]);
      uint2* vd = reinterpret_cast<uint2*>(&lds[buf][1][tok * ROW + cb * 8]);
      kd[0] = make_uint2(kr[r][0], kr[r][1]);
      kd[1] = make_uint2(kr[r][2], kr[r][3]);
      vd[0] = make_uint2(vr[r][0], vr[r][1]);
      vd[1] = make_uint2(vr[r][2], vr[r][3]);
    }
  };

  const int ntiles = (n1 - n0 + TILE - 1) / TILE;
  if (ntiles > 0) {
    fetch(n0);
    stage(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) fetch(n0 + (it + 1) * TILE);
    const uint16_t* kl = lds[buf][0];
    const uint16_t* vl = lds[buf][1];
#pragma unroll
    for (int s = 0; s < TILE / 16; ++s) {
      const int tb = s * 16 + g * 8;
      u32x4 kfrag[4], vfrag;
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const int d = J * 32 + col;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          kfrag[J][e] = (uint32_t)kl[(tb + 2 * e) * ROW + d] |
                        ((uint32_t)kl[(tb + 2 * e + 1) * ROW + d] << 16);
      }
      {
        const int d = wave * 32 + col;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vfrag[e] = (uint32_t)vl[(tb + 2 * e) * ROW + d] |
                     ((uint32_t)vl[(tb + 2 * e + 1) * ROW + d] << 16);
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        accG[J] = mfma32x32x16(as_bf16x8(kfrag[wave]), as_bf16x8(kfrag[J]), accG[J]);
        accU[J] = mfma32x32x16(as_bf16x8(vfrag), as_bf16x8(kfrag[J]), accU[J]);
      }
    }
    if (it + 1 < ntiles) stage(buf ^ 1);
    __syncthreads();
  }

  float* Gd = partial + (size_t)wg * 2 * D * D;
  float* Ud = Gd + D * D;
#pragma unroll
  for (int J = 0; J < 4; ++J) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wave * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      Gd[m * D + J * 32 + col] = c2 * accG[J][r];
      Ud[m * D + J * 32 + col] = c * accU[J][r];
    }
  }
}

__global__ __launch_bounds__(256, 2) void gdn_output_mfma128(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const uint16_t* __restrict__ states,
    int N, int nco, int chunk) {
  constexpr int D = GD;
  constexpr int TILE = 64;
  constexpr int ROW = D + 8;  // 272-byte pitch: 16-byte fragment reads spread over all banks
  constexpr int LPT = TILE * (D / 8) / 256;  // 4
  __shared__ __align__(16) uint16_t lds[2][TILE * ROW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const long wg = blockIdx.x;
  const long bhf = wg / nco;
  const int n0 = (int)(wg % nco) * chunk;
  const int n1 = min(N, n0 + chunk);

  // A operands: rows 32*wave + col of S_f, dims 16s + 8g .. +7, hi and lo planes
  const uint16_t* hi = states + (size_t)bhf * 2 * D * D;
  const uint16_t* lo = hi + D * D;
  u32x4 ahi[8], alo[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const size_t off = (size_t)(wave * 32 + col) * D + s * 16 + g * 8;
    ahi[s] = ld16(hi + off);
    alo[s] = ld16(lo + off);
  }

  const uint16_t* qf = q + (size_t)bhf * N * D;
  uint16_t* of = o + (size_t)bhf * N * D;
  u32x4 qr[LPT];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const int n = t0 + tok;
      qr[r] = (n < n1) ? ld16(qf + (size_t)n * D + cb * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      *reinterpret_cast<u32x4*>(&lds[buf][tok * ROW + cb * 8]) = qr[r];
    }
  };

  const int ntiles = (n1 - n0 + TILE - 1) / TILE;
  if (ntiles > 0) {
    fetch(n0);
    stage(0);
  }
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int t0 = n0 + it * TILE;
    if (it + 1 < ntiles) fetch(t0 + TILE);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      floatx16 acc = {};
      const uint16_t* qrow = &lds[buf][(half * 32 + col) * ROW + g * 8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(qrow + s * 16);
        acc = mfma32x32x16(as_bf16x8(ahi[s]), as_bf16x8(b), acc);
        acc = mfma32x32x16(as_bf16x8(alo[s]), as_bf16x8(b), acc);
      }
      const int t = t0 + half * 32 + col;
      if (t < n1) {
        uint16_t* orow = of + (size_t)t * D + wave * 32 + 4 * g;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint2 w;
          w.x = pack_bf16x2(acc[4 * q4 + 0], acc[4 * q4 + 1]);
          w.y = pack_bf16x2(acc[4 * q4 + 2], acc[4 * q4 + 3]);
          *reinterpret_cast<uint2*>(orow + 8 * q4) = w;
        }
      }
    }
    if (it + 1 < ntiles) stage(buf ^ 1);
    __syncthreads();
  }
}

}  // namespace

bool gdn_has_mfma(int D, int dtype) { return dtype == DT_BF16 && D == GD; }

hipError_t launch_gdn_gram_mfma(int D, const void* k, const void* v, float* partial, float c,
                                float c2, long bhf, int N, int nc, int chunk, hipStream_t st) {
  if (D != GD) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gdn_gram_mfma128, dim3((unsigned)(bhf * nc)), dim3(256), 0, st,
                     (const uint16_t*)k, (const uint16_t*)v, partial, c, c2, N, nc, chunk);
  return hipGetLastError();
}

hipError_t launch_gdn_output_mfma(int D, const void* q, void* o, const void* states, long bhf,
                                  int N, int nco, int chunk, hipStream_t st) {
  if (D != GD) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gdn_output_mfma128, dim3((unsigned)(bhf * nco)), dim3(256), 0, st,
                     (const uint16_t*)q, (uint16_t*)o, (const uint16_t*)states, N, nco, chunk);
  return hipGetLastError();
}

}  // namespace linscan
