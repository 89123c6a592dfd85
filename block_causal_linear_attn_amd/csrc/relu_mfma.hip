// relu_mfma.hip -- bf16 MFMA kernels of the ReLU block-causal linear-attention
// scan for head dims 32 and 64 (SANA-Video's linear attention: ReLU feature map,
// cumulative D x D state plus normaliser, extended frame block by frame block).
//
// Summary pass: the per-frame contributions dS = V^T phi(K), dz = 1^T phi(K)
// contract over tokens, the strided axis of the [N][D] tiles, so each wave
// stages its 64-token K and V tiles in its own LDS slice and gathers 8 tokens
// of one dimension per lane as an MFMA operand.  The normaliser rides on the
// same MFMA with an all-ones A operand.
//
// Output pass: o = S phi(q) contracts over the key dimension, which is
// contiguous in q, so each lane loads 16-byte query fragments straight from
// HBM as the MFMA B operand; S is split once into bf16 hi + lo terms (16
// significant bits) held in registers, giving fp32-grade numerators from two
// bf16 MFMAs.  The denominator z . phi(q) is an fp32 dot product on the VALU.
#include "device_common.h"
#include "kernels.h"

namespace linscan {

namespace {

template <int D>
__global__ __launch_bounds__(256, 2) void relu_summary_mfma(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, float* __restrict__ partial,
    int N, int nc, int chunk) {
  constexpr int DB = D / 32;            // 32-wide dimension blocks
  constexpr int TILE = 64;              // tokens per wave per step
  constexpr int ROW = D + 4;            // LDS row pitch (bf16): +8 bytes keeps gathers conflict-free
  constexpr int CPR = D / 8;            // 16-byte chunks per token row
  constexpr int LPT = TILE * CPR / 64;  // 16-byte loads per lane per tensor per tile
  constexpr int OUT = D * D + D;
  __shared__ __align__(16) uint16_t lds[4][2][TILE * ROW];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, col = lane & 31;
  const long wg = blockIdx.x;
  const long bhf = wg / nc;
  const int n0 = (int)(wg % nc) * chunk;
  const int n1 = min(N, n0 + chunk);
  const uint16_t* kf = k + (size_t)bhf * N * D;
  const uint16_t* vf = v + (size_t)bhf * N * D;
  uint16_t* kl = lds[wave][0];
  uint16_t* vl = lds[wave][1];

  floatx16 acc[DB][DB];
  floatx16 accz[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    accz[i] = floatx16{};
#pragma unroll
    for (int j = 0; j < DB; ++j) acc[i][j] = floatx16{};
  }
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

  for (int t0 = n0 + wave * TILE; t0 < n1; t0 += 4 * TILE) {
    // stage this wave's tile: token rows of K (ReLU applied) and V
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 64 + lane;
      const int tok = ci / CPR, cb = ci % CPR;
      const int n = t0 + tok;
      u32x4 kk = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (n < n1) {
        kk = ld16(kf + (size_t)n * D + cb * 8);
        vv = ld16(vf + (size_t)n * D + cb * 8);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[e] = relu_bf16x2(kk[e]);
      uint2* kd = reinterpret_cast<uint2*>(kl + tok * ROW + cb * 8);
      uint2* vd = reinterpret_cast<uint2*>(vl + tok * ROW + cb * 8);
      kd[0] = make_uint2(kk[0], kk[1]);
      kd[1] = make_uint2(kk[2], kk[3]);
      vd[0] = make_uint2(vv[0], vv[1]);
      vd[1] = make_uint2(vv[2], vv[3]);
    }
    __builtin_amdgcn_wave_barrier();
    // 16 tokens per MFMA k-step; lane group g takes tokens 8g..8g+7 of the step
#pragma unroll
    for (int s = 0; s < TILE / 16; ++s) {
      const int tb = s * 16 + g * 8;
      u32x4 af[DB], bfr[DB];
#pragma unroll
      for (int blk = 0; blk < DB; ++blk) {
        const int d = blk * 32 + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          af[blk][e] = (uint32_t)vl[(tb + 2 * e) * ROW + d] |
                       ((uint32_t)vl[(tb + 2 * e + 1) * ROW + d] << 16);
          bfr[blk][e] = (uint32_t)kl[(tb + 2 * e) * ROW + d] |
                        ((uint32_t)kl[(tb + 2 * e + 1) * ROW + d] << 16);
        }
      }
#pragma unroll
      for (int j = 0; j < DB; ++j) {
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i][j] = mfma32x32x16(as_bf16x8(af[i]), as_bf16x8(bfr[j]), acc[i][j]);
        accz[j] = mfma32x32x16(as_bf16x8(ones), as_bf16x8(bfr[j]), accz[j]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // fixed-order reduction of the four waves' partial sums through LDS
  __syncthreads();
  float* red = reinterpret_cast<float*>(&lds[0][0][0]);
  static_assert(4 * OUT * 4 <= (int)sizeof(lds), "reduction buffer exceeds LDS tile space");
  float* mine = red + wave * OUT;
#pragma unroll
  for (int i = 0; i < DB; ++i) {
#pragma unroll
    for (int j = 0; j < DB; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        mine[m * D + j * 32 + col] = acc[i][j][r];
      }
    }
  }
  if (g == 0) {
#pragma unroll
    for (int j = 0; j < DB; ++j) mine[D * D + j * 32 + col] = accz[j][0];
  }
  __syncthreads();
  float* dst = partial + (size_t)wg * OUT;
  for (int e = threadIdx.x; e < OUT; e += 256)
    dst[e] = ((red[e] + red[OUT + e]) + red[2 * OUT + e]) + red[3 * OUT + e];
}

template <int D>
__global__ __launch_bounds__(256) void relu_output_mfma(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const float* __restrict__ prefix,
    float eps, int N, int nco, int chunk) {
  constexpr int DB = D / 32;  // 32-row blocks of S (output dims)
  constexpr int KS = D / 16;  // 16-dim k-steps over the key dimension
  constexpr int TILE = 32;    // tokens per wave per step

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, col = lane & 31;
  const long wg = blockIdx.x;
  const long bhf = wg / nco;
  const int n0 = (int)(wg % nco) * chunk;
  const int n1 = min(N, n0 + chunk);
  const float* Sf = prefix + (size_t)bhf * (D * D + D);
  const float* zf = Sf + D * D;

  // A operands: S[32I + col][16s + 8g + e] as bf16 hi and lo terms
  u32x4 ahi[DB][KS], alo[DB][KS];
#pragma unroll
  for (int I = 0; I < DB; ++I) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float* src = Sf + (size_t)(I * 32 + col) * D + s * 16 + g * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint16_t h0, l0, h1, l1;
        split_bf16(src[2 * e], h0, l0);
        split_bf16(src[2 * e + 1], h1, l1);
        ahi[I][s][e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        alo[I][s][e] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
    }
  }
  float zr[KS][8];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) zr[s][e] = zf[s * 16 + g * 8 + e];

  for (int t0 = n0 + wave * TILE; t0 < n1; t0 += 4 * TILE) {
    const int t = t0 + col;
    const bool valid = t < n1;
    const uint16_t* qrow = q + ((size_t)bhf * N + (valid ? t : n0)) * D;
    u32x4 b[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      b[s] = ld16(qrow + s * 16 + g * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) b[s][e] = relu_bf16x2(b[s][e]);
    }
    float den = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        den = fmaf(zr[s][2 * e], bf16lo_to_f32(b[s][e]), den);
        den = fmaf(zr[s][2 * e + 1], bf16hi_to_f32(b[s][e]), den);
      }
    }
    den += __shfl_xor(den, 32);  // the partner lane holds the token's other dims
    const float inv = 1.0f / (den + eps);
    uint16_t* orow = o + ((size_t)bhf * N + t) * D;
#pragma unroll
    for (int I = 0; I < DB; ++I) {
      floatx16 acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        acc = mfma32x32x16(as_bf16x8(ahi[I][s]), as_bf16x8(b[s]), acc);
        acc = mfma32x32x16(as_bf16x8(alo[I][s]), as_bf16x8(b[s]), acc);
      }
      if (valid) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint2 w;
          w.x = pack_bf16x2(acc[4 * q4 + 0] * inv, acc[4 * q4 + 1] * inv);
          w.y = pack_bf16x2(acc[4 * q4 + 2] * inv, acc[4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + I * 32 + 8 * q4 + 4 * g) = w;
        }
      }
    }
  }
}

}  // namespace

bool relu_has_mfma(int D, int dtype) { return dtype == DT_BF16 && (D == 32 || D == 64); }

hipError_t launch_relu_summary_mfma(int D, const void* k, const void* v, float* partial, long bhf,
                                    int N, int nc, int chunk, hipStream_t st) {
  dim3 grid((unsigned)(bhf * nc)), block(256);
  if (D == 32)
    hipLaunchKernelGGL(relu_summary_mfma<32>, grid, block, 0, st, (const uint16_t*)k,
                       (const uint16_t*)v, partial, N, nc, chunk);
  else if (D == 64)
    hipLaunchKernelGGL(relu_summary_mfma<64>, grid, block, 0, st, (const uint16_t*)k,
                       (const uint16_t*)v, partial, N, nc, chunk);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_relu_output_mfma(int D, const void* q, void* o, const float* prefix, float eps,
                                   long bhf, int N, int nco, int chunk, hipStream_t st) {
  dim3 grid((unsigned)(bhf * nco)), block(256);
  if (D == 32)
    hipLaunchKernelGGL(relu_output_mfma<32>, grid, block, 0, st, (const uint16_t*)q, (uint16_t*)o,
                       prefix, eps, N, nco, chunk);
  else if (D == 64)
    hipLaunchKernelGGL(relu_output_mfma<64>, grid, block, 0, st, (const uint16_t*)q, (uint16_t*)o,
                       prefix, eps, N, nco, chunk);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace linscan
