// relu_items.h -- bf16 MFMA work items of the ReLU block-causal linear-attention
// scan for head dims 32 and 64 (SANA-Video's linear attention: ReLU feature map,
// cumulative D x D state plus normaliser, extended frame block by frame block).
//
// Summary pass: the per-frame contributions dS = V^T phi(K), dz = 1^T phi(K)
// contract over tokens, the strided axis of the [N][D] tiles, so each wave
// stages its 64-token K and V tiles in its own LDS slice and gathers 8 tokens
// of one dimension per lane as an MFMA operand with two LDS transpose reads
// (ds_read_b64_tr_b16).  The next tile's HBM loads are in flight meanwhile.
// The normaliser rides on the same MFMA with an all-ones A operand.
//
// Output pass: each workgroup first forms its frame's state from the initial
// state and the summary partials (the block-causal prefix), then o = S phi(q)
// contracts over the key dimension, which is contiguous in q, so each lane
// loads 16-byte query fragments straight from HBM as the MFMA B operand; S is
// split once into bf16 hi + lo terms (16 significant bits) held in registers,
// giving fp32-grade numerators from two bf16 MFMAs.  The denominator
// z . phi(q) is an fp32 dot product on the VALU.
#pragma once

#include "device_common.h"

namespace linscan {

// LDS bytes the summary item needs: four waves' K and V tiles, or the
// reduction of their partial sums if that is larger.
template <int D>
constexpr int relu_summary_lds_bytes() {
  return 4 * 2 * 64 * D * 2 > 4 * (D * D + D) * 4 ? 4 * 2 * 64 * D * 2 : 4 * (D * D + D) * 4;
}

// Work item `wg` = (frame of one head) * nc + token chunk: dS, dz partials of
// the chunk -> partial[wg]; item (frame 0, chunk 0) of each head also copies
// (S0, z0) into init[head].
// PRO: 0 without the per-token prologue, 1 with it, 2 with it and the rotary
// embedding (separate instantiations keep the registers of the simpler items).
// PAIR (D = 64, PRO = 0): the head is a pair of heads of dim 32 (dims 0-31
// and 32-63); only the diagonal blocks of dS are formed, the others stay zero.
template <int D, int PRO = 0, bool PAIR = false>
__device__ __forceinline__ void relu_summary_item(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, float* __restrict__ partial,
    const float* S0, const float* z0, float* __restrict__ init, int F, int N, int nc, int chunk,
    long wg, uint8_t* lds_raw, TokLayout L, Prologue P) {
  constexpr int DB = D / 32;            // 32-wide dimension blocks
  constexpr int TILE = 64;              // tokens per wave per step
  constexpr int ROW = D;                // unpadded rows, chunks swizzled by token
  constexpr int CPR = D / 8;            // 16-byte chunks per token row
  constexpr int LPT = TILE * CPR / 64;  // 16-byte loads per lane per tensor per tile
  constexpr int OUT = D * D + D;
  static_assert(!PAIR || (D == 64 && PRO == 0), "head pairs: two heads of dim 32, no prologue");
  typedef uint16_t TileT[2][TILE * ROW];
  TileT* lds = reinterpret_cast<TileT*>(lds_raw);  // [4 waves][K, V][TILE * ROW]

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, col = lane & 31;
  const long bhf = wg / nc;
  const int n0 = (int)(wg % nc) * chunk;
  const int n1 = min(N, n0 + chunk);
  const uint16_t* kf = k + L.base(bhf);
  const uint16_t* vf = v + L.base(bhf);
  uint16_t* kl = lds[wave][0];
  uint16_t* vl = lds[wave][1];
  // the prologue's key weights of the head (RMSNorm), in LDS after the tiles
  float* wl = reinterpret_cast<float*>(lds_raw + relu_summary_lds_bytes<D>());
  if (PRO && P.wk) {
    if (threadIdx.x < D) wl[threadIdx.x] = P.wk[(size_t)((bhf / L.F) % L.H) * D + threadIdx.x];
    __syncthreads();
  }

  floatx16 acc[DB][DB];
  floatx16 accz[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    accz[i] = floatx16{};
#pragma unroll
    for (int j = 0; j < DB; ++j) acc[i][j] = floatx16{};
  }
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  // with the rotary embedding: this lane's sums of the unrotated features of
  // its channels 8 (lane % CPR) .. + 7 (the staged tiles hold rotated ones)
  float zk[8] = {};

  // the next tile's rows are loaded into registers while the current tile is
  // contracted.  Every load is issued (rows past the chunk re-read its first
  // token) and such rows are zeroed when staged: loads under a lane condition
  // would make the compiler wait for every load in flight before staging.
  // (PRO == 2 at D = 32: the rotary table rows of the tile's chunks come with
  // them; at D = 64 they do not fit in registers and are read when staged)
  constexpr bool RPRE = PRO == 2 && LPT <= 4;
  u32x4 kr[LPT], vr[LPT];
  Rot8 rr[RPRE ? LPT : 1];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 64 + lane;
      const int n = t0 + ci / CPR, cb = ci % CPR;
      const size_t off = (size_t)(n < n1 ? n : n0) * L.sn + cb * 8;
      // keys and values non-temporal: a 10-frame call at H70 D32 N3600 ran
      // 140.5 -> 120.9 us; the same hint on the queries or the output
      // stores made it slower (147 and 122 us)
      kr[r] = ld16_stream(kf + off);
      vr[r] = ld16_stream(vf + off);
      if (RPRE) rr[RPRE ? r : 0] = rot8_load(P.rope8(bhf % F, n < n1 ? n : n0, cb, D));
    }
  };
  int t0 = n0 + wave * TILE;
  if (t0 < n1) fetch(t0);
  for (; t0 < n1; t0 += 4 * TILE) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 64 + lane;
      const int tok = ci / CPR, cb = ci % CPR;
      const bool live = t0 + tok < n1;
      u32x4 kk = live ? kr[r] : u32x4{0u, 0u, 0u, 0u};
      const u32x4 vv = live ? vr[r] : u32x4{0u, 0u, 0u, 0u};
      if (PRO == 2) {  // CPR consecutive lanes hold the CPR chunks of token `tok`
        // RMSNorm, the feature map, then the rotation (numerator only): the
        // normaliser sums the unrotated features
        float wk8[8] = {};
        if (P.wk) {
          const float4 a = *reinterpret_cast<const float4*>(wl + 8 * cb), b = *reinterpret_cast<const float4*>(wl + 8 * cb + 4);
          wk8[0] = a.x, wk8[1] = a.y, wk8[2] = a.z, wk8[3] = a.w, wk8[4] = b.x, wk8[5] = b.y, wk8[6] = b.z, wk8[7] = b.w;
        }
        Prologue Pf = P;
        Pf.relu = 1;
        float pre[8];
        kk = prologue_bf16x8(kk, wk8, P.wk != nullptr, Pf, true, 1.0 / D,
                             [](double x) { return group_sum_f64<CPR>(x); },
                             true, RPRE ? rr[RPRE ? r : 0] : rot8_load(P.rope8(bhf % F, live ? t0 + tok : n0, cb, D)),
                             pre);
#pragma unroll
        for (int e = 0; e < 8; ++e) zk[e] += pre[e];
      } else {
        if (PRO && P.wk) {  // CPR consecutive lanes hold the CPR chunks of token `tok`
          float wk8[8];
          const float4 a = *reinterpret_cast<const float4*>(wl + 8 * cb), b = *reinterpret_cast<const float4*>(wl + 8 * cb + 4);
          wk8[0] = a.x, wk8[1] = a.y, wk8[2] = a.z, wk8[3] = a.w, wk8[4] = b.x, wk8[5] = b.y, wk8[6] = b.z, wk8[7] = b.w;
          kk = prologue_bf16x8(kk, wk8, true, P, true, 1.0 / D, [](double x) { return group_sum_f64<CPR>(x); });
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[e] = relu_bf16x2(kk[e]);
      }
      uint2* kd = reinterpret_cast<uint2*>(kl + swz_offset<CPR>(tok, cb));
      uint2* vd = reinterpret_cast<uint2*>(vl + swz_offset<CPR>(tok, cb));
      kd[0] = make_uint2(kk[0], kk[1]);
      kd[1] = make_uint2(kk[2], kk[3]);
      vd[0] = make_uint2(vv[0], vv[1]);
      vd[1] = make_uint2(vv[2], vv[3]);
    }
    if (t0 + 4 * TILE < n1) fetch(t0 + 4 * TILE);
    __builtin_amdgcn_wave_barrier();
    // 16 tokens per MFMA k-step
#pragma unroll
    for (int s = 0; s < TILE / 16; ++s) {
      u32x4 af[DB], bfr[DB];
#pragma unroll
      for (int blk = 0; blk < DB; ++blk) {
        af[blk] = gather_tokens_32_swz<CPR>(vl, s * 16, blk * 32, lane);
        bfr[blk] = gather_tokens_32_swz<CPR>(kl, s * 16, blk * 32, lane);
      }
#pragma unroll
      for (int j = 0; j < DB; ++j) {
#pragma unroll
        for (int i = 0; i < DB; ++i)
          if (!PAIR || i == j) acc[i][j] = mfma32x32x16(as_bf16x8(af[i]), as_bf16x8(bfr[j]), acc[i][j]);
        if (PRO != 2) accz[j] = mfma32x32x16(as_bf16x8(ones), as_bf16x8(bfr[j]), accz[j]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // fixed-order reduction of the four waves' partial sums through LDS
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds_raw);
  static_assert(4 * OUT * 4 <= relu_summary_lds_bytes<D>(), "reduction buffer exceeds LDS tile space");
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
  if (PRO == 2) {
    // lanes lane % CPR + CPR m hold the same channels: sum over m
#pragma unroll
    for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) zk[e] += __shfl_xor(zk[e], o);
    if (lane < CPR) {
#pragma unroll
      for (int e = 0; e < 8; ++e) mine[D * D + lane * 8 + e] = zk[e];
    }
  } else if (g == 0) {
#pragma unroll
    for (int j = 0; j < DB; ++j) mine[D * D + j * 32 + col] = accz[j][0];
  }
  __syncthreads();
  float* dst = partial + (size_t)wg * OUT;
  for (int e = threadIdx.x; e < OUT; e += 256)
    dst[e] = ((red[e] + red[OUT + e]) + red[2 * OUT + e]) + red[3 * OUT + e];
  relu_copy_init<D, PAIR>(S0, z0, init, wg, F, nc);
}

// Row pitch (bf16) of the per-wave output staging tile [32 tokens][D + 8].
template <int D>
constexpr int relu_ostage_pitch() { return D + 8; }
// LDS bytes the output item needs: the frame state (fp32) and four per-wave
// output staging tiles.
template <int D>
constexpr int relu_output_lds_bytes() { return (D * (D + 4) + D) * 4 + 4 * 32 * relu_ostage_pitch<D>() * 2; }

// Work item `wg` = (frame of one head) * nco + token chunk: the frame's state
// from init + partials, then o = S phi(q) / (z . phi(q) + eps) for the chunk;
// the last frame's chunk-0 item writes the final state.
// PAIR (D = 64, PRO = 0): a pair of heads of dim 32 with a block-diagonal
// state; each head's rows take its own denominator, and the final state goes
// out per head.
template <int D, int PRO = 0, bool PAIR = false>
__device__ __forceinline__ void relu_output_item(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const float* __restrict__ partial,
    const float* __restrict__ init, float* S_out, float* z_out, float eps, int F, int N, int nc,
    int bfr, int nco, int chunk, long wg, uint8_t* lds_raw, TokLayout L, Prologue P) {
  constexpr int DB = D / 32;  // 32-row blocks of S (output dims)
  constexpr int KS = D / 16;  // 16-dim k-steps over the key dimension
  static_assert(!PAIR || (D == 64 && PRO == 0), "head pairs: two heads of dim 32, no prologue");
  // 32-token groups per wave per step: two at D = 64 (with four, the
  // fragments and the prologue's fp64 RMSNorm do not fit in registers; with
  // none, 35 heads x 10 frames x 3600 tokens still ran 175 -> 166 us with two)
  constexpr int U = D >= 64 ? 2 : 4;
  constexpr int STEP = 4 * U * 32;  // tokens per workgroup step
  constexpr int PITCH = D + 4;
  float* Ss = reinterpret_cast<float*>(lds_raw);  // [D][PITCH]
  float* zs = Ss + D * PITCH;                      // [D]
  constexpr int OP = relu_ostage_pitch<D>();
  // this wave's [32][OP] bf16 staging tile: MFMA results are scattered over
  // lanes by dimension, so they pass through LDS to leave as whole rows
  uint16_t* ost = reinterpret_cast<uint16_t*>(lds_raw + (D * PITCH + D) * 4) + (threadIdx.x >> 6) * 32 * OP;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, col = lane & 31;
  const long bhf = wg / nco;
  const long bh = bhf / F;
  const int f = (int)(bhf % F);
  const int n0 = (int)(wg % nco) * chunk;
  const int n1 = min(N, n0 + chunk);

  // the state this frame reads: initial state plus every frame of its block and before
  relu_frame_state<D>(partial, init, bh, f, F, nc, bfr, Ss, PITCH, zs);
  // the prologue's query weights of the head (RMSNorm), in LDS after the rest
  float* wql = reinterpret_cast<float*>(lds_raw + relu_output_lds_bytes<D>());
  if (PRO && P.wq && threadIdx.x < D) wql[threadIdx.x] = P.wq[(size_t)(bh % L.H) * D + threadIdx.x];
  __syncthreads();
  if (f == F - 1 && wg % nco == 0) {  // the last frame's state is the call's final state
    for (int e = threadIdx.x; e < D * D; e += 256) {
      constexpr int DH = D / 2;
      const int m = e / D, n = e % D;
      if (PAIR) {
        if (S_out && m / DH == n / DH)
          S_out[((size_t)2 * bh + m / DH) * DH * DH + (m % DH) * DH + n % DH] = Ss[m * PITCH + n];
      } else if (S_out) {
        S_out[(size_t)bh * D * D + e] = Ss[m * PITCH + n];
      }
    }
    if (z_out && threadIdx.x < D) z_out[(size_t)bh * D + threadIdx.x] = zs[threadIdx.x];
  }

  // A operands: S[32I + col][16s + 8g + e] as bf16 hi and lo terms
  u32x4 ahi[DB][KS], alo[DB][KS];
#pragma unroll
  for (int I = 0; I < DB; ++I) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float* src = Ss + (I * 32 + col) * PITCH + s * 16 + g * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 hl = split_bf16x2(src[2 * e], src[2 * e + 1]);
        ahi[I][s][e] = hl.x;
        alo[I][s][e] = hl.y;
      }
    }
  }
  float zr[KS][8];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) zr[s][e] = zs[s * 16 + g * 8 + e];

  const uint16_t* qf = q + L.base(bhf);
  uint16_t* of = o + L.base(bhf);
  // U groups of 32 tokens per wave; the next step's query fragments are in
  // flight while the current ones are contracted
  struct Step {
    u32x4 b[U][KS];
  };
  auto load = [&](Step& X, int t0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * 32 + col;
      const uint16_t* qrow = qf + (size_t)(t < n1 ? t : n0) * L.sn + g * 8;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        X.b[u][s] = ld16(qrow + s * 16);
      }
    }
  };
  // FULL: every token of the group step is inside the chunk, so the stores
  // need no lane condition (a store under a condition would make the
  // compiler wait for every memory operation in flight before the next
  // group's loads are used)
  // PRO == 2: the rotary table rows of group u + 1 are read while group u is
  // computed (rows of the chunks 2 s + g this lane holds); at D = 64 they do
  // not fit in registers and are read where used
  constexpr bool OPRE = PRO == 2 && KS <= 2;
  constexpr int RK = OPRE ? KS : 1;
  auto rot_rows = [&](Rot8 (&r)[RK], int t) {
#pragma unroll
    for (int s = 0; s < RK; ++s) r[s] = rot8_load(P.rope8(f, t < n1 ? t : n0, 2 * s + g, D));
  };
  auto compute = [&](Step& X, int t0, const bool full) {
    auto& b = X.b;
    Rot8 rcur[RK], rnext[RK];
    if (OPRE) rot_rows(rcur, t0 + col);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (OPRE && u + 1 < U) rot_rows(rnext, t0 + (u + 1) * 32 + col);
      if (PRO == 1 && P.wq) {  // RMSNorm of token col's query: this lane holds its dims 16 s + 8 g + 0..7
        // in fp64, rounded once to bf16 (as prologue_bf16x8)
        double ss = 0.0;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const double x0 = bf16lo_to_f32(b[u][s][e]), x1 = bf16hi_to_f32(b[u][s][e]);
            ss = fma(x0, x0, fma(x1, x1, ss));
          }
        ss += __shfl_xor(ss, 32);  // the partner lane holds the token's other dims
        const double inv = rsqrt_f64(fma(ss, 1.0 / D, (double)P.eps));
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const float4 a = *reinterpret_cast<const float4*>(wql + 16 * s + 8 * g);
          const float4 c = *reinterpret_cast<const float4*>(wql + 16 * s + 8 * g + 4);
          const float wv[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            b[u][s][e] = pack_bf16x2_f64((double)bf16lo_to_f32(b[u][s][e]) * (double)wv[2 * e] * inv,
                                         (double)bf16hi_to_f32(b[u][s][e]) * (double)wv[2 * e + 1] * inv);
        }
      }
      float den = 0.0f, inv2 = 0.0f;
      if (PRO == 2) {
        // fp64: RMSNorm (weights), the feature map, the normaliser's dot
        // product on the unrotated features, then the rotation; one rounding
        double inv = 1.0;
        if (P.wq) {
          double ss = 0.0;
#pragma unroll
          for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const double x0 = bf16lo_to_f32(b[u][s][e]), x1 = bf16hi_to_f32(b[u][s][e]);
              ss = fma(x0, x0, fma(x1, x1, ss));
            }
          ss += __shfl_xor(ss, 32);
          inv = rsqrt_f64(fma(ss, 1.0 / D, (double)P.eps));
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          double x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16lo_to_f32(b[u][s][e]);
            x[2 * e + 1] = bf16hi_to_f32(b[u][s][e]);
          }
          if (P.wq) {
            const float4 a = *reinterpret_cast<const float4*>(wql + 16 * s + 8 * g);
            const float4 c = *reinterpret_cast<const float4*>(wql + 16 * s + 8 * g + 4);
            const float wv[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = x[e] * (double)wv[e] * inv;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[e] = signbit(x[e]) ? 0.0 : x[e];
            den = fmaf(zr[s][e], (float)x[e], den);
          }
          const int tq = t0 + u * 32 + col;
          rope_rotate8(x, OPRE ? rcur[OPRE ? s : 0] : rot8_load(P.rope8(f, tq < n1 ? tq : n0, 2 * s + g, D)));
#pragma unroll
          for (int e = 0; e < 4; ++e) b[u][s][e] = pack_bf16x2_f64(x[2 * e], x[2 * e + 1]);
        }
      } else {
        // PAIR: den holds the first head's sum (k-steps s < KS / 2), den2 the second's
        float den2 = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          float& d = PAIR && s >= KS / 2 ? den2 : den;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            b[u][s][e] = relu_bf16x2(b[u][s][e]);
            d = fmaf(zr[s][2 * e], bf16lo_to_f32(b[u][s][e]), d);
            d = fmaf(zr[s][2 * e + 1], bf16hi_to_f32(b[u][s][e]), d);
          }
        }
        if (PAIR) {
          den2 += __shfl_xor(den2, 32);
          inv2 = 1.0f / (den2 + eps);
        }
      }
      den += __shfl_xor(den, 32);  // the partner lane holds the token's other dims
      const float inv1 = 1.0f / (den + eps);
#pragma unroll
      for (int I = 0; I < DB; ++I) {
        const float inv = PAIR && I == 1 ? inv2 : inv1;
        floatx16 acc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if (PAIR && s / (KS / 2) != I) continue;  // the other head's block of S is zero
          acc = mfma32x32x16(as_bf16x8(ahi[I][s]), as_bf16x8(b[u][s]), acc);
          acc = mfma32x32x16(as_bf16x8(alo[I][s]), as_bf16x8(b[u][s]), acc);
        }
        // lane (col, g) holds token col's dims I*32 + 8 q4 + 4 g + 0..3
        uint16_t* srow = ost + col * OP + I * 32 + 4 * g;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint2 w;
          w.x = pack_bf16x2(acc[4 * q4 + 0] * inv, acc[4 * q4 + 1] * inv);
          w.y = pack_bf16x2(acc[4 * q4 + 2] * inv, acc[4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(srow + 8 * q4) = w;
        }
      }
      __builtin_amdgcn_wave_barrier();
      // whole rows out: D/8 lanes per token, 16 bytes each, consecutive lanes
      // on consecutive bytes
      constexpr int LPR = D / 8;        // lanes per token row
      constexpr int TPI = 64 / LPR;     // tokens per store instruction
#pragma unroll
      for (int i = 0; i < 32 / TPI; ++i) {
        const int tl = i * TPI + lane / LPR, cb = lane % LPR;
        const u32x4 w = *reinterpret_cast<const u32x4*>(ost + tl * OP + cb * 8);
        const int tt = t0 + u * 32 + tl;
        if (full || tt < n1) st16(of + (size_t)tt * L.sn + cb * 8, w);
      }
      __builtin_amdgcn_wave_barrier();
      if (OPRE) {
#pragma unroll
        for (int s = 0; s < RK; ++s) rcur[s] = rnext[s];
      }
    }
  };
  // This wave's steps of U * 32 tokens start at n0 + wave * U * 32 and every
  // STEP after; the first nfull of them lie inside the chunk, at most one
  // more is partial.  Loads past the chunk re-read its first token, so every
  // load is issued unconditionally; the main loop has no branch.
  if (n0 >= n1) return;
  const int first = n0 + wave * U * 32;
  const int nfull = first + U * 32 <= n1 ? (n1 - first - U * 32) / STEP + 1 : 0;
  Step b0, b1;
  int t0 = first;
  load(b0, t0);
  int k = 0;
  for (; k + 2 <= nfull; k += 2, t0 += 2 * STEP) {
    load(b1, t0 + STEP);
    compute(b0, t0, true);
    load(b0, t0 + 2 * STEP);
    compute(b1, t0 + STEP, true);
  }
  // b0 holds step k: one more full step and/or a partial one
  if (k < nfull) {
    load(b1, t0 + STEP);
    compute(b0, t0, true);
    if (t0 + STEP < n1) compute(b1, t0 + STEP, false);
  } else if (t0 < n1) {
    compute(b0, t0, false);
  }
}

}  // namespace linscan
