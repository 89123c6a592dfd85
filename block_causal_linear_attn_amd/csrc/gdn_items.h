// gdn_items.h -- bf16 MFMA work items of the frame-wise Gated DeltaNet scan for
// head dim 128 (SANA-WM's frame-wise GDN: one state update per latent frame
// from all of its spatial tokens, keys scaled by 1/sqrt(D*N)).
//
// Gram pass: per frame, G = c^2 K^T K and U = c V^T K (each 128 x 128) are 16
// blocks of 32 x 32 apiece.  Wave w owns block row w of both, so every wave
// needs all four key fragments and one value fragment per 16-token k-step.
// The workgroup stages 64-token K and V tiles in LDS (double buffered, next
// tile's HBM loads in flight while the current one is contracted; rows
// unpadded with their 16-byte chunks swizzled by token) and each lane gathers
// 8 tokens of one dimension per operand with two LDS transpose reads.  Inputs are exact bf16
// products accumulated in fp32; c and c^2 are applied once at the end.
//
// Output pass: o = S_f q.  Wave w computes output dims [32w, 32w + 32) from
// S_f's rows held in registers as bf16 hi + lo terms (written by the scan),
// against 64-token query tiles staged once per workgroup in LDS.  The lo term
// matters: o sums 128 products that often cancel, and S rounded to bf16
// alone would leave an error of 2^-9 of the products' size in such outputs.
#pragma once

#include "device_common.h"
#include "sync.h"

namespace linscan {

constexpr int GD = 128;
// bytes of one (frame, token chunk) record: beta*G hi and lo planes (bf16) + beta*U (fp32)
constexpr size_t kRecBytes = 8 * (size_t)GD * GD;

constexpr int kGramLds = 2 * 2 * 64 * GD * 2;
constexpr int kGramDepth = 2;  // tiles in flight per gram item
// per-token gates of the two staged tiles, after the tiles (gated items only)
constexpr int kGateLds = 2 * 64 * 4;
// the prologue's key weights of the item's head, after the gates
constexpr int kPrologueLds = GD * 4;

// The prologue's weights of head h (zero past DI) into LDS, then a barrier;
// a no-op without weights.
__device__ __forceinline__ void stage_weights(const float* w, long h, int DI, float* wl) {
  if (!w) return;
  if (threadIdx.x < GD) wl[threadIdx.x] = (int)threadIdx.x < DI ? w[(size_t)h * DI + threadIdx.x] : 0.0f;
  __syncthreads();
}
// The 8 weights of channels 8 cb .. 8 cb + 7 from LDS (two 16-byte reads).
__device__ __forceinline__ void weights8_lds(const float* wl, int cb, float (&wt)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(wl + 8 * cb);
  const float4 b = *reinterpret_cast<const float4*>(wl + 8 * cb + 4);
  wt[0] = a.x, wt[1] = a.y, wt[2] = a.z, wt[3] = a.w, wt[4] = b.x, wt[5] = b.y, wt[6] = b.z, wt[7] = b.w;
}

// Work item `wg` = (frame of one head) * nc + token chunk: the chunk's record
// (beta*G hi/lo planes, beta*U) -> rec + wg * kRecBytes.  DI is the head dim
// of the tensors (112 or 128); the items work on 128 dims, the dims past DI
// being zero.
//
// TG (per-token update gate): `beta` holds one gate per token, [B*H*F][N],
// and token n's terms of G and U carry its gate: G = sum_n b_n k_n k_n^T,
// U = sum_n b_n v_n k_n^T (times c^2 and c).  The gates of a tile go to LDS
// with it, and each MFMA's A operands (this wave's key and value fragments,
// 8 tokens per lane) are scaled by their tokens' gates and split into bf16
// hi + lo terms, each contracted against the exact B operand: twice the
// MFMAs, products to ~2^-17.  (Rounding the scaled operand to bf16 alone
// leaves errors of 2^-9 of single products, which outputs that cancel, such
// as a query nearly orthogonal to the keys, turn into large relative errors.)
// The record then carries no further gate factor.
//
// PRO: keys pass through the per-token prologue P when it is on (see
// prologue_bf16x8); a separate instantiation, so that calls without it keep
// the registers its fp64 arithmetic takes.
template <int DI = GD, bool TG = false, bool PRO = false>
__device__ __forceinline__ void gdn_gram_item(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ beta,
    uint8_t* __restrict__ rec, float c, float c2, int N, int nc, int chunk, long wg, uint8_t* lds_raw,
    TokLayout L, Prologue P) {
  constexpr int D = GD;
  constexpr int CI = DI / 8;  // 16-byte chunks per token row in memory
  constexpr int TILE = 64;
  constexpr int ROW = D;  // unpadded rows, chunks swizzled by token (conflict-free transpose reads)
  constexpr int C = D / 8;
  constexpr int LPT = TILE * (D / 8) / 256;  // 16-byte loads per thread per tensor per tile (4)
  typedef uint16_t TileT[2][TILE * ROW];
  TileT* lds = reinterpret_cast<TileT*>(lds_raw);  // [buffer][K, V][TILE * ROW]
  float(*gl)[TILE] = reinterpret_cast<float(*)[TILE]>(lds_raw + kGramLds);  // [buffer][token] gates (TG)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const long bhf = wg / nc;
  const int n0 = (int)(wg % nc) * chunk;
  const int n1 = min(N, n0 + chunk);
  const uint16_t* kf = k + L.base(bhf);
  const uint16_t* vf = v + L.base(bhf);
  const float* gf = TG ? beta + (size_t)bhf * N : beta;  // token gates of the frame (TG)
  // the prologue's key weights of the head, in LDS after the gates
  float* wl = reinterpret_cast<float*>(lds_raw + kGramLds + kGateLds);
  if (PRO) stage_weights(P.wk, (bhf / L.F) % L.H, DI, wl);
  auto row16 = [](double x) { return group_sum_f64<16>(x); };

  floatx16 accG[4], accU[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    accG[j] = floatx16{};
    accU[j] = floatx16{};
  }

  // Tiles of the chunk are fetched into a ring of kGramDepth register sets
  // (tile t in set t % kGramDepth until staged), so that many tiles are in
  // flight while one is contracted from LDS.  The loop body has no branch: it
  // runs a whole number of ring passes, tiles past the chunk are staged as
  // zeros (every row fails the token check) and add nothing, and fetches past
  // the chunk re-read its last tile.  A load or stage under a condition would
  // make the compiler wait for every load in flight at every stage.
  constexpr int DEPTH = PRO ? 1 : kGramDepth;
  struct Regs {
    u32x4 k[LPT], v[LPT];
    float b;  // gate of token tid % 64 of the tile (TG)
  };
  Regs R[DEPTH];
  auto fetch = [&](Regs& X, int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const int n = t0 + tok;
      const size_t off = (size_t)(n < n1 ? n : n0) * L.sn + (cb < CI ? cb : CI - 1) * 8;
      // plain loads: the GDN call at 720p 60 s ran 1170 -> 1139 us against
      // non-temporal ones (the output stores stay non-temporal)
      X.k[r] = ld16(kf + off);
      X.v[r] = ld16(vf + off);
    }
    if (TG) X.b = gf[t0 + (tid & 63) < n1 ? t0 + (tid & 63) : n0];
  };
  auto stage = [&](const Regs& X, int buf, int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const bool live = t0 + tok < n1 && cb < CI;
      const u32x4 kk = live ? X.k[r] : u32x4{0u, 0u, 0u, 0u};
      const u32x4 vv = live ? X.v[r] : u32x4{0u, 0u, 0u, 0u};
      uint2* kd = reinterpret_cast<uint2*>(&lds[buf][0][swz_offset<C>(tok, cb)]);
      uint2* vd = reinterpret_cast<uint2*>(&lds[buf][1][swz_offset<C>(tok, cb)]);
      kd[0] = make_uint2(kk[0], kk[1]);
      kd[1] = make_uint2(kk[2], kk[3]);
      vd[0] = make_uint2(vv[0], vv[1]);
      vd[1] = make_uint2(vv[2], vv[3]);
    }
    if (TG && tid < TILE) gl[buf][tid] = X.b;
    if (PRO && P.on_k()) {
      // the prologue on the staged key chunks, in place, one chunk at a time
      // (each thread reads back only what it wrote; the 16 lanes of a DPP row
      // hold the 16 chunks of token `tok`)
#pragma unroll 1
      for (int r = 0; r < LPT; ++r) {
        const int ci = r * 256 + tid;
        const int tok = ci >> 4, cb = ci & 15;
        uint2* kd = reinterpret_cast<uint2*>(&lds[buf][0][swz_offset<C>(tok, cb)]);
        const uint2 a = kd[0], b = kd[1];
        float wk8[8];
        weights8_lds(wl, cb, wk8);
        // rotary table row of this token (rows past the chunk: a real token's)
        const Rot8 rot = P.rope() ? rot8_load(P.rope8(bhf % L.F, t0 + tok < n1 ? t0 + tok : n0, cb < CI ? cb : 0, DI))
                                  : Rot8{};
        const u32x4 kk =
            prologue_bf16x8(u32x4{a.x, a.y, b.x, b.y}, wk8, P.wk != nullptr, P, true, 1.0 / DI, row16, P.rope(), rot);
        kd[0] = make_uint2(kk[0], kk[1]);
        kd[1] = make_uint2(kk[2], kk[3]);
      }
    }
  };
  auto contract = [&](int buf) {
    const uint16_t* kl = lds[buf][0];
    const uint16_t* vl = lds[buf][1];
#pragma unroll
    for (int s = 0; s < TILE / 16; ++s) {
      u32x4 kfrag[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) kfrag[J] = gather_tokens_32_swz<C>(kl, s * 16, J * 32, lane);
      const u32x4 vfrag = gather_tokens_32_swz<C>(vl, s * 16, wave * 32, lane);
      if (TG) {  // gates of this lane's tokens s*16 + 8g + 0..7
        const float4* gb = reinterpret_cast<const float4*>(&gl[buf][s * 16 + 8 * g]);
        const float4 g0 = gb[0], g1 = gb[1];
        u32x4 kh, kl2, vh, vl2;
        scale_split_bf16x8(kfrag[wave], g0, g1, kh, kl2);
        scale_split_bf16x8(vfrag, g0, g1, vh, vl2);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          accG[J] = mfma32x32x16(as_bf16x8(kh), as_bf16x8(kfrag[J]), accG[J]);
          accG[J] = mfma32x32x16(as_bf16x8(kl2), as_bf16x8(kfrag[J]), accG[J]);
          accU[J] = mfma32x32x16(as_bf16x8(vh), as_bf16x8(kfrag[J]), accU[J]);
          accU[J] = mfma32x32x16(as_bf16x8(vl2), as_bf16x8(kfrag[J]), accU[J]);
        }
        continue;
      }
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        accG[J] = mfma32x32x16(as_bf16x8(kfrag[wave]), as_bf16x8(kfrag[J]), accG[J]);
        accU[J] = mfma32x32x16(as_bf16x8(vfrag), as_bf16x8(kfrag[J]), accU[J]);
      }
    }
  };

  const int ntiles = (n1 - n0 + TILE - 1) / TILE;
  if (ntiles > 0) {
    const int tlast = n0 + (ntiles - 1) * TILE;
    const int nsteps = (ntiles + DEPTH - 1) / DEPTH * DEPTH;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) fetch(R[d], min(n0 + d * TILE, tlast));
    stage(R[0], 0, n0);
    fetch(R[0], min(n0 + DEPTH * TILE, tlast));
    __syncthreads();
    for (int it0 = 0; it0 < nsteps; it0 += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int it = it0 + u;
        contract(it & 1);
        Regs& nxt = R[(u + 1) % DEPTH];  // holds tile it + 1
        stage(nxt, (it + 1) & 1, n0 + (it + 1) * TILE);
        fetch(nxt, min(n0 + (it + 1 + DEPTH) * TILE, tlast));
        __syncthreads();
      }
    }
  }

  // record of this (frame, chunk): beta*G as bf16 hi and lo planes (row-major),
  // then beta*U in fp32 with each group of four rows interleaved, element
  // (m, n) at ((m / 4) * D + n) * 4 + m % 4, so that the four rows a scan lane
  // owns in one column are one 16-byte load
  const float bf = TG ? 1.0f : beta[bhf];
  const float gs = c2 * bf, us = c * bf;
  uint16_t* Ghi = reinterpret_cast<uint16_t*>(rec + (size_t)wg * kRecBytes);
  uint16_t* Glo = Ghi + D * D;
  float* Ud = reinterpret_cast<float*>(Glo + D * D);
#pragma unroll
  for (int J = 0; J < 4; ++J) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wave * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      uint16_t h, l;
      split_bf16(gs * accG[J][r], h, l);
      Ghi[m * D + J * 32 + col] = h;
      Glo[m * D + J * 32 + col] = l;
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int m0 = wave * 32 + 8 * q4 + 4 * g;  // rows m0 .. m0 + 3 sit in regs 4 q4 .. 4 q4 + 3
      float4 u4 = make_float4(us * accU[J][4 * q4], us * accU[J][4 * q4 + 1], us * accU[J][4 * q4 + 2],
                              us * accU[J][4 * q4 + 3]);
      *reinterpret_cast<float4*>(Ud + ((size_t)(m0 >> 2) * D + J * 32 + col) * 4) = u4;
    }
  }
}

// Row-split gram pass, for calls with few frames: work item `item` =
// (frame of one head) * 4 + w computes block row w (rows 32w .. 32w + 31) of
// beta*G and beta*U over all of the frame's tokens, so the four items of a
// frame write disjoint parts of one record and no partial records need to be
// summed.  Each 64-token tile stages K (all dims) and the w-th 32 dims of V
// in LDS; wave j accumulates G(w, j) = sum k_w k_j^T and U(w, j) = sum v_w k_j^T
// (two accumulators), which leaves registers for several tiles in flight.  The
// four items of a frame read K four times, from HBM once and otherwise from
// their XCD's L2.
constexpr int kGramRowsKRow = GD, kGramRowsVRow = 32;  // unpadded; K chunks swizzled by token
constexpr int kGramRowsDepth = 4;  // tiles in flight per workgroup
constexpr int kGramRowsLds = 2 * 64 * (kGramRowsKRow + kGramRowsVRow) * 2;  // RB = 32 (+ kGateLds with TG)

// TG: per-token gates as in gdn_gram_item (the A operands, key and value
// fragments, scaled and split into hi + lo before each MFMA pair; gates in
// LDS after the tiles).
// LDS bytes of the row-split gram accumulation over RB-row blocks: double
// buffered 64-token tiles of K (all dims) and of the block's RB dims of V.
template <int RB>
constexpr int gram_rows_lds() { return 2 * 64 * (GD + RB) * 2; }

// The accumulation of the row-split gram item over rows RB*w .. RB*w + RB - 1
// (RB = 32 or 64, NB = RB / 32 blocks of 32 rows): wave j of the workgroup
// ends with G(32 (NB w + b), j) = sum k k_j^T over those rows in accG[b] and
// U(32 (NB w + b), j) = sum v k_j^T in accU[b] (unscaled), over all N tokens
// of frame bhf (one head's frame).
template <int DI = GD, bool TG = false, bool PRO = false, int RB = 32>
__device__ __forceinline__ void gram_rows_accumulate(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ beta, int N,
    long bhf, int w, uint8_t* lds_raw, TokLayout L, Prologue P, floatx16 (&accG)[RB / 32],
    floatx16 (&accU)[RB / 32]) {
  static_assert(RB == 32 || RB == 64, "row blocks of 32 or 64 rows");
  constexpr int D = GD;
  constexpr int NB = RB / 32;
  constexpr int CI = DI / 8;  // 16-byte chunks per token row in memory
  constexpr int TILE = 64;
  constexpr int KROW = kGramRowsKRow, VROW = RB;
  constexpr int VCH = RB / 8;                 // 16-byte chunks of a token's V slice
  constexpr int KLPT = TILE * (D / 8) / 256;  // 16-byte K loads per thread per tile (4)
  constexpr int VLPT = TILE * VCH / 256;      // 16-byte V loads per thread per tile (1 or 2)
  uint16_t* kl[2] = {reinterpret_cast<uint16_t*>(lds_raw),
                     reinterpret_cast<uint16_t*>(lds_raw) + TILE * KROW};
  uint16_t* vl[2] = {reinterpret_cast<uint16_t*>(lds_raw) + 2 * TILE * KROW,
                     reinterpret_cast<uint16_t*>(lds_raw) + 2 * TILE * KROW + TILE * VROW};
  float(*gl)[TILE] = reinterpret_cast<float(*)[TILE]>(lds_raw + gram_rows_lds<RB>());  // [buffer][token] gates (TG)

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5;
  const uint16_t* kf = k + L.base(bhf);
  const uint16_t* vf = v + L.base(bhf);
  const float* gf = TG ? beta + (size_t)bhf * N : beta;  // token gates of the frame (TG)
  float* wl = reinterpret_cast<float*>(lds_raw + gram_rows_lds<RB>() + kGateLds);  // the prologue's key weights
  if (PRO) stage_weights(P.wk, (bhf / L.F) % L.H, DI, wl);
  auto row16 = [](double x) { return group_sum_f64<16>(x); };

#pragma unroll
  for (int b = 0; b < NB; ++b) {
    accG[b] = floatx16{};
    accU[b] = floatx16{};
  }
  struct Regs {
    u32x4 k[KLPT], v[VLPT];
    float b;  // gate of token tid % 64 of the tile (TG)
  };
  constexpr int DEPTH = PRO ? 2 : kGramRowsDepth;
  Regs R[DEPTH];
  // K: token ci >> 4, 16-byte chunk ci & 15; V: token ci / VCH, chunk
  // ci % VCH of the block's RB dims.  Every load is issued (rows past the
  // frame re-read token 0) and such rows are zeroed when staged, so that the
  // compiler can count the loads in flight instead of waiting for all of them.
  auto fetch = [&](Regs& R, int t0) {
#pragma unroll
    for (int r = 0; r < KLPT; ++r) {
      const int ci = r * 256 + tid;
      const int n = t0 + (ci >> 4);
      R.k[r] = ld16(kf + (size_t)(n < N ? n : 0) * L.sn + ((ci & 15) < CI ? (ci & 15) : CI - 1) * 8);
    }
#pragma unroll
    for (int r = 0; r < VLPT; ++r) {
      const int ci = r * 256 + tid;
      const int n = t0 + ci / VCH, vc = VCH * w + ci % VCH;
      R.v[r] = ld16(vf + (size_t)(n < N ? n : 0) * L.sn + (vc < CI ? vc : CI - 1) * 8);
    }
    if (TG) R.b = gf[t0 + (tid & 63) < N ? t0 + (tid & 63) : 0];
  };
  auto stage = [&](const Regs& R, int buf, int t0) {
    // keep the zeroing of rows past the frame here: hoisted to the top of
    // the unrolled pass, the selects of every set of the ring made the
    // compiler wait for all loads in flight (vmcnt(0)) once per pass
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < KLPT; ++r) {
      const int ci = r * 256 + tid;
      const u32x4 kk = t0 + (ci >> 4) < N && (ci & 15) < CI ? R.k[r] : u32x4{0u, 0u, 0u, 0u};
      uint2* kd = reinterpret_cast<uint2*>(kl[buf] + swz_offset<KROW / 8>(ci >> 4, ci & 15));
      kd[0] = make_uint2(kk[0], kk[1]);
      kd[1] = make_uint2(kk[2], kk[3]);
    }
    if (PRO && P.on_k()) {  // in place on the staged chunks, one at a time (as in gdn_gram_item)
#pragma unroll 1
      for (int r = 0; r < KLPT; ++r) {
        const int ci = r * 256 + tid;
        uint2* kd = reinterpret_cast<uint2*>(kl[buf] + swz_offset<KROW / 8>(ci >> 4, ci & 15));
        const uint2 a = kd[0], b = kd[1];
        float wk8[8];
        weights8_lds(wl, ci & 15, wk8);
        const int n = t0 + (ci >> 4);
        const Rot8 rot = P.rope() ? rot8_load(P.rope8(bhf % L.F, n < N ? n : 0, (ci & 15) < CI ? (ci & 15) : 0, DI))
                                  : Rot8{};
        const u32x4 kk =
            prologue_bf16x8(u32x4{a.x, a.y, b.x, b.y}, wk8, P.wk != nullptr, P, true, 1.0 / DI, row16, P.rope(), rot);
        kd[0] = make_uint2(kk[0], kk[1]);
        kd[1] = make_uint2(kk[2], kk[3]);
      }
    }
#pragma unroll
    for (int r = 0; r < VLPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci / VCH, ch = ci % VCH;
      const u32x4 vv = t0 + tok < N && VCH * w + ch < CI ? R.v[r] : u32x4{0u, 0u, 0u, 0u};
      uint2* vd = reinterpret_cast<uint2*>(vl[buf] + swz_offset<VCH>(tok, ch));
      vd[0] = make_uint2(vv[0], vv[1]);
      vd[1] = make_uint2(vv[2], vv[3]);
    }
    if (TG && tid < TILE) gl[buf][tid] = R.b;
  };
  auto contract = [&](int buf) {
#pragma unroll
    for (int s = 0; s < TILE / 16; ++s) {
      const u32x4 kj = gather_tokens_32_swz<KROW / 8>(kl[buf], s * 16, 32 * wave, lane);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x4 kw = gather_tokens_32_swz<KROW / 8>(kl[buf], s * 16, RB * w + 32 * b, lane);
        const u32x4 vw = gather_tokens_32_swz<VCH>(vl[buf], s * 16, 32 * b, lane);
        if (TG) {  // gates of this lane's tokens s*16 + 8g + 0..7, hi + lo (see gdn_gram_item)
          const float4* gb = reinterpret_cast<const float4*>(&gl[buf][s * 16 + 8 * g]);
          const float4 g0 = gb[0], g1 = gb[1];
          u32x4 kh, kl2, vh, vl2;
          scale_split_bf16x8(kw, g0, g1, kh, kl2);
          scale_split_bf16x8(vw, g0, g1, vh, vl2);
          accG[b] = mfma32x32x16(as_bf16x8(kh), as_bf16x8(kj), accG[b]);
          accG[b] = mfma32x32x16(as_bf16x8(kl2), as_bf16x8(kj), accG[b]);
          accU[b] = mfma32x32x16(as_bf16x8(vh), as_bf16x8(kj), accU[b]);
          accU[b] = mfma32x32x16(as_bf16x8(vl2), as_bf16x8(kj), accU[b]);
        } else {
          accG[b] = mfma32x32x16(as_bf16x8(kw), as_bf16x8(kj), accG[b]);
          accU[b] = mfma32x32x16(as_bf16x8(vw), as_bf16x8(kj), accU[b]);
        }
      }
    }
  };

  // tile t sits in register set t % DEPTH from its fetch until it is staged,
  // so DEPTH tiles stay in flight while one is contracted from LDS (the loop
  // runs DEPTH tiles per pass so that every set index is a constant).  The
  // loop body has no branch: it runs a whole number of passes, tiles past the
  // end are staged as zeros (every row fails the token check) and add
  // nothing, and fetches past the end re-read the last tile (from L2).  A
  // fetch or stage under a branch would leave the compiler unable to count
  // the loads in flight, and it would wait for all of them at every stage.
  const int ntiles = (N + TILE - 1) / TILE;  // >= 1: callers have N > 0
  const int tlast = (ntiles - 1) * TILE;
  const int nsteps = (ntiles + DEPTH - 1) / DEPTH * DEPTH;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fetch(R[d], min(d * TILE, tlast));
  stage(R[0], 0, 0);
  fetch(R[0], min(DEPTH * TILE, tlast));
  __syncthreads();
  for (int it0 = 0; it0 < nsteps; it0 += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int it = it0 + u;
      contract(it & 1);
      Regs& nxt = R[(u + 1) % DEPTH];  // holds tile it + 1
      stage(nxt, (it + 1) & 1, (it + 1) * TILE);
      fetch(nxt, min((it + 1 + DEPTH) * TILE, tlast));
      __syncthreads();
    }
  }
}

// Block (rows row0 .. row0 + 31, cols of wave `wave`) of beta*G as bf16 hi/lo
// planes of a record (row-major, see gdn_gram_item), from the wave's
// accumulator of that block times gs.
__device__ __forceinline__ void store_rows_bg(uint16_t* Ghi, int row0, const floatx16& accG, float gs) {
  constexpr int D = GD;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, col = lane & 31;
  uint16_t* Glo = Ghi + D * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = row0 + 8 * (r >> 2) + 4 * g + (r & 3);
    uint16_t h, l;
    split_bf16(gs * accG[r], h, l);
    Ghi[m * D + wave * 32 + col] = h;
    Glo[m * D + wave * 32 + col] = l;
  }
}

template <int DI = GD, bool TG = false, bool PRO = false>
__device__ __forceinline__ void gdn_gram_rows_item(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ beta,
    uint8_t* __restrict__ rec, float c, float c2, int N, long item, uint8_t* lds_raw, TokLayout L,
    Prologue P) {
  constexpr int D = GD;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, col = lane & 31;
  const long bhf = item >> 2;
  const int w = (int)(item & 3);
  floatx16 accG[1], accU[1];
  gram_rows_accumulate<DI, TG, PRO, 32>(k, v, beta, N, bhf, w, lds_raw, L, P, accG, accU);

  // block (w, wave) of the record: beta*G hi/lo planes and beta*U (layout as in gdn_gram_item)
  const float bf = TG ? 1.0f : beta[bhf];
  const float gs = c2 * bf, us = c * bf;
  uint16_t* Ghi = reinterpret_cast<uint16_t*>(rec + (size_t)bhf * kRecBytes);
  float* Ud = reinterpret_cast<float*>(Ghi + 2 * D * D);
  store_rows_bg(Ghi, 32 * w, accG[0], gs);
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int m0 = w * 32 + 8 * q4 + 4 * g;
    float4 u4 = make_float4(us * accU[0][4 * q4], us * accU[0][4 * q4 + 1], us * accU[0][4 * q4 + 2],
                            us * accU[0][4 * q4 + 3]);
    *reinterpret_cast<float4*>(Ud + ((size_t)(m0 >> 2) * D + wave * 32 + col) * 4) = u4;
  }
}

// One workgroup per (batch*head, 16-row block of S); a head's eight row
// blocks get block ids that are equal mod 8, so they run on one XCD and
// share its L2 copy of each frame's record.  Per frame:
//   S_rows <- alpha (S_rows - S_rows (beta G)) + beta U
// The product runs as three bf16 MFMAs on hi/lo splits of S and beta G
// (dropping only lo*lo), accumulated in fp32; S stays fp32 in registers (C
// layout) and in a double-buffered LDS copy that feeds the next frame's A
// operands.  G is symmetric, so the B operand (8 consecutive k of column n)
// is read as 16 contiguous bytes of row n.
//
// The frame loop is a dependency chain, so it is kept free of branches and
// light on memory instructions: records are fetched two frames ahead into a
// register ring (always issued, with the frame index clamped at the end;
// fused into one launch with the gram items, a frame's record is loaded once
// its flag is up, straight from the XCD's L2),
// the decays of up to kAlphaWin frames sit in LDS, and each frame's state is
// written back with two 16-byte stores per thread from the LDS copy.  MULTI
// handles frames split into several token chunks (one record per chunk).
constexpr int kAlphaWin = 2048;
constexpr int kScanRB = 16, kScanPitch = GD + 4;
// LDS bytes of a scan item over RB rows
template <int RB>
constexpr int scan_lds_bytes() { return 2 * RB * kScanPitch * 4 + kAlphaWin * 4; }
constexpr int kScanLds = scan_lds_bytes<kScanRB>();

// Scan item of rows [r0, r0 + RB) of head `head`'s state over all F frames
// (RB = 16 or 32: one or two 16-row sub-blocks per wave).
// rchunk > 0: the reversed scan that resets at chunk boundaries.  Step f of
// the loop then works on frame phys(f): the frames of each chunk of rchunk
// frames (from frame 0) in decreasing order; the first step of a chunk uses
// a decay of 0, which drops the previous chunk's state (S <- beta U).
// FUSED: records come from gram items of the same launch (wait for gflags
// before each frame, one flag per token chunk) and each frame's state is
// announced on sflags[(head * F + f) * 8 + r0 / RB] for the output items.
template <bool MULTI, bool FUSED, int RB = kScanRB, int DI = GD>
__device__ __forceinline__ void gdn_scan_item(
    const uint8_t* __restrict__ rec, const float* __restrict__ alpha, const float* S0,
    uint16_t* __restrict__ states, float* S_out, long head, int r0, int F, int nc, uint8_t* lds_raw,
    const uint64_t* gflags, uint64_t* sflags, uint64_t epoch, uint32_t* err, int gpf = 0, int rchunk = 0) {
  // gram flags per frame: one per record chunk, or gpf when the frame's record
  // is written in gpf disjoint parts
  const int nfl = gpf > 0 ? gpf : nc;
  constexpr int D = GD, PITCH = kScanPitch;
  constexpr int SB = RB / 16;  // 16-row sub-blocks
  static_assert(RB == 16 || RB == 32, "scan items cover 16 or 32 rows");
  typedef float RowsT[RB][PITCH];
  RowsT* Ss = reinterpret_cast<RowsT*>(lds_raw);                         // [2][RB][PITCH]
  float* As = reinterpret_cast<float*>(lds_raw + 2 * RB * PITCH * 4);    // [kAlphaWin]
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;

  float s[SB][2][4];
#pragma unroll
  for (int sb = 0; sb < SB; ++sb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * sb + 4 * lg + r, n = 32 * wave + 16 * nb + lr;
        s[sb][nb][r] = S0 && r0 + m < DI && n < DI ? S0[(size_t)head * DI * DI + (size_t)(r0 + m) * DI + n] : 0.0f;
        Ss[0][m][n] = s[sb][nb][r];
      }

  struct Rec {
    u32x4 hi[2][4], lo[2][4];
    float u[SB][2][4];
  };
  const size_t hf0 = (size_t)head * F;
  auto phys = [&](int f) {
    if (rchunk <= 0) return f;
    const int c0 = f / rchunk * rchunk;
    return c0 + min(rchunk, F - c0) - 1 - (f - c0);
  };
  // load_rec and store_state take physical frames
  auto load_rec = [&](int f, int cidx, Rec& R) {
    const uint8_t* base = rec + ((hf0 + f) * nc + cidx) * kRecBytes;
    const uint16_t* gh = reinterpret_cast<const uint16_t*>(base);
    const uint16_t* gl = gh + D * D;
    const float* U = reinterpret_cast<const float*>(gl + D * D);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = 32 * wave + 16 * nb + lr;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const size_t off = (size_t)n * D + 32 * s4 + 8 * lg;
        R.hi[nb][s4] = ld16(gh + off);
        R.lo[nb][s4] = ld16(gl + off);
      }
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const float4 u4 =
            *reinterpret_cast<const float4*>(U + ((size_t)(((r0 + 16 * sb) >> 2) + lg) * D + n) * 4);
        R.u[sb][nb][0] = u4.x;
        R.u[sb][nb][1] = u4.y;
        R.u[sb][nb][2] = u4.z;
        R.u[sb][nb][3] = u4.w;
      }
    }
  };
  // S_f leaves for the output pass from the LDS copy the next frame reads
  // anyway: each thread splits 8 consecutive entries of a row and writes
  // them to the hi and lo planes with two 16-byte stores (per 16 rows)
  auto store_state = [&](int f, int buf) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      const int row = 16 * sb + (tid >> 4), c0 = 8 * (tid & 15);
      const float* src = &Ss[buf][row][c0];
      const float4 x0 = *reinterpret_cast<const float4*>(src);
      const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
      const uint2 p0 = split_bf16x2(x0.x, x0.y), p1 = split_bf16x2(x0.z, x0.w);
      const uint2 p2 = split_bf16x2(x1.x, x1.y), p3 = split_bf16x2(x1.z, x1.w);
      uint16_t* hp = states + (hf0 + f) * 2 * D * D + (size_t)(r0 + row) * D + c0;
      st16(hp, u32x4{p0.x, p1.x, p2.x, p3.x});
      st16(hp + D * D, u32x4{p0.y, p1.y, p2.y, p3.y});
    }
  };
  // hi*hi, hi*lo and lo*hi go to three accumulators: independent MFMA
  // chains overlap their latencies instead of queueing behind each other
  auto mfma3 = [&](floatx4 (&acc)[3], const u32x4& ah, const u32x4& al, const u32x4& bh_, const u32x4& bl_) {
    acc[0] = mfma16x16x32(as_bf16x8(ah), as_bf16x8(bh_), acc[0]);
    acc[1] = mfma16x16x32(as_bf16x8(ah), as_bf16x8(bl_), acc[1]);
    acc[2] = mfma16x16x32(as_bf16x8(al), as_bf16x8(bh_), acc[2]);
  };

  Rec R0, R1;
  if (!FUSED && F > 0) {
    load_rec(phys(0), 0, R0);
    load_rec(phys(min(1, F - 1)), 0, R1);
  }

  auto frame = [&](int f, Rec& R) {
    const int cur = f & 1;
    const int pf = phys(f);
    if (FUSED) {
      // this frame's records are published by gram items; the previous
      // frame's state (stored by every thread) is announced once all are done
      __builtin_amdgcn_s_waitcnt(0);
      wait_all(&gflags[(hf0 + pf) * nfl], nfl, epoch, err);
      if (f > 0 && tid == 0)
        __hip_atomic_store(&sflags[(hf0 + phys(f - 1)) * 8 + r0 / RB], epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      load_rec(pf, 0, R);
    }
    const float a = As[f % kAlphaWin];
    // A operands: this workgroup's rows of S_{f-1}, split into bf16 hi + lo
    u32x4 ahi[SB][4], alo[SB][4];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const float* src = &Ss[cur][16 * sb + lr][32 * s4 + 8 * lg];
        const float4 x0 = *reinterpret_cast<const float4*>(src);
        const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
        const uint2 p0 = split_bf16x2(x0.x, x0.y), p1 = split_bf16x2(x0.z, x0.w);
        const uint2 p2 = split_bf16x2(x1.x, x1.y), p3 = split_bf16x2(x1.z, x1.w);
        ahi[sb][s4] = u32x4{p0.x, p1.x, p2.x, p3.x};
        alo[sb][s4] = u32x4{p0.y, p1.y, p2.y, p3.y};
      }
    floatx4 acc3[SB][2][3];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int t = 0; t < 3; ++t) acc3[sb][nb][t] = floatx4{};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          mfma3(acc3[sb][nb], ahi[sb][s4], alo[sb][s4], R.hi[nb][s4], R.lo[nb][s4]);
    float uf[SB][2][4];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) uf[sb][nb][r] = R.u[sb][nb][r];
    if (MULTI) {
      for (int cidx = 1; cidx < nc; ++cidx) {  // the frame's further token chunks
        Rec T;
        load_rec(pf, cidx, T);
#pragma unroll
        for (int sb = 0; sb < SB; ++sb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
              mfma3(acc3[sb][nb], ahi[sb][s4], alo[sb][s4], T.hi[nb][s4], T.lo[nb][s4]);
#pragma unroll
            for (int r = 0; r < 4; ++r) uf[sb][nb][r] += T.u[sb][nb][r];
          }
      }
    }
    // refill this ring slot two frames ahead (the last record again at the end)
    if (!FUSED) load_rec(phys(min(f + 2, F - 1)), 0, R);
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * sb + 4 * lg + r, n = 32 * wave + 16 * nb + lr;
          const float prod = acc3[sb][nb][0][r] + (acc3[sb][nb][1][r] + acc3[sb][nb][2][r]);
          s[sb][nb][r] = a * (s[sb][nb][r] - prod) + uf[sb][nb][r];
          Ss[cur ^ 1][m][n] = s[sb][nb][r];
        }
    __syncthreads();
    store_state(pf, cur ^ 1);
  };

  for (int w0 = 0; w0 < F; w0 += kAlphaWin) {
    const int w1 = min(F, w0 + kAlphaWin);
    for (int i = tid; i < w1 - w0; i += 256)
      As[i] = rchunk > 0 && (w0 + i) % rchunk == 0 ? 0.0f : alpha[hf0 + phys(w0 + i)];
    __syncthreads();
    int f = w0;
    for (; f + 2 <= w1; f += 2) {
      frame(f, R0);
      frame(f + 1, R1);
    }
    if (f < w1) frame(f, R0);  // window tail (kAlphaWin is even, so slot f % 2 == 0)
    __syncthreads();  // As is rewritten for the next window
  }
  if (FUSED && F > 0) publish(&sflags[(hf0 + phys(F - 1)) * 8 + r0 / RB], epoch);
  if (S_out) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = r0 + 16 * sb + 4 * lg + r, cl = 32 * wave + 16 * nb + lr;
          if (row < DI && cl < DI) S_out[(size_t)head * DI * DI + (size_t)row * DI + cl] = s[sb][nb][r];
        }
  }
}

// The scan item of the single launches (fused and phased), rows r0 .. r0 + 31
// of head `head`'s state over all F frames, with the next frame's record
// requested while the current frame is computed.  beta G of a frame (hi and
// lo planes, 64 KB) comes straight from memory into LDS
// (global_load_lds_dwordx4, no registers), beta U's rows into a second set
// of registers; each wave checks whether the next frame's record flags are
// up once it has read the current frame's operands and, if so, requests its
// quarter of the next record right away, else at the next frame's start.  The
// frame's compute and state stores then overlap the record's latency, which
// otherwise sits on the chain once per frame.  Waves decide on their own (no
// barrier depends on the choice); every wave waits for its own loads and then
// for all waves before the operands are read.
//
// LDS: the state rows, fp32 [32][128] with float4 chunks XOR-swizzled by row
// (single buffered: read as A operands at a frame's start, rewritten at its
// end), and one frame's beta G, bf16 [hi, lo][128][128] with 16-byte chunks
// XOR-swizzled by row so that the 16 rows one quarter-wave reads fall on
// distinct banks.  80 KB in all: two items per CU.  The decays come from
// scalar loads one frame ahead.  nfl: gram flags per frame (1, or 4 when the
// record is written in four parts).  rchunk: as gdn_scan_item.
constexpr int kScanPfRows = 32;
constexpr int kScanPfLds = kScanPfRows * GD * 4 + 2 * GD * GD * 2;

template <int DI = GD>
__device__ __forceinline__ void gdn_scan_item_pf(
    const uint8_t* __restrict__ rec, const float* __restrict__ alpha, const float* S0,
    uint16_t* __restrict__ states, float* S_out, long head, int r0, int F, uint8_t* lds_raw,
    const uint64_t* gflags, uint64_t* sflags, uint64_t epoch, uint32_t* err, int nfl, int rchunk) {
  constexpr int D = GD, RB = kScanPfRows, SB = RB / 16;
  float* Ss = reinterpret_cast<float*>(lds_raw);
  uint8_t* Gl = lds_raw + RB * D * 4;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  // element (m, n) of the LDS state rows
  auto sidx = [](int m, int n) { return m * D + (((n >> 2) ^ (m & 15)) << 2) + (n & 3); };
  const size_t hf0 = (size_t)head * F;
  auto phys = [&](int f) {
    if (rchunk <= 0) return f;
    const int c0 = f / rchunk * rchunk;
    return c0 + min(rchunk, F - c0) - 1 - (f - c0);
  };
  // the decay of step f (a reversed chunk's first step starts from zero)
  auto decay = [&](int f) { return rchunk > 0 && f % rchunk == 0 ? 0.0f : alpha[hf0 + phys(f)]; };

  float s[SB][2][4];
#pragma unroll
  for (int sb = 0; sb < SB; ++sb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * sb + 4 * lg + r, n = 32 * wave + 16 * nb + lr;
        s[sb][nb][r] = S0 && r0 + m < DI && n < DI ? S0[(size_t)head * DI * DI + (size_t)(r0 + m) * DI + n] : 0.0f;
        Ss[sidx(m, n)] = s[sb][nb][r];
      }

  typedef float UT[SB][2][4];
  // this wave's quarter of frame pf's beta G into LDS (chunk P of the 4096
  // 16-byte chunks: plane P / 2048, row (P / 16) % 128, swizzled chunk P % 16)
  auto request_bg = [&](int pf) {
    const uint8_t* base = rec + (hf0 + pf) * kRecBytes;
    // rolled: the loads write LDS, not registers, so nothing waits on them here
#pragma unroll 1
    for (int j = 0; j < 16; ++j) {
      const int P = wave * 1024 + j * 64 + lane;
      const int plane = P >> 11, n = (P >> 4) & (D - 1), c = (P & 15) ^ (n & 15);
      __builtin_amdgcn_global_load_lds(base + (size_t)plane * D * D * 2 + (size_t)n * D * 2 + c * 16,
                                       (__attribute__((address_space(3))) void*)(Gl + (wave * 1024 + j * 64) * 16),
                                       16, 0, 0);
    }
  };
  auto request_u = [&](int pf, UT& u) {
    const float* U = reinterpret_cast<const float*>(rec + (hf0 + pf) * kRecBytes + (size_t)4 * D * D);
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int n = 32 * wave + 16 * nb + lr;
        const float4 u4 = *reinterpret_cast<const float4*>(U + ((size_t)(((r0 + 16 * sb) >> 2) + lg) * D + n) * 4);
        u[sb][nb][0] = u4.x;
        u[sb][nb][1] = u4.y;
        u[sb][nb][2] = u4.z;
        u[sb][nb][3] = u4.w;
      }
  };
  // the record flags of frame pf are all up (wave-uniform)
  auto ready = [&](int pf) {
    bool ok = true;
    if (lane < nfl) ok = __hip_atomic_load(&gflags[(hf0 + pf) * nfl + lane], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == epoch;
    return __ballot(!ok) == 0;
  };
  auto wave_wait = [&](int pf) {
    int spins = 0;
    while (!ready(pf)) {
      if (++spins > kSpinLimit) {
        if (lane == 0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  };
  auto store_state = [&](int pf) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      const int row = 16 * sb + (tid >> 4), c0 = 8 * (tid & 15);
      const float4 x0 = *reinterpret_cast<const float4*>(&Ss[sidx(row, c0)]);
      const float4 x1 = *reinterpret_cast<const float4*>(&Ss[sidx(row, c0 + 4)]);
      const uint2 p0 = split_bf16x2(x0.x, x0.y), p1 = split_bf16x2(x0.z, x0.w);
      const uint2 p2 = split_bf16x2(x1.x, x1.y), p3 = split_bf16x2(x1.z, x1.w);
      uint16_t* hp = states + (hf0 + pf) * 2 * D * D + (size_t)(r0 + row) * D + c0;
      st16(hp, u32x4{p0.x, p1.x, p2.x, p3.x});
      st16(hp + D * D, u32x4{p0.y, p1.y, p2.y, p3.y});
    }
  };

  UT U0, U1;
  bool asked = false;  // this wave has requested the next frame's record
  float a_next = 0.0f;
  if (F > 0) {
    wave_wait(phys(0));
    request_bg(phys(0));
    request_u(phys(0), U0);
    a_next = decay(0);
  }
  // step f: its record was requested into LDS and `u`; `un` takes the next one
  auto frame = [&](int f, UT& u, UT& un) {
    const int pf = phys(f);
    const float a = a_next;
    __builtin_amdgcn_s_waitcnt(0);  // this frame's record, and the previous frame's state stores
    if (f > 0 && tid == 0)
      __hip_atomic_store(&sflags[(hf0 + phys(f - 1)) * 8 + r0 / RB], epoch, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    // S_{f-1} (this item's rows) times beta G: per k-step s4, B operands beta
    // G(k, n) for k = 32 s4 + 8 lg .. + 7, n = 32 wave + 16 nb + lr (G is
    // symmetric: row n's chunk k / 8) and A operands, the rows of S_{f-1}
    // split into bf16 hi + lo, straight from LDS
    floatx4 acc[SB][2][2];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[sb][nb][0] = acc[sb][nb][1] = floatx4{};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      u32x4 bhi[2], blo[2], ahi[SB], alo[SB];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int n = 32 * wave + 16 * nb + lr, pc = (4 * s4 + lg) ^ (n & 15);
        bhi[nb] = *reinterpret_cast<const u32x4*>(Gl + (size_t)n * D * 2 + pc * 16);
        blo[nb] = *reinterpret_cast<const u32x4*>(Gl + (size_t)(D + n) * D * 2 + pc * 16);
      }
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const int m = 16 * sb + lr, n0 = 32 * s4 + 8 * lg;
        const float4 x0 = *reinterpret_cast<const float4*>(&Ss[sidx(m, n0)]);
        const float4 x1 = *reinterpret_cast<const float4*>(&Ss[sidx(m, n0 + 4)]);
        const uint2 p0 = split_bf16x2(x0.x, x0.y), p1 = split_bf16x2(x0.z, x0.w);
        const uint2 p2 = split_bf16x2(x1.x, x1.y), p3 = split_bf16x2(x1.z, x1.w);
        ahi[sb] = u32x4{p0.x, p1.x, p2.x, p3.x};
        alo[sb] = u32x4{p0.y, p1.y, p2.y, p3.y};
      }
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          acc[sb][nb][0] = mfma16x16x32(as_bf16x8(ahi[sb]), as_bf16x8(bhi[nb]), acc[sb][nb][0]);
          acc[sb][nb][1] = mfma16x16x32(as_bf16x8(ahi[sb]), as_bf16x8(blo[nb]), acc[sb][nb][1]);
          acc[sb][nb][1] = mfma16x16x32(as_bf16x8(alo[sb]), as_bf16x8(bhi[nb]), acc[sb][nb][1]);
        }
    }
    __syncthreads();  // every wave is done with beta G's buffer and the state rows
    if (f + 1 < F) {
      const int pn = phys(f + 1);
      asked = ready(pn);
      if (asked) {
        request_bg(pn);
        request_u(pn, un);
      }
      a_next = decay(f + 1);
    }
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * sb + 4 * lg + r, n = 32 * wave + 16 * nb + lr;
          s[sb][nb][r] = a * (s[sb][nb][r] - (acc[sb][nb][0][r] + acc[sb][nb][1][r])) + u[sb][nb][r];
          Ss[sidx(m, n)] = s[sb][nb][r];
        }
    __syncthreads();
    store_state(pf);
    if (f + 1 < F && !asked) {  // the next record was not ready: wait for it now
      const int pn = phys(f + 1);
      wave_wait(pn);
      request_bg(pn);
      request_u(pn, un);
    }
  };
  int f = 0;
  for (; f + 2 <= F; f += 2) {
    frame(f, U0, U1);
    frame(f + 1, U1, U0);
  }
  if (f < F) frame(f, U0, U1);
  if (F > 0) publish(&sflags[(hf0 + phys(F - 1)) * 8 + r0 / RB], epoch);
  if (S_out) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = r0 + 16 * sb + 4 * lg + r, cl = 32 * wave + 16 * nb + lr;
          if (row < DI && cl < DI) S_out[(size_t)head * DI * DI + (size_t)row * DI + cl] = s[sb][nb][r];
        }
  }
}

constexpr int kOutPitch = GD + 8;
// Q tiles (double buffered) and output staging tiles (double buffered), bf16
constexpr int kOutLds = 2 * 64 * kOutPitch * 2 + 2 * 64 * kOutPitch * 2;

// Work item `wg` = (frame of one head) * nco + token chunk: o = S_f q.
// With wflags, the state is announced by nw flags equal to epoch: the item
// issues its first query loads, then waits for them, then reads the state.
template <int DI = GD, bool PRO = false>
__device__ __forceinline__ void gdn_output_item(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const uint16_t* __restrict__ states,
    int N, int nco, int chunk, long wg, uint8_t* lds_raw, TokLayout L, Prologue P,
    const uint64_t* wflags = nullptr, int nw = 0, uint64_t epoch = 0, uint32_t* err = nullptr) {
  constexpr int D = GD;
  constexpr int CI = DI / 8;  // 16-byte chunks per token row in memory
  constexpr int TILE = 64;
  constexpr int ROW = D + 8;  // 272-byte pitch: 16-byte fragment reads spread over all banks
  constexpr int LPT = TILE * (D / 8) / 256;  // 4
  typedef uint16_t TileT[TILE * ROW];
  TileT* lds = reinterpret_cast<TileT*>(lds_raw);               // [buffer][TILE * ROW] query tiles
  TileT* ost = reinterpret_cast<TileT*>(lds_raw + 2 * TILE * ROW * 2);  // [buffer][TILE * ROW] outputs

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const long bhf = wg / nco;
  const int n0 = (int)(wg % nco) * chunk;
  const int n1 = min(N, n0 + chunk);

  // A operands: rows 32*wave + col of S_f, dims 16s + 8g .. +7, hi and lo planes
  const uint16_t* hi = states + (size_t)bhf * 2 * D * D;
  const uint16_t* lo = hi + D * D;
  u32x4 ahi[8], alo[8];
  auto load_state = [&]() {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const size_t off = (size_t)(wave * 32 + col) * D + s * 16 + g * 8;
      ahi[s] = ld16(hi + off);
      alo[s] = ld16(lo + off);
    }
  };
  if (!wflags) load_state();

  const uint16_t* qf = q + L.base(bhf);
  uint16_t* of = o + L.base(bhf);
  // query tiles come in through two register sets (tile t in set t % 2
  // until staged), so two tiles are in flight while one is contracted
  struct Regs {
    u32x4 q[LPT];
  };
  auto fetch = [&](Regs& X, int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const int n = t0 + tok;
      // rows past the chunk re-read its first token: their outputs are never stored
      // (dims past DI re-read a real chunk: S_f is zero in those columns)
      X.q[r] = ld16(qf + (size_t)(n < n1 ? n : n0) * L.sn + (cb < CI ? cb : CI - 1) * 8);
    }
  };
  float wq8[8];  // the prologue's query weights of this thread's channels (chunk tid % 16)
  if (PRO) load_weights8(P.wq, (bhf / L.F) % L.H, DI, (tid & 15) * 8, wq8);
  auto row16 = [](double x) { return group_sum_f64<16>(x); };
  // t0: the first token of the staged tile (its rows past the chunk hold token n0)
  auto stage = [&](const Regs& X, int buf, int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      // with the prologue, chunks past DI (which re-read a real chunk) are
      // zeroed out of the token's sums
      const u32x4 qq = PRO && P.on_q() && cb >= CI ? u32x4{0u, 0u, 0u, 0u} : X.q[r];
      *reinterpret_cast<u32x4*>(&lds[buf][tok * ROW + cb * 8]) = qq;
    }
    if (PRO && P.on_q()) {  // in place on the staged chunks, one at a time (as in gdn_gram_item)
#pragma unroll 1
      for (int r = 0; r < LPT; ++r) {
        const int ci = r * 256 + tid;
        const int tok = ci >> 4, cb = ci & 15;
        u32x4* qd = reinterpret_cast<u32x4*>(&lds[buf][tok * ROW + cb * 8]);
        const Rot8 rot = P.rope() ? rot8_load(P.rope8(bhf % L.F, t0 + tok < n1 ? t0 + tok : n0, cb < CI ? cb : 0, DI))
                                  : Rot8{};
        *qd = prologue_bf16x8(*qd, wq8, P.wq != nullptr, P, false, 1.0 / DI, row16, P.rope(), rot);
      }
    }
  };

  // Full tiles run in pairs without any branch in the loop body (a load or
  // store under a condition would make the compiler wait for every memory
  // operation in flight); fetches past the end re-read the last tile, and a
  // last, partial tile stores under a token check after the loop.
  if (n0 >= n1) return;
  const int ntiles = (n1 - n0 + TILE - 1) / TILE;
  const int nfull = (n1 - n0) / TILE;
  const int tlast = n0 + (ntiles - 1) * TILE;
  Regs R0, R1;
  fetch(R0, n0);
  fetch(R1, min(n0 + TILE, tlast));
  if (wflags) {  // the state's producers run in this launch: query loads are in flight meanwhile
    wait_all(wflags, nw, epoch, err);
    load_state();
  }
  stage(R0, 0, n0);
  fetch(R0, min(n0 + 2 * TILE, tlast));
  __syncthreads();
  // a tile's outputs leave as whole 256-byte rows (16 lanes per token, 16
  // bytes each) from its staging buffer
  auto drain = [&](int it, const bool full) {
    const int t0 = n0 + it * TILE;
#pragma unroll
    for (int r = 0; r < TILE * (D / 8) / 256; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const u32x4 w = *reinterpret_cast<const u32x4*>(&ost[it & 1][tok * ROW + cb * 8]);
      if ((full || t0 + tok < n1) && cb < CI) st16_stream(of + (size_t)(t0 + tok) * L.sn + cb * 8, w);
    }
  };
  // tile `it` is in LDS buffer it % 2; nxt holds tile it + 1 and is refilled with tile it + 3
  auto tile = [&](int it, Regs& nxt, const bool full) {
    const int buf = it & 1;
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
      // lane (col, g) of wave w holds token half*32 + col, dims 32 w + 8 q4 + 4 g + 0..3
      uint16_t* srow = &ost[buf][(half * 32 + col) * ROW + wave * 32 + 4 * g];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint2 w;
        w.x = pack_bf16x2(acc[4 * q4 + 0], acc[4 * q4 + 1]);
        w.y = pack_bf16x2(acc[4 * q4 + 2], acc[4 * q4 + 3]);
        *reinterpret_cast<uint2*>(srow + 8 * q4) = w;
      }
    }
    stage(nxt, buf ^ 1, min(n0 + (it + 1) * TILE, tlast));  // the next tile (past the end: a copy of the last, never read)
    fetch(nxt, min(n0 + (it + 3) * TILE, tlast));
    __syncthreads();
    drain(it, full);
  };
  int it = 0;
  for (; it + 2 <= nfull; it += 2) {
    tile(it, R1, true);
    tile(it + 1, R0, true);
  }
  // R1 holds tile it + 1: at most one more full tile, then at most one partial one
  if (it < nfull) {
    tile(it, R1, true);
    if (it + 1 < ntiles) tile(it + 1, R0, false);
  } else if (it < ntiles) {
    tile(it, R1, false);
  }
}


// Single-frame calls: kStepItems = 2 work items (head, w) per head whose only
// frame is the call's.  Item w forms rows 64w .. 64w + 63 of the head's new
// state and the outputs of token chunk w of kStepChunks:
//  1. G and U rows 64w .. over all tokens (gram_rows_accumulate, two 32-row
//     blocks per wave);
//  2. beta G rows 64w .. to the head's record as hi/lo planes; flag
//     gflags[4 head + w]; S0's rows 64w .. start loading into LDS;
//  3. once the head's flags are up, S1 rows 64w .. =
//     alpha (S0 rows - S0 rows . beta G) + beta U rows: wave j forms columns
//     32j .. 32j + 31 from beta G's rows 32j .. (G is symmetric, so they are
//     its columns) and its own accumulators U(rows, j);
//  4. S1 rows 64w .. to S_out (fp32) and to the head's state as hi/lo planes,
//     whole 16-byte stores through LDS; flag sflags[8 head + w];
//  5. the output item of token chunk w, which issues its first query loads
//     before waiting for the head's state flags.
// The launch adds output-only items for the remaining chunks (gdn_output_item
// waiting for the state flags), which prefetch their query tiles meanwhile.
// No separate scan items, and U never leaves registers.  Two items per head
// read K twice (the second time mostly from L2) and read V in whole 128-byte
// lines.  The items of a head wait for each other; their block ids lie
// within 16 of each other, so only items of the (at most 8) heads at the
// dispatch frontier can wait for a partner not yet dispatched, and every
// other waiting item's partner is running.  S_out may equal S0: each item
// reads only its own rows of S0, before writing them.
constexpr int kStepItems = 2, kStepRows = GD / kStepItems, kStepChunks = 4;
constexpr int kStepPitch = GD + 4;  // fp32 LDS rows of S0 / S1
constexpr int kStepLds = gram_rows_lds<kStepRows>() + kGateLds + kPrologueLds;
static_assert(kStepRows * kStepPitch * 4 <= gram_rows_lds<kStepRows>(), "state rows fit in the tile LDS");

template <int DI, bool TG, bool PRO>
__device__ __forceinline__ void gdn_step_item(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, uint16_t* __restrict__ o,
    uint8_t* __restrict__ rec, uint16_t* __restrict__ states, const float* S0, float* S_out, float c, float c2,
    int N, int chunko, long head, int w, uint64_t* gflags, uint64_t* sflags, uint64_t epoch, uint32_t* err,
    int rchunk, uint8_t* lds_raw, TokLayout L, Prologue P) {
  constexpr int D = GD, RB = kStepRows, NB = RB / 32, NW = kStepItems, PITCH = kStepPitch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  floatx16 accG[NB], accU[NB];
  gram_rows_accumulate<DI, TG, PRO, RB>(k, v, beta, N, head, w, lds_raw, L, P, accG, accU);
  const float bf = TG ? 1.0f : beta[head];
  const uint16_t* Ghi = reinterpret_cast<const uint16_t*>(rec + (size_t)head * kRecBytes);
#pragma unroll
  for (int b = 0; b < NB; ++b) store_rows_bg(const_cast<uint16_t*>(Ghi), RB * w + 32 * b, accG[b], c2 * bf);
  publish(&gflags[head * 4 + w], epoch);  // also: every wave is past the tile loop, LDS is free

  // S rows RB w .. as fp32 in LDS, [RB][PITCH], zero past DI
  float(*Sl)[PITCH] = reinterpret_cast<float(*)[PITCH]>(lds_raw);
  const bool with_s0 = S0 && rchunk <= 0;  // a reversed chunk starts from zero
  const float a = with_s0 ? alpha[head] : 0.0f;
  const float us = c * bf;
  floatx16 s1[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) s1[b][r] = us * accU[b][r];
  if (with_s0) {
    // 16-byte chunks: row i / 32, float4 i % 32 (dims 4 (i % 32) ..), loaded
    // before the wait so that they arrive meanwhile
    const float* S0h = S0 + (size_t)head * DI * DI;
    constexpr int CPT = RB * (D / 4) / 256;  // chunks per thread (8)
    float4 x[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int i = j * 256 + tid, row = RB * w + i / 32, d0 = 4 * (i % 32);
      x[j] = *reinterpret_cast<const float4*>(S0h + (size_t)(row < DI ? row : 0) * DI + (d0 < DI ? d0 : 0));
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int i = j * 256 + tid, row = RB * w + i / 32, d0 = 4 * (i % 32);
      *reinterpret_cast<float4*>(&Sl[i / 32][d0]) =
          row < DI && d0 < DI ? x[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    wait_all(&gflags[head * 4], NW, epoch, err);  // (its barrier also orders the LDS writes)
    // B operand: beta G(k, 32 wave + (lane & 31)) for k = 16 s + 8 g .. + 7,
    // i.e. row 32 wave + (lane & 31) of the symmetric beta G
    const uint16_t* Glo = Ghi + D * D;
    u32x4 bh[8], bl[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const size_t off = (size_t)(32 * wave + col) * D + 16 * s + 8 * g;
      bh[s] = ld16(Ghi + off);
      bl[s] = ld16(Glo + off);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // A operand: S0 row RB w + 32 b + (lane & 31), dims 16 s + 8 g .. + 7, as hi + lo
      floatx16 acc[2] = {floatx16{}, floatx16{}};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float* src = &Sl[32 * b + col][16 * s + 8 * g];
        const float4 x0 = *reinterpret_cast<const float4*>(src);
        const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
        const uint2 p0 = split_bf16x2(x0.x, x0.y), p1 = split_bf16x2(x0.z, x0.w);
        const uint2 p2 = split_bf16x2(x1.x, x1.y), p3 = split_bf16x2(x1.z, x1.w);
        const u32x4 ahi = u32x4{p0.x, p1.x, p2.x, p3.x}, alo = u32x4{p0.y, p1.y, p2.y, p3.y};
        acc[0] = mfma32x32x16(as_bf16x8(ahi), as_bf16x8(bh[s]), acc[0]);
        acc[1] = mfma32x32x16(as_bf16x8(ahi), as_bf16x8(bl[s]), acc[1]);
        acc[1] = mfma32x32x16(as_bf16x8(alo), as_bf16x8(bh[s]), acc[1]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float s0 = Sl[32 * b + 8 * (r >> 2) + 4 * g + (r & 3)][32 * wave + col];
        s1[b][r] = a * (s0 - (acc[0][r] + acc[1][r])) + s1[b][r];
      }
    }
    __syncthreads();  // every wave has read S0's rows: S1 may replace them
  }
  // S1 rows through LDS, then whole 16-byte stores: the hi/lo planes of the
  // state (8 entries per thread and row) and S_out (4 entries, rows and dims below DI)
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) Sl[32 * b + 8 * (r >> 2) + 4 * g + (r & 3)][32 * wave + col] = s1[b][r];
  __syncthreads();
  uint16_t* Shi = states + (size_t)head * 2 * D * D;
#pragma unroll
  for (int j = 0; j < RB * (D / 8) / 256; ++j) {
    const int i = j * 256 + tid, row = i / 16, c0 = 8 * (i % 16);
    const float4 x0 = *reinterpret_cast<const float4*>(&Sl[row][c0]);
    const float4 x1 = *reinterpret_cast<const float4*>(&Sl[row][c0 + 4]);
    const uint2 p0 = split_bf16x2(x0.x, x0.y), p1 = split_bf16x2(x0.z, x0.w);
    const uint2 p2 = split_bf16x2(x1.x, x1.y), p3 = split_bf16x2(x1.z, x1.w);
    uint16_t* hp = Shi + (size_t)(RB * w + row) * D + c0;
    st16(hp, u32x4{p0.x, p1.x, p2.x, p3.x});
    st16(hp + D * D, u32x4{p0.y, p1.y, p2.y, p3.y});
  }
  if (S_out) {
    float* So = S_out + (size_t)head * DI * DI;
#pragma unroll
    for (int j = 0; j < RB * (D / 4) / 256; ++j) {
      const int i = j * 256 + tid, row = RB * w + i / 32, d0 = 4 * (i % 32);
      if (row < DI && d0 < DI)
        *reinterpret_cast<float4*>(So + (size_t)row * DI + d0) = *reinterpret_cast<const float4*>(&Sl[i / 32][d0]);
    }
  }
  publish(&sflags[head * 8 + w], epoch);  // its barrier: the output item may reuse the LDS
  gdn_output_item<DI, PRO>(q, o, states, N, kStepChunks, chunko, head * kStepChunks + w, lds_raw, L, P,
                           &sflags[head * 8], NW, epoch, err);
}

}  // namespace linscan
