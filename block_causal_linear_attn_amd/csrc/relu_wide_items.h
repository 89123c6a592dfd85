// relu_wide_items.h -- bf16 MFMA work items of the ReLU block-causal
// linear-attention scan for wide heads (head dims 112 and 128; SANA-Video's
// linear attention: ReLU feature map, cumulative D x D state plus normaliser).
//
// At these widths a D x D partial per wave (the layout of the narrow items)
// no longer fits in registers, so the work is split by rows of the state:
// tensors are taken as 128 dims wide, the dims past the head dim being zero
// (they add nothing to any sum), and wave w owns rows [32w, 32w + 32).
//
// Summary items, np per (head, frame) (np = 1 when there are enough frames
// and heads to fill the chip): dS = V^T phi(K) over one run of the frame's
// tokens.  The workgroup stages 64-token K and V tiles in LDS (ring of
// register sets in flight, rows unpadded with their 16-byte chunks swizzled
// by token; phi applied to K when staged) and each lane gathers 8 tokens of
// one dimension per MFMA operand with two LDS transpose reads.  dz = 1^T phi(K)
// comes from a padding row (head dim 112: value dim 112 is set to 1, so row
// 112 of dS is dz) or, at head dim 128, from one more MFMA with an all-ones
// A operand.  Every part writes its sums as a record.
//
// Prefix items, four per head (32 rows of the state each), add the parts of
// each frame to a running sum held in registers and write the cumulative
// state of every frame, so no later reader has to sum partials and a frame's
// hand-off moves 16 KB per item instead of reloading the previous 66 KB
// state.  (A decoupled look-back over earlier frames' own sums was measured
// slower: every item then reads several 66 KB records from L2 at once.)
//
// Output item, one per (head, frame, token chunk): reads the one cumulative
// state its frame sees (the last frame of its block), splits S into bf16 hi +
// lo terms (16 significant bits) held as MFMA A operands, and contracts
// 64-token query tiles staged in LDS.  The denominator z . phi(q) is formed
// when a tile is staged: each thread holds 8 dims of a token, and 16 lanes
// finish the sum with DPP row reductions.
#pragma once

#include "device_common.h"
#include "sync.h"

namespace linscan {

constexpr int kReluWide = 128;                                   // padded head dim
constexpr int kReluWideRec = kReluWide * kReluWide + kReluWide;  // floats per cumulative record
constexpr int kReluWideDepth = 2;                                // tiles in flight per summary item
constexpr int kReluWideSumLds = 2 * 2 * 64 * kReluWide * 2;      // K, V tiles, double buffered (+ weights)
constexpr int kReluWideOutPitch = kReluWide + 8;
// query tiles and output staging tiles (double buffered, bf16) + per-token denominators
constexpr int kReluWideOutLds = 4 * 64 * kReluWideOutPitch * 2 + 2 * 64 * 4;

// Summary item `part` (of np) of frame f of head bh.  The frame's tiles of 64
// tokens are split into np runs of consecutive tiles, one per part; the part
// writes the sums over its run (dS and dz) to parts[(bh * F + f) * np + part]
// (a record in accumulator order) and publishes the flag of the same index
// in pflags.  The prefix items add them up frame by frame.
template <int DI>
__device__ __forceinline__ void relu_wide_summary_item(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int F, int N, long bh, int f, int np,
    int part, float* __restrict__ parts, uint64_t* __restrict__ pflags, uint64_t epoch, uint8_t* lds_raw,
    TokLayout L, Prologue P) {
  constexpr int D = kReluWide;
  constexpr int CI = DI / 8;  // 16-byte chunks per token row in memory
  constexpr int TILE = 64;
  constexpr int C = D / 8;                   // chunks per (padded) LDS row
  constexpr int LPT = TILE * (D / 8) / 256;  // 16-byte loads per thread per tensor per tile (4)
  typedef uint16_t TileT[2][TILE * D];
  TileT* lds = reinterpret_cast<TileT*>(lds_raw);  // [buffer][K, V][TILE * D]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const long bhf = bh * F + f;
  const uint16_t* kf = k + L.base(bhf);
  const uint16_t* vf = v + L.base(bhf);
  // the prologue's key weights of the head (RMSNorm), in LDS after the tiles
  float* wl = reinterpret_cast<float*>(lds_raw + kReluWideSumLds);
  if (P.wk) {
    if (tid < D) wl[tid] = tid < DI ? P.wk[(size_t)(bh % L.H) * DI + tid] : 0.0f;
    __syncthreads();
  }

  // z: with DI < 128, value dim DI (zero padding) is set to 1 for every live
  // token, so row DI of dS is dz at no cost; at DI = 128 an MFMA with an
  // all-ones A operand forms it (register 0 of accz holds z[32 wave + col])
  constexpr bool ZROW = DI < D;
  // With the rotary embedding the staged keys are rotated, so neither way
  // gives dz: each thread sums the unrotated features of its channel chunk
  // (tid % 16) instead (ZV), and the padding row stays zero.
  const bool ZV = P.rope();
  float zk[8] = {};
  floatx16 acc[4], accz = {};
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = floatx16{};
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

  // this part's tokens [nb, ne): a run of tpp whole tiles (the last part's may be shorter or empty)
  const int tpp = ((N + TILE - 1) / TILE + np - 1) / np;
  const int nb = min(N, part * tpp * TILE), ne = min(N, nb + tpp * TILE);

  // Tile t sits in register set t % DEPTH from its fetch until it is staged.
  // The loop runs a whole number of ring passes with no branch: tiles past
  // the run are staged as zeros and add nothing, fetches past the run
  // re-read its last tile, and dims past DI re-read a real chunk and are
  // zeroed when staged.  (A load or stage under a condition would make the
  // compiler wait for every load in flight at each stage.)
  constexpr int DEPTH = kReluWideDepth;
  struct Regs {
    u32x4 k[LPT], v[LPT];
  };
  Regs R[DEPTH];
  auto fetch = [&](Regs& X, int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const int n = t0 + tok;
      const size_t off = (size_t)(n < ne ? n : nb) * L.sn + (cb < CI ? cb : CI - 1) * 8;
      X.k[r] = ld16_stream(kf + off);
      X.v[r] = ld16_stream(vf + off);
    }
  };
  auto stage = [&](const Regs& X, int buf, int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const bool live = t0 + tok < ne && cb < CI;
      u32x4 kk = live ? X.k[r] : u32x4{0u, 0u, 0u, 0u};
      float wk8[8] = {};
      if (P.wk) {  // the 16 lanes of a DPP row hold the 16 chunks of token `tok`
        const float4 a = *reinterpret_cast<const float4*>(wl + 8 * cb), b = *reinterpret_cast<const float4*>(wl + 8 * cb + 4);
        wk8[0] = a.x, wk8[1] = a.y, wk8[2] = a.z, wk8[3] = a.w, wk8[4] = b.x, wk8[5] = b.y, wk8[6] = b.z, wk8[7] = b.w;
      }
      if (ZV) {  // RMSNorm, the feature map, the unrotated sum, then the rotation
        Prologue Pf = P;
        Pf.relu = 1;
        float pre[8];
        kk = prologue_bf16x8(kk, wk8, P.wk != nullptr, Pf, true, 1.0 / DI,
                             [](double x) { return group_sum_f64<16>(x); },
                             true, rot8_load(P.rope8(f, t0 + tok < ne ? t0 + tok : nb, cb < CI ? cb : 0, DI)), pre);
#pragma unroll
        for (int e = 0; e < 8; ++e) zk[e] += pre[e];
      } else {
        if (P.wk) kk = prologue_bf16x8(kk, wk8, true, P, true, 1.0 / DI, [](double x) { return group_sum_f64<16>(x); });
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[e] = relu_bf16x2(kk[e]);
      }
      u32x4 vv = live ? X.v[r] : u32x4{0u, 0u, 0u, 0u};
      if (ZROW && !ZV) vv[0] = t0 + tok < ne && cb == CI ? 0x3f80u : vv[0];  // v[token][DI] = 1
      uint2* kd = reinterpret_cast<uint2*>(&lds[buf][0][swz_offset<C>(tok, cb)]);
      uint2* vd = reinterpret_cast<uint2*>(&lds[buf][1][swz_offset<C>(tok, cb)]);
      kd[0] = make_uint2(kk[0], kk[1]);
      kd[1] = make_uint2(kk[2], kk[3]);
      vd[0] = make_uint2(vv[0], vv[1]);
      vd[1] = make_uint2(vv[2], vv[3]);
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
#pragma unroll
      for (int J = 0; J < 4; ++J) acc[J] = mfma32x32x16(as_bf16x8(vfrag), as_bf16x8(kfrag[J]), acc[J]);
      if (!ZROW && !ZV) accz = mfma32x32x16(as_bf16x8(ones), as_bf16x8(kfrag[wave]), accz);
    }
  };

  const int ntiles = (ne - nb + TILE - 1) / TILE;
  if (ntiles > 0) {
    const int tlast = nb + (ntiles - 1) * TILE;
    const int nsteps = (ntiles + DEPTH - 1) / DEPTH * DEPTH;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) fetch(R[d], min(nb + d * TILE, tlast));
    stage(R[0], 0, nb);
    fetch(R[0], min(nb + DEPTH * TILE, tlast));
    __syncthreads();
    for (int it0 = 0; it0 < nsteps; it0 += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int it = it0 + u;
        contract(it & 1);
        Regs& nxt = R[(u + 1) % DEPTH];  // holds tile it + 1
        stage(nxt, (it + 1) & 1, nb + (it + 1) * TILE);
        fetch(nxt, min(nb + (it + 1 + DEPTH) * TILE, tlast));
        __syncthreads();
      }
    }
  }

  // ZV: the frame's dz[c] in LDS (the tiles are no longer read): lanes
  // l, l + 16, l + 32, l + 48 of a wave hold chunk l % 16, then the four
  // waves' sums are added in a fixed order
  float* zred = reinterpret_cast<float*>(lds_raw);  // [4][128]
  float dz = 0.0f;                                 // thread tid < 128: dz[tid]
  if (ZV) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      zk[e] += __shfl_xor(zk[e], 16);
      zk[e] += __shfl_xor(zk[e], 32);
    }
    if (ntiles > 0 && lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) zred[wave * D + lane * 8 + e] = zk[e];
    }
    __syncthreads();
    if (ntiles > 0 && tid < D) dz = ((zred[tid] + zred[D + tid]) + zred[2 * D + tid]) + zred[3 * D + tid];
  }

  // A part record holds acc[J][4 i .. 4 i + 3] of thread t as the float4 at
  // (4 J + i) * 256 + t, then the item's own z entries (accz register 0 at
  // 32 wave + col, or dz at tid; with ZROW, z is row DI of the S part) from
  // float D * D on.
  float* rec = parts + ((size_t)bhf * np + part) * kReluWideRec;
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      reinterpret_cast<float4*>(rec)[(4 * J + i) * 256 + tid] =
          make_float4(acc[J][4 * i], acc[J][4 * i + 1], acc[J][4 * i + 2], acc[J][4 * i + 3]);
  if (!ZROW && !ZV && g == 0) rec[D * D + wave * 32 + col] = accz[0];
  if (ZV && tid < D) rec[D * D + tid] = ntiles > 0 ? dz : 0.0f;
  publish(&pflags[(size_t)bhf * np + part], epoch);
}

// Prefix item (head bh, row block w): rows 32w .. 32w + 31 of the head's
// cumulative state at the end of each block of bfr frames.  The running sum
// starts from the initial state (S0, z0; zero where NULL) and stays in
// registers.  Frames go in groups of up to kPrefixRecs part records: one
// wait for the group's records (one flag per thread), all their loads in
// flight, then the adds frame by frame in the order p = 0, 1, ...; a block's
// last frame f writes the rows to cum[bh][f] (row-major S, then z at float
// D * D), and the group's block ends get their flags
// flags[(bh * F + f) * 4 + w] once its records are complete (with release:
// all flags at the end, after one agent-scope release, for output items on
// other XCDs).  Records of other frames are never written.  Ten 1-frame
// blocks with a wait, a record pair's load and a store each kept the output
// items waiting about 20 us after the last summary.  The last frame's rows
// also go to (S_out, z_out), which may alias (S0, z0): every element is
// written by the thread that read it.  Thread T = 64 j + l holds, of each part record, the float4s
// (4 j + i) * 256 + 64 w + l, i = 0..3: S[32 w + 8 i + 4 (l / 32) + e][32 j +
// l % 32], e = 0..3 (the accumulator layout of the summary items' wave w),
// and thread T < 32 the normaliser entry z[32 w + T] where it has its own
// slot (head dim 128 or the rotary embedding; with the padding row, z is
// row DI of S and its copy is written from there).  Four items per head
// shorten each block's hand-off to 16 KB per item, and the records of a
// head's frames are consecutive, so a block is one run of records.
constexpr int kPrefixRecs = 8;  // part records in flight per prefix item
template <int DI>
__device__ __forceinline__ void relu_wide_prefix_item(
    float* __restrict__ cum, const float* S0, const float* z0, float* S_out, float* z_out, int F, int bfr, long bh,
    int w, int np, const float* __restrict__ parts, const uint64_t* __restrict__ pflags, uint64_t* __restrict__ flags,
    uint64_t epoch, uint32_t* err, bool zv, bool release) {
  constexpr int D = kReluWide;
  constexpr bool ZROW = DI < D;
  const int T = threadIdx.x, j = T >> 6, l = T & 63;
  const int g = l >> 5, col = l & 31, n = 32 * j + col;
  const bool zslot = !ZROW || zv;  // z has its own entries (else it is row DI)
  auto row = [&](int i, int e) { return 32 * w + 8 * i + 4 * g + e; };
  float acc[4][4];
  float z = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = row(i, e);
      float x = 0.0f;
      if (S0 && m < DI && n < DI) x = S0[(size_t)bh * DI * DI + (size_t)m * DI + n];
      if (!zslot && z0 && m == DI && n < DI) x = z0[(size_t)bh * DI + n];
      acc[i][e] = x;
    }
  if (zslot && T < 32 && z0 && 32 * w + T < DI) z = z0[(size_t)bh * DI + 32 * w + T];
  auto add = [&](const float4 (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][0] += x[i].x, acc[i][1] += x[i].y, acc[i][2] += x[i].z, acc[i][3] += x[i].w;
  };
  auto load = [&](const float* rec, float4 (&x)[4], float& zx) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = reinterpret_cast<const float4*>(rec)[(4 * j + i) * 256 + 64 * w + l];
    zx = zslot && T < 32 ? rec[D * D + 32 * w + T] : 0.0f;
  };
  // the rows of frame f's cumulative state to cum[bh][f] (and the last frame's
  // to S_out, z_out)
  auto write_frame = [&](int f) {
    float* cur = cum + (size_t)(bh * F + f) * kReluWideRec;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cur[(size_t)row(i, e) * D + n] = acc[i][e];
        if (!zslot && row(i, e) == DI) cur[D * D + n] = acc[i][e];
      }
    if (zslot && T < 32) cur[D * D + 32 * w + T] = z;
    if (f == F - 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = row(i, e);
          if (S_out && m < DI && n < DI) S_out[(size_t)bh * DI * DI + (size_t)m * DI + n] = acc[i][e];
          if (!zslot && z_out && m == DI && n < DI) z_out[(size_t)bh * DI + n] = acc[i][e];
        }
      if (zslot && T < 32 && z_out && 32 * w + T < DI) z_out[(size_t)bh * DI + 32 * w + T] = z;
    }
  };
  auto block_end = [&](int f) { return (f + 1) % bfr == 0 || f == F - 1; };
  // frames in groups of kPrefixRecs / np: one wait for the group's part
  // records, all their loads in flight at once (past the group: re-reads of
  // its last record, not added), then the adds in frame and part order
  const int gf = np < kPrefixRecs ? kPrefixRecs / np : 1;
  for (int fa = 0; fa < F; fa += gf) {
    const int fb = min(F, fa + gf);
    const long r0 = (bh * F + fa) * np, r1 = (bh * F + fb) * np;
    wait_all(&pflags[r0], (int)(r1 - r0), epoch, err);
    float4 x[kPrefixRecs][4];
    float zx[kPrefixRecs];
#pragma unroll
    for (int u = 0; u < kPrefixRecs; ++u)
      load(parts + (size_t)(r0 + u < r1 ? r0 + u : r1 - 1) * kReluWideRec, x[u], zx[u]);
#pragma unroll
    for (int u = 0; u < kPrefixRecs; ++u) {
      if (r0 + u < r1) {
        add(x[u]), z += zx[u];
        if ((u + 1) % np == 0 && block_end(fa + (u + 1) / np - 1)) write_frame(fa + (u + 1) / np - 1);
      }
    }
    if (!release) {  // the group's records are complete: the flags of its block ends
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0)
        for (int f = fa; f < fb; ++f)
          if (block_end(f))
            __hip_atomic_store(&flags[(size_t)(bh * F + f) * 4 + w], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (release) {  // one write-back of the L2 for all records, then every block's flag
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      for (int f0 = 0; f0 < F; f0 += bfr)
        __hip_atomic_store(&flags[(size_t)(bh * F + min(F, f0 + bfr) - 1) * 4 + w], epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Output item `wg` = (frame of one head) * nco + token chunk:
// o = S phi(q) / (z . phi(q) + eps) with (S, z) = cum[bh][fend - 1], fend the
// end of the frame's block of bfr frames.  The record is ready once the four
// flags at wflags equal epoch (NULL: the caller has waited for it).
template <int DI>
__device__ __forceinline__ void relu_wide_output_item(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const float* __restrict__ cum, float eps,
    int F, int N, int bfr, int nco, int chunk, long wg, uint8_t* lds_raw, TokLayout L, Prologue P,
    const uint64_t* wflags, uint64_t epoch, uint32_t* err, bool acquire) {
  constexpr int D = kReluWide;
  constexpr int CI = DI / 8;  // 16-byte chunks per token row in memory
  constexpr int TILE = 64;
  constexpr int ROW = kReluWideOutPitch;     // 272-byte pitch: 16-byte fragment reads spread over all banks
  constexpr int LPT = TILE * (D / 8) / 256;  // 4
  typedef uint16_t TileT[TILE * ROW];
  TileT* lds = reinterpret_cast<TileT*>(lds_raw);                       // [buffer] phi(q) tiles
  TileT* ost = reinterpret_cast<TileT*>(lds_raw + 2 * TILE * ROW * 2);  // [buffer] output tiles
  float(*den)[TILE] = reinterpret_cast<float(*)[TILE]>(lds_raw + 4 * TILE * ROW * 2);  // [buffer][token]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, col = lane & 31;
  const long bhf = wg / nco;
  const long bh = bhf / F;
  const int f = (int)(bhf % F);
  const int fend = min(F, (f / bfr + 1) * bfr);
  const int n0 = (int)(wg % nco) * chunk;
  const int n1 = min(N, n0 + chunk);
  if (n0 >= n1) return;

  const uint16_t* qf = q + L.base(bhf);
  uint16_t* of = o + L.base(bhf);
  struct Regs {
    u32x4 q[LPT];
  };
  auto fetch = [&](Regs& X, int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const int n = t0 + tok;
      // rows past the chunk re-read its first token: their outputs are never
      // stored; dims past DI re-read a real chunk and are zeroed when staged
      X.q[r] = ld16_stream(qf + (size_t)(n < n1 ? n : n0) * L.sn + (cb < CI ? cb : CI - 1) * 8);
    }
  };
  // the first three query tiles are in flight while the item waits for the
  // cumulative record of its block (tile t in register set t % 3 until staged)
  const int ntiles = (n1 - n0 + TILE - 1) / TILE;
  const int nfull = (n1 - n0) / TILE;
  const int tlast = n0 + (ntiles - 1) * TILE;
  Regs R0, R1, R2;
  fetch(R0, n0);
  fetch(R1, min(n0 + TILE, tlast));
  fetch(R2, min(n0 + 2 * TILE, tlast));
  if (wflags) {
    if (acquire)
      wait_all_acquire(wflags, 4, epoch, err);
    else
      wait_all(wflags, 4, epoch, err);
  }
  // A operands: S[32 wave + col][16 s + 8 g + e] as bf16 hi and lo terms
  const float* rec = cum + ((size_t)bh * F + fend - 1) * kReluWideRec;
  u32x4 ahi[8], alo[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float* src = rec + (wave * 32 + col) * D + s * 16 + g * 8;
    const float4 x0 = *reinterpret_cast<const float4*>(src);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
    const uint2 p0 = split_bf16x2(x0.x, x0.y), p1 = split_bf16x2(x0.z, x0.w);
    const uint2 p2 = split_bf16x2(x1.x, x1.y), p3 = split_bf16x2(x1.z, x1.w);
    ahi[s] = u32x4{p0.x, p1.x, p2.x, p3.x};
    alo[s] = u32x4{p0.y, p1.y, p2.y, p3.y};
  }
  // the 8 normaliser entries of the dims this thread stages (chunk tid % 16)
  float zr[8];
  {
    const float4 z0 = *reinterpret_cast<const float4*>(rec + D * D + (tid & 15) * 8);
    const float4 z1 = *reinterpret_cast<const float4*>(rec + D * D + (tid & 15) * 8 + 4);
    zr[0] = z0.x, zr[1] = z0.y, zr[2] = z0.z, zr[3] = z0.w;
    zr[4] = z1.x, zr[5] = z1.y, zr[6] = z1.z, zr[7] = z1.w;
  }

  float wq8[8];  // the prologue's query weights of this thread's channels (chunk tid % 16)
  load_weights8(P.wq, bh % L.H, DI, (tid & 15) * 8, wq8);
  // phi(q) into LDS buffer buf, and each token's denominator into den[buf];
  // t0: the tile's first token (its rows past the chunk hold token n0)
  auto stage = [&](const Regs& X, int buf, int t0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      u32x4 w = cb < CI ? X.q[r] : u32x4{0u, 0u, 0u, 0u};
      float d = 0.0f;
      if (P.rope()) {  // the denominator takes the unrotated features, the numerator the rotated ones
        Prologue Pf = P;
        Pf.relu = 1;
        float pre[8];
        w = prologue_bf16x8(w, wq8, P.wq != nullptr, Pf, false, 1.0 / DI,
                            [](double x) { return group_sum_f64<16>(x); },
                            true, rot8_load(P.rope8(f, t0 + tok < n1 ? t0 + tok : n0, cb < CI ? cb : 0, DI)), pre);
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(zr[e], pre[e], d);
      } else {
        if (P.wq) w = prologue_bf16x8(w, wq8, true, P, false, 1.0 / DI, [](double x) { return group_sum_f64<16>(x); });
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[e] = relu_bf16x2(w[e]);
          d = fmaf(zr[2 * e], bf16lo_to_f32(w[e]), d);
          d = fmaf(zr[2 * e + 1], bf16hi_to_f32(w[e]), d);
        }
      }
      *reinterpret_cast<u32x4*>(&lds[buf][tok * ROW + cb * 8]) = w;
      d = group_sum<16>(d);  // the 16 lanes of a DPP row hold the 16 chunks of this token
      if (cb == 0) den[buf][tok] = d;
    }
  };

  // query tiles keep coming in through the three register sets, so three
  // tiles are in flight while one is contracted
  stage(R0, 0, n0);
  fetch(R0, min(n0 + 3 * TILE, tlast));
  __syncthreads();
  // a tile's outputs leave as whole rows (16-byte chunks, consecutive lanes on
  // consecutive bytes) from its staging buffer
  auto drain = [&](int it, const bool full) {
    const int t0 = n0 + it * TILE;
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int ci = r * 256 + tid;
      const int tok = ci >> 4, cb = ci & 15;
      const u32x4 w = *reinterpret_cast<const u32x4*>(&ost[it & 1][tok * ROW + cb * 8]);
      if ((full || t0 + tok < n1) && cb < CI) st16_stream(of + (size_t)(t0 + tok) * L.sn + cb * 8, w);
    }
  };
  // tile `it` is in LDS buffer it % 2; nxt holds tile it + 1 and is refilled with tile it + 4
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
      const float inv = 1.0f / (den[buf][half * 32 + col] + eps);
      // lane (col, g) of wave w holds token half*32 + col, dims 32 w + 8 q4 + 4 g + 0..3
      uint16_t* srow = &ost[buf][(half * 32 + col) * ROW + wave * 32 + 4 * g];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        uint2 w;
        w.x = pack_bf16x2(acc[4 * q4 + 0] * inv, acc[4 * q4 + 1] * inv);
        w.y = pack_bf16x2(acc[4 * q4 + 2] * inv, acc[4 * q4 + 3] * inv);
        *reinterpret_cast<uint2*>(srow + 8 * q4) = w;
      }
    }
    stage(nxt, buf ^ 1, min(n0 + (it + 1) * TILE, tlast));  // the next tile (past the end: a copy of the last, never read)
    fetch(nxt, min(n0 + (it + 4) * TILE, tlast));
    __syncthreads();
    drain(it, full);
  };
  // Full tiles run in threes with no branch in the loop body; a last,
  // partial tile stores under a token check after the loop.
  int it = 0;
  for (; it + 3 <= nfull; it += 3) {
    tile(it, R1, true);
    tile(it + 1, R2, true);
    tile(it + 2, R0, true);
  }
  // R1, R2 and R0 hold tiles it + 1 .. it + 3: at most two more full tiles,
  // then at most one partial one
  if (it + 2 <= nfull) {
    tile(it, R1, true);
    tile(it + 1, R2, true);
    if (it + 2 < ntiles) tile(it + 2, R0, false);
  } else if (it + 1 <= nfull) {
    tile(it, R1, true);
    if (it + 1 < ntiles) tile(it + 1, R2, false);
  } else if (it < ntiles) {
    tile(it, R1, false);
  }
}

}  // namespace linscan
