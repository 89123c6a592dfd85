// device_common.h -- small device helpers shared by the gfx950 scan kernels:
// bf16 packing, the ReLU feature map on packed bf16, hi/lo splitting of fp32
// values into two bf16 terms, and the MFMA operand types.
//
// MFMA conventions used throughout (wave64, gfx950):
//   v_mfma_f32_32x32x16_bf16  A: lane l holds row (l & 31), 8 k-slots of group (l >> 5)
//                             B: lane l holds col (l & 31), the same 8 k-slots
//                             C: lane l, reg r holds C[8*(r>>2) + 4*(l>>5) + (r&3)][l & 31]
//   v_mfma_f32_16x16x32_bf16  A: lane l holds row (l & 15), 8 k-slots of group (l >> 4)
//                             B: lane l holds col (l & 15), the same 8 k-slots
//                             C: lane l, reg r holds C[4*(l>>4) + r][l & 15]
//   v_mfma_f32_16x16x4_f32    A: lane l holds A[l & 15][l >> 4]
//                             B: lane l holds B[l >> 4][l & 15]
//                             C: lane l, reg r holds C[4*(l>>4) + r][l & 15]
// Only the C layouts matter for correctness of a contraction: A and B share
// their k-slot assignment, so any consistent placement of the contracted index
// (tokens or dimensions) into the slots sums over all of it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace linscan {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32); NaN stays NaN.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ReLU on two packed bf16 values: a value whose sign bit is set becomes +0.
// As 16-bit integers, exactly those values are negative, so a signed max
// with zero implements it (v_pk_max_i16).
__device__ __forceinline__ uint32_t relu_bf16x2(uint32_t w) {
  shortx2 s = __builtin_bit_cast(shortx2, w);
  shortx2 zero = {0, 0};
  s = __builtin_elementwise_max(s, zero);
  return __builtin_bit_cast(uint32_t, s);
}
__device__ __forceinline__ float relu_f32(float x) { return signbit(x) ? 0.0f : x; }

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi): 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}
// Two values at once, packed: .x = (bf16(x0), bf16(x1)) hi terms, .y the lo terms.
__device__ __forceinline__ uint2 split_bf16x2(float x0, float x1) {
  const uint32_t hi = pack_bf16x2(x0, x1);
  return make_uint2(hi, pack_bf16x2(x0 - bf16lo_to_f32(hi), x1 - bf16hi_to_f32(hi)));
}

// Sum over groups of G consecutive lanes (G = 4, 8 or 16, within a DPP row),
// every lane of a group getting the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 4 || G == 8 || G == 16, "groups of 4, 8 or 16 lanes");
  auto add = [](float v, int s) { return v + __int_as_float(s); };
  x = add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lanes ^1
  x = add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lanes ^2
  if (G >= 8) x = add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // half-row mirror
  if (G >= 16) x = add(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row mirror
  return x;
}

// fp64 -> bf16, round to nearest even in one step: the 45 dropped bits of
// the double's fraction decide, so no second rounding (as through fp32) can
// move a value that lies just off a halfway point onto it.  For finite values
// in the normal fp32 range.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  u += ((1ull << 44) - 1) + ((u >> 45) & 1ull);
  u &= ~((1ull << 45) - 1);
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;  // exact: 8 significant bits
}
__device__ __forceinline__ uint32_t pack_bf16x2_f64(double lo, double hi) {
  return f64_to_bf16(lo) | (f64_to_bf16(hi) << 16);
}

// 1 / sqrt(v) for normal v > 0, to within a few fp64 ulps: the hardware
// estimate (about 2^-29 relative error) and two Newton steps, which square the
// error each time.  Cheaper than a correctly rounded square root and
// division, and far inside what could change a later rounding to bf16.
__device__ __forceinline__ double rsqrt_f64(double v) {
  double y = __builtin_amdgcn_rsq(v);
  const double h = 0.5 * v;
  y = y * fma(-h * y, y, 1.5);
  y = y * fma(-h * y, y, 1.5);
  return y;
}

// A 64-bit value from another lane of the DPP row, as two 32-bit moves.
// Every control used here reads a lane of the same row, so no lane falls
// back to the old value: with bound_ctrl the moves need no zeroed
// destination (8 fewer instructions per 16-lane sum).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long u = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(u & 0xffffffffll), CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(u >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double(((long long)hi << 32) | (long long)(uint32_t)lo);
}
// group_sum in fp64.
template <int G>
__device__ __forceinline__ double group_sum_f64(double x) {
  static_assert(G == 4 || G == 8 || G == 16, "groups of 4, 8 or 16 lanes");
  x += dpp_f64<0xB1>(x);
  x += dpp_f64<0x4E>(x);
  if (G >= 8) x += dpp_f64<0x141>(x);
  if (G >= 16) x += dpp_f64<0x140>(x);
  return x;
}

// The (cos, sin) of the rotary embedding of 4 channel pairs (one lane's 8
// channels): a = pairs 0 and 1, b = pairs 2 and 3.
struct Rot8 {
  float4 a, b;
};
__device__ __forceinline__ Rot8 rot8_load(const float* cs) {
  return Rot8{*reinterpret_cast<const float4*>(cs), *reinterpret_cast<const float4*>(cs + 4)};
}
// The rotary embedding of 4 channel pairs held as fp64.
__device__ __forceinline__ void rope_rotate8(double (&x)[8], const Rot8& r) {
  const float4 a = r.a, b = r.b;
  const float c[4] = {a.x, a.z, b.x, b.z}, s[4] = {a.y, a.w, b.y, b.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double x0 = x[2 * j], x1 = x[2 * j + 1];
    x[2 * j] = x0 * (double)c[j] - x1 * (double)s[j];
    x[2 * j + 1] = x0 * (double)s[j] + x1 * (double)c[j];
  }
}

// The prologue (see Prologue) on 8 channels of one token, held by one lane as
// packed bf16; `red` completes a per-token fp64 sum over the lanes that hold
// the token's other channels (every lane calls it: DPP or cross-lane
// exchange).  wt: the RMSNorm weights of these 8 channels (zero past the head
// dim), inv_d = 1 / D.  Returns the result rounded to bf16.
//
// The arithmetic is fp64 and the result is rounded once, from fp64: rounding
// to bf16 picks one of two neighbours, and an fp32 chain (a few rounding
// errors of 2^-24) picks the other neighbour than the exact value for about
// one channel in 10^4 to 10^5.  One such 2^-8 step in a key moves every later
// state, and outputs that cancel (a query nearly orthogonal to the state's
// rows) turn it into a large relative error.  In fp64 the chance is ~2^-40.
//
// rope: rotate the 4 channel pairs by rot (their rows of the tables,
// Prologue::rope8).  pre: if not nullptr, receives the 8 values before the
// rotation, as fp32.
template <typename Red>
__device__ __forceinline__ u32x4 prologue_bf16x8(u32x4 w, const float (&wt)[8], bool norm, const Prologue& P,
                                                 bool is_k, double inv_d, Red red, bool rope = false,
                                                 const Rot8& rot = Rot8{}, float* pre = nullptr) {
  double x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16lo_to_f32(w[e]);
    x[2 * e + 1] = bf16hi_to_f32(w[e]);
  }
  if (norm && is_k && P.l2) {
    // RMSNorm's factor is positive and the same for every channel of the
    // token: the ReLU keeps it and the L2 scale below removes it, so only the
    // weights remain (x * w exact in fp64)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= (double)wt[e];
  } else if (norm) {
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fma(x[e], x[e], ss);
    const double inv = rsqrt_f64(fma(red(ss), inv_d, (double)P.eps));
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * (double)wt[e] * inv;  // x * w exact in fp64
  }
  // Without the rotation or the L2 scale the ReLU is applied to the rounded
  // bf16 values (one packed integer max per two): the rounding keeps every
  // sign, so the result is the same.  The rotation mixes channels and the L2
  // sum needs the ReLU's values, so there it comes first.
  const bool relu_early = P.relu && (rope || (is_k && P.l2));
  if (relu_early) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = signbit(x[e]) ? 0.0 : x[e];
  }
  if (is_k && P.l2) {
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fma(x[e], x[e], ss);
    ss = red(ss);
    const double inv = ss > 0.0 ? rsqrt_f64(ss) : 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] *= inv;
  }
  if (pre) {
#pragma unroll
    for (int e = 0; e < 8; ++e) pre[e] = (float)x[e];
  }
  if (rope) rope_rotate8(x, rot);
  u32x4 out = {pack_bf16x2_f64(x[0], x[1]), pack_bf16x2_f64(x[2], x[3]), pack_bf16x2_f64(x[4], x[5]),
               pack_bf16x2_f64(x[6], x[7])};
  if (P.relu && !relu_early) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = relu_bf16x2(out[e]);
  }
  return out;
}

// The 8 RMSNorm weights of channels c0 .. c0 + 7 of head h (zero at and past
// channel DI, or all zero without weights), loaded without a branch on the
// lane: past DI the address is clamped and the values are zeroed.
__device__ __forceinline__ void load_weights8(const float* w, long h, int DI, int c0, float (&wt)[8]) {
  const float* p = w ? w + (size_t)h * DI + (c0 < DI ? c0 : 0) : nullptr;
  const float4 a = p ? *reinterpret_cast<const float4*>(p) : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 b = p ? *reinterpret_cast<const float4*>(p + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  const bool in = c0 < DI;
  wt[0] = in ? a.x : 0.f, wt[1] = in ? a.y : 0.f, wt[2] = in ? a.z : 0.f, wt[3] = in ? a.w : 0.f;
  wt[4] = in ? b.x : 0.f, wt[5] = in ? b.y : 0.f, wt[6] = in ? b.z : 0.f, wt[7] = in ? b.w : 0.f;
}

// The 8 bf16 values of an MFMA operand fragment (element e in half e % 2 of
// word e / 2) times 8 fp32 factors, as bf16 hi + lo terms (16 significant
// bits), so that MFMAs on hi and on lo together take products with the
// scaled values to about fp32 accuracy.
__device__ __forceinline__ void scale_split_bf16x8(u32x4 w, float4 s0, float4 s1, u32x4& hi, u32x4& lo) {
  const uint2 p0 = split_bf16x2(bf16lo_to_f32(w[0]) * s0.x, bf16hi_to_f32(w[0]) * s0.y);
  const uint2 p1 = split_bf16x2(bf16lo_to_f32(w[1]) * s0.z, bf16hi_to_f32(w[1]) * s0.w);
  const uint2 p2 = split_bf16x2(bf16lo_to_f32(w[2]) * s1.x, bf16hi_to_f32(w[2]) * s1.y);
  const uint2 p3 = split_bf16x2(bf16lo_to_f32(w[3]) * s1.z, bf16hi_to_f32(w[3]) * s1.w);
  hi = u32x4{p0.x, p1.x, p2.x, p3.x};
  lo = u32x4{p0.y, p1.y, p2.y, p3.y};
}

// ds_read_b64_tr_b16 (gfx950 LDS transpose read).  Within each group of 16
// lanes, output lane i, element r is 16-bit element (i % 4) of the 8 bytes
// addressed by lane 4r + i/4 of the same group.  So if lane j of a group
// points at row t0 + j/4, columns c0 + 4(j%4) .. +3 of a row-major bf16 tile,
// lane i receives column c0 + i of rows t0 .. t0+3: four tokens of one
// dimension, the layout an MFMA operand wants when tokens are contracted.
typedef short shortx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  shortx4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)((__attribute__((address_space(3))) uint16_t*)p));
  return __builtin_bit_cast(uint2, r);
}
// MFMA 32x32x16 operand of one 32-wide dimension block: lane l gets dimension
// col0 + (l & 31) of tokens t0 + 8 (l >> 5) + e, e = 0..7, from a row-major
// [token][pitch] bf16 LDS tile (pitch a multiple of 4 elements).
template <int PITCH>
__device__ __forceinline__ u32x4 gather_tokens_32(const uint16_t* tile, int t0, int col0, int lane) {
  const int q = lane >> 4, j = lane & 15;
  const uint16_t* p = tile + (t0 + 8 * (q >> 1) + (j >> 2)) * PITCH + col0 + 16 * (q & 1) + 4 * (j & 3);
  const uint2 a = lds_read_tr16(p);
  const uint2 b = lds_read_tr16(p + 4 * PITCH);
  return u32x4{a.x, a.y, b.x, b.y};
}

// Unpadded token-major LDS tiles of C 16-byte chunks per token row, with the
// chunk index XOR-swizzled by token so that the four tokens one half-wave of
// a transpose read touches (64 bytes each) fall on distinct LDS banks:
// 256-byte rows (C = 16) swizzle by token % 4, 128-byte rows (C = 8) by
// (token / 2) % 2; 64-byte rows (C = 4) tile the 64 banks unswizzled.
template <int C>
__device__ __forceinline__ int chunk_swizzle(int token) {
  static_assert(C == 4 || C == 8 || C == 16, "rows of 4, 8 or 16 chunks");
  return C == 16 ? (token & 3) << 2 : C == 8 ? ((token >> 1) & 1) << 2 : 0;
}
// element offset of (token, 16-byte chunk) in such a tile
template <int C>
__device__ __forceinline__ int swz_offset(int token, int chunk) {
  return token * C * 8 + ((chunk ^ chunk_swizzle<C>(token)) << 3);
}
// gather_tokens_32 on a swizzled tile of C chunks per row (col0 a multiple of 32)
template <int C>
__device__ __forceinline__ u32x4 gather_tokens_32_swz(const uint16_t* tile, int t0, int col0, int lane) {
  const int q = lane >> 4, j = lane & 15;
  const int token = t0 + 8 * (q >> 1) + (j >> 2);
  const int d = col0 + 16 * (q & 1) + 4 * (j & 3);
  const uint16_t* p = tile + swz_offset<C>(token, d >> 3) + (d & 7);
  const uint2 a = lds_read_tr16(p);
  const uint2 b = lds_read_tr16(p + 4 * C * 8);  // token + 4: same swizzle
  return u32x4{a.x, a.y, b.x, b.y};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16x16x4f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16-byte global load / store through 32-bit words.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// The same for data touched once (token tensors): non-temporal, so that the
// stream does not push out of the caches what other work items of the launch
// still have to read.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ReLU scan: the state (S_f, z_f) frame f reads, written to LDS by the whole
// workgroup: the initial state of head bh plus the chunk partials of every
// frame up to the end of f's block (blocks of `bfr` frames from frame 0; a
// block reads the state after all of its own frames).  `partial` holds
// [bh][frame][chunk] records of D*D + D floats, `init` [bh] records.
// Partial loads are issued eight at a time so their latencies overlap.
template <int D>
__device__ __forceinline__ void relu_frame_state(const float* __restrict__ partial,
                                                 const float* __restrict__ init, long bh, int f,
                                                 int F, int nc, int bfr, float* Ss, int pitch,
                                                 float* zs) {
  constexpr int OUT = D * D + D;
  const int fend = min(F, (f / bfr + 1) * bfr);
  const int cnt = fend * nc;
  const float* P = partial + (size_t)bh * F * nc * OUT;
  for (int e = threadIdx.x; e < OUT; e += blockDim.x) {
    float acc = init[(size_t)bh * OUT + e];
    int i = 0;
    for (; i + 8 <= cnt; i += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = P[(size_t)(i + j) * OUT + e];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += v[j];
    }
    for (; i < cnt; ++i) acc += P[(size_t)i * OUT + e];
    if (e < D * D)
      Ss[(e / D) * pitch + e % D] = acc;
    else
      zs[e - D * D] = acc;
  }
}

// ReLU scan: workgroup (frame 0, chunk 0) of each head copies the initial
// state (or zeros) into the workspace, so that later kernels never read
// state_in and state_out may alias it.
// PAIR: head bh is the pair of heads 2 bh and 2 bh + 1 of dim D / 2, whose
// states S0 holds one after the other; the pair's state is block-diagonal.
template <int D, bool PAIR = false>
__device__ __forceinline__ void relu_copy_init(const float* S0, const float* z0, float* init, long wg,
                                               int F, int nc) {
  constexpr int OUT = D * D + D;
  constexpr int DH = D / 2;
  if (wg % ((long)F * nc) != 0) return;
  const long bh = wg / ((long)F * nc);
  for (int e = threadIdx.x; e < OUT; e += blockDim.x) {
    float x = 0.0f;
    if (e < D * D) {
      const int m = e / D, n = e % D;
      if (PAIR) {
        if (S0 && m / DH == n / DH) x = S0[((size_t)2 * bh + m / DH) * DH * DH + (m % DH) * DH + n % DH];
      } else if (S0) {
        x = S0[(size_t)bh * D * D + e];
      }
    } else if (z0) {  // (the pair's two normalisers are adjacent: the same index)
      x = z0[(size_t)bh * D + e - D * D];
    }
    init[(size_t)bh * OUT + e] = x;
  }
}

// Token-tensor element types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
  // an fp64 result in this precision (one rounding)
  static __device__ __forceinline__ float round(double x) { return (float)x; }
};
template <> struct Elem<uint16_t> {  // bf16 bits
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
  static __device__ __forceinline__ float round(double x) { return __uint_as_float(f64_to_bf16(x) << 16); }
};

// One channel of the prologue in fp64: x w s1 (RMSNorm factor s1, weight w;
// s1 = w = 1 without it), then ReLU, then the L2 factor s2 (1 without it).
__device__ __forceinline__ double prologue_chan(float x, float w, double s1, int relu, double s2) {
  double y = (double)x * (double)w * s1;
  if (relu) y = signbit(y) ? 0.0 : y;
  return y * s2;
}

}  // namespace linscan
