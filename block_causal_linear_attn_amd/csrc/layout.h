// layout.h -- element strides of the token tensors q, k, v, o.
//
// A token tensor is indexed [b][h][f][n][d] with d contiguous; the library's
// default is the packed [B][H][F][N][D] layout, and any layout whose four
// outer strides are given, such as [B][F][N][H][D] (frames and tokens outer,
// heads inner), is read and written in place.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace linscan {

struct TokLayout {
  long long sb = 0, sh = 0, sf = 0, sn = 0;  // element strides of batch, head, frame, token
  int H = 1, F = 1;
  // Heads whose rows share 128-byte lines (layouts with heads interleaved in a
  // token row and rows shorter than a line) run in groups of hg on one XCD, so
  // a line is fetched into one L2 rather than into hg of them.
  int hg = 1;
  // element offset of token 0 of frame f of head (b, h), with bhf = (b*H + h)*F + f
  __host__ __device__ __forceinline__ size_t base(long bhf) const {
    const long f = bhf % F, bh = bhf / F;
    return (size_t)((bh / H) * sb + (bh % H) * sh + f * sf);
  }
  // Head (b*H + h) served by work-item slot `slot` of a launch whose block ids
  // put slot % 8 on XCD slot % 8: with hg > 1, slots 8m + x for m = hg*j ..
  // hg*j + hg - 1 (one XCD) serve hg consecutive heads.  A bijection on
  // [0, bhp) when bhp is a multiple of 8*hg.
  __host__ __device__ __forceinline__ long head_of_slot(long slot) const {
    const long m = slot / 8, x = slot % 8;
    return hg * (8 * (m / hg) + x) + m % hg;
  }
  __host__ __device__ static TokLayout packed(int H, int F, int N, int D) {
    TokLayout L;
    L.sn = D;
    L.sf = (long long)N * D;
    L.sh = (long long)F * N * D;
    L.sb = (long long)H * F * N * D;
    L.H = H > 0 ? H : 1;
    L.F = F > 0 ? F : 1;
    return L;
  }
};

// The per-token prologue applied to q and k as they are loaded, before the
// scan's own feature map and key scale: RMSNorm over the D channels of a
// head with per-(head, channel) weights, then (GDN) ReLU, then (GDN, keys)
// division by the L2 norm, then (GDN) the rotary position embedding.
// Results enter the contractions rounded to bf16.
struct Prologue {
  const float* wq = nullptr;  // [H][D] RMSNorm weights of q, or nullptr: no norm on q
  const float* wk = nullptr;  // [H][D] RMSNorm weights of k, or nullptr: no norm on k
  float eps = 1e-6f;
  int relu = 0;               // ReLU on q and k after the norm
  int l2 = 0;                 // keys divided by their L2 norm
  // Rotary embedding: channel pair (2i, 2i+1) of a token of frame f (of the
  // call) and index n turns by the angle whose (cos, sin) is row roff + f,
  // pair i of rf ([T][rpf][2]) for i < rpf, else row n, pair i - rpf of rt
  // ([N][D/2 - rpf][2]).  rpf is a multiple of 4, so the 8 channels of one
  // 16-byte chunk take one table.
  const float* rf = nullptr;
  const float* rt = nullptr;
  int rpf = 0;
  int roff = 0;
  __host__ __device__ bool rope() const { return rf != nullptr || rt != nullptr; }
  __host__ __device__ bool on_q() const { return wq != nullptr || relu || rope(); }
  __host__ __device__ bool on_k() const { return wk != nullptr || relu || l2 || rope(); }
  // (cos, sin) of channel chunk c (pairs 4c .. 4c + 3, 8 floats, 16-byte
  // aligned) of token n of frame f, for head dim D
  __host__ __device__ const float* rope8(long f, long n, int c, int D) const { return rope1(f, n, 4 * c, D); }
  // (cos, sin) of channel pair p of token n of frame f
  __host__ __device__ const float* rope1(long f, long n, int p, int D) const {
    return p < rpf ? rf + ((size_t)(roff + f) * rpf + p) * 2 : rt + ((size_t)n * (D / 2 - rpf) + (p - rpf)) * 2;
  }
};

}  // namespace linscan
