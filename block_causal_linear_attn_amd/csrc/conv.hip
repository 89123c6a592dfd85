// conv.hip -- block-causal temporal convolution of kernel 3 along frames (the
// SANA-Video Causal Mix-FFN's temporal mixing).
//
// For every channel (h, d) and token n, with blocks of `bfr` frames from
// frame 0 of the call:
//   y_f = w0 x_{f-1} + w1 x_f + w2 x_{f+1} + bias
// where the next-frame tap sees zero when frame f ends its block (or the
// call), and x_{-1} is the carried last frame of the previous block.
//
// The op moves each input and output byte once, so it is bound by HBM.  One
// thread owns 16 bytes of channels (8 bf16 or 4 fp32) of one token and walks
// all frames: the frame-to-frame window stays in registers, so x is read
// once (not three times), and consecutive threads cover consecutive 16-byte
// chunks of a frame's contiguous N x D slab, so every load and store is
// coalesced.  Frames go in groups of 8: the loads of a group (with the next
// group's first frame) are issued before any is used.
#include "device_common.h"
#include "kernels.h"

namespace linscan {

namespace {

constexpr int kConvGroup = 8;  // frames per group

template <typename T>
struct ConvVec;
template <>
struct ConvVec<uint16_t> {  // 8 bf16
  static constexpr int kN = 8;
  static __device__ __forceinline__ void unpack(u32x4 w, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16lo_to_f32(w[e]);
      x[2 * e + 1] = bf16hi_to_f32(w[e]);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float* x) {
    return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
  }
};
template <>
struct ConvVec<float> {  // 4 fp32
  static constexpr int kN = 4;
  static __device__ __forceinline__ void unpack(u32x4 w, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
  }
  static __device__ __forceinline__ u32x4 pack(const float* x) {
    return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
  }
};

// One thread per (b*h, token, 16-byte channel chunk); `cells` = B*H*N*chunks.
template <typename T>
__global__ __launch_bounds__(256) void temporal_conv3_kernel(const T* __restrict__ x, const float* __restrict__ w,
                                                             const float* __restrict__ bias, const T* carry_in,
                                                             T* __restrict__ y, T* carry_out, long cells, int H,
                                                             int F, int N, int D, int bfr) {
  using V = ConvVec<T>;
  constexpr int E = V::kN;
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= cells) return;
  const int chunks = D / E;
  const long bhn = t / chunks;  // (b*h) * N + n
  const int d0 = (int)(t % chunks) * E;
  const long bh = bhn / N;
  const int h = (int)(bh % H);
  const size_t frame = (size_t)N * D;                               // elements per frame slab
  const T* xs = x + (size_t)bh * F * frame + (size_t)(bhn % N) * D + d0;  // frame 0 of this cell
  T* ys = y + (size_t)bh * F * frame + (size_t)(bhn % N) * D + d0;

  // taps of this thread's channels: w[h][d0 + e][0..2], the bias and the
  // carried frame.  Optional operands are loaded from a valid stand-in
  // address and replaced by zero afterwards: a load under a condition would
  // make the compiler wait for all of these loads before the first frame
  // loads are issued (measured 84 -> 67 us at 322 MB).
  const size_t cell = (size_t)bhn * D + d0;  // offset in [B][H][N][D]
  const float* wp = w + ((size_t)h * D + d0) * 3;
  const float* bp = bias ? bias + (size_t)h * D + d0 : wp;
  const T* cp = carry_in ? carry_in + cell : xs;
  float w0[E], w1[E], w2[E], bs[E], prev[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    w0[e] = wp[3 * e];
    w1[e] = wp[3 * e + 1];
    w2[e] = wp[3 * e + 2];
    bs[e] = bp[e];
  }
  V::unpack(ld16(cp), prev);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bs[e] = bias ? bs[e] : 0.0f;
    prev[e] = carry_in ? prev[e] : 0.0f;
  }
  u32x4 last = {0u, 0u, 0u, 0u};  // x_{F-1}, for carry_out
  for (int f0 = 0; f0 < F; f0 += kConvGroup) {
    // frames f0 .. f0 + 8 (the last one only as the next-frame tap), all in
    // flight before the first is used.  Frames past the call are not loaded:
    // measured at 10-frame blocks, skipping them (74 -> 66 us at 322 MB)
    // beats re-reading the last frame, even though the loads under a
    // condition make the first use wait for all of them.
    u32x4 raw[kConvGroup + 1];
#pragma unroll
    for (int i = 0; i <= kConvGroup; ++i)
      raw[i] = f0 + i < F ? ld16_stream(xs + (size_t)(f0 + i) * frame) : u32x4{0u, 0u, 0u, 0u};
    float cur[E];
    V::unpack(raw[0], cur);
#pragma unroll
    for (int i = 0; i < kConvGroup; ++i) {
      const int f = f0 + i;
      if (f >= F) break;
      const bool ends = (f + 1) % bfr == 0 || f + 1 == F;
      float nxt[E], out[E];
      V::unpack(raw[i + 1], nxt);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xn = ends ? 0.0f : nxt[e];
        out[e] = fmaf(w2[e], xn, fmaf(w1[e], cur[e], fmaf(w0[e], prev[e], bs[e])));
        prev[e] = cur[e];
        cur[e] = nxt[e];
      }
      st16_stream(ys + (size_t)f * frame, V::pack(out));
      if (f == F - 1) last = raw[i];
    }
  }
  // the carry is read above before it is written here, by this thread only,
  // so carry_out may be carry_in
  if (carry_out) st16(carry_out + cell, last);
}

}  // namespace

hipError_t launch_temporal_conv3(int dtype, const void* x, const float* w, const float* bias, const void* carry_in,
                                 void* y, void* carry_out, long BH, int H, int F, int N, int D, int bfr,
                                 hipStream_t st) {
  const int E = dtype == DT_BF16 ? 8 : 4;
  const long cells = BH * N * (long)(D / E);
  if (cells == 0) return hipSuccess;
  const dim3 grid((unsigned)((cells + 255) / 256)), block(256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(temporal_conv3_kernel<uint16_t>, grid, block, 0, st, (const uint16_t*)x, w, bias,
                       (const uint16_t*)carry_in, (uint16_t*)y, (uint16_t*)carry_out, cells, H, F, N, D, bfr);
  else
    hipLaunchKernelGGL(temporal_conv3_kernel<float>, grid, block, 0, st, (const float*)x, w, bias,
                       (const float*)carry_in, (float*)y, (float*)carry_out, cells, H, F, N, D, bfr);
  return hipGetLastError();
}

}  // namespace linscan
