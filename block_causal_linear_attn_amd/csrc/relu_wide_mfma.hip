// relu_wide_mfma.hip -- the single-launch bf16 MFMA ReLU linear-attention scan
// for wide heads (head dims 112 and 128), built from relu_wide_items.h.
//
// Block ids run over units of B*H padded to a multiple of 8 items, head-minor,
// so all items of a head share one XCD and hand off through its L2 (padding
// items leave at once).  Units np f .. np f + np - 1 hold the np summary parts
// of frame f, part np - 1 first and part 0 last; after the F frames' summary
// units come the output units, frame by frame, one item per head and token
// chunk.  Part 0 of a frame waits for the frame's other parts (earlier units
// of the same frame) and for part 0 of the previous frame (an earlier frame);
// an output item waits for part 0 of the last frame of its block.  Every
// item waited on has a lower block id, and block ids dispatch in order, so it
// is running or done and every wait ends.  All summaries are dispatched
// before any output item: output items wait for a chain through all earlier
// frames, so one dispatched early would only hold a slot that a later frame's
// summary needs to start (measured: at 20 heads x 10 frames x 3600 tokens,
// head dim 112, 162 us with all summaries first against 190 us with output
// items of frame f dispatched beside summaries of frame f + 1).
#include "relu_wide_items.h"
#include "kernels.h"

#include <type_traits>

namespace linscan {

namespace {

constexpr int kReluWideLds = kReluWideSumLds + kReluWide * 4 > kReluWideOutLds ? kReluWideSumLds + kReluWide * 4
                                                                                : kReluWideOutLds;

template <int DI>
__global__ __launch_bounds__(256, 2) void relu_wide_fused_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ cum, const float* S0, const float* z0, float* S_out,
    float* z_out, float eps, long bh_n, long bhp, int F, int N, int bfr, int nco, int chunko, int np,
    uint64_t* __restrict__ flags, uint64_t epoch, uint32_t* err, TokLayout L, Prologue P) {
  __shared__ __align__(16) uint8_t lds[kReluWideLds];
  const long b = blockIdx.x;
  const long bh = L.head_of_slot(b % bhp);
  const long u = b / bhp;  // unit: one item per head
  if (bh >= bh_n) return;
  const long bhf_n = bh_n * F;
  if (u < (long)np * F) {
    // the parts' records follow the F cumulative records of every head, their
    // flags the frames' flags
    const int f = (int)(u / np), part = np - 1 - (int)(u % np);
    relu_wide_summary_item<DI>(k, v, cum, S0, z0, S_out, z_out, F, N, bh, f, np, part,
                               cum + (size_t)bhf_n * kReluWideRec, flags + bhf_n, flags, epoch, err, lds, L, P);
    return;
  }
  const long r = u - (long)np * F;
  const int f = (int)(r / nco), c = (int)(r % nco);
  const int fend = min(F, (f / bfr + 1) * bfr);
  wait_all(&flags[bh * F + fend - 1], 1, epoch, err);
  relu_wide_output_item<DI>(q, o, cum, eps, F, N, bfr, nco, chunko, (bh * F + f) * nco + c, lds, L, P);
}

template <typename Body>
hipError_t with_wide_dim(int D, Body body) {
  if (D == 128) return body(std::integral_constant<int, 128>{});
  if (D == 112) return body(std::integral_constant<int, 112>{});
  return hipErrorInvalidValue;
}

}  // namespace

bool relu_wide_mfma(int D, int dtype) { return dtype == DT_BF16 && (D == 112 || D == 128); }

hipError_t launch_relu_wide_fused_mfma(const ScanArgs& a, long bhp, uint64_t* flags, uint64_t epoch,
                                       uint32_t* err, hipStream_t st) {
  return with_wide_dim(a.D, [&](auto di) {
    constexpr int DI = decltype(di)::value;
    const long grid = (long)a.F * bhp * (a.nc + a.nco);
    hipLaunchKernelGGL(relu_wide_fused_mfma<DI>, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.partial, a.S0, a.z0, a.S_out,
                       a.z_out, a.eps, a.bh, bhp, a.F, a.N, a.bfr, a.nco, a.chunko, a.nc, flags, epoch, err, a.L,
                       a.P);
    return hipGetLastError();
  });
}

}  // namespace linscan
