// relu_wide_mfma.hip -- the single-launch bf16 MFMA ReLU linear-attention scan
// for wide heads (head dims 112 and 128), built from relu_wide_items.h.
//
// Block ids run over units of B*H padded to a multiple of 8 items, head-minor,
// so all items of a head share one XCD and hand off through its L2 (padding
// items leave at once).  Units np f .. np f + np - 1 hold the np summary parts
// of frame f; after the F frames' summary units come four prefix units (one
// item per 32 rows of a head's state, each walking all frames), then the
// output units, frame by frame, one item per head and token chunk.  A prefix
// item waits for the parts of each frame (earlier units); an output item
// waits for the four prefix items' flags of the last frame of its block.
// Every item waited on has a lower block id, and block ids dispatch in order,
// so it is running or done and every wait ends.  All summaries are
// dispatched before any output item: an output item dispatched early would
// only hold a slot that a later frame's summary needs to start (measured: at
// 20 heads x 10 frames x 3600 tokens, head dim 112, 162 us with all summaries
// first against 190 us with output items of frame f dispatched beside
// summaries of frame f + 1).
//
// When B*H is not a multiple of 8 and F > 1 (spread), one XCD per head would leave
// some XCDs with a head more than others (20 heads: 3 on XCDs 0-3, 2 on
// 4-7), and the output phase would end on the busy ones.  The output items
// then run over consecutive block ids without padding, so every XCD takes
// the same share; their records cross XCDs, so each prefix item writes back
// its L2 once, after its last frame, before setting its flags, and each
// output item takes an acquire fence after its wait.  At 20 heads x 10
// frames x 3600 tokens, head dim 112: 164 -> 157 us.  Summaries stay on their
// head's XCD: releasing each of them (400 write-backs) cost 14 us more.
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
    uint64_t* __restrict__ flags, uint64_t epoch, uint32_t* err, TokLayout L, Prologue P, int spread) {
  __shared__ __align__(16) uint8_t lds[kReluWideLds];
  const long b = blockIdx.x;
  const long nfront = ((long)np * F + 4) * bhp;
  if (spread && b >= nfront) {
    // output items over (frame, chunk, head), head-minor without padding:
    // consecutive block ids, so the items of a head land on every XCD
    const long i = b - nfront;
    const long head = i % bh_n, rest = i / bh_n;
    const int f = (int)(rest / nco), c = (int)(rest % nco);
    const int fend = min(F, (f / bfr + 1) * bfr);
    relu_wide_output_item<DI>(q, o, cum, eps, F, N, bfr, nco, chunko, (head * F + f) * nco + c, lds, L, P,
                              &flags[(head * F + fend - 1) * 4], epoch, err, true);
    return;
  }
  const long bh = L.head_of_slot(b % bhp);
  const long u = b / bhp;  // unit: one item per head
  if (bh >= bh_n) return;
  const long bhf_n = bh_n * F;
  // the parts' records follow the F cumulative records of every head, their
  // flags the cumulative records' four row-block flags per frame
  float* parts = cum + (size_t)bhf_n * kReluWideRec;
  uint64_t* pflags = flags + bhf_n * 4;
  // which item this unit is: a summary part (frame f, part c), a prefix item
  // (row block c) or an output item (frame f, chunk c)
  int kind, f = 0, c;
  if (u < (long)np * F) {
    kind = 0, f = (int)(u / np), c = (int)(u % np);
  } else if (u < (long)np * F + 4) {
    kind = 1, c = (int)(u - (long)np * F);
  } else {
    const long r = u - (long)np * F - 4;
    kind = 2, f = (int)(r / nco), c = (int)(r % nco);
  }
  if (kind == 0) {
    relu_wide_summary_item<DI>(k, v, F, N, bh, f, np, c, parts, pflags, epoch, lds, L, P);
    return;
  }
  if (kind == 1) {
    relu_wide_prefix_item<DI>(cum, S0, z0, S_out, z_out, F, bfr, bh, c, np, parts, pflags, flags, epoch, err, P.rope(),
                              spread != 0);
    return;
  }
  const int fend = min(F, (f / bfr + 1) * bfr);
  relu_wide_output_item<DI>(q, o, cum, eps, F, N, bfr, nco, chunko, (bh * F + f) * nco + c, lds, L, P,
                            &flags[(bh * F + fend - 1) * 4], epoch, err, false);
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
    // (one-frame calls keep every item on its head's XCD: there the prefix
    // items' write-back sits on the whole call's critical path, 42.7 -> 50.6 us
    // at 20 heads x 3600 tokens, head dim 112)
    const int spread = a.bh % 8 != 0 && a.L.hg == 1 && a.F > 1;
    const long grid = (long)a.F * bhp * a.nc + bhp * 4 + (long)a.F * (spread ? a.bh : bhp) * a.nco;
    hipLaunchKernelGGL(relu_wide_fused_mfma<DI>, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.partial, a.S0, a.z0, a.S_out,
                       a.z_out, a.eps, a.bh, bhp, a.F, a.N, a.bfr, a.nco, a.chunko, a.nc, flags, epoch, err, a.L,
                       a.P, spread);
    return hipGetLastError();
  });
}

}  // namespace linscan
