// relu_mfma.hip -- the single-launch bf16 MFMA ReLU linear-attention scan
// (head dims 32 and 64), built from the work items in relu_items.h.
//
// relu_fused_mfma runs one call in a single launch: summary items of each
// frame interleaved with output items of earlier frames.  An output item waits (bounded spin)
// until the summaries of its frame's block and every earlier frame of its
// head are published; since every item it waits on has a lower block id and
// block ids dispatch in order, those items are running or done, so the wait
// ends.  Every item of a head gets block ids equal to the head modulo 8, so
// they share one XCD and exchange partials through its L2.  With PAIR the
// items run a pair of heads of dim 32 as one head of dim 64 (block-diagonal
// state), for layouts where the pair shares every 128-byte token segment.
#include "relu_items.h"
#include "kernels.h"
#include "sync.h"

#include <type_traits>

namespace linscan {

namespace {

// Block ids run over steps j = 0, 1, ...: step j holds the summary items of
// frame j (nc per head, one per token chunk of the frame) and then the output
// items of frame j - lag (one per head and token chunk), so summaries of later frames
// stream while earlier frames' outputs are written.  lag >= block_frames
// keeps every summary an output item waits for at a lower block id.  Within
// a step items are head-minor with B*H padded to BHp (a multiple of 8);
// padding items leave at once.
// Head dim 32 with RMSNorm (PRO 1) is held to three workgroups per CU (at
// most 168 registers, 164 used), as without the prologue: with two, its
// fp64 load stage had too few waves to hide behind (10-frame call at H70
// N3600: 168 -> 143 us, 117 us without the prologue).
template <int D, int PRO, bool PAIR = false>
__global__ __launch_bounds__(256, (D == 32 && PRO == 1) ? 3 : 2) void relu_fused_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ partial, float* __restrict__ init, const float* S0,
    const float* z0, float* S_out, float* z_out, float eps, long bh_n, long bhp, int F, int N, int bfr,
    int nc, int chunk, int nco, int chunko, int lag, uint64_t* __restrict__ flags, uint64_t epoch, uint32_t* err,
    TokLayout L, Prologue P) {
  // (each item keeps the prologue's D weights after its own LDS)
  constexpr int LDS = (relu_summary_lds_bytes<D>() > relu_output_lds_bytes<D>() ? relu_summary_lds_bytes<D>()
                                                                                 : relu_output_lds_bytes<D>()) +
                      D * 4;
  __shared__ __align__(16) uint8_t lds[LDS];
  const long b = blockIdx.x;
  const long bh = L.head_of_slot(b % bhp);
  const long u = b / bhp;  // unit: one item per head
  if (bh >= bh_n) return;
  const long head_units = (long)lag * nc, mid_units = (long)(F - lag) * (nc + nco);
  bool summary;
  int f, c;
  if (u < head_units) {
    summary = true;
    f = (int)(u / nc);
    c = (int)(u % nc);
  } else if (u < head_units + mid_units) {
    const long j = lag + (u - head_units) / (nc + nco), r = (u - head_units) % (nc + nco);
    summary = r < nc;
    f = summary ? (int)j : (int)(j - lag);
    c = summary ? (int)r : (int)(r - nc);
  } else {
    const long r = u - head_units - mid_units;
    summary = false;
    f = F - lag + (int)(r / nco);
    c = (int)(r % nco);
  }
  if (summary) {
    relu_summary_item<D, PRO, PAIR>(k, v, partial, S0, z0, init, F, N, nc, chunk, (bh * F + f) * nc + c, lds, L,
                                    P);
    publish(&flags[(bh * F + f) * nc + c], epoch);
    return;
  }
  const int fend = min(F, (f / bfr + 1) * bfr);
  wait_all(&flags[bh * F * nc], fend * nc, epoch, err);
  relu_output_item<D, PRO, PAIR>(q, o, partial, init, S_out, z_out, eps, F, N, nc, bfr, nco, chunko,
                                 (bh * F + f) * nco + c, lds, L, P);
}

}  // namespace
bool relu_has_mfma(int D, int dtype) { return dtype == DT_BF16 && (D == 32 || D == 64 || relu_wide_mfma(D, dtype)); }

hipError_t launch_relu_fused_mfma(const ScanArgs& a, long bhp, uint64_t* flags, uint64_t epoch,
                                  uint32_t* err, hipStream_t st) {
  const long grid = (long)a.F * bhp * (a.nc + a.nco);
  // the prologue's instantiation: 0 none, 1 RMSNorm, 2 with the rotary embedding
  const int pro = a.P.rope() ? 2 : (a.P.wq != nullptr || a.P.wk != nullptr) ? 1 : 0;
  auto pick = [&](auto d) {
    constexpr int D = decltype(d)::value;
    return pro == 2 ? relu_fused_mfma<D, 2> : pro == 1 ? relu_fused_mfma<D, 1> : relu_fused_mfma<D, 0>;
  };
  auto run = [&](auto kern) {
    // three rounds of the resident slots: at B1 H70 D32 N3600 one 10-frame call
    // 120.9 -> 118.0 us (lag 5 -> 10), 24 heads x 60 frames 266 -> 257 us, the
    // 480p call (H70 F21 N1560) 117.4 -> 118.6 us, against 1.25 rounds
    const int lag = fused_lag(device_slots((const void*)kern), bhp * (a.nc + a.nco), a.bfr, a.F, 3.0);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.partial, a.init, a.S0, a.z0, a.S_out, a.z_out, a.eps,
                       a.bh, bhp, a.F, a.N, a.bfr, a.nc, a.chunk, a.nco, a.chunko, lag, flags, epoch, err, a.L,
                       a.P);
    return hipGetLastError();
  };
  if (a.pair) {  // head pairs of dim 32 as heads of dim 64 (no prologue)
    if (a.D != 64 || pro != 0) return hipErrorInvalidValue;
    return run(relu_fused_mfma<64, 0, true>);
  }
  if (a.D == 32) return run(pick(std::integral_constant<int, 32>{}));
  if (a.D == 64) return run(pick(std::integral_constant<int, 64>{}));
  return hipErrorInvalidValue;
}

}  // namespace linscan
