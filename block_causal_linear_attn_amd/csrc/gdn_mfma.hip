// gdn_mfma.hip -- kernels and launchers of the bf16 MFMA frame-wise Gated
// DeltaNet scan (head dim 128), built from the work items in gdn_items.h.
//
// gdn_fused_mfma runs one call in a single launch.  Block ids start with the
// scan items (four 32-row blocks per head), followed by the streaming items
// in frame order: for each step j the gram items of frame j and the output
// items of frame j - L, with L chosen so that output items arrive about when
// their frame's state is ready instead of holding slots while they wait.
// Scan items wait for the gram records of each frame, output items wait for
// the four row blocks of their frame's state.  Every item a wait depends on
// is either dispatched earlier or, for the scan items, a gram item that can
// still find a free slot because scan items fill at most a quarter of the
// device's slots; the library only picks this kernel when that holds
// (gdn_fused_fits: 4*B*H within a quarter of the slots the device holds of
// it), which leaves room for other launches running alongside.  All
// items of a head share one XCD (block id equal to the head modulo 8), so
// records and per-frame states are read back from that XCD's L2 shortly
// after they are written, and the scan's frame-to-frame chain overlaps the
// HBM streaming.
#include "gdn_items.h"
#include "kernels.h"

#include <type_traits>

namespace linscan {

namespace {

template <int DI, bool TG, bool PRO>
__global__ __launch_bounds__(256, 2) void gdn_gram_mfma128(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ beta,
    uint8_t* __restrict__ rec, float c, float c2, int N, int nc, int chunk, TokLayout L, Prologue P) {
  __shared__ __align__(16) uint8_t lds[kGramLds + kGateLds + kPrologueLds];
  gdn_gram_item<DI, TG, PRO>(k, v, beta, rec, c, c2, N, nc, chunk, blockIdx.x, lds, L, P);
}

template <bool MULTI, int DI>
__global__ __launch_bounds__(256) void gdn_scan_mfma128(
    const uint8_t* __restrict__ rec, const float* __restrict__ alpha, const float* S0,
    uint16_t* __restrict__ states, float* S_out, long bh, int F, int nc, int rchunk) {
  __shared__ __align__(16) uint8_t lds[kScanLds];
  const long b = blockIdx.x;
  const long head = (b / 64) * 8 + (b % 8);
  if (head >= bh) return;  // whole workgroup leaves together
  gdn_scan_item<MULTI, false, kScanRB, DI>(rec, alpha, S0, states, S_out, head, (int)((b / 8) % 8) * kScanRB, F, nc,
                                           lds, nullptr, nullptr, 0, nullptr, 0, rchunk);
}

template <int DI, bool PRO>
__global__ __launch_bounds__(256, 2) void gdn_output_mfma128(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const uint16_t* __restrict__ states,
    int N, int nco, int chunk, TokLayout L, Prologue P) {
  __shared__ __align__(16) uint8_t lds[kOutLds];
  gdn_output_item<DI, PRO>(q, o, states, N, nco, chunk, blockIdx.x, lds, L, P);
}

constexpr int kFusedRB = GD / kGdnFusedRowBlocks;  // rows of S per fused scan item

constexpr int lds_max(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

// TG: `beta` holds per-token gates [B*H*F][N] (see gdn_gram_item).
// PRO: the per-token prologue may be on (see gdn_gram_item).
template <bool MULTI, int DI, bool TG, bool PRO>
__global__ __launch_bounds__(256, 2) void gdn_fused_mfma128(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, uint16_t* __restrict__ o,
    uint8_t* __restrict__ rec, uint16_t* __restrict__ states, const float* S0, float* S_out, float c,
    float c2, long bh_n, long bhp, int F, int N, int nc, int chunk, int nco, int chunko, int lag,
    uint64_t* __restrict__ gflags, uint64_t* __restrict__ sflags, uint64_t epoch, uint32_t* err, int rchunk,
    TokLayout L, Prologue P) {
  // one record per frame: the prefetching scan item; several: the chunk-summing one
  constexpr int kSL = MULTI ? scan_lds_bytes<kFusedRB>() : kScanPfLds;
  constexpr int LDS = lds_max(kGramLds + kGateLds + kPrologueLds, kSL, kOutLds);
  constexpr int NRB = kGdnFusedRowBlocks;
  static_assert(MULTI || kFusedRB == kScanPfRows, "prefetching scan items cover 32 rows");
  __shared__ __align__(16) uint8_t lds[LDS];
  const long b = blockIdx.x;
  const long nscan = (bhp / 8) * 8 * NRB;
  if (b < nscan) {
    // eight heads x NRB row blocks per group; a head's row blocks keep its XCD
    const long head = L.head_of_slot((b / (8 * NRB)) * 8 + (b % 8));
    if (head >= bh_n) return;
    if (MULTI)
      gdn_scan_item<MULTI, true, kFusedRB, DI>(rec, alpha, S0, states, S_out, head, (int)((b / 8) % NRB) * kFusedRB,
                                               F, nc, lds, gflags, sflags, epoch, err, 0, rchunk);
    else
      gdn_scan_item_pf<DI>(rec, alpha, S0, states, S_out, head, (int)((b / 8) % NRB) * kFusedRB, F, lds, gflags,
                           sflags, epoch, err, 1, rchunk);
    return;
  }
  const long s = b - nscan;
  const long bh = L.head_of_slot(s % bhp);
  const long u = s / bhp;  // unit: one item per head
  if (bh >= bh_n) return;
  // units of step j: the gram chunks of frame j (j < F), then the output
  // chunks of frame j - lag (j >= lag)
  long j, r;
  const long head_units = (long)lag * nc, mid_units = (long)(F - lag) * (nc + nco);
  int f, cidx;
  bool gram;
  if (u < head_units) {
    gram = true;
    f = (int)(u / nc);
    cidx = (int)(u % nc);
  } else if (u < head_units + mid_units) {
    j = lag + (u - head_units) / (nc + nco);
    r = (u - head_units) % (nc + nco);
    gram = r < nc;
    f = gram ? (int)j : (int)(j - lag);
    cidx = gram ? (int)r : (int)(r - nc);
  } else {
    r = u - head_units - mid_units;
    gram = false;
    f = F - lag + (int)(r / nco);
    cidx = (int)(r % nco);
  }
  if (gram) {
    gdn_gram_item<DI, TG, PRO>(k, v, beta, rec, c, c2, N, nc, chunk, (bh * F + f) * nc + cidx, lds, L, P);
    publish(&gflags[(bh * F + f) * nc + cidx], epoch);
  } else {
    wait_all(&sflags[(bh * F + f) * 8], NRB, epoch, err);
    gdn_output_item<DI, PRO>(q, o, states, N, nco, chunko, (bh * F + f) * nco + cidx, lds, L, P);
  }
}

// One call in a single launch for any number of heads: block ids run over
// the row-split gram items of every (frame, head, row block), then the scan
// items (four 32-row blocks per head), then the output items of every
// (frame, chunk, head), each phase head-minor with B*H padded to BHp (a
// multiple of 8) so that a head's items share one XCD.  Every wait is for
// items with lower block ids, which dispatch first, so the waits end
// whatever the number of heads.  For single-frame calls the scan has no
// frame chain and the phases overlap across heads; longer calls run the
// chain once all records are in.
template <int DI, bool TG, bool PRO>
__global__ __launch_bounds__(256, 2) void gdn_phased_mfma128(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, uint16_t* __restrict__ o,
    uint8_t* __restrict__ rec, uint16_t* __restrict__ states, const float* S0, float* S_out, float c,
    float c2, long bh_n, long bhp, int F, int N, int nco, int chunko, uint64_t* __restrict__ gflags,
    uint64_t* __restrict__ sflags, uint64_t epoch, uint32_t* err, int rchunk, TokLayout L, Prologue P) {
  constexpr int RB = kScanPfRows, NRB = GD / RB;
  constexpr int LDS = lds_max(kGramRowsLds + kGateLds + kPrologueLds, kScanPfLds, kOutLds);
  __shared__ __align__(16) uint8_t lds[LDS];
  const long b = blockIdx.x;
  const long ngram = bhp * F * 4, nscan = bhp * NRB;
  if (b < ngram) {
    const long bh = L.head_of_slot(b % bhp), r = b / bhp;  // r = f * 4 + row block
    if (bh >= bh_n) return;
    const long item = (bh * F + r / 4) * 4 + r % 4;
    gdn_gram_rows_item<DI, TG, PRO>(k, v, beta, rec, c, c2, N, item, lds, L, P);
    publish(&gflags[item], epoch);
    return;
  }
  if (b < ngram + nscan) {
    const long bs = b - ngram;
    const long head = L.head_of_slot(bs % bhp);
    if (head >= bh_n) return;
    gdn_scan_item_pf<DI>(rec, alpha, S0, states, S_out, head, (int)(bs / bhp) * RB, F, lds, gflags, sflags, epoch,
                         err, 4, rchunk);
    return;
  }
  const long bo = b - ngram - nscan;
  const long bh = L.head_of_slot(bo % bhp), r = bo / bhp;  // r = f * nco + chunk
  if (bh >= bh_n) return;
  const int f = (int)(r / nco);
  wait_all(&sflags[(bh * F + f) * 8], NRB, epoch, err);
  gdn_output_item<DI, PRO>(q, o, states, N, nco, chunko, bh * F * nco + r, lds, L, P);
}

// Single-frame calls (the chunk-causal denoising step): one item per (head,
// 64-row block) does the gram rows, the state update of its rows and one of
// the frame's kStepChunks output chunks (gdn_step_item); block id b < 2 bhp
// serves head slot (b / 16) * 8 + b % 8 and row block (b / 8) % 2, so a head's
// two items share an XCD and lie 8 block ids apart.  The output-only items of
// the other chunks follow with the same mapping: they wait for the state
// items, which have lower block ids.
template <int DI, bool TG, bool PRO>
__global__ __launch_bounds__(256, 2) void gdn_step_mfma128(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ alpha, const float* __restrict__ beta, uint16_t* __restrict__ o,
    uint8_t* __restrict__ rec, uint16_t* __restrict__ states, const float* S0, float* S_out, float c,
    float c2, long bh_n, long bhp, int N, int chunko, uint64_t* __restrict__ gflags, uint64_t* __restrict__ sflags,
    uint64_t epoch, uint32_t* err, int rchunk, TokLayout L, Prologue P) {
  constexpr int LDS = lds_max(kStepLds, kOutLds, 0);
  __shared__ __align__(16) uint8_t lds[LDS];
  constexpr int NO = kStepChunks - kStepItems;  // output-only items per head
  const long b = blockIdx.x, nstep = bhp * kStepItems;
  if (b < nstep) {
    const long head = L.head_of_slot((b / (8 * kStepItems)) * 8 + b % 8);
    if (head >= bh_n) return;  // a padded slot: its partner is padded too
    gdn_step_item<DI, TG, PRO>(q, k, v, alpha, beta, o, rec, states, S0, S_out, c, c2, N, chunko, head,
                               (int)((b / 8) % kStepItems), gflags, sflags, epoch, err, rchunk, lds, L, P);
    return;
  }
  const long bo = b - nstep;
  const long head = L.head_of_slot((bo / (8 * NO)) * 8 + bo % 8);
  if (head >= bh_n) return;
  gdn_output_item<DI, PRO>(q, o, states, N, kStepChunks, chunko, head * kStepChunks + kStepItems + (bo / 8) % NO,
                           lds, L, P, &sflags[head * 8], kStepItems, epoch, err);
}

}  // namespace
// The prologue does some work (the kernels take it as a template switch).
static bool pro_on(const Prologue& P) { return P.on_k() || P.on_q(); }

// Head dims with an MFMA path: 128, and 112 (the items run on 128 dims with
// the last 16 zero).
bool gdn_has_mfma(int D, int dtype) { return dtype == DT_BF16 && (D == GD || D == 112); }

// Instantiate `body` with the head dim as a compile-time constant.
template <typename Body>
hipError_t with_head_dim(int D, Body body) {
  if (D == GD) return body(std::integral_constant<int, GD>());
  if (D == 112) return body(std::integral_constant<int, 112>());
  return hipErrorInvalidValue;
}

hipError_t launch_gdn_phased_mfma(const ScanArgs& a, long bhp, uint64_t* gflags, uint64_t* sflags, uint64_t epoch,
                                  uint32_t* err, hipStream_t st) {
  const long grid = bhp * (long)a.F * 4 + bhp * (GD / 32) + bhp * (long)a.F * a.nco;
  const float* gates = a.tg ? a.gate : a.beta;
  return with_head_dim(a.D, [&](auto di) {
    constexpr int DI = decltype(di)::value;
    if (a.tg && pro_on(a.P)) return hipErrorInvalidValue;  // not instantiated: no entry point combines them
    auto kern = a.tg ? gdn_phased_mfma128<DI, true, false>
                     : (pro_on(a.P) ? gdn_phased_mfma128<DI, false, true> : gdn_phased_mfma128<DI, false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, a.alpha, gates, (uint16_t*)a.o, (uint8_t*)a.partial,
                       (uint16_t*)a.states, a.S0, a.S_out, a.c, a.c2, a.bh, bhp, a.F, a.N, a.nco, a.chunko, gflags,
                       sflags, epoch, err, a.rchunk, a.L, a.P);
    return hipGetLastError();
  });
}

hipError_t launch_gdn_step_mfma(const ScanArgs& a, long bhp, uint64_t* gflags, uint64_t* sflags, uint64_t epoch,
                                uint32_t* err, hipStream_t st) {
  if (a.F != 1 || a.N <= 0 || a.nco != kStepChunks) return hipErrorInvalidValue;
  const long grid = bhp * kStepChunks;
  const float* gates = a.tg ? a.gate : a.beta;
  return with_head_dim(a.D, [&](auto di) {
    constexpr int DI = decltype(di)::value;
    if (a.tg && pro_on(a.P)) return hipErrorInvalidValue;  // not instantiated: no entry point combines them
    auto kern = a.tg ? gdn_step_mfma128<DI, true, false>
                     : (pro_on(a.P) ? gdn_step_mfma128<DI, false, true> : gdn_step_mfma128<DI, false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, a.alpha, gates, (uint16_t*)a.o, (uint8_t*)a.partial,
                       (uint16_t*)a.states, a.S0, a.S_out, a.c, a.c2, a.bh, bhp, a.N, a.chunko, gflags, sflags,
                       epoch, err, a.rchunk, a.L, a.P);
    return hipGetLastError();
  });
}

hipError_t launch_gdn_gram_mfma(int D, const void* k, const void* v, const float* gates, bool tg, void* rec,
                                float c, float c2, long bhf, int N, int nc, int chunk, const TokLayout& L,
                                const Prologue& P, hipStream_t st) {
  return with_head_dim(D, [&](auto di) {
    constexpr int DI = decltype(di)::value;
    if (tg && pro_on(P)) return hipErrorInvalidValue;
    auto kern = tg ? gdn_gram_mfma128<DI, true, false>
                   : (pro_on(P) ? gdn_gram_mfma128<DI, false, true> : gdn_gram_mfma128<DI, false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)(bhf * nc)), dim3(256), 0, st, (const uint16_t*)k, (const uint16_t*)v,
                       gates, (uint8_t*)rec, c, c2, N, nc, chunk, L, P);
    return hipGetLastError();
  });
}

hipError_t launch_gdn_scan_mfma(int D, const void* rec, const float* alpha, const float* S0,
                                void* states, float* S_out, long bh, int F, int nc, int rchunk, hipStream_t st) {
  const long groups = (bh + 7) / 8;  // eight heads x eight row blocks per group of 64 workgroups
  return with_head_dim(D, [&](auto di) {
    constexpr int DI = decltype(di)::value;
    if (nc == 1)
      hipLaunchKernelGGL((gdn_scan_mfma128<false, DI>), dim3((unsigned)(groups * 64)), dim3(256), 0, st,
                         (const uint8_t*)rec, alpha, S0, (uint16_t*)states, S_out, bh, F, nc, rchunk);
    else
      hipLaunchKernelGGL((gdn_scan_mfma128<true, DI>), dim3((unsigned)(groups * 64)), dim3(256), 0, st,
                         (const uint8_t*)rec, alpha, S0, (uint16_t*)states, S_out, bh, F, nc, rchunk);
    return hipGetLastError();
  });
}

hipError_t launch_gdn_output_mfma(int D, const void* q, void* o, const void* states, long bhf,
                                  int N, int nco, int chunk, const TokLayout& L, const Prologue& P, hipStream_t st) {
  return with_head_dim(D, [&](auto di) {
    constexpr int DI = decltype(di)::value;
    auto kern = pro_on(P) ? gdn_output_mfma128<DI, true> : gdn_output_mfma128<DI, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(bhf * nco)), dim3(256), 0, st,
                       (const uint16_t*)q, (uint16_t*)o, (const uint16_t*)states, N, nco, chunk, L, P);
    return hipGetLastError();
  });
}

// The fused kernel instance a call with these switches runs (nc > 1: MULTI).
static const void* gdn_fused_kernel(int D, bool tg, bool pro, int nc) {
  const void* k = nullptr;
  (void)with_head_dim(D, [&](auto di) {
    constexpr int DI = decltype(di)::value;
    auto kern = nc == 1 ? (tg ? gdn_fused_mfma128<false, DI, true, false>
                              : (pro ? gdn_fused_mfma128<false, DI, false, true> : gdn_fused_mfma128<false, DI, false, false>))
                        : (tg ? gdn_fused_mfma128<true, DI, true, false>
                              : (pro ? gdn_fused_mfma128<true, DI, false, true> : gdn_fused_mfma128<true, DI, false, false>));
    k = (const void*)kern;
    return hipSuccess;
  });
  return k;
}

bool gdn_fused_fits(int D, bool tg, bool pro, int nc, long bh) {
  const void* k = gdn_fused_kernel(D, tg, pro, nc);
  return k != nullptr && bh * kGdnFusedRowBlocks * 4 <= device_slots(k);
}

hipError_t launch_gdn_fused_mfma(const ScanArgs& a, long bhp, uint64_t* gflags, uint64_t* sflags,
                                 uint64_t epoch, uint32_t* err, hipStream_t st) {
  const long grid = bhp * kGdnFusedRowBlocks + bhp * a.F * (a.nc + a.nco);
  const float* gates = a.tg ? a.gate : a.beta;
  return with_head_dim(a.D, [&](auto di) {
    constexpr int DI = decltype(di)::value;
    if (a.tg && pro_on(a.P)) return hipErrorInvalidValue;
    const bool pro = pro_on(a.P);
    auto kern = a.nc == 1
                    ? (a.tg ? gdn_fused_mfma128<false, DI, true, false>
                            : (pro ? gdn_fused_mfma128<false, DI, false, true> : gdn_fused_mfma128<false, DI, false, false>))
                    : (a.tg ? gdn_fused_mfma128<true, DI, true, false>
                            : (pro ? gdn_fused_mfma128<true, DI, false, true> : gdn_fused_mfma128<true, DI, false, false>));
    // gram items lead the output items by three rounds of the resident slots
    // (as in the ReLU launch): the 720p 60 s call (B1 H24, lag 12 -> 28) ran
    // 1141 -> 1114 us, against 1.25 rounds.  An output item's state needs the
    // records of every frame of its chunk (reversed scan): lag >= rchunk
    // keeps those gram items at lower block ids.
    const int lag = fused_lag(device_slots((const void*)kern) - bhp * kGdnFusedRowBlocks, bhp * (a.nc + a.nco),
                              a.rchunk > 0 ? a.rchunk : 1, a.F, 3.0);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, a.alpha, gates, (uint16_t*)a.o, (uint8_t*)a.partial,
                       (uint16_t*)a.states, a.S0, a.S_out, a.c, a.c2, a.bh, bhp, a.F, a.N, a.nc, a.chunk, a.nco,
                       a.chunko, lag, gflags, sflags, epoch, err, a.rchunk, a.L, a.P);
    return hipGetLastError();
  });
}

}  // namespace linscan
