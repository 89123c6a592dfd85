// linscan_api.cpp -- the C ABI of liblinscan: argument checks, workspace
// planning and kernel dispatch.  Every check runs before the first launch, so
// a rejected call enqueues nothing and touches no output.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <random>
#include <string>
#include <vector>

#include "../../include/linscan.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

ls_status fail(ls_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ls_status ok() { return LS_OK; }

bool supported_d(int D) {
  return D == 16 || D == 32 || D == 48 || D == 64 || D == 80 || D == 96 || D == 112 || D == 128;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspaces start with a 256-byte header whose first word is the fault word.
constexpr size_t kHeaderBytes = 256;

// Epochs tag the flags of one launch: a 64-bit sequence that starts from a
// random value per process, so flags left in a reused workspace never match.
uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{0};
  static std::once_flag once;
  std::call_once(once, [] {
    std::random_device rd;
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    counter.store(((((uint64_t)rd()) << 32) ^ rd() ^ (t * 0x9e3779b97f4a7c15ull)) | 1ull);
  });
  uint64_t e = counter.fetch_add(1);
  return e ? e : counter.fetch_add(1);
}

struct Dims {
  long bh = 0;      // B*H
  long bhf = 0;     // B*H*F
  size_t elems = 0; // B*H*F*N*D
  size_t esize = 0; // bytes per token element
};

ls_status check_shape(const ls_shape* s, Dims* d) {
  if (!s) return fail(LS_ERR_NULL_POINTER, "shape is NULL");
  if (s->B < 0 || s->H < 0 || s->F < 0 || s->N < 0)
    return fail(LS_ERR_BAD_SHAPE, "negative dimension (B=%d H=%d F=%d N=%d)", s->B, s->H, s->F, s->N);
  if (!supported_d(s->D))
    return fail(LS_ERR_UNSUPPORTED_HEAD_DIM, "head dim D=%d not in {16,32,48,64,80,96,112,128}", s->D);
  if (s->dtype != LS_DTYPE_FP32 && s->dtype != LS_DTYPE_BF16)
    return fail(LS_ERR_BAD_DTYPE, "dtype %d is neither LS_DTYPE_FP32 nor LS_DTYPE_BF16", s->dtype);
  // sizes must stay well inside 2^62 elements and 2^31 workgroups
  const double el = (double)s->B * s->H * s->F * s->N * s->D;
  const double bhf = (double)s->B * s->H * s->F;
  if (el > 4.0e18 || bhf > 1.0e9)
    return fail(LS_ERR_BAD_SHAPE, "shape too large (B*H*F*N*D = %.3g)", el);
  d->bh = (long)s->B * s->H;
  d->bhf = d->bh * s->F;
  d->elems = (size_t)d->bhf * s->N * s->D;
  d->esize = s->dtype == LS_DTYPE_BF16 ? 2 : 4;
  return LS_OK;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// [a, a+na) and [b, b+nb) overlap (empty ranges never do)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// The layout of the token tensors: packed [B][H][F][N][D] when `st` is NULL,
// else the caller's element strides (D contiguous).  Strides must keep every
// token row 16-byte aligned and map distinct (b, h, f, n) to disjoint rows:
// sorted by stride, the dims with more than one index must nest (each stride
// at least the previous stride times the previous extent, the smallest at
// least D).  *span = bytes from the base to the end of the last row.
ls_status token_layout(const ls_shape* s, const Dims& d, const ls_strides* st, linscan::TokLayout* L,
                       size_t* span) {
  *L = linscan::TokLayout::packed(s->H, s->F, s->N, s->D);
  *span = d.elems * d.esize;
  if (!st || d.elems == 0) return LS_OK;
  const long long str[4] = {st->batch, st->head, st->frame, st->token};
  const long long ext[4] = {s->B, s->H, s->F, s->N};
  int idx[4] = {0, 1, 2, 3};
  for (int i = 0; i < 4; ++i) {
    if (str[i] < 0 || str[i] > (1LL << 40))
      return fail(LS_ERR_BAD_PARAM, "stride %lld out of range [0, 2^40]", str[i]);
    if ((str[i] * (long long)d.esize) % 16 != 0)
      return fail(LS_ERR_MISALIGNED, "stride %lld elements is not a multiple of 16 bytes", str[i]);
  }
  for (int i = 1; i < 4; ++i)  // insertion sort of the dims by stride
    for (int j = i; j > 0 && str[idx[j]] < str[idx[j - 1]]; --j) {
      const int t = idx[j];
      idx[j] = idx[j - 1];
      idx[j - 1] = t;
    }
  long long need = s->D;  // the next stride that keeps rows disjoint
  double last = 0.0;      // element offset of the last row
  for (int i = 0; i < 4; ++i) {
    const int k = idx[i];
    if (ext[k] <= 1) continue;
    if (str[k] < need)
      return fail(LS_ERR_BAD_PARAM, "strides overlap rows: stride %lld < %lld", str[k], need);
    need = str[k] * ext[k];
    last += (double)str[k] * (double)(ext[k] - 1);
  }
  if ((last + s->D) * d.esize > 4.0e18) return fail(LS_ERR_BAD_SHAPE, "strided span too large");
  L->sb = st->batch;
  L->sh = st->head;
  L->sf = st->frame;
  L->sn = st->token;
  // heads adjacent in a token row with rows that do not fill whole 128-byte
  // lines share lines with their neighbours: group them onto one XCD, when
  // there are enough groups (4 per XCD) to keep the XCDs evenly loaded
  const long long row = (long long)s->D * d.esize;
  if (s->H > 1 && st->head == s->D && row % 128 != 0) {
    long long a = row, b = 128;
    while (b) {
      const long long t = a % b;
      a = b;
      b = t;
    }
    const int hg = (int)(128 / a);
    if (d.bh / hg >= 32) L->hg = hg;
  }
  *span = (size_t)((last + s->D) * d.esize);
  return LS_OK;
}

// The per-token prologue of a call (nullptr: none); `gdn` allows the GDN-only
// parts (ReLU, L2 of keys).  Weights are [H][D] fp32, 16-byte aligned.
// The prologue's read-only buffers (weights, rotary tables), for the
// overlap checks against outputs.
struct ProBufs {
  const void* p[4] = {nullptr, nullptr, nullptr, nullptr};
  size_t n[4] = {0, 0, 0, 0};
};

ls_status prologue_of(const ls_prologue* pr, const ls_shape* s, bool gdn, linscan::Prologue* P, ProBufs* bufs) {
  *P = linscan::Prologue();
  *bufs = ProBufs();
  if (!pr) return LS_OK;
  if (pr->relu != 0 && pr->relu != 1) return fail(LS_ERR_BAD_PARAM, "prologue relu must be 0 or 1");
  if (pr->l2_keys != 0 && pr->l2_keys != 1) return fail(LS_ERR_BAD_PARAM, "prologue l2_keys must be 0 or 1");
  if (!gdn && (pr->relu || pr->l2_keys))
    return fail(LS_ERR_BAD_PARAM, "the ReLU scan applies its own feature map: prologue relu and l2_keys must be 0");
  if ((pr->q_weight || pr->k_weight) && (!(pr->eps > 0.0f) || !isfinite(pr->eps)))
    return fail(LS_ERR_BAD_PARAM, "prologue eps=%g must be finite and > 0", (double)pr->eps);
  if (misaligned(pr->q_weight) || misaligned(pr->k_weight))
    return fail(LS_ERR_MISALIGNED, "prologue weights must be 16-byte aligned");
  const size_t w_bytes = (size_t)s->H * s->D * sizeof(float);
  bufs->p[0] = pr->q_weight, bufs->n[0] = pr->q_weight ? w_bytes : 0;
  bufs->p[1] = pr->k_weight, bufs->n[1] = pr->k_weight ? w_bytes : 0;
  if (pr->rope_frame || pr->rope_token) {
    const int half = s->D / 2, pf = pr->rope_frame_pairs;
    if (pf < 0 || pf > half || pf % 4 != 0)
      return fail(LS_ERR_BAD_PARAM, "rope_frame_pairs=%d must be a multiple of 4 in [0, D/2=%d]", pf, half);
    if (pf > 0 && !pr->rope_frame) return fail(LS_ERR_NULL_POINTER, "rope_frame is NULL but rope_frame_pairs=%d", pf);
    if (pf < half && !pr->rope_token)
      return fail(LS_ERR_NULL_POINTER, "rope_token is NULL but %d pairs turn by token", half - pf);
    if (pr->rope_frame_offset < 0 || (pf > 0 && (long long)pr->rope_frame_offset + s->F > pr->rope_frames))
      return fail(LS_ERR_BAD_PARAM, "rope_frame_offset=%d + F=%d exceeds rope_frames=%lld", pr->rope_frame_offset,
                  s->F, pr->rope_frames);
    if (misaligned(pr->rope_frame) || misaligned(pr->rope_token))
      return fail(LS_ERR_MISALIGNED, "rotary tables must be 16-byte aligned");
    if (pf > 0) {
      P->rf = pr->rope_frame;
      bufs->p[2] = pr->rope_frame, bufs->n[2] = (size_t)pr->rope_frames * pf * 2 * sizeof(float);
    }
    if (pf < half) {
      P->rt = pr->rope_token;
      bufs->p[3] = pr->rope_token, bufs->n[3] = (size_t)s->N * (half - pf) * 2 * sizeof(float);
    }
    P->rpf = pf;
    P->roff = pr->rope_frame_offset;
  }
  P->wq = pr->q_weight;
  P->wk = pr->k_weight;
  P->eps = pr->eps;
  P->relu = pr->relu;
  P->l2 = pr->l2_keys;
  return LS_OK;
}

// Token chunking: enough workgroups to fill 256 CUs several times over, with
// chunks of at least `min_chunk` tokens (a multiple of `quantum`).
void plan_chunks(long frames, int N, int target_wg, int min_chunk, int quantum, int* nc, int* chunk) {
  if (N <= 0 || frames <= 0) {
    *nc = 1;
    *chunk = N > 0 ? N : 1;
    return;
  }
  long want = (target_wg + frames - 1) / frames;
  long max_nc = N / min_chunk;
  if (max_nc < 1) max_nc = 1;
  if (want < 1) want = 1;
  if (want > max_nc) want = max_nc;
  int ch = (int)((N + want - 1) / want);
  ch = (ch + quantum - 1) / quantum * quantum;
  *chunk = ch;
  *nc = (N + ch - 1) / ch;
}

struct ReluPlan {
  bool mfma, fused, wide;
  int nc, chunk, nco, chunko;
  size_t partial_off, init_off, flags_off, bytes;
};

ReluPlan relu_plan(const ls_shape* s, const Dims& d) {
  ReluPlan p;
  p.mfma = linscan::relu_has_mfma(s->D, s->dtype);
  p.fused = p.mfma;  // one launch: summary items then output items
  p.wide = linscan::relu_wide_mfma(s->D, s->dtype);
  // summary: whole frames per item unless there are too few frames to fill
  // the chip (the fused launch always uses whole frames); each output item
  // sums the partials of its frame and all earlier ones, so fewer partials
  // per frame keep that read small
  if (p.fused) {
    p.nc = 1;
    p.chunk = s->N > 0 ? s->N : 1;
    // wide heads: a frame's summary is split over up to 8 parts (runs of at
    // least 6 tiles of 64 tokens) while all parts of all frames still fit in
    // the device's 512 resident slots of this kernel (2 per CU), so that few
    // heads or frames still fill the chip; part 0 adds the others' sums
    if (p.wide) {
      const long tiles = (s->N + 63) / 64;
      while (p.nc < 8 && (p.nc + 1) * d.bhf <= 512 && tiles >= 6 * (p.nc + 1)) ++p.nc;
    } else {
      // narrow heads: up to 4 token chunks of at least 512 tokens per frame
      // while the summary items stay within one per CU (the rollout's
      // one-frame calls); output items then sum nc partials per frame
      while (p.nc < 4 && (p.nc + 1) * d.bhf <= 256 && s->N / (p.nc + 1) >= 512) ++p.nc;
      if (p.nc > 1) {
        p.chunk = (s->N + p.nc - 1) / p.nc;
        p.chunk = (p.chunk + 63) / 64 * 64;
        p.nc = (s->N + p.chunk - 1) / p.chunk;
      }
    }
  } else {
    plan_chunks(d.bhf, s->N, 512, 512, 64, &p.nc, &p.chunk);
  }
  // output items: wide heads aim at about 1000 (about two per resident slot,
  // measured best at 20 heads x 10 frames x 3600 tokens) and take chunks down
  // to 128 tokens when there are few frames (one frame: 52 -> 45 us); head
  // dim 64 aims at about 512, since each output item sums the partials of
  // every earlier frame (35 heads x 10 frames x 3600 tokens: 166 -> 153 us);
  // head dim 32 at about 2800 (70 heads x 10 frames x 3600 tokens: four
  // chunks per frame, 118.8 -> 117.7 us against three)
  plan_chunks(d.bhf, s->N, p.wide ? 1000 : s->D == 64 ? 512 : 2800, p.wide ? 128 : 512, 128, &p.nco, &p.chunko);
  // wide heads keep one cumulative record per frame, 128 dims wide, then one
  // record per summary part, and no init copy; their flags: four row blocks
  // per cumulative record, then one per part
  const size_t out = p.wide ? (size_t)128 * 128 + 128 : (size_t)s->D * s->D + s->D;
  const size_t recs = p.wide ? (size_t)d.bhf * (p.nc + 1) : (size_t)d.bhf * p.nc;
  const size_t nflags = p.wide ? (size_t)d.bhf * (p.nc + 4) : (size_t)d.bhf * p.nc;
  p.partial_off = kHeaderBytes;
  p.init_off = align_up(p.partial_off + recs * out * sizeof(float), 256);
  p.flags_off = align_up(p.init_off + (p.wide ? 0 : (size_t)d.bh * out * sizeof(float)), 256);
  p.bytes = align_up(p.flags_off + (p.fused ? nflags * sizeof(uint64_t) : 0), 256);
  return p;
}

struct GdnPlan {
  bool mfma, fused, phased, step;
  int nc, chunk, nco, chunko;
  size_t partial_off, states_off, gflags_off, sflags_off, bytes;
};

// fused_ok: the device has room for the fused launch's resident scan items
// (the caller checks gdn_fused_fits; workspace sizes cover both answers).
GdnPlan gdn_plan(const ls_shape* s, const Dims& d, bool fused_ok) {
  GdnPlan p;
  p.mfma = linscan::gdn_has_mfma(s->D, s->dtype);
  // one launch with the scan items alongside the streaming items when there
  // are frames to overlap and the scan items take at most a quarter of the
  // device's workgroup slots (B*H <= 32 on an MI355X): they stay resident
  // waiting for gram items that come later in dispatch order, which need
  // free slots even if calls on other streams occupy the rest (see the header)
  p.fused = p.mfma && fused_ok && d.bh * linscan::kGdnFusedRowBlocks <= 128 && s->F >= 2 && s->N > 0;
  // every other MFMA call with tokens: gram, scan and output phases in one
  // launch
  p.phased = p.mfma && !p.fused && s->N > 0;
  // a chunk's G/U partials are 8 D^2 bytes: keep chunks long enough that they
  // stay small next to the chunk's own key/value bytes
  if (p.phased) {  // row-split gram items: one record per frame
    p.nc = 1;
    p.chunk = s->N;
  } else {
    plan_chunks(d.bhf, s->N, 1024, 1024, 64, &p.nc, &p.chunk);
  }
  // output items: about 2048; one-frame calls run the step launch, whose
  // items output the frame in four chunks
  plan_chunks(d.bhf, s->N, 2048, 64, 64, &p.nco, &p.chunko);
  p.step = p.phased && s->F == 1;
  if (p.step) {
    p.nco = 4;
    p.chunko = (s->N + 3) / 4;
  }
  // records and per-frame states of the MFMA kernels always cover 128 dims
  const size_t Dw = p.mfma ? 128 : (size_t)s->D;
  const size_t dd = Dw * Dw;
  p.partial_off = kHeaderBytes;
  p.states_off = align_up(p.partial_off + (size_t)d.bhf * p.nc * 2 * dd * sizeof(float), 256);
  const bool flags = p.fused || p.phased;
  // per-frame states: fp32 for the generic kernels, bf16 hi + lo for the MFMA ones
  p.gflags_off = align_up(p.states_off + (size_t)d.bhf * dd * sizeof(float), 256);
  const size_t gflags_per_frame = p.phased ? 4 : (size_t)p.nc;
  p.sflags_off = align_up(p.gflags_off + (flags ? (size_t)d.bhf * gflags_per_frame * sizeof(uint64_t) : 0), 256);
  p.bytes = align_up(p.sflags_off + (flags ? (size_t)d.bhf * 8 * sizeof(uint64_t) : 0), 256);
  return p;
}

ls_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return LS_OK;
}

// ---- optional per-kernel event timing (diagnostics) ----------------------
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
constexpr size_t kMaxProfRecords = 65536;
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof_records;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (which enqueues one kernel on `st`) between two events when
// profiling is on.
template <typename Fn>
hipError_t timed(const char* name, hipStream_t st, Fn&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_on && g_prof_records.size() < kMaxProfRecords) {
      a = prof_event();
      b = prof_event();
    }
  }
  if (a && b) (void)hipEventRecord(a, st);
  hipError_t e = launch();
  if (a && b) {
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_records.push_back({name, a, b});
  }
  return e;
}

// Head dim 32 in bf16 with an even head count may run as pairs of heads of
// dim 64 (when the layout puts a pair in one 128-byte row segment): the
// shape and dims of that launch.
bool relu_pair_shape(const ls_shape* s) {
  return s->D == 32 && s->dtype == LS_DTYPE_BF16 && s->H % 2 == 0 && linscan::relu_has_mfma(64, linscan::DT_BF16);
}
void relu_pair_dims(const ls_shape* s, const Dims& d, ls_shape* ps, Dims* pd) {
  *ps = *s;
  ps->H = s->H / 2;
  ps->D = 64;
  *pd = d;
  pd->bh = d.bh / 2;
  pd->bhf = d.bhf / 2;
}

}  // namespace

namespace linscan {

ls_status set_error(ls_status st, const char* msg) { return fail(st, "%s", msg); }

ls_status gdn_forward_plain(const ls_shape* s, float key_scale, const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, void* o, const float* state_in, float* state_out,
                            void* workspace, size_t workspace_bytes, uint32_t* fault, void* stream);

}  // namespace linscan

extern "C" {

int ls_version(void) { return LINSCAN_VERSION; }

ls_status ls_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = true;
  return LS_OK;
}

int ls_profile_end(ls_kernel_stat* stats, int max_stats) {
  std::vector<ProfRecord> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = false;
    recs.swap(g_prof_records);
  }
  std::vector<ls_kernel_stat> agg;
  int rc = 0;
  for (const ProfRecord& r : recs) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      rc = -1;
    size_t i = 0;
    while (i < agg.size() && strcmp(agg[i].name, r.name) != 0) ++i;
    if (i == agg.size()) {
      ls_kernel_stat s0;
      memset(&s0, 0, sizeof(s0));
      snprintf(s0.name, sizeof(s0.name), "%s", r.name);
      agg.push_back(s0);
    }
    agg[i].launches += 1;
    agg[i].total_ms += ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (const ProfRecord& r : recs) {
      g_prof_pool.push_back(r.start);
      g_prof_pool.push_back(r.stop);
    }
  }
  for (size_t i = 0; i < agg.size() && (int)i < max_stats; ++i) stats[i] = agg[i];
  return rc < 0 ? -1 : (int)agg.size();
}

const char* ls_last_error(void) { return g_last_error.c_str(); }

const char* ls_status_string(ls_status st) {
  switch (st) {
    case LS_OK: return "ok";
    case LS_ERR_NULL_POINTER: return "a required pointer is NULL";
    case LS_ERR_BAD_SHAPE: return "invalid shape";
    case LS_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head dimension";
    case LS_ERR_BAD_DTYPE: return "unsupported dtype";
    case LS_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case LS_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case LS_ERR_BAD_PARAM: return "invalid scalar parameter";
    case LS_ERR_HIP: return "HIP runtime error";
    case LS_ERR_INTERNAL: return "internal error";
    case LS_ERR_ALIASING: return "output overlaps an input";
  }
  return "unknown status";
}

size_t ls_relu_block_workspace_size(const ls_shape* s) {
  Dims d;
  if (check_shape(s, &d) != LS_OK) return 0;
  size_t bytes = relu_plan(s, d).bytes;
  if (relu_pair_shape(s)) {  // enough for either launch: the layout is not known here
    ls_shape ps;
    Dims pd;
    relu_pair_dims(s, d, &ps, &pd);
    bytes = std::max(bytes, relu_plan(&ps, pd).bytes);
  }
  return bytes;
}

size_t ls_gdn_frame_workspace_size(const ls_shape* s) {
  Dims d;
  if (check_shape(s, &d) != LS_OK) return 0;
  // enough for the fused and the phased launch: which one runs depends on the device
  return std::max(gdn_plan(s, d, true).bytes, gdn_plan(s, d, false).bytes);
}

// Both ReLU entry points: packed token tensors (strides NULL) or strided ones.
static ls_status relu_forward(const ls_shape* s, const ls_strides* strides, const ls_prologue* pro,
                              int block_frames, float eps, const void* q, const void* k, const void* v, void* o,
                              const float* state_in,
                              const float* norm_in, float* state_out, float* norm_out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  Dims d;
  ls_status st = check_shape(s, &d);
  if (st != LS_OK) return st;
  if (block_frames < 1) return fail(LS_ERR_BAD_PARAM, "block_frames=%d < 1", block_frames);
  if (!(eps > 0.0f) || !isfinite(eps)) return fail(LS_ERR_BAD_PARAM, "eps=%g must be finite and > 0", (double)eps);
  const int D = s->D;
  linscan::TokLayout layout;
  size_t tok_bytes = 0;  // bytes each token tensor spans
  if ((st = token_layout(s, d, strides, &layout, &tok_bytes)) != LS_OK) return st;
  linscan::Prologue prolog;
  ProBufs pbufs;
  if ((st = prologue_of(pro, s, false, &prolog, &pbufs)) != LS_OK) return st;
  const size_t state_bytes = (size_t)d.bh * D * D * sizeof(float);
  const size_t norm_bytes = (size_t)d.bh * D * sizeof(float);
  if (d.bh == 0) return ok();
  if (tok_bytes > 0 && (!q || !k || !v || !o))
    return fail(LS_ERR_NULL_POINTER, "q, k, v and o are required when F*N > 0");
  if ((tok_bytes && (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o))) ||
      misaligned(state_in) || misaligned(norm_in) || misaligned(state_out) || misaligned(norm_out) ||
      misaligned(workspace))
    return fail(LS_ERR_MISALIGNED, "token tensors, states and workspace must be 16-byte aligned");
  // outputs may not overlap inputs, except the documented in-place state update
  const void* ins[5] = {q, k, v, state_in, norm_in};
  const size_t in_n[5] = {tok_bytes, tok_bytes, tok_bytes, state_in ? state_bytes : 0,
                          norm_in ? norm_bytes : 0};
  for (int i = 0; i < 5; ++i) {
    if (overlap(o, tok_bytes, ins[i], in_n[i])) return fail(LS_ERR_ALIASING, "o overlaps an input");
    if (state_out && !(i == 3 && state_out == state_in) && overlap(state_out, state_bytes, ins[i], in_n[i]))
      return fail(LS_ERR_ALIASING, "state_out overlaps an input other than state_in");
    if (norm_out && !(i == 4 && norm_out == norm_in) && overlap(norm_out, norm_bytes, ins[i], in_n[i]))
      return fail(LS_ERR_ALIASING, "norm_out overlaps an input other than norm_in");
  }
  if (overlap(o, tok_bytes, state_out, state_out ? state_bytes : 0) ||
      overlap(o, tok_bytes, norm_out, norm_out ? norm_bytes : 0) ||
      overlap(state_out, state_out ? state_bytes : 0, norm_out, norm_out ? norm_bytes : 0))
    return fail(LS_ERR_ALIASING, "outputs overlap each other");
  for (int i = 0; i < 4; ++i)
    if (overlap(o, tok_bytes, pbufs.p[i], pbufs.n[i]) ||
        overlap(state_out, state_out ? state_bytes : 0, pbufs.p[i], pbufs.n[i]) ||
        overlap(norm_out, norm_out ? norm_bytes : 0, pbufs.p[i], pbufs.n[i]) ||
        overlap(workspace, workspace ? workspace_bytes : 0, pbufs.p[i], pbufs.n[i]))
      return fail(LS_ERR_ALIASING, "an output or the workspace overlaps the prologue weights");

  hipStream_t hs = (hipStream_t)stream;
  if (s->F == 0 || s->N == 0) {
    // no tokens: the state passes through unchanged
    // (a NULL source means zeros: each range is either all copied or all zeroed)
    const bool cs = state_out && state_out != state_in, cn = norm_out && norm_out != norm_in;
    if (cs && (st = hip_check(linscan::launch_carry(state_in, state_out, state_bytes / 4, nullptr, nullptr, 0,
                                                    state_in == nullptr, hs), "state copy")) != LS_OK)
      return st;
    if (cn && (st = hip_check(linscan::launch_carry(norm_in, norm_out, norm_bytes / 4, nullptr, nullptr, 0,
                                                    norm_in == nullptr, hs), "norm copy")) != LS_OK)
      return st;
    return ok();
  }
  // Heads of dim 32 stored next to each other in every token row share each
  // 128-byte line in pairs; each pair (2i, 2i + 1) then runs as one head of
  // dim 64, so that one work item reads the whole line (no prologue).
  const bool pair = relu_pair_shape(s) && layout.sh == 32 && !prolog.rope() && !prolog.wq && !prolog.wk;
  ls_shape ps;
  Dims pd;
  if (pair) relu_pair_dims(s, d, &ps, &pd);
  const ReluPlan p = pair ? relu_plan(&ps, pd) : relu_plan(s, d);
  // the documented size, whichever launch the layout picks
  const size_t need = ls_relu_block_workspace_size(s);
  if (!workspace) return fail(LS_ERR_NULL_POINTER, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(LS_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  for (int i = 0; i < 5; ++i)
    if (overlap(workspace, need, ins[i], in_n[i]))
      return fail(LS_ERR_ALIASING, "workspace overlaps an input");
  if (overlap(workspace, need, o, tok_bytes) || overlap(workspace, need, state_out, state_out ? state_bytes : 0) ||
      overlap(workspace, need, norm_out, norm_out ? norm_bytes : 0))
    return fail(LS_ERR_ALIASING, "workspace overlaps an output");

  char* ws = (char*)workspace;
  linscan::ScanArgs a;
  a.D = D;
  a.dtype = s->dtype;
  a.relu = true;
  a.mfma = p.mfma;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.S0 = state_in;
  a.z0 = norm_in;
  a.S_out = state_out;
  a.z_out = norm_out;
  a.partial = (float*)(ws + p.partial_off);
  a.init = (float*)(ws + p.init_off);
  a.eps = eps;
  a.bh = d.bh;
  a.bhf = d.bhf;
  a.F = s->F;
  a.N = s->N;
  a.nc = p.nc;
  a.chunk = p.chunk;
  a.nco = p.nco;
  a.chunko = p.chunko;
  a.bfr = block_frames;
  a.L = layout;
  a.P = prolog;
  if (pair) {
    a.pair = true;
    a.D = 64;
    a.bh = pd.bh;
    a.bhf = pd.bhf;
    a.L.H = ps.H;
    a.L.sh = 2 * layout.sh;
    a.L.hg = 1;
  }
  if (p.fused) {
    const long bhp = (a.bh + 8 * a.L.hg - 1) / (8 * a.L.hg) * (8 * a.L.hg);
    uint64_t* flags = (uint64_t*)(ws + p.flags_off);
    uint32_t* err = (uint32_t*)ws;
    const uint64_t epoch = next_epoch();
    if (p.wide)
      return hip_check(
          timed("relu_wide_fused", hs, [&] { return linscan::launch_relu_wide_fused_mfma(a, bhp, flags, epoch, err, hs); }),
          "relu wide fused");
    return hip_check(timed("relu_fused", hs, [&] { return linscan::launch_relu_fused_mfma(a, bhp, flags, epoch, err, hs); }),
                     "relu fused");
  }
  if ((st = hip_check(timed("relu_summary", hs, [&] { return linscan::launch_relu_summary(a, hs); }),
                      "relu summary")) != LS_OK)
    return st;
  if ((st = hip_check(timed("relu_output", hs, [&] { return linscan::launch_relu_output(a, hs); }),
                      "relu output")) != LS_OK)
    return st;
  return ok();
}

// The GDN entry points: beta per frame ([B*H*F]) or, with token_gate, per
// token ([B*H*F][N]); rchunk > 0 runs the reversed scan in chunks of rchunk
// frames (no state in or out).  `fault` receives the kernels' fault word
// (nullptr: the workspace's first word).
static ls_status gdn_forward(const ls_shape* s, const ls_strides* strides, const ls_prologue* pro, float key_scale,
                             const void* q,
                             const void* k, const void* v, const float* alpha, const float* beta, bool token_gate,
                             int rchunk, void* o, const float* state_in, float* state_out, void* workspace,
                             size_t workspace_bytes, void* stream, uint32_t* fault = nullptr) {
  g_last_error.clear();
  Dims d;
  ls_status st = check_shape(s, &d);
  if (st != LS_OK) return st;
  if (!isfinite(key_scale)) return fail(LS_ERR_BAD_PARAM, "key_scale is not finite");
  const int D = s->D;
  linscan::TokLayout layout;
  size_t tok_bytes = 0;  // bytes each token tensor spans
  if ((st = token_layout(s, d, strides, &layout, &tok_bytes)) != LS_OK) return st;
  linscan::Prologue prolog;
  ProBufs pbufs;
  if ((st = prologue_of(pro, s, true, &prolog, &pbufs)) != LS_OK) return st;
  const size_t state_bytes = (size_t)d.bh * D * D * sizeof(float);
  const size_t gate_bytes = (size_t)d.bhf * (token_gate ? (size_t)s->N : 1) * sizeof(float);
  const size_t alpha_bytes = (size_t)d.bhf * sizeof(float);
  if (d.bh == 0) return ok();
  if (tok_bytes > 0 && (!q || !k || !v || !o))
    return fail(LS_ERR_NULL_POINTER, "q, k, v and o are required when F*N > 0");
  if (s->F > 0 && (!alpha || (!beta && gate_bytes > 0)))
    return fail(LS_ERR_NULL_POINTER, "alpha and beta are required when F > 0");
  if ((tok_bytes && (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o))) ||
      misaligned(state_in) || misaligned(state_out) || misaligned(workspace))
    return fail(LS_ERR_MISALIGNED, "token tensors, states and workspace must be 16-byte aligned");
  if (((uintptr_t)alpha & 3u) || ((uintptr_t)beta & 3u))
    return fail(LS_ERR_MISALIGNED, "alpha and beta must be 4-byte aligned");
  const void* ins[6] = {q, k, v, alpha, beta, state_in};
  const size_t in_n[6] = {tok_bytes, tok_bytes, tok_bytes, alpha_bytes, gate_bytes,
                          state_in ? state_bytes : 0};
  for (int i = 0; i < 6; ++i) {
    if (overlap(o, tok_bytes, ins[i], in_n[i])) return fail(LS_ERR_ALIASING, "o overlaps an input");
    if (state_out && !(i == 5 && state_out == state_in) && overlap(state_out, state_bytes, ins[i], in_n[i]))
      return fail(LS_ERR_ALIASING, "state_out overlaps an input other than state_in");
  }
  if (overlap(o, tok_bytes, state_out, state_out ? state_bytes : 0))
    return fail(LS_ERR_ALIASING, "outputs overlap each other");
  for (int i = 0; i < 4; ++i)
    if (overlap(o, tok_bytes, pbufs.p[i], pbufs.n[i]) ||
        overlap(state_out, state_out ? state_bytes : 0, pbufs.p[i], pbufs.n[i]) ||
        overlap(workspace, workspace ? workspace_bytes : 0, pbufs.p[i], pbufs.n[i]))
      return fail(LS_ERR_ALIASING, "an output or the workspace overlaps the prologue weights or rotary tables");

  hipStream_t hs = (hipStream_t)stream;
  if (s->F == 0) {
    if (state_out && state_out != state_in)
      return hip_check(linscan::launch_carry(state_in, state_out, state_bytes / 4, nullptr, nullptr, 0,
                                             state_in == nullptr, hs), "state copy");
    return ok();
  }
  const size_t need = ls_gdn_frame_workspace_size(s);
  if (!workspace) return fail(LS_ERR_NULL_POINTER, "workspace is NULL (need %zu bytes)", need);
  if (workspace_bytes < need)
    return fail(LS_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  for (int i = 0; i < 6; ++i)
    if (overlap(workspace, need, ins[i], in_n[i])) return fail(LS_ERR_ALIASING, "workspace overlaps an input");
  if (overlap(workspace, need, o, tok_bytes) || overlap(workspace, need, state_out, state_out ? state_bytes : 0))
    return fail(LS_ERR_ALIASING, "workspace overlaps an output");
  GdnPlan p = gdn_plan(s, d, true);
  if (p.fused && !linscan::gdn_fused_fits(D, token_gate, prolog.on_k() || prolog.on_q(), p.nc, d.bh))
    p = gdn_plan(s, d, false);

  // keys are scaled by c = 1/sqrt(D*N) unless the caller gives a scale; with
  // no tokens there is nothing to scale
  double c = key_scale > 0.0f ? (double)key_scale : (s->N > 0 ? 1.0 / sqrt((double)D * s->N) : 0.0);
  char* ws = (char*)workspace;
  linscan::ScanArgs a;
  a.D = D;
  a.dtype = s->dtype;
  a.relu = false;
  a.mfma = p.mfma;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.alpha = alpha;
  a.beta = token_gate ? nullptr : beta;
  a.gate = token_gate ? beta : nullptr;
  a.tg = token_gate;
  a.rchunk = rchunk;
  a.L = layout;
  a.P = prolog;
  a.S0 = state_in;
  a.S_out = state_out;
  a.partial = (float*)(ws + p.partial_off);
  a.states = ws + p.states_off;
  a.c = (float)c;
  a.c2 = (float)(c * c);
  a.bh = d.bh;
  a.bhf = d.bhf;
  a.F = s->F;
  a.N = s->N;
  a.nc = p.nc;
  a.chunk = p.chunk;
  a.nco = p.nco;
  a.chunko = p.chunko;
  if (p.fused || p.phased) {
    const long bhp = (d.bh + 8 * layout.hg - 1) / (8 * layout.hg) * (8 * layout.hg);
    uint64_t* gflags = (uint64_t*)(ws + p.gflags_off);
    uint64_t* sflags = (uint64_t*)(ws + p.sflags_off);
    uint32_t* err = fault ? fault : (uint32_t*)ws;
    const uint64_t epoch = next_epoch();
    if (p.fused)
      return hip_check(timed("gdn_fused", hs, [&] {
                         return linscan::launch_gdn_fused_mfma(a, bhp, gflags, sflags, epoch, err, hs);
                       }), "gdn fused");
    if (p.step)
      return hip_check(timed("gdn_step", hs, [&] {
                         return linscan::launch_gdn_step_mfma(a, bhp, gflags, sflags, epoch, err, hs);
                       }), "gdn step");
    return hip_check(timed("gdn_phased", hs, [&] {
                       return linscan::launch_gdn_phased_mfma(a, bhp, gflags, sflags, epoch, err, hs);
                     }), "gdn phased");
  }
  if ((st = hip_check(timed("gdn_gram", hs, [&] { return linscan::launch_gdn_gram(a, hs); }), "gdn gram")) != LS_OK)
    return st;
  if ((st = hip_check(timed("gdn_scan", hs, [&] { return linscan::launch_gdn_scan(a, hs); }), "gdn scan")) != LS_OK)
    return st;
  if (s->N > 0)
    if ((st = hip_check(timed("gdn_output", hs, [&] { return linscan::launch_gdn_output(a, hs); }),
                        "gdn output")) != LS_OK)
      return st;
  return ok();
}

ls_status ls_relu_block_forward(const ls_shape* s, int block_frames, float eps, const void* q,
                                const void* k, const void* v, void* o, const float* state_in,
                                const float* norm_in, float* state_out, float* norm_out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return relu_forward(s, nullptr, nullptr, block_frames, eps, q, k, v, o, state_in, norm_in, state_out, norm_out,
                      workspace, workspace_bytes, stream);
}

ls_status ls_relu_block_forward_strided(const ls_shape* s, const ls_strides* strides, int block_frames, float eps,
                                        const void* q, const void* k, const void* v, void* o,
                                        const float* state_in, const float* norm_in, float* state_out,
                                        float* norm_out, void* workspace, size_t workspace_bytes, void* stream) {
  return relu_forward(s, strides, nullptr, block_frames, eps, q, k, v, o, state_in, norm_in, state_out, norm_out,
                      workspace, workspace_bytes, stream);
}

ls_status ls_gdn_frame_forward_strided(const ls_shape* s, const ls_strides* strides, float key_scale, const void* q,
                                       const void* k, const void* v, const float* alpha, const float* beta, void* o,
                                       const float* state_in, float* state_out, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return gdn_forward(s, strides, nullptr, key_scale, q, k, v, alpha, beta, false, 0, o, state_in, state_out, workspace,
                     workspace_bytes, stream);
}

ls_status ls_relu_block_forward_prologue(const ls_shape* s, const ls_prologue* prologue, int block_frames, float eps,
                                         const void* q, const void* k, const void* v, void* o,
                                         const float* state_in, const float* norm_in, float* state_out,
                                         float* norm_out, void* workspace, size_t workspace_bytes, void* stream) {
  return relu_forward(s, nullptr, prologue, block_frames, eps, q, k, v, o, state_in, norm_in, state_out, norm_out,
                      workspace, workspace_bytes, stream);
}

ls_status ls_gdn_frame_forward_prologue(const ls_shape* s, const ls_prologue* prologue, float key_scale, const void* q,
                                        const void* k, const void* v, const float* alpha, const float* beta, void* o,
                                        const float* state_in, float* state_out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return gdn_forward(s, nullptr, prologue, key_scale, q, k, v, alpha, beta, false, 0, o, state_in, state_out,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

ls_status linscan::gdn_forward_plain(const ls_shape* s, float key_scale, const void* q, const void* k, const void* v,
                                     const float* alpha, const float* beta, void* o, const float* state_in,
                                     float* state_out, void* workspace, size_t workspace_bytes, uint32_t* fault,
                                     void* stream) {
  return gdn_forward(s, nullptr, nullptr, key_scale, q, k, v, alpha, beta, false, 0, o, state_in, state_out, workspace,
                     workspace_bytes, stream, fault);
}

extern "C" {

ls_status ls_gdn_frame_forward(const ls_shape* s, float key_scale, const void* q, const void* k,
                               const void* v, const float* alpha, const float* beta, void* o,
                               const float* state_in, float* state_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return gdn_forward(s, nullptr, nullptr, key_scale, q, k, v, alpha, beta, false, 0, o, state_in, state_out, workspace,
                     workspace_bytes, stream);
}

ls_status ls_gdn_frame_forward_token_gate(const ls_shape* s, float key_scale, const void* q, const void* k,
                                          const void* v, const float* alpha, const float* beta, void* o,
                                          const float* state_in, float* state_out, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return gdn_forward(s, nullptr, nullptr, key_scale, q, k, v, alpha, beta, true, 0, o, state_in, state_out, workspace,
                     workspace_bytes, stream);
}

ls_status ls_gdn_frame_forward_reversed(const ls_shape* s, int chunk_frames, float key_scale, const void* q,
                                        const void* k, const void* v, const float* alpha, const float* beta,
                                        void* o, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (chunk_frames < 1) return fail(LS_ERR_BAD_PARAM, "chunk_frames must be >= 1 (got %d)", chunk_frames);
  return gdn_forward(s, nullptr, nullptr, key_scale, q, k, v, alpha, beta, false, chunk_frames, o, nullptr, nullptr,
                     workspace, workspace_bytes, stream);
}

ls_status ls_temporal_conv3(const ls_shape* s, int block_frames, const void* x, const float* weight,
                            const float* bias, const void* carry_in, void* y, void* carry_out, void* stream) {
  g_last_error.clear();
  if (!s) return fail(LS_ERR_NULL_POINTER, "shape is NULL");
  if (s->B < 0 || s->H < 0 || s->F < 0 || s->N < 0)
    return fail(LS_ERR_BAD_SHAPE, "negative dimension (B=%d H=%d F=%d N=%d)", s->B, s->H, s->F, s->N);
  if (s->dtype != LS_DTYPE_FP32 && s->dtype != LS_DTYPE_BF16)
    return fail(LS_ERR_BAD_DTYPE, "dtype %d is neither LS_DTYPE_FP32 nor LS_DTYPE_BF16", s->dtype);
  const size_t esize = s->dtype == LS_DTYPE_BF16 ? 2 : 4;
  if (s->D < 1 || s->D > 65536 || (s->D * esize) % 16 != 0)
    return fail(LS_ERR_BAD_SHAPE, "channels D=%d must be in [1, 65536] and a multiple of %zu", s->D, 16 / esize);
  if ((double)s->B * s->H * s->F * s->N * s->D > 4.0e18 || (double)s->B * s->H * s->N * s->D / (16 / esize) > 2.0e11)
    return fail(LS_ERR_BAD_SHAPE, "shape too large");
  if (block_frames < 1) return fail(LS_ERR_BAD_PARAM, "block_frames must be >= 1 (got %d)", block_frames);
  const long BH = (long)s->B * s->H;
  const size_t frame_bytes = (size_t)BH * s->N * s->D * esize;  // one frame of every (b, h): carry size
  const size_t tok_bytes = frame_bytes * s->F;
  const size_t w_bytes = (size_t)s->H * s->D * 3 * sizeof(float), b_bytes = (size_t)s->H * s->D * sizeof(float);
  if (frame_bytes == 0) return ok();
  if (tok_bytes > 0 && (!x || !y || !weight)) return fail(LS_ERR_NULL_POINTER, "x, y and weight are required when F > 0");
  if (misaligned(x) || misaligned(y) || misaligned(weight) || misaligned(bias) || misaligned(carry_in) ||
      misaligned(carry_out))
    return fail(LS_ERR_MISALIGNED, "tensors must be 16-byte aligned");
  const void* ins[4] = {x, weight, bias, carry_in};
  const size_t in_n[4] = {tok_bytes, weight ? w_bytes : 0, bias ? b_bytes : 0, carry_in ? frame_bytes : 0};
  for (int i = 0; i < 4; ++i) {
    if (overlap(y, tok_bytes, ins[i], in_n[i])) return fail(LS_ERR_ALIASING, "y overlaps an input");
    if (carry_out && !(i == 3 && carry_out == carry_in) && overlap(carry_out, frame_bytes, ins[i], in_n[i]))
      return fail(LS_ERR_ALIASING, "carry_out overlaps an input other than carry_in");
  }
  if (overlap(y, tok_bytes, carry_out, carry_out ? frame_bytes : 0)) return fail(LS_ERR_ALIASING, "y overlaps carry_out");
  hipStream_t hs = (hipStream_t)stream;
  if (s->F == 0) {  // no frames: the carried frame passes through
    if (carry_out && carry_out != carry_in)
      return hip_check(linscan::launch_carry((const float*)carry_in, (float*)carry_out, frame_bytes / 4, nullptr,
                                             nullptr, 0, carry_in == nullptr, hs),
                       "carry copy");
    return ok();
  }
  const int dt = s->dtype == LS_DTYPE_BF16 ? linscan::DT_BF16 : linscan::DT_F32;
  return hip_check(timed("temporal_conv3", hs, [&] {
                     return linscan::launch_temporal_conv3(dt, x, weight, bias, carry_in, y, carry_out, BH, s->H,
                                                           s->F, s->N, s->D, block_frames, hs);
                   }), "temporal conv");
}

ls_status ls_state_carry(int B, int H, int D, const float* state_src, const float* norm_src,
                         float* state_dst, float* norm_dst, int reset, void* stream) {
  g_last_error.clear();
  if (B < 0 || H < 0) return fail(LS_ERR_BAD_SHAPE, "negative dimension (B=%d H=%d)", B, H);
  if (!supported_d(D)) return fail(LS_ERR_UNSUPPORTED_HEAD_DIM, "head dim D=%d unsupported", D);
  const size_t bh = (size_t)B * H;
  if (bh == 0) return ok();
  if (!state_dst) return fail(LS_ERR_NULL_POINTER, "state_dst is NULL");
  if (!reset && !state_src) return fail(LS_ERR_NULL_POINTER, "state_src is NULL (and reset == 0)");
  if (misaligned(state_src) || misaligned(state_dst) || misaligned(norm_src) || misaligned(norm_dst))
    return fail(LS_ERR_MISALIGNED, "states must be 16-byte aligned");
  const size_t sb = bh * D * D * sizeof(float), nb = bh * D * sizeof(float);
  const bool with_norm = norm_dst && (reset || norm_src);
  if (!reset) {
    if (state_src != state_dst && overlap(state_src, sb, state_dst, sb))
      return fail(LS_ERR_ALIASING, "state_src and state_dst partially overlap");
    if (with_norm && norm_src != norm_dst && overlap(norm_src, nb, norm_dst, nb))
      return fail(LS_ERR_ALIASING, "norm_src and norm_dst partially overlap");
  }
  if (with_norm && overlap(state_dst, sb, norm_dst, nb))
    return fail(LS_ERR_ALIASING, "state_dst and norm_dst overlap");
  hipStream_t hs = (hipStream_t)stream;
  // state and normaliser move in one launch
  const bool do_state = reset || state_src != state_dst;
  const bool do_norm = with_norm && (reset || norm_src != norm_dst);
  if (!do_state && !do_norm) return ok();
  ls_status st = hip_check(timed("state_carry", hs, [&] {
                             return linscan::launch_carry(state_src, state_dst, do_state ? sb / 4 : 0,
                                                          norm_src, norm_dst, do_norm ? nb / 4 : 0, reset, hs);
                           }), "state carry");
  if (st != LS_OK) return st;
  return ok();
}

}  // extern "C"
