// kernels.h -- host-side launchers of the scan kernels (internal to liblinscan).
//
// Each launcher enqueues one kernel on `st` and returns the launch status.
// Shapes have been validated by the C-ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "layout.h"

namespace linscan {

enum { DT_F32 = 0, DT_BF16 = 1 };

// MFMA fast paths exist for these (dtype, head dim) pairs; every other
// supported pair runs the generic kernels.
bool relu_has_mfma(int D, int dtype);
bool gdn_has_mfma(int D, int dtype);
// The ReLU MFMA pairs served by the wide (head dims 112, 128) items.
bool relu_wide_mfma(int D, int dtype);

// Everything a launcher may need for one call (pointers are device pointers).
struct ScanArgs {
  int D = 0, dtype = 0;
  bool relu = false, mfma = false;
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  void* o = nullptr;
  const float* alpha = nullptr;
  const float* beta = nullptr;   // GDN update gate per frame [B*H*F]
  const float* gate = nullptr;   // GDN update gate per token [B*H*F][N] (tg; beta is then NULL)
  bool tg = false;               // GDN gates per token
  int rchunk = 0;                // GDN: > 0 for the reversed scan in chunks of rchunk frames
  const float* S0 = nullptr;   // initial state (NULL = zeros)
  const float* z0 = nullptr;   // initial ReLU normaliser (NULL = zeros)
  float* S_out = nullptr;
  float* z_out = nullptr;
  float* partial = nullptr;    // per (frame, chunk) summaries (workspace)
  float* init = nullptr;       // ReLU: copy of the initial state (workspace)
  void* states = nullptr;      // GDN: state after every frame (workspace)
  float c = 0.0f, c2 = 0.0f;   // GDN key scale and its square
  float eps = 0.0f;            // ReLU normaliser epsilon
  long bh = 0, bhf = 0;        // B*H, B*H*F
  int F = 0, N = 0;
  int nc = 1, chunk = 1;       // token chunks of the summary/gram pass
  int nco = 1, chunko = 1;     // token chunks of the output pass
  int bfr = 1;                 // ReLU frames per causal block
  // ReLU, head dim 32 with heads interleaved in each token row: heads 2i and
  // 2i + 1 (one 128-byte row segment) run as one head of dim 64 whose state
  // is block-diagonal; D, bh, bhf and L then describe the head pairs, while
  // S0, z0, S_out, z_out keep the per-head layout [B*H][32][32], [B*H][32]
  bool pair = false;
  TokLayout L;                 // element strides of q, k, v, o
  Prologue P;                  // per-token prologue of q and k
};
using GenArgs = ScanArgs;

// ReLU path ---------------------------------------------------------------
// Per (frame, token chunk): dS = sum v phi(k)^T, dz = sum phi(k) ->
// partial[(bhf * nc + chunk)][D*D + D]; (frame 0, chunk 0) of each head also
// copies (S0, z0) into init[bh].
hipError_t launch_relu_summary(const ScanArgs& a, hipStream_t st);
// Per (frame, token chunk): (S_f, z_f) = init + partials of every frame up to
// the end of f's block; o = S_f phi(q) / (z_f . phi(q) + eps); the last
// frame's state goes to (S_out, z_out).
hipError_t launch_relu_output(const ScanArgs& a, hipStream_t st);

// Gated DeltaNet path -----------------------------------------------------
// Per (frame, token chunk): G = c2 * sum k k^T, U = c * sum v k^T
// -> partial[(bhf * nc + chunk)], 8 D^2 bytes each.  Generic kernels store
// G and U in fp32; the MFMA kernels store beta*G as bf16 hi/lo planes and
// beta*U in fp32 (beta of the frame folded in).
hipError_t launch_gdn_gram(const ScanArgs& a, hipStream_t st);
// Per (batch, head, 16-row block of S): S <- alpha S (I - beta G) + beta U for
// every frame in order; the state after each frame goes to `states` (fp32 for
// the generic kernels, bf16 hi/lo planes for the MFMA kernels), the last one
// to S_out.
hipError_t launch_gdn_scan(const ScanArgs& a, hipStream_t st);
// Per (frame, token chunk): o = S_f q.
hipError_t launch_gdn_output(const ScanArgs& a, hipStream_t st);

// One launch for a whole call (MFMA paths): work items exchange partials,
// records and states through flags set to `epoch`; `err` is set if a bounded
// wait timed out.  bhp = B*H rounded up to a multiple of 8.
//  ReLU: flags[B*H*F*nc], one per summary item (frame, token chunk).
hipError_t launch_relu_fused_mfma(const ScanArgs& a, long bhp, uint64_t* flags, uint64_t epoch,
                                  uint32_t* err, hipStream_t st);
//  ReLU, wide heads: `partial` holds the cumulative state of every frame,
//  [B*H*F][128*128 + 128] floats (S row-major, then z; 128 dims wide, zero
//  past D), then [B*H*F][nc] records of the summary parts (nc parts per
//  frame); flags[B*H*F][4] mark the cumulative states' row blocks complete,
//  flags[B*H*F*4 ..][nc] the parts.  `init` is unused.
hipError_t launch_relu_wide_fused_mfma(const ScanArgs& a, long bhp, uint64_t* flags, uint64_t epoch,
                                       uint32_t* err, hipStream_t st);
//  GDN: gflags[B*H*F*nc] (records), sflags[B*H*F*8] (row blocks of states,
//  kGdnFusedRowBlocks of the 8 used); only when gdn_fused_fits, so that scan
//  items never take more than a quarter of the device's slots.
constexpr int kGdnFusedRowBlocks = 4;
// The fused GDN kernel for (head dim D, per-token gates, prologue, nc token
// chunks per frame) keeps its B*H*kGdnFusedRowBlocks scan items within a
// quarter of the slots the current device holds of it.
bool gdn_fused_fits(int D, bool tg, bool pro, int nc, long bh);
hipError_t launch_gdn_fused_mfma(const ScanArgs& a, long bhp, uint64_t* gflags, uint64_t* sflags,
                                 uint64_t epoch, uint32_t* err, hipStream_t st);

// Workgroups of 256 threads of `kernel` that the current device holds at
// once (occupancy per CU x CUs), cached per (kernel, device); 512 if the
// runtime cannot tell.
int device_slots(const void* kernel);

// Frames by which the consumer items of a fused launch trail their producers
// so that a consumer is dispatched about when its inputs become ready: the
// producers of one frame take about as long as the slots need to turn over
// `rounds` times, i.e. rounds * slots / items_per_step steps of dispatch, plus
// one step.  At least `min_lag`, at most F.
int fused_lag(long slots, long items_per_step, int min_lag, int F, double rounds);

//  GDN, any B*H (N > 0): row-split gram items of all frames (four per frame,
//  one record per frame: nc must be 1), then scan items, then output items,
//  in one launch; gflags[B*H*F*4], sflags[B*H*F*8].
hipError_t launch_gdn_phased_mfma(const ScanArgs& a, long bhp, uint64_t* gflags, uint64_t* sflags,
                                  uint64_t epoch, uint32_t* err, hipStream_t st);

//  GDN, single-frame calls (F = 1, N > 0): two items per head, each the gram
//  rows, state rows and one output chunk, then two output-only items per
//  head (nco = 4 chunks of chunko); workspace and flags as the phased launch.
hipError_t launch_gdn_step_mfma(const ScanArgs& a, long bhp, uint64_t* gflags, uint64_t* sflags,
                                uint64_t epoch, uint32_t* err, hipStream_t st);

// Generic (VALU) summary and output kernels of either path.
hipError_t launch_summary_generic(const ScanArgs& a, hipStream_t st);
hipError_t launch_output_generic(const ScanArgs& a, hipStream_t st);

// Block-causal temporal convolution of kernel 3 along frames (x, y, carries
// in `dtype`; F >= 1; D a multiple of 16 bytes of elements): see conv.hip.
hipError_t launch_temporal_conv3(int dtype, const void* x, const float* w, const float* bias, const void* carry_in,
                                 void* y, void* carry_out, long BH, int H, int F, int N, int D, int bfr,
                                 hipStream_t st);

// Copy n0 floats src0 -> dst0 and n1 floats src1 -> dst1 (or zero both
// destinations when `reset`) in one launch.
hipError_t launch_carry(const float* src0, float* dst0, size_t n0, const float* src1, float* dst1,
                        size_t n1, int reset, hipStream_t st);

}  // namespace linscan
