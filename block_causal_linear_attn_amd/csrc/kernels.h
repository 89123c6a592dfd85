// kernels.h -- host-side launchers of the scan kernels (internal to liblinscan).
//
// Each launcher enqueues one kernel on `st` and returns the launch status.
// Shapes have been validated by the C-ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace linscan {

enum { DT_F32 = 0, DT_BF16 = 1 };

// MFMA fast paths exist for these (dtype, head dim) pairs; every other
// supported pair runs the generic kernels.
bool relu_has_mfma(int D, int dtype);
bool gdn_has_mfma(int D, int dtype);

// ReLU path ---------------------------------------------------------------
// Per (frame, token chunk): dS = sum v phi(k)^T and dz = sum phi(k) over the
// chunk's tokens -> partial[(bhf * nc + chunk)][D*D + D].
hipError_t launch_relu_summary(int D, bool mfma, int dtype, const void* k, const void* v,
                               float* partial, long bhf, int N, int nc, int chunk,
                               hipStream_t st);
// Per (batch, head): block-causal inclusive prefix of the partials, starting
// from (S0, z0) -> prefix[bhf][D*D + D]; final state -> (S_out, z_out).
hipError_t launch_relu_prefix(int D, const float* partial, const float* S0, const float* z0,
                              float* prefix, float* S_out, float* z_out, long bh, int F, int nc,
                              int block_frames, hipStream_t st);
// Per (frame, token chunk): o = S_f phi(q) / (z_f . phi(q) + eps).
hipError_t launch_relu_output(int D, bool mfma, int dtype, const void* q, void* o,
                              const float* prefix, float eps, long bhf, int N, int nco, int chunk,
                              hipStream_t st);

// Gated DeltaNet path -----------------------------------------------------
// Per (frame, token chunk): G = c2 * sum k k^T, U = c * sum v k^T
// -> partial[(bhf * nc + chunk)][2][D*D].
hipError_t launch_gdn_gram(int D, bool mfma, int dtype, const void* k, const void* v,
                           float* partial, float c, float c2, long bhf, int N, int nc, int chunk,
                           hipStream_t st);
// Per (batch, head, 16-row block of S): S <- alpha S (I - beta G) + beta U for
// every frame in order; the state after each frame goes to `states` (fp32, or
// split into bf16 hi/lo planes when `hilo`), the last one to S_out.
hipError_t launch_gdn_scan(int D, bool hilo, const float* partial, const float* alpha,
                           const float* beta, const float* S0, void* states, float* S_out,
                           long bh, int F, int nc, hipStream_t st);
// Per (frame, token chunk): o = S_f q.
hipError_t launch_gdn_output(int D, bool mfma, int dtype, const void* q, void* o,
                             const void* states, long bhf, int N, int nco, int chunk,
                             hipStream_t st);

// Copy n floats src -> dst, or zero dst when `reset`.
hipError_t launch_carry(const float* src, float* dst, size_t n, int reset, hipStream_t st);

}  // namespace linscan
