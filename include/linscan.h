/*
 * linscan.h -- C ABI of liblinscan, the block-causal linear-attention scan on
 * AMD Instinct MI355X (gfx950).
 *
 * The scan keeps one fixed-size D x D state per (batch, head) and walks the
 * latent frames of a video in order, so memory does not grow with video
 * length.  Two update rules are provided:
 *
 *  - ReLU linear attention with a cumulative state and normaliser, extended
 *    block by block and cached between blocks ("SANA-Video: Efficient Video
 *    Generation with Block Linear Diffusion Transformer", ICLR 2026 oral talk
 *    transcript, passage on the block KV cache of linear attention; feature
 *    map ReLU and the rule that a block attends to itself and to earlier
 *    blocks: the SANA-Video practical guide, section on core mechanisms);
 *  - frame-wise Gated DeltaNet, one update per latent frame over all of the
 *    frame's spatial tokens, with decay alpha and update gate beta
 *    ("SANA-WM: Efficient Minute-Scale World Modeling with Hybrid Linear
 *    Diffusion Transformer", section 3 Method, hybrid GDN/softmax attention),
 *    keys scaled by 1/sqrt(D*N) with N the spatial tokens per frame (SANA-WM
 *    digest, paragraph on stabilising the spatial explosion, which also
 *    states that this scaling keeps the transition's spectral norm <= 1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Token tensors q, k, v, o are contiguous [B][H][F][N][D], D fastest,
 *    either fp32 or bf16 (ls_shape.dtype); o has the dtype of the inputs and
 *    bf16 outputs are rounded to nearest even from fp32.  The *_strided
 *    entry points take other layouts (ls_strides below).
 *  - The state S is fp32 [B][H][D][D] with S[i][j], i a value dimension and
 *    j a key dimension, so that a query reads o = S q.  The ReLU normaliser
 *    z is fp32 [B][H][D].  Gates alpha, beta are fp32 [B][H][F].
 *  - Every pointer is a DEVICE pointer (hipMalloc'd or equivalent) except
 *    the ls_shape pointer, which is host memory read during the call.
 *  - Token tensors, states and the workspace must be 16-byte aligned.
 *  - Supported head dims: D in {16, 32, 48, 64, 80, 96, 112, 128}.
 *  - A call only enqueues work on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns; results are ready once the stream reaches that
 *    point.  All argument checks run on the host before anything is
 *    enqueued: on any error nothing is launched, no output is touched and
 *    the status names the reason (ls_last_error() gives details).  A device
 *    fault surfaces at the caller's next synchronisation.
 *  - The first 4 bytes of a workspace are its fault word.  Calls that run
 *    as a single launch (bf16 at head dims 32, 64, 112 and 128 for the ReLU
 *    scan, bf16 at head dims 112 and 128 for the GDN scan whenever it has
 *    tokens) hand data between
 *    their work items through flags with bounded waits; if a wait ever gave
 *    up, the call's results are invalid and the fault word becomes nonzero.
 *    The library never clears it; callers that check it zero it beforehand.
 *  - Concurrency: every wait of these launches is for work dispatched
 *    earlier in the same launch, with one exception.  A GDN call with
 *    F >= 2 and B*H <= 32 whose 4*B*H scan work-groups fit in a quarter of
 *    the device's slots for that kernel (B*H <= 32 on an MI355X) keeps them
 *    resident for its whole run, waiting for work-groups of the same launch
 *    that still need free slots (other calls take a launch whose waits all
 *    point at earlier work).  Up to three such calls may run concurrently on
 *    different streams whatever else runs; a fourth could find every slot
 *    taken by waiting work, and its waits would time out (fault word set).
 *  - The caller owns every buffer, including the workspace.  The library
 *    never allocates device memory and carries nothing from one call to the
 *    next (the optional profiling session below only keeps HIP events).
 *    Calls on different streams are safe when their outputs and workspaces
 *    differ (within the concurrency limit above).
 *  - A dimension of size zero is legal: B*H == 0 does nothing; F == 0 copies
 *    the initial state to the output state; N == 0 gives frames without
 *    tokens (the ReLU state is unchanged, the GDN state still decays).
 */
#ifndef LINSCAN_H
#define LINSCAN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LINSCAN_VERSION 200 /* major*100 + minor */

typedef enum {
  LS_OK = 0,
  LS_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  LS_ERR_BAD_SHAPE = 2,           /* a negative dimension, or sizes overflow */
  LS_ERR_UNSUPPORTED_HEAD_DIM = 3,
  LS_ERR_BAD_DTYPE = 4,
  LS_ERR_MISALIGNED = 5,          /* a pointer is not 16-byte aligned */
  LS_ERR_WORKSPACE_TOO_SMALL = 6,
  LS_ERR_BAD_PARAM = 7,           /* eps <= 0, block_frames < 1, non-finite scale ... */
  LS_ERR_HIP = 8,                 /* a HIP runtime call or kernel launch failed */
  LS_ERR_INTERNAL = 9,
  LS_ERR_ALIASING = 10            /* an output overlaps an input it must not overlap */
} ls_status;

typedef enum { LS_DTYPE_FP32 = 0, LS_DTYPE_BF16 = 1 } ls_dtype;

/* Shape of one call.  F is the number of frames handled by THIS call. */
typedef struct {
  int B, H, F, N, D;
  int dtype; /* ls_dtype of q, k, v, o */
} ls_shape;

/*
 * Element strides of the token tensors q, k, v and o (all four share them;
 * D stays contiguous), for the *_strided entry points: element (b, h, f, n, d)
 * sits at b*batch + h*head + f*frame + n*token + d.  For example [B][F][N][H][D]
 * (tokens of all heads interleaved) has token = H*D, head = D, frame = N*H*D,
 * batch = F*N*H*D.  Each stride times the element size must be a multiple of
 * 16 bytes (LS_ERR_MISALIGNED), and distinct (b, h, f, n) must map to
 * disjoint rows: sorted by stride, the dimensions with more than one index
 * must nest, each stride at least the previous stride times the previous
 * extent and the smallest at least D (LS_ERR_BAD_PARAM otherwise).
 */
typedef struct {
  long long batch, head, frame, token;
} ls_strides;

/*
 * Per-token prologue of the *_prologue entry points, applied to q and k as
 * the scan loads them (SANA-WM digest, paragraph on context parallelism and
 * the fused kernel: RMSNorm, ReLU and the key scaling fused into the GDN
 * scan; SANA-Video's linear attention normalises q and k before its ReLU
 * feature map).  For each token row x (the D channels of one head):
 *   RMSNorm  x <- x / sqrt(mean(x^2) + eps) * weight[h][:]   (weight not NULL)
 *   ReLU     x <- max(x, 0)                                   (GDN, relu = 1)
 *   L2       x <- x / |x|, 0 staying 0                        (GDN keys, l2_keys = 1)
 *   RoPE     (rope_frame or rope_token not NULL) channel pair (2i, 2i+1)
 *            of q and k turns by its token's angle:
 *              (x0, x1) <- (x0 cos - x1 sin, x0 sin + x1 cos)
 *            with (cos, sin) = rope_frame[rope_frame_offset + f][i] for the
 *            first rope_frame_pairs pairs (by frame f of the call) and
 *            rope_token[n][i - rope_frame_pairs] for the rest (by token n)
 *            (SANA-WM digest, same paragraph: the fused kernel also prepares
 *            the positional encoding; SANA-Video's guide, core mechanisms:
 *            3D RoPE in the linear attention)
 * in that order, before the key scale (GDN).  The ReLU scan applies its
 * feature map phi after RMSNorm; with the rotary embedding it rotates phi(q)
 * and phi(k) for the numerator only and keeps the unrotated features in the
 * normaliser, which stays positive:
 *     S += v (R phi(k))^T,  z += phi(k),  o = S (R phi(q)) / (z . phi(q) + eps).
 * The arithmetic is fp64; what enters the contractions is rounded once to the
 * token precision (bf16: nearest, ties to even), as a separate exact pass
 * writing the token dtype would give, and the normaliser sums the unrotated
 * features in fp32.
 */
typedef struct {
  const float* q_weight;  /* [H][D] fp32 RMSNorm weights of q, or NULL: q not normalised */
  const float* k_weight;  /* [H][D] fp32 RMSNorm weights of k, or NULL */
  float eps;              /* RMSNorm epsilon, finite and > 0 when a weight is given */
  int relu;               /* GDN only: 1 = ReLU on q and k after their norms */
  int l2_keys;            /* GDN only: 1 = keys divided by their L2 norm */
  /* The rotary embedding (both NULL: none).  Tables are fp32, 16-byte
   * aligned, read only: rope_frame [rope_frames][rope_frame_pairs][2] (needed
   * when rope_frame_pairs > 0) and rope_token [N][D/2 - rope_frame_pairs][2]
   * (needed when rope_frame_pairs < D/2).  rope_frame_pairs is a multiple of 4
   * in [0, D/2]; rope_frame_offset >= 0 and rope_frame_offset + F <=
   * rope_frames (LS_ERR_BAD_PARAM / LS_ERR_NULL_POINTER / LS_ERR_MISALIGNED). */
  const float* rope_frame;
  const float* rope_token;
  int rope_frame_pairs;
  int rope_frame_offset;
  long long rope_frames;
} ls_prologue;

/*
 * Workspace bytes ls_relu_block_forward (and its _strided and _prologue
 * variants) needs for `shape`, 0 if the shape is invalid.  The size depends on
 * the shape only: it covers every block size and token layout.
 */
size_t ls_relu_block_workspace_size(const ls_shape* shape);

/*
 * ReLU block-causal linear attention over the F frames of one call.
 *
 * Frames are grouped into blocks of `block_frames` consecutive frames,
 * counted from frame 0 of this call (1 = frame-causal).  With phi = ReLU
 * (phi(x) = 0 when x has its sign bit set, else x), the state and normaliser
 * start from (state_in, norm_in) (zeros when NULL).  For each block in
 * order, every token of the block adds v phi(k)^T to S and phi(k) to z; then
 * every token of the block reads
 *     o = (S phi(q)) / (z . phi(q) + eps),
 * i.e. a block sees itself and all earlier blocks.  The final (S, z) are
 * written to (state_out, norm_out) when those are non-NULL; state_out may
 * equal state_in and norm_out may equal norm_in (in place), other overlaps
 * between outputs and inputs are rejected with LS_ERR_ALIASING.
 *
 *   q, k, v   [B][H][F][N][D] inputs (dtype of shape)
 *   o         [B][H][F][N][D] output (may not be NULL unless N*F == 0)
 *   eps       > 0 (1e-6 in the video workloads)
 *   workspace >= ls_relu_block_workspace_size(shape, block_frames) bytes,
 *             contents ignored on entry and undefined on return.
 */
ls_status ls_relu_block_forward(const ls_shape* shape, int block_frames, float eps,
                                const void* q, const void* k, const void* v, void* o,
                                const float* state_in, const float* norm_in,
                                float* state_out, float* norm_out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * ls_relu_block_forward with token tensors in the layout `strides` (NULL:
 * packed [B][H][F][N][D]).  Workspace size and everything else as there.
 * Layouts that interleave heads inside a token row ([B][F][N][H][D], head
 * stride D) share 128-byte lines between heads at D = 32: with bf16 tokens
 * and an even head count, heads 2i and 2i + 1 then run in one work item, so
 * each line is read once (results bit for bit those of the packed call).
 */
ls_status ls_relu_block_forward_strided(const ls_shape* shape, const ls_strides* strides, int block_frames,
                                        float eps, const void* q, const void* k, const void* v, void* o,
                                        const float* state_in, const float* norm_in, float* state_out,
                                        float* norm_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ls_relu_block_forward with the per-token prologue `prologue` (NULL: none;
 * relu and l2_keys must be 0: the scan applies its own ReLU feature map;
 * RMSNorm and the rotary embedding as described at ls_prologue).
 * Weights 16-byte aligned (LS_ERR_MISALIGNED) and not overlapping any output
 * or the workspace (LS_ERR_ALIASING); a bad eps or flag is LS_ERR_BAD_PARAM.
 * Workspace size and everything else as ls_relu_block_forward.
 */
ls_status ls_relu_block_forward_prologue(const ls_shape* shape, const ls_prologue* prologue, int block_frames,
                                         float eps, const void* q, const void* k, const void* v, void* o,
                                         const float* state_in, const float* norm_in, float* state_out,
                                         float* norm_out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes ls_gdn_frame_forward needs for `shape` (0 if invalid). */
size_t ls_gdn_frame_workspace_size(const ls_shape* shape);

/*
 * Frame-wise Gated DeltaNet over the F frames of one call.
 *
 * With c = key_scale when key_scale > 0, else c = 1/sqrt(D*N), and S starting
 * from state_in (zeros when NULL), each frame f in order does
 *     G = sum_n (c k_n)(c k_n)^T,   U = sum_n v_n (c k_n)^T   (frame f's tokens)
 *     S <- alpha_f S (I - beta_f G) + beta_f U
 *     o_n = S q_n   for every token n of frame f (the updated state).
 * No feature map or normalisation is applied to q, k or v; callers that want
 * unit-norm keys normalise them beforehand.  alpha and beta are not range
 * checked on the device; their intended domain is [0, 1].
 *
 *   alpha, beta [B][H][F] fp32
 *   o           [B][H][F][N][D] output
 *   state_in    [B][H][D][D] or NULL (zeros)
 *   state_out   [B][H][D][D] or NULL (not written); may equal state_in
 *   workspace   >= ls_gdn_frame_workspace_size(shape) bytes
 */
ls_status ls_gdn_frame_forward(const ls_shape* shape, float key_scale,
                               const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta, void* o,
                               const float* state_in, float* state_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * ls_gdn_frame_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument.  The scan's records, per-frame states
 * and flags live in a static device array of LS_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends; the call
 * itself allocates nothing.  A call whose ls_gdn_frame_workspace_size exceeds
 * that size is rejected with LS_ERR_WORKSPACE_TOO_SMALL before anything is
 * enqueued (64 MiB holds, for example, the single-frame step of B4 H24 D128
 * N920, 19 MB).
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs clearing between calls): calls that overlap
 * in time on one GPU (concurrent streams, or host threads) race and give
 * undefined results; serialise them.
 *
 * fault_word: a device pointer to 4 bytes (4-byte aligned) that the kernels
 * OR a nonzero value into if a bounded wait gave up (the results are then
 * invalid), or NULL (not reported).  The library never clears it.
 * Everything else, including the error behaviour, as ls_gdn_frame_forward.
 */
#define LS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ls_status ls_gdn_frame_forward_noalloc(const ls_shape* shape, float key_scale,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta, void* o,
                                       const float* state_in, float* state_out,
                                       unsigned int* fault_word, void* stream);

/*
 * ls_gdn_frame_forward with token tensors in the layout `strides` (NULL:
 * packed [B][H][F][N][D]).  Workspace size and everything else as there.
 */
ls_status ls_gdn_frame_forward_strided(const ls_shape* shape, const ls_strides* strides, float key_scale,
                                       const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta, void* o,
                                       const float* state_in, float* state_out,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * ls_gdn_frame_forward with the per-token prologue `prologue` (NULL: none),
 * which runs before the key scale.  Argument checks of the weights as for
 * ls_relu_block_forward_prologue; everything else as ls_gdn_frame_forward.
 */
ls_status ls_gdn_frame_forward_prologue(const ls_shape* shape, const ls_prologue* prologue, float key_scale,
                                        const void* q, const void* k, const void* v,
                                        const float* alpha, const float* beta, void* o,
                                        const float* state_in, float* state_out,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Frame-wise Gated DeltaNet with a per-token update gate (SANA-WM summary,
 * section 3 Method, item "Hybrid GDN/Softmax Attention": a decay and a
 * per-token update gate control what the state keeps).  As
 * ls_gdn_frame_forward, except that beta holds one gate per token and each
 * token's terms of the frame's matrices carry its gate:
 *     G = sum_n beta_n (c k_n)(c k_n)^T,   U = sum_n beta_n v_n (c k_n)^T
 *     S <- alpha_f S (I - G) + U
 *     o_n = S q_n   for every token n of frame f.
 * With beta_n = beta_f for every token of frame f this is
 * ls_gdn_frame_forward.  The bf16 kernels apply each gate to one operand of
 * the token products, rounded to bf16 (the other operand stays exact).
 *
 *   alpha [B][H][F] fp32;  beta [B][H][F][N] fp32 (4-byte aligned)
 *   everything else, including the workspace size
 *   (ls_gdn_frame_workspace_size) and the error behaviour, as
 *   ls_gdn_frame_forward.
 */
ls_status ls_gdn_frame_forward_token_gate(const ls_shape* shape, float key_scale,
                                          const void* q, const void* k, const void* v,
                                          const float* alpha, const float* beta, void* o,
                                          const float* state_in, float* state_out,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Reversed frame-wise Gated DeltaNet that resets at chunk boundaries (SANA-WM
 * summary, section 3 Method, item "Chunk-causal deployment": a reversed GDN
 * scan, reset at each chunk boundary, gives each frame context from the later
 * frames of its chunk without leaking across chunks).  Frames are cut into
 * chunks of chunk_frames from frame 0 (the last one may be shorter); each
 * chunk is scanned from its last frame to its first, from a zero state, with
 * each frame's own gates and the update of ls_gdn_frame_forward:
 *     S <- alpha_f S (I - beta_f G_f) + beta_f U_f,   o_n = S q_n (tokens of f).
 * There is no initial or final state.  chunk_frames < 1 is LS_ERR_BAD_PARAM;
 * every other argument, the workspace size (ls_gdn_frame_workspace_size) and
 * the error behaviour are those of ls_gdn_frame_forward.
 */
ls_status ls_gdn_frame_forward_reversed(const ls_shape* shape, int chunk_frames, float key_scale,
                                        const void* q, const void* k, const void* v,
                                        const float* alpha, const float* beta, void* o,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-causal temporal convolution of kernel 3 along frames: the temporal
 * mixing of SANA-Video's Causal Mix-FFN (practical guide, section on core
 * mechanisms: a causal temporal convolution of kernel size 3 in the FFN;
 * talk transcript, passage on causal FFN with temporal convolution: blocks
 * are separated by a zero frame, so a block never sees the next one, and the
 * last frame of a block is handed to the next block, which sees it).
 *
 * For every channel (h, d) and token n, with blocks of block_frames frames
 * from frame 0 of the call,
 *     y_f = w[h][d][0] x_{f-1} + w[h][d][1] x_f + w[h][d][2] x_{f+1} + bias[h][d]
 * where x_{f+1} is zero when frame f ends its block or the call, and x_{-1}
 * is carry_in (zeros when NULL).  Accumulation is fp32; bf16 outputs are
 * rounded to nearest even.
 *
 *   shape       B, H, F, N and D = channels per (b, h): any multiple of 8
 *               (bf16) or 4 (fp32) up to 65536 (not limited to head dims)
 *   x, y        [B][H][F][N][D] of shape->dtype; y may not overlap an input
 *   weight      [H][D][3] fp32 taps on frames f-1, f, f+1
 *   bias        [H][D] fp32, or NULL
 *   carry_in    [B][H][N][D] of shape->dtype, or NULL
 *   carry_out   [B][H][N][D] of shape->dtype, or NULL: receives x_{F-1} (the
 *               carry of the next call); may equal carry_in.  With F = 0 it
 *               receives carry_in (or zeros).
 * All pointers 16-byte aligned; no workspace.  block_frames < 1 is
 * LS_ERR_BAD_PARAM; other errors as for the scans.
 */
ls_status ls_temporal_conv3(const ls_shape* shape, int block_frames, const void* x, const float* weight,
                            const float* bias, const void* carry_in, void* y, void* carry_out, void* stream);

/*
 * Block-autoregressive hand-off of the carried state: the state a finished
 * block leaves behind becomes the cache the next block starts from (SANA-Video
 * talk, block KV cache passage: the state of block i is cached and block i+1
 * adds its own contribution to it).
 *
 * reset == 0: copy state_src -> state_dst ([B][H][D][D] fp32) and, when both
 *             norm pointers are non-NULL, norm_src -> norm_dst ([B][H][D]).
 * reset != 0: zero state_dst (and norm_dst when non-NULL); the sources are
 *             ignored and may be NULL.
 * Source and destination may not partially overlap (identical is a no-op).
 */
ls_status ls_state_carry(int B, int H, int D, const float* state_src, const float* norm_src,
                         float* state_dst, float* norm_dst, int reset, void* stream);

/*
 * Diagnostics: per-kernel timing with HIP events.
 *
 * Between ls_profile_begin() and ls_profile_end(), every kernel the library
 * launches (from any thread, on any stream) is bracketed by two HIP events
 * recorded on the stream it runs on.  ls_profile_end() waits for those
 * events, fills up to `max_stats` entries (one per kernel kind, in first-
 * launch order) with the launch count and the summed event-to-event time,
 * and returns the number of kernel kinds seen (or -1 on a HIP error).  The
 * event records add a few microseconds per launch, so time throughput with
 * profiling off.  At most 65536 launches are recorded per session.
 */
typedef struct {
  char name[32];
  int launches;
  double total_ms;
} ls_kernel_stat;

ls_status ls_profile_begin(void);
int ls_profile_end(ls_kernel_stat* stats, int max_stats);

/* Static description of a status code. */
const char* ls_status_string(ls_status status);

/* Details of the last non-OK status returned on the calling thread ("" if none). */
const char* ls_last_error(void);

/* LINSCAN_VERSION of the built library. */
int ls_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LINSCAN_H */
