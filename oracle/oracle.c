/*
 * oracle.c -- plain fp64 CPU reference for the block-causal linear-attention
 * scan.  TEST INFRASTRUCTURE: only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code, header
 * or constant with the GPU library and never calls into it.
 *
 * Everything here is a direct loop over frames and tokens in the order the
 * pages describe, with double-precision arithmetic throughout.  Token
 * tensors arrive as float32 (bf16 and fp32 inputs widen to float32 without
 * rounding); states arrive and leave as float64.
 *
 * Layout: token tensors are [B][H][F][N][D] row-major (D fastest); the state
 * S is [B][H][D][D] with S[i][j], i indexing value dimensions and j key
 * dimensions, so a query reads out o = S q; the normaliser z is [B][H][D];
 * the gates alpha, beta are [B][H][F].
 *
 * Sources:
 *  - ReLU linear attention with a cumulative D x D state that is cached and
 *    extended block by block: "SANA-Video: Efficient Video Generation with
 *    Block Linear Diffusion Transformer" (ICLR 2026 oral, talk transcript),
 *    the passage on the block KV cache of linear attention; feature map ReLU
 *    per the "SANA-Video practical guide" (lpnh.cn), section on core
 *    mechanisms (attn_type LiteLAReLURope), which also states that each block
 *    attends to itself and the blocks before it.
 *  - Frame-wise Gated DeltaNet with a D x D state updated once per latent
 *    frame from all of that frame's spatial tokens, decay alpha and update
 *    gate beta: "SANA-WM: Efficient Minute-Scale World Modeling with Hybrid
 *    Linear Diffusion Transformer" (paperlayer.ai summary), section 3 Method,
 *    item "Hybrid GDN/Softmax Attention"; key scaling by 1/sqrt(D*S) with S the
 *    spatial tokens per frame: the SANA-WM digest (seosoyoung.eiaserinnys.me),
 *    paragraph on stabilising the spatial explosion.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *  - the ReLU normaliser is o = (S phi(q)) / (z . phi(q) + eps);
 *  - outputs of a block read the state AFTER that block's own tokens were
 *    added (a block sees itself);
 *  - the GDN frame update is S <- alpha S (I - beta G) + beta U with
 *    G = sum_n (c k_n)(c k_n)^T and U = sum_n v_n (c k_n)^T over the frame's
 *    tokens, and the frame's outputs read the updated S;
 *  - phi(x) = 0 when x carries a negative sign, else x (ReLU; -0 maps to 0).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

int oracle_version(void) { return 1; }

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double relu(double x) { return signbit(x) ? 0.0 : x; }

/* offset of token n of frame f of head (b*H + h) in a [B][H][F][N][D] tensor */
static size_t tok(long bh, int f, int n, int F, int N, int D) {
  return (((size_t)bh * F + f) * N + n) * (size_t)D;
}

/*
 * ReLU block-causal linear attention.
 * Frames are grouped into blocks of `block_frames` consecutive frames starting
 * at frame 0 of this call.  For each block in order: every token of the block
 * adds v phi(k)^T to S and phi(k) to z; then every token of the block reads
 * o = S phi(q) / (z . phi(q) + eps).
 * q, k, v: [B][H][F][N][D] float32.  S0, z0: initial state / normaliser or
 * NULL for zeros.  o (may be NULL to skip outputs), S_out, z_out (may be NULL).
 */
int oracle_relu_block(int B, int H, int F, int N, int D, int block_frames, double eps,
                      const float* q, const float* k, const float* v,
                      const double* S0, const double* z0,
                      double* o, double* S_out, double* z_out, int nthreads) {
  if (B < 1 || H < 1 || F < 1 || N < 1 || D < 1 || block_frames < 1) return ORACLE_BAD_ARG;
  if (!k || !v || (o && !q)) return ORACLE_BAD_ARG;
  int status = ORACLE_OK;
  long heads = (long)B * H;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
  for (long bh = 0; bh < heads; ++bh) {
    double* S = (double*)calloc((size_t)D * D, sizeof(double));
    double* z = (double*)calloc((size_t)D, sizeof(double));
    double* feat = (double*)malloc((size_t)D * sizeof(double));
    if (!S || !z || !feat) {
      status = ORACLE_NO_MEMORY;
      free(S); free(z); free(feat);
      continue;
    }
    if (S0) memcpy(S, S0 + (size_t)bh * D * D, (size_t)D * D * sizeof(double));
    if (z0) memcpy(z, z0 + (size_t)bh * D, (size_t)D * sizeof(double));

    for (int f0 = 0; f0 < F; f0 += block_frames) {
      int f1 = f0 + block_frames < F ? f0 + block_frames : F;
      /* 1. the block's keys and values extend the cached state */
      for (int f = f0; f < f1; ++f) {
        for (int n = 0; n < N; ++n) {
          const float* kn = k + tok(bh, f, n, F, N, D);
          const float* vn = v + tok(bh, f, n, F, N, D);
          for (int j = 0; j < D; ++j) feat[j] = relu((double)kn[j]);
          for (int i = 0; i < D; ++i)
            for (int j = 0; j < D; ++j) S[(size_t)i * D + j] += (double)vn[i] * feat[j];
          for (int j = 0; j < D; ++j) z[j] += feat[j];
        }
      }
      /* 2. the block's queries read the state that now includes the block */
      if (o) {
        for (int f = f0; f < f1; ++f) {
          for (int n = 0; n < N; ++n) {
            const float* qn = q + tok(bh, f, n, F, N, D);
            double* on = o + tok(bh, f, n, F, N, D);
            for (int j = 0; j < D; ++j) feat[j] = relu((double)qn[j]);
            double den = 0.0;
            for (int j = 0; j < D; ++j) den += z[j] * feat[j];
            den += eps;
            for (int i = 0; i < D; ++i) {
              double num = 0.0;
              for (int j = 0; j < D; ++j) num += S[(size_t)i * D + j] * feat[j];
              on[i] = num / den;
            }
          }
        }
      }
    }
    if (S_out) memcpy(S_out + (size_t)bh * D * D, S, (size_t)D * D * sizeof(double));
    if (z_out) memcpy(z_out + (size_t)bh * D, z, (size_t)D * sizeof(double));
    free(S); free(z); free(feat);
  }
  return status;
}

/*
 * Block-causal linear attention with separate numerator and denominator
 * features, for the ReLU scan with a rotary position embedding: the SANA-Video
 * practical guide (section on core mechanisms) names the attention
 * LiteLAReLURope, a ReLU linear attention with RoPE, and the talk (passage on
 * the 3D RoPE) adds the rotary embedding to the linear attention.  Rotated
 * features can be negative, so they serve the numerator only and the
 * normaliser keeps the unrotated ReLU features (the pages give no formula;
 * this keeps the denominator positive):
 *   S += v kn^T and z += kd for every token of a block, then
 *   o = S qn / (z . qd + eps) for every token of the block.
 * qn, kn, qd, kd: [B][H][F][N][D] float64 features (the caller applies the
 * feature map and the rotation); v float32; S0, z0, o, S_out, z_out as in
 * oracle_relu_block.
 */
int oracle_linear_block_split(int B, int H, int F, int N, int D, int block_frames, double eps,
                              const double* qn, const double* kn, const double* qd, const double* kd,
                              const float* v, const double* S0, const double* z0, double* o, double* S_out,
                              double* z_out, int nthreads) {
  if (B < 1 || H < 1 || F < 1 || N < 1 || D < 1 || block_frames < 1) return ORACLE_BAD_ARG;
  if (!kn || !kd || !v || (o && (!qn || !qd))) return ORACLE_BAD_ARG;
  int status = ORACLE_OK;
  long heads = (long)B * H;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
  for (long bh = 0; bh < heads; ++bh) {
    double* S = (double*)calloc((size_t)D * D, sizeof(double));
    double* z = (double*)calloc((size_t)D, sizeof(double));
    if (!S || !z) {
      status = ORACLE_NO_MEMORY;
      free(S); free(z);
      continue;
    }
    if (S0) memcpy(S, S0 + (size_t)bh * D * D, (size_t)D * D * sizeof(double));
    if (z0) memcpy(z, z0 + (size_t)bh * D, (size_t)D * sizeof(double));
    for (int f0 = 0; f0 < F; f0 += block_frames) {
      int f1 = f0 + block_frames < F ? f0 + block_frames : F;
      for (int f = f0; f < f1; ++f) {
        for (int n = 0; n < N; ++n) {
          const size_t t = tok(bh, f, n, F, N, D);
          for (int i = 0; i < D; ++i)
            for (int j = 0; j < D; ++j) S[(size_t)i * D + j] += (double)v[t + i] * kn[t + j];
          for (int j = 0; j < D; ++j) z[j] += kd[t + j];
        }
      }
      if (o) {
        for (int f = f0; f < f1; ++f) {
          for (int n = 0; n < N; ++n) {
            const size_t t = tok(bh, f, n, F, N, D);
            double den = 0.0;
            for (int j = 0; j < D; ++j) den += z[j] * qd[t + j];
            den += eps;
            for (int i = 0; i < D; ++i) {
              double num = 0.0;
              for (int j = 0; j < D; ++j) num += S[(size_t)i * D + j] * qn[t + j];
              o[t + i] = num / den;
            }
          }
        }
      }
    }
    if (S_out) memcpy(S_out + (size_t)bh * D * D, S, (size_t)D * D * sizeof(double));
    if (z_out) memcpy(z_out + (size_t)bh * D, z, (size_t)D * sizeof(double));
    free(S); free(z);
  }
  return status;
}

/*
 * Frame-wise Gated DeltaNet.
 * c = key_scale if key_scale > 0, else 1/sqrt(D*N).  For each frame f in order:
 *   G = sum_n (c k_n)(c k_n)^T,  U = sum_n v_n (c k_n)^T   (frame f's tokens)
 *   M = I - beta_f G,  S <- alpha_f (S M) + beta_f U
 *   o_n = S q_n for every token n of frame f.
 * alpha, beta: [B][H][F] float32.  S0: [B][H][D][D] or NULL for zeros.
 * o may be NULL (state only); S_out may be NULL.
 */
int oracle_gdn_frame(int B, int H, int F, int N, int D, double key_scale,
                     const float* q, const float* k, const float* v,
                     const float* alpha, const float* beta, const double* S0,
                     double* o, double* S_out, int nthreads) {
  if (B < 1 || H < 1 || F < 1 || N < 1 || D < 1) return ORACLE_BAD_ARG;
  if (!k || !v || !alpha || !beta || (o && !q)) return ORACLE_BAD_ARG;
  const double c = key_scale > 0.0 ? key_scale : 1.0 / sqrt((double)D * (double)N);
  int status = ORACLE_OK;
  long heads = (long)B * H;
  size_t DD = (size_t)D * D;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
  for (long bh = 0; bh < heads; ++bh) {
    double* S = (double*)calloc(DD, sizeof(double));
    double* G = (double*)malloc(DD * sizeof(double));
    double* U = (double*)malloc(DD * sizeof(double));
    double* M = (double*)malloc(DD * sizeof(double));
    double* T = (double*)malloc(DD * sizeof(double));
    double* kt = (double*)malloc((size_t)D * sizeof(double));
    if (!S || !G || !U || !M || !T || !kt) {
      status = ORACLE_NO_MEMORY;
      free(S); free(G); free(U); free(M); free(T); free(kt);
      continue;
    }
    if (S0) memcpy(S, S0 + (size_t)bh * DD, DD * sizeof(double));

    for (int f = 0; f < F; ++f) {
      const double a = (double)alpha[(size_t)bh * F + f];
      const double b = (double)beta[(size_t)bh * F + f];
      /* 1. the frame's key Gram matrix and value-key matrix, keys scaled by c */
      memset(G, 0, DD * sizeof(double));
      memset(U, 0, DD * sizeof(double));
      for (int n = 0; n < N; ++n) {
        const float* kn = k + tok(bh, f, n, F, N, D);
        const float* vn = v + tok(bh, f, n, F, N, D);
        for (int j = 0; j < D; ++j) kt[j] = c * (double)kn[j];
        for (int i = 0; i < D; ++i) {
          for (int j = 0; j < D; ++j) {
            G[(size_t)i * D + j] += kt[i] * kt[j];
            U[(size_t)i * D + j] += (double)vn[i] * kt[j];
          }
        }
      }
      /* 2. transition: S <- alpha S (I - beta G) + beta U */
      for (int i = 0; i < D; ++i)
        for (int j = 0; j < D; ++j)
          M[(size_t)i * D + j] = (i == j ? 1.0 : 0.0) - b * G[(size_t)i * D + j];
      for (int i = 0; i < D; ++i) {
        for (int j = 0; j < D; ++j) {
          double acc = 0.0;
          for (int l = 0; l < D; ++l) acc += S[(size_t)i * D + l] * M[(size_t)l * D + j];
          T[(size_t)i * D + j] = acc;
        }
      }
      for (size_t e = 0; e < DD; ++e) S[e] = a * T[e] + b * U[e];
      /* 3. the frame's queries read the updated state */
      if (o) {
        for (int n = 0; n < N; ++n) {
          const float* qn = q + tok(bh, f, n, F, N, D);
          double* on = o + tok(bh, f, n, F, N, D);
          for (int i = 0; i < D; ++i) {
            double acc = 0.0;
            for (int j = 0; j < D; ++j) acc += S[(size_t)i * D + j] * (double)qn[j];
            on[i] = acc;
          }
        }
      }
    }
    if (S_out) memcpy(S_out + (size_t)bh * DD, S, DD * sizeof(double));
    free(S); free(G); free(U); free(M); free(T); free(kt);
  }
  return status;
}

/*
 * Frame-wise Gated DeltaNet with a per-token update gate.  The SANA-WM
 * summary (paperlayer.ai), section 3 Method, item "Hybrid GDN/Softmax
 * Attention", names a decay and a per-token update gate; with one update per
 * frame the gate of token n weights that token's contribution:
 *   G = sum_n beta_n (c k_n)(c k_n)^T,  U = sum_n beta_n v_n (c k_n)^T
 *   S <- alpha_f S (I - G) + U ;  o_n = S q_n for the frame's tokens.
 * With beta_n equal to beta_f for every token this is oracle_gdn_frame.
 * alpha: [B][H][F]; beta: [B][H][F][N] float32.  Other arguments as there.
 */
int oracle_gdn_frame_token_gate(int B, int H, int F, int N, int D, double key_scale,
                                const float* q, const float* k, const float* v,
                                const float* alpha, const float* beta, const double* S0,
                                double* o, double* S_out, int nthreads) {
  if (B < 1 || H < 1 || F < 1 || N < 1 || D < 1) return ORACLE_BAD_ARG;
  if (!k || !v || !alpha || !beta || (o && !q)) return ORACLE_BAD_ARG;
  const double c = key_scale > 0.0 ? key_scale : 1.0 / sqrt((double)D * (double)N);
  int status = ORACLE_OK;
  long heads = (long)B * H;
  size_t DD = (size_t)D * D;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
  for (long bh = 0; bh < heads; ++bh) {
    double* S = (double*)calloc(DD, sizeof(double));
    double* G = (double*)malloc(DD * sizeof(double));
    double* U = (double*)malloc(DD * sizeof(double));
    double* T = (double*)malloc(DD * sizeof(double));
    double* kt = (double*)malloc((size_t)D * sizeof(double));
    if (!S || !G || !U || !T || !kt) {
      status = ORACLE_NO_MEMORY;
      free(S); free(G); free(U); free(T); free(kt);
      continue;
    }
    if (S0) memcpy(S, S0 + (size_t)bh * DD, DD * sizeof(double));

    for (int f = 0; f < F; ++f) {
      const double a = (double)alpha[(size_t)bh * F + f];
      /* 1. gate-weighted Gram and value-key matrices of the frame, keys scaled by c */
      memset(G, 0, DD * sizeof(double));
      memset(U, 0, DD * sizeof(double));
      for (int n = 0; n < N; ++n) {
        const double bn = (double)beta[((size_t)bh * F + f) * N + n];
        const float* kn = k + tok(bh, f, n, F, N, D);
        const float* vn = v + tok(bh, f, n, F, N, D);
        for (int j = 0; j < D; ++j) kt[j] = c * (double)kn[j];
        for (int i = 0; i < D; ++i) {
          for (int j = 0; j < D; ++j) {
            G[(size_t)i * D + j] += bn * kt[i] * kt[j];
            U[(size_t)i * D + j] += bn * (double)vn[i] * kt[j];
          }
        }
      }
      /* 2. transition: S <- alpha (S - S G) + U */
      for (int i = 0; i < D; ++i) {
        for (int j = 0; j < D; ++j) {
          double acc = 0.0;
          for (int l = 0; l < D; ++l) acc += S[(size_t)i * D + l] * G[(size_t)l * D + j];
          T[(size_t)i * D + j] = S[(size_t)i * D + j] - acc;
        }
      }
      for (size_t e = 0; e < DD; ++e) S[e] = a * T[e] + U[e];
      /* 3. the frame's queries read the updated state */
      if (o) {
        for (int n = 0; n < N; ++n) {
          const float* qn = q + tok(bh, f, n, F, N, D);
          double* on = o + tok(bh, f, n, F, N, D);
          for (int i = 0; i < D; ++i) {
            double acc = 0.0;
            for (int j = 0; j < D; ++j) acc += S[(size_t)i * D + j] * (double)qn[j];
            on[i] = acc;
          }
        }
      }
    }
    if (S_out) memcpy(S_out + (size_t)bh * DD, S, DD * sizeof(double));
    free(S); free(G); free(U); free(T); free(kt);
  }
  return status;
}

/*
 * Reversed frame-wise Gated DeltaNet that resets at chunk boundaries.  The
 * SANA-WM summary (paperlayer.ai), section 3 Method, item "Chunk-causal
 * deployment": a reversed GDN scan, reset at each chunk boundary, gives every
 * frame context from the later frames of its own chunk without leaking
 * across chunks.  Frames are cut into chunks of `chunk` frames from frame 0
 * (the last chunk may be shorter); within each chunk the state starts at
 * zero at the chunk's LAST frame and the frames are taken in decreasing
 * order, each with its own gates:
 *   G, U of frame f as in oracle_gdn_frame;  S <- alpha_f S (I - beta_f G) + beta_f U
 *   o_n = S q_n for the tokens of frame f.
 * No initial or final state.  Other arguments as in oracle_gdn_frame.
 */
int oracle_gdn_frame_reversed(int B, int H, int F, int N, int D, int chunk, double key_scale,
                              const float* q, const float* k, const float* v,
                              const float* alpha, const float* beta, double* o, int nthreads) {
  if (B < 1 || H < 1 || F < 1 || N < 1 || D < 1 || chunk < 1) return ORACLE_BAD_ARG;
  if (!q || !k || !v || !alpha || !beta || !o) return ORACLE_BAD_ARG;
  const double c = key_scale > 0.0 ? key_scale : 1.0 / sqrt((double)D * (double)N);
  int status = ORACLE_OK;
  long heads = (long)B * H;
  size_t DD = (size_t)D * D;
#ifdef _OPENMP
  if (nthreads < 1) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
#endif
  for (long bh = 0; bh < heads; ++bh) {
    double* S = (double*)malloc(DD * sizeof(double));
    double* G = (double*)malloc(DD * sizeof(double));
    double* U = (double*)malloc(DD * sizeof(double));
    double* T = (double*)malloc(DD * sizeof(double));
    double* kt = (double*)malloc((size_t)D * sizeof(double));
    if (!S || !G || !U || !T || !kt) {
      status = ORACLE_NO_MEMORY;
      free(S); free(G); free(U); free(T); free(kt);
      continue;
    }
    for (int c0 = 0; c0 < F; c0 += chunk) {
      const int c1 = c0 + chunk < F ? c0 + chunk : F;
      memset(S, 0, DD * sizeof(double));  /* reset at the chunk boundary */
      for (int f = c1 - 1; f >= c0; --f) {
        const double a = (double)alpha[(size_t)bh * F + f];
        const double b = (double)beta[(size_t)bh * F + f];
        memset(G, 0, DD * sizeof(double));
        memset(U, 0, DD * sizeof(double));
        for (int n = 0; n < N; ++n) {
          const float* kn = k + tok(bh, f, n, F, N, D);
          const float* vn = v + tok(bh, f, n, F, N, D);
          for (int j = 0; j < D; ++j) kt[j] = c * (double)kn[j];
          for (int i = 0; i < D; ++i) {
            for (int j = 0; j < D; ++j) {
              G[(size_t)i * D + j] += kt[i] * kt[j];
              U[(size_t)i * D + j] += (double)vn[i] * kt[j];
            }
          }
        }
        /* S <- alpha (S - beta S G) + beta U */
        for (int i = 0; i < D; ++i) {
          for (int j = 0; j < D; ++j) {
            double acc = 0.0;
            for (int l = 0; l < D; ++l) acc += S[(size_t)i * D + l] * G[(size_t)l * D + j];
            T[(size_t)i * D + j] = S[(size_t)i * D + j] - b * acc;
          }
        }
        for (size_t e = 0; e < DD; ++e) S[e] = a * T[e] + b * U[e];
        for (int n = 0; n < N; ++n) {
          const float* qn = q + tok(bh, f, n, F, N, D);
          double* on = o + tok(bh, f, n, F, N, D);
          for (int i = 0; i < D; ++i) {
            double acc = 0.0;
            for (int j = 0; j < D; ++j) acc += S[(size_t)i * D + j] * (double)qn[j];
            on[i] = acc;
          }
        }
      }
    }
    free(S); free(G); free(U); free(T); free(kt);
  }
  return status;
}

/*
 * Block-causal temporal convolution of kernel 3 along frames (the Causal
 * Mix-FFN).  The SANA-Video practical guide (lpnh.cn), section on core
 * mechanisms, gives the FFN a causal temporal convolution of kernel size 3;
 * the SANA-Video talk, passage on causal FFN with temporal convolution,
 * separates blocks by a zero frame in training (a block cannot see the next
 * one) and hands the last frame of one block to the next (a block sees the
 * previous block's last frame).  Per channel (h, d) and token n, with blocks
 * of block_frames frames from frame 0:
 *   y_f = w[0] x_{f-1} + w[1] x_f + w[2] x_{f+1} + bias
 * where x_{f+1} is 0 when frame f ends its block (or the call), and x_{-1}
 * is the carried frame (zero when carry is NULL).
 * x: [B][H][F][N][D] float32; w: [H][D][3]; bias: [H][D] or NULL;
 * carry: [B][H][N][D] or NULL.  y: [B][H][F][N][D] float64;
 * carry_out: [B][H][N][D] float64 = x_{F-1}, or NULL.
 */
int oracle_temporal_conv3(int B, int H, int F, int N, int D, int block_frames, const float* x,
                          const float* w, const float* bias, const float* carry, double* y,
                          double* carry_out) {
  if (B < 1 || H < 1 || F < 1 || N < 1 || D < 1 || block_frames < 1) return ORACLE_BAD_ARG;
  if (!x || !w || !y) return ORACLE_BAD_ARG;
  for (long bh = 0; bh < (long)B * H; ++bh) {
    const int h = (int)(bh % H);
    for (int f = 0; f < F; ++f) {
      const int ends_block = (f + 1) % block_frames == 0 || f + 1 == F;
      for (int n = 0; n < N; ++n) {
        for (int d = 0; d < D; ++d) {
          const size_t cell = ((size_t)bh * N + n) * D + d;
          double prev = 0.0, next = 0.0;
          if (f > 0)
            prev = (double)x[tok(bh, f - 1, n, F, N, D) + d];
          else if (carry)
            prev = (double)carry[cell];
          if (!ends_block) next = (double)x[tok(bh, f + 1, n, F, N, D) + d];
          const float* wt = w + ((size_t)h * D + d) * 3;
          double acc = (double)wt[0] * prev + (double)wt[1] * (double)x[tok(bh, f, n, F, N, D) + d] +
                       (double)wt[2] * next;
          if (bias) acc += (double)bias[(size_t)h * D + d];
          y[tok(bh, f, n, F, N, D) + d] = acc;
        }
      }
    }
    if (carry_out)
      for (int n = 0; n < N; ++n)
        for (int d = 0; d < D; ++d)
          carry_out[((size_t)bh * N + n) * D + d] = (double)x[tok(bh, F - 1, n, F, N, D) + d];
  }
  return ORACLE_OK;
}
