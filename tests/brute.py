"""Independent fp64 formulations used to pin the oracle (tiny sizes only).

None of these re-types the oracle's recurrence: each one states the same
mathematical object another way, so that a dropped term, a wrong visibility
rule, a transposed state or a misplaced gate in the oracle shows up as a
mismatch.

- relu_masked_sum: block-causal ReLU linear attention written as a masked
  quadratic sum over token pairs (scores phi(q).phi(k), no state at all).
- delta_rule_tokens: the token-wise gated delta rule in its error-correcting
  form S <- alpha S + beta (v - alpha S k) k^T, which the frame-wise rule must
  reduce to when a frame holds one token.
- affine_composite: the (A, B) summary of an interval of an affine recurrence
  S_end = S_start A + B, read off any state-to-state map by probing it with
  S_start = 0 and S_start = I.
"""
import numpy as np


def relu(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(np.signbit(x), 0.0, x)


def relu_masked_sum(q, k, v, block_frames=1, eps=1e-6, S0=None, z0=None):
    """Quadratic form of block-causal ReLU linear attention.

    o_i = [sum_{j: blk(j) <= blk(i)} (phi q_i . phi k_j) v_j + S0 phi q_i]
          / [sum_{j: blk(j) <= blk(i)} (phi q_i . phi k_j) + z0 . phi q_i + eps]
    Returns o [B,H,F,N,D], S [B,H,D,D], z [B,H,D].
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, F, N, D = k.shape
    o = np.zeros_like(q)
    S = np.zeros((B, H, D, D))
    z = np.zeros((B, H, D))
    blk = np.repeat(np.arange(F) // block_frames, N)          # block of each token
    visible = blk[None, :] <= blk[:, None]                     # [i, j]
    for b in range(B):
        for h in range(H):
            pq = relu(q[b, h].reshape(F * N, D))
            pk = relu(k[b, h].reshape(F * N, D))
            vv = v[b, h].reshape(F * N, D)
            s0 = np.zeros((D, D)) if S0 is None else np.asarray(S0, np.float64)[b, h]
            zz0 = np.zeros(D) if z0 is None else np.asarray(z0, np.float64)[b, h]
            scores = (pq @ pk.T) * visible                      # [F*N, F*N]
            num = scores @ vv + pq @ s0.T
            den = scores.sum(axis=1) + pq @ zz0 + eps
            o[b, h] = (num / den[:, None]).reshape(F, N, D)
            S[b, h] = s0 + sum(np.outer(vv[t], pk[t]) for t in range(F * N))
            z[b, h] = zz0 + pk.sum(axis=0)
    return o, S, z


def delta_rule_tokens(q, k, v, alpha, beta, S0=None, key_scale=None):
    """Token-wise gated delta rule, error-correcting form, one token per frame.

    q, k, v: [F, D] (one head), alpha, beta: [F].  Keys are scaled by
    key_scale (default 1/sqrt(D), i.e. 1/sqrt(D*N) with N = 1).
    S <- alpha S + beta (v - alpha S k~) k~^T ;  o = S q.
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    F, D = k.shape
    c = 1.0 / np.sqrt(D) if key_scale is None else key_scale
    S = np.zeros((D, D)) if S0 is None else np.array(S0, dtype=np.float64)
    outs = []
    for f in range(F):
        kt = c * k[f]
        pred = alpha[f] * (S @ kt)                 # what the decayed memory returns for k~
        S = alpha[f] * S + beta[f] * np.outer(v[f] - pred, kt)
        outs.append(S @ q[f])
    return np.array(outs), S


def affine_composite(step, D):
    """(A, B) with step(S) == S @ A + B for an affine map on D x D states."""
    B = step(np.zeros((D, D)))
    A = step(np.eye(D)) - B
    return A, B
