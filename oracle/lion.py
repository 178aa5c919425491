"""Float64 oracle of LION-s selective-decay bidirectional linear attention.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Source: "Linear Attention for Efficient Bidirectional Sequence Modeling",
section "方法详解" (method details):
  * key design 1 (bidirectional mask): M^F_ij = prod_{k=j+1..i} lambda_k on and
    below the diagonal, M^B_ij = prod_{k=i+1..j} lambda_k on and above it, and
    M = M^F + M^B - I so the diagonal counts once.
  * overall framework: full linear attention Y = Scale(Q K^T (.) M) V.
  * key design 2 (Theorem 3.1): the forward and backward RNNs, each with the
    diagonal correction -1/2 k_i v_i^T.
  * three instantiations table: Lion-s uses lambda_i = sigmoid(W x_i + b).
  * training strategy: feature map phi(x) = (SiLU(x) + 0.5) / ||SiLU(x) + 0.5||.

Readings taken where the page leaves a step open (each is listed in the design doc):
  * Scale(.) is row normalisation: Y = diag(P 1)^-1 P V with P = phi(Q) phi(K)^T (.) M,
    the same normaliser that the linear-attention denominator carries.
  * the feature map is applied to q and k (not v), the norm is the L2 norm over
    the head dimension.
  * per head: q, k, v are x W_Q^h, x W_K^h, x W_V^h (no conv, no key gate) and
    lambda_i^h = sigmoid(x_i . w_lam^h + b_lam^h).
  * the RNN outputs of both directions are combined by adding numerators and
    denominators: y_i = sum_dir q_i^T (S_i^dir - k_i v_i^T / 2) /
    sum_dir q_i^T (z_i^dir - k_i / 2), with S^B_i = lambda_{i+1} S^B_{i+1} + k_i v_i^T
    (the index of M^B in key design 1).
  * packed variable-length input: the mask never connects two sequences.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def feature_map(u):
    """(SiLU(u) + 0.5) / ||SiLU(u) + 0.5||_2 over the last axis."""
    f = u * sigmoid(u) + 0.5
    return f / np.linalg.norm(f, axis=-1, keepdims=True)


def feature_map_backward(u, dphi):
    """Vector-Jacobian product of feature_map at u."""
    sg = sigmoid(u)
    f = u * sg + 0.5
    n = np.linalg.norm(f, axis=-1, keepdims=True)
    p = f / n
    df = (dphi - p * np.sum(dphi * p, axis=-1, keepdims=True)) / n
    dsilu = sg * (1.0 + u * (1.0 - sg))
    return df * dsilu


def decay_mask(lam):
    """M = M^F + M^B - I built from the products of key design 1 (one sequence)."""
    lam = _f64(lam)
    L = lam.shape[0]
    MF = np.zeros((L, L))
    for i in range(L):
        # M^F[i, j] = prod_{k=j+1..i} lam_k for j <= i: running product leftwards from j = i
        MF[i, i] = 1.0
        if i > 0:
            MF[i, :i] = np.cumprod(lam[1:i + 1][::-1])[::-1]
    MB = MF.T.copy()                 # prod_{k=i+1..j} lam_k for j >= i is the transpose
    return MF + MB - np.eye(L)


def _heads(xb, w_q, w_k, w_v, w_lam, b_lam, h, dh):
    cols = slice(h * dh, (h + 1) * dh)
    return (xb @ w_q[:, cols], xb @ w_k[:, cols], xb @ w_v[:, cols], xb @ w_lam[h] + b_lam[h])


def core_full(q, k, v, a):
    """One sequence and head: Y = Scale(phi(Q) phi(K)^T (.) M) V with lambda = sigmoid(a)."""
    q, k, v, a = map(_f64, (q, k, v, a))
    M = decay_mask(sigmoid(a))
    P = (feature_map(q) @ feature_map(k).T) * M
    return (P @ v) / P.sum(axis=1, keepdims=True)


def core_rnn(q, k, v, a):
    """One sequence and head: bidirectional RNN form of Theorem 3.1 with the
    -1/2 k_i v_i^T correction.

    The forward scan runs S^F_i = lam_i S^F_{i-1} + k_i [v_i | 1]^T from the
    sequence start, the backward scan S^B_i = lam_{i+1} S^B_{i+1} + k_i [v_i | 1]^T
    from its end; the appended 1 carries the normaliser."""
    q, k, v, a = map(_f64, (q, k, v, a))
    L, dh = v.shape
    lam = sigmoid(a)
    fq, fk = feature_map(q), feature_map(k)
    v1 = np.concatenate([v, np.ones((L, 1))], axis=1)
    SF = np.zeros((L, dh, dh + 1))
    SB = np.zeros((L, dh, dh + 1))
    state = np.zeros((dh, dh + 1))
    for i in range(L):
        state = lam[i] * state + np.outer(fk[i], v1[i])
        SF[i] = state
    state = np.zeros((dh, dh + 1))
    for i in range(L - 1, -1, -1):
        carry = lam[i + 1] * state if i + 1 < L else state
        state = carry + np.outer(fk[i], v1[i])
        SB[i] = state
    y = np.zeros((L, dh))
    for i in range(L):
        half = 0.5 * np.outer(fk[i], v1[i])
        acc = fq[i] @ (SF[i] - half) + fq[i] @ (SB[i] - half)
        y[i] = acc[:dh] / acc[dh]
    return y


def _suffix_block_sums(E):
    """For every k: sum of E[i, j] over i >= k, j < k (block below-left of (k, k))."""
    L = E.shape[0]
    out = np.zeros(L)
    if L == 0:
        return out
    Z = E[::-1].cumsum(axis=0)[::-1].cumsum(axis=1)   # Z[k, c] = sum_{i>=k, j<=c} E[i, j]
    out[1:] = Z[np.arange(1, L), np.arange(0, L - 1)]
    return out


def core_full_vjp(q, k, v, a, dy):
    """Gradients (dq, dk, dv, da) of sum(Y * dY) for core_full.

    With P = G (.) M, G = phi(Q) phi(K)^T, r = P 1, Y = diag(r)^-1 P V:
      dV = P^T (dY / r),   dP_ij = (dY_i . V_j - dY_i . Y_i) / r_i,
      dG = dP (.) M -> dphi(Q) = dG phi(K), dphi(K) = dG^T phi(Q),
      dM = dP (.) G; every off-diagonal M_ij is a product of lam_k over
      min(i,j) < k <= max(i,j), so dlam_k = sum over those pairs of dM_ij M_ij / lam_k,
      and da_k = dlam_k lam_k (1 - lam_k).
    """
    q, k, v, a, dy = map(_f64, (q, k, v, a, dy))
    lam = sigmoid(a)
    M = decay_mask(lam)
    fq, fk = feature_map(q), feature_map(k)
    G = fq @ fk.T
    P = G * M
    r = P.sum(axis=1)
    Y = (P @ v) / r[:, None]
    dyr = dy / r[:, None]
    dv = P.T @ dyr
    dP = dyr @ v.T - np.sum(dyr * Y, axis=1)[:, None]
    dG = dP * M
    dfq = dG @ fk
    dfk = dG.T @ fq
    E = dP * G * M                      # dM_ij * M_ij
    np.fill_diagonal(E, 0.0)
    # pairs whose product contains lam_k: (i >= k, j < k) and (i < k, j >= k)
    dlam_lam = _suffix_block_sums(E) + _suffix_block_sums(E.T)   # dlam_k * lam_k
    da = dlam_lam * (1.0 - lam)
    return feature_map_backward(q, dfq), feature_map_backward(k, dfk), dv, da


def _layer(x, cu, w_q, w_k, w_v, w_lam, b_lam, num_heads, core):
    x, w_q, w_k, w_v, w_lam, b_lam = map(_f64, (x, w_q, w_k, w_v, w_lam, b_lam))
    H = num_heads
    dh = w_q.shape[1] // H
    y = np.zeros((x.shape[0], H * dh))
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        if e0 == s0:
            continue
        xb = x[s0:e0]
        for h in range(H):
            q, k, v, a = _heads(xb, w_q, w_k, w_v, w_lam, b_lam, h, dh)
            y[s0:e0, h * dh:(h + 1) * dh] = core(q, k, v, a)
    return y


def forward_full(x, cu, w_q, w_k, w_v, w_lam, b_lam, num_heads):
    """LION-s layer, full masked form, all sequences and heads -> y [T, H*d_h]."""
    return _layer(x, cu, w_q, w_k, w_v, w_lam, b_lam, num_heads, core_full)


def forward_rnn(x, cu, w_q, w_k, w_v, w_lam, b_lam, num_heads):
    """LION-s layer, bidirectional RNN form, all sequences and heads -> y [T, H*d_h]."""
    return _layer(x, cu, w_q, w_k, w_v, w_lam, b_lam, num_heads, core_rnn)


def backward_full(x, cu, w_q, w_k, w_v, w_lam, b_lam, dy, num_heads):
    """Gradients of sum(y * dy) for forward_full, through the projections of
    q, k, v and the decay logit a = x w_lam^h + b_lam^h.

    Returns dict dx, dw_q, dw_k, dw_v, dw_lam, db_lam (float64), plus da [T, H],
    the gradient of the decay logit a of every token and head (db_lam is its sum
    over the tokens, dw_lam = x^T da)."""
    x, w_q, w_k, w_v, w_lam, b_lam, dy = map(_f64, (x, w_q, w_k, w_v, w_lam, b_lam, dy))
    H = num_heads
    dh = w_q.shape[1] // H
    dx = np.zeros_like(x)
    dw_q, dw_k, dw_v = np.zeros_like(w_q), np.zeros_like(w_k), np.zeros_like(w_v)
    dw_lam, db_lam = np.zeros_like(w_lam), np.zeros_like(b_lam)
    da_all = np.zeros((x.shape[0], H))
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        if e0 == s0:
            continue
        xb = x[s0:e0]
        for h in range(H):
            cols = slice(h * dh, (h + 1) * dh)
            q, k, v, a = _heads(xb, w_q, w_k, w_v, w_lam, b_lam, h, dh)
            dq, dk, dv, da = core_full_vjp(q, k, v, a, dy[s0:e0, cols])
            dw_q[:, cols] += xb.T @ dq
            dw_k[:, cols] += xb.T @ dk
            dw_v[:, cols] += xb.T @ dv
            dw_lam[h] += xb.T @ da
            db_lam[h] += da.sum()
            da_all[s0:e0, h] = da
            dx[s0:e0] += dq @ w_q[:, cols].T + dk @ w_k[:, cols].T + dv @ w_v[:, cols].T \
                + da[:, None] * w_lam[h][None, :]
    return dict(dx=dx, dw_q=dw_q, dw_k=dw_k, dw_v=dw_v, dw_lam=dw_lam, db_lam=db_lam, da=da_all)
