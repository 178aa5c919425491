"""Float64 oracle of the Gated Bidirectional Linear Attention (GBLA) layer.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Source: "Gated Bidirectional Linear Attention for Generative Retrieval", section
"核心方法" (core method):
  * 2. BLA, Eq. (2)/(3): y_i = phi(q_i)^T sum_j phi(k_j) v_j^T / phi(q_i)^T sum_j phi(k_j),
    with phi(x) = elu(x) + 1.
  * 3. GBLA (1) Conv1D, Eq. (4): X~ = Conv1d(X); Q, K, V are projections of X~.
  * 3. GBLA (2) key gating, Eq. (5)/(6): every key is scaled by a per-token
    scalar gate g_j before it enters the state S = sum_j g_j phi(k_j) v_j^T and
    the normaliser z = sum_j g_j phi(k_j).
  * 3. GBLA (3) gated RMSNorm, Eq. (7): the attention output O of every head is
    RMS-normalised and multiplied by SiLU(X~ W_R^h) (optional, `w_r`).
  * "多头" (multi-head): every head has its own W_Q^h, W_K^h, W_V^h, w_g^h, W_R^h.

Readings taken where the page leaves a step open (each is listed in the design doc):
  * conv: depthwise, causal, kernel 4, no bias; tap 3 multiplies the current
    token, tap k the token 3-k steps back; zero left padding at the start of
    every packed sequence (no mixing across sequences).
  * gate: sigmoid(x~_j . w_g^h + b_g^h) per token and head (the default); the
    page's literal softmax-over-the-sequence gate is available as gate="softmax".
  * no 1/sqrt(d_h) scale, no epsilon in the denominator, no projection biases;
    the output is the concatenation of the heads. Without `w_r` the readout
    ends at O (Eq. (5)); with it, Eq. (7) is applied per head:
    y_i = gamma (.) O_i / sqrt(mean_c O_ic^2 + eps) (.) SiLU(x~_i W_R^h), the
    mean over the head's d_h features, eps added inside the root, and gamma
    [d_h] the usual learnable RMSNorm scale, shared by the heads (None = 1).
  * packed variable-length input: rows [cu[b], cu[b+1]) form sequence b and
    every sum over j runs over that sequence only.

The backward is derived by hand from the same equations (chain rule); it is
pinned by central finite differences in the tests.
"""
from __future__ import annotations

import numpy as np

CONV_WIDTH = 4


def phi(u):
    """elu(u) + 1 (alpha = 1): u + 1 for u > 0, exp(u) for u <= 0."""
    return np.where(u > 0, u + 1.0, np.exp(np.minimum(u, 0.0)))


def dphi(u):
    """Derivative of elu(u) + 1: 1 for u > 0, exp(u) for u <= 0."""
    return np.where(u > 0, 1.0, np.exp(np.minimum(u, 0.0)))


def sigmoid(s):
    return 1.0 / (1.0 + np.exp(-s))


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def causal_conv(x, cu, conv_w):
    """Depthwise causal Conv1d of Eq. (4), restarted at every sequence start.

    x~_t[c] = sum_{k=0..3} conv_w[c, k] * x_{t-3+k}[c], where rows before the
    start of t's sequence count as zero.
    """
    x, w = _f64(x), _f64(conv_w)
    out = np.zeros_like(x)
    K = w.shape[1]
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        for k in range(K):
            shift = K - 1 - k          # source token is `shift` steps back
            if shift >= e - s:
                continue
            out[s + shift:e] += w[:, k] * x[s:e - shift]
    return out


def causal_conv_backward(dxt, x, cu, conv_w):
    """Gradients of causal_conv with respect to x and conv_w."""
    dxt, x, w = _f64(dxt), _f64(x), _f64(conv_w)
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    K = w.shape[1]
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        for k in range(K):
            shift = K - 1 - k
            if shift >= e - s:
                continue
            # forward: out[s+shift:e] += w[:, k] * x[s:e-shift]
            dx[s:e - shift] += w[:, k] * dxt[s + shift:e]
            dw[:, k] += np.sum(dxt[s + shift:e] * x[s:e - shift], axis=0)
    return dx, dw


def silu(u):
    return u * sigmoid(u)


def dsilu(u):
    sg = sigmoid(u)
    return sg * (1.0 + u * (1.0 - sg))


def output_gate(O, r, gamma, eps):
    """Eq. (7) for one head: RmsNorm(O) (.) SiLU(r), O and r [L, d_h]."""
    rms = np.sqrt(np.mean(O * O, axis=1, keepdims=True) + eps)
    g = 1.0 if gamma is None else gamma[None, :]
    return g * (O / rms) * silu(r)


def output_gate_backward(O, r, gamma, eps, dy):
    """Vector-Jacobian product of output_gate: returns (dO, dr, dgamma or None).

    With rho = sqrt(mean(O^2) + eps), n = O / rho and a = gamma (.) SiLU(r):
      dn = dy (.) a,  dO = (dn - n mean(n (.) dn)) / rho,
      dr = dy (.) gamma (.) n (.) SiLU'(r),  dgamma = sum_i dy_i (.) n_i (.) SiLU(r_i)."""
    dh = O.shape[1]
    rho = np.sqrt(np.mean(O * O, axis=1, keepdims=True) + eps)
    n = O / rho
    g = np.ones(dh) if gamma is None else gamma
    dn = dy * g[None, :] * silu(r)
    dO = (dn - n * np.sum(n * dn, axis=1, keepdims=True) / dh) / rho
    dr = dy * g[None, :] * n * dsilu(r)
    dgamma = None if gamma is None else np.sum(dy * n * silu(r), axis=0)
    return dO, dr, dgamma


def _gate(s, gate):
    if gate == "sigmoid":
        return sigmoid(s)
    if gate == "softmax":       # softmax over the tokens of one sequence (page's Eq. (5) gate)
        e = np.exp(s - s.max())
        return e / e.sum()
    raise ValueError(gate)


def _heads(x_t, w_q, w_k, w_v, w_g, b_g, h, dh):
    cols = slice(h * dh, (h + 1) * dh)
    q = x_t @ w_q[:, cols]
    k = x_t @ w_k[:, cols]
    v = x_t @ w_v[:, cols]
    s = x_t @ w_g[h] + b_g[h]
    return q, k, v, s


def forward(x, cu, conv_w, w_q, w_k, w_v, w_g, b_g, num_heads, gate="sigmoid", w_r=None, gamma=None, eps=1e-6):
    """GBLA forward, Eqs. (4)-(6), linear (state-first) order of Eq. (3), and
    with w_r [d, H*d_h] the gated RMSNorm output of Eq. (7).

    Returns (y [T, H*d_h], S [N, H, d_h, d_h], z [N, H, d_h]).
    """
    x, w_q, w_k, w_v, w_g, b_g = map(_f64, (x, w_q, w_k, w_v, w_g, b_g))
    w_r = None if w_r is None else _f64(w_r)
    gamma = None if gamma is None else _f64(gamma)
    T = x.shape[0]
    H = num_heads
    dh = w_q.shape[1] // H
    N = len(cu) - 1
    xt = causal_conv(x, cu, conv_w)
    y = np.zeros((T, H * dh))
    S_all = np.zeros((N, H, dh, dh))
    z_all = np.zeros((N, H, dh))
    for b in range(N):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        if e0 == s0:
            continue
        xb = xt[s0:e0]
        for h in range(H):
            q, k, v, s = _heads(xb, w_q, w_k, w_v, w_g, b_g, h, dh)
            g = _gate(s, gate)
            qf = phi(q)
            kt = g[:, None] * phi(k)            # K~ = g (.) phi(K), Eq. (6)
            S = kt.T @ v                        # sum_j g_j phi(k_j) v_j^T
            z = kt.sum(axis=0)                  # sum_j g_j phi(k_j)
            O = (qf @ S) / (qf @ z)[:, None]
            if w_r is not None:
                O = output_gate(O, xb @ w_r[:, h * dh:(h + 1) * dh], gamma, eps)
            y[s0:e0, h * dh:(h + 1) * dh] = O
            S_all[b, h], z_all[b, h] = S, z
    return y, S_all, z_all


def forward_quadratic(x, cu, conv_w, w_q, w_k, w_v, w_g, b_g, num_heads, gate="sigmoid", w_r=None, gamma=None,
                      eps=1e-6):
    """Brute-force GBLA forward: Eq. (5) evaluated as an explicit L x L
    similarity sim_ij = g_j phi(q_i)^T phi(k_j), row-normalised (then Eq. (7)
    if w_r is given). Use for small L."""
    x, w_q, w_k, w_v, w_g, b_g = map(_f64, (x, w_q, w_k, w_v, w_g, b_g))
    H = num_heads
    dh = w_q.shape[1] // H
    xt = causal_conv(x, cu, conv_w)
    y = np.zeros((x.shape[0], H * dh))
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        if e0 == s0:
            continue
        xb = xt[s0:e0]
        for h in range(H):
            q, k, v, s = _heads(xb, w_q, w_k, w_v, w_g, b_g, h, dh)
            g = _gate(s, gate)
            sim = (phi(q) @ phi(k).T) * g[None, :]
            O = (sim @ v) / sim.sum(axis=1, keepdims=True)
            if w_r is not None:
                O = output_gate(O, xb @ _f64(w_r)[:, h * dh:(h + 1) * dh], None if gamma is None else _f64(gamma),
                                eps)
            y[s0:e0, h * dh:(h + 1) * dh] = O
    return y


def backward(x, cu, conv_w, w_q, w_k, w_v, w_g, b_g, dy, num_heads, gate="sigmoid", w_r=None, gamma=None,
             eps=1e-6):
    """Gradients of sum(y * dy) for the layer of `forward`.

    Per sequence and head, with q~ = phi(q), k~ = g phi(k), num_i = q~_i^T S,
    den_i = q~_i . z, y_i = num_i / den_i:
      dn_i   = dy_i / den_i,           dden_i = -(dy_i . y_i) / den_i
      dq~_i  = S dn_i + dden_i z,      dS = sum_i q~_i dn_i^T,  dz = sum_i dden_i q~_i
      dk~_j  = dS v_j + dz,            dv_j = dS^T k~_j
      dphi(k)_j = g_j dk~_j,           dg_j = phi(k_j) . dk~_j
      dq = dq~ (.) phi'(q),  dk = dphi(k) (.) phi'(k),  ds = dg g (1 - g)  (sigmoid)
    then the projection and conv chain rule of Eq. (4). With w_r, dy is first
    taken back through Eq. (7) (output_gate_backward) to the gradient of O and
    of r = x~ W_R^h.

    Returns dict with dx, dconv_w, dw_q, dw_k, dw_v, dw_g, db_g (float64),
    ds [T, H], the gradient with respect to the gate logits s, and with w_r
    also dw_r (and dgamma if gamma is given).
    """
    x, w_q, w_k, w_v, w_g, b_g, dy = map(_f64, (x, w_q, w_k, w_v, w_g, b_g, dy))
    w_r = None if w_r is None else _f64(w_r)
    gamma = None if gamma is None else _f64(gamma)
    dw_r = None if w_r is None else np.zeros_like(w_r)
    dgamma = None if gamma is None else np.zeros_like(gamma)
    H = num_heads
    dh = w_q.shape[1] // H
    xt = causal_conv(x, cu, conv_w)
    dxt = np.zeros_like(xt)
    dw_q, dw_k, dw_v = np.zeros_like(w_q), np.zeros_like(w_k), np.zeros_like(w_v)
    dw_g, db_g = np.zeros_like(w_g), np.zeros_like(b_g)
    ds_all = np.zeros((x.shape[0], H))
    for b in range(len(cu) - 1):
        s0, e0 = int(cu[b]), int(cu[b + 1])
        if e0 == s0:
            continue
        xb = xt[s0:e0]
        for h in range(H):
            cols = slice(h * dh, (h + 1) * dh)
            q, k, v, s = _heads(xb, w_q, w_k, w_v, w_g, b_g, h, dh)
            g = _gate(s, gate)
            qf, kf = phi(q), phi(k)
            kt = g[:, None] * kf
            S, z = kt.T @ v, kt.sum(axis=0)
            den = qf @ z
            y = (qf @ S) / den[:, None]
            dyb = dy[s0:e0, cols]
            if w_r is not None:          # Eq. (7): back to dO (dyb from here on) and dr
                dyb, dr, dgam = output_gate_backward(y, xb @ w_r[:, cols], gamma, eps, dyb)
                dw_r[:, cols] += xb.T @ dr
                if gamma is not None:
                    dgamma += dgam
            dn = dyb / den[:, None]
            dden = -np.sum(dyb * y, axis=1) / den
            dqf = dn @ S.T + dden[:, None] * z[None, :]
            dS = qf.T @ dn
            dz = qf.T @ dden
            dkt = v @ dS.T + dz[None, :]
            dv = kt @ dS
            dkf = g[:, None] * dkt
            dg = np.sum(kf * dkt, axis=1)
            if gate == "sigmoid":
                ds = dg * g * (1.0 - g)
            else:
                ds = g * (dg - np.sum(g * dg))
            dq = dqf * dphi(q)
            dk = dkf * dphi(k)
            dw_q[:, cols] += xb.T @ dq
            dw_k[:, cols] += xb.T @ dk
            dw_v[:, cols] += xb.T @ dv
            dw_g[h] += xb.T @ ds
            db_g[h] += ds.sum()
            ds_all[s0:e0, h] = ds
            dxt[s0:e0] += dq @ w_q[:, cols].T + dk @ w_k[:, cols].T + dv @ w_v[:, cols].T \
                + ds[:, None] * w_g[h][None, :]
            if w_r is not None:
                dxt[s0:e0] += dr @ w_r[:, cols].T
    dx, dconv = causal_conv_backward(dxt, x, cu, conv_w)
    out = dict(dx=dx, dconv_w=dconv, dw_q=dw_q, dw_k=dw_k, dw_v=dw_v, dw_g=dw_g, db_g=db_g, ds=ds_all)
    if w_r is not None:
        out["dw_r"] = dw_r
        if gamma is not None:
            out["dgamma"] = dgamma
    return out
