"""Pins of the float64 LION-s oracle against facts the LION page fixes.

The mask is checked against its closed forms (the log-cumulative form and the
KMS matrix of the fixed-decay instantiation), the full form against the
independently coded bidirectional RNN of Theorem 3.1, and the backward against
central finite differences and float64 autograd.
"""
import numpy as np
import pytest
import torch

from oracle import lion


def test_mask_symmetric_unit_diagonal_and_log_cumsum_closed_form():
    rng = np.random.default_rng(0)
    lam = 1 / (1 + np.exp(-rng.normal(2, 1, 23)))
    M = lion.decay_mask(lam)
    np.testing.assert_array_equal(np.diag(M), 1.0)
    np.testing.assert_allclose(M, M.T, rtol=1e-14)
    A = np.cumsum(np.log(lam))
    np.testing.assert_allclose(M, np.exp(-np.abs(A[:, None] - A[None, :])), rtol=1e-12)


def test_mask_constant_decay_is_kms_matrix():
    for lam0 in (0.5, 0.9):
        M = lion.decay_mask(np.full(7, lam0))
        i = np.arange(7)
        np.testing.assert_allclose(M, lam0 ** np.abs(i[:, None] - i[None, :]), rtol=1e-14)


def test_mask_no_decay_is_all_ones():
    np.testing.assert_array_equal(lion.decay_mask(np.ones(5)), np.ones((5, 5)))


def test_feature_map_unit_norm_and_positive():
    u = np.random.default_rng(1).standard_normal((50, 16)) * 3
    f = lion.feature_map(u)
    assert np.all(f > 0)
    np.testing.assert_allclose(np.linalg.norm(f, axis=1), 1.0, rtol=1e-14)


def _core_inputs(rng, L, dh=5):
    return (rng.standard_normal((L, dh)), rng.standard_normal((L, dh)),
            rng.standard_normal((L, dh)), rng.normal(1.5, 1.5, L))


@pytest.mark.parametrize("L", [1, 2, 7, 40])
def test_full_form_equals_bidirectional_rnn(L):
    rng = np.random.default_rng(L)
    q, k, v, a = _core_inputs(rng, L)
    np.testing.assert_allclose(lion.core_full(q, k, v, a), lion.core_rnn(q, k, v, a), rtol=1e-11, atol=1e-13)


def test_layer_full_equals_rnn_packed():
    rng = np.random.default_rng(3)
    lens = [9, 1, 30]
    cu = np.concatenate([[0], np.cumsum(lens)])
    d, H, dh = 8, 2, 4
    x = rng.standard_normal((cu[-1], d))
    ws = [rng.standard_normal((d, H * dh)) / np.sqrt(d) for _ in range(3)]
    wl, bl = rng.standard_normal((H, d)) / np.sqrt(d), np.full(H, 3.0)
    y1 = lion.forward_full(x, cu, *ws, wl, bl, H)
    y2 = lion.forward_rnn(x, cu, *ws, wl, bl, H)
    np.testing.assert_allclose(y1, y2, rtol=1e-11, atol=1e-13)


def test_no_decay_reduces_to_plain_bidirectional_linear_attention():
    """lambda -> 1 (a -> +inf) gives the all-ones mask: every query sees the
    same global sums, so y_i = phi(q_i)^T (sum_j phi(k_j) v_j^T) / phi(q_i)^T sum_j phi(k_j)."""
    rng = np.random.default_rng(4)
    q, k, v, _ = _core_inputs(rng, 12)
    y = lion.core_full(q, k, v, np.full(12, 800.0))
    fq, fk = lion.feature_map(q), lion.feature_map(k)
    np.testing.assert_allclose(y, (fq @ (fk.T @ v)) / (fq @ fk.sum(0))[:, None], rtol=1e-12)


def test_single_token_and_convexity():
    rng = np.random.default_rng(5)
    q, k, v, a = _core_inputs(rng, 1)
    np.testing.assert_allclose(lion.core_full(q, k, v, a), v, rtol=1e-14)
    q, k, v, a = _core_inputs(rng, 30)
    y = lion.core_full(q, k, v, a)
    assert np.all(y >= v.min(0) - 1e-12) and np.all(y <= v.max(0) + 1e-12)


def test_first_token_decay_is_never_used():
    """M^B uses lambda_{i+1..j} and M^F lambda_{j+1..i}: lambda_0 appears in no product."""
    rng = np.random.default_rng(6)
    q, k, v, a = _core_inputs(rng, 9)
    a2 = a.copy()
    a2[0] += 5.0
    np.testing.assert_array_equal(lion.core_full(q, k, v, a), lion.core_full(q, k, v, a2))
    _, _, _, da = lion.core_full_vjp(q, k, v, a, rng.standard_normal((9, 5)))
    assert da[0] == 0.0


def test_core_vjp_finite_differences():
    rng = np.random.default_rng(7)
    L = 8
    q, k, v, a = _core_inputs(rng, L, dh=3)
    dy = rng.standard_normal((L, 3))
    grads = lion.core_full_vjp(q, k, v, a, dy)
    args = [q, k, v, a]
    eps = 1e-6
    for n, (arr, g) in enumerate(zip(args, grads)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = [x.copy() for x in args], [x.copy() for x in args]
            ap[n][idx] += eps
            am[n][idx] -= eps
            num[idx] = (np.sum(lion.core_full(*ap) * dy) - np.sum(lion.core_full(*am) * dy)) / (2 * eps)
        err = np.max(np.abs(num - g)) / max(1e-12, np.max(np.abs(num)))
        assert err < 1e-6, (n, err)


def test_layer_backward_matches_float64_autograd():
    rng = np.random.default_rng(8)
    lens = [6, 19]
    cu = np.concatenate([[0], np.cumsum(lens)])
    d, H, dh = 8, 2, 4
    x = rng.standard_normal((cu[-1], d))
    w = [rng.standard_normal((d, H * dh)) / np.sqrt(d) for _ in range(3)]
    wl, bl = rng.standard_normal((H, d)) / np.sqrt(d), np.full(H, 1.0)
    dy = rng.standard_normal((cu[-1], H * dh))
    g = lion.backward_full(x, cu, *w, wl, bl, dy, H)

    t = [torch.tensor(a, requires_grad=True) for a in (x, *w, wl, bl)]
    tx, tq, tk, tv, twl, tbl = t

    def fm(u):
        f = torch.nn.functional.silu(u) + 0.5
        return f / f.norm(dim=-1, keepdim=True)

    ys = []
    for b in range(len(lens)):
        s, e = int(cu[b]), int(cu[b + 1])
        xb = tx[s:e]
        heads = []
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            q, k, v = fm(xb @ tq[:, c]), fm(xb @ tk[:, c]), xb @ tv[:, c]
            logl = torch.nn.functional.logsigmoid(xb @ twl[h] + tbl[h])
            A = torch.cumsum(logl, 0)
            M = torch.exp(-(A[:, None] - A[None, :]).abs())
            P = (q @ k.T) * M
            heads.append((P @ v) / P.sum(1, keepdim=True))
        ys.append(torch.cat(heads, 1))
    (torch.cat(ys) * torch.from_numpy(dy)).sum().backward()
    for tt, key in zip(t, ["dx", "dw_q", "dw_k", "dw_v", "dw_lam", "db_lam"]):
        np.testing.assert_allclose(g[key], tt.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=key)


def test_euler_identity_in_value_weights():
    rng = np.random.default_rng(9)
    lens = [12, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    d, H, dh = 6, 2, 3
    x = rng.standard_normal((cu[-1], d))
    w = [rng.standard_normal((d, H * dh)) for _ in range(3)]
    wl, bl = rng.standard_normal((H, d)), np.full(H, 3.0)
    dy = rng.standard_normal((cu[-1], H * dh))
    y = lion.forward_full(x, cu, *w, wl, bl, H)
    g = lion.backward_full(x, cu, *w, wl, bl, dy, H)
    np.testing.assert_allclose(np.sum(w[2] * g["dw_v"]), np.sum(y * dy), rtol=1e-11)


def test_decay_logit_gradient_sums_to_the_bias_and_weight_gradients():
    """The per-token logit gradient da that backward_full returns is the one its
    weight gradients are built from: db_lam = sum_t da_t and dw_lam = x^T da
    per head (a = x w_lam + b_lam is affine in both). db_lam and dw_lam are
    themselves pinned by finite differences elsewhere in this file."""
    rng = np.random.default_rng(71)
    lens = [9, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    d, H, dh = 6, 2, 3
    x = rng.standard_normal((cu[-1], d))
    w = [rng.standard_normal((d, H * dh)) for _ in range(3)]
    wl, bl = rng.standard_normal((H, d)), np.full(H, 1.5)
    dy = rng.standard_normal((cu[-1], H * dh))
    g = lion.backward_full(x, cu, *w, wl, bl, dy, H)
    assert g["da"].shape == (cu[-1], H)
    np.testing.assert_allclose(g["da"].sum(axis=0), g["db_lam"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(x.T @ g["da"], g["dw_lam"].T, rtol=1e-12, atol=1e-12)
