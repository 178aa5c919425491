"""Pins of the float64 GBLA oracle against facts the equations fix.

Every test here checks the oracle against something other than itself: a
library routine (torch conv1d), the brute-force quadratic form of Eq. (5),
closed-form special cases, invariants of Eqs. (2)-(6), and central finite
differences / float64 autograd for the hand-derived backward. The pages print
no worked numeric example for this layer, so there is no golden fixture.
"""
import numpy as np
import pytest
import torch

from oracle import gbla


def _rand_problem(rng, lens, d=12, H=2, dh=4, gate_bias=0.0, wscale=1.0):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    D = H * dh
    p = dict(
        x=rng.standard_normal((T, d)),
        cu=cu,
        conv_w=rng.uniform(-0.5, 0.5, (d, 4)),
        w_q=rng.standard_normal((d, D)) * wscale / np.sqrt(d),
        w_k=rng.standard_normal((d, D)) * wscale / np.sqrt(d),
        w_v=rng.standard_normal((d, D)) * wscale / np.sqrt(d),
        w_g=rng.standard_normal((H, d)) / np.sqrt(d),
        b_g=np.full(H, gate_bias) + rng.standard_normal(H) * 0.3,
    )
    return p, H


def _fwd(p, H, **kw):
    return gbla.forward(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"], p["b_g"], H, **kw)


# ---------------------------------------------------------------- conv (Eq. 4)

def test_conv_matches_torch_conv1d():
    """Causal depthwise conv == torch conv1d (cross-correlation) with 3 zeros of
    left padding, run on every sequence separately."""
    rng = np.random.default_rng(0)
    lens = [1, 2, 7, 30]
    cu = np.concatenate([[0], np.cumsum(lens)])
    d = 5
    x = rng.standard_normal((cu[-1], d))
    w = rng.standard_normal((d, 4))
    got = gbla.causal_conv(x, cu, w)
    for b in range(len(lens)):
        xb = torch.from_numpy(x[cu[b]:cu[b + 1]].T[None])            # [1, d, L]
        ref = torch.nn.functional.conv1d(xb, torch.from_numpy(w)[:, None, :], padding=3, groups=d)
        ref = ref[0, :, :lens[b]].T.numpy()
        np.testing.assert_allclose(got[cu[b]:cu[b + 1]], ref, rtol=1e-13, atol=1e-13)


def test_conv_shift_kernel_restarts_at_sequence_start():
    rng = np.random.default_rng(1)
    lens = [3, 1, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((cu[-1], 4))
    w = np.zeros((4, 4))
    w[:, 2] = 1.0                                     # one step back
    got = gbla.causal_conv(x, cu, w)
    for b in range(len(lens)):
        s, e = cu[b], cu[b + 1]
        assert np.all(got[s] == 0.0)
        np.testing.assert_array_equal(got[s + 1:e], x[s:e - 1])


def test_conv_backward_matches_autograd():
    rng = np.random.default_rng(2)
    lens = [4, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((cu[-1], 3))
    w = rng.standard_normal((3, 4))
    g = rng.standard_normal(x.shape)
    dx, dw = gbla.causal_conv_backward(g, x, cu, w)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    outs = []
    for b in range(len(lens)):
        xb = xt[cu[b]:cu[b + 1]].T[None]
        o = torch.nn.functional.conv1d(xb, wt[:, None, :], padding=3, groups=3)[0, :, :lens[b]].T
        outs.append(o)
    (torch.cat(outs) * torch.from_numpy(g)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- forward

@pytest.mark.parametrize("gate", ["sigmoid", "softmax"])
def test_linear_form_equals_quadratic_brute_force(gate):
    """Eq. (3)/(6) state-first evaluation == explicit L x L similarity of Eq. (5)."""
    rng = np.random.default_rng(3)
    p, H = _rand_problem(rng, [1, 5, 17, 64], d=16, H=2, dh=8)
    y, _, _ = _fwd(p, H, gate=gate)
    yq = gbla.forward_quadratic(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"],
                                p["w_g"], p["b_g"], H, gate=gate)
    np.testing.assert_allclose(y, yq, rtol=1e-12, atol=1e-13)


def test_single_token_output_is_its_value():
    rng = np.random.default_rng(4)
    p, H = _rand_problem(rng, [1, 1, 1], d=8, H=2, dh=4)
    y, _, _ = _fwd(p, H)
    xt = gbla.causal_conv(p["x"], p["cu"], p["conv_w"])
    np.testing.assert_allclose(y, xt @ p["w_v"], rtol=1e-12, atol=1e-14)


def test_output_is_convex_combination_of_values():
    rng = np.random.default_rng(5)
    p, H = _rand_problem(rng, [9, 33], d=8, H=2, dh=4, wscale=3.0)
    y, _, _ = _fwd(p, H)
    v = gbla.causal_conv(p["x"], p["cu"], p["conv_w"]) @ p["w_v"]
    for b in range(2):
        s, e = p["cu"][b], p["cu"][b + 1]
        lo, hi = v[s:e].min(axis=0), v[s:e].max(axis=0)
        assert np.all(y[s:e] >= lo - 1e-12) and np.all(y[s:e] <= hi + 1e-12)


def test_uniform_gate_drops_out():
    """w_g = 0 gives every token the same gate, so the bias cannot matter and
    the layer reduces to plain BLA; the softmax gate gives the same output."""
    rng = np.random.default_rng(6)
    p, H = _rand_problem(rng, [7, 20], d=8, H=2, dh=4)
    p["w_g"] = np.zeros_like(p["w_g"])
    outs = []
    for bias in (-3.0, 0.0, 2.5):
        p["b_g"] = np.full(H, bias)
        outs.append(_fwd(p, H)[0])
    outs.append(_fwd(p, H, gate="softmax")[0])
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=1e-12, atol=1e-14)


def test_permutation_equivariance_without_conv():
    """With the identity conv (tap 3 = 1) every token is mixed only through the
    global sums, so permuting a sequence's tokens permutes its outputs."""
    rng = np.random.default_rng(7)
    p, H = _rand_problem(rng, [11, 6], d=8, H=2, dh=4)
    p["conv_w"] = np.zeros_like(p["conv_w"])
    p["conv_w"][:, 3] = 1.0
    y, _, _ = _fwd(p, H)
    perm = np.concatenate([rng.permutation(11), 11 + rng.permutation(6)])
    p2 = dict(p, x=p["x"][perm])
    y2, _, _ = _fwd(p2, H)
    np.testing.assert_allclose(y2, y[perm], rtol=1e-12, atol=1e-14)


def test_packed_equals_separate_and_isolated():
    rng = np.random.default_rng(8)
    lens = [5, 13, 1, 8]
    p, H = _rand_problem(rng, lens, d=8, H=2, dh=4)
    y, S, z = _fwd(p, H)
    cu = p["cu"]
    for b in range(len(lens)):
        s, e = cu[b], cu[b + 1]
        pb = dict(p, x=p["x"][s:e], cu=np.array([0, e - s]))
        yb, Sb, zb = _fwd(pb, H)
        np.testing.assert_allclose(y[s:e], yb, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(S[b], Sb[0], rtol=1e-13, atol=1e-14)
    # perturbing sequence 1 leaves every other sequence untouched (bitwise)
    x2 = p["x"].copy()
    x2[cu[1]:cu[2]] += 1.0
    y2, _, _ = _fwd(dict(p, x=x2), H)
    mask = np.ones(len(y), bool)
    mask[cu[1]:cu[2]] = False
    np.testing.assert_array_equal(y2[mask], y[mask])
    assert not np.allclose(y2[~mask], y[~mask])


def test_empty_sequences_are_allowed():
    rng = np.random.default_rng(9)
    p, H = _rand_problem(rng, [0, 4, 0, 3, 0], d=8, H=1, dh=4)
    y, S, z = _fwd(p, H)
    assert np.all(S[0] == 0) and np.all(S[2] == 0) and np.all(S[4] == 0)
    pb = dict(p, cu=np.array([0, 4, 7]))
    np.testing.assert_allclose(y, _fwd(pb, H)[0], rtol=0, atol=0)


# ---------------------------------------------------------------- backward

def _loss(p, H, dy, gate):
    return float(np.sum(_fwd(p, H, gate=gate)[0] * dy))


@pytest.mark.parametrize("gate", ["sigmoid", "softmax"])
def test_backward_central_finite_differences(gate):
    rng = np.random.default_rng(10)
    p, H = _rand_problem(rng, [3, 6], d=6, H=2, dh=3, wscale=2.0)
    dy = rng.standard_normal((9, 6))
    g = gbla.backward(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"],
                      p["b_g"], dy, H, gate=gate)
    names = dict(x="dx", conv_w="dconv_w", w_q="dw_q", w_k="dw_k", w_v="dw_v", w_g="dw_g", b_g="db_g")
    eps = 1e-6
    for key, gkey in names.items():
        base = p[key]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            pp, pm = base.copy(), base.copy()
            pp[idx] += eps
            pm[idx] -= eps
            num[idx] = (_loss(dict(p, **{key: pp}), H, dy, gate)
                        - _loss(dict(p, **{key: pm}), H, dy, gate)) / (2 * eps)
        # true zeros (db_g under the shift-invariant softmax gate) need the atol
        np.testing.assert_allclose(g[gkey], num, rtol=1e-6, atol=1e-8, err_msg=key)


def test_backward_matches_float64_autograd():
    """An independent derivation: torch float64 autograd through Eqs. (4)-(6)."""
    rng = np.random.default_rng(11)
    lens = [17, 40]
    p, H = _rand_problem(rng, lens, d=16, H=2, dh=8)
    dy = rng.standard_normal((57, 16))
    g = gbla.backward(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"],
                      p["b_g"], dy, H)
    t = {k: torch.tensor(v, requires_grad=True) for k, v in p.items() if k != "cu"}
    dh = 8
    ys = []
    for b in range(len(lens)):
        s, e = int(p["cu"][b]), int(p["cu"][b + 1])
        xb = t["x"][s:e].T[None]
        xt = torch.nn.functional.conv1d(xb, t["conv_w"][:, None, :], padding=3, groups=16)[0, :, :e - s].T
        heads = []
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            q, k, v = xt @ t["w_q"][:, c], xt @ t["w_k"][:, c], xt @ t["w_v"][:, c]
            gg = torch.sigmoid(xt @ t["w_g"][h] + t["b_g"][h])
            fq, fk = torch.nn.functional.elu(q) + 1, torch.nn.functional.elu(k) + 1
            kt = gg[:, None] * fk
            heads.append((fq @ (kt.T @ v)) / (fq @ kt.sum(0))[:, None])
        ys.append(torch.cat(heads, 1))
    (torch.cat(ys) * torch.from_numpy(dy)).sum().backward()
    pairs = dict(x="dx", conv_w="dconv_w", w_q="dw_q", w_k="dw_k", w_v="dw_v", w_g="dw_g", b_g="db_g")
    for k, gk in pairs.items():
        np.testing.assert_allclose(g[gk], t[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


def test_backward_euler_identity_in_value_weights():
    """y is homogeneous of degree 1 in W_V, so <W_V, dW_V> = <y, dY> exactly."""
    rng = np.random.default_rng(12)
    p, H = _rand_problem(rng, [10, 25], d=8, H=2, dh=4)
    dy = rng.standard_normal((35, 8))
    y, _, _ = _fwd(p, H)
    g = gbla.backward(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"],
                      p["b_g"], dy, H)
    np.testing.assert_allclose(np.sum(p["w_v"] * g["dw_v"]), np.sum(y * dy), rtol=1e-12)


def test_backward_gate_bias_gradient_vanishes_when_gate_cannot_matter():
    rng = np.random.default_rng(13)
    p, H = _rand_problem(rng, [10, 25], d=8, H=2, dh=4)
    dy = rng.standard_normal((35, 8))
    # softmax over the sequence is shift invariant: a bias shift changes nothing
    g = gbla.backward(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"],
                      p["b_g"], dy, H, gate="softmax")
    np.testing.assert_allclose(g["db_g"], 0.0, atol=1e-12)
    # sigmoid gate with w_g = 0: uniform gates, the output does not depend on b_g
    p["w_g"] = np.zeros_like(p["w_g"])
    g = gbla.backward(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"],
                      p["b_g"], dy, H)
    np.testing.assert_allclose(g["db_g"], 0.0, atol=1e-12)


# ---------------------------------------------------------------- gated RMSNorm output (Eq. 7)

def _gated(rng, p, H, dh, with_gamma=True):
    d = p["x"].shape[1]
    w_r = rng.standard_normal((d, H * dh)) / np.sqrt(d)
    gamma = 1.0 + 0.3 * rng.standard_normal(dh) if with_gamma else None
    return w_r, gamma


@pytest.mark.parametrize("with_gamma", [True, False])
@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_output_gate_matches_torch_rms_norm(with_gamma, eps):
    """Eq. (7) for one head == torch's rms_norm over the head dimension times
    SiLU of the gate pre-activation (a library routine, not a retyped formula)."""
    rng = np.random.default_rng(40)
    O = rng.standard_normal((23, 8)) * 0.7
    r = rng.standard_normal((23, 8)) * 2.0
    gamma = rng.standard_normal(8) if with_gamma else None
    got = gbla.output_gate(O, r, gamma, eps)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(O), (8,), weight=None if gamma is None else
                                       torch.from_numpy(gamma), eps=eps) * torch.nn.functional.silu(torch.from_numpy(r))
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("gate", ["sigmoid", "softmax"])
def test_output_gate_linear_form_equals_quadratic_brute_force(gate):
    rng = np.random.default_rng(41)
    p, H = _rand_problem(rng, [1, 5, 17, 40], d=16, H=2, dh=8)
    w_r, gamma = _gated(rng, p, H, 8)
    y, _, _ = _fwd(p, H, gate=gate, w_r=w_r, gamma=gamma, eps=1e-5)
    yq = gbla.forward_quadratic(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"], p["b_g"], H,
                                gate=gate, w_r=w_r, gamma=gamma, eps=1e-5)
    np.testing.assert_allclose(y, yq, rtol=1e-12, atol=1e-13)


def test_output_gate_rows_have_unit_rms_before_the_gate():
    """With gamma = 1, y / SiLU(r) is O / rms(O): its mean square over a head's
    features is mean(O^2) / (mean(O^2) + eps), exactly 1 for eps = 0."""
    rng = np.random.default_rng(42)
    p, H = _rand_problem(rng, [9, 30], d=8, H=2, dh=4)
    w_r, _ = _gated(rng, p, H, 4)
    y0, _, _ = _fwd(p, H)
    xt = gbla.causal_conv(p["x"], p["cu"], p["conv_w"])
    for eps in (0.0, 0.05):
        y, _, _ = _fwd(p, H, w_r=w_r, eps=eps)
        u = y / gbla.silu(xt @ w_r)
        for h in range(H):
            c = slice(4 * h, 4 * h + 4)
            ms0 = np.mean(y0[:, c] ** 2, axis=1)
            np.testing.assert_allclose(np.mean(u[:, c] ** 2, axis=1), ms0 / (ms0 + eps), rtol=1e-10)


def test_output_gate_removes_the_value_scale():
    """For eps = 0, y is homogeneous of degree 0 in W_V (O scales with W_V and
    the RMSNorm removes it): scaling W_V leaves y unchanged and <W_V, dW_V> = 0;
    y is linear in gamma, so <gamma, dgamma> = <y, dy>."""
    rng = np.random.default_rng(43)
    p, H = _rand_problem(rng, [10, 25], d=8, H=2, dh=4)
    w_r, gamma = _gated(rng, p, H, 4)
    dy = rng.standard_normal((35, 8))
    y, _, _ = _fwd(p, H, w_r=w_r, gamma=gamma, eps=0.0)
    y3, _, _ = _fwd(dict(p, w_v=3.0 * p["w_v"]), H, w_r=w_r, gamma=gamma, eps=0.0)
    np.testing.assert_allclose(y3, y, rtol=1e-12, atol=1e-14)
    g = gbla.backward(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"], p["b_g"], dy, H,
                      w_r=w_r, gamma=gamma, eps=0.0)
    assert abs(np.sum(p["w_v"] * g["dw_v"])) < 1e-12 * np.sum(np.abs(p["w_v"] * g["dw_v"]))
    np.testing.assert_allclose(np.sum(gamma * g["dgamma"]), np.sum(y * dy), rtol=1e-12)


@pytest.mark.parametrize("gate", ["sigmoid", "softmax"])
def test_output_gate_backward_central_finite_differences(gate):
    rng = np.random.default_rng(44)
    p, H = _rand_problem(rng, [3, 6], d=6, H=2, dh=3, wscale=2.0)
    w_r, gamma = _gated(rng, p, H, 3)
    dy = rng.standard_normal((9, 6))
    eps = 1e-3
    kw = dict(gate=gate, eps=eps)

    def loss(q, wr, gm):
        return float(np.sum(_fwd(q, H, w_r=wr, gamma=gm, **kw)[0] * dy))

    g = gbla.backward(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"], p["b_g"], dy, H,
                      w_r=w_r, gamma=gamma, **kw)
    h = 1e-6
    names = dict(x="dx", conv_w="dconv_w", w_q="dw_q", w_k="dw_k", w_v="dw_v", w_g="dw_g", b_g="db_g")
    for key, gkey in names.items():
        base = p[key]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            pp, pm = base.copy(), base.copy()
            pp[idx] += h
            pm[idx] -= h
            num[idx] = (loss(dict(p, **{key: pp}), w_r, gamma) - loss(dict(p, **{key: pm}), w_r, gamma)) / (2 * h)
        np.testing.assert_allclose(g[gkey], num, rtol=1e-6, atol=1e-8, err_msg=key)
    for name, base in (("dw_r", w_r), ("dgamma", gamma)):
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            pp, pm = base.copy(), base.copy()
            pp[idx] += h
            pm[idx] -= h
            if name == "dw_r":
                num[idx] = (loss(p, pp, gamma) - loss(p, pm, gamma)) / (2 * h)
            else:
                num[idx] = (loss(p, w_r, pp) - loss(p, w_r, pm)) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_output_gate_backward_matches_float64_autograd():
    """An independent derivation: torch float64 autograd through Eqs. (4)-(7),
    with torch's own rms_norm and silu."""
    rng = np.random.default_rng(45)
    lens = [17, 40]
    p, H = _rand_problem(rng, lens, d=16, H=2, dh=8)
    w_r, gamma = _gated(rng, p, H, 8)
    dy = rng.standard_normal((57, 16))
    eps = 1e-4
    g = gbla.backward(p["x"], p["cu"], p["conv_w"], p["w_q"], p["w_k"], p["w_v"], p["w_g"], p["b_g"], dy, H,
                      w_r=w_r, gamma=gamma, eps=eps)
    t = {k: torch.tensor(v, requires_grad=True) for k, v in p.items() if k != "cu"}
    t["w_r"] = torch.tensor(w_r, requires_grad=True)
    t["gamma"] = torch.tensor(gamma, requires_grad=True)
    F = torch.nn.functional
    dh = 8
    ys = []
    for b in range(len(lens)):
        s, e = int(p["cu"][b]), int(p["cu"][b + 1])
        xt = F.conv1d(t["x"][s:e].T[None], t["conv_w"][:, None, :], padding=3, groups=16)[0, :, :e - s].T
        heads = []
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            q, k, v = xt @ t["w_q"][:, c], xt @ t["w_k"][:, c], xt @ t["w_v"][:, c]
            gg = torch.sigmoid(xt @ t["w_g"][h] + t["b_g"][h])
            fq, fk = F.elu(q) + 1, F.elu(k) + 1
            kt = gg[:, None] * fk
            O = (fq @ (kt.T @ v)) / (fq @ kt.sum(0))[:, None]
            heads.append(F.rms_norm(O, (dh,), weight=t["gamma"], eps=eps) * F.silu(xt @ t["w_r"][:, c]))
        ys.append(torch.cat(heads, 1))
    (torch.cat(ys) * torch.from_numpy(dy)).sum().backward()
    pairs = dict(x="dx", conv_w="dconv_w", w_q="dw_q", w_k="dw_k", w_v="dw_v", w_g="dw_g", b_g="db_g", w_r="dw_r",
                 gamma="dgamma")
    for k, gk in pairs.items():
        np.testing.assert_allclose(g[gk], t[k].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)
