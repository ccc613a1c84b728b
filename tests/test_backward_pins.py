"""Pins of the backward oracle (oracle.prefill_backward) to facts outside its
own formulas (CPU only).

* central finite differences of the forward oracle's loss sum(dout * out)
  on tiny inputs -- every element of q, k, v and r, so a wrong sign, a
  dropped term, a transposed operand or a mis-sheared dr fails;
* torch.autograd through the forward oracle's logit rows and a library
  softmax, on larger inputs (GQA, windows, E beyond T);
* closed forms: a window of one key, and a single token, make out_i = v_i,
  so dq = dk = dr = 0 and dv is dout summed over the group's heads;
* invariants: rows of the softmax sum to one (sum over keys of dv), the
  gradient w.r.t. the logits sums to zero per row (sum over keys of dk, and
  dr = 0 for a bias constant over distance), alpha = 0 gives dq = dk = 0;
* the log-scale identity: log-scale on equals log-scale off with alpha*s and
  P*s;
* row / key sampling returns the same numbers as the full computation.
"""

import pytest
import torch

import oracle


def _case(B=1, T=7, Hq=4, Hkv=2, D=4, d_r=3, E=4, seed=0, p_scale=0.7):
    g = torch.Generator().manual_seed(seed)
    rnd = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)  # noqa: E731
    return dict(q=rnd(B, T, Hq, D), k=rnd(B, T, Hkv, D), v=rnd(B, T, Hkv, D), r=rnd(B, T, Hq, d_r),
                P=rnd(d_r, E) * p_scale, dout=rnd(B, T, Hq, D))


def _loss(x, alpha, E, W, log_scale=False):
    out, _ = oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], alpha, E, W, log_scale)
    return float((out * x["dout"]).sum())


@pytest.mark.parametrize("W", [0, 3])
def test_backward_matches_central_differences(W):
    x = _case()
    alpha, E = 0.9, 4
    dq, dk, dv, dr = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], alpha, E, W)
    eps = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("r", dr)):
        t = x[name]
        fd = torch.empty_like(t)
        flat, fdf = t.view(-1), fd.view(-1)
        for i in range(flat.numel()):
            keep = float(flat[i])
            flat[i] = keep + eps
            lp = _loss(x, alpha, E, W)
            flat[i] = keep - eps
            lm = _loss(x, alpha, E, W)
            flat[i] = keep
            fdf[i] = (lp - lm) / (2 * eps)
        assert torch.allclose(grad, fd, atol=1e-7, rtol=1e-6), f"d{name}: max diff {float((grad - fd).abs().max())}"


def _autograd(x, alpha, E, W):
    """Gradients by torch.autograd of sum(dout * softmax(logit_rows) @ V)."""
    q, k, v, r = (x[n].clone().requires_grad_(True) for n in ("q", "k", "v", "r"))
    B, T, Hq, _ = q.shape
    G = Hq // k.shape[2]
    pos = torch.arange(T)
    loss = 0.0
    for b in range(B):
        for h in range(Hq):
            lg = oracle.logit_rows(q[b, :, h], r[b, :, h], pos, k[b, :, h // G], x["P"], alpha, E, W, 1.0)
            o = torch.softmax(lg, dim=1) @ v[b, :, h // G]
            loss = loss + (o * x["dout"][b, :, h]).sum()
    loss.backward()
    return q.grad, k.grad, v.grad, r.grad


@pytest.mark.parametrize("T,Hq,Hkv,E,W", [(40, 4, 2, 12, 0), (40, 4, 1, 12, 9), (33, 2, 2, 50, 0), (30, 8, 2, 7, 7)])
def test_backward_matches_autograd(T, Hq, Hkv, E, W):
    x = _case(B=2, T=T, Hq=Hq, Hkv=Hkv, D=16, d_r=8, E=E, seed=T + E, p_scale=1.5)
    alpha = 0.3
    got = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], alpha, E, W)
    ref = _autograd(x, alpha, E, W)
    for name, a, b in zip("qkvr", got, ref):
        assert torch.allclose(a, b, atol=1e-12, rtol=1e-10), f"d{name}: max diff {float((a - b).abs().max())}"


@pytest.mark.parametrize("T,W", [(9, 1), (1, 0)])
def test_backward_single_visible_key_closed_form(T, W):
    x = _case(T=T, Hq=4, Hkv=2)
    dq, dk, dv, dr = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], 0.8, 4, W)
    assert torch.equal(dq, torch.zeros_like(dq)) and torch.equal(dk, torch.zeros_like(dk))
    assert torch.equal(dr, torch.zeros_like(dr))
    want = x["dout"].view(1, T, 2, 2, 4).sum(dim=3)  # dout summed over each kv head's query heads
    assert torch.allclose(dv, want, atol=1e-14)


def test_backward_sums_over_keys():
    x = _case(B=2, T=20, Hq=4, Hkv=2, D=6, d_r=5, E=6, seed=3)
    dq, dk, dv, dr = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], 0.5, 6, 5)
    # rows of p sum to one: sum_j dv_j = sum over queries and the group's heads of dout
    want = x["dout"].view(2, 20, 2, 2, 6).sum(dim=(1, 3))
    assert torch.allclose(dv.sum(dim=1), want, atol=1e-12)
    # the gradient w.r.t. each row's logits sums to zero: sum_j dk_j = 0
    assert dk.sum(dim=1).abs().max() < 1e-12


def test_backward_constant_bias_has_no_effect():
    """All columns of P equal and E >= T: every visible key gets the same bias,
    so dr = 0 and dq, dk, dv equal those with no bias."""
    x = _case(B=1, T=12, Hq=2, Hkv=1, D=5, d_r=3, E=16, seed=4)
    x["P"] = x["P"][:, :1].repeat(1, 16)
    dq, dk, dv, dr = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], 0.7, 16, 0)
    assert dr.abs().max() < 1e-12
    dq0, dk0, dv0, _ = oracle.prefill_backward(x["q"], x["k"], x["v"], None, None, x["dout"], 0.7, 0, 0)
    for a, b in ((dq, dq0), (dk, dk0), (dv, dv0)):
        assert torch.allclose(a, b, atol=1e-12)


def test_backward_alpha_zero_has_no_qk_gradient():
    x = _case(T=10, seed=5)
    dq, dk, dv, dr = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], 0.0, 4, 0)
    assert torch.equal(dq, torch.zeros_like(dq)) and torch.equal(dk, torch.zeros_like(dk))
    assert dr.abs().max() > 1e-3 and dv.abs().max() > 1e-3


def test_backward_gqa_equals_summed_mha():
    x = _case(B=1, T=15, Hq=6, Hkv=2, D=4, d_r=3, E=5, seed=6)
    g = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], 0.6, 5, 0)
    km, vm = x["k"].repeat_interleave(3, dim=2), x["v"].repeat_interleave(3, dim=2)
    m = oracle.prefill_backward(x["q"], km, vm, x["r"], x["P"], x["dout"], 0.6, 5, 0)
    assert torch.allclose(g[0], m[0], atol=1e-13) and torch.allclose(g[3], m[3], atol=1e-13)
    assert torch.allclose(g[1], m[1].view(1, 15, 2, 3, 4).sum(dim=3), atol=1e-13)
    assert torch.allclose(g[2], m[2].view(1, 15, 2, 3, 4).sum(dim=3), atol=1e-13)


def test_backward_log_scale_identity():
    """Log-scale on (s = ln T / ln 4096 = 7/6 at T = 16384) equals log-scale
    off with alpha*s and P*s."""
    T = 16384
    x = _case(B=1, T=T, Hq=2, Hkv=1, D=4, d_r=2, E=6, seed=7)
    s = oracle.scale_factor(T, True)
    assert abs(s - 7.0 / 6.0) < 1e-15
    rows, keys = [0, 5, 9000, T - 1], [0, 3, 9000, T - 2]
    a = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], 0.5, 6, 8, True, rows, keys)
    b = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"] * s, x["dout"], 0.5 * s, 6, 8, False, rows,
                                keys)
    for u, w in zip(a, b):
        assert torch.allclose(u, w, atol=1e-13, rtol=1e-12)
    c = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], 0.5, 6, 8, False, rows, keys)
    assert (a[0] - c[0]).abs().max() > 1e-3  # the scale is not a no-op here


def test_backward_sampling_equals_full():
    x = _case(B=2, T=25, Hq=4, Hkv=2, D=4, d_r=3, E=6, seed=8)
    full = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], 0.6, 6, 7, row_block=4)
    rows, keys = [24, 3, 0, 11], [0, 24, 12, 7]
    part = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"], x["P"], x["dout"], 0.6, 6, 7, rows=rows,
                                   key_rows=keys)
    assert torch.allclose(part[0], full[0][:, rows], atol=1e-14) and torch.allclose(part[3], full[3][:, rows],
                                                                                     atol=1e-14)
    assert torch.allclose(part[1], full[1][:, keys], atol=1e-14) and torch.allclose(part[2], full[2][:, keys],
                                                                                     atol=1e-14)
