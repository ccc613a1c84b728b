"""Pins of the prologue oracle (CPU only): ShortConv against torch's conv1d
and closed forms, RMSNorm against torch's rms_norm and the unit-RMS
invariant, and the chunking invariance of the carried state.  A slip in the
oracle -- a reversed filter, a tap on the wrong side, a dropped residual, a
norm over the wrong axis, a stale state row -- fails at least one."""

import pytest
import torch
import torch.nn.functional as F

import oracle


def _r(shape, g, scale=1.0):
    return torch.randn(*shape, generator=g, dtype=torch.float64) * scale


def test_short_conv_zero_filter_is_identity():
    g = torch.Generator().manual_seed(1)
    x = _r((7, 5), g)
    assert torch.equal(oracle.short_conv(x, torch.zeros(5, 4, dtype=torch.float64)), x)


def test_short_conv_current_tap_doubles():
    g = torch.Generator().manual_seed(2)
    x = _r((6, 3), g)
    w = torch.zeros(3, 4, dtype=torch.float64)
    w[:, 0] = 1.0
    assert torch.equal(oracle.short_conv(x, w), 2 * x)


@pytest.mark.parametrize("d", [1, 2, 3])
def test_short_conv_shift_taps(d):
    """w[:, d] = 1: y[t] = x[t] + x[t-d], with x[t-d] from the state before the chunk."""
    g = torch.Generator().manual_seed(3 + d)
    x, st = _r((6, 4), g), _r((3, 4), g)
    w = torch.zeros(4, 4, dtype=torch.float64)
    w[:, d] = 1.0
    y = oracle.short_conv(x, w, st)
    full = torch.cat([st, x])
    for t in range(6):
        assert torch.equal(y[t], x[t] + full[3 + t - d])
    y0 = oracle.short_conv(x, w)  # no state: zeros before the chunk
    for t in range(6):
        assert torch.equal(y0[t], x[t] + (x[t - d] if t >= d else torch.zeros(4, dtype=torch.float64)))


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_short_conv_equals_depthwise_conv1d(W):
    """Library routine: a depthwise causal conv1d (cross-correlation with the
    filter reversed) over the state-padded rows, plus the residual."""
    g = torch.Generator().manual_seed(10 + W)
    n, C = 9, 6
    x, w, st = _r((n, C), g), _r((C, W), g), _r((3, C), g)
    y = oracle.short_conv(x, w, st)
    xs = torch.cat([st, x]).t().unsqueeze(0)            # [1, C, 3 + n]
    wk = torch.zeros(C, 4, dtype=torch.float64)
    wk[:, :W] = w
    ker = wk.flip(1).unsqueeze(1)                        # [C, 1, 4]: ker[k] = w[3 - k]
    ref = F.conv1d(xs, ker, groups=C)[0].t() + x         # [n, C]
    assert torch.allclose(y, ref, rtol=0, atol=1e-12)


def test_rms_norm_equals_torch_and_has_unit_rms():
    g = torch.Generator().manual_seed(20)
    x, wt = _r((5, 3, 16), g, 3.0), _r((16,), g)
    assert torch.allclose(oracle.rms_norm(x, wt, 1e-6), F.rms_norm(x, (16,), wt, 1e-6), rtol=0, atol=1e-12)
    y = oracle.rms_norm(x, torch.ones(16, dtype=torch.float64), 0.0)
    assert torch.allclose((y * y).mean(-1), torch.ones(5, 3, dtype=torch.float64), rtol=0, atol=1e-12)
    assert torch.allclose(oracle.rms_norm(7.5 * x, wt, 0.0), oracle.rms_norm(x, wt, 0.0), rtol=0, atol=1e-12)


def _case(B_lens, Hq=4, Hkv=2, D=8, W=4, seed=0):
    g = torch.Generator().manual_seed(seed)
    N = sum(B_lens)
    qs = [0]
    for n in B_lens:
        qs.append(qs[-1] + n)
    return dict(q=_r((N, Hq, D), g), k=_r((N, Hkv, D), g), v=_r((N, Hkv, D), g), conv_k=_r((Hkv * D, W), g, 0.5),
                conv_v=_r((Hkv * D, W), g, 0.5), q_norm_w=_r((D,), g), k_norm_w=_r((D,), g), q_start=qs)


def test_prologue_is_the_composition_of_its_parts():
    c = _case([5, 1, 7])
    q_out, k_new, v_new, st = oracle.prologue(c["q"], c["k"], c["v"], c["conv_k"], c["conv_v"], c["q_norm_w"],
                                              c["k_norm_w"], 1e-6, c["q_start"])
    assert torch.allclose(q_out, F.rms_norm(c["q"], (8,), c["q_norm_w"], 1e-6), rtol=0, atol=1e-12)
    qs = c["q_start"]
    for b in range(3):
        rows = slice(qs[b], qs[b + 1])
        n = qs[b + 1] - qs[b]
        kc = oracle.short_conv(c["k"][rows].reshape(n, 16), c["conv_k"])
        assert torch.allclose(k_new[rows], F.rms_norm(kc.reshape(n, 2, 8), (8,), c["k_norm_w"], 1e-6), atol=1e-12)
        assert torch.allclose(v_new[rows].reshape(n, 16), oracle.short_conv(c["v"][rows].reshape(n, 16), c["conv_v"]),
                              atol=1e-12)
        # state: the last three raw rows, zeros where the sequence is shorter
        raw_k = torch.cat([torch.zeros(3, 16, dtype=torch.float64), c["k"][rows].reshape(n, 16)])[-3:]
        assert torch.equal(st[b, 0], raw_k)


@pytest.mark.parametrize("split", [1, 2, 3, 5])
def test_prologue_chunks_with_carried_state_equal_one_call(split):
    """A sequence processed in two calls, the first call's state_out fed to the
    second, gives the rows and final state of one call over the whole sequence."""
    c = _case([8], seed=split)
    args = (c["conv_k"], c["conv_v"], c["q_norm_w"], c["k_norm_w"], 1e-5)
    whole = oracle.prologue(c["q"], c["k"], c["v"], *args, [0, 8])
    a = oracle.prologue(c["q"][:split], c["k"][:split], c["v"][:split], *args, [0, split])
    b = oracle.prologue(c["q"][split:], c["k"][split:], c["v"][split:], *args, [0, 8 - split], state=a[3])
    for i in range(3):
        assert torch.allclose(torch.cat([a[i], b[i]]), whole[i], rtol=0, atol=1e-12)
    assert torch.equal(b[3], whole[3])


def test_cache_positions_follow_extend():
    assert oracle.cache_positions([0, 2, 2, 5], [4, 9, 3]) == [(0, 2), (0, 3), (2, 0), (2, 1), (2, 2)]
