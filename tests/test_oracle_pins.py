"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each check ties the oracle to something it does not compute itself: a
hand-worked example (tests/golden/), a scalar brute-force transcription of the
definitions, library softmax attention (torch SDPA) on special cases, closed
forms and invariants.  A plausible slip in the oracle -- a dropped term, a
wrong sign or index in the shear, an off-by-one at rel_extent or the window
edge, a transposed P, a wrong GQA mapping or scale -- fails at least one.
"""

import json
import math
import os

import pytest
import torch
import torch.nn.functional as F

import oracle
from transformer_attention_query_amd import inputs as tinputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _rand(shape, gen, scale=1.0):
    return torch.randn(*shape, generator=gen, dtype=torch.float64) * scale


def _small_case(B=1, T=9, Hq=2, Hkv=1, D=8, d_r=4, E=5, seed=0, p_scale=0.7):
    g = torch.Generator().manual_seed(seed)
    return dict(q=_rand((B, T, Hq, D), g), k=_rand((B, T, Hkv, D), g), v=_rand((B, T, Hkv, D), g),
                r=_rand((B, T, Hq, d_r), g), P=_rand((d_r, E), g, p_scale))


def _sdpa(q, k, v, mask, scale):
    """torch SDPA in fp64; q [B,T,Hq,D], k/v [B,T,Hkv,D] expanded to Hq by repeat_interleave."""
    G = q.shape[2] // k.shape[2]
    qh = q.permute(0, 2, 1, 3)
    kh = k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vh = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)
    return o.permute(0, 2, 1, 3)


def _visible(T, W):
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    vis = j <= i
    if W > 0:
        vis = vis & (i - j < W)
    return vis


# ---------------------------------------------------------------- golden example

def test_golden_worked_example_logits_and_rows():
    g = json.load(open(GOLDEN))
    t = lambda x: torch.tensor(x, dtype=torch.float64)  # noqa: E731
    q, k, v, r = t(g["q"]), t(g["k"]), t(g["v"]), t(g["r"])
    P = t(g["P_dr_by_E"])
    T = q.shape[0]
    for case in g["cases"]:
        lg = oracle.logit_rows(q, r, torch.arange(T), k, P, case["alpha"], 2, case["window"], 1.0)
        want = torch.tensor([[float("-inf") if x is None else float(x) for x in row] for row in case["logits"]],
                            dtype=torch.float64)
        assert torch.equal(lg, want), (case, lg)
        out, lse = oracle.prefill(q[None, :, None], k[None, :, None], v[None, :, None], r[None, :, None], P,
                                  case["alpha"], 2, case["window"])
        for row, o in case["out_rows"].items():
            assert torch.allclose(out[0, int(row), 0], t(o), atol=1e-15, rtol=0)
        for row, l in case["lse_rows"].items():
            val = 4.0 + math.log(2.0) if l == "4 + ln 2" else float(l)
            assert abs(lse[0, 0, int(row)].item() - val) < 1e-14
        # the remaining rows: softmax of the hand logits against v
        w = torch.softmax(want, dim=1)
        assert torch.allclose(out[0, :, 0], w @ v, atol=1e-14, rtol=0)


def test_log_scale_constants():
    g = json.load(open(GOLDEN))
    for L, s in g["log_scale_constants"]["values"]:
        assert abs(oracle.scale_factor(L, True) - s) < 1e-15
        assert oracle.scale_factor(L, False) == 1.0


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("T,Hq,Hkv,E,W,alpha", [
    (1, 1, 1, 3, 0, 0.35),
    (7, 2, 1, 0, 0, 0.35),
    (9, 2, 1, 1, 0, 0.35),
    (9, 4, 2, 5, 0, 0.35),
    (12, 2, 2, 12, 3, 0.5),
    (16, 4, 1, 4, 1, 0.35),
    (16, 2, 1, 20, 6, 1.0),
    (13, 3, 1, 13, 16, 0.2),
])
def test_brute_force_matches_oracle(T, Hq, Hkv, E, W, alpha):
    c = _small_case(B=2, T=T, Hq=Hq, Hkv=Hkv, E=max(E, 1), seed=T * 31 + E)
    out, lse = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], alpha, E, W)
    bo, bl = oracle.brute_force_prefill(c["q"].tolist(), c["k"].tolist(), c["v"].tolist(), c["r"].tolist(),
                                        c["P"].tolist(), alpha, E, W)
    assert torch.allclose(out, torch.tensor(bo, dtype=torch.float64), atol=1e-12, rtol=0)
    assert torch.allclose(lse, torch.tensor(bl, dtype=torch.float64), atol=1e-12, rtol=0)


# ---------------------------------------------------------------- library reductions

@pytest.mark.parametrize("W", [0, 1, 4, 50])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1), (6, 2)])
def test_zero_P_is_softmax_attention(W, Hq, Hkv):
    T = 23
    c = _small_case(B=2, T=T, Hq=Hq, Hkv=Hkv, D=16, E=8, seed=W + Hq)
    P0 = torch.zeros_like(c["P"])
    alpha = 0.3
    out, _ = oracle.prefill(c["q"], c["k"], c["v"], c["r"], P0, alpha, 8, W)
    ref = _sdpa(c["q"], c["k"], c["v"], _visible(T, W), alpha)
    assert torch.allclose(out, ref, atol=1e-12, rtol=0)


@pytest.mark.parametrize("E,W", [(1, 0), (5, 0), (11, 4), (30, 0), (6, 9)])
def test_sheared_bias_form_equals_definition(E, W):
    """Sheared-bias route (dense bias built entry by entry + library attention)
    equals the per-score definition."""
    T, Hq = 14, 2
    c = _small_case(B=1, T=T, Hq=Hq, Hkv=1, D=8, d_r=4, E=E, seed=E * 7 + W, p_scale=1.5)
    alpha = 0.4
    out, _ = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], alpha, E, W)
    sb = oracle.sheared_bias(c["r"][0], c["P"], T, E)                     # [T, H, T]
    mask = torch.where(_visible(T, W), 0.0, float("-inf")).to(torch.float64)
    attn_mask = sb.permute(1, 0, 2)[None] + mask                          # [1, H, T, T]
    ref = _sdpa(c["q"], c["k"], c["v"], attn_mask, alpha)
    assert torch.allclose(out, ref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("T,E,W", [(20, 6, 0), (20, 1, 0), (33, 10, 15), (12, 12, 0)])
def test_bias_stops_exactly_at_rel_extent(T, E, W):
    """alpha=0, r=e0 and P[0,:]=c: keys with i-j < E weigh e^c, farther visible keys weigh 1."""
    D, d_r, cval = 8, 4, 1.7
    g = torch.Generator().manual_seed(5)
    v = _rand((1, T, 1, D), g)
    q = _rand((1, T, 1, D), g)
    k = _rand((1, T, 1, D), g)
    r = torch.zeros(1, T, 1, d_r, dtype=torch.float64)
    r[..., 0] = 1.0
    P = torch.zeros(d_r, E, dtype=torch.float64)
    P[0, :] = cval
    out, lse = oracle.prefill(q, k, v, r, P, 0.0, E, W)
    ec = math.exp(cval)
    for i in range(T):
        lo = 0 if W == 0 else max(0, i - W + 1)
        near = [j for j in range(lo, i + 1) if i - j < E]
        far = [j for j in range(lo, i + 1) if i - j >= E]
        num = ec * v[0, near, 0].sum(0) + (v[0, far, 0].sum(0) if far else 0.0)
        den = ec * len(near) + len(far)
        assert torch.allclose(out[0, i, 0], num / den, atol=1e-13, rtol=0)
        assert abs(lse[0, 0, i].item() - math.log(den)) < 1e-13


@pytest.mark.parametrize("d0", [0, 1, 8])
def test_shear_direction_and_offset(d0):
    """alpha=0, r=e0, P[0,d0]=30: query i >= d0 puts weight e^30 on key i-d0 exactly."""
    T, E, D, d_r = 17, 9, 8, 4
    g = torch.Generator().manual_seed(d0)
    v = _rand((1, T, 1, D), g)
    q = _rand((1, T, 1, D), g)
    k = _rand((1, T, 1, D), g)
    r = torch.zeros(1, T, 1, d_r, dtype=torch.float64)
    r[..., 0] = 1.0
    P = torch.zeros(d_r, E, dtype=torch.float64)
    P[0, d0] = 30.0
    out, _ = oracle.prefill(q, k, v, r, P, 0.0, E, 0)
    big = math.exp(30.0)
    for i in range(T):
        if i >= d0:
            others = [j for j in range(i + 1) if j != i - d0]
            num = big * v[0, i - d0, 0] + (v[0, others, 0].sum(0) if others else 0.0)
            want = num / (big + len(others))
        else:
            want = v[0, : i + 1, 0].mean(0)
        assert torch.allclose(out[0, i, 0], want, atol=1e-13, rtol=0)


def test_constant_bias_rows_are_shift_invariant():
    """All P columns equal and E >= T: the bias is constant per row, so output equals P = 0."""
    T = 15
    c = _small_case(B=1, T=T, Hq=2, Hkv=1, E=T + 3, seed=3)
    col = c["P"][:, :1]
    Pc = col.expand(-1, T + 3).contiguous()
    out, _ = oracle.prefill(c["q"], c["k"], c["v"], c["r"], Pc, 0.5, T + 3, 0)
    out0, _ = oracle.prefill(c["q"], c["k"], c["v"], c["r"], torch.zeros_like(Pc), 0.5, T + 3, 0)
    assert torch.allclose(out, out0, atol=1e-12, rtol=0)


def test_window_at_least_T_equals_full_causal():
    T = 21
    c = _small_case(B=1, T=T, Hq=2, Hkv=1, E=7, seed=4)
    full, lf = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.5, 7, 0)
    for W in (T, T + 5):
        win, lw = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.5, 7, W)
        assert torch.equal(full, win) and torch.equal(lf, lw)


def test_window_one_and_single_token_return_v():
    c = _small_case(B=1, T=11, Hq=2, Hkv=1, E=4, seed=6)
    out, _ = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.5, 4, 1)
    assert torch.allclose(out, c["v"].repeat_interleave(2, dim=2), atol=1e-15, rtol=0)
    c1 = _small_case(B=1, T=1, Hq=2, Hkv=1, E=4, seed=7)
    out1, _ = oracle.prefill(c1["q"], c1["k"], c1["v"], c1["r"], c1["P"], 0.5, 4, 0)
    assert torch.allclose(out1, c1["v"].repeat_interleave(2, dim=2), atol=1e-15, rtol=0)


@pytest.mark.parametrize("W", [0, 5])
def test_weights_are_a_distribution(W):
    """Rows sum to one and masked entries are exactly zero; with V = identity the
    output row *is* the weight row."""
    T = 12
    c = _small_case(B=1, T=T, Hq=2, Hkv=1, D=T, E=6, seed=8)
    w = oracle.attention_weights(c["q"], c["k"], c["r"], c["P"], 0.5, 6, W)
    assert torch.allclose(w.sum(-1), torch.ones(1, 2, T, dtype=torch.float64), atol=1e-12, rtol=0)
    assert torch.all(w[..., ~_visible(T, W)] == 0)
    eye = torch.eye(T, dtype=torch.float64)[None, :, None, :]             # v_j = e_j
    out, _ = oracle.prefill(c["q"], c["k"], eye, c["r"], c["P"], 0.5, 6, W)
    assert torch.allclose(out[0].permute(1, 0, 2), w[0], atol=1e-14, rtol=0)


def test_log_scale_is_scaled_alpha_and_P():
    """Log-scale on == log-scale off with alpha*s and P*s (s scales q and the rel logits)."""
    T = 4100                                     # just above 4096 so s > 1
    s = oracle.scale_factor(T, True)
    assert s > 1.0
    c = _small_case(B=1, T=T, Hq=2, Hkv=1, D=8, d_r=4, E=40, seed=9)
    rows = [0, 1, 39, 40, 2000, T - 1]
    a, la = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.3, 40, 0, True, rows=rows)
    b, lb = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"] * s, 0.3 * s, 40, 0, False, rows=rows)
    assert torch.allclose(a, b, atol=1e-12, rtol=0) and torch.allclose(la, lb, atol=1e-10, rtol=0)
    # and it is not a no-op
    c2, _ = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.3, 40, 0, False, rows=rows)
    assert (a - c2).abs().max() > 1e-6


def test_gqa_equals_mha_with_repeated_kv():
    c = _small_case(B=2, T=10, Hq=6, Hkv=2, E=5, seed=10)
    a, la = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.5, 5, 3)
    k3 = c["k"].repeat_interleave(3, dim=2)
    v3 = c["v"].repeat_interleave(3, dim=2)
    b, lb = oracle.prefill(c["q"], k3, v3, c["r"], c["P"], 0.5, 5, 3)
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("log_scale,W,L", [(False, 0, 30), (False, 7, 30), (True, 0, 5000), (False, 0, 1)])
def test_decode_equals_last_prefill_row(log_scale, W, L):
    c = _small_case(B=2, T=L, Hq=4, Hkv=2, D=8, d_r=4, E=12, seed=L + W)
    pre, lpre = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.4, 12, W, log_scale, rows=[L - 1])
    dec, ldec = oracle.decode(c["q"][:, L - 1], c["k"], c["v"], c["r"][:, L - 1], c["P"], 0.4, 12, W, log_scale)
    assert torch.allclose(dec, pre[:, 0], atol=1e-13, rtol=0)
    assert torch.allclose(ldec, lpre[:, :, 0], atol=1e-12, rtol=0)


def test_row_subset_equals_full():
    c = _small_case(B=2, T=40, Hq=2, Hkv=1, E=9, seed=11)
    full, lf = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.5, 9, 0, row_block=7)
    rows = [0, 3, 17, 39]
    sub, ls = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.5, 9, 0, rows=rows)
    assert torch.allclose(sub, full[:, rows], atol=1e-14, rtol=0)
    assert torch.allclose(ls, lf[:, :, rows], atol=1e-14, rtol=0)


def test_rel_logits_entrywise_and_basis():
    g = torch.Generator().manual_seed(12)
    r = _rand((3, 2, 5), g)
    P = _rand((5, 7), g)
    rl = oracle.rel_logits(r, P, 1.5)
    for t in range(3):
        for h in range(2):
            for d in range(7):
                want = 1.5 * math.fsum(r[t, h, c].item() * P[c, d].item() for c in range(5))
                assert abs(rl[t, h, d].item() - want) < 1e-12
    # r = e_c picks row c of P (P's columns are indexed by distance)
    eye = torch.eye(5, dtype=torch.float64)
    assert torch.equal(oracle.rel_logits(eye, P), P)


def test_oracle_accepts_bf16_inputs_exactly():
    """The oracle upcasts the exact device values; no re-rounding on the way."""
    c = tinputs.make_prefill_inputs(1, 12, 2, 1, 16, 16, 6, "bf16", seed=3)
    a, _ = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.25, 6, 0)
    b, _ = oracle.prefill(*(c[n].double() for n in ("q", "k", "v", "r", "P")), 0.25, 6, 0)
    assert torch.equal(a, b)


# ---------------------------------------------------------------- extend (chunked prefill over a cache)

def _extend_from_full(seqs, n_new):
    """Pack the last n_new[b] rows of full sequences (dicts of [1,T,...] tensors) as extend inputs."""
    q = torch.cat([c["q"][0, c["q"].shape[1] - n:] for c, n in zip(seqs, n_new)])
    r = torch.cat([c["r"][0, c["r"].shape[1] - n:] for c, n in zip(seqs, n_new)])
    Lcap = max(c["k"].shape[1] for c in seqs)
    Hkv, D = seqs[0]["k"].shape[2], seqs[0]["k"].shape[3]
    k = torch.zeros(len(seqs), Lcap, Hkv, D, dtype=torch.float64)
    v = torch.zeros_like(k)
    for b, c in enumerate(seqs):
        k[b, :c["k"].shape[1]] = c["k"][0]
        v[b, :c["v"].shape[1]] = c["v"][0]
    q_start = [0]
    for n in n_new:
        q_start.append(q_start[-1] + n)
    return q, r, k, v, q_start, [c["q"].shape[1] for c in seqs]


@pytest.mark.parametrize("log_scale,W", [(False, 0), (False, 6), (True, 0)])
def test_extend_rows_equal_prefill_of_whole_sequence(log_scale, W):
    """Chunked prefill is exact: the new rows over a cached prefix are the last
    rows of the prefill of the whole sequence (s from its full length)."""
    Ts = [4200, 4500] if log_scale else [23, 40]
    n_new = [5, 17]
    seqs = [_small_case(B=1, T=T, Hq=4, Hkv=2, D=8, d_r=4, E=9, seed=T) for T in Ts]
    for c in seqs:
        c["P"] = seqs[0]["P"]
    q, r, k, v, q_start, kv_len = _extend_from_full(seqs, n_new)
    out, lse = oracle.extend(q, k, v, r, seqs[0]["P"], 0.4, 9, W, log_scale, q_start, kv_len)
    for b, (c, n) in enumerate(zip(seqs, n_new)):
        T = c["q"].shape[1]
        rows = list(range(T - n, T))
        ref, lref = oracle.prefill(c["q"], c["k"], c["v"], c["r"], c["P"], 0.4, 9, W, log_scale, rows=rows)
        assert torch.allclose(out[q_start[b]:q_start[b + 1]], ref[0], atol=1e-13, rtol=0)
        assert torch.allclose(lse[:, q_start[b]:q_start[b + 1]], lref[0], atol=1e-12, rtol=0)


def test_extend_matches_brute_force_and_skips_empty_sequences():
    """Scalar brute force on tiny sequences; a sequence with no new rows
    contributes nothing, and one with no prefix is a plain prefill."""
    seqs = [_small_case(B=1, T=T, Hq=2, Hkv=1, D=4, d_r=3, E=4, seed=30 + T) for T in (7, 5, 6)]
    for c in seqs:
        c["P"] = seqs[0]["P"]
    n_new = [3, 0, 6]
    q, r, k, v, q_start, kv_len = _extend_from_full(seqs, n_new)
    out, lse = oracle.extend(q, k, v, r, seqs[0]["P"], 0.6, 4, 0, False, q_start, kv_len)
    for b, (c, n) in enumerate(zip(seqs, n_new)):
        if n == 0:
            continue
        T = c["q"].shape[1]
        bo, bl = oracle.brute_force_prefill(c["q"].tolist(), c["k"].tolist(), c["v"].tolist(), c["r"].tolist(),
                                            c["P"].tolist(), 0.6, 4, 0)
        for t in range(n):
            i = T - n + t
            for h in range(2):
                assert max(abs(x - y) for x, y in zip(out[q_start[b] + t, h].tolist(), bo[0][i][h])) < 1e-12
                assert abs(lse[h, q_start[b] + t].item() - bl[0][h][i]) < 1e-12


def test_extend_paged_cache_equals_contiguous():
    """A paged cache (pages at a shuffled permutation of slots) holds the same rows."""
    x = tinputs.make_extend_inputs([70, 9, 64], [11, 9, 1], 4, 2, 16, 16, 12, "bf16", seed=4, page_size=8)
    qs, kl = x["q_start"].tolist(), x["kv_len"].tolist()
    a, la = oracle.extend(x["q"], x["k"], x["v"], x["r"], x["P"], 0.3, 12, 0, False, qs, kl)
    b, lb = oracle.extend(x["q"], x["k_pages"], x["v_pages"], x["r"], x["P"], 0.3, 12, 0, False, qs, kl,
                          block_table=x["block_table"].tolist(), page_size=8)
    assert torch.equal(a, b) and torch.equal(la, lb)
    # the page permutation really is a permutation (no two pages share a slot)
    used = [x["block_table"][bb, p].item() for bb, L in enumerate(kl) for p in range((L + 7) // 8)]
    assert sorted(used) == list(range(len(used)))


@pytest.mark.parametrize("log_scale", [False, True])
def test_decode_equals_extend_of_one_row(log_scale):
    L = 4300 if log_scale else 50
    c = _small_case(B=2, T=L, Hq=4, Hkv=2, D=8, d_r=4, E=12, seed=77)
    dec, ldec = oracle.decode(c["q"][:, L - 1], c["k"], c["v"], c["r"][:, L - 1], c["P"], 0.4, 12, 0, log_scale)
    ext, lext = oracle.extend(c["q"][:, L - 1], c["k"], c["v"], c["r"][:, L - 1], c["P"], 0.4, 12, 0, log_scale,
                              [0, 1, 2], [L, L])
    assert torch.allclose(ext, dec, atol=1e-13, rtol=0)
    assert torch.allclose(lext, ldec.t(), atol=1e-12, rtol=0)
