"""GPU parity of the attention prologue (rel_attn_prologue) through the C ABI
against the fp64 oracle: fresh sequences and continued ones (carried state),
contiguous and paged caches, sequences with no new token or fewer new tokens
than the filter's reach, token blocks that span several sequences, widths 1..4,
in-place q, fp32, and the full 8192-token shape of the bench.

Tolerance (the pages state none for this step; derived from the arithmetic):
the kernel computes in fp32 and rounds each output once to the dtype, so a
bf16 output is within half a bf16 ulp (2^-9 relative) of the exact value plus
the fp32 error; the test allows |got - ref| <= 2^-8 |ref| + 1e-4.  fp32
outputs: |got - ref| <= 1e-5 |ref| + 1e-5.  Cache rows that no new token maps
to, and the raw state rows, must be bit-identical to what they were / to the
input rows."""

import zlib

import pytest
import torch

import oracle
import transformer_attention_query_amd as ra
from transformer_attention_query_amd import inputs as tinputs

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _close(got, ref, dtype, what):
    got = got.detach().cpu().to(torch.float64)
    ref = ref.to(torch.float64)
    rel, ab = (2.0 ** -8, 1e-4) if dtype == torch.bfloat16 else (1e-5, 1e-5)
    err = (got - ref).abs()
    bound = rel * ref.abs() + ab
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {err.numel()} entries off; worst "
                           f"{float((err - bound).max()):.3e} over the bound")


def _run(x, page_size, with_state, in_place=False, state_out=True):
    xd = {n: t.cuda() for n, t in x.items()}
    paged = page_size > 0
    kc = (xd["k_pages"] if paged else xd["k_cache"]).clone()
    vc = (xd["v_pages"] if paged else xd["v_cache"]).clone()
    B = xd["kv_len"].shape[0]
    Hkv, D = xd["k"].shape[1], xd["k"].shape[2]
    so = torch.full((B, 2, 3, Hkv * D), 7.0, dtype=xd["q"].dtype, device="cuda") if state_out else None
    q_out = xd["q"].clone() if in_place else None
    q_in = q_out if in_place else xd["q"]
    res = ra.prologue(q_in, xd["k"], xd["v"], xd["conv_k"], xd["conv_v"], xd["q_norm_w"], xd["k_norm_w"], EPS,
                      xd["q_start"], xd["kv_len"], kc, vc, block_table=xd["block_table"] if paged else None,
                      state_in=xd["state_in"] if with_state else None, state_out=so, q_out=q_out)
    torch.cuda.synchronize()
    if in_place:
        assert res.data_ptr() == q_out.data_ptr()
    return res, kc, vc, so


def _check(x, res, kc, vc, so, page_size, with_state, name):
    dt = x["q"].dtype
    qs = x["q_start"].tolist()
    st = x["state_in"] if with_state else None
    q_ref, k_ref, v_ref, s_ref = oracle.prologue(x["q"], x["k"], x["v"], x["conv_k"], x["conv_v"], x["q_norm_w"],
                                                 x["k_norm_w"], EPS, qs, st)
    _close(res, q_ref, dt, f"{name} q_out")
    kc, vc = kc.cpu(), vc.cpu()
    written = set()
    for row, (b, pos) in enumerate(oracle.cache_positions(qs, x["kv_len"].tolist())):
        if page_size > 0:
            slot = (int(x["block_table"][b, pos // page_size]), pos % page_size)
        else:
            slot = (b, pos)
        written.add(slot)
        _close(kc[slot], k_ref[row], dt, f"{name} k cache row {row}")
        _close(vc[slot], v_ref[row], dt, f"{name} v cache row {row}")
    prior_k = x["k_pages"] if page_size > 0 else x["k_cache"]
    prior_v = x["v_pages"] if page_size > 0 else x["v_cache"]
    for i in range(kc.shape[0]):
        for j in range(kc.shape[1]):
            if (i, j) not in written:
                assert torch.equal(kc[i, j], prior_k[i, j]) and torch.equal(vc[i, j], prior_v[i, j]), \
                    f"{name}: cache row {(i, j)} changed though no new token maps to it"
    if so is not None:
        assert torch.equal(so.cpu(), s_ref.to(dt)), f"{name}: state_out differs from the raw rows"


# name, dtype, kv_lens, new_lens, Hq, Hkv, W, page_size, with_state
CASES = [
    ("fresh_one_seq_ragged", "bf16", [300], [300], 8, 1, 4, 0, False),
    ("extend_state_paged16", "bf16", [50, 10, 40, 9], [17, 0, 40, 2], 8, 2, 4, 16, True),
    ("many_short_seqs_one_block", "bf16", [3, 1, 5, 2, 7, 1, 4], [3, 1, 5, 2, 7, 1, 4], 4, 2, 4, 0, True),
    ("decode_rows_paged64", "bf16", [200, 64, 129], [1, 1, 1], 16, 2, 4, 64, True),
    ("width3_contig", "bf16", [70, 33], [20, 33], 4, 1, 3, 0, True),
    ("width1_contig", "bf16", [40], [40], 2, 2, 1, 0, False),
    ("fp32_paged32", "fp32", [90, 200], [90, 45], 4, 2, 4, 32, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prologue_matches_oracle(case):
    name, dt, kv_lens, new_lens, Hq, Hkv, W, page, ws = case
    x = tinputs.make_prologue_inputs(kv_lens, new_lens, Hq, Hkv, 128, W, dt, seed=zlib.crc32(name.encode()) % 1000,
                                     page_size=page, with_state=ws)
    res, kc, vc, so = _run(x, page, ws)
    _check(x, res, kc, vc, so, page, ws, name)


def test_prologue_in_place_q():
    x = tinputs.make_prologue_inputs([64, 30], [64, 12], 8, 1, 128, 4, "bf16", seed=5, with_state=True)
    res, kc, vc, so = _run(x, 0, True, in_place=True)
    _check(x, res, kc, vc, so, 0, True, "in_place")


def test_prologue_chunks_with_carried_state_equal_one_call():
    """Bit-identical: the same sequence in one call, or in two calls with the
    first call's state_out passed to the second."""
    x = tinputs.make_prologue_inputs([100], [100], 4, 2, 128, 4, "bf16", seed=9, with_state=False)
    whole, kw, vw, sw = _run(x, 0, False)
    split = 37
    x1 = dict(x)
    for n in ("q", "k", "v"):
        x1[n] = x[n][:split]
    x1["q_start"] = torch.tensor([0, split], dtype=torch.int32)
    x1["kv_len"] = torch.tensor([split], dtype=torch.int32)
    a, ka, va, sa = _run(x1, 0, False)
    x2 = dict(x)
    for n in ("q", "k", "v"):
        x2[n] = x[n][split:]
    x2["q_start"] = torch.tensor([0, 100 - split], dtype=torch.int32)
    x2["kv_len"] = torch.tensor([100], dtype=torch.int32)
    x2["state_in"] = sa.cpu()
    x2["k_cache"], x2["v_cache"] = ka.cpu(), va.cpu()
    b, kb, vb, sb = _run(x2, 0, True)
    assert torch.equal(torch.cat([a, b]), whole)
    assert torch.equal(kb, kw) and torch.equal(vb, vw) and torch.equal(sb, sw)


def test_prologue_state_only_call_carries_states():
    """No new token at all: state_out receives state_in."""
    x = tinputs.make_prologue_inputs([5, 9], [0, 0], 4, 1, 128, 4, "bf16", seed=3, with_state=True)
    res, kc, vc, so = _run(x, 0, True)
    assert torch.equal(so.cpu(), x["state_in"])


@pytest.mark.parametrize("name", ["prologue_8k", "prologue_decode_64"])
def test_prologue_full_workloads(name):
    w = tinputs.WORKLOADS[name]
    x = tinputs.make_inputs(w, seed=0)
    ws = "state_in" in x
    res, kc, vc, so = _run(x, w.page_size, ws)
    dt = x["q"].dtype
    qs = x["q_start"].tolist()
    q_ref, k_ref, v_ref, s_ref = oracle.prologue(x["q"], x["k"], x["v"], x["conv_k"], x["conv_v"], x["q_norm_w"],
                                                 x["k_norm_w"], EPS, qs, x.get("state_in"))
    _close(res, q_ref, dt, f"{name} q_out")
    pos = oracle.cache_positions(qs, x["kv_len"].tolist())
    idx_b = torch.tensor([b for b, _ in pos])
    idx_p = torch.tensor([p for _, p in pos])
    if w.page_size > 0:
        pg = x["block_table"][idx_b, idx_p // w.page_size].long()
        kg, vg = kc.cpu()[pg, idx_p % w.page_size], vc.cpu()[pg, idx_p % w.page_size]
    else:
        kg, vg = kc.cpu()[idx_b, idx_p], vc.cpu()[idx_b, idx_p]
    _close(kg, k_ref, dt, f"{name} k rows")
    _close(vg, v_ref, dt, f"{name} v rows")
    assert torch.equal(so.cpu(), s_ref.to(dt))
