"""GPU: the two ways the decode kernels get the relative bias, each against
the oracle, with the path taken checked from the outside.

A decode workgroup whose split holds keys within rel_extent of the query
makes the bias of those keys in LDS when the region fits the LDS budget of
the kernel's occupancy; otherwise the rel_logits kernel first writes bias
rows into the workspace, after the split partials, and the split kernel
reads them from there.  The workspace is filled with a sentinel byte before
the call: the bias-row part is overwritten exactly when the pre-pass ran.

The pre-pass cases are the shapes where min(rel_extent, keys per split) is
large next to the LDS budget: sixteen query heads per kv head with E = 2048
(bf16, contiguous and paged, with cache lengths covering every value of
kv_len % 4, which sets the per-sequence shift of the paged bias rows), the
MXFP8 caches, and fp32 at one workgroup per CU with min(E, chunk) >= 1400."""

import zlib

import pytest
import torch

import oracle
import transformer_attention_query_amd as ra
from transformer_attention_query_amd import inputs as tinputs
from parity import assert_close

pytestmark = pytest.mark.gpu

ALPHA = 1.0 / 128 ** 0.5
SENTINEL = 0xA5


def _workspace(B, L, Hq, Hkv, ns, W, E):
    ns, nbytes = ra.decode_plan(B, L, Hq, Hkv, 128, ns, W, E)
    partial = (ns * B * Hq * (128 + 2) * 4 + 255) // 256 * 256
    ws = torch.full((nbytes,), SENTINEL, dtype=torch.uint8, device="cuda")
    return ns, ws, partial


def _prepass_ran(ws, partial):
    torch.cuda.synchronize()
    tail = ws[partial:]
    assert tail.numel() > 0
    return bool((tail != SENTINEL).any().item())


def _seed(name):
    return zlib.crc32(name.encode()) % 1000


# name, dtype, B, L, Hq, Hkv, d_r, E, W, log_scale, num_splits, pre-pass expected
CONTIGUOUS = [
    ("bf16_g16_E2048_s1", "bf16", 1, 3000, 16, 1, 128, 2048, 0, False, 1, True),
    ("bf16_g16_E2048_s2_log", "bf16", 2, 4500, 16, 1, 64, 2048, 0, True, 2, True),
    ("bf16_g16_E2048_W2500", "bf16", 1, 4000, 32, 2, 128, 2048, 2500, False, 1, True),
    ("fp32_g16_E1500_s1", "fp32", 1, 2000, 16, 1, 128, 1500, 0, False, 1, True),
    ("fp32_g16_E2048_s2", "fp32", 2, 3100, 16, 1, 32, 2048, 0, False, 2, True),
    # the in-LDS path next to them
    ("bf16_g8_E1024_lds", "bf16", 2, 3000, 16, 2, 128, 1024, 0, False, 0, False),
    ("fp32_g16_E1024_lds", "fp32", 1, 2000, 16, 1, 128, 1024, 0, False, 1, False),
    # the first splits one quantum longer than the last: the bias keys then
    # span the last two splits
    ("bf16_g8_E1200_lead_s2", "bf16", 2, 2000, 16, 2, 128, 1200, 0, False, 2, False),
    ("bf16_g8_E1024_lead_s4", "bf16", 1, 4000, 16, 2, 128, 1024, 0, False, 4, False),
]


@pytest.mark.parametrize("case", CONTIGUOUS, ids=[c[0] for c in CONTIGUOUS])
def test_decode_bias_path_matches_oracle(case):
    name, dt, B, L, Hq, Hkv, d_r, E, W, ls, ns, prepass = case
    x = tinputs.make_decode_inputs(B, L, Hq, Hkv, 128, d_r, E, dt, seed=_seed(name))
    xd = {n: t.cuda() for n, t in x.items()}
    ns, ws, partial = _workspace(B, L, Hq, Hkv, ns, W, E)
    out, lse = ra.decode(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], ALPHA, E, W, ls, num_splits=ns,
                         workspace=ws)
    assert _prepass_ran(ws, partial) == prepass
    ref, lref = oracle.decode(x["q"], x["k"], x["v"], x["r"], x["P"], ALPHA, E, W, ls)
    assert_close(out, ref, x["q"].dtype, name, lse, lref)


# name, dtype, kv_lens, Hq, Hkv, d_r, E, W, log_scale, page_size, num_splits, pre-pass expected
PAGED = [
    # kv_len % 4 = 0, 1, 2, 3 (and short sequences whose splits are empty)
    ("bf16_g16_E2048_mod4", "bf16", [3000, 2049, 2502, 1999, 7, 640], 16, 1, 128, 2048, 0, False, 64, 1, True),
    ("bf16_g16_E2048_mod4_s2_log", "bf16", [4096, 3333, 2050, 2767], 16, 1, 64, 2048, 0, True, 32, 2, True),
    ("bf16_g16_E2048_W1500", "bf16", [3001, 2222, 1500], 16, 1, 128, 2048, 1500, False, 128, 1, True),
    ("fp32_g16_E1600_mod4", "fp32", [1800, 1601, 1702, 1403], 16, 1, 32, 1600, 0, False, 32, 1, True),
    ("bf16_g16_E600_lds", "bf16", [3000, 2049, 2502, 1999], 16, 1, 128, 600, 0, False, 64, 1, False),
    # two splits, the first one quantum longer: the bias of the shorter
    # sequences spans both, one sequence has no keys in the second
    ("bf16_g8_E1000_lead_s2", "bf16", [2000, 1500, 1999, 64], 16, 2, 128, 1000, 0, False, 64, 2, False),
]


@pytest.mark.parametrize("case", PAGED, ids=[c[0] for c in PAGED])
def test_decode_paged_bias_path_matches_oracle(case):
    name, dt, kv_lens, Hq, Hkv, d_r, E, W, ls, page, ns, prepass = case
    B = len(kv_lens)
    x = tinputs.make_extend_inputs(kv_lens, [1] * B, Hq, Hkv, 128, d_r, E, dt, seed=_seed(name), page_size=page)
    xd = {n: t.cuda() for n, t in x.items()}
    L = max(kv_lens)
    ns, ws, partial = _workspace(B, L, Hq, Hkv, ns, W, E)
    out, lse = ra.decode_paged(xd["q"], xd["k_pages"], xd["v_pages"], xd["r"], xd["P_cols"], ALPHA, E, W, ls,
                               xd["kv_len"], xd["block_table"], L, num_splits=ns, workspace=ws)
    assert _prepass_ran(ws, partial) == prepass
    ref, lref = oracle.extend(x["q"], x["k_pages"], x["v_pages"], x["r"], x["P"], ALPHA, E, W, ls,
                              x["q_start"].tolist(), kv_lens, block_table=x["block_table"].tolist(),
                              page_size=page)
    assert_close(out, ref, x["q"].dtype, name, lse, lref.t())


def test_decode_mx_contiguous_prepass_matches_oracle():
    B, L, Hq, Hkv, d_r, E = 2, 3000, 16, 1, 128, 2048
    x = tinputs.make_decode_inputs(B, L, Hq, Hkv, 128, d_r, E, "bf16", seed=31)
    kc, ks = ra.mx_quantize(x["k"].cuda())
    vc, vs = ra.mx_quantize(x["v"].cuda())
    ns, ws, partial = _workspace(B, L, Hq, Hkv, 1, 0, E)
    out, lse = ra.decode_mx(x["q"].cuda(), kc, ks, vc, vs, x["r"].cuda(), x["P_cols"].cuda(), ALPHA, E, 0, True,
                            num_splits=ns, workspace=ws)
    assert _prepass_ran(ws, partial)
    qd, kd, vd = oracle.mx_round(x["q"]), oracle.mx_round(x["k"]), oracle.mx_round(x["v"])
    ref, lref = oracle.decode(qd, kd, vd, x["r"], x["P"], ALPHA, E, 0, True)
    assert_close(out, ref, torch.bfloat16, "mx contiguous pre-pass", lse, lref)


def test_decode_mx_paged_prepass_matches_oracle():
    kv_lens = [3000, 2049, 2502, 1999]
    Hq, Hkv, d_r, E, page = 16, 1, 128, 2048, 64
    x = tinputs.make_extend_inputs(kv_lens, [1] * 4, Hq, Hkv, 128, d_r, E, "bf16", seed=32, page_size=page)
    kc, ks = ra.mx_quantize(x["k_pages"].cuda())
    vc, vs = ra.mx_quantize(x["v_pages"].cuda())
    L = max(kv_lens)
    ns, ws, partial = _workspace(4, L, Hq, Hkv, 1, 0, E)
    out, lse = ra.decode_mx(x["q"].cuda(), kc, ks, vc, vs, x["r"].cuda(), x["P_cols"].cuda(), ALPHA, E, 0, False,
                            L=L, kv_len=x["kv_len"].cuda(), block_table=x["block_table"].cuda(), num_splits=ns,
                            workspace=ws)
    assert _prepass_ran(ws, partial)
    ref, lref = oracle.extend(oracle.mx_round(x["q"]), oracle.mx_round(x["k"]), oracle.mx_round(x["v"]), x["r"],
                              x["P"], ALPHA, E, 0, False, x["q_start"].tolist(), kv_lens)
    assert_close(out, ref, torch.bfloat16, "mx paged pre-pass", lse, lref.t().contiguous())


@pytest.mark.parametrize("form", ["contiguous", "paged"])
def test_decode_is_deterministic(form):
    """Two calls on the same inputs give the same bits (no atomics, fixed split
    and merge order)."""
    if form == "contiguous":
        x = {n: t.cuda() for n, t in tinputs.make_decode_inputs(8, 8192, 16, 2, 128, 128, 1024, "bf16",
                                                                 seed=33).items()}
        run = lambda: ra.decode(x["q"], x["k"], x["v"], x["r"], x["P_cols"], ALPHA, 1024)  # noqa: E731
    else:
        kv_lens = [8192, 5000, 77, 4097]
        x = {n: t.cuda() for n, t in tinputs.make_extend_inputs(kv_lens, [1] * 4, 16, 2, 128, 128, 1024, "bf16",
                                                                 seed=34, page_size=64).items()}
        run = lambda: ra.decode_paged(x["q"], x["k_pages"], x["v_pages"], x["r"], x["P_cols"], ALPHA,  # noqa: E731
                                      1024, 0, True, x["kv_len"], x["block_table"], 8192)
    a, la = run()
    b, lb = run()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)
