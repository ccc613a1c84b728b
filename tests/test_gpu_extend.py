"""GPU parity of the extend path (new rows of packed sequences over their KV
caches, contiguous or paged) through the C ABI against the fp64 oracle:
prefixes of different lengths, sequences with no prefix, one new row or none,
rows that start in the middle of a tile, windows, the log-scale per sequence,
GQA ratios that take both workgroup shapes, and fp32."""

import zlib

import pytest
import torch

import oracle
import transformer_attention_query_amd as ra
from transformer_attention_query_amd import inputs as tinputs
from parity import assert_close

pytestmark = pytest.mark.gpu

ALPHA = 1.0 / 128 ** 0.5

# name, dtype, kv_lens, new_lens, Hq, Hkv, d_r, E, W, log_scale, page_size (0 = contiguous)
CASES = [
    ("g8_contig", "bf16", [300, 64, 1000], [37, 64, 1], 8, 1, 32, 100, 0, False, 0),
    ("g4_paged32_window", "bf16", [513, 77, 1], [200, 5, 1], 8, 2, 64, 64, 50, False, 32),
    ("g8_paged64_empty_seq", "bf16", [129, 700, 40], [129, 0, 33], 16, 2, 128, 300, 0, False, 64),
    ("mha_paged128_E1", "bf16", [260, 31], [100, 31], 3, 3, 16, 1, 0, False, 128),
    ("g8_log_scale", "bf16", [5000, 4200], [40, 70], 8, 1, 64, 200, 0, True, 64),
    ("fp32_paged32", "fp32", [90, 200], [90, 45], 4, 2, 32, 50, 17, False, 32),
    ("fp32_contig_E0", "fp32", [70, 33], [7, 33], 2, 1, 16, 0, 0, False, 0),
    # eight or more query heads per kv head take the DMA kernel's extend form
    # (contiguous, or paged with a power-of-two page size); other page sizes
    # the tile kernel
    ("g8_paged32_window", "bf16", [513, 77, 1], [200, 5, 1], 8, 1, 64, 64, 50, False, 32),
    ("g8_paged96_tile_kernel", "bf16", [400, 250], [130, 250], 8, 1, 64, 100, 0, False, 96),
    ("g16_contig_window_log", "bf16", [4500, 900], [300, 64], 16, 2, 128, 1024, 700, True, 0),
    ("g8_paged128_ragged", "bf16", [1111, 37, 2050], [111, 37, 1], 8, 1, 128, 1024, 0, False, 128),
]


def _run(x, E, W, ls, page_size, alpha=ALPHA):
    xd = {n: t.cuda() for n, t in x.items()}
    paged = page_size > 0
    new = (xd["q_start"][1:] - xd["q_start"][:-1]).cpu()
    out, lse = ra.extend(xd["q"], xd["k_pages"] if paged else xd["k"], xd["v_pages"] if paged else xd["v"],
                         xd["r"], xd["P_cols"] if E > 0 else None, alpha, E, W, ls, xd["q_start"], xd["kv_len"],
                         int(new.max()), block_table=xd["block_table"] if paged else None)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_extend_matches_oracle(case):
    name, dt, kv_lens, new_lens, Hq, Hkv, d_r, E, W, ls, page = case
    x = tinputs.make_extend_inputs(kv_lens, new_lens, Hq, Hkv, 128, d_r, max(E, 1), dt,
                                   seed=zlib.crc32(name.encode()) % 1000, page_size=page)
    if E == 0:
        x["P_cols"] = x["P_cols"][:0]
    out, lse = _run(x, E, W, ls, page)
    ref, lref = oracle.extend(x["q"], x["k"], x["v"], x["r"], x["P"], ALPHA, E, W, ls,
                              x["q_start"].tolist(), x["kv_len"].tolist())
    assert_close(out, ref, x["q"].dtype, name, lse, lref)


@pytest.mark.parametrize("heads", [(8, 1), (8, 2)], ids=["G8", "G4"])
def test_extend_bias_sensitivity_paged(heads):
    """Large relative logits: a slip in positions, the shear or the page
    mapping changes the output by O(1)."""
    Hq, Hkv = heads
    x = tinputs.make_extend_inputs([600, 333], [150, 90], Hq, Hkv, 128, 64, 200, "bf16", seed=9, page_size=32)
    x["P"] = (x["P"].float() * 50).to(torch.bfloat16)
    x["P_cols"] = x["P"].t().contiguous()
    out, lse = _run(x, 200, 0, False, 32)
    ref, lref = oracle.extend(x["q"], x["k"], x["v"], x["r"], x["P"], ALPHA, 200, 0, False,
                              x["q_start"].tolist(), x["kv_len"].tolist())
    assert_close(out, ref, torch.bfloat16, "P_x50", lse, lref)


def test_extend_of_whole_sequences_equals_prefill():
    """No prefix: extend over T new rows is a prefill of length T (both paths
    against the oracle, and against each other within the tolerance)."""
    T, Hq, Hkv = 300, 8, 1
    x = tinputs.make_extend_inputs([T, T], [T, T], Hq, Hkv, 128, 64, 128, "bf16", seed=21)
    out, lse = _run(x, 128, 0, False, 0)
    q = x["q"].view(2, T, Hq, 128).cuda()
    r = x["r"].view(2, T, Hq, 64).cuda()
    pout, plse = ra.prefill(q, x["k"].cuda(), x["v"].cuda(), r, x["P_cols"].cuda(), ALPHA, 128, 0, False)
    torch.cuda.synchronize()
    ref, lref = oracle.extend(x["q"], x["k"], x["v"], x["r"], x["P"], ALPHA, 128, 0, False,
                              x["q_start"].tolist(), x["kv_len"].tolist())
    assert_close(out, ref, torch.bfloat16, "extend", lse, lref)
    assert_close(pout.view(2 * T, Hq, 128), ref, torch.bfloat16, "prefill",
                 plse.permute(1, 0, 2).reshape(Hq, 2 * T), lref)


# ---------------------------------------------------------------- paged decode

# name, dtype, kv_lens, Hq, Hkv, d_r, E, W, log_scale, page_size, num_splits (0 = plan's choice)
DECODE_CASES = [
    ("g8_mixed_lengths", "bf16", [1, 31, 32, 700, 3000], 8, 1, 32, 100, 0, False, 32, 0),
    ("g4_window_log", "bf16", [4097, 64, 500], 8, 2, 64, 64, 300, True, 64, 0),
    ("g8_forced_splits_short_seq", "bf16", [2050, 40], 16, 2, 128, 1024, 0, False, 128, 8),
    ("mha_E0", "bf16", [129, 257], 2, 2, 16, 0, 0, False, 32, 0),
    ("fp32_paged", "fp32", [257, 1, 90], 4, 2, 32, 40, 0, False, 32, 0),
    ("g8_one_split_mixed", "bf16", [1, 900, 2000], 16, 2, 128, 256, 0, False, 64, 1),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_paged_matches_oracle(case):
    name, dt, kv_lens, Hq, Hkv, d_r, E, W, ls, page, ns = case
    B = len(kv_lens)
    x = tinputs.make_extend_inputs(kv_lens, [1] * B, Hq, Hkv, 128, d_r, max(E, 1), dt,
                                   seed=zlib.crc32(name.encode()) % 1000, page_size=page)
    xd = {n: t.cuda() for n, t in x.items()}
    out, lse = ra.decode_paged(xd["q"], xd["k_pages"], xd["v_pages"], xd["r"], xd["P_cols"][:E] if E else None,
                               ALPHA, E, W, ls, xd["kv_len"], xd["block_table"], max(kv_lens), num_splits=ns)
    torch.cuda.synchronize()
    ref, lref = oracle.extend(x["q"], x["k_pages"], x["v_pages"], x["r"], x["P"], ALPHA, E, W, ls,
                              x["q_start"].tolist(), kv_lens, block_table=x["block_table"].tolist(), page_size=page)
    assert_close(out, ref, x["q"].dtype, name, lse, lref.t())
