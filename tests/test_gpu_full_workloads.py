"""GPU parity at the full sizes of the five named workloads and of the
extend workload, in the launch configuration bench.py times.  The tiny fp32
and 8K sliding-window prefills, both decodes and the extend are compared
over their whole outputs.  The 2x32K causal
prefill, whose full oracle would take minutes, is compared on every 16th
query row counted from the last, plus every tile edge, the rel_extent edge
and the first rows."""

import random

import pytest
import torch

import oracle
import transformer_attention_query_amd as ra
from transformer_attention_query_amd import inputs as tinputs
from parity import assert_close

pytestmark = pytest.mark.gpu


def _rows(T, extra, seed):
    base = {0, 1, 31, 32, 63, 64, 127, 128, 129, 1023, 1024, 1025, 2047, 2048, T // 2, T - 2, T - 1}
    rng = random.Random(seed)
    base |= {rng.randrange(T) for _ in range(extra)}
    return sorted(r for r in base if r < T)


@pytest.mark.parametrize("name", ["tiny_fp32", "swa_prefill_8k", "full_prefill_32k_log"])
def test_prefill_workload(name):
    w = tinputs.WORKLOADS[name]
    x = tinputs.make_inputs(w, seed=0)
    xd = {n: t.cuda() for n, t in x.items()}
    out, lse = ra.prefill(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], w.alpha, w.E, w.W, w.log_scale)
    torch.cuda.synchronize()
    del xd
    if w.T <= 8192:
        ref, lref = oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], w.alpha, w.E, w.W, w.log_scale)
        assert_close(out, ref, x["q"].dtype, name, lse, lref)
        return
    rows = sorted(set(_rows(w.T, 24, 1)) | set(range(w.T - 1, -1, -16)))
    ref, lref = oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], w.alpha, w.E, w.W, w.log_scale, rows=rows)
    assert_close(out[:, rows], ref, x["q"].dtype, name, lse[:, :, rows], lref)


@pytest.mark.parametrize("name", ["decode_64x8k", "decode_1x1m_log"])
def test_decode_workload(name):
    w = tinputs.WORKLOADS[name]
    x = tinputs.make_inputs(w, seed=0)
    xd = {n: t.cuda() for n, t in x.items()}
    out, lse = ra.decode(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], w.alpha, w.E, w.W, w.log_scale,
                         num_splits=w.num_splits)
    torch.cuda.synchronize()
    del xd
    ref, lref = oracle.decode(x["q"], x["k"], x["v"], x["r"], x["P"], w.alpha, w.E, w.W, w.log_scale)
    assert_close(out, ref, x["q"].dtype, name, lse, lref)


def test_extend_workload():
    """extend_4x1k_8k_paged as the bench runs it: four sequences of 8192
    cached keys, the last 1024 of each new, over a paged cache."""
    w = tinputs.WORKLOADS["extend_4x1k_8k_paged"]
    x = tinputs.make_inputs(w, seed=0)
    xd = {n: t.cuda() for n, t in x.items()}
    paged = w.page_size > 0
    out, lse = ra.extend(xd["q"], xd["k_pages"] if paged else xd["k"], xd["v_pages"] if paged else xd["v"], xd["r"],
                         xd["P_cols"], w.alpha, w.E, w.W, w.log_scale, xd["q_start"], xd["kv_len"], w.n_new,
                         block_table=xd["block_table"] if paged else None)
    torch.cuda.synchronize()
    del xd
    ref, lref = oracle.extend(x["q"], x["k"], x["v"], x["r"], x["P"], w.alpha, w.E, w.W, w.log_scale,
                              x["q_start"].tolist(), x["kv_len"].tolist())
    assert_close(out, ref, x["q"].dtype, w.name, lse, lref)
