"""GPU parity of the backward pass (rel_attn_backward) through the C ABI
against the fp64 oracle (oracle.prefill_backward): GQA 8:1, 4:1, 2:1 and MHA,
windows, ragged tails, no bias, E beyond T, d_r not a multiple of 32, the
log-scale, forced head splits, a bias-only case with a large P (shear errors
are then of order one), T = 1 and window 1, and the 8K sliding-window shape
of the bench on sampled rows and keys.

out and lse come from the GPU forward (rel_attn_prefill) on the same inputs,
as a training step would pass them; the oracle recomputes everything from
q, k, v, r, P and dout.

Tolerance (the pages give none for gradients; derived from the arithmetic):
the kernels round P and dS to bf16 for the MFMAs (2^-9 relative each), use
the bf16-rounded forward output in delta, and round each gradient once to
bf16; the errors are of order 2^-8 relative to the terms summed.  Each
gradient tensor must meet rel-L2 <= 1e-2 (the bar of the forward output) and
max-abs <= 2e-2 * max |reference| (the forward's max-abs bar, taken relative
to the tensor's scale, since gradients are not of order one).  Where the exact
gradient is identically zero (a single visible key per row), max-abs <= 1e-5:
only fp32 rounding of delta against dout . v remains."""

import zlib

import pytest
import torch

import oracle
import transformer_attention_query_amd as ra
from transformer_attention_query_amd import inputs as tinputs
from parity import err_stats

pytestmark = pytest.mark.gpu

ALPHA = 1.0 / 128 ** 0.5


def _grad_close(got, ref, what):
    assert got is not None
    assert torch.isfinite(got.float()).all(), f"{what}: non-finite values"
    max_abs, rel_l2 = err_stats(got, ref)
    scale = ref.abs().max().item()
    print(f"{what}: max-abs {max_abs:.3e} (ref max {scale:.3e}), rel-L2 {rel_l2:.3e}")
    if scale == 0.0:
        # exactly zero gradient (one visible key per row): only the rounding of
        # delta = dout . out against dout . v in fp32 may show
        assert max_abs <= 1e-5, f"{what}: max-abs {max_abs:.3e} where the gradient is exactly zero"
        return
    assert rel_l2 <= 1e-2 and max_abs <= 2e-2 * scale, (
        f"{what}: max-abs {max_abs:.3e} vs bar {2e-2 * scale:.3e}, rel-L2 {rel_l2:.3e} vs bar 1e-2")


def _gpu_backward(x, alpha, E, W, ls, head_splits=0):
    xd = {n: t.cuda() for n, t in x.items()}
    pc = xd["P_cols"] if E > 0 else None
    r = xd["r"] if E > 0 else None
    out, lse = ra.prefill(xd["q"], xd["k"], xd["v"], r, pc, alpha, E, W, ls)
    g = ra.backward(xd["q"], xd["k"], xd["v"], r, pc, out, xd["dout"], lse, alpha, E, W, ls,
                    head_splits=head_splits)
    torch.cuda.synchronize()
    return [t.cpu() if t is not None else None for t in g]


def _check(name, x, got, alpha, E, W, ls, rows=None, keys=None):
    P = x["P"] if E > 0 else None
    ref = oracle.prefill_backward(x["q"], x["k"], x["v"], x["r"] if E > 0 else None, P, x["dout"], alpha, E, W, ls,
                                  rows=rows, key_rows=keys)
    dq, dk, dv, dr = got
    if rows is not None:
        dq = dq[:, rows]
        dr = dr[:, rows] if dr is not None else None
    if keys is not None:
        dk, dv = dk[:, keys], dv[:, keys]
    _grad_close(dq, ref[0], f"{name} dq")
    _grad_close(dk, ref[1], f"{name} dk")
    _grad_close(dv, ref[2], f"{name} dv")
    if E > 0:
        _grad_close(dr, ref[3], f"{name} dr")
    else:
        assert dr is None


# name, B, T, Hq, Hkv, d_r, E, W, log_scale
CASES = [
    ("G8_T300_W100_E64", 1, 300, 16, 2, 128, 64, 100, False),
    ("mha_B2_T200_E40", 2, 200, 2, 2, 32, 40, 0, False),
    ("G2_T150_E256_beyond_T", 1, 150, 4, 2, 64, 256, 0, False),
    ("G8_T130_no_bias", 1, 130, 8, 1, 128, 0, 0, False),
    ("G4_T180_dr48_E96", 1, 180, 4, 1, 48, 96, 0, False),
    ("G8_T257_W33_E1000", 1, 257, 8, 1, 128, 1000, 33, False),
    ("G3_T97_E31_W64", 2, 97, 3, 1, 32, 31, 64, False),
    ("T1", 1, 1, 8, 1, 32, 16, 0, False),
    ("G8_T96_W1", 1, 96, 8, 1, 32, 8, 1, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    name, B, T, Hq, Hkv, d_r, E, W, ls = case
    x = tinputs.make_backward_inputs(B, T, Hq, Hkv, 128, d_r, max(E, 1), "bf16", seed=zlib.crc32(name.encode()) % 1000)
    got = _gpu_backward(x, ALPHA, E, W, ls)
    _check(name, x, got, ALPHA, E, W, ls)


def test_backward_bias_only_large_P():
    """alpha = 0 and P x 50: the logits are the relative bias alone, so a
    misplaced shear in the recomputed bias or in dr is an error of order one."""
    x = tinputs.make_backward_inputs(1, 200, 8, 1, 128, 64, 96, "bf16", seed=11)
    x["P"] = (x["P"].float() * 50).to(torch.bfloat16)
    x["P_cols"] = x["P"].t().contiguous()
    got = _gpu_backward(x, 0.0, 96, 0, False)
    assert got[0].abs().max().item() == 0.0 and got[1].abs().max().item() == 0.0  # alpha = 0: no q.k gradient
    _check("bias_only", x, got, 0.0, 96, 0, False)


@pytest.mark.parametrize("splits", [1, 2, 8])
def test_backward_head_splits(splits):
    """Every split of the group's heads gives the oracle's dk and dv."""
    x = tinputs.make_backward_inputs(1, 160, 16, 2, 128, 128, 64, "bf16", seed=21)
    got = _gpu_backward(x, ALPHA, 64, 0, False, head_splits=splits)
    _check(f"splits{splits}", x, got, ALPHA, 64, 0, False)


def test_backward_log_scale_sampled():
    """T = 5000 with the log-scale on (s = ln 5000 / ln 4096 > 1), full causal,
    on sampled rows and keys."""
    T = 5000
    x = tinputs.make_backward_inputs(1, T, 4, 1, 128, 64, 128, "bf16", seed=31)
    got = _gpu_backward(x, ALPHA, 128, 0, True)
    rows = [0, 1, 31, 32, 127, 128, 2048, 4095, 4096, 4999]
    keys = [0, 5, 64, 2000, 4900, 4999]
    _check("log_scale_T5000", x, got, ALPHA, 128, 0, True, rows=rows, keys=keys)


def test_backward_swa_8k_workload_sampled():
    """The bench shape (T = 8192, Hq = 16, Hkv = 2, d_r = 128, E = W = 1024) in
    the launch configuration the bench times, on sampled rows and keys."""
    w = tinputs.WORKLOADS["swa_backward_8k"]
    x = tinputs.make_inputs(w, seed=0)
    got = _gpu_backward(x, w.alpha, w.E, w.W, w.log_scale)
    rows = [0, 1, 33, 1023, 1024, 1025, 4000, 8190, 8191]
    keys = [0, 31, 32, 1000, 4096, 7168, 8191]
    _check("swa_backward_8k", x, got, w.alpha, w.E, w.W, w.log_scale, rows=rows, keys=keys)


def test_backward_full_causal_32k_log_sampled():
    """The 32K full-causal log-scale shape (B = 2, s = 1.25; the dk/dv kernel
    then runs without head splits, longest blocks first), on sampled query
    rows and on keys near the end, which few queries see."""
    B, T, Hq, Hkv, d_r, E = 2, 32768, 16, 2, 128, 1024
    x = tinputs.make_backward_inputs(B, T, Hq, Hkv, 128, d_r, E, "bf16", seed=41)
    ns, _ = ra.backward_plan(B, T, Hq, Hkv)
    assert ns == 1
    got = _gpu_backward(x, ALPHA, E, 0, True)
    rows = [0, 1, 1023, 1024, 20000, 32766, 32767]
    keys = [32700, 32735, 32767]
    _check("causal_32k_log", x, got, ALPHA, E, 0, True, rows=rows, keys=keys)
