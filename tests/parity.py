"""Tolerances and comparison helpers for the GPU-vs-oracle parity tests.

Bars (stated for the workloads and kept for every parity case):
* bf16 inputs, fp32 accumulation: max-abs <= 2e-2 and relative L2 <= 1e-2
  over the compared outputs; lse max-abs <= 1e-3.
* fp32 inputs: max-abs <= 1e-4; lse max-abs <= 1e-5.
* rel_logits (fp32 output of an fp32-accumulated product of exact inputs):
  |gpu - exact| <= 4 * d_r * 2^-24 * s * sum_c |r_c P_c| + 1e-30 per entry.
"""

import torch

TOL = {
    torch.bfloat16: dict(max_abs=2e-2, rel_l2=1e-2, lse=1e-3),
    torch.float32: dict(max_abs=1e-4, rel_l2=1e-4, lse=1e-5),
}


def err_stats(got: torch.Tensor, ref: torch.Tensor):
    g = got.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    diff = g - r
    max_abs = diff.abs().max().item() if diff.numel() else 0.0
    rel_l2 = (diff.norm() / r.norm().clamp_min(1e-300)).item() if diff.numel() else 0.0
    return max_abs, rel_l2


def assert_close(got, ref, dtype, what="out", lse_got=None, lse_ref=None):
    tol = TOL[dtype]
    assert torch.isfinite(got.float()).all(), f"{what}: non-finite values"
    max_abs, rel_l2 = err_stats(got, ref)
    assert max_abs <= tol["max_abs"] and rel_l2 <= tol["rel_l2"], (
        f"{what}: max-abs {max_abs:.3e} (bar {tol['max_abs']}), rel-L2 {rel_l2:.3e} (bar {tol['rel_l2']})")
    if lse_got is not None:
        lmax, _ = err_stats(lse_got, lse_ref)
        assert lmax <= tol["lse"], f"{what}: lse max-abs {lmax:.3e} (bar {tol['lse']})"
    return max_abs, rel_l2
