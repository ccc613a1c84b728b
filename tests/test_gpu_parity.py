"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element
by element, on seeded inputs spanning several tiles, ragged tails and the
degenerate cases (T = 1, window 1, rel_extent 0 or beyond T, MHA, wide GQA)."""

import zlib

import pytest
import torch

import oracle
import transformer_attention_query_amd as ra
from transformer_attention_query_amd import inputs as tinputs
from parity import TOL, assert_close, err_stats

pytestmark = pytest.mark.gpu

ALPHA = 1.0 / 128 ** 0.5


def _cuda(x):
    return {n: t.cuda() for n, t in x.items()}


def _run_prefill(x, alpha, E, W, ls):
    out, lse = ra.prefill(x["q"], x["k"], x["v"], x["r"], x["P_cols"], alpha, E, W, ls)
    torch.cuda.synchronize()
    return out, lse


# name, dtype, B, T, Hq, Hkv, d_r, E, W, log_scale
PREFILL_CASES = [
    ("tiny_fp32_workload", "fp32", 1, 256, 4, 1, 32, 64, 0, False),
    ("T1", "bf16", 1, 1, 8, 1, 32, 16, 0, False),
    ("T17_mha", "bf16", 2, 17, 3, 3, 16, 5, 0, False),
    ("T100_E1", "bf16", 1, 100, 4, 2, 64, 1, 0, False),
    ("T255_W5", "bf16", 1, 255, 4, 1, 32, 40, 5, False),
    ("T300_W1", "bf16", 1, 300, 2, 1, 48, 10, 1, False),
    ("T1000_W100", "bf16", 2, 1000, 8, 1, 128, 300, 100, False),
    ("T700_E0", "bf16", 1, 700, 4, 2, 32, 0, 0, False),
    ("T600_E_beyond_T", "bf16", 1, 600, 4, 1, 128, 2000, 0, False),
    ("T513_W200_E64", "bf16", 1, 513, 16, 2, 128, 64, 200, False),
    ("T1100_E1024_W1024", "bf16", 1, 1100, 8, 1, 128, 1024, 1024, False),
    ("fp32_T300_W70", "fp32", 1, 300, 4, 2, 64, 100, 70, False),
    ("fp32_T129", "fp32", 2, 129, 2, 1, 16, 7, 0, False),
    # eight or more query heads per kv head: 64-key tiles, two distance chunks per tile
    ("G8_T97_E33", "bf16", 2, 97, 8, 1, 16, 33, 0, False),
    ("G8_T160_W1_E1", "bf16", 1, 160, 8, 1, 32, 1, 1, False),
    ("G8_T333_W65_E63", "bf16", 1, 333, 16, 2, 64, 63, 65, False),
    ("G8_T64_E0", "bf16", 1, 64, 8, 1, 32, 0, 0, False),
    ("G8_T700_E600_log", "bf16", 1, 700, 8, 1, 128, 600, 0, True),
    ("G16_T450_W130_E129", "bf16", 1, 450, 16, 1, 48, 129, 130, False),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_matches_oracle(case):
    name, dt, B, T, Hq, Hkv, d_r, E, W, ls = case
    x = tinputs.make_prefill_inputs(B, T, Hq, Hkv, 128, d_r, max(E, 1), dt, seed=zlib.crc32(name.encode()) % 1000)
    if E == 0:
        x["P_cols"] = x["P_cols"][:0]
    xd = _cuda(x)
    out, lse = _run_prefill(xd, ALPHA, E, W, ls)
    ref, lref = oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], ALPHA, E, W, ls)
    assert_close(out, ref, x["q"].dtype, name, lse, lref)


@pytest.mark.parametrize("heads", [(8, 2), (8, 1)], ids=["G4", "G8"])
@pytest.mark.parametrize("W", [0, 300])
@pytest.mark.parametrize("variant", ["P_x50", "alpha_0", "alpha_neg"])
def test_prefill_bias_sensitivity(variant, W, heads):
    """Large-bias variants where a shear or rel_extent slip changes the output by O(1).
    G8 (eight query heads per kv head) takes the eight-heads-per-workgroup kernel;
    alpha <= 0 takes its form that scales every score before the row max."""
    T, E = 777, 200
    Hq, Hkv = heads
    x = tinputs.make_prefill_inputs(1, T, Hq, Hkv, 128, 64, E, "bf16", seed=5)
    alpha = ALPHA
    if variant == "P_x50":
        x["P"] = (x["P"].float() * 50).to(torch.bfloat16)
        x["P_cols"] = x["P"].t().contiguous()
    else:
        alpha = 0.0 if variant == "alpha_0" else -2.0 * ALPHA
        x["P"] = (x["P"].float() * 25).to(torch.bfloat16)
        x["P_cols"] = x["P"].t().contiguous()
    out, lse = _run_prefill(_cuda(x), alpha, E, W, False)
    ref, lref = oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], alpha, E, W)
    assert_close(out, ref, torch.bfloat16, variant, lse, lref)


def test_prefill_log_scale_sampled_rows():
    T, E = 5000, 300
    x = tinputs.make_prefill_inputs(1, T, 4, 1, 128, 64, E, "bf16", seed=11)
    out, lse = _run_prefill(_cuda(x), ALPHA, E, 0, True)
    rows = [0, 1, 299, 300, 301, 2047, 4095, 4096, 4999]
    ref, lref = oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], ALPHA, E, 0, True, rows=rows)
    assert_close(out[:, rows], ref, torch.bfloat16, "log-scale", lse[:, :, rows], lref)


def test_prefill_log_scale_large_bias_eight_heads_per_kv_head():
    """Eight query heads per kv head (the eight-heads-per-workgroup kernel),
    T > 4096 so the log-scale s exceeds 1, and P scaled by 50 so the bias
    dominates the scores: s must multiply both terms, and the band edge at
    rel_extent must sit at the right distance."""
    T, E = 4500, 1024
    x = tinputs.make_prefill_inputs(1, T, 8, 1, 128, 128, E, "bf16", seed=12)
    x["P"] = (x["P"].float() * 50).to(torch.bfloat16)
    x["P_cols"] = x["P"].t().contiguous()
    assert oracle.scale_factor(T, True) > 1.01
    out, lse = _run_prefill(_cuda(x), ALPHA, E, 0, True)
    rows = [0, 1, 31, 32, 1022, 1023, 1024, 1025, 1055, 1056, 2047, 2048, 3000, 4095, 4096, 4097, 4498, 4499]
    ref, lref = oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], ALPHA, E, 0, True, rows=rows)
    assert_close(out[:, rows], ref, torch.bfloat16, "G8 log-scale P x50", lse[:, :, rows], lref)


@pytest.mark.parametrize("alpha_sign,W,T,ls", [(1, 0, 1500, False), (1, 700, 1337, True), (-1, 0, 1100, False)])
def test_prefill_rising_scores_raise_the_running_maximum(alpha_sign, W, T, ls):
    """Scores that climb by more than 12 log2 units every 32 keys (one
    dimension of k ramps with the key index, q holds a constant there), so in
    the eight-heads kernel the exponentials taken against the running maximum
    overflow the accepted sum on every tile and the maximum is raised, O and l
    rescaled and the exponentials redone, tile after tile.  alpha < 0 (with
    the ramp reversed) runs the kernel form that scales every score."""
    E = 256
    x = tinputs.make_prefill_inputs(1, T, 8, 1, 128, 64, E, "bf16", seed=17 + T)
    ramp = torch.arange(T, dtype=torch.float32) * (4.0 * alpha_sign)
    k = x["k"].float()
    k[0, :, 0, 0] = ramp
    x["k"] = k.to(torch.bfloat16)
    q = x["q"].float()
    q[..., 0] = 1.0
    x["q"] = q.to(torch.bfloat16)
    alpha = alpha_sign * ALPHA
    # log2 units per 32 keys: s * log2(e) * |alpha| * 4 * 32
    assert oracle.scale_factor(T, ls) * 1.4427 * ALPHA * 4 * 32 > 16
    out, lse = _run_prefill(_cuda(x), alpha, E, W, ls)
    ref, lref = oracle.prefill(x["q"], x["k"], x["v"], x["r"], x["P"], alpha, E, W, ls)
    assert_close(out, ref, torch.bfloat16, f"rising scores alpha {alpha_sign} W {W}", lse, lref)


def test_prefill_weights_via_identity_v():
    """V = identity makes each output row the attention-weight row: masked
    weights are exactly zero and each row sums to one."""
    T = 100
    x = tinputs.make_prefill_inputs(1, T, 2, 1, 128, 32, 30, "bf16", seed=2)
    eye = torch.zeros(1, T, 1, 128, dtype=torch.bfloat16)
    eye[0, :, 0, :T] = torch.eye(T, dtype=torch.bfloat16)
    x["v"] = eye
    W = 17
    out, _ = _run_prefill(_cuda(x), ALPHA, 30, W, False)
    o = out.float().cpu()[0]                     # [T, H, 128]
    i = torch.arange(T)[:, None]
    j = torch.arange(128)[None, :]
    masked = (j > i) | (i - j >= W)
    assert torch.all(o[masked[:, None, :].expand(-1, 2, -1)] == 0)
    assert torch.allclose(o.sum(-1), torch.ones(T, 2), atol=2e-2)
    w = oracle.attention_weights(x["q"], x["k"], x["r"], x["P"], ALPHA, 30, W)[0]   # [H, T, T]
    assert_close(o[:, :, :T].permute(1, 0, 2), w, torch.bfloat16, "weights")


def test_prefill_is_deterministic():
    x = _cuda(tinputs.make_prefill_inputs(1, 1500, 8, 1, 128, 128, 512, "bf16", seed=3))
    a, la = _run_prefill(x, ALPHA, 512, 0, False)
    b, lb = _run_prefill(x, ALPHA, 512, 0, False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


# ---------------------------------------------------------------- decode

# name, dtype, B, L, Hq, Hkv, d_r, E, W, log_scale, num_splits
DECODE_CASES = [
    ("L1", "bf16", 2, 1, 16, 2, 128, 64, 0, False, 0),
    ("L33_mha", "bf16", 3, 33, 4, 4, 32, 10, 0, False, 0),
    ("L1000_W100", "bf16", 2, 1000, 16, 2, 128, 300, 100, False, 0),
    ("L5000_log_s7", "bf16", 1, 5000, 8, 1, 64, 1024, 0, True, 7),
    ("G32_s3", "bf16", 1, 700, 32, 1, 16, 50, 0, False, 3),
    ("E0", "bf16", 2, 400, 16, 2, 128, 0, 0, False, 0),
    ("E_beyond_L", "bf16", 1, 300, 16, 2, 128, 1024, 0, False, 2),
    ("fp32", "fp32", 2, 513, 8, 2, 32, 64, 0, False, 0),
    ("fp32_W50_s5", "fp32", 1, 777, 4, 1, 48, 100, 50, False, 5),
    # one split: the split kernel normalises and writes the output itself
    ("L2000_s1", "bf16", 2, 2000, 16, 2, 128, 1024, 0, False, 1),
    ("fp32_L600_W200_s1", "fp32", 1, 600, 8, 2, 32, 64, 200, False, 1),
    # bias keys [2800, 3000) begin 12 keys before the end of the middle split
    ("L3000_W700_E200_s3", "bf16", 2, 3000, 16, 2, 128, 200, 700, False, 3),
    # 16 heads per kv head and E = 2048: the in-kernel bias region would not
    # fit the LDS budget, so the bias rows come from the pre-pass
    ("G16_E2048_prepass", "bf16", 1, 3000, 16, 1, 128, 2048, 0, False, 1),
    # eight and sixteen splits; E = 3000 spans a split boundary
    ("L40000_s16", "bf16", 2, 40000, 16, 2, 128, 1024, 0, False, 16),
    ("L40000_s16_log_E3000", "bf16", 1, 40000, 8, 1, 64, 3000, 0, True, 16),
    ("fp32_L20000_s8", "fp32", 1, 20000, 4, 2, 32, 700, 0, False, 8),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_matches_oracle(case):
    name, dt, B, L, Hq, Hkv, d_r, E, W, ls, ns = case
    x = tinputs.make_decode_inputs(B, L, Hq, Hkv, 128, d_r, max(E, 1), dt, seed=zlib.crc32(name.encode()) % 1000)
    if E == 0:
        x["P_cols"] = x["P_cols"][:0]
    xd = _cuda(x)
    out, lse = ra.decode(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], ALPHA, E, W, ls, num_splits=ns)
    torch.cuda.synchronize()
    ref, lref = oracle.decode(x["q"], x["k"], x["v"], x["r"], x["P"], ALPHA, E, W, ls)
    assert_close(out, ref, x["q"].dtype, name, lse, lref)


def test_decode_split_invariance():
    x = _cuda(tinputs.make_decode_inputs(2, 3000, 16, 2, 128, 128, 1024, "fp32", seed=4))
    outs = []
    for ns in (1, 2, 3, 7, 64, 0):
        o, l = ra.decode(x["q"], x["k"], x["v"], x["r"], x["P_cols"], ALPHA, 1024, 0, False, num_splits=ns)
        outs.append((o.cpu(), l.cpu()))
    torch.cuda.synchronize()
    o0, l0 = outs[0]
    for o, l in outs[1:]:
        assert err_stats(o, o0)[0] <= 1e-5 and err_stats(l, l0)[0] <= 1e-5


@pytest.mark.parametrize("ls,W", [(False, 0), (True, 0), (False, 64)])
def test_decode_equals_last_prefill_row(ls, W):
    L = 4500 if ls else 1300
    x = tinputs.make_prefill_inputs(1, L, 8, 2, 128, 64, 256, "fp32", seed=6)
    xd = _cuda(x)
    pre, lpre = _run_prefill(xd, ALPHA, 256, W, ls)
    dec, ldec = ra.decode(xd["q"][:, L - 1].contiguous(), xd["k"], xd["v"], xd["r"][:, L - 1].contiguous(),
                          xd["P_cols"], ALPHA, 256, W, ls)
    torch.cuda.synchronize()
    assert err_stats(dec, pre[:, L - 1])[0] <= 1e-4
    assert err_stats(ldec, lpre[:, :, L - 1])[0] <= 2e-5


# ---------------------------------------------------------------- rel_logits

@pytest.mark.parametrize("dt,n,H,d_r,E,ls,seq", [
    ("bf16", 300, 4, 128, 1000, False, 0),
    ("bf16", 77, 16, 32, 33, True, 32768),
    ("fp32", 129, 2, 48, 130, False, 0),
])
def test_rel_logits_matches_oracle(dt, n, H, d_r, E, ls, seq):
    x = tinputs.make_prefill_inputs(1, n, H, 1, 128, d_r, E, dt, seed=n)
    r = x["r"][0]                                     # [n, H, d_r]
    got = ra.rel_logits(r.cuda(), x["P_cols"].cuda(), ls, seq)
    torch.cuda.synchronize()
    s = oracle.scale_factor(seq if seq else n, ls)
    ref = oracle.rel_logits(r, x["P"], s)
    bound = 4 * d_r * 2.0 ** -24 * s * (r.double().abs() @ x["P"].double().abs()) + 1e-30
    assert torch.all((got.double().cpu() - ref).abs() <= bound)
