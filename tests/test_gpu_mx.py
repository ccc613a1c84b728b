"""GPU parity of the MXFP8 K/V path through the C ABI.

* rel_mx_quantize against the oracle's MX quantiser, bit for bit (codes and
  scales): both take the rounding decision from the same bf16 / fp32 input
  values (rows over twelve binades, all-zero blocks, exact ties).
* rel_attn_decode_mx (contiguous and paged) against the oracle's attention
  on the MXFP8 values of q, k and v (the oracle quantises the bf16 inputs
  itself): the bf16 decode bar -- max-abs <= 2e-2 and rel-L2 <= 1e-2 over
  the output, lse within 1e-3.
* rel_attn_prologue_mx: every written cache value within the MX error bound
  of the oracle's fp64 prologue output (half an E4M3 step, 2^-4 relative, a
  subnormal quantum of the block scale, or the clamp at 448 x scale -- the
  kernel quantises its fp32 values, so a code may differ from the one the
  fp64 value rounds to); q_out and the state equal the bf16 prologue's.
* prologue_mx then decode_mx against the oracle's prologue -> MXFP8 ->
  decode chain.
* rel_attn_extend_mx (contiguous and paged) against the oracle's extend on
  the MXFP8 values of q, k and v, at the bf16 bar; a peaky-query case where
  the rounding of q is visible pins that the kernel quantises q itself."""

import zlib

import pytest
import torch

import oracle
import transformer_attention_query_amd as ra
from transformer_attention_query_amd import inputs as tinputs
from parity import assert_close

pytestmark = pytest.mark.gpu

ALPHA = 1.0 / 128 ** 0.5


def _rows(n, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, 128, generator=g, dtype=torch.float64)
    x *= torch.logspace(-6, 6, n, dtype=torch.float64)[:, None]  # twelve binades of block maxima
    x[3, 32:64] = 0.0                                             # an all-zero block
    x[5, :] = 0.0                                                 # an all-zero row
    # exact E4M3 ties after scaling: block max 448 * 2^-4, others on midpoints
    x[7, :32] = torch.tensor([448.0] + [(1.0 + (2 * k + 1) / 16.0) * 2.0 ** ((k % 9) - 3) for k in range(31)],
                             dtype=torch.float64) * 2.0 ** -4
    return x.to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_mx_quantize_is_bit_exact(dtype):
    x = _rows(200, dtype, 1)
    codes, scales = ra.mx_quantize(x.cuda())
    torch.cuda.synchronize()
    rc, rs = oracle.mx_quantize(x)
    assert torch.equal(scales.cpu(), rs)
    assert torch.equal(codes.cpu(), rc)


def _mx_cache(t):
    """GPU codes and scales of a [.., 128] tensor (moved to the device)."""
    return ra.mx_quantize(t.cuda().contiguous())


# name, B, L, Hq, Hkv, d_r, E, W, log_scale, num_splits (0 = plan's)
CASES = [
    ("g8_ragged", 3, 1000, 16, 2, 128, 256, 0, False, 0),
    ("g4_window_splits", 2, 2500, 8, 2, 64, 300, 700, False, 5),
    ("g8_log_scale", 1, 5000, 8, 1, 32, 100, 0, True, 0),
    ("mha_E0", 2, 333, 4, 4, 32, 0, 0, False, 3),
    ("g16_short", 4, 65, 16, 1, 64, 64, 0, False, 0),
    ("g8_one_split", 2, 1500, 16, 2, 128, 512, 0, False, 1),
    ("g8_16_splits", 1, 40000, 16, 2, 128, 1024, 0, False, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_mx_matches_oracle(case):
    name, B, L, Hq, Hkv, d_r, E, W, ls, ns = case
    x = tinputs.make_decode_inputs(B, L, Hq, Hkv, 128, d_r, max(E, 1), "bf16", seed=zlib.crc32(name.encode()) % 1000)
    kc, ks = _mx_cache(x["k"])
    vc, vs = _mx_cache(x["v"])
    out, lse = ra.decode_mx(x["q"].cuda(), kc, ks, vc, vs, x["r"].cuda(), x["P_cols"].cuda() if E > 0 else None,
                            ALPHA, E, W, ls, num_splits=ns)
    torch.cuda.synchronize()
    qd, kd, vd = oracle.mx_round(x["q"]), oracle.mx_round(x["k"]), oracle.mx_round(x["v"])
    ref, lref = oracle.decode(qd, kd, vd, x["r"], x["P"] if E > 0 else x["P"][:, :0], ALPHA, E, W, ls)
    assert_close(out, ref, torch.bfloat16, name, lse, lref)


@pytest.mark.parametrize("page", [32, 64])
def test_decode_mx_paged_matches_oracle(page):
    kv_lens = [1, 700, 4097, 64]
    x = tinputs.make_extend_inputs(kv_lens, [1] * 4, 16, 2, 128, 64, 200, "bf16", seed=7 + page, page_size=page)
    kc, ks = _mx_cache(x["k_pages"])
    vc, vs = _mx_cache(x["v_pages"])
    q = x["q"].cuda()  # [B, Hq, D]: one new row per sequence
    out, lse = ra.decode_mx(q, kc, ks, vc, vs, x["r"].cuda(), x["P_cols"].cuda(), ALPHA, 200, 0, True,
                            L=max(kv_lens), kv_len=x["kv_len"].cuda(), block_table=x["block_table"].cuda())
    torch.cuda.synchronize()
    ref, lref = oracle.extend(oracle.mx_round(x["q"]), oracle.mx_round(x["k"]), oracle.mx_round(x["v"]), x["r"],
                              x["P"], ALPHA, 200, 0, True, x["q_start"].tolist(), x["kv_len"].tolist())
    assert_close(out, ref, torch.bfloat16, f"paged{page}", lse, lref.t().contiguous())


def _check_mx_rows(codes, scales, ref, what):
    deq = oracle.mx_dequantize(codes.cpu(), scales.cpu())
    s = oracle.mx_dequantize(torch.full_like(codes.cpu(), 0x38), scales.cpu())  # 0x38 = 1.0: the block scale
    err = (deq - ref).abs()
    bound = torch.maximum(ref.abs() * 2.0 ** -4, s * 2.0 ** -10) + 1e-6 * ref.abs()
    clipped = ref.abs() > 448.0 * s
    bad = (err > bound) & ~clipped
    assert not bad.any(), f"{what}: {int(bad.sum())} values outside the MX bound, worst {float((err - bound).max()):.3e}"


@pytest.mark.parametrize("page", [0, 16])
def test_prologue_mx_matches_oracle(page):
    kv_lens, new_lens = [50, 10, 40, 200], [17, 0, 40, 120]
    x = tinputs.make_prologue_inputs(kv_lens, new_lens, 8, 2, 128, 4, "bf16", seed=11 + page, page_size=page,
                                     with_state=True)
    xd = {n: t.cuda() for n, t in x.items()}
    bt = xd["block_table"] if page else None
    shape = (xd["k_pages"] if page else xd["k_cache"]).shape
    kc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    ks = torch.zeros(shape[:3] + (4,), dtype=torch.uint8, device="cuda")
    vs = torch.zeros_like(ks)
    so = torch.empty(4, 2, 3, 256, dtype=torch.bfloat16, device="cuda")
    q_out = ra.prologue_mx(xd["q"], xd["k"], xd["v"], xd["conv_k"], xd["conv_v"], xd["q_norm_w"], xd["k_norm_w"],
                           1e-6, xd["q_start"], xd["kv_len"], kc, ks, vc, vs, block_table=bt,
                           state_in=xd["state_in"], state_out=so)
    # the bf16 prologue on the same inputs: q_out and the state must agree exactly
    kb = (xd["k_pages"] if page else xd["k_cache"]).clone()
    vb = (xd["v_pages"] if page else xd["v_cache"]).clone()
    so2 = torch.empty_like(so)
    q_out2 = ra.prologue(xd["q"], xd["k"], xd["v"], xd["conv_k"], xd["conv_v"], xd["q_norm_w"], xd["k_norm_w"], 1e-6,
                         xd["q_start"], xd["kv_len"], kb, vb, block_table=bt, state_in=xd["state_in"], state_out=so2)
    torch.cuda.synchronize()
    assert torch.equal(q_out, q_out2) and torch.equal(so, so2)
    qs = x["q_start"].tolist()
    _, k_ref, v_ref, _ = oracle.prologue(x["q"], x["k"], x["v"], x["conv_k"], x["conv_v"], x["q_norm_w"],
                                         x["k_norm_w"], 1e-6, qs, x["state_in"])
    pos = oracle.cache_positions(qs, x["kv_len"].tolist())
    ib = torch.tensor([b for b, _ in pos])
    ip = torch.tensor([p for _, p in pos])
    if page:
        pg = x["block_table"][ib, ip // page].long()
        sel = (pg, ip % page)
    else:
        sel = (ib, ip)
    kcc, kss, vcc, vss = kc.cpu(), ks.cpu(), vc.cpu(), vs.cpu()
    _check_mx_rows(kcc[sel], kss[sel], k_ref, f"page{page} k")
    _check_mx_rows(vcc[sel], vss[sel], v_ref, f"page{page} v")


def test_prologue_mx_then_decode_mx_matches_oracle_chain():
    """A fresh batch of sequences: the prologue writes MXFP8 caches, decode
    reads them for each sequence's last token."""
    lens = [300, 77]
    x = tinputs.make_prologue_inputs(lens, lens, 16, 2, 128, 4, "bf16", seed=21, with_state=False)
    xd = {n: t.cuda() for n, t in x.items()}
    shape = xd["k_cache"].shape
    kc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    ks = torch.full(shape[:3] + (4,), 127, dtype=torch.uint8, device="cuda")
    vs = torch.full_like(ks, 127)
    q_out = ra.prologue_mx(xd["q"], xd["k"], xd["v"], xd["conv_k"], xd["conv_v"], xd["q_norm_w"], xd["k_norm_w"],
                           1e-6, xd["q_start"], xd["kv_len"], kc, ks, vc, vs)
    qs = x["q_start"].tolist()
    last = [qs[b + 1] - 1 for b in range(2)]
    q_dec = q_out[last].contiguous()  # [2, Hq, D]: each sequence's last token
    g = torch.Generator().manual_seed(5)
    r = (torch.randn(2, 16, 64, generator=g)).to(torch.bfloat16)
    P = (torch.randn(64, 128, generator=g) * 0.02).to(torch.bfloat16)
    # sequence 1 is shorter than the cache: decode it over a paged view of
    # the same rows, one 32-row page per block (kv_len per sequence)
    L = shape[1]
    page = 32
    npg = (L + page - 1) // page
    kc_p = torch.zeros(2 * npg * page, 2, 128, dtype=torch.uint8, device="cuda")
    vc_p = torch.zeros_like(kc_p)
    ks_p = torch.full((2 * npg * page, 2, 4), 127, dtype=torch.uint8, device="cuda")
    vs_p = torch.full_like(ks_p, 127)
    for b in range(2):
        kc_p[b * npg * page:b * npg * page + L] = kc[b]
        vc_p[b * npg * page:b * npg * page + L] = vc[b]
        ks_p[b * npg * page:b * npg * page + L] = ks[b]
        vs_p[b * npg * page:b * npg * page + L] = vs[b]
    table = torch.tensor([[b * npg + i for i in range(npg)] for b in range(2)], dtype=torch.int32, device="cuda")
    out, lse = ra.decode_mx(q_dec, kc_p.view(2 * npg, page, 2, 128), ks_p.view(2 * npg, page, 2, 4),
                            vc_p.view(2 * npg, page, 2, 128), vs_p.view(2 * npg, page, 2, 4), r.cuda(), P.t().contiguous().cuda(),
                            ALPHA, 128, 0, False, L=L, kv_len=torch.tensor(lens, dtype=torch.int32, device="cuda"),
                            block_table=table)
    torch.cuda.synchronize()
    q_ref, k_ref, v_ref, _ = oracle.prologue(x["q"], x["k"], x["v"], x["conv_k"], x["conv_v"], x["q_norm_w"],
                                             x["k_norm_w"], 1e-6, qs)
    # the oracle's own decode query: its fp64 prologue q, rounded to bf16 like the kernel's q_out
    q_dec_ref = q_ref[last].to(torch.bfloat16)
    assert_close(q_out.cpu(), q_ref, torch.bfloat16, "chain q_out")
    kcache = torch.zeros(2, L, 2, 128, dtype=torch.float64)
    vcache = torch.zeros(2, L, 2, 128, dtype=torch.float64)
    for b in range(2):
        kcache[b, :lens[b]] = k_ref[qs[b]:qs[b + 1]]
        vcache[b, :lens[b]] = v_ref[qs[b]:qs[b + 1]]
    qs1 = [0, 1, 2]
    ref, lref = oracle.extend(oracle.mx_round(q_dec_ref), oracle.mx_round(kcache), oracle.mx_round(vcache), r, P,
                              ALPHA, 128, 0, False, qs1, lens)
    assert_close(out, ref, torch.bfloat16, "chain decode", lse, lref.t().contiguous())


# ---------------------------------------------------------------- extend over MXFP8 caches

# name, kv_lens, new_lens, Hq, Hkv, d_r, E, W, log_scale, page_size (0 = contiguous)
EXTEND_CASES = [
    ("g8_contig", [300, 64, 1000], [37, 64, 1], 8, 1, 32, 100, 0, False, 0),
    ("g4_paged32_window", [513, 77, 1], [200, 5, 1], 8, 2, 64, 64, 50, False, 32),
    ("g8_paged64_empty_seq", [129, 700, 40], [129, 0, 33], 16, 2, 128, 300, 0, False, 64),
    ("mha_paged128_E1", [260, 31], [100, 31], 3, 3, 16, 1, 0, False, 128),
    ("g8_log_scale", [5000, 4200], [40, 70], 8, 1, 64, 200, 0, True, 64),
    ("g16_contig_E0", [700, 333], [300, 333], 16, 1, 32, 0, 0, False, 0),
    ("g2_whole_sequences_E1024", [1500, 1100], [1500, 1100], 4, 2, 128, 1024, 0, False, 0),
]


def _extend_mx(x, E, W, ls, page):
    paged = page > 0
    kc, ks = _mx_cache(x["k_pages"] if paged else x["k"])
    vc, vs = _mx_cache(x["v_pages"] if paged else x["v"])
    new = (x["q_start"][1:] - x["q_start"][:-1])
    out, lse = ra.extend_mx(x["q"].cuda(), kc, ks, vc, vs, x["r"].cuda(), x["P_cols"].cuda() if E > 0 else None,
                            ALPHA, E, W, ls, x["q_start"].cuda(), x["kv_len"].cuda(), int(new.max()),
                            block_table=x["block_table"].cuda() if paged else None)
    torch.cuda.synchronize()
    return out, lse


def _extend_mx_ref(x, E, W, ls):
    """The oracle's extend on the values the MXFP8 rows stand for: q, k and v
    through MXFP8 and back (the kernel quantises each new query row itself)."""
    return oracle.extend(oracle.mx_round(x["q"]), oracle.mx_round(x["k"]), oracle.mx_round(x["v"]), x["r"],
                         x["P"] if E > 0 else x["P"][:, :0], ALPHA, E, W, ls, x["q_start"].tolist(),
                         x["kv_len"].tolist())


@pytest.mark.parametrize("case", EXTEND_CASES, ids=[c[0] for c in EXTEND_CASES])
def test_extend_mx_matches_oracle(case):
    name, kv_lens, new_lens, Hq, Hkv, d_r, E, W, ls, page = case
    x = tinputs.make_extend_inputs(kv_lens, new_lens, Hq, Hkv, 128, d_r, max(E, 1), "bf16",
                                   seed=zlib.crc32(name.encode()) % 1000, page_size=page)
    out, lse = _extend_mx(x, E, W, ls, page)
    ref, lref = _extend_mx_ref(x, E, W, ls)
    assert_close(out, ref, torch.bfloat16, name, lse, lref)


@pytest.mark.parametrize("heads", [(8, 1), (8, 2)], ids=["G8", "G4"])
def test_extend_mx_bias_sensitivity_paged(heads):
    """P x50: the bias dominates the MXFP8 scores, so a slip in the shear, the
    extent edge or the page mapping changes the output by O(1)."""
    Hq, Hkv = heads
    x = tinputs.make_extend_inputs([600, 333], [150, 90], Hq, Hkv, 128, 64, 200, "bf16", seed=19, page_size=32)
    x["P"] = (x["P"].float() * 50).to(torch.bfloat16)
    x["P_cols"] = x["P"].t().contiguous()
    out, lse = _extend_mx(x, 200, 0, False, 32)
    ref, lref = _extend_mx_ref(x, 200, 0, False)
    assert_close(out, ref, torch.bfloat16, "mx P_x50", lse, lref)


def test_extend_mx_query_quantisation_matters():
    """Peaky queries (one value per 32-block scaled by 40) make the MXFP8
    rounding of q visible: the kernel must agree with the oracle on
    mx_round(q), and differ measurably from attention on the unrounded bf16 q.

    The scaled fp8 MFMA sums its 64 products with about 12 bits (measured on
    the device: |error| <= 2e-4 of the sum of |products|), so with these
    large scores the lse bar gets that allowance: 1e-3 + 4e-4 * alpha *
    max_j sum_d |q_d k_jd| per row."""
    x = tinputs.make_extend_inputs([400], [400], 8, 1, 128, 32, 64, "bf16", seed=23)
    q = x["q"].float()
    q[..., ::32] *= 40.0
    x["q"] = q.to(torch.bfloat16)
    out, lse = _extend_mx(x, 64, 0, False, 0)
    ref, lref = _extend_mx_ref(x, 64, 0, False)
    assert_close(out, ref, torch.bfloat16, "mx peaky q")
    qd = oracle.mx_round(x["q"])[:, :, None, :]                    # [T, H, 1, D]
    kd = oracle.mx_round(x["k"])[0, :, 0][None, None, :, :]        # [1, 1, T, D]
    T = qd.shape[0]
    visible = torch.tril(torch.ones(T, T, dtype=torch.bool))[:, None, :]
    absdot = torch.einsum("thd,jd->thj", qd[:, :, 0].abs(), kd[0, 0].abs()).masked_fill(~visible, 0)
    allow = 1e-3 + 4e-4 * ALPHA * absdot.amax(-1).t()             # [H, T]
    err = (lse.cpu().double() - lref).abs()
    assert bool((err <= allow).all()), f"lse error {err.max().item():.3e} beyond the allowance"
    plain, _ = oracle.extend(x["q"], oracle.mx_round(x["k"]), oracle.mx_round(x["v"]), x["r"], x["P"], ALPHA, 64, 0,
                             False, x["q_start"].tolist(), x["kv_len"].tolist())
    assert (plain - ref).abs().max().item() > 5e-2
