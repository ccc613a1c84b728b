"""GPU: rel_attn_decode_noalloc (the decode that runs in the library's fixed
per-device scratch instead of a caller's workspace) against rel_attn_decode
with a workspace, on two calls in a row where the second is smaller, so stale
partials and bias rows left in the scratch by the first call must not leak
into the second.  Both entry points plan the same way and share the kernels,
so their outputs agree bit for bit; each output is also held to the oracle's
parity bar."""

import zlib

import pytest
import torch

import oracle
import transformer_attention_query_amd as ra
from transformer_attention_query_amd import inputs as tinputs
from parity import assert_close

pytestmark = pytest.mark.gpu

ALPHA = 1.0 / 128 ** 0.5


def _inputs(name, dt, B, L, Hq, Hkv, d_r, E):
    x = tinputs.make_decode_inputs(B, L, Hq, Hkv, 128, d_r, max(E, 1), dt, seed=zlib.crc32(name.encode()) % 1000)
    if E == 0:
        x["P_cols"] = x["P_cols"][:0]
    return x, {n: t.cuda() for n, t in x.items()}


def _both(xd, E, W, ls, ns=0):
    ref_out, ref_lse = ra.decode(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], ALPHA, E, W, ls, num_splits=ns)
    got_out, got_lse = ra.decode_noalloc(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], ALPHA, E, W, ls,
                                         num_splits=ns)
    torch.cuda.synchronize()
    return (got_out, got_lse), (ref_out, ref_lse)


# (first call, second call): name, dtype, B, L, Hq, Hkv, d_r, E, W, log_scale
PAIRS = [
    (("bf16_B8_L3000_E512", "bf16", 8, 3000, 16, 2, 128, 512, 0, False),
     ("bf16_B2_L700_E64", "bf16", 2, 700, 16, 2, 128, 64, 0, False)),
    (("bf16_B4_L5000_log_W2000", "bf16", 4, 5000, 32, 2, 64, 1024, 2000, True),
     ("bf16_B1_L333_log", "bf16", 1, 333, 8, 1, 32, 100, 0, True)),
    (("fp32_B3_L2500_E1024", "fp32", 3, 2500, 16, 2, 128, 1024, 0, False),
     ("fp32_B1_L97_W50_E0", "fp32", 1, 97, 4, 2, 16, 0, 50, False)),
    # sixteen query heads per kv head and a long extent: bias rows in the scratch
    (("bf16_G16_B2_L4100_E2048", "bf16", 2, 4100, 16, 1, 128, 2048, 0, False),
     ("bf16_G16_B1_L1500_E1400", "bf16", 1, 1500, 16, 1, 128, 1400, 0, False)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=[p[0][0] + "__then__" + p[1][0] for p in PAIRS])
def test_decode_noalloc_matches_decode_on_two_calls(pair):
    results = []
    for case in pair:
        name, dt, B, L, Hq, Hkv, d_r, E, W, ls = case
        assert ra.decode_plan(B, L, Hq, Hkv, 128, 0, W, E)[1] <= 16 << 20
        x, xd = _inputs(name, dt, B, L, Hq, Hkv, d_r, E)
        got, ref = _both(xd, E, W, ls)
        results.append((case, x, got, ref))
    for case, x, (go, gl), (ro, rl) in results:
        name = case[0]
        assert torch.equal(go, ro), f"{name}: out differs from rel_attn_decode"
        assert torch.equal(gl, rl), f"{name}: lse differs from rel_attn_decode"
        E, W, ls = case[7], case[8], case[9]
        oo, ol = oracle.decode(x["q"], x["k"], x["v"], x["r"], x["P"], ALPHA, E, W, ls)
        assert_close(go, oo, x["q"].dtype, name, gl, ol)


def test_decode_noalloc_split_counts_and_preallocated_outputs():
    """Forced split counts (one split writes the output directly; many use the
    merge), the second call smaller than the first, outputs passed in."""
    x, xd = _inputs("noalloc_splits", "bf16", 2, 3000, 16, 2, 128, 256)
    out = torch.empty_like(xd["q"])
    lse = torch.empty(xd["q"].shape[:2], dtype=torch.float32, device=out.device)
    for ns, B in ((64, 2), (7, 1), (1, 1)):
        q, k, v, r = (xd[n][:B].contiguous() for n in ("q", "k", "v", "r"))
        ref_o, ref_l = ra.decode(q, k, v, r, xd["P_cols"], ALPHA, 256, 0, False, num_splits=ns)
        o, l = ra.decode_noalloc(q, k, v, r, xd["P_cols"], ALPHA, 256, 0, False, num_splits=ns,
                                 out=out[:B], lse=lse[:B])
        torch.cuda.synchronize()
        assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), f"num_splits={ns}, B={B}"


def test_decode_noalloc_takes_no_device_memory():
    """With the outputs passed in, a call leaves the device's free memory as
    it was (the scratch is part of the library's image, not allocated per call)."""
    x, xd = _inputs("noalloc_mem", "bf16", 4, 4096, 16, 2, 128, 1024)
    out = torch.empty_like(xd["q"])
    lse = torch.empty(xd["q"].shape[:2], dtype=torch.float32, device=out.device)
    ra.decode_noalloc(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], ALPHA, 1024, out=out, lse=lse)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        ra.decode_noalloc(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], ALPHA, 1024, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0


def test_decode_noalloc_refuses_beyond_its_scratch():
    """A shape whose plan needs more than 16 MiB raises before any launch."""
    B, L, Hq, Hkv, E = 512, 4096, 32, 2, 1024
    assert ra.decode_plan(B, L, Hq, Hkv, 128, 0, 0, E)[1] > 16 << 20
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, L, Hkv, 128, dtype=torch.bfloat16, device="cuda")
    r = torch.zeros(B, Hq, 16, dtype=torch.bfloat16, device="cuda")
    P = torch.zeros(E, 16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="scratch"):
        ra.decode_noalloc(q, k, k, r, P, ALPHA, E)


def test_decode_noalloc_replays_from_a_captured_graph():
    """The caller it is for: a HIP graph captured around the call (outputs
    passed in, nothing allocated inside), replayed three times with eager
    calls in between that reuse the same scratch on other inputs; every
    replay equals the eager rel_attn_decode result bit for bit."""
    x, xd = _inputs("noalloc_graph", "bf16", 4, 3000, 16, 2, 128, 512)
    y, yd = _inputs("noalloc_graph_other", "bf16", 2, 5000, 16, 2, 128, 1024)
    ref_o, ref_l = ra.decode(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], ALPHA, 512)
    out = torch.empty_like(xd["q"])
    lse = torch.empty(xd["q"].shape[:2], dtype=torch.float32, device=out.device)
    run = lambda: ra.decode_noalloc(xd["q"], xd["k"], xd["v"], xd["r"], xd["P_cols"], ALPHA, 512,  # noqa: E731
                                    out=out, lse=lse)
    run()  # the device's scratch address is looked up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        out.fill_(0)
        lse.fill_(0)
        o2, l2 = ra.decode_noalloc(yd["q"], yd["k"], yd["v"], yd["r"], yd["P_cols"], ALPHA, 1024)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        assert torch.isfinite(o2.float()).all()
