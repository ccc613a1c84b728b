"""C-ABI checks that need no GPU: the library loads, exports every function
include/relattn.h declares, rejects bad arguments on the host before any HIP
call, plans decode splits as a pure function of the shape, and applies the
log-scale reading."""

import ctypes
import os
import re
import threading

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "relattn.h")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_WORKSPACE = 0, -1, -2, -3
RA_BF16, RA_F32 = 1, 2
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


@pytest.fixture(scope="session")
def lib():
    from transformer_attention_query_amd import binding
    if not os.path.exists(binding.library_path()):
        from transformer_attention_query_amd import build
        build.build(verbose=False)
    return binding.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("rel_attn_prefill", "rel_attn_extend", "rel_attn_decode", "rel_attn_decode_paged",
              "rel_attn_decode_plan", "rel_logits", "rel_attn_prologue", "rel_attn_prologue_mx",
              "rel_attn_decode_mx", "rel_mx_quantize", "rel_attn_backward", "rel_attn_backward_plan",
              "rel_attn_last_error", "rel_attn_version", "rel_attn_scale_factor"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), f"{n} declared in relattn.h but not exported"


def test_version(lib):
    assert lib.rel_attn_version() >= 100


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, r=FAKE + 48, P=FAKE + 64, out=FAKE + 80, lse=None,
             dtype=RA_BF16, B=1, T=16, Hq=4, Hkv=2, D=128, d_r=32, alpha=0.1, E=8, W=0, ls=0)
    a.update(kw)
    return lib.rel_attn_prefill(a["q"], a["k"], a["v"], a["r"], a["P"], a["out"], a["lse"], a["dtype"],
                                a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["d_r"], a["alpha"], a["E"],
                                a["W"], a["ls"], None)


def _err(lib):
    return lib.rel_attn_last_error().decode()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(dtype=7), RA_ERR_INVALID_ARG, "dtype"),
    (dict(B=-1), RA_ERR_INVALID_ARG, "B ="),
    (dict(T=-3), RA_ERR_INVALID_ARG, "T ="),
    (dict(Hq=6, Hkv=4), RA_ERR_INVALID_ARG, "multiple"),
    (dict(Hkv=0), RA_ERR_INVALID_ARG, "positive"),
    (dict(E=-1), RA_ERR_INVALID_ARG, "rel_extent"),
    (dict(W=-2), RA_ERR_INVALID_ARG, "window"),
    (dict(ls=2), RA_ERR_INVALID_ARG, "log_scale"),
    (dict(alpha=float("nan")), RA_ERR_INVALID_ARG, "alpha"),
    (dict(D=64), RA_ERR_UNSUPPORTED, "head dim"),
    (dict(d_r=24), RA_ERR_UNSUPPORTED, "d_r"),
    (dict(d_r=256), RA_ERR_UNSUPPORTED, "d_r"),
    (dict(q=None), RA_ERR_INVALID_ARG, "q is NULL"),
    (dict(out=None), RA_ERR_INVALID_ARG, "out is NULL"),
    (dict(r=None), RA_ERR_INVALID_ARG, "r is NULL"),
    (dict(P=None), RA_ERR_INVALID_ARG, "P_cols is NULL"),
    (dict(k=FAKE + 2), RA_ERR_INVALID_ARG, "aligned"),
    (dict(lse=FAKE + 4), RA_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE), RA_ERR_INVALID_ARG, "alias"),
])
def test_prefill_rejects_bad_arguments(lib, kw, code, frag):
    assert _prefill(lib, **kw) == code
    assert frag in _err(lib)


def test_prefill_empty_is_a_noop(lib):
    assert _prefill(lib, B=0) == RA_OK
    assert _prefill(lib, T=0) == RA_OK
    assert _err(lib) == ""


def test_prefill_without_bias_needs_no_r_or_P(lib):
    # E = 0: r and P may be NULL and d_r is not checked; T = 0 keeps it off the GPU
    assert _prefill(lib, E=0, r=None, P=None, d_r=0, T=0) == RA_OK


def _plan(lib, B, L, Hq, Hkv, req=0, W=0, D=128, E=0):
    ns = ctypes.c_int(-1)
    ws = ctypes.c_size_t(0)
    rc = lib.rel_attn_decode_plan(B, L, Hq, Hkv, D, req, W, E, ctypes.byref(ns), ctypes.byref(ws))
    return rc, ns.value, ws.value


def test_decode_plan_is_pure_and_sized():
    from transformer_attention_query_amd import binding
    lib = binding.load_library()
    for (B, L, Hq, Hkv) in [(64, 8192, 16, 2), (1, 1 << 20, 16, 2), (3, 77, 8, 8), (1, 1, 4, 1)]:
        a = _plan(lib, B, L, Hq, Hkv)
        b = _plan(lib, B, L, Hq, Hkv)
        assert a == b and a[0] == RA_OK
        ns = a[1]
        assert 1 <= ns <= (L + 31) // 32
        partial = (ns * B * Hq * (128 + 2) * 4 + 255) // 256 * 256
        assert a[2] >= partial + B * Hq * 32 * 4   # split partials + one (zero) bias row per head
        # with a relative extent the workspace adds one bias row per (sequence, head)
        rc, ns2, ws2 = _plan(lib, B, L, Hq, Hkv, E=1024)
        assert rc == RA_OK and ns2 == ns and ws2 >= partial + B * Hq * 1024 * 4
    # forced split counts are honoured up to one 32-key step per split
    for req in (1, 2, 3, 7, 64):
        rc, ns, _ = _plan(lib, 2, 3000, 16, 2, req)
        assert rc == RA_OK and ns <= req
    rc, ns, _ = _plan(lib, 1, 300, 16, 2, 64)
    assert ns == 2                      # splits hold whole 256-key quanta: 300 keys -> 2
    # a window limits the visible range
    rc, ns, _ = _plan(lib, 1, 100000, 16, 2, 0, 64)
    assert ns <= 2


@pytest.mark.parametrize("args,code", [
    ((1, 0, 16, 2), RA_ERR_INVALID_ARG),
    ((-1, 10, 16, 2), RA_ERR_INVALID_ARG),
    ((1, 10, 16, 3), RA_ERR_INVALID_ARG),
    ((1, 10, 16, 2, 0, 0, 128, -1), RA_ERR_INVALID_ARG),
])
def test_decode_plan_rejects(lib, args, code):
    assert _plan(lib, *args)[0] == code


def test_decode_plan_rejects_other_head_dims(lib):
    assert _plan(lib, 1, 10, 16, 2, D=64)[0] == RA_ERR_UNSUPPORTED


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, r=FAKE + 48, P=FAKE + 64, out=FAKE + 80, lse=None,
             dtype=RA_BF16, B=2, L=300, Hq=16, Hkv=2, D=128, d_r=128, alpha=0.1, E=64, W=0, ls=0,
             ns=0, ws=None, wsb=0)
    a.update(kw)
    return lib.rel_attn_decode(a["q"], a["k"], a["v"], a["r"], a["P"], a["out"], a["lse"], a["dtype"],
                               a["B"], a["L"], a["Hq"], a["Hkv"], a["D"], a["d_r"], a["alpha"], a["E"],
                               a["W"], a["ls"], a["ns"], a["ws"], a["wsb"], None)


def test_decode_with_no_sequences_is_a_no_op(lib):
    """B == 0 plans without dividing by the workgroup count and returns RA_OK
    before touching the workspace (a division by zero here once killed the
    process)."""
    rc, ns, need = _plan(lib, 0, 300, 16, 2, E=64)
    assert rc == RA_OK and ns >= 1
    assert _decode(lib, B=0) == RA_OK


def test_decode_workspace_errors(lib):
    assert _decode(lib) == RA_ERR_WORKSPACE and "NULL" in _err(lib)
    assert _decode(lib, ws=FAKE + 512 + 16, wsb=1 << 30) == RA_ERR_WORKSPACE and "256-byte" in _err(lib)
    _, ns, need = _plan(lib, 2, 300, 16, 2, E=64)
    assert _decode(lib, ws=FAKE * 16, wsb=need - 1) == RA_ERR_WORKSPACE and "smaller" in _err(lib)


@pytest.mark.parametrize("kw,code", [
    (dict(L=0), RA_ERR_INVALID_ARG),
    (dict(ns=-1), RA_ERR_INVALID_ARG),
    (dict(dtype=0), RA_ERR_INVALID_ARG),
    (dict(D=256), RA_ERR_UNSUPPORTED),
    (dict(v=None), RA_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_arguments(lib, kw, code):
    assert _decode(lib, **kw) == code


def _decode_noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, r=FAKE + 48, P=FAKE + 64, out=FAKE + 80, lse=None,
             dtype=RA_BF16, B=2, L=300, Hq=16, Hkv=2, D=128, d_r=128, alpha=0.1, E=64, W=0, ls=0, ns=0)
    a.update(kw)
    return lib.rel_attn_decode_noalloc(a["q"], a["k"], a["v"], a["r"], a["P"], a["out"], a["lse"], a["dtype"],
                                       a["B"], a["L"], a["Hq"], a["Hkv"], a["D"], a["d_r"], a["alpha"], a["E"],
                                       a["W"], a["ls"], a["ns"], None)


NOALLOC_SCRATCH = 16 << 20


@pytest.mark.parametrize("kw,code", [
    (dict(L=0), RA_ERR_INVALID_ARG),
    (dict(ns=-1), RA_ERR_INVALID_ARG),
    (dict(dtype=0), RA_ERR_INVALID_ARG),
    (dict(D=256), RA_ERR_UNSUPPORTED),
    (dict(v=None), RA_ERR_INVALID_ARG),
    (dict(out=FAKE), RA_ERR_INVALID_ARG),
])
def test_decode_noalloc_rejects_bad_arguments(lib, kw, code):
    assert _decode_noalloc(lib, **kw) == code


def test_decode_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """A plan that needs more than the fixed scratch is refused on the host
    (before any HIP call), with the sizes in the message; B == 0 is a no-op."""
    B, L, Hq, Hkv, E = 512, 4096, 32, 2, 1024
    rc, ns, need = _plan(lib, B, L, Hq, Hkv, E=E)
    assert rc == RA_OK and need > NOALLOC_SCRATCH
    assert _decode_noalloc(lib, B=B, L=L, Hq=Hq, Hkv=Hkv, E=E) == RA_ERR_WORKSPACE
    assert str(need) in _err(lib) and str(NOALLOC_SCRATCH) in _err(lib)
    assert _decode_noalloc(lib, B=0) == RA_OK
    # the measured decode shapes fit it
    for B, L in ((64, 8192), (1, 1 << 20)):
        assert _plan(lib, B, L, 16, 2, E=1024)[2] <= NOALLOC_SCRATCH


def test_rel_logits_rejects_bad_arguments(lib):
    f = lib.rel_logits
    assert f(FAKE, FAKE + 16, FAKE + 32, 3, 10, 2, 32, 64, 0, 10, None) == RA_ERR_INVALID_ARG
    assert f(FAKE, FAKE + 16, FAKE + 32, RA_BF16, -1, 2, 32, 64, 0, 10, None) == RA_ERR_INVALID_ARG
    assert f(FAKE, FAKE + 16, FAKE + 32, RA_BF16, 10, 2, 32, 0, 0, 10, None) == RA_ERR_INVALID_ARG
    assert f(FAKE, FAKE + 16, FAKE + 32, RA_BF16, 10, 2, 40, 64, 0, 10, None) == RA_ERR_UNSUPPORTED
    assert f(None, FAKE + 16, FAKE + 32, RA_BF16, 10, 2, 32, 64, 0, 10, None) == RA_ERR_INVALID_ARG
    assert f(FAKE, FAKE + 16, FAKE + 32, RA_BF16, 0, 2, 32, 64, 0, 10, None) == RA_OK


def test_last_error_is_per_thread(lib):
    assert _prefill(lib, dtype=9) == RA_ERR_INVALID_ARG
    seen = {}

    def other():
        seen["msg"] = lib.rel_attn_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "dtype" in _err(lib)


def test_scale_factor_reading(lib):
    f = lib.rel_attn_scale_factor
    assert f(0, 1 << 20) == 1.0
    assert f(1, 4096) == 1.0 and f(1, 100) == 1.0
    assert abs(f(1, 32768) - 1.25) < 1e-15
    assert abs(f(1, 1 << 20) - 5.0 / 3.0) < 1e-15


def _extend(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, r=FAKE, P=FAKE, out=FAKE + 0x1000, lse=None, dtype=RA_BF16, B=2,
             total_q=10, max_q=8, q_start=FAKE, kv_len=FAKE, cache_len=64, block_table=None, max_pages=0,
             num_pages=0, page_size=0, Hq=8, Hkv=1, D=128, d_r=64, alpha=0.1, E=32, W=0, ls=0)
    a.update(kw)
    return lib.rel_attn_extend(a["q"], a["k"], a["v"], a["r"], a["P"], a["out"], a["lse"], a["dtype"], a["B"],
                               a["total_q"], a["max_q"], a["q_start"], a["kv_len"], a["cache_len"],
                               a["block_table"], a["max_pages"], a["num_pages"], a["page_size"], a["Hq"],
                               a["Hkv"], a["D"], a["d_r"], a["alpha"], a["E"], a["W"], a["ls"], None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(block_table=FAKE, page_size=48, max_pages=4, num_pages=8), RA_ERR_UNSUPPORTED, "page_size"),
    (dict(block_table=FAKE, page_size=0, max_pages=4, num_pages=8), RA_ERR_UNSUPPORTED, "page_size"),
    (dict(block_table=FAKE, page_size=64, max_pages=0, num_pages=8), RA_ERR_INVALID_ARG, "max_pages"),
    (dict(cache_len=0), RA_ERR_INVALID_ARG, "cache_len"),
    (dict(q_start=None), RA_ERR_INVALID_ARG, "q_start"),
    (dict(kv_len=FAKE + 2), RA_ERR_INVALID_ARG, "aligned"),
    (dict(max_q=-1), RA_ERR_INVALID_ARG, "max_q"),
    (dict(D=64), RA_ERR_UNSUPPORTED, "head dim"),
    (dict(d_r=40), RA_ERR_UNSUPPORTED, "d_r"),
    (dict(out=FAKE), RA_ERR_INVALID_ARG, "alias"),
    (dict(Hq=6, Hkv=4), RA_ERR_INVALID_ARG, "multiple"),
    (dict(r=None), RA_ERR_INVALID_ARG, "r is NULL"),
])
def test_extend_rejects_bad_arguments(lib, kw, code, frag):
    assert _extend(lib, **kw) == code
    assert frag in lib.rel_attn_last_error().decode()


def test_extend_empty_is_a_noop(lib):
    for kw in (dict(B=0), dict(total_q=0), dict(max_q=0)):
        assert _extend(lib, q=None, k=None, v=None, out=None, q_start=None, kv_len=None, **kw) == RA_OK


def _extend_mx(lib, **kw):
    a = dict(q=FAKE, kc=FAKE + 0x100, ks=FAKE + 0x200, vc=FAKE + 0x300, vs=FAKE + 0x400, r=FAKE + 0x500,
             P=FAKE + 0x600, out=FAKE + 0x1000, lse=None, B=2, total_q=10, max_q=8, q_start=FAKE, kv_len=FAKE,
             cache_len=64, block_table=None, max_pages=0, num_pages=0, page_size=0, Hq=8, Hkv=1, D=128, d_r=64,
             alpha=0.1, E=32, W=0, ls=0)
    a.update(kw)
    return lib.rel_attn_extend_mx(a["q"], a["kc"], a["ks"], a["vc"], a["vs"], a["r"], a["P"], a["out"], a["lse"],
                                  a["B"], a["total_q"], a["max_q"], a["q_start"], a["kv_len"], a["cache_len"],
                                  a["block_table"], a["max_pages"], a["num_pages"], a["page_size"], a["Hq"],
                                  a["Hkv"], a["D"], a["d_r"], a["alpha"], a["E"], a["W"], a["ls"], None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(ks=None), RA_ERR_INVALID_ARG, "scales"),
    (dict(vs=None), RA_ERR_INVALID_ARG, "scales"),
    (dict(kc=None), RA_ERR_INVALID_ARG, "k is NULL"),
    (dict(out=FAKE + 0x200), RA_ERR_INVALID_ARG, "alias"),
    (dict(lse=FAKE + 0x400), RA_ERR_INVALID_ARG, "alias"),
    (dict(block_table=FAKE, page_size=48, max_pages=4, num_pages=8), RA_ERR_UNSUPPORTED, "page_size"),
    (dict(cache_len=0), RA_ERR_INVALID_ARG, "cache_len"),
    (dict(D=64), RA_ERR_UNSUPPORTED, "head dim"),
    (dict(d_r=40), RA_ERR_UNSUPPORTED, "d_r"),
    (dict(q_start=None), RA_ERR_INVALID_ARG, "q_start"),
])
def test_extend_mx_rejects_bad_arguments(lib, kw, code, frag):
    assert _extend_mx(lib, **kw) == code
    assert frag in lib.rel_attn_last_error().decode()


def test_extend_mx_empty_is_a_noop(lib):
    for kw in (dict(B=0), dict(total_q=0), dict(max_q=0)):
        assert _extend_mx(lib, q=None, kc=None, ks=None, vc=None, vs=None, out=None, q_start=None, kv_len=None,
                          **kw) == RA_OK


def _decode_paged(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, r=FAKE, P=FAKE, out=FAKE + 0x1000, lse=None, dtype=RA_BF16, B=2, max_len=100,
             kv_len=FAKE, bt=FAKE, max_pages=4, num_pages=8, page_size=32, Hq=8, Hkv=1, D=128, d_r=64,
             alpha=0.1, E=32, W=0, ls=0, ns=0, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.rel_attn_decode_paged(a["q"], a["k"], a["v"], a["r"], a["P"], a["out"], a["lse"], a["dtype"], a["B"],
                                     a["max_len"], a["kv_len"], a["bt"], a["max_pages"], a["num_pages"],
                                     a["page_size"], a["Hq"], a["Hkv"], a["D"], a["d_r"], a["alpha"], a["E"],
                                     a["W"], a["ls"], a["ns"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(page_size=48), RA_ERR_UNSUPPORTED, "page_size"),
    (dict(max_pages=0), RA_ERR_INVALID_ARG, "max_pages"),
    (dict(bt=None), RA_ERR_INVALID_ARG, "block_table"),
    (dict(kv_len=FAKE + 1), RA_ERR_INVALID_ARG, "aligned"),
    (dict(max_len=0), RA_ERR_INVALID_ARG, "max_len"),
    (dict(D=96), RA_ERR_UNSUPPORTED, "head dim"),
    (dict(out=FAKE), RA_ERR_INVALID_ARG, "alias"),
    (dict(ns=-1), RA_ERR_INVALID_ARG, "num_splits"),
    (dict(), RA_ERR_WORKSPACE, "workspace is NULL"),
    (dict(ws=FAKE + 16, ws_bytes=1 << 30), RA_ERR_WORKSPACE, "256-byte"),
    (dict(ws=FAKE, ws_bytes=16), RA_ERR_WORKSPACE, "smaller"),
])
def test_decode_paged_rejects_bad_arguments(lib, kw, code, frag):
    assert _decode_paged(lib, **kw) == code
    assert frag in lib.rel_attn_last_error().decode()


def _prologue(lib, **kw):
    a = dict(q_in=FAKE, k_in=FAKE + 0x100, v_in=FAKE + 0x200, conv_k=FAKE + 0x300, conv_v=FAKE + 0x400,
             qw=FAKE + 0x500, kw_=FAKE + 0x600, eps=1e-6, st_in=None, st_out=None, q_out=FAKE + 0x700,
             k_cache=FAKE + 0x800, v_cache=FAKE + 0x900, dtype=RA_BF16, B=2, total_q=10, q_start=FAKE + 0xa00,
             kv_len=FAKE + 0xb00, cache_len=64, block_table=None, max_pages=0, num_pages=0, page_size=0,
             Hq=8, Hkv=1, D=128, W=4)
    a.update(kw)
    return lib.rel_attn_prologue(a["q_in"], a["k_in"], a["v_in"], a["conv_k"], a["conv_v"], a["qw"], a["kw_"],
                                 a["eps"], a["st_in"], a["st_out"], a["q_out"], a["k_cache"], a["v_cache"],
                                 a["dtype"], a["B"], a["total_q"], a["q_start"], a["kv_len"], a["cache_len"],
                                 a["block_table"], a["max_pages"], a["num_pages"], a["page_size"], a["Hq"],
                                 a["Hkv"], a["D"], a["W"], None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(W=5), RA_ERR_UNSUPPORTED, "conv_width"),
    (dict(W=0), RA_ERR_UNSUPPORTED, "conv_width"),
    (dict(D=64), RA_ERR_UNSUPPORTED, "head dim"),
    (dict(eps=-1.0), RA_ERR_INVALID_ARG, "eps"),
    (dict(eps=float("inf")), RA_ERR_INVALID_ARG, "eps"),
    (dict(dtype=3), RA_ERR_INVALID_ARG, "dtype"),
    (dict(q_start=None), RA_ERR_INVALID_ARG, "q_start"),
    (dict(kv_len=FAKE + 2), RA_ERR_INVALID_ARG, "aligned"),
    (dict(conv_k=FAKE + 1), RA_ERR_INVALID_ARG, "element size"),
    (dict(k_cache=FAKE + 8), RA_ERR_INVALID_ARG, "16-byte"),
    (dict(k_cache=FAKE + 0x900), RA_ERR_INVALID_ARG, "same buffer"),
    (dict(v_cache=FAKE), RA_ERR_INVALID_ARG, "alias"),
    (dict(q_out=FAKE + 0x100), RA_ERR_INVALID_ARG, "q_out"),
    (dict(st_in=FAKE + 0xc00, st_out=FAKE + 0xc00), RA_ERR_INVALID_ARG, "state_out aliases"),
    (dict(cache_len=0), RA_ERR_INVALID_ARG, "cache_len"),
    (dict(block_table=FAKE + 0xd00, page_size=0, max_pages=4, num_pages=8), RA_ERR_INVALID_ARG, "page_size"),
    (dict(block_table=FAKE + 0xd00, page_size=16, max_pages=0, num_pages=8), RA_ERR_INVALID_ARG, "max_pages"),
    (dict(Hkv=0), RA_ERR_INVALID_ARG, "positive"),
])
def test_prologue_rejects_bad_arguments(lib, kw, code, frag):
    assert _prologue(lib, **kw) == code
    assert frag in lib.rel_attn_last_error().decode()


def test_prologue_empty_is_a_noop(lib):
    nulls = dict(q_in=None, k_in=None, v_in=None, q_out=None, k_cache=None, v_cache=None, conv_k=None,
                 conv_v=None, qw=None, kw_=None, q_start=None, kv_len=None)
    assert _prologue(lib, B=0, **nulls) == RA_OK
    assert _prologue(lib, total_q=0, **nulls) == RA_OK


def _decode_mx(lib, **kw):
    a = dict(q=FAKE, kc=FAKE + 0x100, ks=FAKE + 0x200, vc=FAKE + 0x300, vs=FAKE + 0x400, r=FAKE + 0x500,
             P=FAKE + 0x600, out=FAKE + 0x700, lse=None, B=2, L=100, kv_len=None, bt=None, max_pages=0, num_pages=0,
             page_size=0, Hq=16, Hkv=2, D=128, d_r=64, alpha=0.1, E=32, W=0, ls=0, ns=0, ws=FAKE + 0x1000,
             ws_bytes=1 << 30)
    a.update(kw)
    return lib.rel_attn_decode_mx(a["q"], a["kc"], a["ks"], a["vc"], a["vs"], a["r"], a["P"], a["out"], a["lse"],
                                  a["B"], a["L"], a["kv_len"], a["bt"], a["max_pages"], a["num_pages"],
                                  a["page_size"], a["Hq"], a["Hkv"], a["D"], a["d_r"], a["alpha"], a["E"], a["W"],
                                  a["ls"], a["ns"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(ks=None), RA_ERR_INVALID_ARG, "scales"),
    (dict(kv_len=FAKE + 0x800), RA_ERR_INVALID_ARG, "paged"),
    (dict(bt=FAKE + 0x800), RA_ERR_INVALID_ARG, "kv_len"),
    (dict(bt=FAKE + 0x800, kv_len=FAKE + 0x900, page_size=48, max_pages=4, num_pages=8), RA_ERR_UNSUPPORTED, "page_size"),
    (dict(L=0), RA_ERR_INVALID_ARG, "L = 0"),
    (dict(D=64), RA_ERR_UNSUPPORTED, "head dim"),
    (dict(out=FAKE + 0x300), RA_ERR_INVALID_ARG, "alias"),
    (dict(ws=None), RA_ERR_WORKSPACE, "workspace"),
    (dict(ws_bytes=16), RA_ERR_WORKSPACE, "smaller"),
    (dict(kc=FAKE + 8), RA_ERR_INVALID_ARG, "16-byte"),
])
def test_decode_mx_rejects_bad_arguments(lib, kw, code, frag):
    assert _decode_mx(lib, **kw) == code
    assert frag in lib.rel_attn_last_error().decode()


def test_mx_quantize_rejects_and_noop(lib):
    assert lib.rel_mx_quantize(FAKE, FAKE + 0x100, FAKE + 0x200, RA_BF16, 0, 128, None) == RA_OK
    assert lib.rel_mx_quantize(FAKE, FAKE + 0x100, FAKE + 0x200, RA_BF16, 10, 64, None) == RA_ERR_UNSUPPORTED
    assert lib.rel_mx_quantize(FAKE, FAKE, FAKE + 0x200, RA_BF16, 10, 128, None) == RA_ERR_INVALID_ARG
    assert lib.rel_mx_quantize(FAKE, FAKE + 0x100, None, RA_BF16, 10, 128, None) == RA_ERR_INVALID_ARG
    assert lib.rel_mx_quantize(FAKE, FAKE + 0x100, FAKE + 0x200, 7, 10, 128, None) == RA_ERR_INVALID_ARG
    assert lib.rel_mx_quantize(FAKE, FAKE + 0x100, FAKE + 0x200, RA_BF16, -1, 128, None) == RA_ERR_INVALID_ARG


def _prologue_mx(lib, **kw):
    a = dict(q_in=FAKE, k_in=FAKE + 0x100, v_in=FAKE + 0x200, conv_k=FAKE + 0x300, conv_v=FAKE + 0x400,
             qw=FAKE + 0x500, kw_=FAKE + 0x600, eps=1e-6, st_in=None, st_out=None, q_out=FAKE + 0x700,
             kc=FAKE + 0x800, ks=FAKE + 0x900, vc=FAKE + 0xa00, vs=FAKE + 0xb00, B=2, total_q=10,
             q_start=FAKE + 0xc00, kv_len=FAKE + 0xd00, cache_len=64, block_table=None, max_pages=0, num_pages=0,
             page_size=0, Hq=8, Hkv=1, D=128, W=4)
    a.update(kw)
    return lib.rel_attn_prologue_mx(a["q_in"], a["k_in"], a["v_in"], a["conv_k"], a["conv_v"], a["qw"], a["kw_"],
                                    a["eps"], a["st_in"], a["st_out"], a["q_out"], a["kc"], a["ks"], a["vc"], a["vs"],
                                    a["B"], a["total_q"], a["q_start"], a["kv_len"], a["cache_len"],
                                    a["block_table"], a["max_pages"], a["num_pages"], a["page_size"], a["Hq"],
                                    a["Hkv"], a["D"], a["W"], None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(ks=None), RA_ERR_INVALID_ARG, "scales"),
    (dict(vs=FAKE + 0x900), RA_ERR_INVALID_ARG, "overlap"),
    (dict(ks=FAKE + 0x800), RA_ERR_INVALID_ARG, "overlap"),
    (dict(vs=FAKE), RA_ERR_INVALID_ARG, "alias"),
    (dict(W=5), RA_ERR_UNSUPPORTED, "conv_width"),
    (dict(cache_len=0), RA_ERR_INVALID_ARG, "cache_len"),
])
def test_prologue_mx_rejects_bad_arguments(lib, kw, code, frag):
    assert _prologue_mx(lib, **kw) == code
    assert frag in lib.rel_attn_last_error().decode()


# ---------------------------------------------------------------- backward

def _bplan(lib, B, T, Hq, Hkv, D=128, req=0):
    ns, wb = ctypes.c_int(-7), ctypes.c_size_t(0)
    rc = lib.rel_attn_backward_plan(B, T, Hq, Hkv, D, req, ctypes.byref(ns), ctypes.byref(wb))
    return rc, ns.value, wb.value


def test_backward_plan_is_pure_and_sized(lib):
    rc, ns, wb = _bplan(lib, 1, 8192, 16, 2)
    # 64 blocks of 128 keys x 2 kv heads = 128 workgroups: the 8 heads of a group split in 2
    assert rc == RA_OK and ns == 2
    assert wb == 16 * 8192 * 4 + 2 * 2 * 8192 * 2 * 128 * 4
    assert _bplan(lib, 1, 8192, 16, 2) == (rc, ns, wb)
    rc, ns, wb = _bplan(lib, 2, 32768, 16, 2)
    assert rc == RA_OK and ns == 1 and wb == 2 * 16 * 32768 * 4  # enough blocks: no split, no partials
    assert _bplan(lib, 1, 100, 16, 2, req=4)[:2] == (RA_OK, 4)
    rc, ns, wb = _bplan(lib, 1, 5, 3, 3)  # one head per kv head: nothing to split
    assert rc == RA_OK and ns == 1 and wb == 256


@pytest.mark.parametrize("args,code", [
    ((1, 100, 16, 2, 128, 3), RA_ERR_INVALID_ARG),
    ((1, 100, 16, 2, 128, -1), RA_ERR_INVALID_ARG),
    ((1, 100, 6, 4, 128, 0), RA_ERR_INVALID_ARG),
    ((-1, 100, 16, 2, 128, 0), RA_ERR_INVALID_ARG),
    ((1, 100, 16, 2, 64, 0), RA_ERR_UNSUPPORTED),
])
def test_backward_plan_rejects(lib, args, code):
    assert _bplan(lib, *args)[0] == code


def _backward(lib, **kw):
    a = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, r=FAKE + 48, P=FAKE + 64, out=FAKE + 80, dout=FAKE + 96,
             lse=FAKE + 112, dq=FAKE + 128, dk=FAKE + 144, dv=FAKE + 160, dr=FAKE + 176, dtype=RA_BF16,
             B=1, T=100, Hq=16, Hkv=2, D=128, d_r=128, alpha=0.1, E=64, W=0, ls=0, ns=1, ws=FAKE * 16,
             wsb=1 << 30)
    a.update(kw)
    return lib.rel_attn_backward(a["q"], a["k"], a["v"], a["r"], a["P"], a["out"], a["dout"], a["lse"], a["dq"],
                                 a["dk"], a["dv"], a["dr"], a["dtype"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"],
                                 a["d_r"], a["alpha"], a["E"], a["W"], a["ls"], a["ns"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(dtype=RA_F32), RA_ERR_UNSUPPORTED, "RA_BF16"),
    (dict(dtype=5), RA_ERR_INVALID_ARG, "dtype"),
    (dict(lse=None), RA_ERR_INVALID_ARG, "lse is NULL"),
    (dict(dout=None), RA_ERR_INVALID_ARG, "dout is NULL"),
    (dict(dr=None), RA_ERR_INVALID_ARG, "dr is NULL"),
    (dict(dq=FAKE), RA_ERR_INVALID_ARG, "alias"),
    (dict(dv=FAKE + 144), RA_ERR_INVALID_ARG, "alias"),
    (dict(dk=FAKE * 16), RA_ERR_INVALID_ARG, "alias"),
    (dict(ns=3), RA_ERR_INVALID_ARG, "head_splits"),
    (dict(ns=0), RA_ERR_INVALID_ARG, "head_splits"),
    (dict(ws=None), RA_ERR_WORKSPACE, "NULL"),
    (dict(ws=FAKE * 16 + 16), RA_ERR_WORKSPACE, "256-byte"),
    (dict(wsb=100), RA_ERR_WORKSPACE, "smaller"),
    (dict(d_r=24), RA_ERR_UNSUPPORTED, "d_r"),
    (dict(D=96), RA_ERR_UNSUPPORTED, "head dim"),
])
def test_backward_rejects_bad_arguments(lib, kw, code, frag):
    assert _backward(lib, **kw) == code
    assert frag in _err(lib)


def test_backward_without_bias_needs_no_r_P_or_dr_and_empty_is_a_noop(lib):
    assert _backward(lib, B=0, ws=None, wsb=0) == RA_OK
    assert _backward(lib, T=0, ws=None, wsb=0) == RA_OK
    assert _backward(lib, E=0, r=None, P=None, dr=None, B=0) == RA_OK
