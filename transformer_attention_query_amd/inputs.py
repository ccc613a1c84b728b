"""Seeded synthetic inputs for relative attention, and the named workloads.

This module only draws random numbers and lays them out; it holds none of
the attention arithmetic, so both the HIP path and the CPU oracle can be fed
from it without sharing any computation.

Recipe (the same for every workload): a CPU ``torch.Generator`` seeded with
``seed`` draws, in this order and as float32 standard normals, q, k, v, r and
then P in the shapes below; P is multiplied by ``p_std`` (0.02, i.e.
P ~ N(0, 0.02^2)); every tensor is then rounded to the workload dtype.

* prefill: q [B,T,Hq,D], k [B,T,Hkv,D], v [B,T,Hkv,D], r [B,T,Hq,d_r], P [d_r,E]
* decode:  q [B,Hq,D],   k [B,L,Hkv,D], v [B,L,Hkv,D], r [B,Hq,d_r],   P [d_r,E]
* extend:  q [total_q,Hq,D] (packed new rows), k, v [B,Lcap,Hkv,D] (caches),
           r [total_q,Hq,d_r], P [d_r,E]; then, without further draws, the
           same caches cut into pages of ``page_size`` rows, placed at a
           seeded random permutation of page slots (a block table), when a
           page size is given.

* backward: the prefill tensors, then dout [B,T,Hq,D] (the gradient of the
           loss w.r.t. the attention output), drawn after P.
* prologue: q [N,Hq,D], k [N,Hkv,D], v [N,Hkv,D] (the raw projections of
           N packed new tokens), conv_k, conv_v [Hkv*D,W] times ``conv_std``
           (0.3), q_norm_w, k_norm_w [D] as 1 + 0.1 * normal, then (if asked)
           the state [B,2,3,Hkv*D], then the caches' prior contents
           [B,Lcap,Hkv,D] for k and v, cut into pages as for extend.  The
           pages give no distribution for these weights; the recipe only keeps
           the filter and norm outputs of order one.

P is drawn in the orientation of the method's notation (column d holds the
projection for distance d).  The library takes it distance-major, as
``P_cols`` [E, d_r] with ``P_cols[d] = P[:, d]``: the same numbers, stored so
that the d_r coefficients of one distance are contiguous.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch

__all__ = ["Workload", "WORKLOADS", "make_prefill_inputs", "make_backward_inputs", "make_decode_inputs",
           "make_extend_inputs", "make_prologue_inputs", "make_inputs", "torch_dtype"]


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


@dataclass(frozen=True)
class Workload:
    """One named relative-attention workload (shapes, masks and dtype)."""
    name: str
    kind: str            # "prefill", "backward", "decode", "extend" or "prologue"
    dtype: str           # "bf16" or "fp32"
    B: int
    T: int               # prefill: sequence length; decode, extend: kv length L
    Hq: int
    Hkv: int
    D: int
    d_r: int
    E: int               # rel_extent
    W: int = 0           # sliding window (keys incl. self); 0 = full causal
    log_scale: bool = False
    alpha: float = 1.0 / math.sqrt(128.0)
    num_splits: int = 0  # decode only; 0 = library's choice
    n_new: int = 0       # extend, prologue: new rows per sequence (the last n_new of its T)
    page_size: int = 0   # extend, prologue: rows per KV page; 0 = contiguous caches
    notes: str = field(default="", compare=False)


# The five workloads the kernels are specified and measured on.
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload(
        "tiny_fp32", "prefill", "fp32", B=1, T=256, Hq=4, Hkv=1, D=128, d_r=32, E=64,
        notes="tiny full-causal layer in fp32, GQA 4:1"),
    "swa_prefill_8k": Workload(
        "swa_prefill_8k", "prefill", "bf16", B=1, T=8192, Hq=16, Hkv=2, D=128, d_r=128, E=1024, W=1024,
        notes="sliding-window layer, 1024 keys incl. self, GQA 8:1"),
    "swa_backward_8k": Workload(
        "swa_backward_8k", "backward", "bf16", B=1, T=8192, Hq=16, Hkv=2, D=128, d_r=128, E=1024, W=1024,
        notes="backward of the sliding-window layer: dq, dk, dv, dr at an 8K packed sequence, E = 1024"),
    "full_prefill_32k_log": Workload(
        "full_prefill_32k_log", "prefill", "bf16", B=2, T=32768, Hq=16, Hkv=2, D=128, d_r=128, E=1024,
        log_scale=True, notes="full causal layer with the length log-scale (s = 1.25)"),
    "decode_64x8k": Workload(
        "decode_64x8k", "decode", "bf16", B=64, T=8192, Hq=16, Hkv=2, D=128, d_r=128, E=1024,
        notes="64 sequences x 1 token, kv length 8192, split-KV"),
    "decode_1x1m_log": Workload(
        "decode_1x1m_log", "decode", "bf16", B=1, T=1 << 20, Hq=16, Hkv=2, D=128, d_r=128, E=1024,
        log_scale=True, notes="1 sequence x 1 token, kv length 2^20, log-scale s = 5/3"),
    "decode_paged_64x8k": Workload(
        "decode_paged_64x8k", "extend", "bf16", B=64, T=8192, Hq=16, Hkv=2, D=128, d_r=128, E=1024,
        n_new=1, page_size=64,
        notes="decode_64x8k over a paged cache (64-row pages at shuffled slots), per-sequence lengths"),
    "extend_4x1k_8k_paged": Workload(
        "extend_4x1k_8k_paged", "extend", "bf16", B=4, T=8192, Hq=16, Hkv=2, D=128, d_r=128, E=1024,
        n_new=1024, page_size=64,
        notes="chunked prefill: 4 sequences x 1024 new rows over 7168 cached ones, paged KV (64 rows)"),
    "prologue_8k": Workload(
        "prologue_8k", "prologue", "bf16", B=1, T=8192, Hq=16, Hkv=2, D=128, d_r=0, E=0, n_new=8192,
        notes="attention prologue of an 8192-token prefill: K/V ShortConv (W=4), Q/K RMSNorm, cache write"),
    "prologue_decode_64": Workload(
        "prologue_decode_64", "prologue", "bf16", B=64, T=8192, Hq=16, Hkv=2, D=128, d_r=0, E=0, n_new=1,
        page_size=64, notes="decode-step prologue: 64 sequences x 1 token with carried state, paged KV"),
}


def _draw(gen: torch.Generator, shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def make_prefill_inputs(B: int, T: int, Hq: int, Hkv: int, D: int, d_r: int, E: int,
                        dtype: str = "bf16", seed: int = 0, p_std: float = 0.02,
                        device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """Seeded prefill inputs (see the module docstring for the recipe)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = torch_dtype(dtype)
    q = _draw(gen, (B, T, Hq, D)).to(dt)
    k = _draw(gen, (B, T, Hkv, D)).to(dt)
    v = _draw(gen, (B, T, Hkv, D)).to(dt)
    r = _draw(gen, (B, T, Hq, d_r)).to(dt)
    P = (_draw(gen, (d_r, E)) * p_std).to(dt)
    out = {"q": q, "k": k, "v": v, "r": r, "P": P, "P_cols": P.t().contiguous()}
    if device is not None:
        out = {n: t.to(device) for n, t in out.items()}
    return out


def make_backward_inputs(B: int, T: int, Hq: int, Hkv: int, D: int, d_r: int, E: int,
                         dtype: str = "bf16", seed: int = 0, p_std: float = 0.02,
                         device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """Seeded backward inputs: the prefill inputs of the same seed, then dout."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = torch_dtype(dtype)
    q = _draw(gen, (B, T, Hq, D)).to(dt)
    k = _draw(gen, (B, T, Hkv, D)).to(dt)
    v = _draw(gen, (B, T, Hkv, D)).to(dt)
    r = _draw(gen, (B, T, Hq, d_r)).to(dt)
    P = (_draw(gen, (d_r, E)) * p_std).to(dt)
    dout = _draw(gen, (B, T, Hq, D)).to(dt)
    out = {"q": q, "k": k, "v": v, "r": r, "P": P, "P_cols": P.t().contiguous(), "dout": dout}
    if device is not None:
        out = {n: t.to(device) for n, t in out.items()}
    return out


def make_decode_inputs(B: int, L: int, Hq: int, Hkv: int, D: int, d_r: int, E: int,
                       dtype: str = "bf16", seed: int = 0, p_std: float = 0.02,
                       device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """Seeded decode inputs: one query token per sequence, KV cache of length L."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = torch_dtype(dtype)
    q = _draw(gen, (B, Hq, D)).to(dt)
    k = _draw(gen, (B, L, Hkv, D)).to(dt)
    v = _draw(gen, (B, L, Hkv, D)).to(dt)
    r = _draw(gen, (B, Hq, d_r)).to(dt)
    P = (_draw(gen, (d_r, E)) * p_std).to(dt)
    out = {"q": q, "k": k, "v": v, "r": r, "P": P, "P_cols": P.t().contiguous()}
    if device is not None:
        out = {n: t.to(device) for n, t in out.items()}
    return out


def make_extend_inputs(kv_lens, new_lens, Hq: int, Hkv: int, D: int, d_r: int, E: int,
                       dtype: str = "bf16", seed: int = 0, p_std: float = 0.02, page_size: int = 0,
                       device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """Seeded extend inputs: sequence b has kv_lens[b] cached rows, the last
    new_lens[b] of which are its new query rows (packed in q and r).

    Returns q, r, k, v (contiguous caches [B, Lcap, Hkv, D], Lcap = max kv
    length), P, P_cols, q_start [B+1] and kv_len [B] (int32); with a page size
    also k_pages, v_pages [num_pages, page_size, Hkv, D] and block_table
    [B, max_pages] (int32, unused entries 0).
    """
    B = len(kv_lens)
    assert len(new_lens) == B and all(0 <= n <= L for n, L in zip(new_lens, kv_lens))
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = torch_dtype(dtype)
    total_q = int(sum(new_lens))
    Lcap = max(max(kv_lens), 1)
    q = _draw(gen, (total_q, Hq, D)).to(dt)
    k = _draw(gen, (B, Lcap, Hkv, D)).to(dt)
    v = _draw(gen, (B, Lcap, Hkv, D)).to(dt)
    r = _draw(gen, (total_q, Hq, d_r)).to(dt)
    P = (_draw(gen, (d_r, E)) * p_std).to(dt)
    q_start = torch.tensor([0] + list(torch.cumsum(torch.tensor(list(new_lens)), 0).tolist()), dtype=torch.int32)
    out = {"q": q, "k": k, "v": v, "r": r, "P": P, "P_cols": P.t().contiguous(), "q_start": q_start,
           "kv_len": torch.tensor(list(kv_lens), dtype=torch.int32)}
    if page_size > 0:
        pages = [(L + page_size - 1) // page_size for L in kv_lens]
        max_pages = max(max(pages), 1)
        n_pages = max(sum(pages), 1)
        perm = torch.randperm(n_pages, generator=gen)
        kp = torch.zeros(n_pages, page_size, Hkv, D, dtype=dt)
        vp = torch.zeros(n_pages, page_size, Hkv, D, dtype=dt)
        table = torch.zeros(B, max_pages, dtype=torch.int32)
        slot = 0
        for b, L in enumerate(kv_lens):
            for pg in range(pages[b]):
                dst = int(perm[slot])
                slot += 1
                table[b, pg] = dst
                lo, hi = pg * page_size, min(L, (pg + 1) * page_size)
                kp[dst, :hi - lo] = k[b, lo:hi]
                vp[dst, :hi - lo] = v[b, lo:hi]
        out.update(k_pages=kp, v_pages=vp, block_table=table)
    if device is not None:
        out = {n: t.to(device) for n, t in out.items()}
    return out


def make_prologue_inputs(kv_lens, new_lens, Hq: int, Hkv: int, D: int, W: int = 4, dtype: str = "bf16",
                         seed: int = 0, conv_std: float = 0.3, page_size: int = 0, with_state: bool = True,
                         device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """Seeded prologue inputs: sequence b's last new_lens[b] of kv_lens[b]
    positions are new (packed in q, k, v).  Returns q, k, v, conv_k, conv_v,
    q_norm_w, k_norm_w, q_start [B+1], kv_len [B] (int32), state_in
    [B,2,3,Hkv*D] (with_state), k_cache, v_cache [B,Lcap,Hkv,D] holding prior
    contents and, with a page size, k_pages, v_pages and block_table as for
    extend."""
    B = len(kv_lens)
    assert len(new_lens) == B and all(0 <= n <= L for n, L in zip(new_lens, kv_lens))
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = torch_dtype(dtype)
    N = int(sum(new_lens))
    Lcap = max(max(kv_lens), 1)
    out = {"q": _draw(gen, (N, Hq, D)).to(dt), "k": _draw(gen, (N, Hkv, D)).to(dt),
           "v": _draw(gen, (N, Hkv, D)).to(dt),
           "conv_k": (_draw(gen, (Hkv * D, W)) * conv_std).to(dt), "conv_v": (_draw(gen, (Hkv * D, W)) * conv_std).to(dt),
           "q_norm_w": (1.0 + 0.1 * _draw(gen, (D,))).to(dt), "k_norm_w": (1.0 + 0.1 * _draw(gen, (D,))).to(dt)}
    if with_state:
        out["state_in"] = _draw(gen, (B, 2, 3, Hkv * D)).to(dt)
    kc = _draw(gen, (B, Lcap, Hkv, D)).to(dt)
    vc = _draw(gen, (B, Lcap, Hkv, D)).to(dt)
    out["k_cache"], out["v_cache"] = kc, vc
    out["q_start"] = torch.tensor([0] + list(torch.cumsum(torch.tensor(list(new_lens)), 0).tolist()),
                                  dtype=torch.int32)
    out["kv_len"] = torch.tensor(list(kv_lens), dtype=torch.int32)
    if page_size > 0:
        pages = [(L + page_size - 1) // page_size for L in kv_lens]
        max_pages = max(max(pages), 1)
        n_pages = max(sum(pages), 1)
        perm = torch.randperm(n_pages, generator=gen)
        kp = torch.zeros(n_pages, page_size, Hkv, D, dtype=dt)
        vp = torch.zeros(n_pages, page_size, Hkv, D, dtype=dt)
        table = torch.zeros(B, max_pages, dtype=torch.int32)
        slot = 0
        for b, L in enumerate(kv_lens):
            for pg in range(pages[b]):
                dst = int(perm[slot])
                slot += 1
                table[b, pg] = dst
                lo, hi = pg * page_size, min(L, (pg + 1) * page_size)
                kp[dst, :hi - lo] = kc[b, lo:hi]
                vp[dst, :hi - lo] = vc[b, lo:hi]
        out.update(k_pages=kp, v_pages=vp, block_table=table)
    if device is not None:
        out = {n: t.to(device) for n, t in out.items()}
    return out


def make_inputs(w: Workload, seed: int = 0, device: Optional[str] = None) -> Dict[str, torch.Tensor]:
    """Inputs of a named workload."""
    if w.kind == "prologue":
        return make_prologue_inputs([w.T] * w.B, [w.n_new] * w.B, w.Hq, w.Hkv, w.D, 4, w.dtype, seed,
                                    page_size=w.page_size, with_state=w.n_new < w.T, device=device)
    if w.kind == "extend":
        return make_extend_inputs([w.T] * w.B, [w.n_new] * w.B, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.dtype, seed,
                                  page_size=w.page_size, device=device)
    if w.kind == "backward":
        return make_backward_inputs(w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.dtype, seed, device=device)
    if w.kind == "prefill":
        return make_prefill_inputs(w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.dtype, seed, device=device)
    return make_decode_inputs(w.B, w.T, w.Hq, w.Hkv, w.D, w.d_r, w.E, w.dtype, seed, device=device)
