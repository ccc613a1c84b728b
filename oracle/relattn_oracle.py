"""Plain fp64 CPU oracle for Inkling-style relative attention (forward).

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  The product path (the HIP library and its Python
binding) never imports, links or calls it, and it imports nothing from the
product path.  It takes tensors and returns tensors; where the inputs come
from is not its business.

What it computes is the definition written out, in float64, with the full
logit rows materialised:

* relative logits -- "SGLang and Miles Add Day-0 Support for Inkling",
  section "Attention with Relative Positional Embedding", eq. for
  rel_logits: rel_logits(t,h,d) = r_{t,h} . P[:, d] for distance d in
  [0, rel_extent).  The same definition is restated in the section
  "Customized Efficient Kernels for Train-Inference Consistency".
* the logit -- same section, eq. for l(i,j,h):
  l(i,j,h) = alpha * q_{i,h} . k_{j,h} + 1[0 <= i-j < rel_extent] * rel_logits(i,h,i-j).
* masks -- same section: future keys are masked (causal); "Attention layout"
  paragraph: sliding-window layers keep only recent keys, full layers see
  every past key; both use the relative bias.
* the length-dependent log-scale on q and on the relative logits -- same
  paragraph.  The pages give no formula.  Reading taken here: one scalar per
  call, s = max(1, ln(Lseq) / ln(4096)) with Lseq the sequence length
  (T in prefill, the kv length L in decode); it multiplies q (hence the
  whole alpha*q.k term) and the relative logits, so the whole logit is s*l.
* the sheared-bias form -- section "Relative Logits Optimization", eq. for
  sheared_bias(i,h,j) = rel_logits(i,h,i-j), which the page states is
  equivalent to looking the bias up per score.
* the softmax over keys, the weighted sum of values, and the natural-log
  log-sum-exp of each row (standard attention; the pages add the bias
  "inside the online softmax", i.e. before normalisation).

Readings where the pages are silent (each listed in the design notes):
* P is one [d_r, E] matrix shared by every head and batch entry; column d
  belongs to distance d ("distance bucket" = exact distance i-j).
* r is per query head, like q.
* GQA maps query head h to kv head h // (Hq / Hkv).
* window W >= 1 keeps keys with 0 <= i-j < W (self included); W = 0 means
  full causal.
* decode: the single query sits at position L-1 of its cache and sees keys
  0..L-1 (its own key included).
* extend (chunked prefill over a cache, the "extend" kernels of the SGLang
  page's AMD path): sequence b holds kv_len[b] tokens in its cache, the last
  n_b of which are the new query rows; new row t sits at position
  kv_len[b] - n_b + t.  s uses Lseq = kv_len[b], one scalar per sequence.
  A paged cache stores key j of sequence b in slot j % page_size of page
  block_table[b][j // page_size].

Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (brute force on tiny inputs, a hand-worked
example under ``tests/golden/``, reductions to library softmax attention,
closed forms and invariants).  The log-scale *form*, the sharing of P and
the GQA head mapping are readings, not facts of the pages: those three are
"parity unpinned" against the pages and pinned only to the stated reading.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import torch

__all__ = [
    "scale_factor",
    "rel_logits",
    "logit_rows",
    "sheared_bias",
    "prefill",
    "decode",
    "extend",
    "cache_rows",
    "brute_force_prefill",
    "attention_weights",
]

_LN_4096 = math.log(4096.0)


def scale_factor(seq_len: int, log_scale: bool) -> float:
    """Length-dependent log-scale s (reading of the "Attention layout" paragraph).

    The pages only say full layers may scale q and the relative logits by a
    factor that depends on the length.  Chosen form: s = max(1, ln L / ln 4096),
    so s = 1 up to 4096 tokens, 1.25 at 32768 and 5/3 at 2**20.
    """
    if not log_scale:
        return 1.0
    if seq_len <= 1:
        return 1.0
    return max(1.0, math.log(seq_len) / _LN_4096)


def rel_logits(r: torch.Tensor, P: torch.Tensor, s: float = 1.0) -> torch.Tensor:
    """rel_logits(t,h,d) = s * r_{t,h} . P[:, d]  (eq. for rel_logits).

    r: [..., d_r];  P: [d_r, E] (column d = distance d).  Returns [..., E] fp64.
    """
    return s * (r.to(torch.float64) @ P.to(torch.float64))


def logit_rows(q_rows: torch.Tensor, r_rows: torch.Tensor, q_pos: torch.Tensor,
               K: torch.Tensor, P: Optional[torch.Tensor], alpha: float,
               rel_extent: int, window: int, s: float) -> torch.Tensor:
    """Full logit rows l(i, j) for the queries at positions ``q_pos`` against all keys.

    q_rows [I, D], r_rows [I, d_r], q_pos [I] (int64), K [Tk, D] (key j at position j).
    Returns [I, Tk] fp64 with -inf on masked entries.  This is the eq. for
    l(i,j,h) with the log-scale s applied to q and to the relative logits,
    then the causal / sliding-window mask.
    """
    q64 = q_rows.to(torch.float64)
    K64 = K.to(torch.float64)
    Tk = K64.shape[0]
    dist = q_pos.to(torch.int64)[:, None] - torch.arange(Tk, dtype=torch.int64)[None, :]  # i - j

    # alpha * (s q_i) . k_j
    lg = (s * alpha) * (q64 @ K64.T)

    # + 1[0 <= i-j < E] * s * rel_logits(i, i-j)
    if rel_extent > 0:
        rl = rel_logits(r_rows, P[:, :rel_extent], s)           # [I, E]
        in_band = (dist >= 0) & (dist < rel_extent)
        idx = torch.where(in_band, dist, torch.zeros_like(dist))
        bias = torch.gather(rl, 1, idx)
        lg = lg + torch.where(in_band, bias, torch.zeros_like(bias))

    # causal mask (j > i) and sliding window (i - j >= W)
    masked = dist < 0
    if window > 0:
        masked = masked | (dist >= window)
    return lg.masked_fill(masked, float("-inf"))


def _softmax_rows(lg: torch.Tensor, V: torch.Tensor):
    """Row softmax of logits, weighted sum of V, and natural-log LSE."""
    m = lg.max(dim=1, keepdim=True).values
    e = torch.exp(lg - m)
    z = e.sum(dim=1, keepdim=True)
    o = (e @ V.to(torch.float64)) / z
    lse = (m + torch.log(z)).squeeze(1)
    return o, lse


def attention_weights(q, k, r, P, alpha: float, rel_extent: int, window: int = 0,
                      log_scale: bool = False) -> torch.Tensor:
    """Softmax weights p[b, h, i, j] (fp64) of a prefill call; for the sum-to-one checks."""
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    s = scale_factor(T, log_scale)
    pos = torch.arange(T, dtype=torch.int64)
    w = torch.empty(B, Hq, T, T, dtype=torch.float64)
    for b in range(B):
        for h in range(Hq):
            lg = logit_rows(q[b, :, h], r[b, :, h] if r is not None else None, pos,
                            k[b, :, h // G], P, alpha, rel_extent, window, s)
            w[b, h] = torch.softmax(lg, dim=1)
    return w


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, r: Optional[torch.Tensor],
            P: Optional[torch.Tensor], alpha: float, rel_extent: int, window: int = 0,
            log_scale: bool = False, rows: Optional[Sequence[int]] = None,
            row_block: int = 1024):
    """Relative-attention prefill, self-attention over positions 0..T-1.

    q [B,T,Hq,D], k/v [B,T,Hkv,D], r [B,T,Hq,d_r], P [d_r, E] (any float dtype;
    upcast exactly to fp64).  ``rows`` selects the query positions to compute
    (default: all).  Returns ``out`` [B, n_rows, Hq, D] and ``lse`` [B, Hq, n_rows],
    both fp64.  Row blocks only bound memory; each row sees every key.
    """
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    s = scale_factor(T, log_scale)
    sel = torch.arange(T, dtype=torch.int64) if rows is None else torch.as_tensor(list(rows), dtype=torch.int64)
    n = sel.numel()
    out = torch.empty(B, n, Hq, D, dtype=torch.float64)
    lse = torch.empty(B, Hq, n, dtype=torch.float64)
    for b in range(B):
        for g in range(Hkv):
            K = k[b, :, g].to(torch.float64)
            V = v[b, :, g].to(torch.float64)
            for h in range(g * G, (g + 1) * G):
                for s0 in range(0, n, row_block):
                    pos = sel[s0:s0 + row_block]
                    lg = logit_rows(q[b, pos, h], r[b, pos, h] if rel_extent > 0 else None, pos,
                                    K, P, alpha, rel_extent, window, s)
                    o, l = _softmax_rows(lg, V)
                    out[b, s0:s0 + pos.numel(), h] = o
                    lse[b, h, s0:s0 + pos.numel()] = l
    return out, lse


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, r: Optional[torch.Tensor],
           P: Optional[torch.Tensor], alpha: float, rel_extent: int, window: int = 0,
           log_scale: bool = False):
    """One query token per sequence against its KV cache.

    q [B,Hq,D], k/v [B,L,Hkv,D], r [B,Hq,d_r], P [d_r,E].  The query sits at
    position L-1 and sees keys 0..L-1 (its own key included); s uses Lseq = L.
    Returns out [B,Hq,D] and lse [B,Hq], fp64.
    """
    B, Hq, D = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    s = scale_factor(L, log_scale)
    pos = torch.tensor([L - 1], dtype=torch.int64)
    out = torch.empty(B, Hq, D, dtype=torch.float64)
    lse = torch.empty(B, Hq, dtype=torch.float64)
    for b in range(B):
        for g in range(Hkv):
            K = k[b, :, g].to(torch.float64)
            V = v[b, :, g].to(torch.float64)
            for h in range(g * G, (g + 1) * G):
                lg = logit_rows(q[b, h][None], r[b, h][None] if rel_extent > 0 else None, pos,
                                K, P, alpha, rel_extent, window, s)
                o, l = _softmax_rows(lg, V)
                out[b, h] = o[0]
                lse[b, h] = l[0]
    return out, lse


def cache_rows(cache: torch.Tensor, b: int, n: int, block_table=None, page_size: int = 0) -> torch.Tensor:
    """Rows 0..n-1 of sequence b of a KV cache, as [n, Hkv, D].

    Contiguous cache [B, Lcap, Hkv, D]: rows cache[b, :n].  Paged cache
    [num_pages, page_size, Hkv, D] with ``block_table`` [B][max_pages]: row j
    is slot j % page_size of page block_table[b][j // page_size].
    """
    if block_table is None:
        return cache[b, :n]
    idx = [(int(block_table[b][j // page_size]), j % page_size) for j in range(n)]
    return torch.stack([cache[pg, sl] for pg, sl in idx]) if n > 0 else cache[0, :0]


def extend(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, r: Optional[torch.Tensor],
           P: Optional[torch.Tensor], alpha: float, rel_extent: int, window: int,
           log_scale: bool, q_start: Sequence[int], kv_len: Sequence[int],
           block_table=None, page_size: int = 0, row_block: int = 1024):
    """New query rows of several sequences against their KV caches.

    q [total_q, Hq, D] and r [total_q, Hq, d_r] are packed: rows
    q_start[b] .. q_start[b+1]-1 belong to sequence b.  k/v is a contiguous
    cache [B, Lcap, Hkv, D] or, with ``block_table``, a paged one (see
    ``cache_rows``).  New row t of sequence b sits at position
    kv_len[b] - n_b + t (n_b its number of new rows) and sees the cached keys
    0..position under the causal / window mask, with the bias of the eq. for
    l(i,j,h); s uses Lseq = kv_len[b].  Returns out [total_q, Hq, D] and
    lse [Hq, total_q], fp64.
    """
    total_q, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    B = len(kv_len)
    out = torch.zeros(total_q, Hq, D, dtype=torch.float64)
    lse = torch.zeros(Hq, total_q, dtype=torch.float64)
    for b in range(B):
        L = int(kv_len[b])
        r0, r1 = int(q_start[b]), int(q_start[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        s = scale_factor(L, log_scale)
        Kb = cache_rows(k, b, L, block_table, page_size)
        Vb = cache_rows(v, b, L, block_table, page_size)
        pos_all = torch.arange(L - n, L, dtype=torch.int64)
        for g in range(Hkv):
            K = Kb[:, g].to(torch.float64)
            V = Vb[:, g].to(torch.float64)
            for h in range(g * G, (g + 1) * G):
                for t0 in range(0, n, row_block):
                    pos = pos_all[t0:t0 + row_block]
                    rows = torch.arange(r0 + t0, r0 + t0 + pos.numel())
                    lg = logit_rows(q[rows, h], r[rows, h] if rel_extent > 0 else None, pos,
                                    K, P, alpha, rel_extent, window, s)
                    o, l = _softmax_rows(lg, V)
                    out[rows, h] = o
                    lse[h, rows] = l
    return out, lse


def sheared_bias(r: torch.Tensor, P: torch.Tensor, T: int, rel_extent: int, s: float = 1.0) -> torch.Tensor:
    """Dense sheared bias [T, H, T] built entry by entry (section "Relative
    Logits Optimization", eq. for sheared_bias(i,h,j) = rel_logits(i,h,i-j)),
    zero where i-j lies outside [0, rel_extent).

    r [T, H, d_r], P [d_r, E].  Only for small T: a separate route to the
    same bias as ``logit_rows`` (used by the equivalence check).
    """
    H = r.shape[1]
    out = torch.zeros(T, H, T, dtype=torch.float64)
    r64 = r.to(torch.float64)
    P64 = P.to(torch.float64)
    for i in range(T):
        for j in range(T):
            d = i - j
            if 0 <= d < rel_extent:
                for h in range(H):
                    out[i, h, j] = s * torch.dot(r64[i, h], P64[:, d])
    return out


def brute_force_prefill(q, k, v, r, P, alpha: float, rel_extent: int, window: int = 0,
                        log_scale: bool = False):
    """Scalar pure-Python evaluation of the definitions, for T <= 16.

    Inputs are nested lists (or tensors converted with .tolist()):
    q[b][i][h][x], k/v[b][j][g][x], r[b][i][h][c], P[c][d].  Uses math.fsum and
    math.exp only.  Returns (out[b][i][h][x], lse[b][h][i]).
    """
    B, T, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    G = Hq // Hkv
    s = scale_factor(T, log_scale)
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(T)] for _ in range(B)]
    lse = [[[0.0] * T for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(T):
                logits = {}
                for j in range(T):
                    d = i - j
                    if d < 0 or (window > 0 and d >= window):
                        continue
                    qk = math.fsum(s * q[b][i][h][x] * k[b][j][g][x] for x in range(D))
                    val = alpha * qk
                    if 0 <= d < rel_extent:
                        rl = math.fsum(r[b][i][h][c] * P[c][d] for c in range(len(P)))
                        val += s * rl
                    logits[j] = val
                m = max(logits.values())
                w = {j: math.exp(val - m) for j, val in logits.items()}
                z = math.fsum(w.values())
                for x in range(D):
                    out[b][i][h][x] = math.fsum(w[j] * v[b][j][g][x] for j in w) / z
                lse[b][h][i] = m + math.log(z)
    return out, lse
