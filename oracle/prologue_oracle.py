"""Plain fp64 CPU oracle for the attention prologue.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path; it
imports nothing from the product path.

The prologue is the step right before the attention kernels (page "SGLang
and Miles Add Day-0 Support for Inkling", section "ShortConv Optimization",
paragraph "KV ShortConv + QK-norm + KV store"): the K and V stream short
convolutions, the Q/K RMS normalisation and the KV-cache write, fused into
one kernel.  What each step computes:

* ShortConv -- section "Short Convolution (ShortConv)", its equation: a
  per-channel causal filter over the token axis with a residual,
  y[t,c] = x[t,c] + sum_{d=0}^{W-1} w[c,d] * x[t-d,c], W = 4 in the current
  configurations.  It sits on the K stream before the Q/K normalisation and
  on the V stream (same section, its list of the four places).
* Q/K normalisation -- named "Q/K RMSNorm" in the paragraph above; RMSNorm
  over a head's D channels: y = x / sqrt(mean(x^2) + eps) * g.
* KV-cache write -- the normalised K and the convolved V of each new token
  go to the cache at the token's position.

Readings where the pages are silent (each listed in the design notes):
* The channels of the K (V) ShortConv are the Hkv*D channels of a token's
  K (V) row; w is [Hkv*D, W], w[c, d] multiplying x[t-d, c].
* RMSNorm weights are one D-vector for q and one for k, shared by all heads;
  eps is a parameter.  r passes through the prologue unchanged.
* Positions before a sequence's first token hold zeros.  A chunk that
  continues a sequence (extend) takes the raw (pre-convolution) K and V rows
  of the three positions before it from a per-sequence state
  [2, 3, Hkv*D] (K then V, oldest row first) and returns the state after
  its last token.  With no state, those rows are zeros.
* Sequence b's n_b new tokens sit at cache positions
  kv_len[b] - n_b .. kv_len[b] - 1, as in extend.
* The section "Customized Efficient Kernels for Train-Inference
  Consistency" says the ShortConv kernels accumulate in fp32 and add the
  residual last; the oracle is exact fp64, so the order does not show here.

Parity status: ``short_conv`` is pinned to torch's conv1d (a library
routine) and to closed forms for identity and shift filters; ``rms_norm`` to
torch's rms_norm and to the unit-RMS invariant; ``prologue`` to the chunking
invariance (a sequence in one call equals the same sequence in two calls
with the state carried) and to the composition of the two pinned parts.
The weight-sharing and state-layout readings above are "parity unpinned"
against the pages and pinned only to the stated reading.
"""

from __future__ import annotations

from typing import Optional, Sequence, Tuple

import torch

__all__ = ["STATE_ROWS", "short_conv", "rms_norm", "prologue", "cache_positions"]

STATE_ROWS = 3  # raw rows kept per stream: the W - 1 = 3 positions before a chunk


def short_conv(x: torch.Tensor, w: torch.Tensor, state: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ShortConv of one sequence's new rows (section "Short Convolution").

    x: [n, C] raw rows in position order; w: [C, W] with 1 <= W <= 4;
    state: [3, C] raw rows of the three positions before x (oldest first),
    or None for zeros.  Returns y [n, C] in float64 with
    y[t] = x[t] + sum_d w[:, d] * x[t - d].
    """
    n, C = x.shape
    W = w.shape[1]
    assert 1 <= W <= STATE_ROWS + 1 and w.shape[0] == C
    prev = torch.zeros(STATE_ROWS, C, dtype=torch.float64) if state is None else state.to(torch.float64)
    xs = torch.cat([prev, x.to(torch.float64)], dim=0)  # xs[3 + t] = x[t]
    wd = w.to(torch.float64)
    acc = torch.zeros(n, C, dtype=torch.float64)
    for d in range(W):
        acc += wd[:, d] * xs[STATE_ROWS - d:STATE_ROWS - d + n]
    return acc + x.to(torch.float64)


def rms_norm(x: torch.Tensor, weight: torch.Tensor, eps: float) -> torch.Tensor:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * weight, in float64."""
    x = x.to(torch.float64)
    ms = (x * x).mean(dim=-1, keepdim=True)
    return x / torch.sqrt(ms + eps) * weight.to(torch.float64)


def cache_positions(q_start: Sequence[int], kv_len: Sequence[int]):
    """Cache position of every packed new row: row q_start[b] + t of sequence
    b sits at kv_len[b] - n_b + t.  Returns a list of (b, position) per row."""
    out = []
    for b in range(len(kv_len)):
        n = q_start[b + 1] - q_start[b]
        for t in range(n):
            out.append((b, kv_len[b] - n + t))
    return out


def prologue(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, conv_k: torch.Tensor, conv_v: torch.Tensor,
             q_norm_w: torch.Tensor, k_norm_w: torch.Tensor, eps: float, q_start: Sequence[int],
             state: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """The prologue of a packed batch of new tokens.

    q [N, Hq, D], k and v [N, Hkv, D] are the raw projections of the new
    tokens, packed by sequence (rows q_start[b] .. q_start[b+1]-1 belong to
    sequence b).  state is [B, 2, 3, Hkv*D] or None.  Returns (q_out, k_new,
    v_new, state_out) in float64: q_out = RMSNorm(q) per head, k_new =
    RMSNorm(ShortConv(k)) per head, v_new = ShortConv(v), and state_out
    [B, 2, 3, Hkv*D] = the raw K and V rows of each sequence's last three
    positions (taken from state where the chunk is shorter than three).
    """
    N, Hq, D = q.shape
    Hkv = k.shape[1]
    B = len(q_start) - 1
    C = Hkv * D
    q_out = rms_norm(q, q_norm_w, eps)
    k_new = torch.empty(N, Hkv, D, dtype=torch.float64)
    v_new = torch.empty(N, Hkv, D, dtype=torch.float64)
    state_out = torch.zeros(B, 2, STATE_ROWS, C, dtype=torch.float64)
    for b in range(B):
        a0, a1 = q_start[b], q_start[b + 1]
        n = a1 - a0
        for s, (x, w, dst) in enumerate(((k, conv_k, k_new), (v, conv_v, v_new))):
            st = None if state is None else state[b, s]
            rows = x[a0:a1].reshape(n, C)
            y = short_conv(rows, w, st)
            if s == 0:
                y = rms_norm(y.reshape(n, Hkv, D), k_norm_w, eps)
            dst[a0:a1] = y.reshape(n, Hkv, D)
            prev = torch.zeros(STATE_ROWS, C, dtype=torch.float64) if st is None else st.to(torch.float64)
            state_out[b, s] = torch.cat([prev, rows.to(torch.float64)], dim=0)[-STATE_ROWS:]
    return q_out, k_new, v_new, state_out
