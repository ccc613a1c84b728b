"""Plain fp64 CPU oracle for the backward pass of relative attention.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path; it
imports nothing from the product path.

Page "SGLang and Miles Add Day-0 Support for Inkling", section "Customized
Efficient Kernels for Train-Inference Consistency", paragraph "Relative
attention": the training side differentiates the attention through the
scores and through r, with the relative projection P frozen, at the same
logit definition as serving (rel_logits(i,h,d) = r_{i,h} . P[:, d];
l(i,j,h) = alpha q_{i,h} . k_{j,h} + b(i,j,h)).  The pages give no formulas
for the gradients; these are the chain rule applied to that definition (with
the log-scale s of the forward oracle, so the logit is s * l):

  p_ij   = softmax_j(s l_ij)                     (masked entries 0)
  dp_ij  = dout_i . v_j
  delta_i = sum_j p_ij dp_ij                     (= dout_i . out_i)
  ds_ij  = p_ij (dp_ij - delta_i)                (gradient w.r.t. s l_ij)
  dq_i   = s alpha sum_j ds_ij k_j
  dk_j   = s alpha sum_{i, heads of k's group} ds_ij q_i
  dv_j   = sum_{i, heads of v's group} p_ij dout_i
  dr_i   = s sum_{0 <= d < E, i-d visible} ds_{i,i-d} P[:, d]

for the scalar loss sum(dout * out).  Everything is float64 with the full
logit rows materialised (``logit_rows`` of the forward oracle); ``delta`` is
taken from the probabilities, not from a stored output.

Parity status: pinned by ``tests/test_backward_pins.py`` -- central finite
differences of the (separately pinned) forward oracle on tiny inputs,
torch.autograd through the forward oracle's logits and a library softmax,
closed forms (window 1, a single token), invariants (sum over keys of dv and
dk, shift invariance of the bias) and the log-scale identity.  The readings
of the forward oracle (log-scale form, one shared P, the GQA mapping) carry
over unchanged.
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from .relattn_oracle import logit_rows, scale_factor

__all__ = ["prefill_backward"]


def prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, r: Optional[torch.Tensor],
                     P: Optional[torch.Tensor], dout: torch.Tensor, alpha: float, rel_extent: int,
                     window: int = 0, log_scale: bool = False, rows: Optional[Sequence[int]] = None,
                     key_rows: Optional[Sequence[int]] = None, row_block: int = 512):
    """Gradients of sum(dout * out) of a prefill call, P held fixed.

    q [B,T,Hq,D], k/v [B,T,Hkv,D], r [B,T,Hq,d_r], P [d_r,E], dout [B,T,Hq,D].
    ``rows`` selects the query positions whose dq, dr are returned and
    ``key_rows`` the key positions whose dk, dv are returned (default: all).
    Returns (dq [B,nr,Hq,D], dk [B,nk,Hkv,D], dv [B,nk,Hkv,D], dr [B,nr,Hq,d_r]
    or None when rel_extent == 0), all float64.
    """
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    E = rel_extent
    s = scale_factor(T, log_scale)
    qsel = torch.arange(T) if rows is None else torch.as_tensor(list(rows), dtype=torch.int64)
    ksel = torch.arange(T) if key_rows is None else torch.as_tensor(list(key_rows), dtype=torch.int64)

    # query positions whose rows touch a requested key (j <= i, and i - j < W)
    sees = torch.zeros(T, dtype=torch.bool)
    for j in ksel.tolist():
        sees[j:(T if window <= 0 else min(T, j + window))] = True
    sees[qsel] = True
    qpos = torch.nonzero(sees).flatten()
    q_slot = torch.full((T,), -1, dtype=torch.int64)  # position -> index in rows
    q_slot[qsel] = torch.arange(qsel.numel())

    d_r = r.shape[-1] if r is not None else 0
    dq = torch.zeros(B, qsel.numel(), Hq, D, dtype=torch.float64)
    dr = torch.zeros(B, qsel.numel(), Hq, d_r, dtype=torch.float64) if E > 0 else None
    dk = torch.zeros(B, ksel.numel(), Hkv, D, dtype=torch.float64)
    dv = torch.zeros(B, ksel.numel(), Hkv, D, dtype=torch.float64)
    P64 = P.to(torch.float64)[:, :E] if E > 0 else None

    for b in range(B):
        for g in range(Hkv):
            K = k[b, :, g].to(torch.float64)
            V = v[b, :, g].to(torch.float64)
            for h in range(g * G, (g + 1) * G):
                for s0 in range(0, qpos.numel(), row_block):
                    pos = qpos[s0:s0 + row_block]
                    lg = logit_rows(q[b, pos, h], r[b, pos, h] if E > 0 else None, pos, K, P, alpha, E, window, s)
                    p = torch.softmax(lg, dim=1)                         # [I, T]
                    dO = dout[b, pos, h].to(torch.float64)               # [I, D]
                    dp = dO @ V.T                                        # [I, T]
                    delta = (p * dp).sum(dim=1, keepdim=True)
                    ds = p * (dp - delta)                                # gradient w.r.t. s*l
                    Q = q[b, pos, h].to(torch.float64)
                    # key-side gradients, summed over the heads of kv head g
                    dk[b, :, g] += (s * alpha) * (ds[:, ksel].T @ Q)
                    dv[b, :, g] += p[:, ksel].T @ dO
                    # query-side gradients of the requested rows
                    slot = q_slot[pos]
                    keep = slot >= 0
                    if keep.any():
                        dq[b, slot[keep], h] = (s * alpha) * (ds[keep] @ K)
                        if E > 0:
                            # G[i, d] = ds[i, i - d] for 0 <= d < E (zero where i - d < 0)
                            dist = pos[keep][:, None] - torch.arange(E)[None, :]
                            ok = dist >= 0
                            Gm = torch.gather(ds[keep], 1, torch.where(ok, dist, torch.zeros_like(dist)))
                            Gm = torch.where(ok, Gm, torch.zeros_like(Gm))
                            dr[b, slot[keep], h] = s * (Gm @ P64.T)
    return dq, dk, dv, dr
