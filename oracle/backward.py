"""Reference backward pass of one rank's causal attention in float64 (oracle side, test
infrastructure).

Source: "Add context parallelism" (MaxText PR 1445), Description: context parallelism exists
to train long sequences, so every rank also runs the backward pass of its shard's attention
(queries of its shard against the all-gathered keys and values, under the same reordered
causal mask). The pages give no formulas; the gradients here are those of the forward pass in
``attention.py`` by the chain rule, written out:

* forward, per (b, query head h, row i) over its visible keys j:
  ``s_ij = scale * q_i . k_j``, ``P_ij = exp(s_ij - LSE_i)``, ``O_i = sum_j P_ij v_j``;
* for an upstream gradient dO of O (the loss is ``sum dO * O``):
  ``dV_j = sum_i P_ij dO_i``; ``dP_ij = dO_i . v_j``; ``D_i = sum_j P_ij dP_ij = dO_i . O_i``;
  ``dS_ij = P_ij (dP_ij - D_i)``; ``dQ_i = scale * sum_j dS_ij k_j``;
  ``dK_j = scale * sum_i dS_ij q_i``;
* grouped-query heads: dK and dV of a kv head are the sums over the query heads that read it.

A rank's dK and dV cover the full (gathered) key set but only its own queries' contributions;
summing them over ranks (a reduce-scatter, on several GPUs) gives the full gradients.

All arithmetic is float64 torch CPU ops, one (batch, query head) and one block of query rows
at a time; the block loop only bounds memory, every sum is the plain one above.
"""

import numpy as np
import torch

from .attention import _t64


def causal_attention_bwd_ref(q, k, v, do, q_pos, k_pos, scale, row_block=512):
    """Gradients of causal grouped-query attention.

    q: [B, Sq, Hq, Dqk]; k: [B, Sk, Hkv, Dqk]; v: [B, Sk, Hkv, Dv]; do: [B, Sq, Hq, Dv] (any float
    dtype, numpy or CPU torch). q_pos [Sq], k_pos [Sk]: original positions; key j is visible to
    row i iff ``k_pos[j] <= q_pos[i]``. Every row must see at least one key.

    Returns (dQ [B, Sq, Hq, Dqk], dK [B, Sk, Hkv, Dqk], dV [B, Sk, Hkv, Dv]) float64 numpy.
    """
    q64, k64, v64, do64 = _t64(q), _t64(k), _t64(v), _t64(do)
    B, Sq, Hq, _ = q64.shape
    Sk, Hkv = k64.shape[1], k64.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    q_pos = torch.as_tensor(np.asarray(q_pos, dtype=np.int64))
    k_pos = torch.as_tensor(np.asarray(k_pos, dtype=np.int64))
    dq = torch.zeros_like(q64)
    dk = torch.zeros_like(k64)
    dv = torch.zeros_like(v64)
    for b in range(B):
        for g in range(Hkv):
            kg, vg = k64[b, :, g, :], v64[b, :, g, :]
            for start in range(0, Sq, row_block):
                rows = slice(start, min(Sq, start + row_block))
                visible = k_pos[None, :] <= q_pos[rows][:, None]
                if not bool(visible.any(dim=1).all()):
                    raise ValueError("every query row must see at least one key")
                for h in range(g * G, (g + 1) * G):
                    qi, doi = q64[b, rows, h, :], do64[b, rows, h, :]
                    s = torch.where(visible, scale * (qi @ kg.T), float("-inf"))
                    lse = torch.logsumexp(s, dim=1)
                    p = torch.exp(s - lse[:, None])          # 0 where masked
                    o = p @ vg
                    dp = doi @ vg.T
                    d = (doi * o).sum(dim=1)
                    ds = p * (dp - d[:, None])
                    dq[b, rows, h, :] = scale * (ds @ kg)
                    dk[b, :, g, :] += scale * (ds.T @ qi)
                    dv[b, :, g, :] += p.T @ doi
    return dq.numpy(), dk.numpy(), dv.numpy()


def cp_attention_bwd_ref(q_shard, k_perm, v_perm, do_shard, q_positions, seq, cp, scale):
    """One rank's backward over the full K/V held in load-balanced (gathered) order: dQ of its
    shard rows, and its contribution to dK, dV of every gathered key (in that order)."""
    from .lb_index import load_balance_perm

    if k_perm.shape[1] != seq:
        raise ValueError("k_perm must hold the full sequence")
    return causal_attention_bwd_ref(q_shard, k_perm, v_perm, do_shard, q_positions, load_balance_perm(seq, cp),
                                    scale)
