"""Reference attention in float64 (oracle side, test infrastructure).

Definitions followed:

* Causal self-attention over a context-parallel shard. "Add context parallelism"
  (MaxText PR 1445), Description: each device keeps its shard of query rows and attends over
  the all-gathered keys and values; the attention mask is reordered together with the
  tokens, so a key is visible to a query exactly when the key's original position is not
  after the query's original position (a token sees itself).
* Grouped-query attention: query head ``h`` reads key/value head ``h // G`` with
  ``G = Hq / Hkv`` ("Add Pallas GPU decode attention in Maxtext inference", PR 1066,
  Description: the decode path calls a grouped-query kernel; contiguous groups are the
  reading taken here).
* The result is materialised dot-product attention, the un-sharded comparison the unit
  test of "Add support for EP to context parallelism in self-attention" (PR 2023) uses:
  ``s = scale * q . k`` over visible keys, ``m = max s``, ``l = sum exp(s - m)``,
  ``O = sum exp(s - m) v / l`` and the row log-sum-exp ``LSE = m + ln l`` (natural log of
  the scaled logits). No online rescaling, no tiling.
* Decode: one query per sequence, the newest token, attends to cache entries
  ``0 .. len-1`` of its sequence (PR 1066, Tests: the cache is filled by a prefill and then
  grows to the target length).

All arithmetic is float64; inputs are upcast exactly (bf16 and fp32 values are exact in
float64).
"""

import numpy as np
import torch

from .lb_index import load_balance_perm


def _f64(x):
    """Exact upcast of a numpy array or a CPU torch tensor (any float dtype) to float64 numpy."""
    if hasattr(x, "detach"):  # torch tensor
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _t64(x):
    """Exact upcast to a float64 CPU torch tensor (shares memory with float64 numpy input)."""
    if hasattr(x, "detach"):
        return x.detach().to(device="cpu", dtype=torch.float64)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))


def causal_attention_ref(q, k, v, q_pos, k_pos, scale, rows=None, row_block=256):
    """Masked two-pass softmax attention with grouped-query heads.

    q: [B, Sq, Hq, Dqk]; k: [B, Sk, Hkv, Dqk]; v: [B, Sk, Hkv, Dv] (any float dtype, numpy or
    CPU torch). q_pos: [Sq] original positions of the query rows; k_pos: [Sk] original
    positions of the key rows. A key j is visible to row i iff ``k_pos[j] <= q_pos[i]``.
    rows: optional iterable of query-row indices; only those rows are computed (the rest of
    the returned arrays are NaN).

    The arithmetic is float64 torch CPU ops (matmul, exp, max, sum), one (batch, query head)
    at a time. Returns (O [B, Sq, Hq, Dv] float64, LSE [B, Hq, Sq] float64) as numpy arrays.
    """
    q64, k64, v64 = _t64(q), _t64(k), _t64(v)
    B, Sq, Hq, _ = q64.shape
    Sk, Hkv, Dv = k64.shape[1], k64.shape[2], v64.shape[3]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    q_pos = torch.as_tensor(np.asarray(q_pos, dtype=np.int64))
    k_pos = torch.as_tensor(np.asarray(k_pos, dtype=np.int64))
    row_ids = torch.arange(Sq) if rows is None else torch.as_tensor(np.unique(np.asarray(rows, dtype=np.int64)))

    out = torch.full((B, Sq, Hq, Dv), float("nan"), dtype=torch.float64)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float64)
    for b in range(B):
        for g in range(Hkv):
            kg = k64[b, :, g, :]
            vg = v64[b, :, g, :]
            for start in range(0, len(row_ids), row_block):
                blk = row_ids[start:start + row_block]
                qp = q_pos[blk]
                # keys that can be visible to any row of the block (a selection, not a reorder)
                cand = torch.nonzero(k_pos <= qp.max()).flatten()
                visible = k_pos[cand][None, :] <= qp[:, None]
                kc, vc = kg[cand], vg[cand]
                for h in range(g * G, (g + 1) * G):
                    s = scale * (q64[b, blk, h, :] @ kc.T)
                    s = torch.where(visible, s, float("-inf"))
                    m = s.max(dim=1).values
                    p = torch.exp(s - m[:, None])
                    l = p.sum(dim=1)
                    out[b, blk, h, :] = (p @ vc) / l[:, None]
                    lse[b, h, blk] = m + torch.log(l)
    return out.numpy(), lse.numpy()


def cp_attention_ref(q_shard, k_perm, v_perm, q_positions, seq, cp, scale, rows=None):
    """One rank's causal attention over the full K/V held in load-balanced (gathered) order.

    The key at permuted slot j has original position ``load_balance_perm(seq, cp)[j]``.
    """
    k_pos = load_balance_perm(seq, cp)
    if _f64_len(k_perm) != seq:
        raise ValueError("k_perm must hold the full sequence")
    return causal_attention_ref(q_shard, k_perm, v_perm, q_positions, k_pos, scale, rows=rows)


def _f64_len(x):
    return x.shape[1]


def decode_ref(q, k_cache, v_cache, lengths, scale):
    """Single-token grouped-query decode attention.

    q: [B, Hq, D]; k_cache, v_cache: [B, Hkv, Lmax, D] (cache laid out head-major, each
    (b, kv head) slab contiguous); lengths: [B] valid entries per sequence.
    Entries at index >= lengths[b] are never read, so they may hold anything (NaN included).
    A length of 0 (an empty slice of a cache split along its length) has no key: its
    log-sum-exp is ln 0 = -inf and its output is taken as 0 (a merge gives it weight 0).
    Returns (O [B, Hq, Dv] float64, LSE [B, Hq] float64).
    """
    q64 = _f64(q)
    B, Hq, _ = q64.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    lengths = [int(x) for x in np.asarray(lengths).reshape(-1)]
    Dv = v_cache.shape[3]
    out = np.empty((B, Hq, Dv))
    lse = np.empty((B, Hq))
    for b in range(B):
        n = lengths[b]
        if n < 0:
            raise ValueError("lengths must be >= 0")
        if n == 0:
            out[b] = 0.0
            lse[b] = -np.inf
            continue
        for g in range(Hkv):
            kk = _f64(k_cache[b, g, :n])
            vv = _f64(v_cache[b, g, :n])
            for h in range(g * G, (g + 1) * G):
                s = scale * (kk @ q64[b, h])
                m = s.max()
                p = np.exp(s - m)
                l = p.sum()
                out[b, h] = (p @ vv) / l
                lse[b, h] = m + np.log(l)
    return out, lse


def decode_merge_ref(o_parts, lse_parts):
    """Combine decode results over disjoint slices of the keys ("rename context to
    context_autoregressive", PR 1453: inference context parallelism shards the cache along its
    length). With parts r: M = max_r lse_r, w_r = exp(lse_r - M),
    O = sum_r w_r o_r / sum_r w_r, LSE = M + ln sum_r w_r. Parts with lse = -inf carry no keys and
    are left out; if all are, O = 0 and LSE = -inf.

    o_parts: [R, B, Hq, Dv]; lse_parts: [R, B, Hq]. Returns (O [B, Hq, Dv], LSE [B, Hq]) float64.
    """
    o = _f64(o_parts)
    l = _f64(lse_parts)
    R, B, Hq, Dv = o.shape
    out = np.zeros((B, Hq, Dv))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            live = [r for r in range(R) if l[r, b, h] != -np.inf]
            if not live:
                continue
            m = max(l[r, b, h] for r in live)
            w = {r: np.exp(l[r, b, h] - m) for r in live}
            tot = sum(w.values())
            out[b, h] = sum(w[r] * o[r, b, h] for r in live) / tot
            lse[b, h] = m + np.log(tot)
    return out, lse


def permute_ref(x, seq, cp, row_begin=0, row_count=None):
    """Rows ``[row_begin, row_begin+row_count)`` of ``x`` (natural order, [B, S, ...]) taken in
    load-balanced order: ``y[:, i] = x[:, perm[row_begin + i]]`` (a gather, like ``jnp.take``)."""
    perm = load_balance_perm(seq, cp)
    if row_count is None:
        row_count = seq - row_begin
    idx = perm[row_begin:row_begin + row_count]
    return x[:, idx]


def unpermute_ref(x_window, dst, seq, cp, row_begin=0):
    """Write load-balanced rows back to natural order: ``dst[:, perm[row_begin + i]] = x_window[:, i]``.

    Returns a new array/tensor (``dst`` is not modified)."""
    perm = load_balance_perm(seq, cp)
    n = x_window.shape[1]
    out = dst.clone() if hasattr(dst, "clone") else dst.copy()
    out[:, perm[row_begin:row_begin + n]] = x_window
    return out
