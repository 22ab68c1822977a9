"""Load-balanced token order for context parallelism (oracle side, test infrastructure).

"Add context parallelism" (MaxText PR 1445), Description: to give every device a similar
amount of causal work, the tokens are reordered before sharding. With context parallelism 2
and eight tokens, one device keeps tokens 0,1,6,7 and the other keeps 2,3,4,5.

Reading for general cp (the page shows cp=2 only): the sequence of length S is cut into
2*cp equal chunks of c = S / (2*cp) tokens; rank r keeps chunk r followed by chunk
2*cp-1-r. The permuted sequence is the concatenation of the ranks' shards in rank order,
which is what an all-gather of the shards along the context axis returns.

This module builds the order by concatenating Python ranges, the most literal form of the
chunk rule; it shares nothing with the closed-form index used by the HIP kernels.
"""

import numpy as np


def _chunk_len(seq, cp):
    if cp < 1 or seq < 1 or seq % (2 * cp) != 0:
        raise ValueError(f"sequence length {seq} must be a positive multiple of 2*cp = {2 * cp}")
    return seq // (2 * cp)


def load_balance_perm(seq, cp):
    """Return ``perm`` with ``perm[j]`` = original token position of permuted slot ``j``."""
    c = _chunk_len(seq, cp)
    order = []
    for r in range(cp):
        first = r
        second = 2 * cp - 1 - r
        order.extend(range(first * c, (first + 1) * c))
        order.extend(range(second * c, (second + 1) * c))
    return np.array(order, dtype=np.int64)


def inverse_perm(perm):
    """Inverse permutation: ``inv[p]`` = permuted slot that holds original position ``p``."""
    perm = np.asarray(perm)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm), dtype=perm.dtype)
    return inv


def shard_row_range(seq, cp, rank):
    """Rows ``[begin, end)`` of the permuted sequence that rank ``rank`` holds."""
    c = _chunk_len(seq, cp)
    if not 0 <= rank < cp:
        raise ValueError(f"rank {rank} outside [0, {cp})")
    return rank * 2 * c, (rank + 1) * 2 * c


def shard_positions(seq, cp, rank):
    """Original token positions of rank ``rank``'s query rows, in shard-row order."""
    begin, end = shard_row_range(seq, cp, rank)
    return load_balance_perm(seq, cp)[begin:end]


def contiguous_shard_positions(seq, cp, rank):
    """Positions a rank would hold without load balancing: tokens [rank*S/cp, (rank+1)*S/cp)."""
    if seq % cp != 0 or not 0 <= rank < cp:
        raise ValueError("bad contiguous shard")
    n = seq // cp
    return np.arange(rank * n, (rank + 1) * n, dtype=np.int64)


def causal_pair_count(q_positions, k_positions):
    """Number of (query, key) pairs a causal mask leaves visible (key position <= query position)."""
    kp = np.sort(np.asarray(k_positions))
    return int(np.searchsorted(kp, np.asarray(q_positions), side="right").sum())
