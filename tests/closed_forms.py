"""Closed forms of a rank's attention gradients when all keys of a kv head are equal, used to
check every key and every row at full size (no GPU here: the checks take the gradients as CPU or
GPU tensors). With identical keys each visible key gets probability 1/(pos_i + 1) in row i."""

import numpy as np
import torch

from oracle import lb_index as olb


def bwd_tol(ref):
    """bf16 gradients: |err| <= 2e-2 * max(1, max |ref|) (bf16 P, dS and inputs; fp32 sums)."""
    return 2e-2 * max(1.0, float(np.abs(ref).max()))


def check_identical_keys_bwd(w, cp, rank, do, dq, dv):
    S = w.seq
    c, G = S // (2 * cp), w.hq // w.hkv
    perm = olb.load_balance_perm(S, cp)           # position of gathered key j
    rows = perm[rank * 2 * c:(rank + 1) * 2 * c]  # the rank's row positions, ascending
    assert np.all(np.diff(rows) > 0)
    first = np.searchsorted(rows, perm, side="left")  # first of the rank's rows that sees key j
    seen = first < 2 * c
    do_rows = do[0, torch.from_numpy(rows)]       # [2c, Hq, Dv]
    inv_n = torch.from_numpy(1.0 / (rows + 1.0))[:, None]
    dv = dv[0].cpu()                              # [S, Hkv, Dv], gathered key order
    worst = 0.0
    for g in range(w.hkv):
        contrib = do_rows[:, g * G:(g + 1) * G].double().sum(1) * inv_n      # [2c, Dv]
        suffix = contrib.flip(0).cumsum(0).flip(0)                           # rows i and after
        ref = torch.zeros((S, w.d_v), dtype=torch.float64)
        ref[torch.from_numpy(seen)] = suffix[torch.from_numpy(first[seen])]
        err = float((dv[:, g].double() - ref).abs().max())
        tol = bwd_tol(ref.numpy())
        worst = max(worst, err / tol)
        assert err <= tol, f"dV rank {rank} kv head {g}: max err {err:.3e} > {tol:.3e}"
    dq_max = float(dq.abs().max())
    print(f"  every key's dV within {worst:.3f} of its bound; max |dQ| {dq_max:.3e} (exact 0)", flush=True)
    assert dq_max <= bwd_tol(np.zeros(1))


def check_identical_keys_dk(w, cp, rank, q, v, do, dk):
    """dK with identical keys: dS_ij = (dO_i . v_j - D_i) / n_i for a visible key (n_i = pos_i + 1,
    D_i = dO_i . O_i, O_i the prefix mean of V), so dK_j = scale (M(f_j) v_j - t(f_j)) with f_j the
    first of the rank's rows that sees key j, M(f) the sum over rows i >= f and the group's heads
    of q_i dO_i^T / n_i, and t(f) the same sum of q_i D_i / n_i. M is accumulated from the last row
    down, so every key's value comes from one pass."""
    S = w.seq
    c, G = S // (2 * cp), w.hq // w.hkv
    perm = olb.load_balance_perm(S, cp)
    rows = perm[rank * 2 * c:(rank + 1) * 2 * c]
    first = np.searchsorted(rows, perm, side="left")
    order = np.argsort(first, kind="stable")
    bounds = np.searchsorted(first[order], np.arange(2 * c + 1), side="left")  # keys of row i: order[bounds[i]:bounds[i+1]]
    n = torch.from_numpy(rows + 1.0)
    rows_t = torch.from_numpy(rows)
    dk = dk[0].cpu()                               # [S, Hkv, Dqk], gathered key order
    worst = 0.0
    for g in range(w.hkv):
        hs = slice(g * G, (g + 1) * G)
        qg = q[0, rows_t, hs].double()             # [2c, G, Dqk]
        dog = do[0, rows_t, hs].double()           # [2c, G, Dv]
        vnat = v[0, :, g].double()                 # [S, Dv], natural order
        o_rows = vnat.cumsum(0)[rows_t] / n[:, None]
        dvec = (dog * o_rows[:, None, :]).sum(-1)  # [2c, G]
        t_rows = (qg * (dvec / n[:, None])[..., None]).sum(1)
        t_suf = t_rows.flip(0).cumsum(0).flip(0)   # [2c, Dqk]
        vkeys = vnat[torch.from_numpy(perm)]       # value of gathered key j, [S, Dv]
        ref = torch.zeros((S, w.d_qk), dtype=torch.float64)
        m = torch.zeros((w.d_qk, w.d_v), dtype=torch.float64)
        for i in range(2 * c - 1, -1, -1):
            m += qg[i].T @ dog[i] / n[i]
            lo, hi = bounds[i], bounds[i + 1]
            if hi > lo:
                keys = torch.from_numpy(order[lo:hi])
                ref[keys] = w.scale * (vkeys[keys] @ m.T - t_suf[i])
        err = float((dk[:, g].double() - ref).abs().max())
        tol = bwd_tol(ref.numpy())
        worst = max(worst, err / tol)
        assert err <= tol, f"dK rank {rank} kv head {g}: max err {err:.3e} > {tol:.3e}"
    print(f"  every key's dK within {worst:.3f} of its bound", flush=True)
