"""CPU pins of the identical-key closed forms that check every key and row of the full-size GPU
backward: they must accept the fp64 oracle's gradients exactly (up to rounding) and reject
plausible mistakes (a scaled, shifted or zeroed gradient)."""

import math
import types

import numpy as np
import pytest
import torch

from closed_forms import check_identical_keys_bwd, check_identical_keys_dk
from oracle import backward as obw
from oracle import lb_index as olb


def _case(S, cp, hq, hkv, d, seed):
    w = types.SimpleNamespace(seq=S, hq=hq, hkv=hkv, d_qk=d, d_v=d, scale=1.0 / math.sqrt(d))
    g = torch.Generator().manual_seed(seed)
    q, v, do = (torch.randn(1, S, h, d, generator=g, dtype=torch.float64) for h in (hq, hkv, hq))
    k = torch.randn(1, 1, hkv, d, generator=g, dtype=torch.float64).expand(-1, S, -1, -1).contiguous()
    return w, q, k, v, do


def _oracle(w, cp, rank, q, k, v, do):
    perm = olb.load_balance_perm(w.seq, cp)
    c = w.seq // (2 * cp)
    rows = perm[rank * 2 * c:(rank + 1) * 2 * c]
    out = obw.causal_attention_bwd_ref(q[:, rows], k[:, perm], v[:, perm], do[:, rows], rows, perm, w.scale)
    return tuple(torch.as_tensor(np.asarray(x)) for x in out)


@pytest.mark.parametrize("S,cp,hq,hkv,d", [(64, 2, 4, 2, 16), (96, 1, 2, 2, 8), (128, 4, 6, 3, 8)])
def test_closed_forms_match_oracle(S, cp, hq, hkv, d):
    w, q, k, v, do = _case(S, cp, hq, hkv, d, seed=S + cp)
    for rank in range(cp):
        dq, dk, dv = _oracle(w, cp, rank, q, k, v, do)
        assert float(dq.abs().max()) < 1e-12  # dQ is exactly zero with identical keys
        check_identical_keys_bwd(w, cp, rank, do, dq, dv)
        check_identical_keys_dk(w, cp, rank, q, v, do, dk)


@pytest.mark.parametrize("mistake", ["dk-scaled", "dk-next-key", "dv-scaled", "dv-next-key", "dv-zero", "dq-nonzero"])
def test_closed_forms_reject_mistakes(mistake):
    w, q, k, v, do = _case(64, 2, 4, 2, 16, seed=5)
    dq, dk, dv = _oracle(w, 2, 0, q, k, v, do)
    if mistake == "dk-scaled":
        dk = dk * 1.1
    elif mistake == "dk-next-key":
        dk = torch.roll(dk, 1, dims=1)
    elif mistake == "dv-scaled":
        dv = dv * 1.1
    elif mistake == "dv-next-key":
        dv = torch.roll(dv, 1, dims=1)
    elif mistake == "dv-zero":
        dv = torch.zeros_like(dv)
    else:
        dq = dq + 0.05
    with pytest.raises(AssertionError):
        check_identical_keys_bwd(w, 2, 0, do, dq, dv)
        check_identical_keys_dk(w, 2, 0, q, v, do, dk)
