"""GPU checks of the backward's dQ split at small grids ("Add context parallelism", PR 1445,
Description: ranks balanced in work and hence in time). With a workspace of
cp_attention_bwd_split_workspace_bytes, a grid with about one work item per CU computes dQ of
its heavy row blocks in pieces of their key range, and a merge adds the pieces in a fixed order.

Each case runs the same rank twice, split and unsplit:
- dK and dV come from the same kernel either way and must agree bit for bit;
- dQ differs only in how float32 sums are grouped (a piece's tiles, then the pieces), so the two
  agree to 1e-4 * max(1, max |dQ|);
- both are checked against the oracle at the backward tolerance 2e-2 * max(1, max |ref|)."""

import math

import numpy as np
import pytest
import torch

import context_causal_attention_load_amd as cpa
from context_causal_attention_load_amd import synth
from oracle import backward as obw
from oracle import lb_index as olb

from closed_forms import bwd_tol
from gpu_util import DEV, announce, assert_close

pytestmark = pytest.mark.gpu


def both_ways(q, k, v, do, seq, cp, rank, scale):
    """Forward once, then the backward with a split-sized and with a base-sized workspace."""
    c = seq // (2 * cp)
    kp, vp = cpa.permute(k.to(DEV), cp), cpa.permute(v.to(DEV), cp)
    qs = cpa.permute(q.to(DEV), cp, row_begin=rank * 2 * c, row_count=2 * c)
    dos = cpa.permute(do.to(DEV), cp, row_begin=rank * 2 * c, row_count=2 * c)
    o, lse = cpa.attention_fwd(qs, kp, vp, cp, rank, scale=scale)
    B, Sq, Hq, Dqk = qs.shape
    need = cpa.attention_bwd_split_workspace_bytes(B, seq, Hq, kp.shape[2], Dqk, vp.shape[3], torch.bfloat16, cp,
                                                   rank)
    base = cpa.attention_bwd_workspace_bytes(B, Sq, Hq)
    assert need > base, "this case is meant to split"
    split = cpa.attention_bwd(qs, kp, vp, o, lse, dos, cp, rank, scale=scale, split=True)
    unsplit = cpa.attention_bwd(qs, kp, vp, o, lse, dos, cp, rank, scale=scale, split=False)
    torch.cuda.synchronize()
    return split, unsplit


def compare_split_unsplit(split, unsplit, tag):
    (dq_s, dk_s, dv_s), (dq_u, dk_u, dv_u) = split, unsplit
    assert torch.equal(dk_s, dk_u) and torch.equal(dv_s, dv_u), f"dK/dV differ between split and unsplit ({tag})"
    diff = float((dq_s - dq_u).abs().max())
    ref = max(1.0, float(dq_u.abs().max()))
    print(f"  {tag}: max |dQ split - dQ unsplit| = {diff:.3e} (bound {1e-4 * ref:.3e})", flush=True)
    assert diff <= 1e-4 * ref
    assert bool(torch.isfinite(dq_s).all())


@pytest.mark.parametrize("batch,seq,cp,hq,hkv,d,d_v,ranks,tag", [
    (2, 8000, 4, 2, 2, 128, 128, (0, 3), "ragged chunks"),     # c = 1000: a 256-row block spans both chunks
    (1, 8192, 4, 1, 1, 64, 64, (0, 2), "one head, 8 pieces"),  # one unit: heavy blocks cut into 8 pieces
    (1, 4096, 2, 4, 4, 192, 128, (0, 1), "MLA head dims"),     # Dqk 192, Dv 128
])
def test_backward_dq_split_against_oracle(batch, seq, cp, hq, hkv, d, d_v, ranks, tag):
    q, k, v = synth.prefill_inputs(batch, seq, hq, hkv, d, d_v, torch.bfloat16, seq + d)
    do = synth.prefill_grad(batch, seq, hq, d_v, torch.bfloat16, seq + d + 1)
    perm = olb.load_balance_perm(seq, cp)
    scale = 1.0 / math.sqrt(d)
    c = seq // (2 * cp)
    for r in ranks:
        announce(f"backward dQ split, {tag}: B={batch} S={seq} cp={cp} Hq={hq}/{hkv} D={d}/{d_v} rank {r}")
        split, unsplit = both_ways(q, k, v, do, seq, cp, r, scale)
        compare_split_unsplit(split, unsplit, f"{tag} rank {r}")
        rows = perm[r * 2 * c:(r + 1) * 2 * c]
        dq_r, dk_r, dv_r = obw.causal_attention_bwd_ref(q[:, rows], k[:, perm], v[:, perm], do[:, rows], rows, perm,
                                                        scale)
        assert_close(split[0].cpu().numpy(), dq_r, bwd_tol(dq_r), f"dQ split {tag} r{r}")
        assert_close(split[1].cpu().numpy(), dk_r, bwd_tol(dk_r), f"dK {tag} r{r}")
        assert_close(split[2].cpu().numpy(), dv_r, bwd_tol(dv_r), f"dV {tag} r{r}")


def test_backward_dq_split_llama7b_every_rank():
    """The Llama2-7B shape at cp = 4 (256 work items per rank): every rank split and unsplit.
    (The oracle checks the split path at ranks 0 and 3 in the backward parity tests.)"""
    w = synth.LLAMA2_7B_S8K
    q, k, v = synth.prefill_inputs(w.batch, w.seq, w.hq, w.hkv, w.d_qk, w.d_v, torch.bfloat16, w.seed)
    do = synth.prefill_grad(w.batch, w.seq, w.hq, w.d_v, torch.bfloat16, w.seed + 1000)
    for r in range(4):
        announce(f"backward dQ split, {w.name} cp=4 rank {r}")
        split, unsplit = both_ways(q, k, v, do, w.seq, 4, r, 1.0 / math.sqrt(w.d_qk))
        compare_split_unsplit(split, unsplit, f"{w.name} rank {r}")


def test_backward_dq_split_reuses_a_dirty_workspace():
    """A workspace full of NaN from a previous user gives the same gradients: every partial slot
    a merge reads is written first in the same call."""
    seq, cp, hq, d = 8192, 4, 2, 128
    q, k, v = synth.prefill_inputs(1, seq, hq, hq, d, d, torch.bfloat16, 77)
    do = synth.prefill_grad(1, seq, hq, d, torch.bfloat16, 78)
    c = seq // (2 * cp)
    kp, vp = cpa.permute(k.to(DEV), cp), cpa.permute(v.to(DEV), cp)
    qs = cpa.permute(q.to(DEV), cp, row_begin=0, row_count=2 * c)
    dos = cpa.permute(do.to(DEV), cp, row_begin=0, row_count=2 * c)
    announce("backward dQ split with a NaN-filled workspace")
    o, lse = cpa.attention_fwd(qs, kp, vp, cp, 0)
    need = cpa.attention_bwd_split_workspace_bytes(1, seq, hq, hq, d, d, torch.bfloat16, cp, 0)
    assert need > cpa.attention_bwd_workspace_bytes(1, 2 * c, hq), "this case is meant to split"
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=DEV)
    dirty = cpa.attention_bwd(qs, kp, vp, o, lse, dos, cp, 0, workspace=ws)
    clean = cpa.attention_bwd(qs, kp, vp, o, lse, dos, cp, 0)
    torch.cuda.synchronize()
    for a, b, name in zip(dirty, clean, ("dQ", "dK", "dV")):
        assert torch.equal(a, b), name
    assert np.isfinite(dirty[0].cpu().numpy()).all()
