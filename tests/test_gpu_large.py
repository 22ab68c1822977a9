"""GPU parity at sizes where element offsets pass 2^31 (the largest tensors the boundary accepts
are bounded at 2^40 bytes): the forward, the backward and both decodes index such tensors with
64-bit offsets, and these tests run them there.

Inputs are drawn on the device from a seeded torch generator (they are far too large for the
host generators used elsewhere); K and V are taken as already being in the load-balanced
gathered order, which is all the kernels and the oracle's gathered-order entry points need.
The oracle then checks sampled rows of the first and the last batch element from host copies
of exactly those elements, at the tolerances of the other tests (bf16: 2e-2; backward:
2e-2 * max(1, max |ref|))."""

import math

import numpy as np
import pytest
import torch

import context_causal_attention_load_amd as cpa
from oracle import attention as oatt
from oracle import backward as obw
from oracle import lb_index as olb
from oracle import quant as oq

from closed_forms import bwd_tol
from gpu_util import DEV, announce, assert_close, stratified_rows

pytestmark = pytest.mark.gpu

# Llama3.1-70B-shaped rank: one batch element's query shard (16384 x 64 x 128) and K or V
# (131072 x 8 x 128) each hold 2^27 elements, so batch element 16 starts at element 2^31.
BIG_B, S, CP, HQ, HKV, D = 17, 131072, 8, 64, 8, 128


def dev_randn(shape, gen):
    """bf16 N(0,1) on the device, drawn one leading index at a time (bounded fp32 transients)."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    for i in range(shape[0]):
        out[i] = torch.randn(shape[1:], generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    return out


def big_prefill(seed):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    c = S // (2 * CP)
    q = dev_randn((BIG_B, 2 * c, HQ, D), gen)
    k = dev_randn((BIG_B, S, HKV, D), gen)
    v = dev_randn((BIG_B, S, HKV, D), gen)
    assert (BIG_B - 1) * q[0].numel() >= 2 ** 31 and (BIG_B - 1) * k[0].numel() >= 2 ** 31
    return q, k, v


def test_attention_past_2g_elements():
    """Rank 5's forward over 17 batch elements of the 131072-token shape (the last element's
    query, K and V elements start at offset 2^31): outputs finite everywhere, and stratified
    rows of elements 16 and 0 against the oracle."""
    rank, c = 5, S // (2 * CP)
    announce(f"forward past 2^31 elements: batch {BIG_B}, S={S}, cp={CP}, rank {rank}: drawing inputs")
    q, k, v = big_prefill(seed=1705)
    scale = 1.0 / math.sqrt(D)
    announce("forward past 2^31 elements: attention")
    o, lse = cpa.attention_fwd(q, k, v, CP, rank, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    pos = olb.shard_positions(S, CP, rank)
    rows = stratified_rows(c, 1, seed=rank)
    for b in (BIG_B - 1, 0):
        announce(f"forward past 2^31 elements: oracle on {len(rows)} rows of batch element {b}")
        O_ref, L_ref = oatt.cp_attention_ref(q[b:b + 1, rows].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu(), pos[rows],
                                             S, CP, scale)
        assert_close(o[b:b + 1, rows].float().cpu().numpy(), O_ref, 2e-2, f"O batch element {b}")
        assert_close(lse[b:b + 1, :, rows].cpu().numpy(), L_ref, 2e-2, f"LSE batch element {b}")


def test_backward_past_2g_elements():
    """Rank 2's backward over the same 17 batch elements: dQ on sampled rows of element 16, and
    dK, dV of the keys at the rank's last 48 positions (seen only by the rank's last 48 rows,
    all in the sample), against the oracle; keys past the rank's last position get exactly 0."""
    rank, c = 2, S // (2 * CP)
    announce(f"backward past 2^31 elements: batch {BIG_B}, S={S}, cp={CP}, rank {rank}: drawing inputs")
    q, k, v = big_prefill(seed=1706)
    do = dev_randn(tuple(q.shape), torch.Generator(device=DEV).manual_seed(1707))
    scale = 1.0 / math.sqrt(D)
    announce("backward past 2^31 elements: forward and backward")
    o, lse = cpa.attention_fwd(q, k, v, CP, rank, scale=scale)
    dq, dk, dv = cpa.attention_bwd(q, k, v, o, lse, do, CP, rank, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dq).all()) and bool(torch.isfinite(dk).all()) and bool(torch.isfinite(dv).all())
    b = BIG_B - 1
    perm = olb.load_balance_perm(S, CP)
    shard = perm[rank * 2 * c:(rank + 1) * 2 * c]
    top = (2 * CP - rank) * c  # one past the rank's last position
    rng = np.random.default_rng(rank)
    sel = np.unique(np.concatenate([np.arange(2 * c - 48, 2 * c), rng.integers(0, 2 * c, 8)]))
    announce(f"backward past 2^31 elements: oracle on {len(sel)} rows of batch element {b}")
    dq_r, dk_r, dv_r = obw.causal_attention_bwd_ref(q[b:b + 1, sel].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu(),
                                                    do[b:b + 1, sel].cpu(), shard[sel], perm, scale)
    assert_close(dq[b:b + 1, sel].cpu().numpy(), dq_r, bwd_tol(dq_r), f"dQ batch element {b} sampled rows")
    keys = olb.inverse_perm(perm)[top - 48:top]
    assert_close(dk[b:b + 1, keys].cpu().numpy(), dk_r[:, keys], bwd_tol(dk_r[:, keys]), f"dK batch element {b} last keys")
    assert_close(dv[b:b + 1, keys].cpu().numpy(), dv_r[:, keys], bwd_tol(dv_r[:, keys]), f"dV batch element {b} last keys")
    later = olb.inverse_perm(perm)[top:S:997]
    assert float(dk[b, later].abs().max()) == 0.0 and float(dv[b, later].abs().max()) == 0.0


def test_decode_past_2g_elements():
    """bf16 decode over 160 sequences x 8 kv heads x 16384 cached keys (2.7e9 elements per
    cache), then the int8 quantizer and the int8 decode over the same cache: sampled sequences
    (the last, holding the full length, the first, and one of length 1) against the oracle; the
    last sequence's codes and scales bit for bit."""
    B, hq, hkv, d, L = 160, 48, 8, 128, 16384
    announce(f"decode past 2^31 elements: B={B}, Hq={hq}, Hkv={hkv}, D={d}, Lmax={L}: drawing inputs")
    gen = torch.Generator(device=DEV).manual_seed(160)
    kc = dev_randn((B, hkv, L, d), gen)
    vc = dev_randn((B, hkv, L, d), gen)
    assert (B - 1) * kc[0].numel() >= 2 ** 31
    q = torch.randn((B, hq, d), generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    cgen = torch.Generator("cpu").manual_seed(161)
    lengths = torch.randint(1, L + 1, (B,), generator=cgen, dtype=torch.int64).to(torch.int32)
    lengths[B - 1] = L
    lengths[B // 2] = 1
    scale = 1.0 / math.sqrt(d)
    announce("decode past 2^31 elements: bf16 decode")
    o, lse = cpa.decode(q, kc, vc, lengths.to(DEV), scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    seqs = (B - 1, 0, B // 2)
    for b in seqs:
        O_ref, L_ref = oatt.decode_ref(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(),
                                       lengths[b:b + 1].numpy(), scale)
        assert_close(o[b:b + 1].float().cpu().numpy(), O_ref, 2e-2, f"decode O sequence {b} (length {int(lengths[b])})")
        assert_close(lse[b:b + 1].cpu().numpy(), L_ref, 2e-2, f"decode LSE sequence {b}")

    announce("decode past 2^31 elements: int8 quantizer and int8 decode")
    kq, ks = cpa.quantize_kv(kc)
    vq, vs = cpa.quantize_kv(vc)
    torch.cuda.synchronize()
    kq_r, ks_r = oq.kv_quantize_ref(kc[B - 1:B].cpu())
    got_c, got_s = kq[B - 1:B].cpu().numpy(), ks[B - 1:B].cpu().numpy()
    print(f"  K codes of sequence {B - 1}: {int((got_c != kq_r).sum())} mismatches", flush=True)
    assert np.array_equal(got_c, kq_r)
    assert np.array_equal(got_s.view(np.uint32), ks_r.view(np.uint32))
    del kc, vc
    o8, lse8 = cpa.decode_int8(q, kq, ks, vq, vs, lengths.to(DEV), scale=scale)
    torch.cuda.synchronize()
    for b in seqs:
        O_ref, L_ref = oq.decode_int8_ref(q[b:b + 1].cpu(), kq[b:b + 1].cpu(), ks[b:b + 1].cpu(), vq[b:b + 1].cpu(),
                                          vs[b:b + 1].cpu(), lengths[b:b + 1].numpy(), scale)
        assert_close(o8[b:b + 1].float().cpu().numpy(), O_ref, 2e-2, f"int8 decode O sequence {b}")
        assert_close(lse8[b:b + 1].cpu().numpy(), L_ref, 2e-2, f"int8 decode LSE sequence {b}")
