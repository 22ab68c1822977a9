"""Pins for the CPU oracle: worked example, brute force, library routines, closed forms.

Every check here is independent of the oracle's own code path, so that a plausible mistake
in the oracle (wrong chunk order, strict mask, dropped scale, wrong head group, transposed
operand) fails at least one of them; ``test_planted_mistakes_are_caught`` plants such
mistakes and confirms it.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle import lb_index as olb
from oracle import quant as oq
from oracle import backward as obw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- helpers

def _rand(shape, seed, dtype=np.float64):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape).astype(dtype)


def _brute_force(q, k, v, q_pos, k_pos, scale):
    """Pure-Python loops with math.fsum: the definition written element by element."""
    B, Sq, Hq, Dqk = q.shape
    Sk, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    O = np.zeros((B, Sq, Hq, Dv))
    L = np.zeros((B, Hq, Sq))
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                g = h // G
                s = {}
                for j in range(Sk):
                    if k_pos[j] <= q_pos[i]:
                        s[j] = scale * math.fsum(float(q[b, i, h, d]) * float(k[b, j, g, d]) for d in range(Dqk))
                m = max(s.values())
                w = {j: math.exp(x - m) for j, x in s.items()}
                l = math.fsum(w.values())
                for d in range(Dv):
                    O[b, i, h, d] = math.fsum(w[j] * float(v[b, j, g, d]) for j in w) / l
                L[b, h, i] = m + math.log(l)
    return O, L


def _check_golden(perm_fn):
    with open(os.path.join(GOLDEN, "lb_perm_s8_cp2.txt")) as f:
        lines = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    assert lines
    for ln in lines:
        parts = [p.split() for p in ln.split("|")]
        seq, cp = int(parts[0][0]), int(parts[0][1])
        shards = [[int(x) for x in p] for p in parts[1:]]
        perm = list(perm_fn(seq, cp))
        n = seq // cp
        got = [perm[r * n:(r + 1) * n] for r in range(cp)]
        assert got == shards, (got, shards)


def _check_balance(perm_fn, seq, cp):
    perm = np.asarray(perm_fn(seq, cp))
    assert sorted(perm.tolist()) == list(range(seq))
    n = seq // cp
    counts = [olb.causal_pair_count(perm[r * n:(r + 1) * n], perm) for r in range(cp)]
    # closed form: every rank holds chunk r and chunk 2cp-1-r, c*(S+1) visible pairs
    assert counts == [seq * (seq + 1) // (2 * cp)] * cp, counts


def _check_brute(att_fn, seq, cp, hq, hkv, dqk, dv, seed):
    q = _rand((1, seq, hq, dqk), seed)
    k = _rand((1, seq, hkv, dqk), seed + 1)
    v = _rand((1, seq, hkv, dv), seed + 2)
    scale = 1.0 / math.sqrt(dqk)
    perm = olb.load_balance_perm(seq, cp)
    qp, kp, vp = q[:, perm], k[:, perm], v[:, perm]
    for r in range(cp):
        b0, b1 = olb.shard_row_range(seq, cp, r)
        pos = perm[b0:b1]
        O, L = att_fn(qp[:, b0:b1], kp, vp, pos, perm, scale)
        Ob, Lb = _brute_force(qp[:, b0:b1], kp, vp, pos, perm, scale)
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


def _sdpa_full(q, k, v, scale):
    """torch's CPU fp64 scaled_dot_product_attention (causal) plus torch.logsumexp: library pins."""
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)  # B H S D
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    G = tq.shape[1] // tk.shape[1]
    tk = tk.repeat_interleave(G, dim=1)
    tv = tv.repeat_interleave(G, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale
    S = s.shape[-1]
    causal = torch.ones(S, S, dtype=torch.bool).tril()
    lse = torch.logsumexp(s.masked_fill(~causal, float("-inf")), dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy()


def _check_library(att_fn, seq, cp, hq, hkv, dqk, dv, seed, batch=1):
    q = _rand((batch, seq, hq, dqk), seed)
    k = _rand((batch, seq, hkv, dqk), seed + 1)
    v = _rand((batch, seq, hkv, dv), seed + 2)
    scale = 1.0 / math.sqrt(dqk)
    perm = olb.load_balance_perm(seq, cp)
    inv = olb.inverse_perm(perm)
    qp, kp, vp = q[:, perm], k[:, perm], v[:, perm]
    Os, Ls = [], []
    for r in range(cp):
        b0, b1 = olb.shard_row_range(seq, cp, r)
        O, L = att_fn(qp[:, b0:b1], kp, vp, perm[b0:b1], perm, scale)
        Os.append(O)
        Ls.append(L)
    O_perm = np.concatenate(Os, axis=1)
    L_perm = np.concatenate(Ls, axis=2)
    O_nat = O_perm[:, inv]
    L_nat = L_perm[:, :, inv]
    O_ref, L_ref = _sdpa_full(q, k, v, scale)
    np.testing.assert_allclose(O_nat, O_ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(L_nat, L_ref, rtol=0, atol=1e-10)


def _oracle_att(q, k, v, q_pos, k_pos, scale):
    return oatt.causal_attention_ref(q, k, v, q_pos, k_pos, scale)


# ----------------------------------------------------------------------------- index pins

def test_golden_worked_example():
    _check_golden(olb.load_balance_perm)


@pytest.mark.parametrize("seq,cp", [(8, 1), (8, 2), (8, 4), (512, 2), (8192, 4), (131072, 8), (32768, 4), (96, 3)])
def test_balance_closed_form(seq, cp):
    _check_balance(olb.load_balance_perm, seq, cp)


def test_contiguous_sharding_is_unbalanced():
    # max/mean visible-pair ratio of contiguous shards: 1.5 (S=512,cp=2), 1.875 (S=131072,cp=8)
    for seq, cp, ratio in [(512, 2, 1.5), (8192, 4, 1.75), (131072, 8, 1.875), (32768, 4, 1.75)]:
        allpos = np.arange(seq)
        counts = [olb.causal_pair_count(olb.contiguous_shard_positions(seq, cp, r), allpos) for r in range(cp)]
        mean = seq * (seq + 1) / (2 * cp)
        assert abs(max(counts) / mean - ratio) < 2e-3, (seq, cp, max(counts) / mean)


@pytest.mark.parametrize("seq,cp", [(8, 2), (64, 4), (48, 3), (512, 2), (4096, 8)])
def test_permutation_round_trip_bit_exact(seq, cp):
    perm = olb.load_balance_perm(seq, cp)
    inv = olb.inverse_perm(perm)
    assert (perm[inv] == np.arange(seq)).all() and (inv[perm] == np.arange(seq)).all()
    x = torch.randint(-2**31, 2**31 - 1, (2, seq, 3), dtype=torch.int32)
    y = torch.cat([oatt.permute_ref(x, seq, cp, b0, b1 - b0)
                   for b0, b1 in (olb.shard_row_range(seq, cp, r) for r in range(cp))], dim=1)
    assert torch.equal(y, oatt.permute_ref(x, seq, cp))
    z = torch.zeros_like(x)
    for r in range(cp):
        b0, b1 = olb.shard_row_range(seq, cp, r)
        z = oatt.unpermute_ref(y[:, b0:b1], z, seq, cp, b0)
    assert torch.equal(z, x)


def _golden_rows():
    with open(os.path.join(GOLDEN, "lb_perm_s8_cp2.txt")) as f:
        lines = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    out = []
    for ln in lines:
        parts = [p.split() for p in ln.split("|")]
        out.append((int(parts[0][0]), int(parts[0][1]), [[int(x) for x in p] for p in parts[1:]]))
    return out


def _check_permute_direction(permute_fn, unpermute_fn):
    """The direction of the reference gather and scatter, pinned to the worked example and to the
    chunk rule itself (not to the oracle's index function): permuting the token ids 0..S-1 must
    give the shards printed on the page, rank r's window must read chunk r then chunk 2cp-1-r,
    and scattering the page's permuted ids must give 0..S-1 back. A gather by the inverse
    permutation (gather and scatter confused) gives 0,1,4,5,6,7,2,3 for the example."""
    for seq, cp, shards in _golden_rows():
        ids = torch.arange(seq, dtype=torch.int64)[None]
        got = permute_fn(ids, seq, cp)[0].tolist()
        assert got == [t for sh in shards for t in sh], (got, shards)
        flat = torch.tensor([t for sh in shards for t in sh], dtype=torch.int64)[None]
        back = unpermute_fn(flat, torch.zeros_like(flat), seq, cp)[0].tolist()
        assert back == list(range(seq)), back
    for seq, cp in [(48, 3), (64, 4), (4096, 8)]:
        c = seq // (2 * cp)
        ids = torch.arange(seq, dtype=torch.int64)[None]
        for r in range(cp):
            win = permute_fn(ids, seq, cp, r * 2 * c, 2 * c)[0]
            assert torch.equal(win[:c], torch.arange(r * c, (r + 1) * c)), (seq, cp, r)
            assert torch.equal(win[c:], torch.arange((2 * cp - 1 - r) * c, (2 * cp - r) * c)), (seq, cp, r)
            # scattering the window alone writes exactly the two chunks' ids at their own positions
            z = unpermute_fn(win[None], torch.full_like(ids, -1), seq, cp, r * 2 * c)[0]
            hit = (z >= 0).nonzero().flatten()
            assert torch.equal(z[hit], hit), (seq, cp, r)
            assert len(hit) == 2 * c


def test_permute_ref_direction():
    _check_permute_direction(oatt.permute_ref, oatt.unpermute_ref)


def test_index_rejects_bad_shapes():
    with pytest.raises(ValueError):
        olb.load_balance_perm(10, 2)
    with pytest.raises(ValueError):
        olb.shard_row_range(16, 2, 2)


# ----------------------------------------------------------------------------- attention pins

@pytest.mark.parametrize("seq,cp,hq,hkv,dqk,dv", [
    (8, 1, 2, 2, 4, 4), (8, 2, 4, 2, 4, 4), (16, 4, 2, 1, 3, 5), (16, 2, 4, 4, 6, 4), (12, 3, 2, 2, 4, 4)])
def test_brute_force(seq, cp, hq, hkv, dqk, dv):
    _check_brute(_oracle_att, seq, cp, hq, hkv, dqk, dv, seed=seq * 7 + cp)


@pytest.mark.parametrize("seq,cp,hq,hkv,dqk,dv,batch", [
    (64, 1, 4, 2, 16, 16, 1), (64, 2, 4, 2, 16, 16, 2), (128, 4, 6, 2, 12, 8, 1),
    (256, 8, 8, 8, 16, 16, 1), (96, 3, 4, 1, 8, 8, 1)])
def test_sharded_equals_library_causal_attention(seq, cp, hq, hkv, dqk, dv, batch):
    _check_library(_oracle_att, seq, cp, hq, hkv, dqk, dv, seed=seq + cp, batch=batch)


def test_cp_degrees_agree():
    seq, hq, hkv, d = 128, 4, 2, 16
    q, k, v = _rand((1, seq, hq, d), 1), _rand((1, seq, hkv, d), 2), _rand((1, seq, hkv, d), 3)
    outs = {}
    for cp in (1, 2, 4, 8):
        perm = olb.load_balance_perm(seq, cp)
        inv = olb.inverse_perm(perm)
        Os, Ls = [], []
        for r in range(cp):
            b0, b1 = olb.shard_row_range(seq, cp, r)
            O, L = oatt.cp_attention_ref(q[:, perm][:, b0:b1], k[:, perm], v[:, perm], perm[b0:b1], seq, cp, 0.25)
            Os.append(O)
            Ls.append(L)
        outs[cp] = (np.concatenate(Os, 1)[:, inv], np.concatenate(Ls, 2)[:, :, inv])
    for cp in (2, 4, 8):
        np.testing.assert_allclose(outs[cp][0], outs[1][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(outs[cp][1], outs[1][1], rtol=0, atol=1e-12)


def test_constant_v_returns_v():
    seq, cp = 64, 4
    perm = olb.load_balance_perm(seq, cp)
    q, k = _rand((1, seq, 4, 8), 5), _rand((1, seq, 2, 8), 6)
    vrow = _rand((2, 8), 7)
    v = np.broadcast_to(vrow, (1, seq, 2, 8)).copy()
    for r in range(cp):
        b0, b1 = olb.shard_row_range(seq, cp, r)
        O, _ = oatt.cp_attention_ref(q[:, perm][:, b0:b1], k[:, perm], v[:, perm], perm[b0:b1], seq, cp, 0.3)
        for h in range(4):
            np.testing.assert_allclose(O[0, :, h, :], np.broadcast_to(vrow[h // 2], (b1 - b0, 8)), rtol=0, atol=1e-12)


def test_identical_keys_give_prefix_mean():
    seq, cp, scale = 64, 2, 0.7
    perm = olb.load_balance_perm(seq, cp)
    q, v = _rand((1, seq, 2, 8), 8), _rand((1, seq, 1, 8), 9)
    krow = _rand((8,), 10)
    k = np.broadcast_to(krow, (1, seq, 1, 8)).copy()
    prefix_mean = np.cumsum(v[0, :, 0, :], axis=0) / np.arange(1, seq + 1)[:, None]
    for r in range(cp):
        b0, b1 = olb.shard_row_range(seq, cp, r)
        pos = perm[b0:b1]
        O, L = oatt.cp_attention_ref(q[:, perm][:, b0:b1], k[:, perm], v[:, perm], pos, seq, cp, scale)
        for h in range(2):
            np.testing.assert_allclose(O[0, :, h, :], prefix_mean[pos], rtol=0, atol=1e-12)
            expect = scale * (q[0, pos, h, :] @ krow) + np.log(pos + 1.0)
            np.testing.assert_allclose(L[0, h], expect, rtol=0, atol=1e-12)


def test_position_zero_row_and_lse_bounds():
    seq, cp, scale = 32, 2, 0.5
    perm = olb.load_balance_perm(seq, cp)
    q, k, v = _rand((1, seq, 2, 4), 11), _rand((1, seq, 2, 4), 12), _rand((1, seq, 2, 4), 13)
    b0, b1 = olb.shard_row_range(seq, cp, 0)
    pos = perm[b0:b1]
    O, L = oatt.cp_attention_ref(q[:, perm][:, b0:b1], k[:, perm], v[:, perm], pos, seq, cp, scale)
    i0 = int(np.nonzero(pos == 0)[0][0])
    for h in range(2):
        assert np.array_equal(O[0, i0, h], v[0, 0, h])
        assert L[0, h, i0] == scale * float(q[0, 0, h] @ k[0, 0, h])
    # max_j s_j <= LSE_i <= max_j s_j + ln(n_i)
    for i, p in enumerate(pos):
        for h in range(2):
            s = scale * (k[0, :p + 1, h] @ q[0, p, h])
            assert s.max() - 1e-12 <= L[0, h, i] <= s.max() + math.log(p + 1) + 1e-12


def test_rows_subset_matches_full():
    seq, cp = 128, 4
    perm = olb.load_balance_perm(seq, cp)
    q, k, v = _rand((1, seq, 4, 8), 14), _rand((1, seq, 2, 8), 15), _rand((1, seq, 2, 8), 16)
    b0, b1 = olb.shard_row_range(seq, cp, 1)
    full = oatt.cp_attention_ref(q[:, perm][:, b0:b1], k[:, perm], v[:, perm], perm[b0:b1], seq, cp, 0.3)
    rows = [0, 5, 15, 16, 30, 31]
    part = oatt.cp_attention_ref(q[:, perm][:, b0:b1], k[:, perm], v[:, perm], perm[b0:b1], seq, cp, 0.3, rows=rows)
    np.testing.assert_array_equal(part[0][:, rows], full[0][:, rows])
    np.testing.assert_array_equal(part[1][:, :, rows], full[1][:, :, rows])


# ----------------------------------------------------------------------------- decode pins

def _check_decode(dec_fn):
    B, Hq, Hkv, D, Lmax = 3, 6, 2, 8, 40
    rng = np.random.default_rng(21)
    lengths = np.array([1, 17, 40])
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Hkv, Lmax, D))
    vc = rng.standard_normal((B, Hkv, Lmax, D))
    scale = 0.35
    O, L = dec_fn(q, kc, vc, lengths, scale)
    for b in range(B):
        n = lengths[b]
        # the newest token sits at cache index n-1 and sees keys 0..n-1: last row of causal attention
        qq = q[b][None, None]  # [1, 1, Hq, D]
        kk = kc[b, :, :n].transpose(1, 0, 2)[None]
        vv = vc[b, :, :n].transpose(1, 0, 2)[None]
        Oc, Lc = _brute_force(qq, kk, vv, [n - 1], list(range(n)), scale)
        np.testing.assert_allclose(O[b], Oc[0, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[b], Lc[0, :, 0], rtol=0, atol=1e-12)
        # library routine: non-causal SDPA over the valid prefix
        tq = torch.from_numpy(q[b][:, None, :])  # Hq 1 D
        tk = torch.from_numpy(kc[b, :, :n]).repeat_interleave(Hq // Hkv, 0)
        tv = torch.from_numpy(vc[b, :, :n]).repeat_interleave(Hq // Hkv, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
        np.testing.assert_allclose(O[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)
    # NaN-poisoned tail must not change anything
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(B):
        kc2[b, :, lengths[b]:] = np.nan
        vc2[b, :, lengths[b]:] = np.nan
    O2, L2 = dec_fn(q, kc2, vc2, lengths, scale)
    assert np.array_equal(O2, O) and np.array_equal(L2, L)


def test_decode_pins():
    _check_decode(oatt.decode_ref)


def test_decode_empty_length():
    """A length-0 sequence (an empty slice of a cache split along its length) has LSE = ln 0 =
    -inf and output 0; the other sequences are unaffected."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4, 8))
    kc = rng.standard_normal((2, 2, 6, 8))
    vc = rng.standard_normal((2, 2, 6, 8))
    O, L = oatt.decode_ref(q, kc, vc, [0, 5], 0.3)
    assert np.all(O[0] == 0.0) and np.all(L[0] == -np.inf)
    O1, L1 = oatt.decode_ref(q[1:], kc[1:], vc[1:], [5], 0.3)
    np.testing.assert_array_equal(O[1], O1[0])
    np.testing.assert_array_equal(L[1], L1[0])


def _check_merge(merge_fn):
    """Split invariance: decoding disjoint slices of each cache and merging the results equals
    one decode over the whole cache (slices include empty ones); plus closed forms."""
    B, Hq, Hkv, D, Lmax, W = 3, 4, 2, 8, 40, 16
    rng = np.random.default_rng(31)
    lengths = np.array([40, 17, 1])
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Hkv, Lmax, D))
    vc = rng.standard_normal((B, Hkv, Lmax, D))
    scale = 0.3
    parts_o, parts_l = [], []
    for start in range(0, Lmax, W):
        width = min(W, Lmax - start)
        n = np.clip(lengths - start, 0, width)
        o, l = oatt.decode_ref(q, kc[:, :, start:start + width], vc[:, :, start:start + width], n, scale)
        parts_o.append(o)
        parts_l.append(l)
    O, L = merge_fn(np.stack(parts_o), np.stack(parts_l))
    O_full, L_full = oatt.decode_ref(q, kc, vc, lengths, scale)
    np.testing.assert_allclose(O, O_full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, L_full, rtol=0, atol=1e-12)
    # the same result from the library routine over each valid prefix
    for b in range(B):
        n = lengths[b]
        tk = torch.from_numpy(kc[b, :, :n]).repeat_interleave(Hq // Hkv, 0)
        tv = torch.from_numpy(vc[b, :, :n]).repeat_interleave(Hq // Hkv, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q[b][:, None, :]), tk, tv, scale=scale)
        np.testing.assert_allclose(O[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)
    # closed forms: one part is the identity; two equal parts keep O and add ln 2 to the LSE;
    # all parts empty give O = 0 and LSE = -inf
    O1, L1 = merge_fn(O_full[None], L_full[None])
    np.testing.assert_allclose(O1, O_full, rtol=0, atol=1e-15)
    np.testing.assert_allclose(L1, L_full, rtol=0, atol=1e-15)
    O2, L2 = merge_fn(np.stack([O_full, O_full]), np.stack([L_full, L_full]))
    np.testing.assert_allclose(O2, O_full, rtol=0, atol=1e-15)
    np.testing.assert_allclose(L2, L_full + math.log(2.0), rtol=0, atol=1e-12)
    O3, L3 = merge_fn(np.zeros((2, B, Hq, D)), np.full((2, B, Hq), -np.inf))
    assert np.all(O3 == 0.0) and np.all(L3 == -np.inf)


def test_decode_merge_pins():
    _check_merge(oatt.decode_merge_ref)


# ----------------------------------------------------------------------------- int8 cache pins

def _read_quant_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "kv_quant_rows.txt")):
        if line.startswith("#") or not line.strip():
            continue
        xs, cs, sc = (f.split() for f in line.split("|"))
        rows.append((np.array([float(t) for t in xs], dtype=np.float32), np.array([int(t) for t in cs]),
                     float.fromhex(sc[0])))
    return rows


def _check_quant_golden(quant_fn):
    for x, codes, scale in _read_quant_golden():
        c, s = quant_fn(x[None])
        assert np.array_equal(np.asarray(c)[0].astype(np.int64), codes), (x, c, codes)
        assert float(np.asarray(s)[0]) == scale, (x, s, scale)


def test_quantize_golden_rows():
    _check_quant_golden(oq.kv_quantize_ref)


def _check_quant_invariants(quant_fn):
    """Any correct absmax quantizer: codes in [-127, 127]; the largest |x| of a row maps to
    +-127; every code is the nearest integer to x / scale (within float32 rounding of the
    quotient); dequantized values are within half a step of x."""
    rng = np.random.default_rng(41)
    x = torch.from_numpy(rng.standard_normal((64, 128)) * rng.uniform(0.01, 50, (64, 1))).to(torch.bfloat16)
    c, s = quant_fn(x)
    c = np.asarray(c).astype(np.float64)
    s = np.asarray(s).astype(np.float64)
    xf = x.double().numpy()
    assert c.min() >= -127 and c.max() <= 127
    arg = np.abs(xf).argmax(1)
    assert np.all(np.abs(c[np.arange(64), arg]) == 127)
    assert np.all(np.sign(c[np.arange(64), arg]) == np.sign(xf[np.arange(64), arg]))
    np.testing.assert_allclose(s, np.abs(xf).max(1) / 127, rtol=2 ** -23, atol=0)
    assert np.all(np.abs(xf / s[:, None] - c) <= 0.5 + 1e-5)
    assert np.all(np.abs(xf - c * s[:, None]) <= s[:, None] * (0.5 + 1e-5))


def test_quantize_invariants():
    _check_quant_invariants(oq.kv_quantize_ref)


def _check_decode_int8(dec_fn):
    """Closed forms of decode over a quantized cache (values code * scale)."""
    rng = np.random.default_rng(43)
    B, Hq, Hkv, D, Lmax = 2, 4, 2, 8, 6
    q = rng.standard_normal((B, Hq, D))
    kq = rng.integers(-127, 128, (B, Hkv, Lmax, D)).astype(np.int8)
    vq = rng.integers(-127, 128, (B, Hkv, Lmax, D)).astype(np.int8)
    ks = rng.uniform(0.001, 0.02, (B, Hkv, Lmax)).astype(np.float32)
    vs = rng.uniform(0.5, 2.0, (B, Hkv, Lmax)).astype(np.float32)
    sm = 0.3
    # one key: O is that key's value, LSE its scaled logit
    O, L = dec_fn(q, kq, ks, vq, vs, [1, 1], sm)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            np.testing.assert_allclose(O[b, h], vq[b, g, 0].astype(np.float64) * float(vs[b, g, 0]), rtol=1e-14)
            logit = sm * float(ks[b, g, 0]) * float(np.dot(q[b, h], kq[b, g, 0].astype(np.float64)))
            np.testing.assert_allclose(L[b, h], logit, rtol=1e-12, atol=1e-12)
    # two keys: softmax of two logits written out
    O, L = dec_fn(q, kq, ks, vq, vs, [2, 2], sm)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            a = [sm * float(ks[b, g, j]) * float(q[b, h] @ kq[b, g, j]) for j in range(2)]
            e = [math.exp(t - max(a)) for t in a]
            want = sum(e[j] * vq[b, g, j].astype(np.float64) * float(vs[b, g, j]) for j in range(2)) / sum(e)
            np.testing.assert_allclose(O[b, h], want, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(L[b, h], max(a) + math.log(sum(e)), rtol=1e-12, atol=1e-12)
    # a zero query weighs every key alike: the mean of the values, LSE = ln n
    O, L = dec_fn(np.zeros_like(q), kq, ks, vq, vs, [5, 3], sm)
    for b, n in enumerate([5, 3]):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            want = (vq[b, g, :n].astype(np.float64) * vs[b, g, :n, None].astype(np.float64)).mean(0)
            np.testing.assert_allclose(O[b, h], want, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(L[b, h], math.log(n), rtol=1e-14)
    # scaling the V scales scales O; scaling the K scales by c equals a softmax scale c times larger
    O1, L1 = dec_fn(q, kq, ks, vq, vs, [6, 4], sm)
    O2, L2 = dec_fn(q, kq, ks, vq, (vs * 4).astype(np.float32), [6, 4], sm)
    np.testing.assert_allclose(O2, 4 * O1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=0)
    O3, L3 = dec_fn(q, kq, (ks * 2).astype(np.float32), vq, vs, [6, 4], sm)
    O4, L4 = dec_fn(q, kq, ks, vq, vs, [6, 4], 2 * sm)
    np.testing.assert_allclose(O3, O4, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L3, L4, rtol=1e-12, atol=1e-12)


def test_decode_int8_closed_forms():
    _check_decode_int8(oq.decode_int8_ref)


def test_quantized_decode_approximates_float_decode():
    """Quantizing a bf16 cache and decoding the codes stays close to decoding the bf16 cache:
    per-row absmax int8 keeps each value within amax/254, far below the tolerance used here."""
    rng = np.random.default_rng(47)
    B, Hq, Hkv, D, Lmax = 2, 8, 2, 64, 50
    q = torch.from_numpy(rng.standard_normal((B, Hq, D))).to(torch.bfloat16)
    kc = torch.from_numpy(rng.standard_normal((B, Hkv, Lmax, D))).to(torch.bfloat16)
    vc = torch.from_numpy(rng.standard_normal((B, Hkv, Lmax, D))).to(torch.bfloat16)
    kq, ks = oq.kv_quantize_ref(kc)
    vq, vs = oq.kv_quantize_ref(vc)
    O, L = oq.decode_int8_ref(q, kq, ks, vq, vs, [50, 31], 0.125)
    Of, Lf = oatt.decode_ref(q, kc, vc, [50, 31], 0.125)
    assert np.max(np.abs(O - Of)) < 2e-2 and np.max(np.abs(L - Lf)) < 2e-2
    assert np.max(np.abs(O - Of)) > 0  # the quantization really changed the cache


# ----------------------------------------------------------------------------- backward pins

def _sdpa_grads(q, k, v, do, q_pos, k_pos, scale):
    """torch float64 autograd through the library's masked scaled_dot_product_attention."""
    B, Sq, Hq, _ = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    mask = torch.as_tensor(np.asarray(k_pos))[None, :] <= torch.as_tensor(np.asarray(q_pos))[:, None]
    kk = tk.repeat_interleave(G, dim=2).transpose(1, 2)
    vv = tv.repeat_interleave(G, dim=2).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(tq.transpose(1, 2), kk, vv, attn_mask=mask, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64).transpose(1, 2))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _check_bwd_library(bwd_fn, seq, cp, hq, hkv, dqk, dv, seed, batch=1):
    """Each rank's dQ equals the library autograd dQ at its rows; the ranks' dK and dV summed
    equal the library's (keys compared in gathered order)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, seq, hq, dqk))
    k = rng.standard_normal((batch, seq, hkv, dqk))
    v = rng.standard_normal((batch, seq, hkv, dv))
    do = rng.standard_normal((batch, seq, hq, dv))
    scale = 1.0 / math.sqrt(dqk)
    pos = np.arange(seq)
    dq_ref, dk_ref, dv_ref = _sdpa_grads(q, k, v, do, pos, pos, scale)
    perm = olb.load_balance_perm(seq, cp)
    dk_sum = np.zeros_like(k)
    dv_sum = np.zeros_like(v)
    for r in range(cp):
        b0, b1 = olb.shard_row_range(seq, cp, r)
        rows = perm[b0:b1]
        dq, dk, dv_ = bwd_fn(q[:, rows], k[:, perm], v[:, perm], do[:, rows], rows, perm, scale)
        np.testing.assert_allclose(dq, dq_ref[:, rows], rtol=0, atol=1e-10)
        dk_sum += dk
        dv_sum += dv_
    np.testing.assert_allclose(dk_sum, dk_ref[:, perm], rtol=0, atol=1e-10)
    np.testing.assert_allclose(dv_sum, dv_ref[:, perm], rtol=0, atol=1e-10)


@pytest.mark.parametrize("seq,cp,hq,hkv,dqk,dv,batch", [
    (16, 1, 2, 2, 8, 8, 1),
    (32, 2, 4, 2, 8, 4, 2),
    (64, 4, 6, 3, 12, 8, 1),
])
def test_backward_matches_library_autograd(seq, cp, hq, hkv, dqk, dv, batch):
    _check_bwd_library(obw.causal_attention_bwd_ref, seq, cp, hq, hkv, dqk, dv, 71, batch)


def _forward_loss(q, k, v, do, q_pos, k_pos, scale):
    o, _ = oatt.causal_attention_ref(q, k, v, q_pos, k_pos, scale)
    return float((o * do).sum())


def _check_bwd_finite_differences(bwd_fn):
    """Central differences of L = sum(dO * O) through the forward oracle."""
    rng = np.random.default_rng(73)
    seq, cp = 8, 2
    q = rng.standard_normal((1, 4, 2, 4))
    k = rng.standard_normal((1, seq, 1, 4))
    v = rng.standard_normal((1, seq, 1, 3))
    do = rng.standard_normal((1, 4, 2, 3))
    perm = olb.load_balance_perm(seq, cp)
    rows = perm[4:8]
    scale = 0.7
    dq, dk, dv = bwd_fn(q, k, v, do, rows, perm, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [tuple(int(rng.integers(0, n)) for n in x.shape) for _ in range(6)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _forward_loss(args["q"], args["k"], args["v"], do, rows, perm, scale)
            args[name] = xm
            lm = _forward_loss(args["q"], args["k"], args["v"], do, rows, perm, scale)
            num = (lp - lm) / (2 * h)
            assert abs(num - g[idx]) <= 1e-7 * max(1.0, abs(num)), (name, idx, num, g[idx])


def test_backward_finite_differences():
    _check_bwd_finite_differences(obw.causal_attention_bwd_ref)


def _check_bwd_closed_forms(bwd_fn):
    rng = np.random.default_rng(79)
    seq, hq, hkv, d = 12, 4, 2, 6
    pos = np.arange(seq)
    q = rng.standard_normal((1, seq, hq, d))
    k = rng.standard_normal((1, seq, hkv, d))
    do = rng.standard_normal((1, seq, hq, d))
    # constant V: O does not depend on the scores, so dQ = dK = 0 and dV_j = sum_i P_ij dO_i
    v = np.broadcast_to(rng.standard_normal((1, 1, hkv, d)), (1, seq, hkv, d)).copy()
    dq, dk, dv = bwd_fn(q, k, v, do, pos, pos, 0.5)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    # identical keys: every visible key has P_ij = 1 / (i + 1), so
    # dV_j = sum over query heads of the group and rows i >= j of dO_i / (i + 1)
    k_same = np.broadcast_to(k[:, :1], k.shape).copy()
    v2 = rng.standard_normal((1, seq, hkv, d))
    dq, dk, dv = bwd_fn(q, k_same, v2, do, pos, pos, 0.5)
    G = hq // hkv
    for g in range(hkv):
        for j in range(seq):
            want = sum(do[0, i, h] / (i + 1) for i in range(j, seq) for h in range(g * G, (g + 1) * G))
            np.testing.assert_allclose(dv[0, j, g], want, rtol=1e-12, atol=1e-12)
    # any inputs: the softmax gradient sums to zero over each row, so dK summed over keys is 0
    v3 = rng.standard_normal((1, seq, hkv, d))
    dq, dk, dv = bwd_fn(q, k, v3, do, pos, pos, 0.5)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    assert np.abs(dk).max() > 1e-3


def test_backward_closed_forms():
    _check_bwd_closed_forms(obw.causal_attention_bwd_ref)


# ----------------------------------------------------------------------------- planted mistakes

def _perm_swapped_chunk_order(seq, cp):
    c = seq // (2 * cp)
    out = []
    for r in range(cp):
        out += list(range((2 * cp - 1 - r) * c, (2 * cp - r) * c)) + list(range(r * c, (r + 1) * c))
    return np.array(out)


def _perm_unbalanced(seq, cp):
    c = seq // (2 * cp)
    out = []
    for r in range(cp):
        out += list(range(r * c, (r + 1) * c)) + list(range((cp + r) * c, (cp + r + 1) * c))
    return np.array(out)


def _att_strict_mask(q, k, v, q_pos, k_pos, scale):
    return oatt.causal_attention_ref(q, k, v, np.asarray(q_pos) - 1, k_pos, scale)


def _att_no_scale(q, k, v, q_pos, k_pos, scale):
    return oatt.causal_attention_ref(q, k, v, q_pos, k_pos, 1.0)


def _att_wrong_group(q, k, v, q_pos, k_pos, scale):
    # query head h reads kv head h % Hkv instead of h // G
    Hq, Hkv = q.shape[2], k.shape[2]
    idx = [h % Hkv for h in range(Hq)]
    kk = np.asarray(k)[:, :, idx]
    vv = np.asarray(v)[:, :, idx]
    return oatt.causal_attention_ref(q, kk, vv, q_pos, k_pos, scale)


def _att_transposed_v(q, k, v, q_pos, k_pos, scale):
    vv = np.asarray(v)[:, ::-1]  # values taken from the mirrored token
    return oatt.causal_attention_ref(q, k, vv, q_pos, k_pos, scale)


def _dec_off_by_one(q, kc, vc, lengths, scale):
    return oatt.decode_ref(q, kc, vc, np.asarray(lengths) - 1 + (np.asarray(lengths) == 1), scale)


def _merge_unweighted(o_parts, lse_parts):
    # averages the live parts' outputs instead of weighting them by exp(lse)
    o, l = np.asarray(o_parts, dtype=np.float64), np.asarray(lse_parts, dtype=np.float64)
    live = l != -np.inf
    cnt = np.maximum(live.sum(0), 1)
    O = np.where(live[..., None], o, 0.0).sum(0) / cnt[..., None]
    m = np.where(live, l, -np.inf).max(0)
    L = np.where(np.isfinite(m), m + np.log(np.where(live, np.exp(l - np.where(np.isfinite(m), m, 0)), 0).sum(0)), -np.inf)
    return O, L


def _quant_half_away(x):
    # rounds ties away from zero instead of to even
    codes, scales = oq.kv_quantize_ref(x)
    x32 = np.asarray(x, dtype=np.float32).reshape(-1, np.shape(x)[-1])
    s = scales.reshape(-1)
    out = codes.reshape(x32.shape).copy()
    for i in range(x32.shape[0]):
        if s[i] != 0:
            t = x32[i] / s[i]
            out[i] = np.clip(np.sign(t) * np.floor(np.abs(t) + np.float32(0.5)), -127, 127).astype(np.int8)
    return out.reshape(np.shape(x)), scales


def _dec_int8_k_scale_on_v(q, kq, ks, vq, vs, lengths, scale):
    return oq.decode_int8_ref(q, kq, ks, vq, ks, lengths, scale)


def _dec_int8_no_k_scale(q, kq, ks, vq, vs, lengths, scale):
    return oq.decode_int8_ref(q, kq, np.ones_like(ks), vq, vs, lengths, scale)


def _bwd_no_delta(q, k, v, do, q_pos, k_pos, scale):
    # drops the D_i term of dS: dS = P * dP
    k_pos = np.asarray(k_pos)
    q_pos = np.asarray(q_pos)
    q64, k64, v64, do64 = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Sq, Hq, _ = q64.shape
    Hkv = k64.shape[2]
    G = Hq // Hkv
    dq, dk, dv = np.zeros_like(q64), np.zeros_like(k64), np.zeros_like(v64)
    vis = k_pos[None, :] <= q_pos[:, None]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s_ = np.where(vis, scale * q64[b, :, h] @ k64[b, :, g].T, -np.inf)
            p = np.exp(s_ - s_.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            ds = p * (do64[b, :, h] @ v64[b, :, g].T)
            dq[b, :, h] = scale * ds @ k64[b, :, g]
            dk[b, :, g] += scale * ds.T @ q64[b, :, h]
            dv[b, :, g] += p.T @ do64[b, :, h]
    return dq, dk, dv


def _bwd_dk_unscaled(q, k, v, do, q_pos, k_pos, scale):
    dq, dk, dv = obw.causal_attention_bwd_ref(q, k, v, do, q_pos, k_pos, scale)
    return dq, dk / scale, dv


def _bwd_dv_one_head(q, k, v, do, q_pos, k_pos, scale):
    # keeps only the first query head of each group in dV
    q = np.asarray(q, dtype=np.float64).copy()
    dq, dk, dv = obw.causal_attention_bwd_ref(q, k, v, do, q_pos, k_pos, scale)
    G = q.shape[2] // np.asarray(k).shape[2]
    do0 = np.asarray(do, dtype=np.float64).copy()
    for h in range(q.shape[2]):
        if h % G:
            do0[:, :, h] = 0
    _, _, dv0 = obw.causal_attention_bwd_ref(q, k, v, do0, q_pos, k_pos, scale)
    return dq, dk, dv0


def _permute_by_inverse(x, seq, cp, row_begin=0, row_count=None):
    # gathers with the inverse permutation (gather and scatter confused)
    inv = olb.inverse_perm(olb.load_balance_perm(seq, cp))
    if row_count is None:
        row_count = seq - row_begin
    return x[:, inv[row_begin:row_begin + row_count]]


def _unpermute_by_inverse(x_window, dst, seq, cp, row_begin=0):
    inv = olb.inverse_perm(olb.load_balance_perm(seq, cp))
    out = dst.clone()
    out[:, inv[row_begin:row_begin + x_window.shape[1]]] = x_window
    return out


@pytest.mark.parametrize("check", [
    lambda: _check_golden(_perm_swapped_chunk_order),
    lambda: _check_permute_direction(_permute_by_inverse, _unpermute_by_inverse),
    lambda: _check_permute_direction(oatt.permute_ref, _unpermute_by_inverse),
    lambda: _check_balance(_perm_unbalanced, 64, 4),
    lambda: _check_brute(_att_strict_mask, 8, 2, 2, 2, 4, 4, 3),
    lambda: _check_library(_att_no_scale, 64, 2, 4, 2, 16, 16, 3),
    lambda: _check_library(_att_wrong_group, 64, 2, 4, 2, 16, 16, 3),
    lambda: _check_brute(_att_transposed_v, 8, 2, 2, 1, 4, 4, 3),
    lambda: _check_decode(_dec_off_by_one),
    lambda: _check_merge(_merge_unweighted),
    lambda: _check_quant_golden(_quant_half_away),
    lambda: _check_decode_int8(_dec_int8_k_scale_on_v),
    lambda: _check_decode_int8(_dec_int8_no_k_scale),
    lambda: _check_bwd_library(_bwd_no_delta, 32, 2, 4, 2, 8, 4, 5),
    lambda: _check_bwd_finite_differences(_bwd_dk_unscaled),
    lambda: _check_bwd_library(_bwd_dv_one_head, 32, 2, 4, 2, 8, 4, 5),
], ids=["chunk-order", "permute-by-inverse", "unpermute-by-inverse", "unbalanced", "strict-mask", "no-scale", "wrong-group", "mirrored-v", "decode-length",
        "merge-unweighted", "quant-ties-away", "int8-k-scale-on-v", "int8-no-k-scale", "bwd-no-delta", "bwd-dk-unscaled",
        "bwd-dv-one-head"])
def test_planted_mistakes_are_caught(check):
    with pytest.raises((AssertionError, ValueError, IndexError)):
        check()
