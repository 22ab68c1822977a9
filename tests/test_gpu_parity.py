"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Inputs come from the seeded generators in ``context_causal_attention_load_amd.synth``; the
oracle permutes and computes from the natural-order CPU tensors on its own, so no oracle input
or expected value comes from the GPU. Tolerances: max abs error <= 1e-4 for float32 inputs and
<= 2e-2 for bfloat16 inputs (on O and on LSE); the permutation is compared bit for bit.
"""

import math

import numpy as np
import pytest
import torch

import context_causal_attention_load_amd as cpa
from context_causal_attention_load_amd import synth
from oracle import attention as oatt
from oracle import lb_index as olb

from closed_forms import bwd_tol, check_identical_keys_bwd, check_identical_keys_dk
from gpu_util import (DEV, TOL, Prefill, announce, assert_close, check_rank, describe_rows, sample_rows,
                      stratified_rows)

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------- permutation

@pytest.mark.parametrize("outer,seq,inner,dtype,cp", [
    (1, 512, (4, 64), torch.float32, 2),
    (2, 96, (3,), torch.int32, 3),
    (3, 64, (5,), torch.uint8, 4),        # 5-byte rows: byte path
    (2, 40, (3,), torch.int16, 2),        # 6-byte rows: 2-byte path
    (1, 4096, (2, 4), torch.bfloat16, 8),  # 16-byte rows
    (1, 8192, (32, 128), torch.bfloat16, 4),
])
def test_permute_bit_exact(outer, seq, inner, dtype, cp):
    announce(f"permute outer={outer} seq={seq} inner={inner} {dtype} cp={cp}")
    g = torch.Generator().manual_seed(seq + cp)
    if dtype.is_floating_point:
        x = torch.randn((outer, seq) + inner, generator=g).to(dtype)
    else:
        info = torch.iinfo(dtype)
        x = torch.randint(info.min, info.max, (outer, seq) + inner, generator=g, dtype=torch.int64).to(dtype)
    xd = x.to(DEV)
    full = cpa.permute(xd, cp).cpu()
    assert torch.equal(full, oatt.permute_ref(x, seq, cp))
    c = seq // (2 * cp)
    back = torch.zeros_like(xd)
    for r in range(cp):
        win = cpa.permute(xd, cp, row_begin=r * 2 * c, row_count=2 * c)
        assert torch.equal(win.cpu(), oatt.permute_ref(x, seq, cp, r * 2 * c, 2 * c))
        cpa.unpermute(win, cp, seq, row_begin=r * 2 * c, out=back)
    assert torch.equal(back.cpu(), x)
    # an odd window and its scatter
    b0, n = 3, seq // 2 - 1
    win = cpa.permute(xd, cp, row_begin=b0, row_count=n)
    assert torch.equal(win.cpu(), oatt.permute_ref(x, seq, cp, b0, n))
    dst = torch.zeros_like(x)
    got = cpa.unpermute(win, cp, seq, row_begin=b0, out=torch.zeros_like(xd)).cpu()
    assert torch.equal(got, oatt.unpermute_ref(oatt.permute_ref(x, seq, cp, b0, n), dst, seq, cp, b0))


def test_permute_last_axis_lse_layout():
    announce("permute along the last axis of [B, H, S] fp32")
    B, H, S, cp = 2, 6, 256, 4
    x = torch.randn(B, H, S)
    xd = x.to(DEV)
    y = cpa.permute(xd, cp, dim=2).cpu()
    perm = olb.load_balance_perm(S, cp)
    assert torch.equal(y, x[:, :, perm])
    back = cpa.unpermute(y.to(DEV), cp, S, dim=2).cpu()
    assert torch.equal(back, x)


# ----------------------------------------------------------------------------- attention, small full

SMALL = [
    # name, batch, seq, cps, hq, hkv, dqk, dv, dtype, seed
    ("tiny-cp2-fp32", 1, 512, (2,), 4, 2, 64, 64, torch.float32, 1),
    ("gqa-g4-bf16", 1, 1024, (4, 1), 8, 2, 128, 128, torch.bfloat16, 11),
    ("ragged-c100-bf16", 1, 600, (3,), 6, 3, 128, 128, torch.bfloat16, 12),
    ("mla-192-128-bf16", 1, 512, (2,), 4, 4, 192, 128, torch.bfloat16, 13),
    ("d64-g4-bf16", 1, 256, (1, 2), 4, 1, 64, 64, torch.bfloat16, 14),
    ("batch2-g8-bf16", 2, 384, (2,), 16, 2, 128, 128, torch.bfloat16, 15),
    ("g16-bf16", 1, 256, (2,), 16, 1, 128, 128, torch.bfloat16, 16),
    ("fp32-d128", 1, 256, (2,), 2, 2, 128, 128, torch.float32, 17),
    ("chunk1-bf16", 1, 4, (2, 1), 1, 1, 64, 64, torch.bfloat16, 18),
    ("chunk1-cp4-fp32", 1, 8, (4,), 2, 1, 64, 64, torch.float32, 19),
    # Dqk 192 runs 96-key tiles: a chunk of exactly one tile, one key past it, one short of two
    ("mla-c96-bf16", 1, 384, (2,), 2, 2, 192, 128, torch.bfloat16, 20),
    ("mla-c97-g2-bf16", 1, 388, (2,), 4, 2, 192, 128, torch.bfloat16, 21),
    ("mla-c191-cp3-bf16", 1, 1146, (3,), 2, 1, 192, 128, torch.bfloat16, 22),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_attention_small_all_ranks(case):
    name, batch, seq, cps, hq, hkv, dqk, dv, dtype, seed = case
    pf = Prefill(batch, seq, hq, hkv, dqk, dv, dtype, seed)
    for cp in cps:
        for r in range(cp):
            check_rank(pf, cp, r, tag=name)


SPLIT_CASES = [
    # name, batch, seq, cp, hq, hkv, dqk, dv, seed: shapes whose grids are small enough for the
    # forward to cut heavy row blocks' key ranges into pieces (a workspace is passed)
    ("split-mha-cp1", 1, 2048, 1, 1, 1, 128, 128, 61),
    ("split-gqa-g8", 1, 2048, 2, 16, 2, 128, 128, 62),
    ("split-mla-192", 1, 1024, 2, 2, 2, 192, 128, 63),
    ("split-d64-g4", 1, 2048, 2, 4, 1, 64, 64, 64),
    ("split-ragged-b2", 2, 2400, 3, 2, 2, 128, 128, 65),   # c = 400: row blocks straddle both chunks
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_attention_split_heavy_row_blocks(case):
    """The key-range split of heavy row blocks (cp_attention_fwd_ws): every row of every rank
    against the oracle, and against the unsplit call on the same inputs."""
    name, batch, seq, cp, hq, hkv, dqk, dv, seed = case
    pf = Prefill(batch, seq, hq, hkv, dqk, dv, torch.bfloat16, seed)
    kp, vp = pf.kv_perm(cp)
    c = seq // (2 * cp)
    for r in range(cp):
        need = cpa.attention_fwd_workspace_bytes(batch, seq, hq, hkv, dqk, dv, torch.bfloat16, cp, r)
        announce(f"{name} rank {r}: split workspace {need} bytes")
        assert need > 0, "this shape was chosen to be split"
        ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)  # garbage: contents must not matter
        qs = cpa.permute(pf.qd, cp, row_begin=r * 2 * c, row_count=2 * c)
        o, lse = cpa.attention_fwd(qs, kp, vp, cp, r, scale=pf.scale, workspace=ws)
        o1, lse1 = cpa.attention_fwd(qs, kp, vp, cp, r, scale=pf.scale, split=False)
        torch.cuda.synchronize()
        O_ref, L_ref = pf.oracle_rank(cp, r)
        assert_close(o.float().cpu().numpy(), O_ref, 2e-2, f"{name} split O r{r}")
        assert_close(lse.cpu().numpy(), L_ref, 2e-2, f"{name} split LSE r{r}")
        assert_close(o.float().cpu().numpy(), o1.float().cpu().numpy(), 2e-2, f"{name} split vs unsplit O r{r}")


def test_sharded_outputs_reassemble_to_full_causal_attention():
    """Concatenated, un-permuted per-rank outputs equal un-sharded causal attention (the
    relation the CP unit test of PR 2023 checks), on the GPU and against the oracle."""
    announce("reassemble cp=4 ranks vs cp=1 and vs oracle full causal attention")
    seq, hq, hkv, d, cp = 1024, 8, 2, 128, 4
    pf = Prefill(1, seq, hq, hkv, d, d, torch.bfloat16, 21)
    c = seq // (2 * cp)
    O_nat = torch.zeros((1, seq, hq, d), dtype=torch.bfloat16, device=DEV)
    L_nat = torch.zeros((1, hq, seq), dtype=torch.float32, device=DEV)
    for r in range(cp):
        o, lse = pf.gpu_rank(cp, r)
        cpa.unpermute(o, cp, seq, row_begin=r * 2 * c, out=O_nat)
        cpa.unpermute(lse, cp, seq, dim=2, row_begin=r * 2 * c, out=L_nat)
    o1, l1 = pf.gpu_rank(1, 0)
    nat = np.arange(seq)
    O_ref, L_ref = oatt.causal_attention_ref(pf.q, pf.k, pf.v, nat, nat, pf.scale)
    assert_close(O_nat.float().cpu().numpy(), O_ref, 2e-2, "reassembled O vs oracle")
    assert_close(L_nat.cpu().numpy(), L_ref, 2e-2, "reassembled LSE vs oracle")
    assert_close(O_nat.float().cpu().numpy(), o1.float().cpu().numpy(), 2e-2, "reassembled O vs cp=1")


def test_explicit_positions_match_implicit_and_unbalanced_shard():
    announce("q_positions given explicitly; contiguous (unbalanced) shard positions")
    seq, cp, hq, hkv, d = 512, 2, 4, 2, 128
    pf = Prefill(1, seq, hq, hkv, d, d, torch.bfloat16, 22)
    pos = cpa.lb_positions(seq, cp, 256, 256).to(DEV)
    o_imp, l_imp = pf.gpu_rank(cp, 1)
    o_exp, l_exp = pf.gpu_rank(cp, 1, q_positions=pos)
    assert torch.equal(o_imp, o_exp) and torch.equal(l_imp, l_exp)
    # rows taken contiguously from the natural sequence (no load balance) against permuted K/V
    kp, vp = pf.kv_perm(cp)
    for r in range(cp):
        rows = torch.arange(r * seq // cp, (r + 1) * seq // cp, dtype=torch.int32)
        qs = pf.qd[:, rows.long().to(DEV)].contiguous()
        o, lse = cpa.attention_fwd(qs, kp, vp, cp, r, q_positions=rows.to(DEV), scale=pf.scale)
        O_ref, L_ref = oatt.causal_attention_ref(pf.q[:, rows.long()], oatt.permute_ref(pf.k, seq, cp),
                                                 oatt.permute_ref(pf.v, seq, cp), rows.numpy(),
                                                 olb.load_balance_perm(seq, cp), pf.scale)
        assert_close(o.float().cpu().numpy(), O_ref, 2e-2, f"unbalanced O r={r}")
        assert_close(lse.cpu().numpy(), L_ref, 2e-2, f"unbalanced LSE r={r}")


def test_attention_is_deterministic():
    announce("determinism: two identical calls")
    pf = Prefill(1, 2048, 16, 2, 128, 128, torch.bfloat16, 23)
    a = pf.gpu_rank(2, 1)
    b = pf.gpu_rank(2, 1)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ----------------------------------------------------------------------------- full-size, sampled rows

_FULL = {}


def full_workload(w):
    """One set of full-size inputs at a time (the 131072-token one holds ~3 GB on the host)."""
    if w.name not in _FULL:
        _FULL.clear()
        torch.cuda.empty_cache()
        announce(f"generating {w.name}")
        _FULL[w.name] = Prefill(w.batch, w.seq, w.hq, w.hkv, w.d_qk, w.d_v, w.dtype, w.seed)
    return _FULL[w.name]


@pytest.mark.parametrize("cp", synth.LLAMA2_7B_S8K.cps)
def test_attention_llama7b_every_row(cp):
    """8192-token Llama2-7B-shaped MHA: the complete O and LSE of every rank (every row, every
    head) against the oracle, at cp = 1 (natural order) and at cp = 4 (load-balanced shards)."""
    w = synth.LLAMA2_7B_S8K
    pf = full_workload(w)
    for rank in range(cp):
        check_rank(pf, cp, rank, rows=None, tag=w.name)


def test_attention_contiguous_shards_llama7b():
    """The unbalanced (contiguous) layout the load balance replaces: rank r's rows are
    r*S/cp .. of the natural order and K/V stay in natural order (the call's cp = 1 order with
    explicit positions). Sampled rows of every rank of cp = 4 against plain causal attention."""
    w = synth.LLAMA2_7B_S8K
    pf = full_workload(w)
    cp, S = 4, w.seq
    k_nat, v_nat = pf.k.double(), pf.v.double()
    kpos = np.arange(S)
    for r in range(cp):
        b0, n = r * S // cp, S // cp
        rows = torch.arange(b0, b0 + n, dtype=torch.int32)
        announce(f"contiguous shard r={r} rows {b0}..{b0 + n - 1}")
        o, lse = cpa.attention_fwd(pf.qd[:, b0:b0 + n], pf.kd, pf.vd, 1, 0, q_positions=rows.to(DEV), scale=pf.scale)
        torch.cuda.synchronize()
        pick = sample_rows(n // 2, 24, seed=77 + r)
        O_ref, L_ref = oatt.causal_attention_ref(pf.q[:, b0 + pick], k_nat, v_nat, (b0 + pick), kpos, pf.scale)
        assert_close(o[:, pick].float().cpu().numpy(), O_ref, TOL[pf.dtype], f"contiguous O r={r}")
        assert_close(lse[:, :, pick].cpu().numpy(), L_ref, TOL[pf.dtype], f"contiguous LSE r={r}")


def test_attention_mla_rank0_every_row():
    """Every row and head of rank 0 at the DeepSeek-V3 MLA size (S 32768, cp 4: 8192 rows x 128
    heads, Dqk 192, Dv 128). Rank 0 holds both the shortest chunk (positions 0..4095) and the
    longest (28672..32767)."""
    w = synth.DEEPSEEK_V3_MLA_S32K
    pf = full_workload(w)
    check_rank(pf, w.cps[0], 0, rows=None, tag=w.name)


FULL_CASES = [(w, cp, r) for w in (synth.DEEPSEEK_V3_MLA_S32K, synth.LLAMA31_70B_S131K)
              for cp in w.cps for r in range(cp)]


@pytest.mark.parametrize("w,cp,rank", FULL_CASES, ids=[f"{w.name}-cp{cp}-r{r}" for w, cp, r in FULL_CASES])
def test_attention_full_size_stratified(w, cp, rank):
    """Random-data parity at the DeepSeek-V3 MLA (cp 4) and Llama3.1-70B (cp 8) sizes, every rank:
    the first and last 8 rows of both chunks plus 16 seeded rows for each of the 32 positions in a
    32-row block (about 540 rows), every head, element by element against the oracle."""
    pf = full_workload(w)
    c = w.seq // (2 * cp)
    rows = stratified_rows(c, 16, seed=1000 * cp + rank)
    print(f"  checked rows of rank {rank}: {describe_rows(rows, c)}", flush=True)
    check_rank(pf, cp, rank, rows=rows, tag=w.name)


def test_permute_full_size_llama70b():
    """Full-size gather/scatter of the 131072-token workload (runs after its attention tests so
    the cached inputs are reused)."""
    w = synth.LLAMA31_70B_S131K
    pf = full_workload(w)
    announce(f"permute {w.name}: K full, Q rank-3 window and its scatter")
    assert torch.equal(cpa.permute(pf.kd, 8).cpu(), oatt.permute_ref(pf.k, w.seq, 8))
    c = w.seq // 16
    win = cpa.permute(pf.qd, 8, row_begin=3 * 2 * c, row_count=2 * c)
    assert torch.equal(win.cpu(), oatt.permute_ref(pf.q, w.seq, 8, 3 * 2 * c, 2 * c))
    out = torch.zeros_like(pf.qd)
    cpa.unpermute(win, 8, w.seq, row_begin=3 * 2 * c, out=out)
    pos = torch.from_numpy(olb.shard_positions(w.seq, 8, 3))
    assert torch.equal(out[:, pos.to(DEV)].cpu(), pf.q[:, pos])


@pytest.mark.parametrize("w", [synth.LLAMA31_70B_S131K, synth.DEEPSEEK_V3_MLA_S32K], ids=lambda w: w.name)
def test_attention_full_size_identical_keys_every_row(w):
    """Every row and head of every rank at full size, against a closed form. All keys of a kv
    head are set equal (k_j = k_g, the natural-order row 0), so every visible key gets the same
    weight: O_i is the mean of v_j over the keys with position <= the row's position (a prefix
    mean of V in natural order), and LSE_i = scale * q_i . k_g + ln(pos_i + 1).

    The kernel's probabilities are then exactly 1 and its row sum is the exact count of visible
    keys, so the comparison can be tight: O within bf16 rounding (2^-8 |O| + 1e-5), and LSE within
    2e-5 once the expected logit models the kernel's one documented rounding of the scores' input
    (the query times scale * log2(e) in float32, rounded to bfloat16, then an exact product with
    k_g); what is left is float32 accumulation (observed at most 2.8e-6). A visible-key count off
    by 2e-5 of itself (3 keys at position 131071, 1 key below position 50000) fails the LSE check
    in any row; a wrong row, head or kv group fails both."""
    pf = full_workload(w)
    cp = w.cps[-1]
    S, c = w.seq, w.seq // (2 * cp)
    G = w.hq // w.hkv
    k1d = pf.kd[:, :1].expand(-1, S, -1, -1).contiguous()
    kp = cpa.permute(k1d, cp)
    vp = pf.kv_perm(cp)[1]
    k1 = pf.k[0, 0].double()                                                   # [Hkv, Dqk]
    sl2 = torch.tensor(pf.scale, dtype=torch.float32) * torch.tensor(math.log2(math.e), dtype=torch.float32)
    worst_o = worst_l = 0.0
    for r in range(cp):
        announce(f"{w.name} identical keys, every row: cp={cp} rank={r}")
        qs = cpa.permute(pf.qd, cp, row_begin=r * 2 * c, row_count=2 * c)
        o, lse = cpa.attention_fwd(qs, kp, vp, cp, r, scale=pf.scale)
        torch.cuda.synchronize()
        o, lse = o[0].float().cpu(), lse[0].cpu().double()                    # [Sq, Hq, Dv], [Hq, Sq]
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        pos = torch.from_numpy(olb.shard_positions(S, cp, r)).long()
        cnt = (pos + 1).double()
        for g in range(w.hkv):
            hs = slice(g * G, (g + 1) * G)
            pref = pf.v[0, :, g].double().cumsum(0)[pos] / cnt[:, None]      # [Sq, Dv]
            err_o = (o[:, hs].double() - pref[:, None, :]).abs()
            tol_o = pref.abs()[:, None, :] * 2.0 ** -8 + 1e-5
            bad = err_o > tol_o
            assert not bad.any(), (f"O rank {r} group {g}: {int(bad.sum())} elements beyond bf16 rounding, "
                                   f"max err {float(err_o.max()):.3e}")
            qr = (pf.q[0, pos, hs].float() * sl2).to(torch.bfloat16).double()  # [Sq, G, Dqk]
            lse_ref = (qr @ k1[g]) * math.log(2.0) + torch.log(cnt)[:, None]  # [Sq, G]
            err_l = (lse[hs].T - lse_ref).abs()
            assert float(err_l.max()) <= 2e-5, f"LSE rank {r} group {g}: max err {float(err_l.max()):.3e}"
            worst_o = max(worst_o, float((err_o / tol_o).max()))
            worst_l = max(worst_l, float(err_l.max()))
    print(f"  every row of every rank: O error at most {worst_o:.3f} of its bf16 bound, LSE error at most "
          f"{worst_l:.2e}", flush=True)


def test_tiny_workload_full():
    w = synth.TINY_CP2_F32
    pf = Prefill(w.batch, w.seq, w.hq, w.hkv, w.d_qk, w.d_v, w.dtype, w.seed)
    for r in range(2):
        check_rank(pf, 2, r, tag=w.name)


# ----------------------------------------------------------------------------- decode

def run_decode(lengths, q, kc, vc, scale):
    o, lse = cpa.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lengths.to(DEV), scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def test_decode_full_workload_with_poisoned_tail():
    w = synth.MIXTRAL_8X22B_DECODE
    announce(f"decode {w.name} (NaN beyond each length)")
    lengths, q, kc, vc = synth.workload_decode_inputs(w)
    O_ref, L_ref = oatt.decode_ref(q, kc, vc, lengths.numpy(), w.scale)
    for b in range(w.batch):
        kc[b, :, lengths[b]:] = float("nan")
        vc[b, :, lengths[b]:] = float("nan")
    o, lse = run_decode(lengths, q, kc, vc, w.scale)
    assert_close(o, O_ref, 2e-2, "decode O")
    assert_close(lse, L_ref, 2e-2, "decode LSE")


@pytest.mark.parametrize("batch,hq,hkv,d,max_len,dtype,lens", [
    (4, 48, 8, 128, 2048, torch.bfloat16, [1, 2048, 256, 257]),
    (3, 16, 1, 128, 300, torch.bfloat16, [300, 1, 255]),     # G=16: two P V groups of 8
    (2, 9, 1, 128, 513, torch.bfloat16, [513, 257]),          # G=9: P V groups of 5 and 4
    (3, 24, 2, 128, 800, torch.bfloat16, [800, 1, 256]),      # G=12: groups of 6 and 6
    (2, 26, 2, 128, 600, torch.bfloat16, [600, 299]),         # G=13: groups of 7 and 6
    (2, 17, 1, 128, 300, torch.bfloat16, [300, 45]),          # G=17: matrix-core kernel, blocks of 16 + 1
    (2, 32, 1, 128, 1000, torch.bfloat16, [1000, 513]),       # G=32: two full head blocks
    (3, 96, 2, 128, 700, torch.bfloat16, [700, 1, 257]),      # G=48, two kv heads
    (2, 20, 1, 128, 64, torch.float32, [64, 33]),             # fp32, G=20: the generic kernel
    (5, 160, 5, 128, 900, torch.bfloat16, [900, 1, 256, 257, 613]),  # 25 (sequence, kv head) pairs
    (3, 32, 4, 64, 2048, torch.bfloat16, [2048, 1, 1500]),    # D=64, G=8: 8 lanes per V row
    (3, 24, 2, 64, 300, torch.bfloat16, [300, 17, 256]),      # D=64, G=12: the generic kernel
    (2, 8, 8, 64, 513, torch.float32, [513, 17]),
    (5, 12, 4, 64, 1000, torch.bfloat16, [999, 1000, 512, 3, 768]),
    (2, 4, 2, 128, 64, torch.float32, [64, 33]),
    # caches up to 1024 keys take 128-key splits in the v_dot2 kernels, longer ones 256
    (3, 12, 2, 128, 1024, torch.bfloat16, [1024, 128, 129]),
    (3, 12, 2, 128, 1025, torch.bfloat16, [1025, 1024, 1]),
    (2, 8, 2, 64, 128, torch.bfloat16, [128, 127]),
    (2, 8, 2, 64, 129, torch.bfloat16, [129, 128]),
    # 12 kv heads: workgroups are placed by kv head on 8 XCDs, so heads 8..11 form a second group
    (2, 24, 12, 128, 700, torch.bfloat16, [700, 300]),
    (2, 36, 12, 64, 200, torch.float32, [200, 1]),
])
def test_decode_edge_lengths(batch, hq, hkv, d, max_len, dtype, lens):
    announce(f"decode B={batch} Hq={hq} Hkv={hkv} D={d} Lmax={max_len} {dtype} lens={lens}")
    lengths, q, kc, vc = synth.decode_inputs(batch, hq, hkv, d, max_len, 1, max_len, dtype, seed=batch + d)
    lengths = torch.tensor(lens, dtype=torch.int32)
    scale = 1.0 / math.sqrt(d)
    O_ref, L_ref = oatt.decode_ref(q, kc, vc, lengths.numpy(), scale)
    for b in range(batch):
        kc[b, :, lens[b]:] = float("nan")
        vc[b, :, lens[b]:] = float("nan")
    o, lse = run_decode(lengths, q, kc, vc, scale)
    tol = TOL[dtype]
    assert_close(o, O_ref, tol, "decode O")
    assert_close(lse, L_ref, tol, "decode LSE")


def test_decode_llama405b_shape():
    """Llama3.1-405B-shaped decode (128 query heads over 8 kv heads, G = 16, D = 128) over
    8 sequences of mixed length up to 4096, NaN past every length."""
    announce("decode Llama3.1-405B shape: B=8, Hq=128, Hkv=8, D=128, Lmax=4096")
    lengths, q, kc, vc = synth.decode_inputs(8, 128, 8, 128, 4096, 1, 4096, torch.bfloat16, seed=405)
    lengths[0] = 4096
    scale = 1.0 / math.sqrt(128)
    O_ref, L_ref = oatt.decode_ref(q, kc, vc, lengths.numpy(), scale)
    for b in range(8):
        kc[b, :, lengths[b]:] = float("nan")
        vc[b, :, lengths[b]:] = float("nan")
    o, lse = run_decode(lengths, q, kc, vc, scale)
    assert_close(o, O_ref, 2e-2, "decode O")
    assert_close(lse, L_ref, 2e-2, "decode LSE")


def test_decode_llama32_1b_shape():
    """Llama3.2-1B-shaped decode (32 query heads over 8 kv heads, head dim 64) over 16
    sequences of mixed length up to 4096, NaN past every length."""
    announce("decode Llama3.2-1B shape: B=16, Hq=32, Hkv=8, D=64, Lmax=4096")
    lengths, q, kc, vc = synth.decode_inputs(16, 32, 8, 64, 4096, 1, 4096, torch.bfloat16, seed=321)
    lengths[3] = 4096
    scale = 1.0 / math.sqrt(64)
    O_ref, L_ref = oatt.decode_ref(q, kc, vc, lengths.numpy(), scale)
    for b in range(16):
        kc[b, :, lengths[b]:] = float("nan")
        vc[b, :, lengths[b]:] = float("nan")
    o, lse = run_decode(lengths, q, kc, vc, scale)
    assert_close(o, O_ref, 2e-2, "decode O")
    assert_close(lse, L_ref, 2e-2, "decode LSE")


def test_decode_zero_length():
    """A length of 0 (an empty cache slice) gives O = 0 and LSE = -inf; other rows unchanged."""
    announce("decode with a zero length")
    lengths, q, kc, vc = synth.decode_inputs(3, 12, 4, 128, 300, 1, 300, torch.bfloat16, seed=9)
    lengths = torch.tensor([0, 300, 41], dtype=torch.int32)
    o, lse = run_decode(lengths, q, kc, vc, 1.0 / math.sqrt(128))
    assert np.all(np.asarray(o)[0] == 0.0) and np.all(np.asarray(lse)[0] == -np.inf)
    O_ref, L_ref = oatt.decode_ref(q, kc, vc, lengths.numpy(), 1.0 / math.sqrt(128))
    assert_close(np.asarray(o)[1:], O_ref[1:], 2e-2, "decode O (non-empty rows)")
    assert_close(np.asarray(lse)[1:], L_ref[1:], 2e-2, "decode LSE (non-empty rows)")


@pytest.mark.parametrize("shape", ["mixtral-8x22b-b24", "fp32-small"])
def test_decode_length_sharded_merge(shape):
    """A cache split along its length into R shards (inference context parallelism): decode on
    each shard's own cache slice, then gqa_decode_merge, against one oracle decode over the whole
    cache. Short sequences leave later shards empty."""
    if shape == "mixtral-8x22b-b24":
        w = synth.MIXTRAL_8X22B_DECODE
        lengths, q, kc, vc = synth.workload_decode_inputs(w)
        scale, R, tol = w.scale, 4, 2e-2
    else:
        lengths, q, kc, vc = synth.decode_inputs(3, 8, 2, 64, 96, 1, 96, torch.float32, seed=13)
        lengths = torch.tensor([96, 33, 5], dtype=torch.int32)
        scale, R, tol = 0.125, 3, 1e-4
    Lmax = kc.shape[2]
    W = Lmax // R
    announce(f"length-sharded decode {shape}: {R} shards of {W}")
    o_parts, l_parts = [], []
    for r in range(R):
        n = torch.clamp(lengths - r * W, 0, W).to(torch.int32)
        o, lse = cpa.decode(q.to(DEV), kc[:, :, r * W:(r + 1) * W].contiguous().to(DEV),
                            vc[:, :, r * W:(r + 1) * W].contiguous().to(DEV), n.to(DEV), scale=scale)
        o_parts.append(o)
        l_parts.append(lse)
    O, L = cpa.decode_merge(torch.stack(o_parts), torch.stack(l_parts))
    torch.cuda.synchronize()
    O_ref, L_ref = oatt.decode_ref(q, kc, vc, lengths.numpy(), scale)
    assert_close(O.float().cpu().numpy(), O_ref, tol, f"sharded decode O ({shape})")
    assert_close(L.cpu().numpy(), L_ref, tol, f"sharded decode LSE ({shape})")


@pytest.mark.parametrize("R,B,Hq,D,dtype", [
    (1, 3, 5, 128, torch.bfloat16),
    (4, 24, 48, 128, torch.bfloat16),   # the length-sharded Mixtral decode's merge
    (8, 2, 6, 64, torch.float32),
    (5, 2, 3, 200, torch.bfloat16),     # D not a multiple of 64: threads past it store nothing
    (9, 2, 4, 128, torch.float32),      # more parts than the unrolled kernel takes
    (3, 2, 3, 300, torch.float32),      # D above 256
])
def test_decode_merge_against_oracle(R, B, Hq, D, dtype):
    """gqa_decode_merge on random partials against the oracle's merge: some parts empty
    (log-sum-exp -inf) with NaN in their outputs, which must not reach the result, and one
    (b, h) with every part empty (O = 0, LSE = -inf)."""
    announce(f"decode merge R={R} B={B} Hq={Hq} D={D} {dtype}")
    g = torch.Generator().manual_seed(R * 1000 + D)
    o = torch.randn((R, B, Hq, D), generator=g).to(dtype)
    lse = (torch.rand((R, B, Hq), generator=g) * 10 - 5).float()
    empty = torch.rand((R, B, Hq), generator=g) < 0.3
    empty[:, 0, 0] = True  # every part of (0, 0) empty
    if R > 1:
        empty[0, 1, 0] = False
        empty[1:, 1, 0] = True  # (1, 0): one live part
    lse[empty] = -float("inf")
    o[empty] = float("nan")
    O, L = cpa.decode_merge(o.to(DEV), lse.to(DEV))
    torch.cuda.synchronize()
    O_ref, L_ref = oatt.decode_merge_ref(o, lse)
    tol = TOL[dtype]
    assert_close(O.float().cpu().numpy(), O_ref, tol, "merge O")
    Lg = L.cpu().numpy()
    assert np.isneginf(Lg[0, 0]) and np.isneginf(L_ref[0, 0])
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(Lg), fin)
    assert_close(Lg[fin], L_ref[fin], tol, "merge LSE")


def test_decode_workspace_reuse():
    """One workspace (garbage-filled) serves repeated calls and a smaller batch afterwards."""
    announce("decode workspace reuse")
    B, hq, hkv, d, lmax = 6, 12, 2, 128, 700
    ws = torch.full((cpa.decode_workspace_bytes(B, hq, hkv, lmax, d),), 0x7F, dtype=torch.uint8, device=DEV)
    for it, (b, seed) in enumerate([(6, 31), (6, 32), (3, 33)]):
        lengths, q, kc, vc = synth.decode_inputs(b, hq, hkv, d, lmax, 1, lmax, torch.bfloat16, seed=seed)
        o, lse = cpa.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), lengths.to(DEV), workspace=ws)
        torch.cuda.synchronize()
        O_ref, L_ref = oatt.decode_ref(q, kc, vc, lengths.numpy(), 1.0 / math.sqrt(d))
        assert_close(o.float().cpu().numpy(), O_ref, 2e-2, f"decode O call {it}")
        assert_close(lse.cpu().numpy(), L_ref, 2e-2, f"decode LSE call {it}")


# ----------------------------------------------------------------------------- int8 cache

from oracle import quant as oq  # noqa: E402


@pytest.mark.parametrize("rows,d,dtype", [
    (24 * 8 * 64, 128, torch.bfloat16),   # 64 cache positions of the Mixtral-shaped cache
    (1000, 128, torch.float32),
    (37, 64, torch.bfloat16),
    (5, 100, torch.float32),              # a row length that is not a multiple of the wave
    (3, 1, torch.bfloat16),
])
def test_quantize_bit_exact(rows, d, dtype):
    """Codes and scales of the HIP quantizer equal the oracle's bit for bit (both take every
    rounding decision in float32). Includes zero rows, rows with one large outlier and a row whose
    absmax is negative."""
    announce(f"kv quantize rows={rows} d={d} {dtype}")
    gen = torch.Generator("cpu").manual_seed(rows + d)
    x = (torch.randn((rows, d), generator=gen) * torch.rand((rows, 1), generator=gen) * 8).to(dtype)
    x[0] = 0
    if rows > 2:
        x[1, d // 2] = -1000.0
        x[2] = x[2].abs()
        x[2, 0] = -3 * x[2].abs().max()
    codes, scales = cpa.quantize_kv(x.to(DEV))
    torch.cuda.synchronize()
    c_ref, s_ref = oq.kv_quantize_ref(x)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    bad = int((got_c != c_ref).sum())
    print(f"  code mismatches {bad}, scale mismatches {int((got_s != s_ref).sum())}", flush=True)
    assert bad == 0
    assert np.array_equal(got_s.view(np.uint32), s_ref.view(np.uint32))


def run_decode_int8(lengths, q, kq, ks, vq, vs, scale, workspace=None):
    o, lse = cpa.decode_int8(q.to(DEV), kq.to(DEV), ks.to(DEV), vq.to(DEV), vs.to(DEV), lengths.to(DEV),
                             scale=scale, workspace=workspace)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def test_decode_int8_full_workload_with_poisoned_tail():
    """Mixtral-8x22B-shaped decode batch over an int8 cache; scales past each length are NaN and
    codes there are -128 (a value the quantizer never writes): neither may leak into the result."""
    w = synth.MIXTRAL_8X22B_DECODE
    announce(f"int8 decode {w.name} (poisoned beyond each length)")
    lengths, q, kq, ks, vq, vs = synth.workload_decode_int8_inputs(w)
    O_ref, L_ref = oq.decode_int8_ref(q, kq, ks, vq, vs, lengths.numpy(), w.scale)
    for b in range(w.batch):
        n = int(lengths[b])
        ks[b, :, n:] = float("nan")
        vs[b, :, n:] = float("nan")
        kq[b, :, n:] = -128
        vq[b, :, n:] = -128
    o, lse = run_decode_int8(lengths, q, kq, ks, vq, vs, w.scale)
    assert_close(o, O_ref, 2e-2, "int8 decode O")
    assert_close(lse, L_ref, 2e-2, "int8 decode LSE")


@pytest.mark.parametrize("batch,hq,hkv,max_len,lens", [
    (4, 48, 8, 2048, [1, 2048, 256, 257]),
    (3, 16, 1, 300, [300, 1, 255]),          # G = 16: one full head block
    (2, 40, 2, 513, [513, 17]),              # G = 20: two head blocks, the second partial
    (2, 64, 2, 130, [64, 130]),              # G = 32
    (5, 12, 4, 1000, [999, 1000, 512, 3, 768]),
    (2, 1, 1, 1, [1, 1]),                    # one key, one head
    (2, 36, 12, 600, [600, 129]),            # 12 kv heads: a second group of kv heads per XCD
])
def test_decode_int8_edge_lengths(batch, hq, hkv, max_len, lens):
    announce(f"int8 decode B={batch} Hq={hq} Hkv={hkv} Lmax={max_len} lens={lens}")
    lengths, q, kq, ks, vq, vs = synth.decode_int8_inputs(batch, hq, hkv, 128, max_len, 1, max_len,
                                                          seed=batch + hq + max_len)
    lengths = torch.tensor(lens, dtype=torch.int32)
    scale = 1.0 / math.sqrt(128)
    O_ref, L_ref = oq.decode_int8_ref(q, kq, ks, vq, vs, lengths.numpy(), scale)
    for b in range(batch):
        ks[b, :, lens[b]:] = float("nan")
        vs[b, :, lens[b]:] = float("nan")
    o, lse = run_decode_int8(lengths, q, kq, ks, vq, vs, scale)
    assert_close(o, O_ref, 2e-2, "int8 decode O")
    assert_close(lse, L_ref, 2e-2, "int8 decode LSE")


def test_decode_int8_zero_length_and_workspace_reuse():
    """Length 0 gives O = 0, LSE = -inf; a garbage-filled workspace serves two calls in a row,
    the second with a smaller batch."""
    announce("int8 decode: zero length, workspace reuse")
    B, hq, hkv, lmax = 4, 24, 4, 700
    ws = torch.full((cpa.decode_workspace_bytes(B, hq, hkv, lmax, 128),), 0x7F, dtype=torch.uint8, device=DEV)
    for it, (b, seed) in enumerate([(4, 51), (2, 52)]):
        lengths, q, kq, ks, vq, vs = synth.decode_int8_inputs(b, hq, hkv, 128, lmax, 1, lmax, seed=seed)
        lengths[0] = 0
        o, lse = run_decode_int8(lengths, q, kq, ks, vq, vs, 1.0 / math.sqrt(128), workspace=ws)
        assert np.all(o[0] == 0.0) and np.all(lse[0] == -np.inf)
        O_ref, L_ref = oq.decode_int8_ref(q, kq, ks, vq, vs, lengths.numpy(), 1.0 / math.sqrt(128))
        assert_close(o[1:], O_ref[1:], 2e-2, f"int8 decode O call {it}")
        assert_close(lse[1:], L_ref[1:], 2e-2, f"int8 decode LSE call {it}")


def test_quantize_then_decode_int8():
    """The cache-writer path: a bf16 cache quantized on the GPU and decoded from its codes, against
    the oracle's own quantization and decode of the same bf16 cache."""
    announce("quantize bf16 cache then int8 decode")
    lengths, q, kc, vc = synth.decode_inputs(6, 48, 8, 128, 1100, 1, 1100, torch.bfloat16, seed=61)
    kq, ks = cpa.quantize_kv(kc.to(DEV))
    vq, vs = cpa.quantize_kv(vc.to(DEV))
    o, lse = cpa.decode_int8(q.to(DEV), kq, ks, vq, vs, lengths.to(DEV))
    torch.cuda.synchronize()
    kq_r, ks_r = oq.kv_quantize_ref(kc)
    vq_r, vs_r = oq.kv_quantize_ref(vc)
    O_ref, L_ref = oq.decode_int8_ref(q, kq_r, ks_r, vq_r, vs_r, lengths.numpy(), 1.0 / math.sqrt(128))
    assert_close(o.float().cpu().numpy(), O_ref, 2e-2, "quantize + int8 decode O")
    assert_close(lse.cpu().numpy(), L_ref, 2e-2, "quantize + int8 decode LSE")


# ----------------------------------------------------------------------------- backward

from oracle import backward as obw  # noqa: E402


def run_bwd_rank(qd, kd, vd, dod, seq, cp, rank, scale, kp=None, vp=None):
    """GPU: permute the shard's Q and dO and the full K/V, forward, then backward."""
    c = seq // (2 * cp)
    if kp is None:
        kp, vp = cpa.permute(kd, cp), cpa.permute(vd, cp)
    qs = cpa.permute(qd, cp, row_begin=rank * 2 * c, row_count=2 * c)
    dos = cpa.permute(dod, cp, row_begin=rank * 2 * c, row_count=2 * c)
    o, lse = cpa.attention_fwd(qs, kp, vp, cp, rank, scale=scale)
    dq, dk, dv = cpa.attention_bwd(qs, kp, vp, o, lse, dos, cp, rank, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_bwd_full(batch, seq, cp, hq, hkv, d, ranks, seed, tag, d_v=None):
    d_v = d if d_v is None else d_v
    q, k, v = synth.prefill_inputs(batch, seq, hq, hkv, d, d_v, torch.bfloat16, seed)
    do = synth.prefill_grad(batch, seq, hq, d_v, torch.bfloat16, seed + 1000)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    kp, vp = cpa.permute(kd, cp), cpa.permute(vd, cp)
    perm = olb.load_balance_perm(seq, cp)
    scale = 1.0 / math.sqrt(d)
    c = seq // (2 * cp)
    for r in ranks:
        announce(f"backward {tag} cp={cp} rank={r}")
        dq, dk, dv = run_bwd_rank(qd, kd, vd, dod, seq, cp, r, scale, kp, vp)
        rows = perm[r * 2 * c:(r + 1) * 2 * c]
        dq_r, dk_r, dv_r = obw.causal_attention_bwd_ref(q[:, rows], k[:, perm], v[:, perm], do[:, rows], rows, perm,
                                                        scale)
        assert_close(dq.cpu().numpy(), dq_r, bwd_tol(dq_r), f"dQ {tag} r{r}")
        assert_close(dk.cpu().numpy(), dk_r, bwd_tol(dk_r), f"dK {tag} r{r}")
        assert_close(dv.cpu().numpy(), dv_r, bwd_tol(dv_r), f"dV {tag} r{r}")


@pytest.mark.parametrize("batch,seq,cp,hq,hkv,d,ranks", [
    (1, 512, 2, 4, 2, 64, (0, 1)),
    (2, 400, 2, 4, 1, 128, (0, 1)),     # c = 100: partial key tiles and query blocks
    (1, 1024, 4, 16, 2, 128, (0, 3)),   # G = 8
    (1, 256, 1, 2, 2, 64, (0,)),        # cp = 1: plain causal attention
])
def test_backward_small(batch, seq, cp, hq, hkv, d, ranks):
    check_bwd_full(batch, seq, cp, hq, hkv, d, ranks, seed=seq + hq, tag=f"B{batch} S{seq} Hq{hq}/{hkv} D{d}")


def test_backward_mla_shape_small():
    """MLA-style head dims (q/k 192 = 128 + 64 rotary, v 128) at a small size, both ranks."""
    check_bwd_full(1, 768, 2, 4, 4, 192, (0, 1), seed=23, tag="MLA Dqk192 Dv128", d_v=128)


@pytest.mark.parametrize("batch,seq,hq,hkv,ranks", [
    (1, 640, 8, 2, (0, 1)),  # G = 4, c = 160: two 64-key tiles and a 32-key tail per chunk
    (2, 312, 6, 3, (1,)),    # G = 2, batch 2, c = 78
    (1, 388, 4, 2, (0, 1)),  # c = 97: one 64-key tile and a 33-key tail per chunk
])
def test_backward_mla_dims_grouped_heads(batch, seq, hq, hkv, ranks):
    """Dqk 192, Dv 128 with several query heads per kv head: the dkdv kernel at these head dims
    walks the query heads of its kv head inside its stage loop, and dq reads the shared K/V."""
    check_bwd_full(batch, seq, 2, hq, hkv, 192, ranks, seed=seq + 7 * hq, d_v=128,
                   tag=f"B{batch} S{seq} Hq{hq}/{hkv} Dqk192 Dv128")


def test_backward_contiguous_shard_positions():
    """Explicit q_positions: a contiguous (unbalanced) shard of the natural order, K/V natural."""
    seq, hq, hkv, d = 512, 4, 2, 64
    q, k, v = synth.prefill_inputs(1, seq, hq, hkv, d, d, torch.bfloat16, 17)
    do = synth.prefill_grad(1, seq, hq, d, torch.bfloat16, 18)
    rows = np.arange(256, 512)
    pos = torch.tensor(rows, dtype=torch.int32, device=DEV)
    announce("backward contiguous shard with explicit positions")
    qs, dos = q[:, 256:].contiguous().to(DEV), do[:, 256:].contiguous().to(DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    o, lse = cpa.attention_fwd(qs, kd, vd, 1, 0, q_positions=pos, scale=0.125)
    dq, dk, dv = cpa.attention_bwd(qs, kd, vd, o, lse, dos, 1, 0, q_positions=pos, scale=0.125)
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = obw.causal_attention_bwd_ref(q[:, 256:], k, v, do[:, 256:], rows, np.arange(seq), 0.125)
    assert_close(dq.cpu().numpy(), dq_r, bwd_tol(dq_r), "dQ contiguous")
    assert_close(dk.cpu().numpy(), dk_r, bwd_tol(dk_r), "dK contiguous")
    assert_close(dv.cpu().numpy(), dv_r, bwd_tol(dv_r), "dV contiguous")


def test_backward_llama7b_s8192():
    w = synth.LLAMA2_7B_S8K
    check_bwd_full(w.batch, w.seq, 4, w.hq, w.hkv, w.d_qk, (0, 3), seed=w.seed, tag=w.name)


def sampled_bwd_check(w, cp, rank):
    """One rank at its real shape. dQ on sampled rows; dK, dV at the keys of the last 48
    positions of the rank's upper chunk (seen only by the rank's rows at those positions, all of
    which are in the sample); keys past the rank's last position are exactly 0; and dK sums to ~0
    over the keys of each kv head (the softmax gradient sums to zero)."""
    S = w.seq
    c = S // (2 * cp)
    announce(f"backward {w.name} rank {rank} (sampled)")
    q, k, v = synth.workload_prefill_inputs(w)
    do = synth.workload_prefill_grad(w)
    perm = olb.load_balance_perm(S, cp)
    scale = w.scale
    dq, dk, dv = run_bwd_rank(q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), S, cp, rank, scale)
    shard = perm[rank * 2 * c:(rank + 1) * 2 * c]
    top = (2 * cp - rank) * c            # one past the rank's last position
    p0 = top - 48
    rng = np.random.default_rng(rank)
    sel = np.unique(np.concatenate([np.arange(2 * c - 48, 2 * c), rng.integers(0, 2 * c, 8)]))
    rows = shard[sel]
    dq_r, dk_r, dv_r = obw.causal_attention_bwd_ref(q[:, rows], k[:, perm], v[:, perm], do[:, rows], rows, perm, scale)
    assert_close(dq[:, sel].cpu().numpy(), dq_r, bwd_tol(dq_r), f"dQ rank {rank} sampled rows")
    inv = olb.inverse_perm(perm)
    keys = inv[p0:top]
    assert_close(dk[:, keys].cpu().numpy(), dk_r[:, keys], bwd_tol(dk_r[:, keys]), f"dK rank {rank} last keys")
    assert_close(dv[:, keys].cpu().numpy(), dv_r[:, keys], bwd_tol(dv_r[:, keys]), f"dV rank {rank} last keys")
    if top < S:
        later = inv[top:S:997]
        assert float(dk[:, later].abs().max()) == 0.0 and float(dv[:, later].abs().max()) == 0.0
    ssum = dk.sum(dim=1).abs().max().item()
    scale_ref = dk.abs().sum(dim=1).max().item()
    print(f"  sum_j dK_j: max |.| {ssum:.3e} against max sum_j |dK_j| {scale_ref:.3e}", flush=True)
    assert ssum <= 1e-2 * scale_ref


@pytest.mark.parametrize("rank", [0, 3])
def test_backward_deepseek_mla_full_size_sampled(rank):
    sampled_bwd_check(synth.DEEPSEEK_V3_MLA_S32K, 4, rank)


@pytest.mark.parametrize("rank", [0, 7])
def test_backward_llama70b_full_size_sampled(rank):
    sampled_bwd_check(synth.LLAMA31_70B_S131K, 8, rank)


def test_backward_llama70b_identical_keys_every_key():
    """Every key's dV and dK and every row's dQ of ranks 0 and 7 at the 131072-token shape,
    against closed forms (dK: check_identical_keys_dk). With all keys of a kv head equal (k_j = k_g, the natural-order row 0), each visible key
    gets probability 1/(pos_i + 1) in row i, so dV_j is the sum, over the rank's rows i with
    pos_i >= kpos_j and over the G query heads of the group, of dO_i / (pos_i + 1): a suffix sum
    over the rows in position order. dQ is 0: dQ_i = scale * k_g * sum_j dS_ij, and the dS of a
    row sums to zero. Tolerance as for the other backward checks, 2e-2 * max(1, max |ref|)."""
    w = synth.LLAMA31_70B_S131K
    cp, S = w.cps[0], w.seq
    announce(f"backward {w.name} identical keys, every key: generating inputs")
    q, k, v = synth.workload_prefill_inputs(w)
    do = synth.workload_prefill_grad(w)
    qd, vd, dod = q.to(DEV), v.to(DEV), do.to(DEV)
    k1d = k[:, :1].expand(-1, S, -1, -1).contiguous().to(DEV)
    kp, vp = cpa.permute(k1d, cp), cpa.permute(vd, cp)
    for rank in (0, 7):
        announce(f"backward {w.name} identical keys, every key: rank {rank}")
        dq, dk, dv = run_bwd_rank(qd, k1d, vd, dod, S, cp, rank, w.scale, kp, vp)
        check_identical_keys_bwd(w, cp, rank, do, dq, dv)
        check_identical_keys_dk(w, cp, rank, q, v, do, dk)


def test_backward_mla_identical_keys_every_key():
    """The DeepSeek-V3 MLA shape (Dqk 192, Dv 128, 128 kv heads), ranks 0 and 3 at cp = 4: every
    key's dV and every row's dQ against the identical-key closed forms (dK there is covered by
    the sampled check; its row-by-row closed form over 128 kv heads is too slow for the suite)."""
    w = synth.DEEPSEEK_V3_MLA_S32K
    cp, S = w.cps[0], w.seq
    announce(f"backward {w.name} identical keys, every key: generating inputs")
    q, k, v = synth.workload_prefill_inputs(w)
    do = synth.workload_prefill_grad(w)
    qd, vd, dod = q.to(DEV), v.to(DEV), do.to(DEV)
    k1d = k[:, :1].expand(-1, S, -1, -1).contiguous().to(DEV)
    kp, vp = cpa.permute(k1d, cp), cpa.permute(vd, cp)
    for rank in (0, cp - 1):
        announce(f"backward {w.name} identical keys, every key: rank {rank}")
        dq, dk, dv = run_bwd_rank(qd, k1d, vd, dod, S, cp, rank, w.scale, kp, vp)
        check_identical_keys_bwd(w, cp, rank, do, dq, dv)
