"""Seeded sweep of random shapes against the oracle, beside the hand-picked cases: odd context
parallel degrees (3, 5, 6), query-to-kv head ratios from 1 to 16, ragged chunk lengths (down
to one token), batches of 1 to 3, every supported head-dim pair and both dtypes, for the
forward (with and without the split of heavy row blocks), the backward and the bf16, fp32 and
int8-cache decodes. The shapes are drawn once from a fixed seed, so every run checks the same
ones, and each case prints its shape before it runs. Tolerances are those of the other parity
tests: 1e-4 for fp32, 2e-2 for bf16, 2e-2 * max(1, max |ref|) for the gradients."""

import math

import numpy as np
import pytest
import torch

import context_causal_attention_load_amd as cpa
from context_causal_attention_load_amd import synth
from oracle import attention as oatt
from oracle import quant as oq

from gpu_util import DEV, TOL, Prefill, announce, assert_close, check_rank
from test_gpu_parity import check_bwd_full

pytestmark = pytest.mark.gpu

BF16_DIMS = [(64, 64), (128, 128), (192, 128)]
F32_DIMS = [(64, 64), (128, 128)]


def _prefill_cases(n, seed, bf16_only=False):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = torch.bfloat16 if bf16_only or rng.random() < 0.75 else torch.float32
        dims = BF16_DIMS if dtype == torch.bfloat16 else F32_DIMS
        dqk, dv = dims[rng.integers(len(dims))]
        cp = int(rng.choice([1, 2, 3, 4, 5, 6, 8]))
        c = int(rng.choice([1, 2, 31, 32, 33, int(rng.integers(3, 129))]))
        hkv = int(rng.integers(1, 5))
        g = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
        while hkv * g > 32:
            g //= 2
        batch = int(rng.choice([1, 1, 2, 3]))
        ranks = list(range(cp)) if cp <= 4 else sorted({0, cp // 2, cp - 1})
        name = f"s{i}-{'bf16' if dtype == torch.bfloat16 else 'f32'}-d{dqk}-cp{cp}-c{c}-hq{hkv * g}-hkv{hkv}-b{batch}"
        cases.append((name, batch, 2 * cp * c, cp, hkv * g, hkv, dqk, dv, dtype, 1000 + i, ranks))
    return cases


FWD_CASES = _prefill_cases(24, seed=20261203)
BWD_CASES = _prefill_cases(8, seed=20261204, bf16_only=True)


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_attention_random_shapes(case):
    name, batch, seq, cp, hq, hkv, dqk, dv, dtype, seed, ranks = case
    pf = Prefill(batch, seq, hq, hkv, dqk, dv, dtype, seed)
    for r in ranks:
        check_rank(pf, cp, r, tag=name)
        if dtype == torch.bfloat16:
            check_rank(pf, cp, r, tag=name, split=False)


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_random_shapes(case):
    name, batch, seq, cp, hq, hkv, dqk, dv, dtype, seed, ranks = case
    check_bwd_full(batch, seq, cp, hq, hkv, dqk, ranks, seed, name, d_v=dv)


def _decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 13))
        g = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
        while hkv * g > 96:
            g //= 2
        batch = int(rng.integers(1, 7))
        max_len = int(rng.choice([1, 255, 256, 257, int(rng.integers(2, 3000))]))
        lens = rng.integers(0, max_len + 1, batch)
        lens[rng.integers(batch)] = max_len
        name = f"d{i}-{'bf16' if dtype == torch.bfloat16 else 'f32'}-D{d}-hq{hkv * g}-hkv{hkv}-b{batch}-L{max_len}"
        cases.append((name, batch, hkv * g, hkv, d, max_len, dtype, [int(x) for x in lens], 2000 + i))
    return cases


DEC_CASES = _decode_cases(12, seed=20261205)


@pytest.mark.parametrize("case", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_decode_random_shapes(case):
    """bf16 or fp32 decode with NaN past every length; with bf16 queries and D = 128, also the
    int8-cache decode over the oracle's quantization of the same cache."""
    name, batch, hq, hkv, d, max_len, dtype, lens, seed = case
    announce(f"{name} lens={lens}")
    _, q, kc, vc = synth.decode_inputs(batch, hq, hkv, d, max_len, 1, max_len, dtype, seed=seed)
    lengths = torch.tensor(lens, dtype=torch.int32)
    scale = 1.0 / math.sqrt(d)
    O_ref, L_ref = oatt.decode_ref(q, kc, vc, lengths.numpy(), scale)
    kcn, vcn = kc.clone(), vc.clone()
    for b in range(batch):
        kcn[b, :, lens[b]:] = float("nan")
        vcn[b, :, lens[b]:] = float("nan")
    o, lse = cpa.decode(q.to(DEV), kcn.to(DEV), vcn.to(DEV), lengths.to(DEV), scale=scale)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    empty = np.array(lens) == 0
    assert np.all(o[empty] == 0.0) and np.all(lse[empty] == -np.inf)
    tol = TOL[dtype]
    assert_close(o[~empty], O_ref[~empty], tol, f"{name} decode O")
    assert_close(lse[~empty], L_ref[~empty], tol, f"{name} decode LSE")
    if dtype == torch.bfloat16 and d == 128:
        kq, ks = oq.kv_quantize_ref(kc)
        vq, vs = oq.kv_quantize_ref(vc)
        O8, L8 = oq.decode_int8_ref(q, kq, ks, vq, vs, lengths.numpy(), scale)
        o8, lse8 = cpa.decode_int8(q.to(DEV), torch.from_numpy(kq).to(DEV), torch.from_numpy(ks).to(DEV),
                                   torch.from_numpy(vq).to(DEV), torch.from_numpy(vs).to(DEV), lengths.to(DEV),
                                   scale=scale)
        torch.cuda.synchronize()
        o8, lse8 = o8.float().cpu().numpy(), lse8.cpu().numpy()
        assert np.all(o8[empty] == 0.0) and np.all(lse8[empty] == -np.inf)
        assert_close(o8[~empty], O8[~empty], 2e-2, f"{name} int8 decode O")
        assert_close(lse8[~empty], L8[~empty], 2e-2, f"{name} int8 decode LSE")
