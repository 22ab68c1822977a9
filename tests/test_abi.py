"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, its host
index helper agrees with the oracle's independent construction, and every argument check
fails with the documented status before any HIP call."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import context_causal_attention_load_amd as cpa
from context_causal_attention_load_amd import binding
from oracle import lb_index as olb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cpa.library_path()):
        from context_causal_attention_load_amd import build

        build.build()
    return cpa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("cp_load_balance_permute", "cp_load_balance_unpermute", "cp_attention_fwd",
                 "cp_attention_fwd_ws", "cp_attention_fwd_workspace_bytes", "gqa_decode_attention_noalloc",
                 "gqa_decode_attention", "gqa_decode_workspace_bytes", "cpattn_last_error",
                 "cp_load_balance_source_index", "cp_load_balance_positions", "gqa_decode_merge",
                 "gqa_decode_attention_int8kv", "kv_cache_quantize_int8", "cp_attention_bwd",
                 "cp_attention_bwd_workspace_bytes", "cp_attention_bwd_split_workspace_bytes"):
        assert must in names, names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(cpa.library_path())
    for name in declared_functions():
        assert hasattr(raw, name), f"missing export {name}"


@pytest.mark.parametrize("seq,cp", [(8, 1), (8, 2), (8, 4), (96, 3), (512, 2), (8192, 4), (131072, 8)])
def test_source_index_matches_oracle(lib, seq, cp):
    perm = olb.load_balance_perm(seq, cp)
    got = cpa.lb_positions(seq, cp).numpy()
    assert np.array_equal(got, perm)
    for r in range(cp):
        b0, b1 = olb.shard_row_range(seq, cp, r)
        assert np.array_equal(cpa.lb_positions(seq, cp, b0, b1 - b0).numpy(), olb.shard_positions(seq, cp, r))
    for j in (0, seq // 2, seq - 1):
        assert cpa.lb_source_index(seq, cp, j) == perm[j]


def test_source_index_rejects(lib):
    assert lib.cp_load_balance_source_index(10, 2, 0) == -1
    assert lib.cp_load_balance_source_index(8, 0, 0) == -1
    assert lib.cp_load_balance_source_index(8, 2, 8) == -1
    assert lib.cp_load_balance_source_index(8, 2, -1) == -1


FAKE = ctypes.c_void_p(4096)  # never dereferenced: every call below fails its host checks first


def _status_and_message(lib, rc):
    return rc, lib.cpattn_last_error().decode()


@pytest.mark.parametrize("args,substr", [
    ((FAKE, ctypes.c_void_p(1 << 20), 1, 10, 16, 2, 0, 10, None), "multiple of 2*cp"),
    ((FAKE, ctypes.c_void_p(1 << 20), 1, 8, 16, 0, 0, 8, None), "cp must be"),
    ((FAKE, ctypes.c_void_p(1 << 20), 1, 8, 0, 2, 0, 8, None), "row_bytes"),
    ((FAKE, ctypes.c_void_p(1 << 20), 1, 8, 16, 2, 4, 8, None), "window"),
    ((FAKE, ctypes.c_void_p(1 << 20), 1, 8, 16, 2, -1, 2, None), "window"),
    ((None, ctypes.c_void_p(1 << 20), 1, 8, 16, 2, 0, 8, None), "null"),
    ((FAKE, ctypes.c_void_p(4096 + 64), 1, 8, 16, 2, 0, 8, None), "overlap"),
    ((FAKE, ctypes.c_void_p(1 << 20), -1, 8, 16, 2, 0, 8, None), "outer"),
])
def test_permute_argument_errors(lib, args, substr):
    for fn in (lib.cp_load_balance_permute, lib.cp_load_balance_unpermute):
        rc, msg = _status_and_message(lib, fn(*args))
        assert rc == binding.CPA_EINVAL and substr in msg, (rc, msg)


def test_permute_empty_is_ok_without_device(lib):
    assert lib.cp_load_balance_permute(None, None, 0, 8, 16, 2, 0, 8, None) == 0
    assert lib.cp_load_balance_permute(None, None, 1, 8, 16, 2, 3, 0, None) == 0


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, pos=None, o=ctypes.c_void_p(1 << 30), lse=None, batch=1, seq=512, sq=256,
             hq=4, hkv=2, dqk=64, dv=64, dtype=binding.CPA_F32, scale=0.125, cp=2, rank=0)
    a.update(kw)
    rc = lib.cp_attention_fwd(a["q"], a["k"], a["v"], a["pos"], a["o"], a["lse"], a["batch"], a["seq"], a["sq"],
                              a["hq"], a["hkv"], a["dqk"], a["dv"], a["dtype"], a["scale"], a["cp"], a["rank"], None)
    return _status_and_message(lib, rc)


@pytest.mark.parametrize("kw,status,substr", [
    (dict(seq=502), binding.CPA_EINVAL, "multiple of 2*cp"),
    (dict(rank=2), binding.CPA_EINVAL, "rank"),
    (dict(rank=-1), binding.CPA_EINVAL, "rank"),
    (dict(hq=3), binding.CPA_EINVAL, "multiple of hkv"),
    (dict(scale=0.0), binding.CPA_EINVAL, "softmax_scale"),
    (dict(scale=float("nan")), binding.CPA_EINVAL, "softmax_scale"),
    (dict(sq=100), binding.CPA_EINVAL, "without q_positions"),
    (dict(dtype=7), binding.CPA_EINVAL, "dtype"),
    (dict(dqk=96, dv=96), binding.CPA_ENOTSUP, "not supported"),
    (dict(dqk=192, dv=128), binding.CPA_ENOTSUP, "not supported"),  # fp32 has no MLA variant
    (dict(q=None), binding.CPA_EINVAL, "null"),
    (dict(k=ctypes.c_void_p(4100)), binding.CPA_EINVAL, "aligned"),
    (dict(lse=ctypes.c_void_p(4098)), binding.CPA_EINVAL, "lse"),
    (dict(pos=ctypes.c_void_p(4098), sq=10), binding.CPA_EINVAL, "q_positions"),
])
def test_attention_argument_errors(lib, kw, status, substr):
    rc, msg = _fwd(lib, **kw)
    assert rc == status and substr in msg, (rc, msg)


def test_attention_fwd_workspace_bytes(lib):
    # the 8192-token MHA shape at cp = 4 (256 work items) is split; the 131072-token GQA and the
    # 32768-token MLA shapes (4096 work items per rank) and float32 are not; bad arguments give 0
    bf16, f32 = binding.CPA_BF16, binding.CPA_F32
    assert all(lib.cp_attention_fwd_workspace_bytes(1, 8192, 32, 32, 128, 128, bf16, 4, r) > 0 for r in range(4))
    assert lib.cp_attention_fwd_workspace_bytes(1, 8192, 32, 32, 128, 128, bf16, 1, 0) == 0
    assert lib.cp_attention_fwd_workspace_bytes(1, 131072, 64, 8, 128, 128, bf16, 8, 3) == 0
    assert lib.cp_attention_fwd_workspace_bytes(1, 32768, 128, 128, 192, 128, bf16, 4, 0) == 0
    assert lib.cp_attention_fwd_workspace_bytes(1, 2048, 1, 1, 128, 128, f32, 1, 0) == 0
    assert lib.cp_attention_fwd_workspace_bytes(1, 2047, 1, 1, 128, 128, bf16, 1, 0) == 0
    assert lib.cp_attention_fwd_workspace_bytes(1, 2048, 1, 1, 96, 96, bf16, 1, 0) == 0
    assert lib.cp_attention_fwd_workspace_bytes(1, 2048, 1, 1, 128, 128, bf16, 2, 2) == 0


def _dq_split_bytes_expected(batch, seq, hq, hkv, d_qk, cp, rank):
    """The dQ split's workspace restated from its rules: 256-row blocks (MHA: one head per
    workgroup), 64-key tiles, split only below 512 work items; pieces of tau = max(16, tiles x
    units / 256) tiles; one partial slot per piece of every cut row block."""
    c = seq // (2 * cp)
    sq = 2 * c
    sqp = -(-sq // 32) * 32
    base = 2 * batch * hq * sqp * 4 + sqp * 4 + 2 * (sqp // 32) * 4
    base = -(-base // 256) * 256
    g = hq // hkv
    hpw = math.gcd(g, 8)
    bm = 32 * (8 // hpw)
    nrb = -(-sq // bm)
    units = batch * hkv * (g // hpw)
    if units * nrb >= 512:
        return base
    pos = olb.shard_positions(seq, cp, rank)
    tpc = -(-c // 64)
    tiles = []
    for rb in range(nrb):
        qmax = int(pos[min(sq, (rb + 1) * bm) - 1])
        imax = min(qmax // c, 2 * cp - 1)
        tiles.append(imax * tpc + min(-(-(qmax - imax * c + 1) // 64), tpc))
    tau = max(16, -(-(sum(tiles) * units) // 256))
    slots = sum(n for n in (-(-t_ // tau) for t_ in tiles) if n > 1)
    if slots == 0:
        return base
    return base + units * slots * bm * hpw * d_qk * 4


def test_attention_bwd_split_workspace_bytes(lib):
    # the 8192-token MHA shape at cp = 4 (256 work items) splits dQ on every rank; the cp = 1
    # and 131072-token shapes have enough work items and need only the base workspace
    bf16, f32 = binding.CPA_BF16, binding.CPA_F32
    for r in range(4):
        got = lib.cp_attention_bwd_split_workspace_bytes(1, 8192, 32, 32, 128, 128, bf16, 4, r)
        assert got == _dq_split_bytes_expected(1, 8192, 32, 32, 128, 4, r), r
        assert got > lib.cp_attention_bwd_workspace_bytes(1, 2048, 32), r
    for args in ((1, 8192, 32, 32, 128, 128, bf16, 1, 0), (1, 131072, 64, 8, 128, 128, bf16, 8, 3),
                 (1, 32768, 128, 128, 192, 128, bf16, 4, 0)):
        b, s, hq, hkv, dqk, dv, dt, cp, r = args
        got = lib.cp_attention_bwd_split_workspace_bytes(*args)
        assert got == lib.cp_attention_bwd_workspace_bytes(b, s // cp, hq) == _dq_split_bytes_expected(
            b, s, hq, hkv, dqk, cp, r), args
    # a ragged small GQA shape: batch 2, 8 kv heads of 2 query heads
    assert lib.cp_attention_bwd_split_workspace_bytes(2, 4096, 16, 8, 64, 64, bf16, 2, 1) == \
        _dq_split_bytes_expected(2, 4096, 16, 8, 64, 2, 1)
    for bad in ((1, 2048, 1, 1, 128, 128, f32, 1, 0), (1, 2047, 1, 1, 128, 128, bf16, 1, 0),
                (1, 2048, 1, 1, 96, 96, bf16, 1, 0), (1, 2048, 1, 1, 128, 128, bf16, 2, 2),
                (0, 2048, 1, 1, 128, 128, bf16, 1, 0), (1, 2048, 3, 2, 128, 128, bf16, 1, 0)):
        assert lib.cp_attention_bwd_split_workspace_bytes(*bad) == 0, bad


def test_attention_fwd_ws_argument_errors(lib):
    rc = lib.cp_attention_fwd_ws(FAKE, FAKE, FAKE, None, FAKE, None, 1, 8192, 2048, 32, 32, 128, 128,
                                 binding.CPA_BF16, 0.088, 4, 0, ctypes.c_void_p(4100), 1 << 30, None)
    rc, msg = _status_and_message(lib, rc)
    assert rc == binding.CPA_EINVAL and "workspace" in msg, (rc, msg)
    rc = lib.cp_attention_fwd_ws(FAKE, FAKE, FAKE, None, FAKE, None, 1, 8192, 2048, 32, 32, 128, 128,
                                 binding.CPA_BF16, 0.088, 4, 4, FAKE, 1 << 30, None)
    rc, msg = _status_and_message(lib, rc)
    assert rc == binding.CPA_EINVAL and "rank" in msg, (rc, msg)


def test_attention_empty_is_ok_without_device(lib):
    assert _fwd(lib, batch=0)[0] == 0
    assert _fwd(lib, sq=0, pos=FAKE)[0] == 0


def _bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, pos=None, dq=FAKE, dk=FAKE, dv=FAKE, batch=1,
             seq=512, sq=256, hq=4, hkv=2, dqk=64, dv_=64, dtype=binding.CPA_BF16, scale=0.125, cp=2, rank=0,
             ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    rc = lib.cp_attention_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["pos"], a["dq"], a["dk"],
                              a["dv"], a["batch"], a["seq"], a["sq"], a["hq"], a["hkv"], a["dqk"], a["dv_"],
                              a["dtype"], a["scale"], a["cp"], a["rank"], a["ws"], a["ws_bytes"], None)
    return _status_and_message(lib, rc)


@pytest.mark.parametrize("kw,status,substr", [
    (dict(seq=502), binding.CPA_EINVAL, "multiple of 2*cp"),
    (dict(rank=2), binding.CPA_EINVAL, "rank"),
    (dict(hq=3), binding.CPA_EINVAL, "multiple of hkv"),
    (dict(scale=-0.5), binding.CPA_EINVAL, "softmax_scale"),
    (dict(sq=100), binding.CPA_EINVAL, "without q_positions"),
    (dict(dtype=binding.CPA_F32), binding.CPA_ENOTSUP, "not supported"),
    (dict(dqk=96, dv_=96), binding.CPA_ENOTSUP, "not supported"),
    (dict(dtype=5), binding.CPA_EINVAL, "dtype"),
    (dict(lse=None), binding.CPA_EINVAL, "null"),
    (dict(dk=ctypes.c_void_p(4100)), binding.CPA_EINVAL, "aligned"),
    (dict(lse=ctypes.c_void_p(4098)), binding.CPA_EINVAL, "aligned"),
    (dict(ws_bytes=64), binding.CPA_EINVAL, "workspace"),
])
def test_attention_bwd_argument_errors(lib, kw, status, substr):
    rc, msg = _bwd(lib, **kw)
    assert rc == status and substr in msg, (rc, msg)


def test_attention_bwd_empty_is_ok_without_device(lib):
    assert _bwd(lib, batch=0)[0] == 0
    assert _bwd(lib, sq=0, pos=FAKE)[0] == 0


def test_attention_bwd_workspace_size(lib):
    # log2-LSE and D per (b, h, padded row), positions per padded row, min/max per 32-row block,
    # rounded up to 256 bytes (where the dQ split's partial slots begin)
    def up256(n):
        return -(-n // 256) * 256
    assert cpa.attention_bwd_workspace_bytes(1, 16384, 64) == up256(2 * 64 * 16384 * 4 + 16384 * 4 + 2 * 512 * 4)
    assert cpa.attention_bwd_workspace_bytes(2, 100, 4) == up256(2 * 2 * 4 * 128 * 4 + 128 * 4 + 2 * 4 * 4)
    assert cpa.attention_bwd_workspace_bytes(0, 100, 4) == 0


def _dec(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lengths=FAKE, o=FAKE, lse=None, batch=24, hq=48, hkv=8, d=128, max_len=2048,
             dtype=binding.CPA_BF16, scale=0.088, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    rc = lib.gqa_decode_attention(a["q"], a["k"], a["v"], a["lengths"], a["o"], a["lse"], a["batch"], a["hq"],
                                  a["hkv"], a["d"], a["max_len"], a["dtype"], a["scale"], a["ws"], a["ws_bytes"], None)
    return _status_and_message(lib, rc)


@pytest.mark.parametrize("kw,status,substr", [
    (dict(hq=50), binding.CPA_EINVAL, "multiple of hkv"),
    (dict(max_len=0), binding.CPA_EINVAL, "max_len"),
    (dict(scale=-1.0), binding.CPA_EINVAL, "softmax_scale"),
    (dict(d=96), binding.CPA_ENOTSUP, "head dim"),
    (dict(lengths=None), binding.CPA_EINVAL, "null"),
    (dict(ws_bytes=16), binding.CPA_EINVAL, "workspace"),
    (dict(v=ctypes.c_void_p(4104)), binding.CPA_EINVAL, "aligned"),
    (dict(dtype=3), binding.CPA_EINVAL, "dtype"),
])
def test_decode_argument_errors(lib, kw, status, substr):
    rc, msg = _dec(lib, **kw)
    assert rc == status and substr in msg, (rc, msg)


def _dec_noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lengths=FAKE, o=FAKE, lse=None, batch=24, hq=48, hkv=8, d=128, max_len=2048,
             dtype=binding.CPA_BF16, scale=0.088)
    a.update(kw)
    rc = lib.gqa_decode_attention_noalloc(a["q"], a["k"], a["v"], a["lengths"], a["o"], a["lse"], a["batch"],
                                          a["hq"], a["hkv"], a["d"], a["max_len"], a["dtype"], a["scale"], None)
    return _status_and_message(lib, rc)


@pytest.mark.parametrize("kw,status,substr", [
    (dict(hq=50), binding.CPA_EINVAL, "multiple of hkv"),
    (dict(max_len=0), binding.CPA_EINVAL, "max_len"),
    (dict(scale=float("nan")), binding.CPA_EINVAL, "softmax_scale"),
    (dict(d=96), binding.CPA_ENOTSUP, "head dim"),
    (dict(o=None), binding.CPA_EINVAL, "null"),
    (dict(q=ctypes.c_void_p(4104)), binding.CPA_EINVAL, "aligned"),
    (dict(batch=64, hq=64, max_len=8192), binding.CPA_EINVAL, "static scratch"),
])
def test_decode_noalloc_argument_errors(lib, kw, status, substr):
    rc, msg = _dec_noalloc(lib, **kw)
    assert rc == status and substr in msg, (rc, msg)


def test_decode_noalloc_empty_is_ok_without_device(lib):
    assert _dec_noalloc(lib, batch=0)[0] == 0


def _merge(lib, **kw):
    a = dict(o_parts=FAKE, lse_parts=FAKE, o=FAKE, lse=None, parts=4, batch=24, hq=48, d=128, dtype=binding.CPA_BF16)
    a.update(kw)
    rc = lib.gqa_decode_merge(a["o_parts"], a["lse_parts"], a["o"], a["lse"], a["parts"], a["batch"], a["hq"], a["d"],
                              a["dtype"], None)
    return _status_and_message(lib, rc)


@pytest.mark.parametrize("kw,status,substr", [
    (dict(parts=0), binding.CPA_EINVAL, "parts"),
    (dict(batch=-1), binding.CPA_EINVAL, ">= 0"),
    (dict(d=0), binding.CPA_EINVAL, "d must"),
    (dict(dtype=7), binding.CPA_EINVAL, "dtype"),
    (dict(o=None), binding.CPA_EINVAL, "null"),
    (dict(lse_parts=ctypes.c_void_p(4098)), binding.CPA_EINVAL, "aligned"),
    (dict(o_parts=ctypes.c_void_p(4097)), binding.CPA_EINVAL, "aligned"),
])
def test_decode_merge_argument_errors(lib, kw, status, substr):
    rc, msg = _merge(lib, **kw)
    assert rc == status and substr in msg, (rc, msg)


def test_decode_merge_empty_is_ok_without_device(lib):
    assert _merge(lib, batch=0)[0] == 0
    assert _merge(lib, hq=0)[0] == 0


def _dec8(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, lengths=FAKE, o=FAKE, lse=None, batch=24, hq=48, hkv=8, d=128,
             max_len=2048, scale=0.088, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    rc = lib.gqa_decode_attention_int8kv(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["lengths"], a["o"], a["lse"],
                                         a["batch"], a["hq"], a["hkv"], a["d"], a["max_len"], a["scale"], a["ws"],
                                         a["ws_bytes"], None)
    return _status_and_message(lib, rc)


@pytest.mark.parametrize("kw,status,substr", [
    (dict(hq=50), binding.CPA_EINVAL, "multiple of hkv"),
    (dict(batch=-1), binding.CPA_EINVAL, "batch"),
    (dict(max_len=0), binding.CPA_EINVAL, "max_len"),
    (dict(scale=float("inf")), binding.CPA_EINVAL, "softmax_scale"),
    (dict(d=64), binding.CPA_ENOTSUP, "head dim"),
    (dict(batch=70000), binding.CPA_EINVAL, "65535"),
    (dict(ks=None), binding.CPA_EINVAL, "null"),
    (dict(ws_bytes=1024), binding.CPA_EINVAL, "workspace"),
    (dict(k=ctypes.c_void_p(4104)), binding.CPA_EINVAL, "aligned"),
    (dict(vs=ctypes.c_void_p(4098)), binding.CPA_EINVAL, "aligned"),
])
def test_decode_int8_argument_errors(lib, kw, status, substr):
    rc, msg = _dec8(lib, **kw)
    assert rc == status and substr in msg, (rc, msg)


def test_decode_int8_empty_is_ok_without_device(lib):
    assert _dec8(lib, batch=0)[0] == 0


def _quant(lib, **kw):
    a = dict(x=FAKE, codes=FAKE, scales=FAKE, rows=100, d=128, dtype=binding.CPA_BF16)
    a.update(kw)
    rc = lib.kv_cache_quantize_int8(a["x"], a["codes"], a["scales"], a["rows"], a["d"], a["dtype"], None)
    return _status_and_message(lib, rc)


@pytest.mark.parametrize("kw,status,substr", [
    (dict(rows=-1), binding.CPA_EINVAL, "rows"),
    (dict(d=0), binding.CPA_EINVAL, "d must"),
    (dict(dtype=9), binding.CPA_EINVAL, "dtype"),
    (dict(codes=None), binding.CPA_EINVAL, "null"),
    (dict(x=ctypes.c_void_p(4097)), binding.CPA_EINVAL, "aligned"),
    (dict(x=ctypes.c_void_p(4098), dtype=binding.CPA_F32), binding.CPA_EINVAL, "aligned"),
    (dict(scales=ctypes.c_void_p(4102)), binding.CPA_EINVAL, "aligned"),
    (dict(rows=1 << 34), binding.CPA_EINVAL, "too large"),
])
def test_quantize_argument_errors(lib, kw, status, substr):
    rc, msg = _quant(lib, **kw)
    assert rc == status and substr in msg, (rc, msg)


def test_quantize_empty_is_ok_without_device(lib):
    assert _quant(lib, rows=0)[0] == 0


def test_decode_workspace_size(lib):
    # (max, sum, D outputs) per (sequence, query head, split of 256 keys)
    assert cpa.decode_workspace_bytes(24, 48, 8, 2048, 128) == 24 * 48 * 8 * 130 * 4
    assert cpa.decode_workspace_bytes(1, 1, 1, 1, 64) == 66 * 4
    # short caches (max_len <= 1024) take 128-key splits
    assert cpa.decode_workspace_bytes(24, 48, 8, 512, 128) == 24 * 48 * 4 * 130 * 4
    assert cpa.decode_workspace_bytes(2, 4, 1, 1024, 64) == 2 * 4 * 8 * 66 * 4
    assert cpa.decode_workspace_bytes(2, 4, 1, 1025, 64) == 2 * 4 * 5 * 66 * 4
    assert cpa.decode_workspace_bytes(0, 48, 8, 2048, 128) == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch

    with pytest.raises(ValueError):
        cpa.permute(torch.zeros(1, 8, 4), 2)
