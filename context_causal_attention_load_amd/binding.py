"""ctypes binding of libcpattn.so (include/cpattn.h).

Argument marshalling only: torch tensors are checked for device, dtype and contiguity and
passed as raw pointers with the current HIP stream. Every computation runs in the library's
HIP kernels; there is no CPU path. A missing library raises ``CpattnError`` on first use.
"""

import ctypes
import math
import os

import torch

from .build import OUT as _LIB_PATH

CPA_OK, CPA_EINVAL, CPA_ENOTSUP, CPA_EHIP = 0, -22, -95, -1000
CPA_F32, CPA_BF16 = 0, 1

_DTYPES = {torch.float32: CPA_F32, torch.bfloat16: CPA_BF16}

_lib = None


class CpattnError(RuntimeError):
    def __init__(self, func, status, message):
        super().__init__(f"{func} failed with status {status}: {message}")
        self.status = status
        self.func = func


def library_path():
    return _LIB_PATH


def load_library():
    """Load libcpattn.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise CpattnError("load_library", CPA_EHIP,
                          f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python -m context_causal_attention_load_amd.build)")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.cpattn_last_error.restype = ctypes.c_char_p
    lib.cpattn_last_error.argtypes = []
    lib.cp_load_balance_source_index.restype = i64
    lib.cp_load_balance_source_index.argtypes = [i64, i32, i64]
    lib.cp_load_balance_positions.restype = ctypes.c_int
    lib.cp_load_balance_positions.argtypes = [i64, i32, i64, i64, vp]
    for name in ("cp_load_balance_permute", "cp_load_balance_unpermute"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, i64, i64, i64, i32, i64, i64, vp]
    lib.cp_attention_fwd.restype = ctypes.c_int
    lib.cp_attention_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                     f32, i32, i32, vp]
    lib.cp_attention_fwd_workspace_bytes.restype = ctypes.c_size_t
    lib.cp_attention_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.cp_attention_fwd_ws.restype = ctypes.c_int
    lib.cp_attention_fwd_ws.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                        f32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.gqa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.gqa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.gqa_decode_attention.restype = ctypes.c_int
    lib.gqa_decode_attention.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                         vp, ctypes.c_size_t, vp]
    lib.gqa_decode_attention_noalloc.restype = ctypes.c_int
    lib.gqa_decode_attention_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp]
    lib.gqa_decode_merge.restype = ctypes.c_int
    lib.gqa_decode_merge.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.gqa_decode_attention_int8kv.restype = ctypes.c_int
    lib.gqa_decode_attention_int8kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                                vp, ctypes.c_size_t, vp]
    lib.cp_attention_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.cp_attention_bwd_workspace_bytes.argtypes = [i32, i32, i32]
    lib.cp_attention_bwd_split_workspace_bytes.restype = ctypes.c_size_t
    lib.cp_attention_bwd_split_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.cp_attention_bwd.restype = ctypes.c_int
    lib.cp_attention_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     i32, f32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.kv_cache_quantize_int8.restype = ctypes.c_int
    lib.kv_cache_quantize_int8.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    _lib = lib
    return lib


def _check(name, status):
    if status != CPA_OK:
        msg = load_library().cpattn_last_error().decode(errors="replace")
        raise CpattnError(name, status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_gpu(*tensors):
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous (no implicit copies are made)")


def _check_buf(t, shape, dtype, name):
    """A caller-provided output must have exactly the shape and dtype the call writes: the
    library receives a raw pointer and cannot see how large the buffer is."""
    if t is not None and (tuple(t.shape) != tuple(shape) or t.dtype != dtype):
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


# ---------------------------------------------------------------------------- index helpers

def lb_source_index(seq, cp, j):
    """Original position of permuted slot j (host helper of the library)."""
    return int(load_library().cp_load_balance_source_index(seq, cp, j))


def lb_positions(seq, cp, row_begin=0, row_count=None):
    """int32 CPU tensor of original positions for permuted slots [row_begin, row_begin+row_count)."""
    if row_count is None:
        row_count = seq - row_begin
    out = torch.empty(row_count, dtype=torch.int32)
    _check("cp_load_balance_positions",
           load_library().cp_load_balance_positions(seq, cp, row_begin, row_count,
                                                    ctypes.c_void_p(out.data_ptr())))
    return out


# ---------------------------------------------------------------------------- permutation

def _fold(x, dim):
    dim = dim % x.dim()
    outer = math.prod(x.shape[:dim])
    row_bytes = math.prod(x.shape[dim + 1:]) * x.element_size()
    return outer, x.shape[dim], row_bytes


def permute(x, cp, dim=1, row_begin=0, row_count=None, out=None):
    """Gather permuted slots [row_begin, row_begin+row_count) of ``x`` (original order along
    ``dim``): ``out.select(dim, i) = x.select(dim, src(row_begin + i))``."""
    _need_gpu(x, out)
    outer, seq, row_bytes = _fold(x, dim)
    if row_count is None:
        row_count = seq - row_begin
    shape = list(x.shape)
    shape[dim % x.dim()] = row_count
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif list(out.shape) != shape or out.dtype != x.dtype:
        raise ValueError(f"out must be {shape} {x.dtype}")
    _check("cp_load_balance_permute",
           load_library().cp_load_balance_permute(_ptr(x), _ptr(out), outer, seq, row_bytes, cp,
                                                  row_begin, row_count, _stream(x.device)))
    return out


def unpermute(x, cp, seq, dim=1, row_begin=0, out=None):
    """Scatter permuted slots [row_begin, row_begin + x.shape[dim]) back to original order:
    ``out.select(dim, src(row_begin + i)) = x.select(dim, i)``. Other rows of ``out`` keep their
    contents (a new ``out`` is zero-filled)."""
    _need_gpu(x, out)
    outer, row_count, row_bytes = _fold(x, dim)
    shape = list(x.shape)
    shape[dim % x.dim()] = seq
    if out is None:
        out = torch.zeros(shape, dtype=x.dtype, device=x.device)
    elif list(out.shape) != shape or out.dtype != x.dtype:
        raise ValueError(f"out must be {shape} {x.dtype}")
    _check("cp_load_balance_unpermute",
           load_library().cp_load_balance_unpermute(_ptr(x), _ptr(out), outer, seq, row_bytes, cp,
                                                    row_begin, row_count, _stream(x.device)))
    return out


# ---------------------------------------------------------------------------- attention

def attention_fwd_workspace_bytes(batch, seq, hq, hkv, d_qk, d_v, dtype, cp, rank):
    """Workspace bytes the forward uses to split heavy row blocks of the rank's own shard (0: none)."""
    return int(load_library().cp_attention_fwd_workspace_bytes(batch, seq, hq, hkv, d_qk, d_v, _DTYPES[dtype], cp,
                                                                rank))


def attention_fwd(q_shard, k, v, cp, rank, q_positions=None, scale=None, out=None, lse=None,
                  want_lse=True, workspace=None, split=True):
    """One rank's causal GQA attention over all-gathered K/V in load-balanced order.

    q_shard [B, Sq, Hq, Dqk]; k [B, S, Hkv, Dqk]; v [B, S, Hkv, Dv]; q_positions int32 [Sq] on
    the GPU or None (the rank's own shard). Returns (O [B, Sq, Hq, Dv], LSE [B, Hq, Sq] fp32).
    With ``split`` (the default) a shape whose grid is too small to balance itself gets a
    workspace (``workspace``, or a new one) and the library splits its heavy row blocks;
    ``split=False`` calls cp_attention_fwd, which never splits.
    """
    _need_gpu(q_shard, k, v, q_positions, out, lse)
    if q_shard.dtype not in _DTYPES or k.dtype != q_shard.dtype or v.dtype != q_shard.dtype:
        raise ValueError("q, k, v must share dtype float32 or bfloat16")
    B, Sq, Hq, Dqk = q_shard.shape
    S, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if k.shape != (B, S, Hkv, Dqk) or v.shape[:3] != (B, S, Hkv):
        raise ValueError("k/v shapes do not match q")
    if q_positions is not None and (q_positions.dtype != torch.int32 or q_positions.shape != (Sq,)):
        raise ValueError("q_positions must be int32 [Sq]")
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    _check_buf(out, (B, Sq, Hq, Dv), q_shard.dtype, "out")
    _check_buf(lse, (B, Hq, Sq), torch.float32, "lse")
    if out is None:
        out = torch.empty((B, Sq, Hq, Dv), dtype=q_shard.dtype, device=q_shard.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q_shard.device)
    ws_need = 0
    if split and q_positions is None:
        ws_need = attention_fwd_workspace_bytes(B, S, Hq, Hkv, Dqk, Dv, q_shard.dtype, cp, rank)
    if ws_need > 0:
        _need_gpu(workspace)
        if workspace is None:
            workspace = torch.empty(ws_need, dtype=torch.uint8, device=q_shard.device)
        _check("cp_attention_fwd_ws",
               load_library().cp_attention_fwd_ws(_ptr(q_shard), _ptr(k), _ptr(v), _ptr(q_positions), _ptr(out),
                                                  _ptr(lse), B, S, Sq, Hq, Hkv, Dqk, Dv, _DTYPES[q_shard.dtype],
                                                  float(scale), cp, rank, _ptr(workspace),
                                                  workspace.numel() * workspace.element_size(),
                                                  _stream(q_shard.device)))
        return out, lse
    _check("cp_attention_fwd",
           load_library().cp_attention_fwd(_ptr(q_shard), _ptr(k), _ptr(v), _ptr(q_positions), _ptr(out),
                                           _ptr(lse), B, S, Sq, Hq, Hkv, Dqk, Dv, _DTYPES[q_shard.dtype],
                                           float(scale), cp, rank, _stream(q_shard.device)))
    return out, lse


def decode_workspace_bytes(batch, hq, hkv, max_len, d):
    return int(load_library().gqa_decode_workspace_bytes(batch, hq, hkv, max_len, d))


def decode(q, k_cache, v_cache, lengths, scale=None, workspace=None, out=None, lse=None, want_lse=True):
    """GQA single-token decode. q [B, Hq, D]; caches [B, Hkv, Lmax, D]; lengths int32 [B] (GPU).
    Returns (O [B, Hq, D], LSE [B, Hq] fp32)."""
    _need_gpu(q, k_cache, v_cache, lengths, workspace, out, lse)
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and caches must share dtype float32 or bfloat16")
    B, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, Hkv, Lmax, D) or v_cache.shape != (B, Hkv, Lmax, D):
        raise ValueError("cache shapes do not match q")
    if lengths.dtype != torch.int32 or lengths.shape != (B,):
        raise ValueError("lengths must be int32 [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_workspace_bytes(B, Hq, Hkv, Lmax, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_buf(out, (B, Hq, D), q.dtype, "out")
    _check_buf(lse, (B, Hq), torch.float32, "lse")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check("gqa_decode_attention",
           load_library().gqa_decode_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lengths), _ptr(out),
                                               _ptr(lse), B, Hq, Hkv, D, Lmax, _DTYPES[q.dtype], float(scale),
                                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                                               _stream(q.device)))
    return out, lse


def decode_noalloc(q, k_cache, v_cache, lengths, out, lse=None, scale=None):
    """decode() for callers that cannot allocate: the split partials live in the library's static
    device scratch, and ``out`` (and ``lse``, optional) must be given, so no device memory is
    allocated here either. Calls that overlap on one GPU race (they share the scratch)."""
    _need_gpu(q, k_cache, v_cache, lengths, out, lse)
    if q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and caches must share dtype float32 or bfloat16")
    B, Hq, D = q.shape
    Hkv, Lmax = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, Hkv, Lmax, D) or v_cache.shape != (B, Hkv, Lmax, D):
        raise ValueError("cache shapes do not match q")
    if lengths.dtype != torch.int32 or lengths.shape != (B,):
        raise ValueError("lengths must be int32 [B]")
    if out is None:
        raise ValueError("out must be given (this call allocates nothing)")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check_buf(out, (B, Hq, D), q.dtype, "out")
    _check_buf(lse, (B, Hq), torch.float32, "lse")
    _check("gqa_decode_attention_noalloc",
           load_library().gqa_decode_attention_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lengths),
                                                       _ptr(out), _ptr(lse), B, Hq, Hkv, D, Lmax, _DTYPES[q.dtype],
                                                       float(scale), _stream(q.device)))
    return out, lse


def decode_merge(o_parts, lse_parts, out=None, lse=None, want_lse=True):
    """Combine decode results of disjoint cache slices (a cache sharded along its length).
    o_parts [R, B, Hq, D]; lse_parts [R, B, Hq] fp32 (natural log, -inf = empty slice).
    Returns (O [B, Hq, D], LSE [B, Hq] fp32)."""
    _need_gpu(o_parts, lse_parts, out, lse)
    if o_parts.dtype not in _DTYPES:
        raise ValueError("o_parts must be float32 or bfloat16")
    R, B, Hq, D = o_parts.shape
    if lse_parts.dtype != torch.float32 or tuple(lse_parts.shape) != (R, B, Hq):
        raise ValueError("lse_parts must be float32 [R, B, Hq]")
    _check_buf(out, (B, Hq, D), o_parts.dtype, "out")
    _check_buf(lse, (B, Hq), torch.float32, "lse")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=o_parts.dtype, device=o_parts.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=o_parts.device)
    _check("gqa_decode_merge",
           load_library().gqa_decode_merge(_ptr(o_parts), _ptr(lse_parts), _ptr(out), _ptr(lse), R, B, Hq, D,
                                           _DTYPES[o_parts.dtype], _stream(o_parts.device)))
    return out, lse


def quantize_kv(x, codes=None, scales=None):
    """Int8 absmax quantization of every row (last dim) of x (bf16 or fp32, GPU): one float32
    scale per row. Returns (codes int8 of x's shape, scales float32 of x.shape[:-1])."""
    _need_gpu(x, codes, scales)
    if x.dtype not in _DTYPES:
        raise ValueError("x must be float32 or bfloat16")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if codes.dtype != torch.int8 or codes.shape != x.shape:
        raise ValueError("codes must be int8 of x's shape")
    if scales.dtype != torch.float32 or scales.shape != x.shape[:-1]:
        raise ValueError("scales must be float32 of x.shape[:-1]")
    _check("kv_cache_quantize_int8",
           load_library().kv_cache_quantize_int8(_ptr(x), _ptr(codes), _ptr(scales), rows, d, _DTYPES[x.dtype],
                                                 _stream(x.device)))
    return codes, scales


def decode_int8(q, k_codes, k_scales, v_codes, v_scales, lengths, scale=None, workspace=None, out=None, lse=None,
                want_lse=True):
    """GQA single-token decode over an int8 cache. q [B, Hq, 128] bf16; codes int8 [B, Hkv, Lmax,
    128]; scales float32 [B, Hkv, Lmax]; lengths int32 [B] (GPU). Returns (O [B, Hq, 128] bf16,
    LSE [B, Hq] fp32)."""
    _need_gpu(q, k_codes, k_scales, v_codes, v_scales, lengths, workspace, out, lse)
    if q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16")
    if k_codes.dtype != torch.int8 or v_codes.dtype != torch.int8:
        raise ValueError("codes must be int8")
    if k_scales.dtype != torch.float32 or v_scales.dtype != torch.float32:
        raise ValueError("scales must be float32")
    B, Hq, D = q.shape
    Hkv, Lmax = k_codes.shape[1], k_codes.shape[2]
    if k_codes.shape != (B, Hkv, Lmax, D) or v_codes.shape != (B, Hkv, Lmax, D):
        raise ValueError("code cache shapes do not match q")
    if k_scales.shape != (B, Hkv, Lmax) or v_scales.shape != (B, Hkv, Lmax):
        raise ValueError("scales must be [B, Hkv, Lmax]")
    if lengths.dtype != torch.int32 or lengths.shape != (B,):
        raise ValueError("lengths must be int32 [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_workspace_bytes(B, Hq, Hkv, Lmax, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_buf(out, (B, Hq, D), q.dtype, "out")
    _check_buf(lse, (B, Hq), torch.float32, "lse")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check("gqa_decode_attention_int8kv",
           load_library().gqa_decode_attention_int8kv(_ptr(q), _ptr(k_codes), _ptr(v_codes), _ptr(k_scales),
                                                      _ptr(v_scales), _ptr(lengths), _ptr(out), _ptr(lse), B, Hq,
                                                      Hkv, D, Lmax, float(scale), _ptr(workspace),
                                                      workspace.numel() * workspace.element_size(),
                                                      _stream(q.device)))
    return out, lse


def attention_bwd_workspace_bytes(batch, sq, hq):
    return int(load_library().cp_attention_bwd_workspace_bytes(batch, sq, hq))


def attention_bwd_split_workspace_bytes(batch, seq, hq, hkv, d_qk, d_v, dtype, cp, rank):
    """Workspace bytes with which the backward also splits the dQ of heavy row blocks of the
    rank's own shard (equal to attention_bwd_workspace_bytes(batch, seq // cp, hq) when the shape
    is not split; 0 for invalid arguments)."""
    return int(load_library().cp_attention_bwd_split_workspace_bytes(batch, seq, hq, hkv, d_qk, d_v, _DTYPES[dtype],
                                                                     cp, rank))


def attention_bwd(q_shard, k, v, o, lse, d_o, cp, rank, q_positions=None, scale=None, workspace=None, dq=None,
                  dk=None, dv=None, split=True):
    """Backward of attention_fwd for one rank (bf16). Inputs as for attention_fwd plus its O and
    LSE and dO [B, Sq, Hq, Dv]. Returns float32 (dQ [B, Sq, Hq, Dqk], dK [B, S, Hkv, Dqk],
    dV [B, S, Hkv, Dv]), dK/dV in the gathered key order and holding this rank's share.

    With ``split`` (the default) a new workspace is sized so that a grid too small to balance
    itself computes dQ of its heavy row blocks in pieces (the library decides from the
    workspace's size); ``split=False`` sizes it for the unsplit call. A caller's ``workspace``
    is used as given."""
    _need_gpu(q_shard, k, v, o, lse, d_o, q_positions, workspace, dq, dk, dv)
    if q_shard.dtype != torch.bfloat16 or k.dtype != q_shard.dtype or v.dtype != q_shard.dtype:
        raise ValueError("q, k and v must be bfloat16")
    if o.dtype != q_shard.dtype or d_o.dtype != q_shard.dtype:
        raise ValueError("o and d_o must have q's dtype")
    B, Sq, Hq, Dqk = q_shard.shape
    S, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if k.shape != (B, S, Hkv, Dqk) or v.shape[:3] != (B, S, Hkv):
        raise ValueError("k and v shapes do not match q")
    if o.shape != (B, Sq, Hq, Dv) or d_o.shape != (B, Sq, Hq, Dv):
        raise ValueError("o and d_o must be [B, Sq, Hq, Dv]")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, Sq):
        raise ValueError("lse must be float32 [B, Hq, Sq]")
    if q_positions is not None and (q_positions.dtype != torch.int32 or q_positions.shape != (Sq,)):
        raise ValueError("q_positions must be int32 [Sq]")
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    dev = q_shard.device
    if workspace is None:
        need = attention_bwd_workspace_bytes(B, Sq, Hq)
        if split and q_positions is None:
            need = max(need, attention_bwd_split_workspace_bytes(B, S, Hq, Hkv, Dqk, Dv, q_shard.dtype, cp, rank))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check_buf(dq, (B, Sq, Hq, Dqk), torch.float32, "dq")
    _check_buf(dk, (B, S, Hkv, Dqk), torch.float32, "dk")
    _check_buf(dv, (B, S, Hkv, Dv), torch.float32, "dv")
    if dq is None:
        dq = torch.empty((B, Sq, Hq, Dqk), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((B, S, Hkv, Dqk), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((B, S, Hkv, Dv), dtype=torch.float32, device=dev)
    _check("cp_attention_bwd",
           load_library().cp_attention_bwd(_ptr(q_shard), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(d_o),
                                           _ptr(q_positions), _ptr(dq), _ptr(dk), _ptr(dv), B, S, Sq, Hq, Hkv, Dqk,
                                           Dv, _DTYPES[q_shard.dtype], float(scale), cp, rank, _ptr(workspace),
                                           workspace.numel() * workspace.element_size(), _stream(dev)))
    return dq, dk, dv
