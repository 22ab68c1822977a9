"""The allocation-free decode entry point (gqa_decode_attention_noalloc) against the workspace
entry point (gqa_decode_attention), through the C ABI, on two calls in a row: the 24-sequence
Mixtral-8x22B-shaped batch, then a smaller fp32 batch, so the second call runs over the first
call's leftovers in the library's static scratch. Both entry points run the same kernels, so the
outputs must agree bit for bit (which is inside the 2e-2 / 1e-4 parity bar)."""

import ctypes

import pytest
import torch

import context_causal_attention_load_amd as cpa
from context_causal_attention_load_amd import binding, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _noalloc_raw(q, kc, vc, lengths, o, lse, scale):
    """Straight through the C ABI, no binding checks: returns the status."""
    lib = cpa.load_library()
    B, Hq, D = q.shape
    Hkv, Lmax = kc.shape[1], kc.shape[2]
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return lib.gqa_decode_attention_noalloc(ptr(q), ptr(kc), ptr(vc), ptr(lengths), ptr(o), ptr(lse), B, Hq, Hkv, D,
                                            Lmax, binding._DTYPES[q.dtype], float(scale),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("dummy", [0])
def test_noalloc_decode_matches_workspace_decode(dummy):
    w = synth.MIXTRAL_8X22B_DECODE
    cases = [
        ("mixtral-b24", w.batch, w.hq, w.hkv, w.d, w.max_len, w.len_min, w.len_max, w.dtype, w.seed),
        ("small-fp32", 3, 12, 4, 64, 700, 1, 700, torch.float32, 71),
    ]
    for name, B, Hq, Hkv, D, Lmax, lo, hi, dtype, seed in cases:
        print(f"\n[gpu case] noalloc decode {name}: B={B} Hq={Hq} Hkv={Hkv} D={D} Lmax={Lmax} {dtype}", flush=True)
        lengths, q, kc, vc = synth.decode_inputs(B, Hq, Hkv, D, Lmax, lo, hi, dtype, seed)
        qd, kd, vd, ld = q.to(DEV), kc.to(DEV), vc.to(DEV), lengths.to(DEV)
        o_ref, l_ref = cpa.decode(qd, kd, vd, ld)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, float("nan"))
        rc = _noalloc_raw(qd, kd, vd, ld, o, lse, 1.0 / D ** 0.5)
        assert rc == binding.CPA_OK, cpa.load_library().cpattn_last_error()
        torch.cuda.synchronize()
        diff = (o.float() - o_ref.float()).abs().max().item()
        print(f"  max |O_noalloc - O_workspace| = {diff:.3e}", flush=True)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
        # the binding's wrapper of the same call
        o2 = torch.empty_like(o_ref)
        cpa.decode_noalloc(qd, kd, vd, ld, o2)
        torch.cuda.synchronize()
        assert torch.equal(o2, o_ref)


def test_noalloc_decode_refuses_more_than_its_scratch():
    B, Hq, Hkv, D, Lmax = 64, 64, 8, 128, 8192   # 68 MB of partials > 16 MiB
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((B, Hkv, 16, D), dtype=torch.bfloat16, device=DEV)  # never read: the call is refused first
    ld = torch.zeros(B, dtype=torch.int32, device=DEV)
    o = torch.zeros_like(q)
    lib = cpa.load_library()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = lib.gqa_decode_attention_noalloc(ptr(q), ptr(kc), ptr(kc), ptr(ld), ptr(o), None, B, Hq, Hkv, D, Lmax,
                                          binding.CPA_BF16, 0.088, None)
    msg = lib.cpattn_last_error().decode()
    assert rc == binding.CPA_EINVAL and "static scratch" in msg, (rc, msg)
