"""The binding rejects caller-provided output buffers of the wrong shape or dtype before any
launch: the library receives raw pointers and could not tell that a buffer is too small."""

import pytest
import torch

import context_causal_attention_load_amd as cpa

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _t(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype, device=DEV)


def test_attention_fwd_rejects_wrong_outputs():
    q, k, v = _t((1, 64, 4, 64)), _t((1, 128, 2, 64)), _t((1, 128, 2, 64))
    with pytest.raises(ValueError, match="out must be"):
        cpa.attention_fwd(q, k, v, 1, 0, q_positions=torch.arange(64, dtype=torch.int32, device=DEV),
                          out=_t((1, 32, 4, 64)))
    with pytest.raises(ValueError, match="out must be"):
        cpa.attention_fwd(q, k, v, 1, 0, q_positions=torch.arange(64, dtype=torch.int32, device=DEV),
                          out=_t((1, 64, 4, 64), torch.float32))
    with pytest.raises(ValueError, match="lse must be"):
        cpa.attention_fwd(q, k, v, 1, 0, q_positions=torch.arange(64, dtype=torch.int32, device=DEV),
                          lse=_t((1, 4, 32), torch.float32))


def test_backward_rejects_wrong_outputs():
    q, k, v = _t((1, 64, 4, 64)), _t((1, 128, 2, 64)), _t((1, 128, 2, 64))
    o, do, lse = _t((1, 64, 4, 64)), _t((1, 64, 4, 64)), _t((1, 4, 64), torch.float32)
    pos = torch.arange(64, dtype=torch.int32, device=DEV)
    for name, kw in (("dq", dict(dq=_t((1, 64, 4, 32), torch.float32))),
                     ("dk", dict(dk=_t((1, 64, 2, 64), torch.float32))),
                     ("dv", dict(dv=_t((1, 128, 2, 64)))),):
        with pytest.raises(ValueError, match=f"{name} must be"):
            cpa.attention_bwd(q, k, v, o, lse, do, 1, 0, q_positions=pos, **kw)


def test_decodes_reject_wrong_outputs():
    q = _t((2, 8, 128))
    kc, vc = _t((2, 2, 64, 128)), _t((2, 2, 64, 128))
    lengths = torch.tensor([10, 64], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="out must be"):
        cpa.decode(q, kc, vc, lengths, out=_t((2, 4, 128)))
    with pytest.raises(ValueError, match="lse must be"):
        cpa.decode(q, kc, vc, lengths, lse=_t((2, 8), torch.bfloat16))
    codes = torch.zeros((2, 2, 64, 128), dtype=torch.int8, device=DEV)
    scales = _t((2, 2, 64), torch.float32)
    with pytest.raises(ValueError, match="out must be"):
        cpa.decode_int8(q, codes, scales, codes, scales, lengths, out=_t((2, 8, 64)))
    with pytest.raises(ValueError, match="lse must be"):
        cpa.decode_merge(_t((3, 2, 8, 128)), _t((3, 2, 8), torch.float32), lse=_t((2, 9), torch.float32))
