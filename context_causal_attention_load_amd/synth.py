"""Seeded synthetic inputs and workload shapes.

This module only draws random numbers and names shapes; it holds none of the attention or
load-balancing arithmetic, so both the HIP path's tests and the CPU oracle can take their
inputs from it.

Workload shapes stand in for the models the source pages test with: Llama2-7B (MHA, 32
heads of 128) and Llama3.1-70B at 131072 tokens (64 query heads, 8 KV heads) from "Add
context parallelism" (PR 1445, Tests); a DeepSeek-V3-style MLA attention (128 heads, q/k
head dim 192 = 128 + 64 rotary, v head dim 128) from "Add support for EP to context
parallelism in self-attention" (PR 2023, Tests); and a Mixtral-8x22B decode batch of 24 with
prefill 1024 / target 2048 (48 query heads, 8 KV heads) from the inference benchmark command
of "rename context to context_autoregressive" (issue 1453, Tests). Only the attention
shapes are used; values are N(0, 1).

Recipe: ``torch.Generator("cpu").manual_seed(seed)``; Q, then K, then V are drawn as
float32 N(0,1) in natural token order, token chunk by token chunk (``TOKEN_CHUNK`` tokens
per draw, all batches of a chunk at once), then rounded to the workload dtype with
round-to-nearest-even (``Tensor.to``). The backward pass's upstream gradient dO is drawn the same way as Q from a generator of its own
(seed + 1000 for a named workload). Decode draws ``lengths`` (uniform integers in
[len_min, len_max]) first, then q, then the K cache and the V cache over the full maximum
length. The int8-cache decode draws ``lengths`` and q the same way, then for K and then V
the codes (float32 N(0,1) times 40, rounded, clipped to [-127, 127]: the spread of absmax-int8
codes of Gaussian rows) and then one positive float32 scale per cached row, uniform in
[2.5/127, 3.5/127] (the absmax of 128 N(0,1) values divided by 127).
"""

from dataclasses import dataclass, field
import math

import torch

TOKEN_CHUNK = 4096


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    batch: int
    seq: int
    cps: tuple
    hq: int
    hkv: int
    d_qk: int
    d_v: int
    dtype: torch.dtype
    seed: int

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d_qk)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    hq: int
    hkv: int
    d: int
    max_len: int
    len_min: int
    len_max: int
    dtype: torch.dtype
    seed: int

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)


TINY_CP2_F32 = PrefillWorkload("tiny-cp2-gqa-fp32-s512", 1, 512, (2,), 4, 2, 64, 64, torch.float32, 1)
LLAMA2_7B_S8K = PrefillWorkload("llama2-7b-mha-bf16-s8192", 1, 8192, (1, 4), 32, 32, 128, 128, torch.bfloat16, 2)
LLAMA31_70B_S131K = PrefillWorkload("llama3.1-70b-gqa-bf16-s131072-cp8", 1, 131072, (8,), 64, 8, 128, 128, torch.bfloat16, 3)
DEEPSEEK_V3_MLA_S32K = PrefillWorkload("deepseek-v3-mla-bf16-s32768-cp4", 1, 32768, (4,), 128, 128, 192, 128, torch.bfloat16, 4)
MIXTRAL_8X22B_DECODE = DecodeWorkload("mixtral-8x22b-gqa-decode-b24-l2048", 24, 48, 8, 128, 2048, 1024, 2048, torch.bfloat16, 5)

PREFILL_WORKLOADS = (TINY_CP2_F32, LLAMA2_7B_S8K, LLAMA31_70B_S131K, DEEPSEEK_V3_MLA_S32K)


def _draw(gen, shape, dtype, token_axis=1):
    """N(0,1) float32 draws, chunked along ``token_axis``, rounded to ``dtype``."""
    n = shape[token_axis]
    out = torch.empty(shape, dtype=dtype)
    for t0 in range(0, n, TOKEN_CHUNK):
        t1 = min(n, t0 + TOKEN_CHUNK)
        sub = list(shape)
        sub[token_axis] = t1 - t0
        block = torch.randn(sub, generator=gen, dtype=torch.float32)
        out.narrow(token_axis, t0, t1 - t0).copy_(block.to(dtype))
    return out


def prefill_inputs(batch, seq, hq, hkv, d_qk, d_v, dtype, seed):
    """Q [B,S,Hq,Dqk], K [B,S,Hkv,Dqk], V [B,S,Hkv,Dv] in natural token order (CPU tensors)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = _draw(gen, (batch, seq, hq, d_qk), dtype)
    k = _draw(gen, (batch, seq, hkv, d_qk), dtype)
    v = _draw(gen, (batch, seq, hkv, d_v), dtype)
    return q, k, v


def prefill_grad(batch, seq, hq, d_v, dtype, seed):
    """Upstream gradient dO [B, S, Hq, Dv] for the backward pass, N(0,1) in natural token order,
    drawn like Q from its own generator (seeded with ``seed``)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    return _draw(gen, (batch, seq, hq, d_v), dtype)


def workload_prefill_grad(w: PrefillWorkload, seed=None):
    return prefill_grad(w.batch, w.seq, w.hq, w.d_v, w.dtype, 1000 + (w.seed if seed is None else seed))


def workload_prefill_inputs(w: PrefillWorkload, seed=None):
    return prefill_inputs(w.batch, w.seq, w.hq, w.hkv, w.d_qk, w.d_v, w.dtype, w.seed if seed is None else seed)


# Query factors of the rising-logit inputs: powers of two, so every planted value is exact in
# bfloat16 and a power-of-two softmax scale keeps it exact after scaling.
RISE_Q_FACTORS = (0.125, 0.25, 0.5, 1.0, 2.0)


def plant_rising_logits(q, k, step_tokens, step_height, q_factors=RISE_Q_FACTORS):
    """Give the logits a staircase that rises with the key's original position (in place, on
    natural-order CPU tensors Q [B, S, Hq, Dqk] and K [B, S, Hkv, Dqk]).

    Dimension 0 of every key at position u becomes ``step_height * (u // step_tokens)`` and
    dimension 0 of query (position t, head h) becomes ``q_factors[(t + h) % len(q_factors)]``,
    so that dimension adds ``q_factor * step_height * (u // step_tokens)`` to the raw dot product:
    a query's largest logit keeps growing as later keys come in, by an amount per step that
    differs between neighbouring rows and heads. The other dimensions keep their N(0,1) draws.
    Every planted value must be exact in the tensors' dtype (checked)."""
    S = q.shape[1]
    steps = torch.div(torch.arange(S, dtype=torch.int64), step_tokens, rounding_mode="floor")
    kval = (steps * step_height).to(torch.float64)
    if not torch.equal(kval.to(k.dtype).to(torch.float64), kval):
        raise ValueError("planted key values are not exact in the key dtype")
    f = torch.tensor(q_factors, dtype=torch.float64)
    if not torch.equal(f.to(q.dtype).to(torch.float64), f):
        raise ValueError("query factors are not exact in the query dtype")
    hq = q.shape[2]
    idx = (torch.arange(S)[:, None] + torch.arange(hq)[None, :]) % len(q_factors)
    q[:, :, :, 0] = f[idx].to(q.dtype)[None]
    k[:, :, :, 0] = kval.to(k.dtype)[None, :, None]
    return q, k


def decode_inputs(batch, hq, hkv, d, max_len, len_min, len_max, dtype, seed):
    """lengths [B] int32, q [B,Hq,D], k_cache / v_cache [B,Hkv,Lmax,D] (CPU tensors)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    lengths = torch.randint(len_min, len_max + 1, (batch,), generator=gen, dtype=torch.int64).to(torch.int32)
    q = torch.randn((batch, hq, d), generator=gen, dtype=torch.float32).to(dtype)
    k_cache = _draw(gen, (batch, hkv, max_len, d), dtype, token_axis=2)
    v_cache = _draw(gen, (batch, hkv, max_len, d), dtype, token_axis=2)
    return lengths, q, k_cache, v_cache


def decode_int8_inputs(batch, hq, hkv, d, max_len, len_min, len_max, seed):
    """lengths [B] int32, q [B,Hq,D] bf16, then (codes int8 [B,Hkv,Lmax,D], scales float32
    [B,Hkv,Lmax]) for K and for V (CPU tensors)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    lengths = torch.randint(len_min, len_max + 1, (batch,), generator=gen, dtype=torch.int64).to(torch.int32)
    q = torch.randn((batch, hq, d), generator=gen, dtype=torch.float32).to(torch.bfloat16)
    out = []
    for _ in range(2):
        codes = torch.empty((batch, hkv, max_len, d), dtype=torch.int8)
        for t0 in range(0, max_len, TOKEN_CHUNK):
            t1 = min(max_len, t0 + TOKEN_CHUNK)
            block = torch.randn((batch, hkv, t1 - t0, d), generator=gen, dtype=torch.float32)
            codes[:, :, t0:t1] = (block * 40).round().clamp(-127, 127).to(torch.int8)
        scales = (torch.rand((batch, hkv, max_len), generator=gen, dtype=torch.float32) + 2.5) / 127
        out += [codes, scales]
    return (lengths, q, *out)


def workload_decode_int8_inputs(w: DecodeWorkload, seed=None):
    return decode_int8_inputs(w.batch, w.hq, w.hkv, w.d, w.max_len, w.len_min, w.len_max,
                              w.seed if seed is None else seed)


def workload_decode_inputs(w: DecodeWorkload, seed=None):
    return decode_inputs(w.batch, w.hq, w.hkv, w.d, w.max_len, w.len_min, w.len_max, w.dtype,
                         w.seed if seed is None else seed)
