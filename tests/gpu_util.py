"""Helpers shared by the GPU parity tests: device, tolerances, comparison with a printed error
summary, row sampling, and a prefill input holder that permutes on the device with the library
while the oracle permutes its own host copy."""

import math

import numpy as np
import torch

import context_causal_attention_load_amd as cpa
from context_causal_attention_load_amd import synth
from oracle import attention as oatt
from oracle import lb_index as olb

DEV = "cuda:0"
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def announce(msg):
    print(f"\n[gpu case] {msg}", flush=True)


def assert_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    print(f"  {what}: max abs err {err.max():.3e} at {i} (tol {tol:g})", flush=True)
    assert err.max() <= tol, f"{what}: max abs err {err.max():.3e} at {i} > {tol}"


def sample_rows(c, n_random, seed):
    """First/last rows of both chunks of a shard plus seeded random rows (shard has 2c rows)."""
    edge = list(range(min(4, c))) + list(range(max(0, c - 4), c))
    edge += [c + x for x in edge]
    rng = np.random.default_rng(seed)
    rnd = rng.integers(0, 2 * c, n_random).tolist()
    return np.unique(np.array(edge + rnd, dtype=np.int64))


def stratified_rows(c, per_class, seed, block=32, edge=8):
    """Rows of a 2c-row shard for a sampled full-size check: the first and last ``edge`` rows of
    both chunks, plus ``per_class`` seeded rows for every position inside a 32-row block (the
    kernels' row blocks), drawn from different blocks across the whole shard."""
    n = 2 * c
    rows = set()
    for base in (0, c):
        rows.update(range(base, base + min(edge, c)))
        rows.update(range(max(base, base + c - edge), base + c))
    rng = np.random.default_rng(seed)
    nblk = (n + block - 1) // block
    for k in range(min(block, n)):
        cand = np.arange(k, n, block)
        take = min(per_class, len(cand))
        rows.update(rng.choice(cand, take, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def describe_rows(rows, c):
    """One line naming the checked rows: count, per-chunk counts, block-position coverage and the
    rows themselves as ranges."""
    rows = np.asarray(rows)
    spans, start = [], rows[0]
    for a, b in zip(rows[:-1], rows[1:]):
        if b != a + 1:
            spans.append((start, a))
            start = b
    spans.append((start, rows[-1]))
    txt = ",".join(f"{a}" if a == b else f"{a}-{b}" for a, b in spans)
    classes = len(set((rows % 32).tolist()))
    return (f"{len(rows)} rows ({int((rows < c).sum())} in the lower chunk, {int((rows >= c).sum())} in the upper), "
            f"{classes}/32 block positions: {txt}")


class Prefill:
    """Natural-order inputs on host and device, permuted on the device by the library; the
    oracle permutes the host copies itself. ``plant`` (optional) edits the host inputs in place
    before they are copied to the device."""

    def __init__(self, batch, seq, hq, hkv, dqk, dv, dtype, seed, scale=None, plant=None):
        self.seq, self.dtype = seq, dtype
        self.q, self.k, self.v = synth.prefill_inputs(batch, seq, hq, hkv, dqk, dv, dtype, seed)
        if plant is not None:
            plant(self.q, self.k)
        self.qd, self.kd, self.vd = (t.to(DEV) for t in (self.q, self.k, self.v))
        self.scale = 1.0 / math.sqrt(dqk) if scale is None else scale
        self._perm = {}
        self._ref_perm = {}

    def kv_perm(self, cp):
        if cp not in self._perm:
            self._perm[cp] = (cpa.permute(self.kd, cp), cpa.permute(self.vd, cp))
        return self._perm[cp]

    def ref_kv_perm(self, cp):
        if cp not in self._ref_perm:
            self._ref_perm = {cp: (oatt.permute_ref(self.k, self.seq, cp).double(),
                                   oatt.permute_ref(self.v, self.seq, cp).double())}
        return self._ref_perm[cp]

    def gpu_rank(self, cp, rank, q_positions=None, split=True):
        c = self.seq // (2 * cp)
        kp, vp = self.kv_perm(cp)
        qs = cpa.permute(self.qd, cp, row_begin=rank * 2 * c, row_count=2 * c)
        o, lse = cpa.attention_fwd(qs, kp, vp, cp, rank, q_positions=q_positions, scale=self.scale, split=split)
        torch.cuda.synchronize()
        return o, lse

    def oracle_rank(self, cp, rank, rows=None):
        c = self.seq // (2 * cp)
        qs = oatt.permute_ref(self.q, self.seq, cp, rank * 2 * c, 2 * c)
        pos = olb.shard_positions(self.seq, cp, rank)
        kp, vp = self.ref_kv_perm(cp)
        if rows is not None:
            qs, pos = qs[:, rows], pos[rows]
        return oatt.cp_attention_ref(qs, kp, vp, pos, self.seq, cp, self.scale)


def check_rank(pf, cp, rank, rows=None, tag="", split=True):
    announce(f"{tag} attention_fwd cp={cp} rank={rank} rows={'all' if rows is None else len(rows)}"
             f"{'' if split else ' (never split)'}")
    o, lse = pf.gpu_rank(cp, rank, split=split)
    O_ref, L_ref = pf.oracle_rank(cp, rank, rows)
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    if rows is not None:
        o, lse = o[:, rows], lse[:, :, rows]
    tol = TOL[pf.dtype]
    assert_close(o, O_ref, tol, f"{tag} O cp={cp} r={rank}")
    assert_close(lse, L_ref, tol, f"{tag} LSE cp={cp} r={rank}")
