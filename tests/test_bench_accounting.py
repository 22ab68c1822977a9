"""CPU checks of bench.py's accounting: the useful flops and algorithmic bytes that every reported
throughput and roofline fraction divides by, pinned to the oracle's index math (a causal pair
count over the load-balanced positions) and to the figures the design states, and the rule that
a profiled traffic figure is used only while the kernel sources it was taken from are unchanged."""

import hashlib

import numpy as np
import pytest

import bench
from context_causal_attention_load_amd import synth
from oracle import lb_index as olb


@pytest.mark.parametrize("seq,cp,hq,dqk,dv", [(16, 2, 2, 8, 8), (48, 3, 4, 16, 8), (512, 2, 4, 64, 64),
                                              (8192, 4, 32, 128, 128), (4096, 8, 8, 192, 128)])
def test_useful_flops_match_oracle_pair_count(seq, cp, hq, dqk, dv):
    perm = olb.load_balance_perm(seq, cp)
    for r in range(cp):
        pairs = olb.causal_pair_count(olb.shard_positions(seq, cp, r), perm)
        assert bench.useful_flops(seq, cp, hq, dqk, dv) == 2.0 * pairs * hq * (dqk + dv)
        # backward: the five products S, dP, dV, dK, dQ over the same pairs
        assert bench.backward_flops(seq, cp, hq, dqk, dv) == 2.0 * pairs * hq * (3 * dqk + 2 * dv)


def test_headline_figures():
    # one rank of the 131072-token Llama3.1-70B shape at cp = 8: c (S + 1) = 8192 * 131073 pairs
    assert bench.useful_flops(131072, 8, 64, 128, 128) == 35_184_640_524_288
    assert bench.backward_flops(131072, 8, 64, 128, 128) == 87_961_601_310_720
    assert bench.backward_flops(131072, 8, 64, 128, 128) == 2.5 * bench.useful_flops(131072, 8, 64, 128, 128)
    # DeepSeek-V3 MLA shape, one rank at cp = 4
    assert bench.useful_flops(32768, 4, 128, 192, 128) == 10_995_451_822_080


def test_decode_bytes():
    w = synth.MIXTRAL_8X22B_DECODE
    lengths, _, _, _ = synth.workload_decode_inputs(w)
    lens = lengths.numpy().astype(np.int64)
    # every valid cache row of K and V once (bf16), q in, o out, fp32 LSE out, int32 lengths in
    expect = int(lens.sum()) * w.hkv * w.d * 2 * 2 + w.batch * w.hq * w.d * 2 * 2 + w.batch * w.hq * 4 + w.batch * 4
    assert bench.decode_bytes(w, lengths) == expect
    assert bench.decode_bytes(w, lengths) == 150_467_168  # the seed-5 figure the design quotes
    # int8 cache: a byte per code and a float32 scale per valid row, for K and for V
    rows = int(lens.sum()) * w.hkv
    assert bench.decode_int8_bytes(w, lengths) == rows * (w.d + 4) * 2 + w.batch * w.hq * w.d * 4 + w.batch * w.hq * 4 + w.batch * 4
    assert bench.decode_int8_bytes(w, lengths) == 77_872_608


def test_profiled_traffic_only_while_sources_match(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "context_causal_attention_load_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_bytes(b"kernel source\n")
    digest = hashlib.sha256(b"kernel source\n").hexdigest()
    (tmp_path / "profiles" / "p.md").write_text(
        f"# summary\n\ntraffic_bytes_per_launch = 12345\nsource_sha256[k.hip] = {digest}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("p.md", ("k.hip",)) == 12345
    (csrc / "k.hip").write_bytes(b"kernel source, changed\n")
    assert bench.profiled_traffic("p.md", ("k.hip",)) is None
    assert bench.profiled_traffic("missing.md", ("k.hip",)) is None


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU's share; a request for several GPUs ends with a message and a
    non-zero status before anything runs."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
