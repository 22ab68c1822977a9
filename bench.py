"""Benchmark: one context-parallel rank's load-balanced causal GQA attention step on one MI355X.

Workload (default): Llama3.1-70B-shaped attention at 131072 tokens, 64 query heads / 8 KV
heads, head dim 128, bf16, cp = 8 (one rank's 16384-row query shard over the full K/V). One
step = the rank's whole share of the hot path, inputs resident in HBM:
  1. gather its query shard (window r*2c .. (r+1)*2c of the load-balanced order) from Q,
  2. gather its K and V shard into its slice of the all-gathered K/V buffers (the other ranks'
     slices were filled before timing: the all-gather itself needs other GPUs),
  3. causal attention forward over the full K/V (O and LSE),
  4. scatter O and LSE back to original token order.
Step i runs rank i % cp, so the timed steps cover every rank; per-rank times are reported.

After the timed steps (not part of them): every rank's attention kernel with the balanced
shard and with a contiguous shard of the natural order, to show the spread the load balance
removes (`load_balance`; skip with --no-balance-demo); and every rank's backward call
(`backward`; skip with --no-backward).

Also measured: GQA decode (Mixtral-8x22B shape, batch 24, 48/8 heads, D 128, cache 2048 with
lengths uniform in [1024, 2048]), rotating 4 cache copies so reads come from HBM rather than
the 256 MB last-level cache; the same decode over an int8-quantized cache (6 copies); every
rank's attention kernel at the other prefill shapes (`other_configs`: Llama2-7B MHA at 8192
tokens, cp 1 and 4; DeepSeek-V3 MLA at 32768 tokens, cp 4; skip with --no-other-configs); and
the CPU fp64 oracle on a bounded row sample of the same prefill workload (the CPU baseline),
plus the oracle over whole workloads at the small configs (`cpu_baseline.full_configs`). A plain
bf16 GEMM through torch.matmul is timed last as a reference for the matrix-core rate the part
sustains (`gemm_reference`; skip with --no-gemm-reference).

Prints one JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

METRIC = "causal attn fwd TFLOP/s + %MFMA peak (131k CP shard); decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def profiled_traffic(profile, sources):
    """HBM bytes per launch recorded in a committed rocprofv3 summary under profiles/ (FETCH_SIZE
    and WRITE_SIZE, scaled by a plain-copy calibration), or None when the summary is missing or
    any source file of the kernels has changed since the counters were taken: the summary lists
    ``source_sha256[<file>] = <hex>`` for each file and every one must match."""
    import hashlib
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
    except OSError:
        return None
    fields = dict(line.split(" = ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch = ", "source_sha256[")))
    for src in sources:
        try:
            data = open(os.path.join(ROOT, "context_causal_attention_load_amd", "csrc", src), "rb").read()
        except OSError:
            return None
        if fields.get(f"source_sha256[{src}]", "").strip() != hashlib.sha256(data).hexdigest():
            return None
    if "traffic_bytes_per_launch = " not in text:
        return None
    return int(fields["traffic_bytes_per_launch"])


def useful_flops(seq, cp, hq, dqk, dv, batch=1):
    # every rank of a balanced split sees exactly c*(S+1) causal (query, key) pairs
    c = seq // (2 * cp)
    pairs = c * (seq + 1)
    return 2.0 * pairs * hq * (dqk + dv) * batch


def bench_prefill(w, cp, steps, warmup, dev, balance_demo=True, backward=True):
    import context_causal_attention_load_amd as cpa
    from context_causal_attention_load_amd import synth

    q, k, v = synth.workload_prefill_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    del q, k, v
    S, c = w.seq, w.seq // (2 * cp)
    kp, vp = cpa.permute(kd, cp), cpa.permute(vd, cp)  # the all-gathered K/V (all ranks' slices)
    q_shard = torch.empty((w.batch, 2 * c, w.hq, w.d_qk), dtype=w.dtype, device=dev)
    o_shard = torch.empty((w.batch, 2 * c, w.hq, w.d_v), dtype=w.dtype, device=dev)
    lse_shard = torch.empty((w.batch, w.hq, 2 * c), dtype=torch.float32, device=dev)
    o_nat = torch.zeros((w.batch, S, w.hq, w.d_v), dtype=w.dtype, device=dev)
    lse_nat = torch.zeros((w.batch, w.hq, S), dtype=torch.float32, device=dev)
    assert w.batch == 1, "the K/V slice update below assumes batch 1"

    def step(r, ev=None):
        b0 = r * 2 * c
        cpa.permute(qd, cp, row_begin=b0, row_count=2 * c, out=q_shard)
        cpa.permute(kd, cp, row_begin=b0, row_count=2 * c, out=kp[:, b0:b0 + 2 * c])
        cpa.permute(vd, cp, row_begin=b0, row_count=2 * c, out=vp[:, b0:b0 + 2 * c])
        if ev is not None:
            ev[0].record()
        cpa.attention_fwd(q_shard, kp, vp, cp, r, scale=w.scale, out=o_shard, lse=lse_shard)
        if ev is not None:
            ev[1].record()
        cpa.unpermute(o_shard, cp, S, row_begin=b0, out=o_nat)
        cpa.unpermute(lse_shard, cp, S, dim=2, row_begin=b0, out=lse_nat)

    for i in range(warmup):
        step(i % cp)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    step_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step_evs[i][0].record()
        step(i % cp, evs[i])
        step_evs[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    step_ms = [a.elapsed_time(b) for a, b in step_evs]
    per_rank = {}
    for i in range(steps):
        per_rank.setdefault(i % cp, []).append(step_ms[i])
    out = dict(wall_s=wall, attn_ms=attn_ms, step_ms=step_ms,
               per_rank_ms={r: sum(v) / len(v) for r, v in sorted(per_rank.items())},
               flops=useful_flops(S, cp, w.hq, w.d_qk, w.d_v, w.batch))
    if balance_demo:
        out["balance"] = balance_demo_ms(w, cp, qd, kd, vd, kp, vp, q_shard, o_shard, lse_shard)
    if backward:
        out["backward"] = backward_ms(w, cp, kp, vp, qd, q_shard, o_shard, lse_shard)
    return out


def backward_flops(seq, cp, hq, dqk, dv, batch=1):
    """Useful backward flops of one rank: the five products over visible (query, key, head)
    triples, S = QK^T and dQ, dK (2 Dqk each), dP = dO V^T and dV (2 Dv each)."""
    c = seq // (2 * cp)
    return 2.0 * c * (seq + 1) * hq * (3 * dqk + 2 * dv) * batch


def backward_ms(w, cp, kp, vp, qd, q_shard, o_shard, lse_shard):
    """After the timed forward steps: for every rank, its forward (untimed) then its backward call
    (prep + dq + dkdv kernels), timed with HIP events on the launch stream. dO is a seeded
    N(0,1) draw on the device (timing only)."""
    import context_causal_attention_load_amd as cpa

    S, c = w.seq, w.seq // (2 * cp)
    gen = torch.Generator(device=qd.device).manual_seed(1000 + w.seed)
    d_o = torch.randn((w.batch, 2 * c, w.hq, w.d_v), generator=gen, device=qd.device, dtype=torch.float32).to(w.dtype)
    dq = torch.empty((w.batch, 2 * c, w.hq, w.d_qk), dtype=torch.float32, device=qd.device)
    dk = torch.empty((w.batch, S, w.hkv, w.d_qk), dtype=torch.float32, device=qd.device)
    dv = torch.empty((w.batch, S, w.hkv, w.d_v), dtype=torch.float32, device=qd.device)
    ws = torch.empty(cpa.attention_bwd_workspace_bytes(w.batch, 2 * c, w.hq), dtype=torch.uint8, device=qd.device)

    def run(r, ev=None):
        cpa.permute(qd, cp, row_begin=r * 2 * c, row_count=2 * c, out=q_shard)
        cpa.attention_fwd(q_shard, kp, vp, cp, r, scale=w.scale, out=o_shard, lse=lse_shard)
        if ev is not None:
            ev[0].record()
        cpa.attention_bwd(q_shard, kp, vp, o_shard, lse_shard, d_o, cp, r, scale=w.scale, workspace=ws, dq=dq,
                          dk=dk, dv=dv)
        if ev is not None:
            ev[1].record()

    run(0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(cp)]
    for r in range(cp):
        run(r, evs[r])
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return dict(ms=ms, flops=backward_flops(S, cp, w.hq, w.d_qk, w.d_v, w.batch))


def balance_demo_ms(w, cp, qd, kd, vd, kp, vp, q_shard, o_shard, lse_shard):
    """Outside the timed steps: every rank's attention kernel time with the load-balanced shard
    (chunks r and 2cp-1-r) and with a contiguous shard (rows r*S/cp .. of the natural order,
    K/V in natural order, given as explicit positions), one launch each after a warm-up."""
    import context_causal_attention_load_amd as cpa

    S, c = w.seq, w.seq // (2 * cp)

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    balanced, contiguous = [], []
    for r in range(cp):
        b0 = r * 2 * c
        cpa.permute(qd, cp, row_begin=b0, row_count=2 * c, out=q_shard)
        balanced.append(timed(lambda: cpa.attention_fwd(q_shard, kp, vp, cp, r, scale=w.scale, out=o_shard,
                                                        lse=lse_shard)))
        rows = torch.arange(b0, b0 + 2 * c, dtype=torch.int32, device=qd.device)
        q_rows = qd[:, b0:b0 + 2 * c]
        contiguous.append(timed(lambda: cpa.attention_fwd(q_rows, kd, vd, 1, 0, q_positions=rows, scale=w.scale,
                                                          out=o_shard, lse=lse_shard)))

    def spread(v):
        return max(v) / (sum(v) / len(v))

    return {"balanced_attn_ms_per_rank": [round(x, 3) for x in balanced],
            "contiguous_attn_ms_per_rank": [round(x, 3) for x in contiguous],
            "balanced_max_over_mean": round(spread(balanced), 4),
            "contiguous_max_over_mean": round(spread(contiguous), 4),
            "contiguous_max_over_mean_closed_form": round((2 * cp - 1) / cp, 4)}


def decode_bytes(w, lengths, elt=2):
    """Algorithmic HBM bytes of one decode call: the valid K and V rows of every sequence and kv
    head (elt bytes per element), q read and o written, the fp32 LSE written, the int32 lengths."""
    kv_bytes = int(lengths.sum()) * w.hkv * w.d * elt * 2
    io_bytes = w.batch * w.hq * w.d * elt * 2 + w.batch * w.hq * 4 + w.batch * 4
    return kv_bytes + io_bytes


def decode_int8_bytes(w, lengths):
    """The same over an int8 cache: one byte per K and V code plus a float32 scale per valid row
    of K and of V; q and o stay bf16."""
    rows = int(lengths.sum()) * w.hkv
    kv_bytes = rows * w.d * 2 + rows * 4 * 2
    io_bytes = w.batch * w.hq * w.d * 2 * 2 + w.batch * w.hq * 4 + w.batch * 4
    return kv_bytes + io_bytes


def _time_calls(call, iters):
    """Times ``call(i)`` two ways on the current stream: each call between its own pair of HIP
    events (sorted per-call milliseconds), and ``iters`` calls back to back between one pair
    (milliseconds per call, as a decode loop issues them)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i in range(iters):
        evs[i][0].record()
        call(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(iters):
        call(i)
    t1.record()
    torch.cuda.synchronize()
    return ms, t0.elapsed_time(t1) / iters


def _time_graph(call, check, reps=24, replays=10):
    """GPU time per call of a short call: ``reps`` calls captured in one HIP graph and replayed
    ``replays`` times between one pair of events, so the host's per-call launch cost does not
    enter (for calls of a few microseconds it exceeds the kernels). ``check()`` returns the
    call's outputs; after the replays they must equal those of an eager call bit for bit, else
    the figure is withheld (None)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [x.clone() for x in check()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            call(i)
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    call(reps - 1)  # eager again: the last captured call's inputs
    torch.cuda.synchronize()
    eager_last = [x.clone() for x in check()]
    g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(eager_last, check()))
    del g, eager
    return t0.elapsed_time(t1) / (replays * reps) if same else None


def gemm_reference(dev, n=16384, iters=10):
    """Sustained rate of a plain bf16 GEMM (n x n x n through torch.matmul, i.e. the vendor BLAS)
    on this part in the same run: a reference for how much of the spec-sheet matrix-core peak the
    part holds under load, so the attention kernel's fraction of peak can be read against it. Not
    part of the attention path."""
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del a, b, c
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"shape": f"{n}x{n}x{n} bf16 torch.matmul", "ms": round(ms, 3), "tflops": round(tf, 1),
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def other_configs_ms(dev, iters=5, bwd_iters=3):
    """Every rank's attention kernel at the other prefill shapes (the 8192-token Llama2-7B MHA at
    cp = 1 and cp = 4, the 32768-token DeepSeek-V3 MLA shape at cp = 4): HIP-event time of one
    launch after a warm-up, median of ``iters``; then every rank's backward call, median of
    ``bwd_iters``. Inputs are seeded N(0,1) draws on the device (timing only; these shapes'
    parity is in the tests)."""
    import context_causal_attention_load_amd as cpa
    from context_causal_attention_load_amd import synth

    out = []
    for w in (synth.LLAMA2_7B_S8K, synth.DEEPSEEK_V3_MLA_S32K):
        gen = torch.Generator(device=dev).manual_seed(w.seed)
        qd, kd, vd = (torch.randn((w.batch, w.seq, h, d), generator=gen, device=dev, dtype=torch.float32).to(w.dtype)
                      for h, d in ((w.hq, w.d_qk), (w.hkv, w.d_qk), (w.hkv, w.d_v)))
        for cp in w.cps:
            c = w.seq // (2 * cp)
            kp, vp = cpa.permute(kd, cp), cpa.permute(vd, cp)
            o = torch.empty((w.batch, 2 * c, w.hq, w.d_v), dtype=w.dtype, device=dev)
            lse = torch.empty((w.batch, w.hq, 2 * c), dtype=torch.float32, device=dev)
            # the split of heavy row blocks (small grids) gets its workspace before timing
            need = max(cpa.attention_fwd_workspace_bytes(w.batch, w.seq, w.hq, w.hkv, w.d_qk, w.d_v, w.dtype, cp, r)
                       for r in range(cp))
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            d_o = torch.randn((w.batch, 2 * c, w.hq, w.d_v), generator=gen, device=dev,
                              dtype=torch.float32).to(w.dtype)
            dq = torch.empty((w.batch, 2 * c, w.hq, w.d_qk), dtype=torch.float32, device=dev)
            dk = torch.empty((w.batch, w.seq, w.hkv, w.d_qk), dtype=torch.float32, device=dev)
            dv = torch.empty((w.batch, w.seq, w.hkv, w.d_v), dtype=torch.float32, device=dev)
            # the backward's workspace also holds the dQ pieces of heavy row blocks (small grids)
            bbase = cpa.attention_bwd_workspace_bytes(w.batch, 2 * c, w.hq)
            bneed = max(cpa.attention_bwd_split_workspace_bytes(w.batch, w.seq, w.hq, w.hkv, w.d_qk, w.d_v, w.dtype,
                                                                cp, r) for r in range(cp))
            bws = torch.empty(max(bneed, bbase), dtype=torch.uint8, device=dev)
            ms, bms = [], []
            for r in range(cp):
                qs = cpa.permute(qd, cp, row_begin=r * 2 * c, row_count=2 * c)
                cpa.attention_fwd(qs, kp, vp, cp, r, scale=w.scale, out=o, lse=lse, workspace=ws)
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
                for a, b in evs:
                    a.record()
                    cpa.attention_fwd(qs, kp, vp, cp, r, scale=w.scale, out=o, lse=lse, workspace=ws)
                    b.record()
                torch.cuda.synchronize()
                ms.append(sorted(a.elapsed_time(b) for a, b in evs)[iters // 2])
                def bwd(qs=qs, r=r):
                    cpa.attention_bwd(qs, kp, vp, o, lse, d_o, cp, r, scale=w.scale, workspace=bws, dq=dq, dk=dk, dv=dv)

                bwd()
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(bwd_iters)]
                for a, b in evs:
                    a.record()
                    bwd()
                    b.record()
                torch.cuda.synchronize()
                bms.append(sorted(a.elapsed_time(b) for a, b in evs)[bwd_iters // 2])
            flops = useful_flops(w.seq, cp, w.hq, w.d_qk, w.d_v, w.batch)
            avg = sum(ms) / len(ms)
            tf = flops / (avg * 1e-3) / 1e12
            bflops = backward_flops(w.seq, cp, w.hq, w.d_qk, w.d_v, w.batch)
            bavg = sum(bms) / len(bms)
            btf = bflops / (bavg * 1e-3) / 1e12
            out.append({"workload": f"{w.name} cp={cp}", "ms_per_rank": [round(x, 3) for x in ms],
                        "rank_max_over_mean": round(max(ms) / avg, 4), "heavy_row_blocks_split": need > 0,
                        "useful_flop_per_rank": flops, "tflops": round(tf, 1),
                        "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                        "backward": {"ms_per_rank": [round(x, 3) for x in bms],
                                     "rank_max_over_mean": round(max(bms) / bavg, 4),
                                     "heavy_row_blocks_dq_split": bneed > bbase, "useful_flop_per_rank": bflops,
                                     "tflops": round(btf, 1), "frac_of_bf16_peak": round(btf / PEAK_BF16_TFLOPS, 4)}})
            del d_o, dq, dk, dv, bws
        del qd, kd, vd
    return out


def bench_decode(w, iters, dev, copies=4):
    import context_causal_attention_load_amd as cpa
    from context_causal_attention_load_amd import synth

    lengths, q, kc, vc = synth.workload_decode_inputs(w)
    qd, ld = q.to(dev), lengths.to(dev)
    caches = [(kc.to(dev), vc.to(dev))]
    for _ in range(copies - 1):
        caches.append((caches[0][0].clone(), caches[0][1].clone()))
    ws = torch.empty(cpa.decode_workspace_bytes(w.batch, w.hq, w.hkv, w.max_len, w.d), dtype=torch.uint8, device=dev)
    out = torch.empty((w.batch, w.hq, w.d), dtype=w.dtype, device=dev)
    lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=dev)
    for i in range(copies):
        cpa.decode(qd, caches[i][0], caches[i][1], ld, scale=w.scale, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()

    def call(i):
        kci, vci = caches[i % copies]
        cpa.decode(qd, kci, vci, ld, scale=w.scale, workspace=ws, out=out, lse=lse)

    ms, b2b = _time_calls(call, iters)
    alg = decode_bytes(w, lengths)
    med = ms[len(ms) // 2]
    return dict(median_ms=med, min_ms=ms[0], b2b_ms=b2b, bytes=alg, gbs=alg / (med * 1e-3) / 1e9,
                b2b_gbs=alg / (b2b * 1e-3) / 1e9)


def bench_decode_sharded(w, iters, dev, shards=4, copies=6):
    """The decode batch with its cache split along the length into ``shards`` equal slices, one
    per rank of an inference context-parallel job: each rank decodes over its own slice (the
    one-GPU part, timed slice by slice, rotating ``copies`` copies of the slice so reads come
    from HBM), then the ranks' (o, LSE) partials, once all-gathered, are combined by
    gqa_decode_merge (timed on its own). The all-gather itself needs a second GPU."""
    import context_causal_attention_load_amd as cpa
    from context_causal_attention_load_amd import synth

    lengths, q, kc, vc = synth.workload_decode_inputs(w)
    W = w.max_len // shards
    qd = q.to(dev)
    o_parts = torch.empty((shards, w.batch, w.hq, w.d), dtype=w.dtype, device=dev)
    l_parts = torch.empty((shards, w.batch, w.hq), dtype=torch.float32, device=dev)
    ws = torch.empty(cpa.decode_workspace_bytes(w.batch, w.hq, w.hkv, W, w.d), dtype=torch.uint8, device=dev)
    per = []
    for r in range(shards):
        n = torch.clamp(lengths - r * W, 0, W).to(torch.int32)
        nd = n.to(dev)
        sl = [(kc[:, :, r * W:(r + 1) * W].contiguous().to(dev), vc[:, :, r * W:(r + 1) * W].contiguous().to(dev))]
        for _ in range(copies - 1):
            sl.append((sl[0][0].clone(), sl[0][1].clone()))

        def call(i, sl=sl, nd=nd, r=r):
            kci, vci = sl[i % copies]
            cpa.decode(qd, kci, vci, nd, scale=w.scale, workspace=ws, out=o_parts[r], lse=l_parts[r])

        for i in range(copies):
            call(i)
        torch.cuda.synchronize()
        ms, b2b = _time_calls(call, iters)
        gms = _time_graph(call, lambda r=r: (o_parts[r], l_parts[r]), reps=4 * copies)
        alg = decode_bytes(w, n)
        per.append(dict(median_ms=ms[len(ms) // 2], b2b_ms=b2b, graph_ms=gms, bytes=alg, keys=int(n.sum())))
        del sl, call
    out = torch.empty((w.batch, w.hq, w.d), dtype=w.dtype, device=dev)
    lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=dev)
    cpa.decode_merge(o_parts, l_parts, out=out, lse=lse)
    torch.cuda.synchronize()
    mms, mb2b = _time_calls(lambda i: cpa.decode_merge(o_parts, l_parts, out=out, lse=lse), iters)
    mgms = _time_graph(lambda i: cpa.decode_merge(o_parts, l_parts, out=out, lse=lse), lambda: (out, lse))
    return dict(shards=per, merge_median_ms=mms[len(mms) // 2], merge_b2b_ms=mb2b, merge_graph_ms=mgms,
                merge_bytes=o_parts.numel() * o_parts.element_size() + l_parts.numel() * 4
                + out.numel() * out.element_size() + lse.numel() * 4)


def bench_decode_int8(w, iters, dev, copies=6):
    """The same decode batch over an int8 cache (codes plus one float32 scale per cached row),
    rotating ``copies`` caches so reads come from HBM."""
    import context_causal_attention_load_amd as cpa
    from context_causal_attention_load_amd import synth

    lengths, q, kq, ks, vq, vs = synth.workload_decode_int8_inputs(w)
    qd, ld = q.to(dev), lengths.to(dev)
    caches = [tuple(t.to(dev) for t in (kq, ks, vq, vs))]
    for _ in range(copies - 1):
        caches.append(tuple(t.clone() for t in caches[0]))
    ws = torch.empty(cpa.decode_workspace_bytes(w.batch, w.hq, w.hkv, w.max_len, w.d), dtype=torch.uint8, device=dev)
    out = torch.empty((w.batch, w.hq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.hq), dtype=torch.float32, device=dev)
    for c in caches:
        cpa.decode_int8(qd, c[0], c[1], c[2], c[3], ld, scale=w.scale, workspace=ws, out=out, lse=lse)
    torch.cuda.synchronize()

    def call(i):
        c = caches[i % copies]
        cpa.decode_int8(qd, c[0], c[1], c[2], c[3], ld, scale=w.scale, workspace=ws, out=out, lse=lse)

    ms, b2b = _time_calls(call, iters)
    alg = decode_int8_bytes(w, lengths)
    med = ms[len(ms) // 2]
    return dict(median_ms=med, min_ms=ms[0], b2b_ms=b2b, bytes=alg, gbs=alg / (med * 1e-3) / 1e9,
                b2b_gbs=alg / (b2b * 1e-3) / 1e9)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, cp, rank, n_rows, seed=0):
    """Time the CPU fp64 oracle (as it is) on a row sample of one rank: its permutes of the
    rank's windows plus attention for the sampled query rows over all heads. The sample is
    stratified: the first and last 8 rows of both chunks, the rest drawn uniformly from the shard.
    Reports useful TFLOP/s on the sampled rows' causal pairs and, from that rate, the time the
    oracle would take for the whole shard (labelled extrapolated)."""
    import numpy as np

    from context_causal_attention_load_amd import synth
    from oracle import attention as oatt
    from oracle import lb_index as olb

    q, k, v = synth.workload_prefill_inputs(w)
    S, c = w.seq, w.seq // (2 * cp)
    rng = np.random.default_rng(seed)
    edge = [x for base in (0, c) for x in list(range(base, base + 8)) + list(range(base + c - 8, base + c))]
    rows = np.unique(np.concatenate([np.array(edge), rng.integers(0, 2 * c, max(0, n_rows - len(edge)))]))
    pos = olb.shard_positions(S, cp, rank)
    t0 = time.perf_counter()
    qs = oatt.permute_ref(q, S, cp, rank * 2 * c, 2 * c)[:, rows]
    kp = oatt.permute_ref(k, S, cp)
    vp = oatt.permute_ref(v, S, cp)
    oatt.cp_attention_ref(qs, kp, vp, pos[rows], S, cp, w.scale)
    dt = time.perf_counter() - t0
    pairs = int((pos[rows] + 1).sum())
    flops = 2.0 * pairs * w.hq * (w.d_qk + w.d_v) * w.batch
    rate = flops / dt
    full = useful_flops(S, cp, w.hq, w.d_qk, w.d_v, w.batch)
    threads = torch.get_num_threads()
    return dict(value=rate / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=(f"{len(rows)} query rows of rank {rank} at S={S}, cp={cp} (first/last 8 rows of both chunks "
                        f"plus uniform random rows), all {w.hq} heads: oracle permutes of the Q window and the full "
                        f"K/V plus fp64 attention, {dt:.1f} s for {flops / 1e12:.3f} useful TFLOP"),
                extrapolated_full_shard_s=round(full / rate, 1),
                cpu_model=_cpu_model(), torch_threads=threads, affinity_cores=len(os.sched_getaffinity(0)),
                seconds=dt)


def cpu_baseline_full_configs():
    """Time the CPU fp64 oracle (as it is) over whole workloads at the small configs: every rank
    of the 512-token cp=2 fp32 case, the 8192-token Llama2-7B shape at cp=1 and every rank at
    cp=4 (each rank's permutes of its windows plus attention over its full shard), and the
    Mixtral-8x22B-shaped decode over the whole batch. Rates are useful causal TFLOP/s for the
    prefills and algorithmic GB/s for the decode."""
    from context_causal_attention_load_amd import synth
    from oracle import attention as oatt
    from oracle import lb_index as olb

    out = []
    for w in (synth.TINY_CP2_F32, synth.LLAMA2_7B_S8K):
        q, k, v = synth.workload_prefill_inputs(w)
        for cp in w.cps:
            S, c = w.seq, w.seq // (2 * cp)
            t0 = time.perf_counter()
            for r in range(cp):
                qs = oatt.permute_ref(q, S, cp, r * 2 * c, 2 * c)
                kp = oatt.permute_ref(k, S, cp)
                vp = oatt.permute_ref(v, S, cp)
                oatt.cp_attention_ref(qs, kp, vp, olb.shard_positions(S, cp, r), S, cp, w.scale)
            dt = time.perf_counter() - t0
            flops = cp * useful_flops(S, cp, w.hq, w.d_qk, w.d_v, w.batch)
            out.append({"workload": f"{w.name} cp={cp}, all {cp} rank(s)", "seconds": round(dt, 3),
                        "value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s"})
    dw = synth.MIXTRAL_8X22B_DECODE
    lengths, q, kc, vc = synth.workload_decode_inputs(dw)
    t0 = time.perf_counter()
    oatt.decode_ref(q, kc, vc, lengths.numpy(), dw.scale)
    dt = time.perf_counter() - t0
    nbytes = decode_bytes(dw, lengths)
    out.append({"workload": dw.name, "seconds": round(dt, 3), "value": round(nbytes / dt / 1e9, 3),
                "unit": "GB/s"})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=24)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-iters", type=int, default=200)
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass timing (after the timed forward steps)")
    ap.add_argument("--no-balance-demo", action="store_true",
                    help="skip the per-rank balanced vs contiguous shard timing (after the timed steps)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the per-rank attention timing at the other prefill shapes")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the plain bf16 GEMM timed as a reference for the part's sustained matrix-core rate")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share (one context-parallel rank) and does not run on more than "
              "one GPU", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    from context_causal_attention_load_amd import synth

    dev = "cuda:0"
    w = synth.LLAMA31_70B_S131K
    cp = w.cps[0]
    pre = bench_prefill(w, cp, args.steps, args.warmup, dev, balance_demo=not args.no_balance_demo,
                        backward=not args.no_backward)
    ms_per_step = sum(pre["step_ms"]) / len(pre["step_ms"])
    value = pre["flops"] / (ms_per_step * 1e-3) / 1e12
    attn_avg_ms = sum(pre["attn_ms"]) / len(pre["attn_ms"])
    achieved = pre["flops"] / (attn_avg_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: one rank's 16384-row query shard over full K/V", "batch": w.batch,
                   "seq_len": w.seq, "cp": cp, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim_qk": w.d_qk,
                   "head_dim_v": w.d_v, "parallelism": "one context-parallel rank (cp=8) per GPU",
                   "ranks_timed": sorted(pre["per_rank_ms"].keys())},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic("attn_fwd_bf16_llama70b_s131072_cp8.md",
                                                 ("attn_fwd.hip", "attn_tiles.h", "common.h")),
                     "traffic_unit": "HBM bytes per launch",
                     "kernel": "attn_fwd_bf16_kernel<128,128>", "kernel_avg_ms": round(attn_avg_ms, 4),
                     "kernel_median_ms": round(sorted(pre["attn_ms"])[len(pre["attn_ms"]) // 2], 4),
                     "kernel_min_ms": round(min(pre["attn_ms"]), 4),
                     "useful_flop_per_launch": pre["flops"]},
        "per_rank_step_ms": {str(r): round(t, 3) for r, t in pre["per_rank_ms"].items()},
    }
    if "balance" in pre:
        result["load_balance"] = pre["balance"]
    if "backward" in pre:
        bw = pre["backward"]
        bms = sum(bw["ms"]) / len(bw["ms"])
        btf = bw["flops"] / (bms * 1e-3) / 1e12
        result["backward"] = {
            "workload": f"{w.name}: one rank's backward (dQ of its shard, its dK/dV share over the full K/V)",
            "value": round(btf, 2), "unit": "TFLOP/s", "ms_per_rank_avg": round(bms, 3),
            "per_rank_ms": {str(r): round(t, 3) for r, t in enumerate(bw["ms"])},
            "roofline": {"bound": "mfma", "achieved": round(btf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(btf / PEAK_BF16_TFLOPS, 4),
                         "traffic": profiled_traffic("attn_bwd_bf16_llama70b_s131072_cp8.md",
                                                     ("attn_bwd.hip", "attn_tiles.h", "common.h")),
                         "traffic_unit": "HBM bytes per call (prep + dq + dkdv)",
                         "kernel": "cp_attention_bwd call (bwd_delta + attn_bwd_dq + attn_bwd_dkdv)",
                         "useful_flop_per_call": bw["flops"]}}
    if not args.no_decode:
        dw = synth.MIXTRAL_8X22B_DECODE
        d = bench_decode(dw, args.decode_iters, dev)
        result["decode"] = {"workload": dw.name, "value": round(d["gbs"], 1), "unit": "GB/s",
                            "median_us": round(d["median_ms"] * 1e3, 2), "min_us": round(d["min_ms"] * 1e3, 2),
                            "back_to_back_us": round(d["b2b_ms"] * 1e3, 2),
                            "back_to_back_gbs": round(d["b2b_gbs"], 1),
                            "roofline": {"bound": "hbm", "achieved": round(d["gbs"], 1), "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": round(d["gbs"] / PEAK_HBM_GBS, 4),
                                         "traffic": profiled_traffic("decode_gqa_mixtral8x22b_b24_l2048.md",
                                                                     ("decode.hip", "common.h")),
                                         "traffic_unit": "HBM bytes per call (split + merge)",
                                         "algorithmic_bytes": d["bytes"]}}
        d8 = bench_decode_int8(dw, args.decode_iters, dev)
        result["decode_int8"] = {
            "workload": dw.name + " with the KV cache quantized to int8 (one float32 scale per cached row)",
            "value": round(d8["gbs"], 1), "unit": "GB/s", "median_us": round(d8["median_ms"] * 1e3, 2),
            "min_us": round(d8["min_ms"] * 1e3, 2), "back_to_back_us": round(d8["b2b_ms"] * 1e3, 2),
            "back_to_back_gbs": round(d8["b2b_gbs"], 1),
            "roofline": {"bound": "hbm", "achieved": round(d8["gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(d8["gbs"] / PEAK_HBM_GBS, 4),
                         "traffic": profiled_traffic("decode_int8_mixtral8x22b_b24_l2048.md",
                                                     ("decode_int8.hip", "decode.hip", "common.h")),
                         "traffic_unit": "HBM bytes per call (split + merge)", "algorithmic_bytes": d8["bytes"]}}
        ds = bench_decode_sharded(dw, args.decode_iters, dev)
        busiest = max(ds["shards"], key=lambda s: s["median_ms"])
        bgbs = busiest["bytes"] / (busiest["median_ms"] * 1e-3) / 1e9
        us = lambda x: None if x is None else round(x * 1e3, 2)
        result["decode_length_sharded"] = {
            "workload": dw.name + f" with the cache split along its length into {len(ds['shards'])} slices "
                        "(one per rank of an inference context-parallel job)",
            "value": round(bgbs, 1), "unit": "GB/s (the slowest rank's slice)",
            "shard_median_us": [round(s["median_ms"] * 1e3, 2) for s in ds["shards"]],
            "shard_back_to_back_us": [round(s["b2b_ms"] * 1e3, 2) for s in ds["shards"]],
            "shard_graph_replay_us": [us(s["graph_ms"]) for s in ds["shards"]],
            "shard_keys": [s["keys"] for s in ds["shards"]],
            "merge_median_us": round(ds["merge_median_ms"] * 1e3, 2),
            "merge_back_to_back_us": round(ds["merge_b2b_ms"] * 1e3, 2),
            "merge_graph_replay_us": us(ds["merge_graph_ms"]),
            "timing_note": "median and back-to-back figures are host-issued calls (each includes the "
                           "binding's checks and a launch); graph-replay figures are GPU time per call",
            "rank_critical_path_us": round((busiest["median_ms"] + ds["merge_median_ms"]) * 1e3, 2),
            "rank_critical_path_graph_replay_us": (
                None if ds["merge_graph_ms"] is None or any(s["graph_ms"] is None for s in ds["shards"])
                else us(max(s["graph_ms"] for s in ds["shards"]) + ds["merge_graph_ms"])),
            "roofline": {"bound": "hbm", "achieved": round(bgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(bgbs / PEAK_HBM_GBS, 4), "traffic": None,
                         "algorithmic_bytes": busiest["bytes"]}}
    if not args.no_other_configs:
        result["other_configs"] = other_configs_ms(dev)
    if not args.no_gemm_reference:
        result["gemm_reference"] = gemm_reference(dev)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, cp, 0, args.cpu_rows)
        cb.pop("seconds")
        result["cpu_baseline"] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in cb.items()}
        result["cpu_baseline"]["full_configs"] = cpu_baseline_full_configs()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
