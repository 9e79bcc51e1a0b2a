#!/usr/bin/env python3
"""Benchmark of the ReSA decode hot path on one MI355X.

Workload (default): one request at 262144 tokens of context through a stack
of 28 independent Qwen2.5-7B-shaped attention layers (28 query heads over 4
KV heads, head dim 128, bf16, block 16, 10% block budget = 1639 of 16384
blocks per KV head).  Inputs are seeded synthetic data (see synth/).

A step is one decoded token through all 28 layers; per layer it runs the
whole sparse path: resa_score_select (with the tail-descriptor refresh of
the block holding the newest token, in the same launch) and
resa_sparse_decode.  The 28-layer step is
captured once into a HIP graph and replayed, so the timing holds GPU work
only (the pages measure kernel time without CPU overhead, §5).  Reported:

* value: microseconds per layer-step (lower is better);
* achieved HBM GB/s of the layer-step on its algorithmic bytes;
* the build's own dense decode (resa_dense_decode) at the same shape;
* the rectification call (window 32) at the same shape, and at the
  rectification workload (4 requests x 131072 tokens, window 64);
* a streaming reference measured in the same run: the runtime's device copy
  at 54 MiB (the sparse decode's size) and at 1 GiB, timed with HIP events;
* roofline of the dominant kernel (sparse decode): the event-timed call, the
  kernel's own duration from the committed kernel trace, the whole step;
* the CPU oracle timed on bounded samples (a 256K layer-step, a 32K
  layer-step, one rectification of a 131K KV head), on every core this
  process may use.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-decode attention µs/layer-step & achieved HBM GB/s at 256K ctx"
PEAK_HBM_GBPS = 8000.0
SEED = 2024
RECT_CHUNK = 32


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_bytes(spec, L, n_sel, e):
    """Bytes the method must move per layer-step (descriptors, selected K/V
    rows, q, fp32 output), per Eq 6's accounting with a 10% attended fraction."""
    H, g, d = spec.num_kv_heads, spec.group_size, spec.head_dim
    M = (L + 15) // 16
    tail_rows = L - (M - 1) * 16
    desc = H * M * 2 * d * e
    kv = H * ((n_sel - 1) * 16 + tail_rows) * 2 * d * e
    q = H * g * d * e
    out = H * g * d * 4
    return {"desc": desc, "kv": kv, "q": q, "out": out, "total": desc + kv + q + out}


def layers_for_fresh_reads(spec, lens, e=2):
    """Number of independent layer caches a timed replay cycles through so
    that the bytes one replay touches (descriptors + selected K/V, at the
    default 10 % budget) exceed 1 GiB, four times the 256 MB last-level
    cache: every step then reads its data from HBM, as in a model whose other
    layers' traffic evicts it between steps.  Between 2 and 256 caches."""
    touched = sum(algorithmic_bytes(spec, L, max(16, -(-((L + 15) // 16) // 10)), e)["total"] for L in lens)
    return max(2, min(256, -(-(1 << 30) // touched)))


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_sparse_attention_resa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_hash):
    """HBM bytes per launch of the sparse decode call and the kernel-trace
    durations of its two kernels, from the committed rocprofv3 summary, if it
    was taken on the current kernel source (else (None, None))."""
    path = os.path.join(ROOT, "profiles", "sparse_decode_traffic_256k.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, None
    if rec.get("kernel_source_hash") != kernel_hash:
        return None, None
    return rec.get("hbm_bytes_per_launch"), rec.get("rocprof_avg_us")


C5_NAME = "qwen7b_ctx131k_b4_rectify"
C2_NAME = "qwen7b_ctx32k_b1"


def oracle_layer_step(O, qs, Ks, Vs, desc, L, scale):
    """One layer-step of the oracle: per KV head the tail block's descriptor,
    the block scores, the selection and attention over the selected blocks."""
    for i in range(len(qs)):
        lo, hi = desc[i]
        lo[-1], hi[-1] = O.block_descriptor(Ks[i], L, (L + 15) // 16 - 1)
        S = O.scores(qs[i], lo, hi)
        blocks = O.select(S)
        O.attend(qs[i], Ks[i], Vs[i], L, blocks, scale)


def time_reps(fn, budget_s, max_reps):
    reps = 0
    t0 = time.perf_counter()
    while reps < 1 or (time.perf_counter() - t0 < budget_s and reps < max_reps):
        fn()
        reps += 1
    return (time.perf_counter() - t0) / reps, reps


def cpu_oracle_legs(O, np, torch, spec4, keep0, scale):
    """The oracle (fp64 NumPy, as it stands) on the host's cores: the 256K
    layer-step (the headline unit), a 32K layer-step and the rectification of
    one 131K KV head at window 64.  The two layer-steps use the workloads'
    seeded synthetic layers (the 256K one is the GPU run's layer 0); the
    rectification's cache is seeded N(0, 1) rows of the same shape (the
    oracle's cost does not depend on the values).  Returns the cpu_baseline
    record."""
    from threadpoolctl import threadpool_limits

    from synth import WORKLOADS, make_layer, make_rectify_inputs

    cores = len(os.sched_getaffinity(0))
    f64 = lambda t: t.float().numpy().astype(np.float64)
    legs = {}
    with threadpool_limits(limits=cores):
        # 256K layer-step (layer 0 of the timed stack)
        q0, k0, v0 = keep0
        H, g = spec4.num_kv_heads, spec4.group_size
        L4 = spec4.seq_lens[0]
        qs = [f64(q0[0, i * g:(i + 1) * g]) for i in range(H)]
        Ks = [f64(k0[0][i]) for i in range(H)]
        Vs = [f64(v0[0][i]) for i in range(H)]
        desc = [O.descriptors(Ks[i], L4) for i in range(H)]  # the cache state before the step (not timed)
        sec, reps = time_reps(lambda: oracle_layer_step(O, qs, Ks, Vs, desc, L4, scale), 10.0, 5)
        legs["ctx256k_layer_step_us"] = round(sec * 1e6, 1)
        legs["ctx256k_reps"] = reps
        del Ks, Vs, desc
        # 32K layer-step
        spec2 = WORKLOADS[C2_NAME]
        inp = make_layer(spec2, seed=SEED, layer=0)
        L2 = spec2.seq_lens[0]
        qs = [f64(inp.q[0, i * g:(i + 1) * g]) for i in range(H)]
        Ks = [f64(inp.keys[0][i]) for i in range(H)]
        Vs = [f64(inp.values[0][i]) for i in range(H)]
        desc = [O.descriptors(Ks[i], L2) for i in range(H)]
        sec, reps = time_reps(lambda: oracle_layer_step(O, qs, Ks, Vs, desc, L2, scale), 4.0, 20)
        legs["ctx32k_layer_step_us"] = round(sec * 1e6, 1)
        legs["ctx32k_reps"] = reps
        del inp, Ks, Vs, desc
        # rectification of one KV head of one 131K request at window 64; the
        # call rectifies 4 requests x 4 KV heads, so the per-call figure is 16x
        spec5 = WORKLOADS[C5_NAME]
        f = spec5.rectify_chunk
        L5 = spec5.seq_lens[0]
        k5 = torch.Generator().manual_seed(SEED)
        K5 = np.asarray(torch.randn((L5, spec5.head_dim), generator=k5).to(torch.bfloat16).float().numpy(),
                        dtype=np.float64)
        V5 = np.asarray(torch.randn((L5, spec5.head_dim), generator=k5).to(torch.bfloat16).float().numpy(),
                        dtype=np.float64)
        qc, kn, vn = make_rectify_inputs(spec5.with_(num_requests=1), 131, f)
        qh, knh, vnh = f64(qc[0, :, :g]), f64(kn[0, :, 0]), f64(vn[0, :, 0])
        sec, reps = time_reps(lambda: O.rectify(qh, knh, vnh, K5, V5, L5, scale), 1.0, 1)
        units = spec5.num_requests * spec5.num_kv_heads
        legs["rectify_131k_f64_us_per_call"] = round(sec * 1e6 * units, 1)
        legs["rectify_sample_kv_heads"] = 1
        del K5, V5
    return {"value": legs["ctx256k_layer_step_us"], "unit": "us/layer-step", "cores": cores, "kind": "oracle",
            "sample": (f"256K: {legs['ctx256k_reps']} layer-step(s) of layer 0 (4 KV heads: tail descriptor, "
                       f"16384 block scores, top-1639 selection, attention over the selected blocks); 32K: "
                       f"{legs['ctx32k_reps']} layer-step(s); rectification: one KV head of one 131072-token "
                       f"request at window 64, scaled by the call's 16 (request, KV head) pairs; "
                       f"NumPy fp64 on {cores} threads"),
            "legs": legs}


def copy_reference(torch, nbytes, reps):
    """The runtime's device copy (torch copy_) of nbytes, timed with HIP events
    over back-to-back copies that cycle through enough buffer pairs to touch
    more than 1 GiB, so no copy reads from the last-level cache.  Returns
    (us per copy, GB/s counting the bytes read and written)."""
    n = nbytes // 2
    nbuf = max(1, min(24, -(-(1 << 30) // nbytes)))
    src = [torch.ones(n, dtype=torch.bfloat16, device="cuda") for _ in range(nbuf)]
    dst = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(nbuf)]
    for j in range(nbuf):
        dst[j].copy_(src[j])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(reps):
        dst[k % nbuf].copy_(src[k % nbuf])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return us, 2 * nbytes / (us * 1e-6) / 1e9


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen7b_ctx256k_l28")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (for profiler runs)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (HBM counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line: context x budget x scoring-mode table (markdown)")
    ap.add_argument("--cycle", action="store_true",
                    help="instead of the headline line: the decoding loop at 256K (32 sparse steps at growing "
                         "lengths, then the rectification of the last 32 positions, per layer), amortised")
    ap.add_argument("--workloads", action="store_true",
                    help="instead of the headline line: every bf16 workload (batch, ragged, 131K + rectify) "
                         "as a markdown table")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_sparse_attention_resa_amd as resa
    from synth import WORKLOADS, make_layer, make_paged

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    resa.load_library()
    torch.cuda.set_device(0)
    if args.sweep:
        return sweep(args)
    if args.workloads:
        return workloads(args)
    if args.cycle:
        return cycle(args)
    spec = WORKLOADS[args.workload]
    assert spec.num_requests == 1 and spec.dtype == "bf16"
    L = spec.seq_lens[0]
    H, g, d = spec.num_kv_heads, spec.group_size, spec.head_dim
    e = 2
    cfg = resa.Config(num_kv_heads=H, group_size=g, head_dim=d, dtype=resa.RESA_BF16)
    nlayers = spec.layers

    # ---------------------------------------------------------------- setup
    t_setup = time.perf_counter()
    layers = []
    keep0 = None
    for l in range(nlayers):
        inp = make_layer(spec, seed=SEED, layer=l, device="cuda")
        pg = make_paged(inp)
        if l == 0 and not args.no_cpu_baseline:
            keep0 = (inp.q.cpu(), [k.cpu() for k in inp.keys], [v.cpu() for v in inp.values])
        kv = resa.PagedKV(pg.k_pool, pg.v_pool, pg.desc_pool, pg.block_table, pg.seq_lens)
        resa.build_descriptors(cfg, kv)
        layers.append({"kv": kv, "q": inp.q})
        del inp
        if (l + 1) % 7 == 0:
            torch.cuda.synchronize()
            log(f"layer {l + 1}/{nlayers} generated")
    mb = layers[0]["kv"].max_blocks
    ms = resa.selection_count(cfg, mb)
    n_sel = resa.selection_count(cfg, (L + 15) // 16)
    for st in layers:
        st["sel_idx"] = torch.empty((1, H, ms), dtype=torch.int32, device="cuda")
        st["sel_cnt"] = torch.empty((1, H), dtype=torch.int32, device="cuda")
        st["out"] = torch.empty((1, H * g, d), dtype=torch.float32, device="cuda")
        st["out_dense"] = torch.empty((1, H * g, d), dtype=torch.float32, device="cuda")
    ws_sel = resa.alloc_workspace(cfg, resa.OP_SCORE_SELECT, 1, mb, ms)
    ws_dec = resa.alloc_workspace(cfg, resa.OP_SPARSE_DECODE, 1, mb, ms)
    ws_den = resa.alloc_workspace(cfg, resa.OP_DENSE_DECODE, 1, mb)
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f}s, {nlayers} layers, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB resident")

    def tail_refresh(st):
        resa.build_descriptors(cfg, st["kv"], None, 1)

    def score_select(st):
        # refresh_tail: the descriptor of the block holding the newest token is
        # recomputed inside the same launch (the incremental block-key-cache update)
        resa.score_select(cfg, st["kv"], st["q"], st["sel_idx"], st["sel_cnt"], ws_sel, refresh_tail=True)

    def sparse_decode(st):
        resa.sparse_decode(cfg, st["kv"], st["q"], st["sel_idx"], st["sel_cnt"], st["out"], ws_dec)

    def dense_decode(st):
        resa.dense_decode(cfg, st["kv"], st["q"], st["out_dense"], ws_den)

    def sparse_step():
        for st in layers:
            score_select(st)
            sparse_decode(st)

    def dense_step():
        for st in layers:
            dense_decode(st)

    def capture(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        torch.cuda.synchronize()
        return graph

    def time_graph(graph, steps, warmup, per_step=None):
        """Mean ms per replay (wall clock between synchronizations, and HIP
        events on the stream); with `per_step` a list, it receives each
        replay's event-timed duration."""
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        w0 = time.perf_counter()
        ev[0].record()
        for k in range(steps):
            graph.replay()
            ev[k + 1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w0) * 1e3 / steps
        if per_step is not None:
            per_step.extend(ev[k].elapsed_time(ev[k + 1]) for k in range(steps))
        return wall, ev[0].elapsed_time(ev[steps]) / steps

    # ---------------------------------------------------------------- sparse step
    g_sparse = capture(sparse_step)
    log("captured sparse step graph")
    step_ms = []
    wall_ms, ev_ms = time_graph(g_sparse, args.steps, args.warmup, per_step=step_ms)
    us_layer = wall_ms * 1e3 / nlayers
    pct = {f"p{q}": round(float(np.percentile(step_ms, q)) * 1e3 / nlayers, 3) for q in (10, 50, 90)}
    log(f"sparse: {wall_ms:.3f} ms/step (events {ev_ms:.3f}), {us_layer:.2f} us/layer-step")

    # Per-call breakdown: each call alone, replayed from a graph over the 28
    # layers and timed with HIP events on the replay stream; the sparse decode
    # figure is the roofline kernel's average launch duration.
    def per_call(fn):
        gr = capture(lambda: [fn(st) for st in layers])
        _, ev = time_graph(gr, max(5, args.steps // 5), 2)
        del gr
        return ev * 1e3 / nlayers  # us

    t_tail = per_call(tail_refresh)
    t_sel = per_call(score_select)
    t_dec = per_call(sparse_decode)
    # the same layer-step through the one-call entry point (at this row length
    # it runs the same kernels as the two calls)
    ws_step = resa.alloc_workspace(cfg, resa.OP_SPARSE_STEP, 1, mb, ms)
    t_step_call = per_call(lambda st: resa.sparse_step(cfg, st["kv"], st["q"], st["sel_idx"], st["sel_cnt"],
                                                       st["out"], ws_step, refresh_tail=True))
    log(f"breakdown us: tail-descriptor call {t_tail:.2f}  score+select (with tail refresh) {t_sel:.2f}  "
        f"sparse decode {t_dec:.2f}  resa_sparse_step {t_step_call:.2f}")

    # ---------------------------------------------------------------- dense
    g_dense = capture(dense_step)
    dwall_ms, dev_ms = time_graph(g_dense, max(5, args.steps // 5), 2)
    us_dense = dwall_ms * 1e3 / nlayers
    log(f"dense: {dwall_ms:.3f} ms/step, {us_dense:.2f} us/layer-step")
    del g_dense

    # ---------------------------------------------------------------- bytes
    ab = algorithmic_bytes(spec, L, n_sel, e)
    dense_bytes = H * L * 2 * d * e + ab["q"] + ab["out"]
    gbps = ab["total"] / (us_layer * 1e-6) / 1e9
    dec_bytes = ab["kv"] + ab["q"] + ab["out"]
    dec_gbps = dec_bytes / (t_dec * 1e-6) / 1e9
    khash = source_hash("decode.hip", "decode_core.h", "attn_frag.h", "resa_internal.h")
    traffic, trace = measured_traffic(khash)
    trace_us = trace.get("decode") if isinstance(trace, dict) else None

    # ---------------------------------------------------------------- check + CPU oracle
    cpu = None
    check = None
    if keep0 is not None:
        import oracle as O

        torch.cuda.synchronize()
        q0, k0, v0 = keep0
        scale = float(np.float32(1 / math.sqrt(d)))
        qs = [q0[0, i * g:(i + 1) * g].float().numpy().astype(np.float64) for i in range(H)]
        Ks = [k0[0][i].float().numpy().astype(np.float64) for i in range(H)]
        Vs = [v0[0][i].float().numpy().astype(np.float64) for i in range(H)]
        log("oracle: building the layer-0 block key cache (not timed)")
        desc = [O.descriptors(Ks[i], L) for i in range(H)]
        # sanity check of the timed GPU outputs of layer 0 against the oracle on the GPU's selection
        sel = layers[0]["sel_idx"].cpu()
        cnt = layers[0]["sel_cnt"].cpu()
        out0 = layers[0]["out"].cpu().numpy()
        errs = []
        for i in range(H):
            blocks = sel[0, i, : int(cnt[0, i])].tolist()
            ref = O.attend(qs[i], Ks[i], Vs[i], L, blocks, scale)
            errs.append(float(np.abs(out0[0, i * g:(i + 1) * g] - ref).max()))
        check = max(errs)
        log(f"layer-0 output vs oracle: max abs err {check:.2e}")
        del Ks, Vs, desc
        log(f"oracle: timing on the host ({len(os.sched_getaffinity(0))} threads)")
        cpu = cpu_oracle_legs(O, np, torch, spec, keep0, scale)
        log(f"oracle: {cpu['legs']}")

    # ---------------------------------------------------------------- rectification
    qc = torch.randn((1, RECT_CHUNK, H * g, d), device="cuda").to(torch.bfloat16)
    kn = torch.randn((1, RECT_CHUNK, H, d), device="cuda").to(torch.bfloat16)
    vn = torch.randn((1, RECT_CHUNK, H, d), device="cuda").to(torch.bfloat16)
    rout = torch.empty((1, RECT_CHUNK, H * g, d), device="cuda")
    ws_rect = resa.alloc_workspace(cfg, resa.OP_DENSE_RECTIFY, 1, mb, chunk=RECT_CHUNK)

    def rectify(st):
        resa.dense_rectify(cfg, st["kv"], qc, kn, vn, rout, ws_rect)

    t_rect = per_call(rectify)  # every replay rewrites the same window
    rect_flops = H * g * sum(4 * d * (L - RECT_CHUNK + t + 1) for t in range(RECT_CHUNK))
    log(f"rectify (window {RECT_CHUNK}): {t_rect:.1f} us/layer, {rect_flops / (t_rect * 1e-6) / 1e12:.1f} TFLOP/s")

    # rectification workload: 4 requests x 131072 tokens, window 64
    spec5 = WORKLOADS[C5_NAME]
    f5 = spec5.rectify_chunk
    inp5 = make_layer(spec5, seed=SEED, layer=0, device="cuda")
    pg5 = make_paged(inp5)
    kv5 = resa.PagedKV(pg5.k_pool, pg5.v_pool, pg5.desc_pool, pg5.block_table, pg5.seq_lens)
    resa.build_descriptors(cfg, kv5)
    lens5 = list(inp5.seq_lens)
    del inp5
    R5 = len(lens5)
    qc5 = torch.randn((R5, f5, H * g, d), device="cuda").to(torch.bfloat16)
    kn5 = torch.randn((R5, f5, H, d), device="cuda").to(torch.bfloat16)
    vn5 = torch.randn((R5, f5, H, d), device="cuda").to(torch.bfloat16)
    rout5 = torch.empty((R5, f5, H * g, d), device="cuda")
    ws_r5 = resa.alloc_workspace(cfg, resa.OP_DENSE_RECTIFY, R5, kv5.max_blocks, chunk=f5)
    gr5 = capture(lambda: resa.dense_rectify(cfg, kv5, qc5, kn5, vn5, rout5, ws_r5))
    # Every replay rewrites the same windows.  One call is under 1 ms, and the
    # first few dozen milliseconds of MFMA work after a pause run slower while
    # the chip ramps up (on a fresh box: 1020, 960, 885, 866 us for the first
    # calls, then 816-841 us on every cache), so the warm-up spans about 40 ms.
    _, ev5 = time_graph(gr5, max(5, args.steps // 5), 48)
    del gr5
    t_rect5 = ev5 * 1e3
    flops5 = H * g * sum(4 * d * (L5 - f5 + t + 1) for L5 in lens5 for t in range(f5))
    kv_bytes5 = sum(H * L5 * 2 * d * e for L5 in lens5)
    log(f"rectify {C5_NAME}: {t_rect5:.1f} us/call, {flops5 / (t_rect5 * 1e-6) / 1e12:.1f} TFLOP/s")
    del kv5, pg5, qc5, kn5, vn5, rout5, ws_r5
    torch.cuda.empty_cache()

    # streaming reference in the same run: the runtime's device copy
    copy54_us, copy54_gbps = copy_reference(torch, 54 << 20, 200)
    copy1g_us, copy1g_gbps = copy_reference(torch, 1 << 30, 20)
    log(f"device copy: 54 MiB {copy54_us:.2f} us ({copy54_gbps:.0f} GB/s read+write), "
        f"1 GiB {copy1g_us:.1f} us ({copy1g_gbps:.0f} GB/s)")

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * 2**20 // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    line = {
        "metric": METRIC,
        "value": round(us_layer, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "requests": 1, "ctx": L, "layers": nlayers, "q_heads": H * g,
                   "kv_heads": H, "head_dim": d, "block": 16, "budget": "1/10", "selected_blocks": n_sel,
                   "step": "28 layers x (score/select with tail-descriptor refresh + sparse decode), HIP graph"},
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes_per_layer_step": ab["total"],
        "us_per_layer_step_percentiles": pct,
        "tokens_per_s": round(1e3 / wall_ms, 1),
        "dense_us_per_layer_step": round(us_dense, 3),
        "speedup_vs_dense": round(us_dense / us_layer, 3),
        "dense_hbm_gbps": round(dense_bytes / (us_dense * 1e-6) / 1e9, 1),
        "breakdown_us": {"score_select_with_tail_refresh": round(t_sel, 2), "sparse_decode": round(t_dec, 2),
                         "standalone_tail_descriptor_call": round(t_tail, 2),
                         "sparse_step_call": round(t_step_call, 2)},
        "rectify_us_per_layer": round(t_rect, 1),
        "rectify_window": RECT_CHUNK,
        "rectify_tflops": round(rect_flops / (t_rect * 1e-6) / 1e12, 2),
        "rectify_c5": {"workload": C5_NAME, "requests": R5, "ctx": lens5[0], "window": f5,
                       "us_per_call": round(t_rect5, 1),
                       "useful_tflops": round(flops5 / (t_rect5 * 1e-6) / 1e12, 1),
                       "frac_of_bf16_mfma_peak": round(flops5 / (t_rect5 * 1e-6) / 2.5e15, 4),
                       "cache_bytes": kv_bytes5,
                       "cache_stream_gbps": round(kv_bytes5 / (t_rect5 * 1e-6) / 1e9, 1)},
        "stream_reference": {"kind": "runtime device copy (torch copy_), HIP events, buffers cycled past the "
                                     "last-level cache; GB/s counts bytes read + written",
                             "copy_54MiB_us": round(copy54_us, 2), "copy_54MiB_gbps": round(copy54_gbps, 1),
                             "copy_1GiB_us": round(copy1g_us, 1), "copy_1GiB_gbps": round(copy1g_gbps, 1)},
        "roofline": {"bound": "hbm",
                     "kernel": "sparse decode call (resa_sparse_decode: decode_kernel + merge_kernel)",
                     "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "bytes_per_launch": dec_bytes, "avg_launch_us": round(t_dec, 3),
                     "timing": "event-timed call: HIP events around graph replays of the call over 28 layers",
                     "trace_kernel": "decode_kernel<bf16_t, 128, true, 8>",
                     "trace_avg_us": trace_us,
                     "trace_kernel_frac": (round(dec_bytes / (trace_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
                                           if trace_us else None),
                     "step_frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "frac_of_copy_54MiB": round(dec_gbps / copy54_gbps, 4),
                     "step_frac_of_copy_54MiB": round(gbps / copy54_gbps, 4),
                     "kernel_source_hash": khash},
        "cpu_baseline": cpu,
        "oracle_check_max_abs_err": check,
    }
    print(json.dumps(line), flush=True)
    return 0


SWEEP_CTX = (16384, 65536, 262144)
SWEEP_BUDGETS = ((1, 50), (1, 20), (1, 10), (1, 5))


def sweep(args):
    """Per layer-step time of the sparse path (resa_sparse_step with the tail
    refresh, and beside it the two calls resa_score_select +
    resa_sparse_decode) for contexts 16K / 64K / 256K, budgets
    2 / 5 / 10 / 20 % and both scoring modes at 10 %, next to the dense decode
    and the rectification of a 32-token window.  Every figure is a HIP-graph
    replay over enough layer caches that one replay touches more than 1 GiB
    (so nothing is served from the 256 MB last-level cache), divided by the
    layer count;
    the two calls of the step are also timed alone.  Printed as a markdown
    table."""
    import torch

    import block_sparse_attention_resa_amd as resa
    from synth import WORKLOADS, make_layer, make_paged

    base = WORKLOADS["qwen7b_ctx256k_l28"]
    H, g, d = base.num_kv_heads, base.group_size, base.head_dim
    rows = []

    def graph_of(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        torch.cuda.synchronize()
        return gr

    def replay_us(gr, n_items, steps=20):
        gr.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            gr.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / steps / n_items

    for L in SWEEP_CTX:
        nl = layers_for_fresh_reads(base, [L])
        spec = base.with_(seq_lens=(L,), layers=nl, name=f"ctx{L}")
        caches = []
        for l in range(nl):
            inp = make_layer(spec, seed=SEED, layer=l, device="cuda")
            pg = make_paged(inp)
            kv = resa.PagedKV(pg.k_pool, pg.v_pool, pg.desc_pool, pg.block_table, pg.seq_lens)
            caches.append({"kv": kv, "q": inp.q})
            del inp
        cfg0 = resa.Config(num_kv_heads=H, group_size=g, head_dim=d, dtype=resa.RESA_BF16)
        for c in caches:
            resa.build_descriptors(cfg0, c["kv"])
        mb = caches[0]["kv"].max_blocks
        torch.cuda.synchronize()
        log(f"sweep: ctx {L}, {nl} layer caches")

        den = [torch.empty((1, H * g, d), device="cuda") for _ in caches]
        ws_den = resa.alloc_workspace(cfg0, resa.OP_DENSE_DECODE, 1, mb)
        gd = graph_of(lambda: [resa.dense_decode(cfg0, c["kv"], c["q"], o, ws_den) for c, o in zip(caches, den)])
        us_dense = replay_us(gd, nl)
        del gd

        f = 32
        qc = torch.randn((1, f, H * g, d), device="cuda").to(torch.bfloat16)
        kn = torch.randn((1, f, H, d), device="cuda").to(torch.bfloat16)
        vn = torch.randn((1, f, H, d), device="cuda").to(torch.bfloat16)
        rout = torch.empty((1, f, H * g, d), device="cuda")
        ws_r = resa.alloc_workspace(cfg0, resa.OP_DENSE_RECTIFY, 1, mb, chunk=f)
        gr = graph_of(lambda: [resa.dense_rectify(cfg0, c["kv"], qc, kn, vn, rout, ws_r) for c in caches])
        us_rect = replay_us(gr, nl, steps=5)  # rewrites the same window each time
        del gr

        variants = [(num, den_, resa.RESA_SCORE_SUM_HEADS) for num, den_ in SWEEP_BUDGETS]
        variants.append((1, 10, resa.RESA_SCORE_MEAN_POOL))
        for num, den_, mode in variants:
            cfg = resa.Config(num_kv_heads=H, group_size=g, head_dim=d, dtype=resa.RESA_BF16, budget_num=num,
                              budget_den=den_, score_mode=mode)
            ms = resa.selection_count(cfg, mb)
            n_sel = resa.selection_count(cfg, (L + 15) // 16)
            st = [{"sel": torch.empty((1, H, ms), dtype=torch.int32, device="cuda"),
                   "cnt": torch.empty((1, H), dtype=torch.int32, device="cuda"),
                   "out": torch.empty((1, H * g, d), device="cuda"), **c} for c in caches]
            ws_s = resa.alloc_workspace(cfg, resa.OP_SCORE_SELECT, 1, mb, ms)
            ws_d = resa.alloc_workspace(cfg, resa.OP_SPARSE_DECODE, 1, mb, ms)
            ws_st = resa.alloc_workspace(cfg, resa.OP_SPARSE_STEP, 1, mb, ms)

            def sel(c):
                resa.score_select(cfg, c["kv"], c["q"], c["sel"], c["cnt"], ws_s, refresh_tail=True)

            def dec(c):
                resa.sparse_decode(cfg, c["kv"], c["q"], c["sel"], c["cnt"], c["out"], ws_d)

            gs = graph_of(lambda: [(sel(c), dec(c)) for c in st])
            us_two = replay_us(gs, nl)
            del gs
            gs = graph_of(lambda: [resa.sparse_step(cfg, c["kv"], c["q"], c["sel"], c["cnt"], c["out"], ws_st,
                                                    refresh_tail=True) for c in st])
            us_step = replay_us(gs, nl)
            del gs
            gsel = graph_of(lambda: [sel(c) for c in st])
            t_sel = replay_us(gsel, nl)
            gdec = graph_of(lambda: [dec(c) for c in st])
            t_dec = replay_us(gdec, nl)
            del gsel, gdec
            desc_b = H * ((L + 15) // 16) * 2 * d * 2
            kv_b = H * ((n_sel - 1) * 16 + (L - ((L + 15) // 16 - 1) * 16)) * 2 * d * 2
            rows.append({"ctx": L, "budget": f"{num}/{den_}", "mode": "sum" if mode == 0 else "mean-pool",
                         "n_sel": n_sel, "us_step": us_step, "us_two": us_two, "us_score_select": t_sel,
                         "us_decode": t_dec,
                         "us_dense": us_dense, "us_rectify_f32": us_rect,
                         "gbps": (desc_b + kv_b) / (us_step * 1e-6) / 1e9,
                         "speedup": us_dense / us_step,
                         "cycle_speedup": us_dense / (us_step + us_rect / f)})
            del st
        del caches, den
        torch.cuda.empty_cache()

    print("| ctx | budget | scoring | blocks | us/layer-step | two calls us | score+select us | sparse decode us "
          "| GB/s (alg.) | dense us | x dense | rectify f=32 us | x dense incl. rectify/32 |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['ctx']} | {r['budget']} | {r['mode']} | {r['n_sel']} | {r['us_step']:.1f} | {r['us_two']:.1f} | "
              f"{r['us_score_select']:.1f} | {r['us_decode']:.1f} | {r['gbps']:.0f} | {r['us_dense']:.1f} | "
              f"{r['speedup']:.2f} | {r['us_rectify_f32']:.0f} | {r['cycle_speedup']:.2f} |")
    return 0


CYCLE_F = 32  # rectification window and period (the analysis page's default f)


def cycle(args):
    """The decoding loop of Algorithm 1 at 256K, timed end to end: for each of
    the 28 layers, CYCLE_F sparse steps at sequence lengths L - f + 1 ... L
    (score/select with the tail-descriptor refresh + sparse decode; the rows
    of those positions are already in the cache), then the rectification of
    the last f positions (row write, descriptor refresh, causal chunk
    attention).  Steps run layer by layer within each step, the
    rectification pass after the f-th step, all captured once in a HIP graph.
    Prints one JSON line: microseconds per layer-step amortised over the
    cycle, next to the dense decode per layer-step on the same caches."""
    import torch

    import block_sparse_attention_resa_amd as resa
    from synth import WORKLOADS, make_layer, make_paged

    spec = WORKLOADS["qwen7b_ctx256k_l28"]
    L = spec.seq_lens[0]
    H, g, d = spec.num_kv_heads, spec.group_size, spec.head_dim
    f = CYCLE_F
    cfg = resa.Config(num_kv_heads=H, group_size=g, head_dim=d, dtype=resa.RESA_BF16)
    layers = []
    for l in range(spec.layers):
        inp = make_layer(spec, seed=SEED, layer=l, device="cuda")
        pg = make_paged(inp)
        kv = resa.PagedKV(pg.k_pool, pg.v_pool, pg.desc_pool, pg.block_table, pg.seq_lens)
        resa.build_descriptors(cfg, kv)
        # one view per step: the same pools and table, the step's sequence length
        steps = [resa.PagedKV(pg.k_pool, pg.v_pool, pg.desc_pool, pg.block_table,
                              torch.tensor([L - f + 1 + t], dtype=torch.int32, device="cuda")) for t in range(f)]
        layers.append({"kv": kv, "steps": steps, "q": inp.q})
        del inp
    torch.cuda.synchronize()
    log(f"cycle: {len(layers)} layer caches, f = {f}")
    mb = layers[0]["kv"].max_blocks
    ms = resa.selection_count(cfg, mb)
    sel_idx = torch.empty((1, H, ms), dtype=torch.int32, device="cuda")
    sel_cnt = torch.empty((1, H), dtype=torch.int32, device="cuda")
    out = torch.empty((1, H * g, d), device="cuda")
    ws_s = resa.alloc_workspace(cfg, resa.OP_SCORE_SELECT, 1, mb, ms)
    ws_d = resa.alloc_workspace(cfg, resa.OP_SPARSE_DECODE, 1, mb, ms)
    ws_n = resa.alloc_workspace(cfg, resa.OP_DENSE_DECODE, 1, mb)
    ws_r = resa.alloc_workspace(cfg, resa.OP_DENSE_RECTIFY, 1, mb, chunk=f)
    gen = torch.Generator(device="cuda").manual_seed(SEED)
    qc = torch.randn((1, f, H * g, d), device="cuda", generator=gen).to(torch.bfloat16)
    kn = torch.randn((1, f, H, d), device="cuda", generator=gen).to(torch.bfloat16)
    vn = torch.randn((1, f, H, d), device="cuda", generator=gen).to(torch.bfloat16)
    rout = torch.empty((1, f, H * g, d), device="cuda")

    def one_cycle():
        for t in range(f):
            for st in layers:
                kv_t = st["steps"][t]
                resa.score_select(cfg, kv_t, st["q"], sel_idx, sel_cnt, ws_s, refresh_tail=True)
                resa.sparse_decode(cfg, kv_t, st["q"], sel_idx, sel_cnt, out, ws_d)
        for st in layers:
            resa.dense_rectify(cfg, st["kv"], qc, kn, vn, rout, ws_r)

    def dense_step():
        for st in layers:
            resa.dense_decode(cfg, st["kv"], st["q"], out, ws_n)

    def graph_of(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        torch.cuda.synchronize()
        return gr

    def replay_ms(gr, n):
        gr.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            gr.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    gc = graph_of(one_cycle)
    ms_cycle = replay_ms(gc, 5)
    del gc
    gd = graph_of(dense_step)
    ms_dense = replay_ms(gd, 10)
    del gd
    nl = len(layers)
    us_cycle = ms_cycle * 1e3 / (f * nl)
    us_dense = ms_dense * 1e3 / nl
    line = {"metric": "decode-loop us/layer-step incl. rectification every 32 steps, 256K ctx",
            "value": round(us_cycle, 3), "unit": "us/layer-step", "n_gpus": 1, "higher_is_better": False,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "qwen7b_ctx256k_l28", "layers": nl, "f": f,
                       "cycle": f"{f} sparse steps at lengths L-{f - 1}..L (score/select with tail refresh + "
                                f"sparse decode) then rectification of the last {f} positions, per layer, HIP graph"},
            "ms_per_cycle": round(ms_cycle, 3), "dense_us_per_layer_step": round(us_dense, 3),
            "speedup_vs_dense": round(us_dense / us_cycle, 3)}
    print(json.dumps(line), flush=True)
    return 0


WORKLOAD_TABLE = ("qwen7b_ctx32k_b1", "qwen7b_ragged_b8", "qwen7b_ctx131k_b4_rectify", "qwen7b_ctx256k_l28")


def workloads(args):
    """The bf16 workloads of the measured configurations, each at its own
    batch and context: per layer-step time of the sparse step
    (resa_sparse_step with the tail refresh, all requests of one layer; and
    beside it the two calls resa_score_select + resa_sparse_decode), decode
    tokens/s over 28 layers (attention only), algorithmic GB/s and its
    fraction of 8 TB/s, the dense decode and the speedup, and the
    rectification of the workload's window (the rectify workload's f, else
    32) with its useful TFLOP/s and fraction of the 2.5 PFLOP/s bf16 MFMA
    peak.  HIP-graph replays over enough layer caches that one replay
    touches more than 1 GiB (no reuse from the last-level cache), divided by
    the layer count.  Printed as a markdown table."""
    import torch

    import block_sparse_attention_resa_amd as resa
    from synth import WORKLOADS, make_layer, make_paged

    def graph_of(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        torch.cuda.synchronize()
        return gr

    def replay_us(gr, n_items, steps):
        gr.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            gr.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / steps / n_items

    rows = []
    for name in WORKLOAD_TABLE:
        spec = WORKLOADS[name]
        H, g, d, e = spec.num_kv_heads, spec.group_size, spec.head_dim, 2
        cfg = resa.Config(num_kv_heads=H, group_size=g, head_dim=d, dtype=resa.RESA_BF16)
        lens = None
        caches = []
        nl = 2
        l = 0
        while l < nl:
            inp = make_layer(spec, seed=SEED, layer=l, device="cuda")
            lens = list(inp.seq_lens)
            if l == 0:
                nl = layers_for_fresh_reads(spec, lens, e)
            pg = make_paged(inp)
            kv = resa.PagedKV(pg.k_pool, pg.v_pool, pg.desc_pool, pg.block_table, pg.seq_lens)
            resa.build_descriptors(cfg, kv)
            caches.append({"kv": kv, "q": inp.q})
            del inp
            l += 1
        R = len(lens)
        mb = caches[0]["kv"].max_blocks
        ms = resa.selection_count(cfg, mb)
        torch.cuda.synchronize()
        log(f"workloads: {name}, {R} requests, {nl} layer caches")
        st = [{"sel": torch.empty((R, H, ms), dtype=torch.int32, device="cuda"),
               "cnt": torch.empty((R, H), dtype=torch.int32, device="cuda"),
               "out": torch.empty((R, H * g, d), device="cuda"), **c} for c in caches]
        ws_s = resa.alloc_workspace(cfg, resa.OP_SCORE_SELECT, R, mb, ms)
        ws_d = resa.alloc_workspace(cfg, resa.OP_SPARSE_DECODE, R, mb, ms)
        ws_n = resa.alloc_workspace(cfg, resa.OP_DENSE_DECODE, R, mb)
        ws_st = resa.alloc_workspace(cfg, resa.OP_SPARSE_STEP, R, mb, ms)

        def two_calls(c):
            resa.score_select(cfg, c["kv"], c["q"], c["sel"], c["cnt"], ws_s, refresh_tail=True)
            resa.sparse_decode(cfg, c["kv"], c["q"], c["sel"], c["cnt"], c["out"], ws_d)

        def step(c):
            resa.sparse_step(cfg, c["kv"], c["q"], c["sel"], c["cnt"], c["out"], ws_st, refresh_tail=True)

        gs = graph_of(lambda: [two_calls(c) for c in st])
        us_two = replay_us(gs, nl, 20)
        del gs
        gs = graph_of(lambda: [step(c) for c in st])
        us_step = replay_us(gs, nl, 20)
        del gs
        gd = graph_of(lambda: [resa.dense_decode(cfg, c["kv"], c["q"], c["out"], ws_n) for c in st])
        us_dense = replay_us(gd, nl, 10)
        del gd

        f = getattr(spec, "rectify_chunk", 0) or 32
        qc = torch.randn((R, f, H * g, d), device="cuda").to(torch.bfloat16)
        kn = torch.randn((R, f, H, d), device="cuda").to(torch.bfloat16)
        vn = torch.randn((R, f, H, d), device="cuda").to(torch.bfloat16)
        rout = torch.empty((R, f, H * g, d), device="cuda")
        ws_r = resa.alloc_workspace(cfg, resa.OP_DENSE_RECTIFY, R, mb, chunk=f)
        gr = graph_of(lambda: [resa.dense_rectify(cfg, c["kv"], qc, kn, vn, rout, ws_r) for c in caches])
        us_rect = replay_us(gr, nl, 5)  # rewrites the same windows each time
        del gr

        alg = 0
        nsel = []
        for L in lens:
            n = resa.selection_count(cfg, (L + 15) // 16)
            nsel.append(n)
            alg += algorithmic_bytes(spec, L, n, e)["total"]
        flops = sum(H * g * 4 * d * (L - f + t + 1) for L in lens for t in range(f))
        gbps = alg / (us_step * 1e-6) / 1e9
        rows.append({"name": name, "R": R, "ctx": f"{min(lens)}" if min(lens) == max(lens) else f"{min(lens)}-{max(lens)}",
                     "nsel": f"{min(nsel)}" if min(nsel) == max(nsel) else f"{min(nsel)}-{max(nsel)}",
                     "us": us_step, "two": us_two, "tok": R / (28 * us_step * 1e-6), "gbps": gbps, "frac": gbps / PEAK_HBM_GBPS,
                     "dense": us_dense, "x": us_dense / us_step, "f": f, "rect": us_rect,
                     "tflops": flops / (us_rect * 1e-6) / 1e12})
        del st, caches, qc, kn, vn, rout
        torch.cuda.empty_cache()

    print("| workload | requests | context | blocks/head | us/layer-step | two calls us | tokens/s (28 layers) "
          "| GB/s (alg.) | of 8 TB/s | dense us | x dense | rectify f | rectify us | rectify TFLOP/s "
          "| of 2.5 PFLOP/s |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['name']} | {r['R']} | {r['ctx']} | {r['nsel']} | {r['us']:.1f} | {r['two']:.1f} | {r['tok']:.0f} | "
              f"{r['gbps']:.0f} | {r['frac'] * 100:.1f} % | {r['dense']:.1f} | {r['x']:.2f} | {r['f']} | "
              f"{r['rect']:.0f} | {r['tflops']:.0f} | {r['tflops'] / 2500 * 100:.1f} % |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
