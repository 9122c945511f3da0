#!/usr/bin/env python3
"""Benchmark of the DSA forward hot path on one MI355X.

One step = one fused forward (lightning-indexer scores -> top-k -> sparse
attention) over one batch of synthetic inputs already resident in HBM.  The
headline workload is MLA-style prefill at L = 32768, k = 2048 (64 indexer heads
x 128 in FP8 e4m3; 128 query heads over 576-wide bf16 latent rows, value width
512, softmax scale 1/sqrt(192)).  After it, the other four workloads (tiny
fp32 L = 256, L = 4096 MQA, decode 64 x 65536, L = 131072 in query tiles of
4096) are timed the same way and reported under "workloads", each stage
against the roofline that bounds it; the CPU oracle is timed on a bounded
sample of every workload.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA prefill tokens/s at L=32K,k=2048 (1 GPU); indexer % FP8 MFMA peak"
PEAK_FP8 = 5.0e15        # dense FP8 MFMA, MI355X
PEAK_BF16 = 2.5e15       # dense BF16 MFMA, MI355X
PEAK_FP32 = 157.3e12     # fp32 vector ALU, MI355X
PEAK_HBM = 8.0e12        # HBM3E bytes/s
HEADLINE = "mla_prefill_L32768"
OTHER_WORKLOADS = ("tiny_fp32_L256", "prefill_L4096", "decode_B64_ctx65536", "prefill_L131072")
# oracle sample per workload: query rows (prefill, evenly spaced over the
# sequence) or sequences (decode); chosen for a few seconds of CPU work each
ORACLE_SAMPLE = {"tiny_fp32_L256": 256, "prefill_L4096": 128, HEADLINE: 384, "decode_B64_ctx65536": 12,
                 "prefill_L131072": 48}

# HBM traffic of one attention launch at the headline workload, from rocprofv3
# FETCH_SIZE / WRITE_SIZE runs scaled by a 1 GiB plain copy measured in the same
# runs (fetch factor 2.0, write factor 1.0).  Valid only for the attention
# source it was measured on; any other source reports null.
ATTN_TRAFFIC = {"source_sha256_16": "e34f4f0fad0bac23", "fetch_bytes": 33821857868.4,
                "write_bytes": 4312926208.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg):
    """Algorithmic work of one forward (causal, no credit for masked work)
    and the bytes each stage must move at least."""
    t_pos = range(cfg.q_pos0, cfg.q_pos0 + cfg.Lq)
    n_all = cfg.B * sum(tp + 1 for tp in t_pos)
    n_sel = cfg.B * sum(min(cfg.k, tp + 1) for tp in t_pos)
    n_topk_read = cfg.B * sum(tp + 1 for tp in t_pos if tp + 1 > cfg.k)
    idx_bytes = 1 if cfg.idx_dtype == "fp8" else 4
    io_bytes = 2 if cfg.io_dtype == "bf16" else 4
    rows = cfg.B * cfg.Lq
    return {
        "rows": rows,
        "indexer_flop": 2.0 * cfg.n_idx_heads * cfg.idx_dim * n_all,
        # query codes, weights and scales once; every key (and its scale) once
        "indexer_bytes": float(rows * cfg.n_idx_heads * (cfg.idx_dim * idx_bytes + 8)
                               + cfg.B * cfg.Lk * (cfg.idx_dim * idx_bytes + 4)),
        "topk_bytes": 4.0 * n_topk_read + 4.0 * rows * cfg.k,
        "attn_flop": 2.0 * cfg.n_heads * (cfg.d_qk + cfg.d_v) * n_sel,
        "attn_gather_bytes": float(io_bytes * cfg.d_qk * n_sel),
        # q and out once, the index lists, the latent rows once
        "attn_unique_bytes": float(rows * cfg.n_heads * (cfg.d_qk + cfg.d_v) * io_bytes + 4 * rows * cfg.k
                                   + cfg.B * cfg.Lk * cfg.d_qk * io_bytes),
    }


def stage_bounds(cfg, work):
    """The roofline each stage is measured against, with its algorithmic
    work: FP8 / BF16 MFMA for the prefill indexer and attention, HBM for the
    top-k and for the decode indexer and gather, fp32 ALU for the fp32 path."""
    fp32 = cfg.idx_dtype == "f32"
    decode = cfg.Lq == 1
    if fp32:
        idx = ("alu", work["indexer_flop"], PEAK_FP32, "TFLOP/s")
        att = ("alu", work["attn_flop"], PEAK_FP32, "TFLOP/s")
    elif decode:
        idx = ("hbm", work["indexer_bytes"], PEAK_HBM, "GB/s")
        att = ("hbm", work["attn_gather_bytes"] + work["attn_unique_bytes"] - cfg.B * cfg.Lk * cfg.d_qk * 2,
               PEAK_HBM, "GB/s")
    else:
        idx = ("mfma", work["indexer_flop"], PEAK_FP8, "TFLOP/s")
        att = ("mfma", work["attn_flop"], PEAK_BF16, "TFLOP/s")
    return {"indexer": idx, "topk": ("hbm", work["topk_bytes"], PEAK_HBM, "GB/s"), "attention": att}


def stage_roofline(cfg, work, stages_ms):
    out = {}
    floor_s = 0.0
    for name, (bound, amount, peak, unit) in stage_bounds(cfg, work).items():
        floor = amount / peak
        floor_s += floor
        t = stages_ms.get(name)
        if t is None:
            continue
        rate = amount / (t * 1e-3)
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        out[name] = {"bound": bound, "achieved": rate / scale, "peak": peak / scale, "unit": unit,
                     "frac": rate / peak, "floor_ms": floor * 1e3, "ms": t}
    return out, floor_s


def attn_traffic_bytes():
    import hashlib
    src = os.path.join(ROOT, "sparse_attention_04_amd", "csrc", "attn_mla.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    if sha != ATTN_TRAFFIC["source_sha256_16"]:
        return None
    return ATTN_TRAFFIC["fetch_bytes"] + ATTN_TRAFFIC["write_bytes"]


def time_steps(fn, steps, stream):
    """Per-call times (ms) of `steps` back-to-back calls, from events recorded
    on `stream` between the calls; the region is bracketed by device
    synchronisation."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def median_ms(fn, steps, stream):
    return statistics.median(time_steps(fn, steps, stream))


def input_side(cfg, dev, stream, steps):
    """The input-side kernels at this workload's sizes, each timed alone (not
    part of the forward step): per-token FP8 quantisation of fp32 q_I and k_I,
    and assembly of the attention queries and latent rows from their
    compressed and rotary parts.  All four are HBM-bound; bytes are the
    algorithmic ones (every input read once, every output written once)."""
    import torch
    import sparse_attention_04_amd as dsa
    g = torch.Generator(device=dev).manual_seed(5)
    B, L, HI, DI, H = cfg.B, cfg.Lq, cfg.n_idx_heads, cfg.idx_dim, cfg.n_heads
    d_rope = cfg.d_qk - cfg.d_v
    res = {}
    qi = torch.randn(B, L, HI, DI, device=dev, generator=g)
    ki = torch.randn(B, cfg.Lk, DI, device=dev, generator=g)
    qc, qs = torch.empty(qi.shape, dtype=torch.uint8, device=dev), torch.empty(B, L, HI, device=dev)
    kc, ks = torch.empty(ki.shape, dtype=torch.uint8, device=dev), torch.empty(B, cfg.Lk, device=dev)
    jobs = [("quantize_q_idx", lambda: dsa.dsa_quantize_e4m3(qi, 2, HI, codes=qc, scales=qs, stream=stream),
             qi.numel() * 5 + qs.numel() * 4),
            ("quantize_k_idx", lambda: dsa.dsa_quantize_e4m3(ki, 1, 1, codes=kc, scales=ks, stream=stream),
             ki.numel() * 5 + ks.numel() * 4)]
    if d_rope >= 8 and cfg.io_dtype == "bf16":
        qn = torch.randn(B, L, H, cfg.d_v, device=dev, generator=g).to(torch.bfloat16)
        qr = torch.randn(B, L, H, d_rope, device=dev, generator=g).to(torch.bfloat16)
        cn = torch.randn(B, cfg.Lk, 1, cfg.d_v, device=dev, generator=g).to(torch.bfloat16)
        cr = torch.randn(B, cfg.Lk, 1, d_rope, device=dev, generator=g).to(torch.bfloat16)
        qo = torch.empty(B, L, H, cfg.d_qk, dtype=torch.bfloat16, device=dev)
        co = torch.empty(B, cfg.Lk, 1, cfg.d_qk, dtype=torch.bfloat16, device=dev)
        jobs += [("rope_assemble_q", lambda: dsa.dsa_rope_assemble(qn, qr, pos0=cfg.q_pos0, out=qo, stream=stream),
                  4 * qo.numel()),
                 ("rope_assemble_kv", lambda: dsa.dsa_rope_assemble(cn, cr, out=co, stream=stream), 4 * co.numel())]
    for name, f, nbytes in jobs:
        f()
        t = median_ms(f, steps, stream)
        res[name] = {"ms": t, "bytes": nbytes, "achieved_gbs": nbytes / (t * 1e-3) / 1e9,
                     "frac_hbm_peak": nbytes / (t * 1e-3) / PEAK_HBM}
        log(f"[bench] input side {name}: {t:.3f} ms ({res[name]['achieved_gbs']:.0f} GB/s)")
    return res


def measured_mfma_peaks(dev, stream):
    """MFMA issue rate and shader clock from the measurement probe
    (measure/libdsa_probe.so): back-to-back independent MFMAs with operands in
    registers, FP8 16x16x128 at two waves per SIMD (the indexer's occupancy)
    and BF16 32x32x16 at one wave per SIMD (the attention's), on
    near-constant and on pseudo-random operands (the clock drops further when
    the operand bits toggle), and at eight waves per SIMD."""
    import torch
    import measure
    sink = torch.empty(256 * 8 * 4 * 4, dtype=torch.float32, device=dev)
    clocks = torch.zeros(256 * 8 * 2 * 4, dtype=torch.int64, device=dev)
    res = {}
    for name, kind, wps, rnd, iters in (("fp8_2_waves_per_simd", 0, 2, False, 20000),
                                        ("fp8_2_waves_per_simd_random", 0, 2, True, 20000),
                                        ("fp8_8_waves_per_simd", 0, 8, False, 5000),
                                        ("bf16_1_wave_per_simd", 1, 1, False, 50000),
                                        ("bf16_1_wave_per_simd_random", 1, 1, True, 50000),
                                        ("bf16_8_waves_per_simd", 1, 8, False, 6000)):
        f = lambda: measure.probe_mfma(kind, wps, iters, rnd, sink=sink, clocks=clocks, stream=stream)
        flop = f()
        t = median_ms(f, 3, stream)
        res[name] = {"tflops": flop / (t * 1e-3) / 1e12, "clock_ghz": measure.clock_ghz(clocks)}
        log(f"[bench] MFMA probe {name}: {res[name]['tflops']:.0f} TFLOP/s at {res[name]['clock_ghz']:.2f} GHz")
    return res


def training_side(cfg, dev, stream, steps):
    """The two training-time steps next to the forward, each timed alone on
    inputs of their own (not part of the forward step):
      - the indexer distillation loss at L = 8192 (dense attention
        probabilities of all heads against the FP8 indexer's scores; two
        Q.K sweeps of 2*H*d_qk FLOP per (query, key) pair, causal);
      - the sparse-attention backward at L = 4096 over the forward's own
        selected sets (Q.K, dO.V, dq, and the two dkv products:
        2*H*(3*d_qk + 2*d_v) FLOP per selected entry)."""
    import torch
    import sparse_attention_04_amd as dsa
    from dsa_inputs import make_inputs
    res = {}
    H, dqk, dv = cfg.n_heads, cfg.d_qk, cfg.d_v
    if cfg.io_dtype != "bf16" or cfg.B != 1:
        return res
    # distillation loss
    L = 8192
    kc = cfg.with_(name="kl_L8192", Lq=L, Lk=L, q_pos0=0, q_tile_rows=0)
    inp = make_inputs(kc, seed=1, device=dev)
    sc = dsa.dsa_indexer_scores(inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["w"],
                                stream=stream)
    kl = torch.empty((1, L), dtype=torch.float32, device=dev)
    f = lambda: dsa.dsa_indexer_kl(inp["q"], inp["kv"], sc, kc.softmax_scale, kl=kl, stream=stream)
    f()
    t = median_ms(f, steps, stream)
    flop = 2.0 * 2 * H * dqk * (L * (L + 1) / 2)
    res["indexer_kl"] = {"workload": f"L={L}, {H} heads x {dqk}", "ms": t, "bound": "mfma",
                         "achieved_tflops": flop / (t * 1e-3) / 1e12, "peak_tflops": PEAK_BF16 / 1e12,
                         "frac": flop / (t * 1e-3) / PEAK_BF16}
    log(f"[bench] training side indexer_kl: {t:.3f} ms ({res['indexer_kl']['frac'] * 100:.1f}% of bf16 peak)")
    del inp, sc, kl
    # sparse-attention backward
    L = 4096
    bc = cfg.with_(name="bwd_L4096", Lq=L, Lk=L, q_pos0=0, q_tile_rows=0)
    inp = make_inputs(bc, seed=2, device=dev)
    fwd = dsa.Forward(1, L, L, bc.k, H, dv, inp["q"].dtype, dev, d_qk=dqk)
    fwd(inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["w"], inp["q"], inp["kv"],
        bc.softmax_scale, stream=stream)
    g = torch.Generator(device=dev).manual_seed(3)
    dout = torch.randn(fwd.out.shape, device=dev, generator=g).to(torch.bfloat16)
    dq = torch.empty((1, L, H, dqk), dtype=torch.float32, device=dev)
    dkv = torch.empty((1, L, dqk), dtype=torch.float32, device=dev)
    ws = torch.empty(max(int(dsa.lib.dsa_sparse_attn_bwd_workspace_size(1, L, L, H, bc.k)), 256), dtype=torch.uint8,
                     device=dev)
    f = lambda: dsa.dsa_sparse_attn_bwd(inp["q"], inp["kv"], fwd.idx, fwd.out, fwd.lse, dout, bc.softmax_scale,
                                        dq=dq, dkv=dkv, workspace=ws, stream=stream)
    f()
    t = median_ms(f, steps, stream)
    n_sel = sum(min(bc.k, tp + 1) for tp in range(L))
    flop = 2.0 * H * (3 * dqk + 2 * dv) * n_sel
    res["attn_backward"] = {"workload": f"L={L}, k={bc.k}, {H} heads, selected sets from the forward", "ms": t,
                            "bound": "dkv: key-major contribution slots (HBM)", "achieved_tflops": flop / (t * 1e-3) / 1e12,
                            "peak_tflops": PEAK_BF16 / 1e12, "frac": flop / (t * 1e-3) / PEAK_BF16,
                            "dkv_contribution_bytes": n_sel * dqk * 4}
    log(f"[bench] training side attn_backward: {t:.3f} ms ({res['attn_backward']['frac'] * 100:.1f}% of bf16 peak)")
    del inp, fwd, dout, dq, dkv, ws
    torch.cuda.empty_cache()
    return res


def forward_runner(cfg, inp, dev, stream, select=0):
    import sparse_attention_04_amd as dsa
    fwd = dsa.Forward(cfg.B, cfg.Lq, cfg.Lk, cfg.k, cfg.n_heads, cfg.d_v, inp["q"].dtype, dev, d_qk=cfg.d_qk,
                      q_tile_rows=cfg.q_tile_rows, select=select)
    run = lambda: fwd(inp["q_idx"], inp.get("q_scale"), inp["k_idx"], inp.get("k_scale"), inp["w"], inp["q"],
                      inp["kv"], cfg.softmax_scale, q_pos0=cfg.q_pos0, stream=stream)
    return fwd, run


def route_times(cfg, inp, dev, stream, steps):
    """The forward by each selection route that takes the workload (score
    tiles; candidate lists, which keep full score rows out of memory), median
    ms, and the route the default (AUTO) takes: the one whose workspace size
    it asks for."""
    import torch
    import sparse_attention_04_amd as dsa
    ws = lambda sel: dsa.dsa_forward_workspace_size(cfg.B, cfg.Lq, cfg.Lk, cfg.k, cfg.n_heads, cfg.d_qk, cfg.d_v,
                                                    inp["q"].dtype, cfg.q_tile_rows, sel)
    out = {}
    routes = {"score_tiles": dsa.SELECT_SCORE_TILES}
    if cfg.idx_dtype == "fp8" and ws(dsa.SELECT_CANDIDATES) > 0:
        routes["candidates"] = dsa.SELECT_CANDIDATES
    for name, sel in routes.items():
        fwd, run = forward_runner(cfg, inp, dev, stream, sel)
        run()
        torch.cuda.synchronize()
        out[name] = median_ms(run, steps, stream)
        del fwd, run
        torch.cuda.empty_cache()
    auto = "candidates" if ("candidates" in routes and ws(dsa.SELECT_AUTO) == ws(dsa.SELECT_CANDIDATES)) \
        else "score_tiles"
    return out, auto


def time_stages(cfg, inp, fwd, dev, stream, steps):
    """Each stage alone through its own entry point, on the forward's inputs
    (the attention on the forward's selected sets).  Workloads the forward runs
    in query tiles time the indexer and the top-k tile by tile (the standalone
    indexer also writes each tile's masked scores); the attention runs once."""
    import torch
    import sparse_attention_04_amd as dsa
    T = cfg.q_tile_rows if cfg.q_tile_rows > 0 else cfg.Lq
    tiles = [(t0, min(T, cfg.Lq - t0)) for t0 in range(0, cfg.Lq, T)]
    assert len(tiles) == 1 or cfg.B == 1
    scores = torch.empty((cfg.B, T, cfg.Lk), dtype=torch.float32, device=dev)
    idx = torch.empty((cfg.B, cfg.Lq, cfg.k), dtype=torch.int32, device=dev)
    out = torch.empty_like(fwd.out)
    lse = torch.empty_like(fwd.lse)
    qs = inp.get("q_scale")

    def f_idx():
        for t0, tc in tiles:
            dsa.dsa_indexer_scores(inp["q_idx"][:, t0:t0 + tc], None if qs is None else qs[:, t0:t0 + tc],
                                   inp["k_idx"], inp.get("k_scale"), inp["w"][:, t0:t0 + tc],
                                   q_pos0=cfg.q_pos0 + t0, scores=scores[:, :tc], stream=stream)

    def f_topk():
        for t0, tc in tiles:
            dsa.dsa_topk(scores[:, :tc], cfg.k, q_pos0=cfg.q_pos0 + t0, idx=idx[:, t0:t0 + tc], stream=stream)

    f_attn = lambda: dsa.dsa_sparse_attn(inp["q"], inp["kv"], fwd.idx, cfg.d_v, cfg.softmax_scale,
                                         q_pos0=cfg.q_pos0, out=out, lse=lse, stream=stream)
    res = {}
    for name, f in (("indexer", f_idx), ("topk", f_topk), ("attention", f_attn)):
        f()
        res[name] = median_ms(f, steps, stream)
        log(f"[bench] {cfg.name} stage {name}: {res[name]:.3f} ms")
    del scores, idx, out, lse
    return res


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(cfg, inp, n_sample):
    """The oracle, as it stands, on a bounded sample of the workload: query
    rows evenly spaced over the sequence (prefill) or whole sequences
    (decode), from the same input bytes (copied to the host).  Each stage is
    timed on the monotonic clock; tokens/s is the sample's rows over the
    sample's time."""
    import numpy as np
    import torch
    import oracle
    fp8 = cfg.idx_dtype == "fp8"
    dt = oracle.E4M3 if fp8 else oracle.F32
    io = oracle.BF16 if cfg.io_dtype == "bf16" else oracle.F32
    if cfg.Lq == 1:
        batches = np.unique(np.linspace(0, cfg.B - 1, min(n_sample, cfg.B)).astype(np.int64))
        plan = [(int(b), np.array([0])) for b in batches]
    else:
        rows = np.unique(np.linspace(0, cfg.Lq - 1, min(n_sample, cfg.Lq)).astype(np.int64))
        plan = [(0, rows)]
    st = {"indexer": 0.0, "topk": 0.0, "attention": 0.0}
    n_rows = 0
    for b, rows in plan:
        rt = torch.as_tensor(rows, device=inp["q"].device)
        host = lambda key: inp[key][b].index_select(0, rt).cpu()
        qi, w, q = host("q_idx"), host("w"), host("q")
        qs = host("q_scale") if fp8 else None
        ki, kv = inp["k_idx"][b].cpu(), inp["kv"][b].cpu()
        ks = inp["k_scale"][b].cpu() if fp8 else None
        t_pos = cfg.q_pos0 + rows
        t0 = time.perf_counter()
        sc = oracle.indexer(qi, qs, ki, ks, w, t_pos, dt)
        t1 = time.perf_counter()
        ix = oracle.topk(sc, t_pos, cfg.k)
        t2 = time.perf_counter()
        oracle.sparse_attn(q, kv, ix, cfg.d_v, cfg.softmax_scale, io)
        t3 = time.perf_counter()
        st["indexer"] += t1 - t0
        st["topk"] += t2 - t1
        st["attention"] += t3 - t2
        n_rows += len(rows)
    total = sum(st.values())
    model, cores = cpu_info()
    full = n_rows == cfg.B * cfg.Lq
    what = ("every row" if full else
            (f"{n_rows} of {cfg.B} sequences" if cfg.Lq == 1 else
             f"{n_rows} query rows evenly spaced over t=0..{cfg.Lq - 1}"))
    return {"value": n_rows / total, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{what} of the same inputs (indexer + top-k + attention per row, fp64), {total:.1f} s",
            "extrapolated": not full, "rows": n_rows, "stage_s": st, "affinity_cpus": cores, "cpu_model": model}


def bench_workload(cfg, dev, stream, steps, warmup, want_oracle):
    """One of the non-headline workloads: forward (median of `steps`), each
    stage alone against its bound, the oracle on a bounded sample."""
    import torch
    from dsa_inputs import make_inputs
    log(f"[bench] {cfg.name}: drawing inputs")
    inp = make_inputs(cfg, seed=0, device=dev)
    torch.cuda.synchronize()
    work = algorithmic(cfg)
    fwd, run = forward_runner(cfg, inp, dev, stream)
    for _ in range(warmup):
        run()
    ms = median_ms(run, steps, stream)
    tokens = cfg.B * cfg.Lq
    log(f"[bench] {cfg.name}: forward {ms:.3f} ms -> {tokens / (ms * 1e-3):.4g} tokens/s")
    routes, route = route_times(cfg, inp, dev, stream, steps)
    stages = time_stages(cfg, inp, fwd, dev, stream, steps)
    roof, floor_s = stage_roofline(cfg, work, stages)
    res = {"tokens_per_s": tokens / (ms * 1e-3), "ms_per_step": ms, "steps": steps, "tokens": tokens,
           "config": {"B": cfg.B, "Lq": cfg.Lq, "Lk": cfg.Lk, "q_pos0": cfg.q_pos0, "k": cfg.k,
                      "n_idx_heads": cfg.n_idx_heads, "idx_dim": cfg.idx_dim, "idx_dtype": cfg.idx_dtype,
                      "n_heads": cfg.n_heads, "d_qk": cfg.d_qk, "d_v": cfg.d_v, "io_dtype": cfg.io_dtype,
                      "q_tile_rows": cfg.q_tile_rows},
           "routes_ms": routes, "route": route,
           "stages_ms": stages, "stage_roofline": roof, "floor_ms": floor_s * 1e3,
           "e2e_frac_of_floor": floor_s / (ms * 1e-3)}
    if want_oracle:
        log(f"[bench] {cfg.name}: oracle on a sample")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, ORACLE_SAMPLE[cfg.name])
        log(f"[bench] {cfg.name}: oracle {res['cpu_baseline']['value']:.3g} tokens/s")
    del inp, fwd, run
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--cpu-rows", type=int, default=ORACLE_SAMPLE[HEADLINE],
                    help="oracle sample size in query rows of the headline workload (0 = no oracle at all)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (counter calibration)")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage timing loops")
    ap.add_argument("--no-training", action="store_true",
                    help="skip the training-side steps (distillation loss, backward), which also run the forward "
                         "kernels at their own sizes")
    ap.add_argument("--no-workloads", action="store_true", help="skip the other four workloads")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              f"the path shards by query rows, but this program measures a single GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    from dsa_inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    log(f"[bench] {cfg.name}: drawing inputs on {torch.cuda.get_device_name(dev)}")
    inp = make_inputs(cfg, seed=0, device=dev)
    torch.cuda.synchronize()
    work = algorithmic(cfg)
    if args.copy_mib > 0:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter readings
        # calibrate the HBM traffic counters of the kernels below
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    fwd, run = forward_runner(cfg, inp, dev, stream)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    step_ms = time_steps(run, args.steps, stream)
    ms = statistics.median(step_ms)
    tokens = cfg.B * cfg.Lq
    log(f"[bench] forward median {ms:.3f} ms/step (mean {statistics.mean(step_ms):.3f}) -> "
        f"{tokens / (ms * 1e-3):.4g} tokens/s")

    res = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_mean": statistics.mean(step_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "L": cfg.Lk, "k": cfg.k,
                   "n_idx_heads": cfg.n_idx_heads, "idx_dim": cfg.idx_dim, "n_heads": cfg.n_heads,
                   "d_qk": cfg.d_qk, "d_v": cfg.d_v, "q_tile_rows": cfg.q_tile_rows},
    }
    if not args.no_stages:
        res["routes_ms"], res["route"] = route_times(cfg, inp, dev, stream, max(1, args.steps))
        log(f"[bench] routes {res['routes_ms']} (default: {res['route']})")
        stages = time_stages(cfg, inp, fwd, dev, stream, max(1, args.steps))
        torch.cuda.empty_cache()
        roof, floor_s = stage_roofline(cfg, work, stages)
        att = roof["attention"]
        res["roofline"] = {"bound": att["bound"], "kernel": "sparse_attn_mla_kernel", "achieved": att["achieved"],
                           "peak": att["peak"], "unit": att["unit"], "frac": att["frac"],
                           "traffic": attn_traffic_bytes() if cfg.name == HEADLINE else None}
        res["indexer_frac_fp8_peak"] = roof["indexer"]["frac"]
        res["stages_ms"] = stages
        res["stage_roofline"] = roof
        res["stage_roofline"]["attention"]["gather_tbs"] = work["attn_gather_bytes"] / (stages["attention"] * 1e-3) / 1e12
        res["floor_ms"] = floor_s * 1e3
        res["e2e_frac_of_floor"] = floor_s / (ms * 1e-3)
        peaks = measured_mfma_peaks(dev, stream)
        res["measured_mfma"] = peaks
        res["indexer_frac_measured_peak"] = (work["indexer_flop"] / (stages["indexer"] * 1e-3) / 1e12 /
                                             peaks["fp8_2_waves_per_simd_random"]["tflops"])
        res["stage_roofline"]["attention"]["frac_measured_peak"] = (
            att["achieved"] / peaks["bf16_1_wave_per_simd_random"]["tflops"])
        res["input_side"] = input_side(cfg, dev, stream, max(1, args.steps))
        torch.cuda.empty_cache()
        if cfg.name == HEADLINE and not args.no_training:
            res["training_side"] = training_side(cfg, dev, stream, max(1, args.steps))
    if args.cpu_rows > 0:
        log(f"[bench] oracle on {args.cpu_rows} sampled rows")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_rows)
    del inp, fwd, run
    torch.cuda.empty_cache()
    if not args.no_workloads and cfg.name == HEADLINE:
        res["workloads"] = {}
        for name in OTHER_WORKLOADS:
            wcfg = CONFIGS[name]
            steps = max(3, args.steps // 2) if name == "prefill_L131072" else max(1, args.steps)
            res["workloads"][name] = bench_workload(wcfg, dev, stream, steps, max(1, args.warmup // 2 + 1),
                                                    args.cpu_rows > 0)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
