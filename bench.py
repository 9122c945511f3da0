#!/usr/bin/env python3
"""Benchmark of the DSA forward hot path on one MI355X.

One step = one fused forward (lightning-indexer scores -> top-k -> sparse
attention) over one batch of synthetic inputs already resident in HBM.  The
default workload is MLA-style prefill at L = 32768, k = 2048 (64 indexer heads
x 128 in FP8 e4m3; 128 query heads over 576-wide bf16 latent rows, value width
512, softmax scale 1/sqrt(192)).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA prefill tokens/s at L=32K,k=2048 (1 GPU); indexer % FP8 MFMA peak"
PEAK_FP8 = 5.0e15        # dense FP8 MFMA, MI355X
PEAK_BF16 = 2.5e15       # dense BF16 MFMA, MI355X
PEAK_HBM = 8.0e12        # HBM3E bytes/s

# HBM traffic of one attention launch at the bench workload, from rocprofv3
# FETCH_SIZE / WRITE_SIZE runs scaled by a 1 GiB plain copy measured in the same
# runs (fetch factor 2.0, write factor 1.0).  Valid only for the attention
# source it was measured on; any other source reports null.
ATTN_TRAFFIC = {"source_sha256_16": "d574ec853ebdf46f", "fetch_bytes": 55110908519.0,
                "write_bytes": 5431578400.0}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg):
    """Algorithmic work of one forward (causal, no credit for masked work)."""
    t_pos = [cfg.q_pos0 + t for t in range(cfg.Lq)]
    n_all = cfg.B * sum(tp + 1 for tp in t_pos)
    n_sel = cfg.B * sum(min(cfg.k, tp + 1) for tp in t_pos)
    n_topk_read = cfg.B * sum(tp + 1 for tp in t_pos if tp + 1 > cfg.k)
    return {
        "indexer_flop": 2.0 * cfg.n_idx_heads * cfg.idx_dim * n_all,
        "attn_flop": 2.0 * cfg.n_heads * (cfg.d_qk + cfg.d_v) * n_sel,
        "topk_bytes": 4.0 * n_topk_read + 4.0 * cfg.B * cfg.Lq * cfg.k,
        "attn_gather_bytes": 2.0 * cfg.d_qk * n_sel,
    }


def attn_traffic_bytes():
    import hashlib
    src = os.path.join(ROOT, "sparse_attention_04_amd", "csrc", "sparse_attn.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    if sha != ATTN_TRAFFIC["source_sha256_16"]:
        return None
    return ATTN_TRAFFIC["fetch_bytes"] + ATTN_TRAFFIC["write_bytes"]


def time_loop(fn, steps, stream):
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


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
        t = time_loop(f, steps, stream)
        res[name] = {"ms": t, "bytes": nbytes, "achieved_gbs": nbytes / (t * 1e-3) / 1e9,
                     "frac_hbm_peak": nbytes / (t * 1e-3) / PEAK_HBM}
        log(f"[bench] input side {name}: {t:.3f} ms ({res[name]['achieved_gbs']:.0f} GB/s)")
    return res


def measured_mfma_peaks(dev, stream):
    """MFMA issue-rate probe (the library's dsa_probe_mfma): back-to-back
    independent MFMAs with operands in registers.  FP8 16x16x128 at two waves
    per SIMD (the indexer's occupancy) and BF16 32x32x16 at one wave per SIMD
    (the attention's), each also at eight waves per SIMD."""
    import torch
    import sparse_attention_04_amd as dsa
    sink = torch.empty(256 * 8 * 4 * 4, dtype=torch.float32, device=dev)
    res = {}
    for name, kind, wps, iters in (("fp8_2_waves_per_simd", 0, 2, 20000), ("fp8_8_waves_per_simd", 0, 8, 5000),
                                   ("bf16_1_wave_per_simd", 1, 1, 50000), ("bf16_8_waves_per_simd", 1, 8, 6000)):
        flop = dsa.dsa_probe_mfma(kind, wps, iters, sink=sink, stream=stream)
        t = time_loop(lambda: dsa.dsa_probe_mfma(kind, wps, iters, sink=sink, stream=stream), 3, stream)
        res[name] = flop / (t * 1e-3) / 1e12
        log(f"[bench] MFMA probe {name}: {res[name]:.0f} TFLOP/s")
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
    t = time_loop(f, steps, stream)
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
    ws = torch.empty(max(int(dsa.lib.dsa_sparse_attn_bwd_workspace_size(1, L, H, bc.k)), 256), dtype=torch.uint8,
                     device=dev)
    f = lambda: dsa.dsa_sparse_attn_bwd(inp["q"], inp["kv"], fwd.idx, fwd.out, fwd.lse, dout, bc.softmax_scale,
                                        dq=dq, dkv=dkv, workspace=ws, stream=stream)
    f()
    t = time_loop(f, steps, stream)
    n_sel = sum(min(bc.k, tp + 1) for tp in range(L))
    flop = 2.0 * H * (3 * dqk + 2 * dv) * n_sel
    res["attn_backward"] = {"workload": f"L={L}, k={bc.k}, {H} heads, selected sets from the forward", "ms": t,
                            "bound": "atomics (dkv scatter)", "achieved_tflops": flop / (t * 1e-3) / 1e12,
                            "peak_tflops": PEAK_BF16 / 1e12, "frac": flop / (t * 1e-3) / PEAK_BF16,
                            "dkv_atomic_adds": n_sel * dqk}
    log(f"[bench] training side attn_backward: {t:.3f} ms ({res['attn_backward']['frac'] * 100:.1f}% of bf16 peak)")
    del inp, fwd, dout, dq, dkv, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg, inp, n_rows):
    """The oracle, as it stands, on a uniform sample of query rows."""
    import numpy as np
    import torch
    import oracle
    rows = np.unique(np.linspace(0, cfg.Lq - 1, n_rows).astype(np.int64))
    rt = torch.as_tensor(rows, device=inp["q"].device)
    b = 0
    qi = inp["q_idx"][b].index_select(0, rt).cpu()
    qs = inp["q_scale"][b].index_select(0, rt).cpu()
    w = inp["w"][b].index_select(0, rt).cpu()
    q = inp["q"][b].index_select(0, rt).cpu()
    ki, ks, kv = inp["k_idx"][b].cpu(), inp["k_scale"][b].cpu(), inp["kv"][b].cpu()
    t_pos = cfg.q_pos0 + rows
    t0 = time.perf_counter()
    sc = oracle.indexer(qi, qs, ki, ks, w, t_pos, oracle.E4M3)
    ix = oracle.topk(sc, t_pos, cfg.k)
    oracle.sparse_attn(q, kv, ix, cfg.d_v, cfg.softmax_scale, oracle.BF16)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{len(rows)} query rows evenly spaced over t=0..{cfg.Lq - 1} of the same inputs "
                      f"(indexer + top-k + attention per row, fp64), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mla_prefill_L32768")
    ap.add_argument("--cpu-rows", type=int, default=768, help="oracle sample size in query rows (0 = skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (counter calibration)")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage timing loops")
    ap.add_argument("--no-training", action="store_true",
                    help="skip the training-side steps (distillation loss, backward), which also run the forward "
                         "kernels at their own sizes")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              f"the path shards by query rows, but this program measures a single GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_04_amd as dsa
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

    fwd = dsa.Forward(cfg.B, cfg.Lq, cfg.Lk, cfg.k, cfg.n_heads, cfg.d_v, inp["q"].dtype, dev, d_qk=cfg.d_qk,
                      q_tile_rows=cfg.q_tile_rows)
    run = lambda: fwd(inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"], inp["w"], inp["q"],
                      inp["kv"], cfg.softmax_scale, q_pos0=cfg.q_pos0, stream=stream)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ms = time_loop(run, args.steps, stream)
    tokens = cfg.B * cfg.Lq
    log(f"[bench] forward {ms:.3f} ms/step -> {tokens / (ms * 1e-3):.4g} tokens/s")

    stages = {}
    if not args.no_stages:
        # each stage alone, on the same stream, same inputs; the attention uses
        # the forward's own selected sets
        scores = torch.empty((cfg.B, cfg.Lq, cfg.Lk), dtype=torch.float32, device=dev)
        idx = torch.empty((cfg.B, cfg.Lq, cfg.k), dtype=torch.int32, device=dev)
        out = torch.empty_like(fwd.out)
        lse = torch.empty_like(fwd.lse)
        f_idx = lambda: dsa.dsa_indexer_scores(inp["q_idx"], inp["q_scale"], inp["k_idx"], inp["k_scale"],
                                               inp["w"], q_pos0=cfg.q_pos0, scores=scores, stream=stream)
        f_topk = lambda: dsa.dsa_topk(scores, cfg.k, q_pos0=cfg.q_pos0, idx=idx, stream=stream)
        f_attn = lambda: dsa.dsa_sparse_attn(inp["q"], inp["kv"], fwd.idx, cfg.d_v, cfg.softmax_scale,
                                             q_pos0=cfg.q_pos0, out=out, lse=lse, stream=stream)
        for name, f in (("indexer", f_idx), ("topk", f_topk), ("attention", f_attn)):
            f()
            stages[name] = time_loop(f, max(1, args.steps), stream)
            log(f"[bench] stage {name}: {stages[name]:.3f} ms")
        del scores, idx, out, lse
        torch.cuda.empty_cache()

    res = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "L": cfg.Lk, "k": cfg.k,
                   "n_idx_heads": cfg.n_idx_heads, "idx_dim": cfg.idx_dim, "n_heads": cfg.n_heads,
                   "d_qk": cfg.d_qk, "d_v": cfg.d_v, "q_tile_rows": cfg.q_tile_rows},
    }
    if stages:
        t_att = stages["attention"] * 1e-3
        t_idx = stages["indexer"] * 1e-3
        t_tk = stages["topk"] * 1e-3
        att = work["attn_flop"] / t_att
        res["roofline"] = {"bound": "mfma", "kernel": "sparse_attn_bf16", "achieved": att / 1e12,
                           "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": att / PEAK_BF16,
                           "traffic": attn_traffic_bytes() if cfg.name == "mla_prefill_L32768" else None}
        res["indexer_frac_fp8_peak"] = work["indexer_flop"] / t_idx / PEAK_FP8
        res["stages_ms"] = stages
        res["stage_roofline"] = {
            "indexer": {"bound": "mfma", "achieved_tflops": work["indexer_flop"] / t_idx / 1e12,
                        "peak_tflops": PEAK_FP8 / 1e12, "frac": work["indexer_flop"] / t_idx / PEAK_FP8},
            "topk": {"bound": "hbm", "achieved_gbs": work["topk_bytes"] / t_tk / 1e9,
                     "peak_gbs": PEAK_HBM / 1e9, "frac": work["topk_bytes"] / t_tk / PEAK_HBM},
            "attention": {"bound": "mfma", "achieved_tflops": att / 1e12, "peak_tflops": PEAK_BF16 / 1e12,
                          "frac": att / PEAK_BF16,
                          "gather_tbs": work["attn_gather_bytes"] / t_att / 1e12},
        }
        floor = max(work["indexer_flop"] / PEAK_FP8, 0) + work["topk_bytes"] / PEAK_HBM + work["attn_flop"] / PEAK_BF16
        res["e2e_frac_of_floor"] = floor / (ms * 1e-3)
        peaks = measured_mfma_peaks(dev, stream)
        res["measured_mfma_tflops"] = peaks
        res["indexer_frac_measured_peak"] = work["indexer_flop"] / t_idx / 1e12 / peaks["fp8_2_waves_per_simd"]
        res["stage_roofline"]["attention"]["frac_measured_peak"] = att / 1e12 / peaks["bf16_1_wave_per_simd"]
        res["input_side"] = input_side(cfg, dev, stream, max(1, args.steps))
        torch.cuda.empty_cache()
        if cfg.name == "mla_prefill_L32768" and not args.no_training:
            res["training_side"] = training_side(cfg, dev, stream, max(1, args.steps))
    if args.cpu_rows > 0:
        log(f"[bench] oracle on {args.cpu_rows} sampled rows")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
