"""Batch-1 decode benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2b|2b_32k|moe|tiny|gemv]

A step is one generation request: ONE kie_decode launch of the workload's
decode length (1024 greedy tokens for the default ~2.1B decoder) from the
same post-prompt state. W untimed steps, then exactly K timed steps bracketed
by torch.cuda.synchronize(); one JSON line is printed. Inputs are seeded and
synthetic and stay resident in HBM; the workload stands in for the pages' 2B
model (25 layers, fp16, batch 1).

The JSON line carries:
  value      whole-job tokens/s (one GPU);
  mbu        (active weight + KV bytes per token) x tok/s / 8 TB/s;
  roofline   algorithmic bytes of one launch / the launch's mean device time
             (HIP events recorded by the library on its stream), against the
             8 TB/s HBM peak; traffic from committed rocprofv3 counter
             summaries when they match the current kernel sources, else null;
  cpu_baseline  the CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from memory_bandwidth_bound_amd import roofline  # noqa: E402

PEAK_GBS = roofline.HBM_PEAK_BYTES_PER_S / 1e9


def kernel_source_hash(probes: bool = False) -> str:
    """Hash of the sources a kernel and its launch are built from: for the
    decode kernel every csrc file but the measurement probes and the batched
    prefill; with probes=True every csrc file."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "memory_bandwidth_bound_amd", "csrc", "*"))):
        if os.path.basename(p) in ("kie_probes.hip", "kie_prefill.hip") and not probes:
            continue
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_traffic(name: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_hash(probes=name.endswith("_probe")):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


WEIGHT_DESC = {"fp16": "fp16 weights", "fp8": "E4M3 weights (dequantised)", "fp4": "E2M1 weights (dequantised)"}
DTYPE = {"fp16": "fp16", "fp8": "fp8-e4m3 weights, fp32 math", "fp4": "fp4-e2m1 weights, fp32 math"}


def describe(cfg) -> str:
    s = (f"{cfg.name} decoder: {cfg.n_layers} layers, d_model {cfg.d_model}, {cfg.n_heads} query / "
         f"{cfg.n_kv_heads} KV heads x {cfg.head_dim}, SwiGLU {cfg.ffn_dim}")
    if cfg.n_experts:
        s += f" x {cfg.n_experts} experts (top-{cfg.top_k})"
    wf = getattr(cfg, "weight_format", "fp16")
    if wf in ("fp8", "fp4"):
        name = "FP8 E4M3" if wf == "fp8" else "FP4 E2M1"
        s += (f", vocab {cfg.vocab}, weights N(0,{cfg.weight_sigma}) held as {name} with one fp32 scale per row "
              f"(quantised at load; embedding fp16); batch 1, ")
    else:
        s += f", vocab {cfg.vocab}, fp16 weights N(0,{cfg.weight_sigma}); batch 1, "
    if cfg.kv_prefill:
        s += f"KV cache pre-filled with {cfg.kv_prefill} seeded positions, "
    else:
        s += f"{cfg.prompt_len}-token prompt, "
    s += f"{cfg.decode_steps} greedy decode steps per request"
    return s


# ----------------------------------------------------------------------------
def cpu_baseline_decode(cfg, W, prompt, target_s: float):
    """The oracle as it stands, timed on this host on a bounded sample: greedy
    decode passes right after the prompt (or the pre-filled cache)."""
    import oracle
    dec = oracle.Decoder(cfg, W)
    if cfg.kv_prefill:
        K, V = synth.make_kv_prefill(cfg)
        dec.set_kv(K, V, synth.make_pending_token(cfg))
        del K, V
    else:
        dec.prefill_batched(prompt)
    t0 = time.perf_counter()
    dec.decode(1)
    t1 = time.perf_counter() - t0
    start = (cfg.kv_prefill or cfg.prompt_len) + 1
    room = cfg.max_seq - start          # positions left in the oracle's KV cache
    n = int(max(1, min(64, room, round(target_s / max(t1, 1e-3)))))
    t0 = time.perf_counter()
    dec.decode(n)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tok/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{n} greedy decode passes of the {cfg.name} decoder at positions "
                      f"{start}..{start + n - 1} (numpy fp32 on the "
                      f"{WEIGHT_DESC.get(getattr(cfg, 'weight_format', 'fp16'), 'fp16 weights')}"
                      f"), after one untimed pass; "
                      f"host os.cpu_count()={os.cpu_count()}"}


def bench_decode(cfg, args):
    import torch
    from memory_bandwidth_bound_amd import kie
    if args.tokens:
        cfg = cfg.with_(decode_steps=args.tokens)
    t_setup = time.perf_counter()
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg)
    m = kie.Model(cfg, W, device="cuda:0")
    m.set_attention_mode(args.attention)
    if cfg.kv_prefill:
        K, V = synth.make_kv_prefill(cfg)
        pend = synth.make_pending_token(cfg)
        m.set_kv(K, V, pend)
        del K, V
        pos0, first = cfg.kv_prefill, pend
    else:
        first, _, _ = m.prefill(prompt)
        pos0 = cfg.prompt_len
    n = cfg.decode_steps
    print(f"# setup {time.perf_counter() - t_setup:.1f}s; decode {n} tokens per step from position {pos0}",
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        m.rewind(pos0, first)
        m.decode(n)
    torch.cuda.synchronize()
    kms = []
    ids_first = None
    t0 = time.perf_counter()
    for _ in range(args.steps):
        m.rewind(pos0, first)
        ids, _, _ = m.decode(n)
        kms.append(m.last_kernel_ms)
        if ids_first is None:
            ids_first = ids
        elif not np.array_equal(ids, ids_first):
            raise RuntimeError("repeated decode requests produced different tokens")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tok_s = args.steps * n / wall
    algo = roofline.decode_bytes(cfg, pos0, n)
    k_ms = float(np.mean(kms))
    per_tok = algo / n
    achieved = algo / (k_ms * 1e-3) / 1e9
    traffic = counters_traffic(f"decode_{cfg.name}")
    line = {
        "metric": "batch-1 decode tokens/sec on 1 MI355X + MBU (% of 8 TB/s HBM)",
        "value": round(tok_s, 2), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[getattr(cfg, "weight_format", "fp16")],
        "data": "synthetic",
        "config": {"workload": describe(cfg), "global_batch": 1, "seq_len": pos0 + n,
                   "decode_tokens_per_step": n, "parallelism": "single GPU, one persistent launch per request",
                   "attention": args.attention},
        "mbu": round(per_tok * tok_s / roofline.HBM_PEAK_BYTES_PER_S, 4),
        "bytes_per_token": per_tok,
        "kernel_ms_mean": round(k_ms, 3),
        "kernel_tok_per_s": round(n / (k_ms * 1e-3), 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4),
                     "traffic": traffic},
        "launches_per_request": 1,
    }
    m.close()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(cfg, W, prompt, args.cpu_seconds)
    return line


def bench_gemv(args):
    import torch
    import oracle
    from memory_bandwidth_bound_amd import kie
    cfg = synth.get_config("gemv")
    shapes = []
    tot_bytes, tot_ms = 0.0, 0.0
    for si, (M, K) in enumerate(cfg.shapes):
        A, x = synth.make_probe(si, M, K)
        mat = 2 * M * K
        copies = max(1, -(-(1 << 30) // mat))       # >= 1 GiB per launch (4x the 256 MB MALL)
        At = torch.from_numpy(A).cuda()
        Ac = At.unsqueeze(0).repeat(copies, 1, 1).contiguous()
        xt = torch.from_numpy(x).cuda()
        for _ in range(args.warmup):
            kie.gemv_probe(Ac, xt, variant=0)
        ms = []
        for _ in range(args.steps):
            _, t = kie.gemv_probe(Ac, xt, variant=0)
            ms.append(t)
        _, t_direct = kie.gemv_probe(Ac, xt, variant=1)
        b = copies * roofline.gemv_bytes(M, K)
        gbs = b / (np.mean(ms) * 1e-3) / 1e9
        shapes.append({"shape": [M, K], "copies": copies, "GB_s": round(gbs, 1),
                       "direct_GB_s": round(b / (t_direct * 1e-3) / 1e9, 1)})
        tot_bytes += b
        tot_ms += float(np.mean(ms))
        del Ac, At
        torch.cuda.empty_cache()
    agg = tot_bytes / (tot_ms * 1e-3) / 1e9
    line = {
        "metric": "GEMV achieved HBM bandwidth (fp16 matrix x vector, fp32 accumulate)",
        "value": round(agg, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(tot_ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "GEMV probe: fp16 row-major 2560x2560, 2560x8192, 8192x2560, 2560x32768 "
                               "x fp16 vector, rotating copies >= 1 GiB per launch", "shapes": shapes},
        "roofline": {"bound": "hbm", "achieved": round(agg, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(agg / PEAK_GBS, 4), "traffic": counters_traffic("gemv_probe")},
    }
    if not args.no_cpu_baseline:
        M, K = cfg.shapes[1]
        A, x = synth.make_probe(1, M, K)
        reps = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            oracle.gemv_f64(A, x)
            reps += 1
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(reps * roofline.gemv_bytes(M, K) / dt / 1e9, 3), "unit": "GB/s",
                                "cores": blas_threads(), "kind": "oracle",
                                "sample": f"{reps} float64 GEMVs of the {M}x{K} fp16 matrix (oracle gemv_f64)"}
    return line


def bench_prefill(args):
    """Prompt processing of the ~2.1B decoder: the 128-token prompt through the
    batched matrix-core prefill (and, for comparison, one persistent launch
    of 128 decode passes); roofline of the GEMM kernel on the prompt's largest
    projection (gate/up: 128 x 16384 x 2560), timed by the library with HIP
    events. Not the decode metric."""
    import torch
    from memory_bandwidth_bound_amd import kie
    cfg = synth.get_config("2b")
    W = synth.make_weights(cfg)
    P = synth.make_prompt(cfg)
    m = kie.Model(cfg, W, device="cuda:0")
    out = {}
    for mode in ("auto", "passes"):
        m.set_prefill_mode(mode)
        for _ in range(args.warmup):
            m.prefill(P)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            m.prefill(P)
        torch.cuda.synchronize()
        out[mode] = (time.perf_counter() - t0) / args.steps
    m.close()
    del W
    n, M, K = len(P), 2 * cfg.ffn_dim, cfg.d_model
    A = torch.randn((n, K), dtype=torch.float32, device="cuda:0")
    Wg = (torch.randn((M, K), device="cuda:0") * 0.02).to(torch.float16)
    kie.gemm_probe(A, Wg)
    ms = float(np.mean([kie.gemm_probe(A, Wg)[1] for _ in range(max(3, args.steps))]))
    flops = 2.0 * n * M * K                          # algorithmic: one product per (row, weight)
    tflops = flops / (ms * 1e-3) / 1e12
    wbytes = 2.0 * M * K + 4.0 * n * K + 4.0 * n * M  # weights once, fp32 activations in, fp32 out
    gbs = wbytes / (ms * 1e-3) / 1e9
    # 128 prompt rows: 2n/2 = 128 FLOP per weight byte, below the ridge of
    # 2.5 PFLOP/s over 8 TB/s (~312): the GEMM's roofline is HBM
    return {"metric": "prefill tokens/sec on 1 MI355X (batched matrix-core prompt processing)",
            "value": round(n / out["auto"], 1), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(out["auto"] * 1e3, 3), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp16 weights, fp16x2 activations, fp32 accumulate",
            "data": "synthetic",
            "config": {"workload": describe(cfg).replace(f", {cfg.decode_steps} greedy decode steps per request",
                                                         "; the prompt only"),
                       "prompt_tokens": n, "passes_ms": round(out["passes"] * 1e3, 3)},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_GBS, 4), "traffic": None,
                         "kernel": f"gemm_mfma {n}x{M}x{K}, {ms:.4f} ms, {tflops:.1f} TFLOP/s of 2500 dense fp16 "
                                   f"(two fp16 MFMAs per step: hi and lo terms)"}}


def bench_copy(args):
    """Counter calibration: a plain device copy of a known size (1 GiB read,
    1 GiB written per launch), timed like the other workloads."""
    import torch
    n = 1 << 30
    src = torch.empty(n // 2, dtype=torch.float16, device="cuda:0").normal_()
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(args.steps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    gbs = 2 * n / (ms * 1e-3) / 1e9
    return {"metric": "device copy bandwidth (read + write)", "value": round(gbs, 1), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
            "data": "synthetic",
            "config": {"workload": "torch copy_ of a 1 GiB fp16 tensor (counter calibration)",
                       "bytes_read": n, "bytes_written": n},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_GBS, 4), "traffic": None}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="2b",
                    help="2b (default), 2b_32k, 2b_fp8, 2b_fp4, moe, moe_fp8, moe_fp4, tiny, gemv, prefill, "
                         "or copy (counter calibration)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attention", choices=("global", "xcd_local"), default="global",
                    help="decode configs: attention at short context on the whole grid (default) or "
                         "recomputed on every XCD")
    ap.add_argument("--tokens", type=int, default=0,
                    help="decode configs: passes per request (default: the workload's request length)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decoder runs on a single GPU and has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        sys.exit("--steps must be >= 1")
    import torch
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.config == "gemv":
        line = bench_gemv(args)
    elif args.config == "prefill":
        line = bench_prefill(args)
    elif args.config == "copy":
        line = bench_copy(args)
    else:
        line = bench_decode(synth.get_config(args.config), args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
