"""PR-Sink hot-path benchmark on one MI355X.

One step = one streamed block of the 480x480 workload (40 heads, d=128,
Q=2700 tokens, K=14400 keys once the cache is full, 40 layers): pose
retrieval (the Dynamic Sink reads the retrieved bank entry in place), 40
layers x 3 denoise-step attention calls, 40 clean-KV writes, and the bank
update (blocks < 20).  With --streams 2 (the default) the clean writes and the
bank update run on a second stream; the library's events order them against
the attention calls.  Inputs are synthetic,
seeded and resident in HBM before the timed region; the attention inputs of a
step cycle through pools of 7 distinct Q/K/V sets so consecutive calls do not
reuse cached keys.

--workload 384x672 runs the same step on the 384x672 bucket (Q=3024,
K=16128) instead.

--attends-per-layer 4 adds the clean forward's own attention call to every
layer (160 calls per block at 40 layers) as a variant; 3, the denoise steps
alone, is the headline step.

Prints one JSON line.  `value` is attention TFLOP/s over the whole step (120
attention calls' algorithmic FLOPs / block time).  The timed blocks carry no
timing markers.  After them, untimed blocks of the same stream measure the
whole pr_sink_attend call (attn_ms_per_call: rotation of the current keys +
attention kernel; one block, HIP events around each call) and the attention
kernel alone (attn_kernel_ms, which the roofline uses; two blocks, HIP events
the library records right around each launch).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "PR-Sink attn ms/call + TFLOP/s (% bf16 MFMA peak), 480×480 block; ms/block stream"
# --workload 384x672 times the 384x672 bucket (H=40, d=128, 24x42 tokens per
# frame: Q=3024, K=16128) the same way; 480x480 is the headline workload
WORKLOADS = ("480x480", "384x672")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
POOL = 7                    # distinct input sets per pool (coprime to the layer count)
KERNEL_BLOCKS = 2           # untimed blocks whose attention kernels carry HIP events


def counter_record(workload):
    """The committed rocprofv3 counter record of the workload (HBM bytes per attention
    launch from FETCH_SIZE / WRITE_SIZE, cross-checked by the DRAM request counters; the
    shader clock and MFMA utilisation), or None when there is none or the attention
    kernel's sources have changed since it was taken."""
    from bounded_kv_cache_pr_amd.profile_summary import attn_source_sha256
    record = os.path.join(ROOT, "profiles", f"attn_bf16_kernel_{workload}_traffic.json")
    try:
        with open(record) as f:
            rec = json.load(f)
        sha = attn_source_sha256()
    except OSError:
        return None
    return rec if rec.get("attn_sources_sha256") == sha else None


def attn_flops(cfg) -> float:
    return 4.0 * cfg.n_heads * cfg.block_tokens * cfg.full_cache_keys * cfg.head_dim


def cpu_baseline(cfg, q, kc, vc, ref_kv_host, block_kv_host, orc, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the same attention call: whole heads
    until ~budget_s of CPU time has been spent."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    done, t_total = 0, 0.0
    for h in range(cfg.n_heads):
        t0 = time.perf_counter()
        orc.attend(q, kc, vc, ref_kv_host, block_kv_host, heads=[h])
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    flops = attn_flops(cfg) * done / cfg.n_heads
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {cfg.n_heads} heads of one {cfg.lat_h * 16}x{cfg.lat_w * 16} "
                      f"attention call (Q={cfg.block_tokens}, K={cfg.full_cache_keys}, "
                      f"d={cfg.head_dim}), numpy fp64, {t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--streams", type=int, choices=(1, 2), default=2,
                    help="2: clean-KV writes and the bank update on a second stream")
    ap.add_argument("--workload", choices=WORKLOADS, default="480x480")
    ap.add_argument("--attends-per-layer", type=int, choices=(3, 4), default=3,
                    help="attention calls per layer and block: the 3 denoise steps, or 4 when the "
                         "clean forward's own attention is counted too (160 calls at 40 layers)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the PR-Sink path here runs on a single MI355X "
              "(no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bounded_kv_cache_pr_amd import binding, build, synth

    if not os.path.exists(build.LIB_PATH):
        build.build_library()
    dev = torch.device("cuda:0")
    base = synth.C3_STREAM_480 if args.workload == "480x480" else synth.C2_384x672
    cfg = base.replace(n_layers=args.layers)
    L, steps = cfg.n_layers, args.attends_per_layer
    n_blocks = args.warmup + args.steps
    seed = args.seed

    cache = binding.PRSinkCache(cfg, device=dev)
    for l in range(L):
        k, v = synth.ref_kv_torch(cfg, l, seed, dev)
        cache.set_ref(l, k, v)
    qkv_pool = [synth.step_qkv_torch(cfg, 10_000 + i, 0, 0, seed, dev) for i in range(POOL)]
    clean_pool = [synth.clean_kv_torch(cfg, 20_000 + i, 0, seed, dev) for i in range(POOL)]
    out = torch.empty_like(qkv_pool[0][0])
    fps = torch.from_numpy(synth.pose_stream(n_blocks + 1 + KERNEL_BLOCKS, seed=seed)).to(dev)
    stream = torch.cuda.current_stream(dev)
    clean_stream = torch.cuda.Stream(dev) if args.streams == 2 else stream
    # whole-call events, recorded on one extra block after the timed region so
    # the timed blocks carry only the kernel events below
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps * L)]
    # events the library records right around its attention kernel (the
    # kernel alone, without the rotation of the current keys before it)
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps * L * KERNEL_BLOCKS)]
    for a, z in kev:  # create the events before handing them over
        a.record(stream)
        z.record(stream)

    def run_block(b, kernel_base=None, call_events=False):
        cache.retrieve(b, fps[b])
        for s in range(steps):
            for l in range(L):
                q, k, v = qkv_pool[(b * steps * L + s * L + l) % POOL]
                if kernel_base is not None:
                    cache.set_attend_events(*kev[kernel_base + s * L + l])
                if call_events:
                    e0, e1 = ev[s * L + l]
                    e0.record(stream)
                    cache.attend(l, q, k, v, out=out)
                    e1.record(stream)
                else:
                    cache.attend(l, q, k, v, out=out)
        with torch.cuda.stream(clean_stream):  # ordered by the library's events
            for l in range(L):
                k, v = clean_pool[(b * L + l) % POOL]
                cache.clean_kv_write(l, k, v)
            cache.bank_update(b)

    cache.set_attend_events()
    for b in range(args.warmup):
        run_block(b)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_block(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    run_block(n_blocks, call_events=True)   # untimed: whole-call durations
    for i in range(KERNEL_BLOCKS):          # untimed: attention kernel durations
        run_block(n_blocks + 1 + i, kernel_base=i * steps * L)
    torch.cuda.synchronize()
    cache.set_attend_events()

    ms_per_block = (t1 - t0) * 1e3 / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    attn_avg_ms = float(np.mean(attn_ms))
    kern_ms = [a.elapsed_time(b) for a, b in kev]
    kern_avg_ms = float(np.mean(kern_ms))
    flops = attn_flops(cfg)
    achieved = flops / (kern_avg_ms * 1e-3) / 1e12
    value = steps * L * flops / (ms_per_block * 1e-3) / 1e12

    T, Kc = cfg.block_tokens, cfg.full_cache_keys
    result = {
        "metric": METRIC if args.workload == "480x480" else METRIC.replace("480×480", "384×672"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_block, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"PR-Sink streamed block at {args.workload}: H={cfg.n_heads}, "
                        f"d={cfg.head_dim}, Q={T}, K={Kc} "
                        f"(Ref {cfg.ref_tokens} + Static/Dynamic/2 window/current {T} each), {L} layers x "
                        f"{steps} attention calls ({'denoise steps' if steps == synth.DENOISE_STEPS else 'denoise steps + the clean forward'}) + {L} clean-KV writes + "
                        "retrieval + bank update",
            "blocks_timed": f"{args.warmup}..{n_blocks - 1}",
            "streams": args.streams,
            "layers": L,
            "attends_per_layer": steps,
        },
        "attn_ms_per_call": round(attn_avg_ms, 5),
        "attn_kernel_ms": round(kern_avg_ms, 5),
        "attn_ms_p10_p50_p90": [round(float(np.percentile(attn_ms, p)), 5) for p in (10, 50, 90)],
        "attn_kernel_tflops": round(achieved, 2),
        "attn_kernel_frac_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "ms_per_block": round(ms_per_block, 3),
        "fps_equiv_12_frames_per_block": round(12.0 / (ms_per_block * 1e-3), 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
    }
    rec = counter_record(args.workload)
    if rec is not None:
        result["roofline"]["traffic"] = rec["traffic_bytes_per_launch"]
        if "shader_clock_ghz" in rec:
            # context, not the fraction of the published peak: the MFMA peak at
            # the shader clock the counter pass measured during this kernel (a
            # separate rocprofv3 run; the clock differs from box to box)
            peak_clk = PEAK_BF16_TFLOPS * rec["shader_clock_ghz"] / 2.4
            result["clock_adjusted"] = {
                "shader_clock_ghz": rec["shader_clock_ghz"],
                "peak_tflops_at_clock": round(peak_clk, 1),
                "frac": round(achieved / peak_clk, 4),
                "mfma_busy_pct": rec.get("mfma_util_pct"),
                "source": f"profiles/attn_bf16_kernel_{args.workload}_traffic.json (counter pass of "
                          "another run)",
            }

    if not args.no_cpu_baseline:
        import oracle as O
        b = n_blocks
        orc = O.PRSinkOracle(cfg)
        fps_h = fps.cpu().numpy()
        t_rb = time.perf_counter()
        for blk in range(n_blocks):
            orc.open_block(blk, fps_h[blk])
            orc.close_block(blk)
        rb_ms = (time.perf_counter() - t_rb) * 1e3 / n_blocks
        orc.open_block(b, fps_h[b])
        host = lambda t: t.float().cpu().numpy()
        l = 0
        q, k, v = (host(x) for x in qkv_pool[0])
        ref_host = tuple(host(x) for x in synth.ref_kv_torch(cfg, l, seed, dev))
        block_host = lambda bid: tuple(host(x) for x in clean_pool[(bid * L + l) % POOL])
        result["cpu_baseline"] = cpu_baseline(cfg, q, k, v, ref_host, block_host, orc,
                                              args.cpu_budget)
        # the oracle's retrieval and bank update, per block (the fill phase's blocks)
        result["cpu_baseline"]["retrieval_bank_ms_per_block"] = round(rb_ms, 3)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
