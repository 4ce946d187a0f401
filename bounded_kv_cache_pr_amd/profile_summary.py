"""Summaries of rocprofv3 runs over bench.py: per-kernel durations, HBM bytes and
rates, the block timeline, and the attention counter record that bench.py
reports as ``roofline.traffic``.

    python -m bounded_kv_cache_pr_amd.profile_summary DIR --workload 480x480 --layers 4 \\
        [--record profiles/attn_bf16_kernel_480x480_traffic.json]

DIR holds one folder per rocprofv3 pass over the same bench.py command
(``rocprofv3 <pass options> --output-format csv -d DIR/<pass> -o run -- python3 bench.py ...``):

    trace   --kernel-trace --stats
    dram    --pmc TCC_EA0_RDREQ_DRAM_32B TCC_EA0_WRREQ_WRITE_DRAM_32B
    fetch   --pmc FETCH_SIZE
    write   --pmc WRITE_SIZE
    clock   --pmc GRBM_COUNT GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES

Missing passes are skipped.  The DRAM request counters count 32-byte units (a
128-byte request counts 4), so bytes = count x 32 with no calibration.
FETCH_SIZE / WRITE_SIZE are scaled by what they read for the Ref Sink's plain
copy (kv_write_kernel: 2 x ref_tokens rows read and written).

Dispatches are sorted into roles by kernel name and order: a block starts at
its retrieve_kernel; a rope_follow launch that the next launch on its queue is
the attention kernel rotates the current keys; one right after a slot_copy
rotates a new bank entry at the Dynamic Sink's place; one before the first
retrieval rotates a Ref Sink.  This module reads profiler output only; it runs
nothing on the GPU.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics as st
from collections import defaultdict

from . import synth

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# what the attention kernel is compiled from
ATTN_SOURCES = ("kernels_attn.hip", "prsink_device.h", "prsink_internal.h")

SHORT = ("attn_bf16_kernel", "attn_f32_kernel", "clean_write_kernel", "rope_follow_kernel",
         "slot_copy_kernel", "kv_write_kernel", "retrieve_kernel", "bank_update_kernel",
         "state_init_kernel")
N_SIMD = 256 * 4
N_XCD = 8


def attn_source_sha256(csrc: str | None = None) -> str:
    """sha256 over the attention kernel's source files (name and bytes of each)."""
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        h.update(name.encode() + b"\0")
        with open(os.path.join(csrc or CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(name: str):
    for k in SHORT:
        if k in name:
            return k
    return None


def load_pass(path: str):
    """Dispatches of one pass, in dispatch order: dicts with kernel, grid, queue,
    start/end (ns) and the counters summed over their instances."""
    trace = os.path.join(path, "run_kernel_trace.csv")
    ctr = os.path.join(path, "run_counter_collection.csv")
    rows = {}
    if os.path.exists(trace):
        with open(trace, newline="") as f:
            for r in csv.DictReader(f):
                k = short_name(r["Kernel_Name"])
                d = int(r["Dispatch_Id"])
                rows[d] = dict(id=d, kernel=k, name=r["Kernel_Name"], queue=int(r["Queue_Id"]),
                               grid=int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
                               start=int(r["Start_Timestamp"]), end=int(r["End_Timestamp"]), ctr={})
    elif os.path.exists(ctr):
        with open(ctr, newline="") as f:
            for r in csv.DictReader(f):
                d = int(r["Dispatch_Id"])
                if d not in rows:
                    rows[d] = dict(id=d, kernel=short_name(r["Kernel_Name"]), name=r["Kernel_Name"],
                                   queue=int(r["Queue_Id"]), grid=int(r["Grid_Size"]),
                                   start=int(r["Start_Timestamp"]), end=int(r["End_Timestamp"]),
                                   ctr=defaultdict(float))
                rows[d]["ctr"][r["Counter_Name"]] += float(r["Counter_Value"])
    else:
        return None
    return [rows[d] for d in sorted(rows)]


def assign_roles(ds):
    """Role and block index of every dispatch (block -1: before the first retrieval)."""
    block = -1
    by_queue = defaultdict(list)
    for d in ds:
        by_queue[d["queue"]].append(d)
    nxt, prv = {}, {}
    for q in by_queue.values():
        for a, b in zip(q, q[1:]):
            nxt[a["id"]], prv[b["id"]] = b, a
    for d in ds:
        k = d["kernel"]
        if k == "retrieve_kernel":
            block += 1
        d["block"] = block
        role = k
        if k == "rope_follow_kernel":
            n, p = nxt.get(d["id"]), prv.get(d["id"])
            if n is not None and n["kernel"] in ("attn_bf16_kernel", "attn_f32_kernel"):
                role = "rope_follow (current keys)"
            elif p is not None and p["kernel"] == "slot_copy_kernel":
                role = "rope_follow (bank entry)"
            elif block < 0:
                role = "rope_follow (Ref Sink)"
            else:
                role = "rope_follow (other)"
        elif k == "clean_write_kernel":
            role = "clean_write (block 0, +Static)" if block == 0 else "clean_write"
        d["role"] = role
    return ds


def algorithmic_bytes(cfg):
    """Bytes each role must move: (read, written)."""
    esz = 2 if cfg.dtype == synth.DTYPE_BF16 else 4
    row = cfg.n_heads * cfg.head_dim * esz
    T, Tr, L, W = cfg.block_tokens, cfg.ref_tokens, cfg.n_layers, cfg.window_slots
    K = cfg.full_cache_keys
    tab = 8 * (cfg.head_dim // 2)          # fp32 (cos, sin) per pair and token
    fp, M = cfg.fp_dim, cfg.bank_size
    return {
        "attn_bf16_kernel": ((T + 2 * K) * row, T * row),
        "attn_f32_kernel": ((T + 2 * K) * row, T * row),
        "rope_follow (current keys)": (T * row + T * tab, T * row),
        "rope_follow (Ref Sink)": (Tr * row + Tr * tab, Tr * row),
        "rope_follow (bank entry)": (L * T * row + T * tab, L * T * row),
        # K, V in; raw K (a block that may still enter the bank: every block of
        # the fill phase, which the profiled runs stay in), V and K rotated at the
        # W-1 window places out
        "clean_write": (2 * T * row + (W - 1) * T * tab, (2 + W - 1) * T * row),
        "clean_write (block 0, +Static)": (2 * T * row + W * T * tab, (2 + W - 1 + 2) * T * row),
        "slot_copy_kernel": (L * T * row, L * T * row),
        "kv_write_kernel": (2 * Tr * row, 2 * Tr * row),
        "retrieve_kernel": (4 * fp + 8 * M * fp, 8 * fp),
        "bank_update_kernel": (8 * fp + 8 * M * fp, 8 * fp),
    }


def med(xs):
    return st.median(xs) if xs else float("nan")


def steady(ds, role, from_block):
    return [d for d in ds if d["role"] == role and d["block"] >= from_block]


def summarise(root, workload, layers):
    base = synth.C3_STREAM_480 if workload == "480x480" else synth.C2_384x672
    cfg = base.replace(n_layers=layers)
    alg = algorithmic_bytes(cfg)
    passes = {}
    for p in ("trace", "dram", "fetch", "write", "clock"):
        ds = load_pass(os.path.join(root, p))
        if ds is not None:
            passes[p] = assign_roles(ds)
    # steady attention and current-key rotation: every segment full (block >= 3)
    first = {"attn_bf16_kernel": 3, "attn_f32_kernel": 3, "rope_follow (current keys)": 3}
    roles = [r for r in alg if any(d["role"] == r for ds in passes.values() for d in ds)]
    table = {}
    for role in roles:
        fb = first.get(role, -1)
        e = {"alg_read": alg[role][0], "alg_write": alg[role][1]}
        if "trace" in passes:
            xs = steady(passes["trace"], role, fb)
            e["n_trace"] = len(xs)
            e["trace_us"] = med([(d["end"] - d["start"]) / 1e3 for d in xs])
        for p, names in (("dram", ("TCC_EA0_RDREQ_DRAM_32B", "TCC_EA0_WRREQ_WRITE_DRAM_32B")),
                         ("fetch", ("FETCH_SIZE",)), ("write", ("WRITE_SIZE",)),
                         ("clock", ("GRBM_COUNT", "GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES",
                                    "SQ_VALU_MFMA_BUSY_CYCLES"))):
            if p not in passes:
                continue
            xs = steady(passes[p], role, fb)
            e[f"{p}_us"] = med([(d["end"] - d["start"]) / 1e3 for d in xs])
            e[f"n_{p}"] = len(xs)
            for n in names:
                e[n] = med([d["ctr"].get(n, 0.0) for d in xs])
        table[role] = e
    # FETCH_SIZE / WRITE_SIZE calibration on the Ref Sink's plain copy
    cal = None
    kv = table.get("kv_write_kernel")
    if kv and kv.get("FETCH_SIZE") and kv.get("WRITE_SIZE"):
        cal = {"fetch_factor": kv["alg_read"] / (kv["FETCH_SIZE"] * 1024),
               "write_factor": kv["alg_write"] / (kv["WRITE_SIZE"] * 1024),
               "fetch_kib": kv["FETCH_SIZE"], "write_kib": kv["WRITE_SIZE"],
               "copy_kib": kv["alg_read"] / 1024}
    for e in table.values():
        if "TCC_EA0_RDREQ_DRAM_32B" in e:
            e["dram_read"] = 32 * e["TCC_EA0_RDREQ_DRAM_32B"]
            e["dram_write"] = 32 * e["TCC_EA0_WRREQ_WRITE_DRAM_32B"]
        if cal and "FETCH_SIZE" in e and "WRITE_SIZE" in e:
            e["fetch_bytes"] = e["FETCH_SIZE"] * 1024 * cal["fetch_factor"]
            e["write_bytes"] = e["WRITE_SIZE"] * 1024 * cal["write_factor"]
        if "GRBM_COUNT" in e and e.get("clock_us"):
            e["clock_ghz"] = e["GRBM_COUNT"] / N_XCD / (e["clock_us"] * 1e3)
            e["mfma_busy_pct"] = 100 * e["SQ_VALU_MFMA_BUSY_CYCLES"] / (
                N_SIMD * e["GRBM_COUNT"] / N_XCD)
    return cfg, passes, table, cal


def timeline(ds, blocks):
    """Per-block breakdown of the trace: block span (retrieval to next retrieval),
    time per role on the attention queue, the rest of that queue's time (idle),
    and busy time on the other queues."""
    starts = {}
    for d in ds:
        if d["kernel"] == "retrieve_kernel":
            starts[d["block"]] = d["start"]
    attn_q = next((d["queue"] for d in ds if d["kernel"] == "attn_bf16_kernel"), None)
    rows = []
    for b in blocks:
        if b not in starts or b + 1 not in starts:
            continue
        t0, t1 = starts[b], starts[b + 1]
        per = defaultdict(float)
        other = 0.0
        for d in ds:
            if d["block"] != b:
                continue
            us = (d["end"] - d["start"]) / 1e3
            if d["queue"] == attn_q:
                per[d["role"]] += us
            else:
                other += us
        span = (t1 - t0) / 1e3
        rows.append(dict(block=b, span_us=span, attn_queue=dict(per),
                         attn_queue_idle_us=span - sum(per.values()), other_queues_busy_us=other))
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    ap.add_argument("--workload", choices=("480x480", "384x672"), default="480x480")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--record", help="write the attention counter record (JSON) here")
    ap.add_argument("--timeline", help="blocks a..b of the trace pass to break down, e.g. 3..12")
    args = ap.parse_args()
    cfg, passes, table, cal = summarise(args.dir, args.workload, args.layers)
    mb = lambda x: f"{x / 1e6:.2f}"
    print(f"| Kernel (role) | n | trace us | alone us | alg read MB | alg write MB | alg TB/s (alone) "
          f"| DRAM read MB | DRAM write MB | DRAM TB/s | FETCH KiB | WRITE KiB |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|")
    for role, e in table.items():
        alone = e.get("dram_us", float("nan"))
        a_tbs = (e["alg_read"] + e["alg_write"]) / (alone * 1e-6) / 1e12 if alone == alone else float("nan")
        d_tbs = ((e["dram_read"] + e["dram_write"]) / (alone * 1e-6) / 1e12) if "dram_read" in e else float("nan")
        print(f"| {role} | {e.get('n_trace', e.get('n_dram', 0))} | {e.get('trace_us', float('nan')):.2f} "
              f"| {alone:.2f} | {mb(e['alg_read'])} | {mb(e['alg_write'])} | {a_tbs:.2f} "
              f"| {mb(e.get('dram_read', float('nan')))} | {mb(e.get('dram_write', float('nan')))} | {d_tbs:.2f} "
              f"| {e.get('FETCH_SIZE', float('nan')):.1f} | {e.get('WRITE_SIZE', float('nan')):.1f} |")
    if cal:
        print(f"\ncalibration: kv_write copy of {cal['copy_kib']:.1f} KiB read + written: FETCH "
              f"{cal['fetch_kib']:.1f} KiB (x{cal['fetch_factor']:.6f}), WRITE {cal['write_kib']:.1f} KiB "
              f"(x{cal['write_factor']:.6f})")
    a = table.get("attn_bf16_kernel")
    if a and "clock_ghz" in a:
        print(f"attention: shader clock {a['clock_ghz']:.3f} GHz, MFMA busy {a['mfma_busy_pct']:.2f} % "
              f"of SIMD-cycles (SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles))")
    if args.timeline and "trace" in passes:
        lo, hi = (int(x) for x in args.timeline.split(".."))
        rows = timeline(passes["trace"], range(lo, hi + 1))
        roles = sorted({r for row in rows for r in row["attn_queue"]})
        print(f"\nblocks {lo}..{hi} (median over {len(rows)} blocks, us): span "
              f"{med([r['span_us'] for r in rows]):.1f}")
        for r in roles:
            print(f"  attention queue, {r}: {med([row['attn_queue'].get(r, 0.0) for row in rows]):.1f}")
        print(f"  attention queue idle: {med([r['attn_queue_idle_us'] for r in rows]):.1f}")
        print(f"  other queues busy: {med([r['other_queues_busy_us'] for r in rows]):.1f}")
    if args.record:
        if not (a and cal and "dram_read" in a):
            raise SystemExit("the record needs the dram, fetch and write passes")
        rec = {
            "kernel": "attn_bf16_kernel<128>",
            "workload": f"{args.workload} block, H={cfg.n_heads}, d={cfg.head_dim}, Q={cfg.block_tokens}, "
                        f"K={cfg.full_cache_keys}",
            "attn_sources_sha256": attn_source_sha256(),
            "dispatches": a["n_fetch"],
            "fetch_size_kib": round(a["FETCH_SIZE"], 1),
            "write_size_kib": round(a["WRITE_SIZE"], 1),
            "fetch_factor": round(cal["fetch_factor"], 6),
            "write_factor": round(cal["write_factor"], 6),
            "calibration": f"kv_write_kernel copy (Ref Sink write) of {cal['copy_kib']:.1f} KiB read + "
                           f"{cal['copy_kib']:.1f} KiB written: FETCH {cal['fetch_kib']:.1f} KiB, "
                           f"WRITE {cal['write_kib']:.1f} KiB",
            "traffic_bytes_per_launch": int(round(a["fetch_bytes"] + a["write_bytes"])),
            "dram_read_bytes_per_launch": int(round(a["dram_read"])),
            "dram_write_bytes_per_launch": int(round(a["dram_write"])),
            "dram_note": "TCC_EA0_RDREQ_DRAM_32B and TCC_EA0_WRREQ_WRITE_DRAM_32B x 32 bytes, no calibration",
            "algorithmic_bytes_per_launch": int(a["alg_read"] + a["alg_write"]),
        }
        if "clock_ghz" in a:
            rec["shader_clock_ghz"] = round(a["clock_ghz"], 3)
            rec["mfma_util_pct"] = round(a["mfma_busy_pct"], 2)
            rec["clock_note"] = ("GRBM_COUNT summed over the 8 XCDs / 8 / dispatch duration; MFMA busy = "
                                 "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_COUNT / 8); steady dispatches, median")
        with open(args.record, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(f"\nwrote {args.record}")


if __name__ == "__main__":
    main()
