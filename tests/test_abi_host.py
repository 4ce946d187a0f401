"""CPU tests of the C ABI: the library loads, exports what include/pr_sink.h
declares, and validates configs, arguments and call order without a GPU
(dry-run caches never touch a device)."""
import os
import re
import sys

import pytest

from bounded_kv_cache_pr_amd import binding, build, synth
from bounded_kv_cache_pr_amd.binding import (PR_SINK_EINVAL, PR_SINK_ENOSPACE, PR_SINK_ESTATE,
                                             PRSinkCache, PRSinkError)

HEADER = os.path.join(build.ROOT, "include", "pr_sink.h")


@pytest.fixture(scope="module", autouse=True)
def built_lib():
    if not os.path.exists(build.LIB_PATH):
        build.build_library()
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(pr_sink_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls_and_library_exports_all():
    names = declared_functions()
    for must in ("pr_sink_cache_init", "pr_sink_retrieve", "pr_sink_bank_update",
                 "pr_sink_attend", "pr_sink_clean_kv_write"):
        assert must in names
    lib = binding.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"
    assert set(names) == set(binding.EXPORTED)


def test_arena_bytes_closed_form():
    for cfg in (synth.C0_TINY, synth.C1_480, synth.C2_384x672, synth.C4_STREAM_672x384):
        esz = 2 if cfg.dtype == synth.DTYPE_BF16 else 4
        pad = lambda n: -(-n // 64) * 64
        slots = 1 + cfg.window_slots + cfg.bank_size  # Static, window, bank (Dynamic reads a bank entry)
        row = cfg.n_heads * cfg.head_dim * esz
        # the Ref slot holds raw K, V and rotated K per layer; a block slot V
        # and rotated K; raw keys are kept for the W window blocks only; a
        # window block is attended at W-1 places, so each window slot keeps
        # W-2 more rotated copies; plus the current block's rotated K
        kv = 3 * cfg.n_layers * row * pad(cfg.ref_tokens) + 2 * cfg.n_layers * row * slots * pad(cfg.block_tokens)
        kv += cfg.window_slots * cfg.n_layers * row * pad(cfg.block_tokens)
        kv += cfg.window_slots * max(0, cfg.window_slots - 2) * cfg.n_layers * row * pad(cfg.block_tokens)
        kv += row * pad(cfg.block_tokens)
        # cos/sin tables of every place (fp32 pairs): the Ref Sink's, then the
        # Static, Dynamic, W-1 window and current places of a block
        kv += 8 * (cfg.head_dim // 2) * (cfg.ref_tokens + (cfg.window_slots + 2) * cfg.block_tokens)
        if cfg.dtype == synth.DTYPE_BF16:
            # split attention jobs: up to 4 pieces of each of up to 32 jobs per
            # XCD (8 XCDs), one fp32 partial record per piece (256 rows x d of
            # O, plus (m, l) per lane), and one counter per split job
            kv += 8 * 32 * 4 * (256 * cfg.head_dim + 1024) * 4 + 8 * 32 * 4
        n = binding.arena_bytes(cfg)
        slack = (slots + 3 + cfg.window_slots) * 4096 + 4 * cfg.n_layers * (slots + 1) * 256 + (1 << 20)
        assert kv <= n <= kv + slack
    # the footprint is a function of the config alone: it grows with layers, not with blocks
    a1 = binding.arena_bytes(synth.C1_480.replace(n_layers=1))
    a2 = binding.arena_bytes(synth.C1_480.replace(n_layers=2))
    assert a2 > a1


@pytest.mark.parametrize("bad", [
    dict(head_dim=96), dict(rope_dims=(44, 42, 40)), dict(rope_dims=(43, 43, 42)),
    dict(n_layers=0), dict(window_slots=0), dict(window_slots=6), dict(bank_size=1),
    dict(bank_size=9), dict(fp_dim=0), dict(rope_theta=0.0), dict(lat_h=0), dict(t0=-1),
    dict(block_frames=0), dict(bank_fill_blocks=-1),
    dict(bank_policy=8), dict(bank_policy=2, bank_stale_blocks=0),
    dict(bank_policy=4, bank_refresh_tau=1.5), dict(bank_policy=4, bank_refresh_tau=float("nan")),
])
def test_invalid_configs_are_rejected(bad):
    cfg = synth.C1_480.replace(**bad)
    with pytest.raises(PRSinkError) as e:
        binding.arena_bytes(cfg)
    assert e.value.code == PR_SINK_EINVAL
    assert binding.last_error()


def test_arena_too_small_is_enospace():
    from ctypes import byref, c_void_p
    cfg = synth.C0_TINY
    c = binding.to_c_config(cfg)
    h = c_void_p()
    need = binding.arena_bytes(cfg)
    rc = binding.lib().pr_sink_cache_init(byref(c), 1 << 20, need - 1, None, byref(h))
    assert rc == PR_SINK_ENOSPACE and not h.value
    rc = binding.lib().pr_sink_cache_init(byref(c), (1 << 20) + 8, need, None, byref(h))
    assert rc == PR_SINK_EINVAL  # misaligned arena


FAKE = 1 << 20  # 16-byte aligned, never dereferenced by a dry-run cache


def _dry(cfg=synth.C0_TINY):
    return PRSinkCache(cfg, dry_run=True)


def _code(fn, *a):
    with pytest.raises(PRSinkError) as e:
        fn(*a)
    return e.value.code


def test_block_protocol_order():
    cfg = synth.C0_TINY
    c = _dry(cfg)
    assert _code(c.retrieve, 0, FAKE) == PR_SINK_ESTATE          # Ref Sink not set
    for l in range(cfg.n_layers):
        c.set_ref(l, FAKE, FAKE)
    assert _code(c.retrieve, 1, FAKE) == PR_SINK_ESTATE          # block 0 first
    assert _code(c.attend, 0, FAKE, FAKE + 16, FAKE + 32, FAKE + 48) == PR_SINK_ESTATE
    assert _code(c.clean_kv_write, 0, FAKE, FAKE) == PR_SINK_ESTATE
    assert _code(c.bank_update, 0) == PR_SINK_ESTATE
    c.retrieve(0, FAKE)
    assert _code(c.retrieve, 1, FAKE) == PR_SINK_ESTATE          # block 0 still open
    assert _code(c.set_ref, 0, FAKE, FAKE) == PR_SINK_ESTATE
    c.attend(0, FAKE, FAKE + 16, FAKE + 32, FAKE + 48)
    assert _code(c.bank_update, 0) == PR_SINK_ESTATE             # clean K/V missing
    c.clean_kv_write(0, FAKE, FAKE)
    assert _code(c.clean_kv_write, 0, FAKE, FAKE) == PR_SINK_ESTATE  # twice
    c.clean_kv_write(1, FAKE, FAKE)
    assert _code(c.bank_update, 1) == PR_SINK_ESTATE
    c.bank_update(0)
    c.retrieve(1, FAKE)


def test_argument_validation():
    cfg = synth.C0_TINY
    c = _dry(cfg)
    assert _code(c.set_ref, 2, FAKE, FAKE) == PR_SINK_EINVAL      # layer out of range
    assert _code(c.set_ref, -1, FAKE, FAKE) == PR_SINK_EINVAL
    assert _code(c.set_ref, 0, 0, FAKE) == PR_SINK_EINVAL         # NULL
    assert _code(c.set_ref, 0, FAKE + 8, FAKE) == PR_SINK_EINVAL  # misaligned
    for l in range(cfg.n_layers):
        c.set_ref(l, FAKE, FAKE)
    assert _code(c.retrieve, 0, FAKE + 2) == PR_SINK_EINVAL       # misaligned fingerprint
    c.retrieve(0, FAKE)
    assert _code(c.attend, 0, FAKE, FAKE + 16, FAKE + 32, FAKE) == PR_SINK_EINVAL  # out aliases q


def test_attend_noalloc_validates_like_attend_and_rejects_blocks_over_64_mib():
    """pr_sink_attend_noalloc takes the same arguments and call order as
    pr_sink_attend; a block whose rotated keys exceed the 64 MiB static scratch
    is rejected with PR_SINK_EINVAL before anything is queued."""
    cfg = synth.C0_TINY
    c = _dry(cfg)
    assert _code(c.attend_noalloc, 0, FAKE, FAKE + 16, FAKE + 32, FAKE + 48) == PR_SINK_ESTATE
    for l in range(cfg.n_layers):
        c.set_ref(l, FAKE, FAKE)
    c.retrieve(0, FAKE)
    c.attend_noalloc(0, FAKE, FAKE + 16, FAKE + 32, FAKE + 48)
    assert _code(c.attend_noalloc, 0, FAKE, FAKE + 16, FAKE + 32, FAKE) == PR_SINK_EINVAL  # out aliases q
    assert _code(c.attend_noalloc, 5, FAKE, FAKE + 16, FAKE + 32, FAKE + 48) == PR_SINK_EINVAL
    # 3 frames x 64 x 64 tokens x 64 heads x 128 dims x 2 bytes = 192 MiB of keys
    big = synth.C1_480.replace(n_layers=1, n_heads=64, lat_h=64, lat_w=64)
    c = _dry(big)
    c.set_ref(0, FAKE, FAKE)
    c.retrieve(0, FAKE)
    c.attend(0, FAKE, FAKE + 16, FAKE + 32, FAKE + 48)  # the arena-backed call has room
    assert _code(c.attend_noalloc, 0, FAKE, FAKE + 16, FAKE + 32, FAKE + 48) == PR_SINK_EINVAL
    assert "64 MiB" in binding.last_error() or "scratch" in binding.last_error()
    # the failed call left the block open and unchanged
    c.clean_kv_write(0, FAKE, FAKE)
    c.bank_update(0)


def test_segment_layout_follows_the_block_protocol():
    cfg = synth.C0_TINY.replace(t0=3)
    c = _dry(cfg)
    for l in range(cfg.n_layers):
        c.set_ref(l, FAKE, FAKE)
    tb, tr = cfg.block_tokens, cfg.ref_tokens
    expect_present = {0: [1, 0, 0, 0, 0, 1], 1: [1, 1, 0, 0, 1, 1], 2: [1, 1, 1, 1, 1, 1],
                      7: [1, 1, 1, 1, 1, 1]}
    for b in range(8):
        c.retrieve(b, FAKE)
        segs = c.segments()
        assert [s[1] for s in segs] == [3 + x for x in (0, 1, 3, 5, 7, 9)]
        if b in expect_present:
            toks = [tr] + [tb] * 5
            assert [s[0] for s in segs] == [t * p for t, p in zip(toks, expect_present[b])]
        for l in range(cfg.n_layers):
            c.clean_kv_write(l, FAKE, FAKE)
        c.bank_update(b)


def test_no_bank_means_no_dynamic_sink():
    cfg = synth.C0_TINY.replace(bank_fill_blocks=0)
    c = _dry(cfg)
    for l in range(cfg.n_layers):
        c.set_ref(l, FAKE, FAKE)
    for b in range(5):
        c.retrieve(b, FAKE)
        assert c.segments()[2][0] == 0
        for l in range(cfg.n_layers):
            c.clean_kv_write(l, FAKE, FAKE)
        c.bank_update(b)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with a message before touching a device."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_bench_counter_record_follows_the_kernel_source(tmp_path, monkeypatch):
    """bench.py reports a rocprofv3 counter record (HBM bytes, clock) only while the hash of
    the attention kernel's sources matches the one the record was taken on."""
    import json
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    from bounded_kv_cache_pr_amd import profile_summary
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    for name in profile_summary.ATTN_SOURCES:
        (csrc / name).write_bytes(f"// {name}\n".encode())
    monkeypatch.setattr(profile_summary, "CSRC", str(csrc))
    (tmp_path / "profiles").mkdir()
    rec = {"attn_sources_sha256": profile_summary.attn_source_sha256(),
           "traffic_bytes_per_launch": 409636192, "shader_clock_ghz": 1.956}
    (tmp_path / "profiles" / "attn_bf16_kernel_480x480_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_record("480x480") == rec
    assert bench.counter_record("384x672") is None          # no record for that workload
    for name in profile_summary.ATTN_SOURCES:                # any of the kernel's sources changed
        (csrc / name).write_bytes(b"// changed\n")
        assert bench.counter_record("480x480") is None
        (csrc / name).write_bytes(f"// {name}\n".encode())
    assert bench.counter_record("480x480") == rec


def test_profile_summary_roles_and_bytes(tmp_path):
    """profile_summary sorts rocprofv3 dispatches into the path's roles (a rope_follow launch
    right before attention on its queue rotates the current keys, one right after a
    slot_copy rotates a bank entry, one before the first retrieval a Ref Sink) and turns
    DRAM request counts into bytes (x 32)."""
    import csv
    from bounded_kv_cache_pr_amd import profile_summary as ps
    names = {"a": "prsink::attn_bf16_kernel<128>(prsink::AttnParams)",
             "r": "prsink::rope_follow_kernel(prsink::RotParams)",
             "k": "prsink::kv_write_kernel(...)", "q": "prsink::retrieve_kernel(...)",
             "c": "prsink::clean_write_kernel(prsink::CleanWrite)",
             "u": "prsink::bank_update_kernel(...)", "s": "prsink::slot_copy_kernel(...)"}
    # (kernel, queue): set-up, then four blocks with the clean path on queue 2
    seq = [("k", 1), ("r", 1)]
    for _ in range(4):
        seq += [("q", 1), ("r", 1), ("a", 1), ("r", 1), ("a", 1), ("c", 2), ("u", 2), ("s", 2), ("r", 2)]
    d = tmp_path / "dram"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Queue_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        t = 0
        for i, (k, q) in enumerate(seq):
            for name, val in (("TCC_EA0_RDREQ_DRAM_32B", 100 + i), ("TCC_EA0_WRREQ_WRITE_DRAM_32B", 10)):
                # counters arrive per hardware instance: two rows that add up
                w.writerow([i + 1, q, 256, names[k], name, val / 2, t, t + 1000 * (i + 1)])
                w.writerow([i + 1, q, 256, names[k], name, val / 2, t, t + 1000 * (i + 1)])
            t += 100000
    ds = ps.assign_roles(ps.load_pass(str(d)))
    roles = [x["role"] for x in ds]
    assert roles[:2] == ["kv_write_kernel", "rope_follow (Ref Sink)"]
    assert roles[3] == "rope_follow (current keys)" and roles[5] == "rope_follow (current keys)"
    assert roles[10] == "rope_follow (bank entry)" and roles[19] == "rope_follow (bank entry)"
    assert roles[7] == "clean_write (block 0, +Static)" and roles[16] == "clean_write"
    assert [x["block"] for x in ds][:3] == [-1, -1, 0] and ds[11]["block"] == 1
    assert ds[4]["ctr"]["TCC_EA0_RDREQ_DRAM_32B"] == 104
    cfg, passes, table, cal = ps.summarise(str(tmp_path), "480x480", 4)
    assert table["attn_bf16_kernel"]["dram_write"] == 320      # steady dispatches: block 3 on
    assert table["attn_bf16_kernel"]["n_dram"] == 2
    # algorithmic bytes of the current-key rotation: T rows + T table rows read, T rows written
    row = cfg.n_heads * cfg.head_dim * 2
    assert table["rope_follow (current keys)"]["alg_read"] == cfg.block_tokens * (row + 4 * cfg.head_dim)
    assert table["attn_bf16_kernel"]["alg_write"] == cfg.block_tokens * row
