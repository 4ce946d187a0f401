"""pr_sink_attend_noalloc against pr_sink_attend, through the C ABI.

The allocation-free entry point keeps the current block's rotated keys in the
library's static device scratch and runs every attention job whole.  Two calls
in a row on one GPU share that scratch, the second on a smaller cache: each
output must match the regular entry point's (bitwise where the regular call
also runs every job whole, to the bf16 bounds where it splits jobs), and each
must match the oracle: whole heads of the large call, the whole small one.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from bounded_kv_cache_pr_amd import binding, synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = torch.device("cuda:0")
BF16_REL, BF16_ABS = 1e-2, 3e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def drive(cfg, seed, n_blocks):
    """A cache with Ref, Static, a Dynamic entry and a full window, block n_blocks open."""
    cache = binding.PRSinkCache(cfg, device=DEV)
    for l in range(cfg.n_layers):
        cache.set_ref(l, *synth.ref_kv_torch(cfg, l, seed, DEV))
    fps = synth.pose_stream(n_blocks + 1, seed=seed)
    for b in range(n_blocks):
        cache.retrieve(b, torch.from_numpy(fps[b]).to(DEV))
        for l in range(cfg.n_layers):
            cache.clean_kv_write(l, *synth.clean_kv_torch(cfg, b, l, seed, DEV))
        cache.bank_update(b)
    cache.retrieve(n_blocks, torch.from_numpy(fps[n_blocks]).to(DEV))
    return cache, fps


def test_noalloc_matches_attend_two_calls_second_smaller():
    big = synth.C1_480.replace(n_layers=1)                      # 2700 tokens x 40 heads: jobs run whole
    small = synth.C1_480.replace(n_layers=1, n_heads=4, lat_h=10, lat_w=10)  # 300 tokens: regular call splits
    seed, b = 11, 6
    for name, cfg in (("480x480", big), ("small", small)):
        log(f"case: noalloc vs attend, {name}, block {b}")
        cache, fps = drive(cfg, seed, b)
        q, kc, vc = synth.step_qkv_torch(cfg, b, 0, 0, seed, DEV)
        ref_out = cache.attend(0, q, kc, vc)
        out = torch.full_like(q, float("nan"))
        cache.attend_noalloc(0, q, kc, vc, out)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        got, want = out.float().cpu().numpy(), ref_out.float().cpu().numpy()
        err, mx = rel_l2(got, want), float(np.abs(got - want).max())
        log(f"{name}: noalloc vs attend rel-L2 {err:.3g} max-abs {mx:.3g}, bitwise {torch.equal(out, ref_out)}")
        if name == "480x480":
            assert torch.equal(out, ref_out)
        assert err <= BF16_REL and mx <= BF16_ABS
        # against the oracle: heads from both ends of the large call, the small one whole
        heads = [0, 7, 24, 39] if name == "480x480" else list(range(cfg.n_heads))
        orc = O.PRSinkOracle(cfg)
        for blk in range(b):
            orc.open_block(blk, fps[blk])
            orc.close_block(blk)
        orc.open_block(b, fps[b])
        host = lambda t: t.float().cpu().numpy()
        ref = orc.attend(host(q), host(kc), host(vc),
                         tuple(host(x) for x in synth.ref_kv_torch(cfg, 0, seed, DEV)),
                         lambda bid: tuple(host(x) for x in synth.clean_kv_torch(cfg, bid, 0, seed, DEV)),
                         heads=heads)
        sub = got[:, heads]
        e2, m2 = rel_l2(sub, ref), float(np.abs(sub - ref).max())
        log(f"{name}: noalloc vs oracle, heads {heads if len(heads) < 8 else 'all'}: rel-L2 {e2:.3g} max-abs {m2:.3g}")
        assert e2 <= BF16_REL and m2 <= BF16_ABS
        cache.close()
