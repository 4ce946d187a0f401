"""Seeded synthetic inputs for the PR-Sink hot path.

This module is the only code shared by the GPU path's tests/benchmarks and the
fp64 CPU oracle's tests.  It holds shapes and random inputs only; none of the
method's arithmetic (RoPE, attention, fingerprint normalisation, retrieval,
bank policy) lives here.

Workload shapes follow the LiveAnimate pages: blocks of 3 latent frames
(= 12 RGB frames) at the 480x480, 384x672 and 672x384 resolution buckets
(LiveAnimate review on paper.rainbus.top, reproducibility paragraph; news
article on jiazhuangai.com, limitations list).  Head count, head dim and the
RoPE band split are those of a 14B Wan-style DiT (40 heads x 128); the pages
give only "14B".  Pose fingerprints are 3 frames x 62 keypoints x (x, y, conf)
= 558 values (review, full-pipeline paragraph), with failed detections
zero-filled (review, novelty and weaknesses paragraphs).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

DTYPE_BF16 = "bf16"
DTYPE_F32 = "f32"


@dataclass(frozen=True)
class PRSinkConfig:
    """Shape of one PR-Sink cache.  Field names mirror the C struct."""

    n_layers: int
    n_heads: int
    head_dim: int
    rope_dims: tuple  # (t, h, w) band widths, each even, summing to head_dim
    rope_theta: float
    lat_h: int
    lat_w: int
    ref_frames: int
    block_frames: int
    window_slots: int = 3
    bank_size: int = 5
    bank_fill_blocks: int = 20
    fp_dim: int = 558
    dtype: str = DTYPE_BF16
    t0: int = 0
    bank_policy: int = 0          # bits: 1 zero-fingerprint fallback, 2 continual, 4 gated refresh
    bank_stale_blocks: int = 1    # continual: blocks unused before an entry may be evicted
    bank_refresh_tau: float = 0.0  # gated: refresh when the best bank dot product is below this

    @property
    def tokens_per_frame(self) -> int:
        return self.lat_h * self.lat_w

    @property
    def block_tokens(self) -> int:
        return self.block_frames * self.tokens_per_frame

    @property
    def ref_tokens(self) -> int:
        return self.ref_frames * self.tokens_per_frame

    @property
    def full_cache_keys(self) -> int:
        """Keys attended once every segment is populated (current block included)."""
        return self.ref_tokens + (self.window_slots + 2) * self.block_tokens

    def replace(self, **kw) -> "PRSinkConfig":
        return dataclasses.replace(self, **kw)


def wan_rope_dims(head_dim: int) -> tuple:
    """Band widths (t, h, w) of the 3D RoPE split used by Wan-style DiTs."""
    s = 2 * (head_dim // 6)
    return (head_dim - 2 * s, s, s)


# The five workloads.  C0 is the tiny fp32 correctness case; C1/C2 are single
# bf16 attention calls at the 480x480 and 384x672 buckets; C3/C4 are streams.
C0_TINY = PRSinkConfig(n_layers=2, n_heads=1, head_dim=64, rope_dims=wan_rope_dims(64),
                       rope_theta=1e4, lat_h=4, lat_w=4, ref_frames=1, block_frames=2,
                       dtype=DTYPE_F32)
C1_480 = PRSinkConfig(n_layers=40, n_heads=40, head_dim=128, rope_dims=wan_rope_dims(128),
                      rope_theta=1e4, lat_h=30, lat_w=30, ref_frames=1, block_frames=3)
C2_384x672 = C1_480.replace(lat_h=24, lat_w=42)
C3_STREAM_480 = C1_480
C4_STREAM_672x384 = C1_480.replace(lat_h=42, lat_w=24)

STREAM_BLOCKS = {"C3": 200, "C4": 240}
DENOISE_STEPS = 3  # attention calls per layer per block (review, full-pipeline paragraph)


# ----------------------------------------------------------------------------
# bf16 input rounding (round-to-nearest-even), applied before either side sees
# the values, so GPU and oracle consume identical numbers.
# ----------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) & 0xFFFFFFFF for k in key])


def normal_tokens(n_tokens: int, cfg: PRSinkConfig, scale: float, *key) -> np.ndarray:
    """[n_tokens][H][d] float32 ~ scale*N(0,1), rounded to bf16 for bf16 configs."""
    x = (_rng(*key).standard_normal((n_tokens, cfg.n_heads, cfg.head_dim)) * scale)
    x = x.astype(np.float32)
    return round_to_bf16(x) if cfg.dtype == DTYPE_BF16 else x


# Stream tags keep the input families apart.
TAG_Q, TAG_KCUR, TAG_VCUR, TAG_KCLEAN, TAG_VCLEAN, TAG_KREF, TAG_VREF = range(1, 8)


def ref_kv(cfg: PRSinkConfig, layer: int, seed: int):
    n = cfg.ref_tokens
    return (normal_tokens(n, cfg, 0.5, seed, TAG_KREF, layer),
            normal_tokens(n, cfg, 0.5, seed, TAG_VREF, layer))


def clean_kv(cfg: PRSinkConfig, block: int, layer: int, seed: int):
    """Raw (pre-RoPE) clean K and V of one block and layer."""
    n = cfg.block_tokens
    return (normal_tokens(n, cfg, 0.5, seed, TAG_KCLEAN, block, layer),
            normal_tokens(n, cfg, 0.5, seed, TAG_VCLEAN, block, layer))


def step_qkv(cfg: PRSinkConfig, block: int, step: int, layer: int, seed: int):
    """Raw Q, K, V of the current (noisy) block at one denoise step and layer."""
    n = cfg.block_tokens
    return (normal_tokens(n, cfg, 1.0, seed, TAG_Q, block, step, layer),
            normal_tokens(n, cfg, 0.5, seed, TAG_KCUR, block, step, layer),
            normal_tokens(n, cfg, 0.5, seed, TAG_VCUR, block, step, layer))


# Device-side generation of the same families for the full-size workloads
# (hundreds of MB per block).  Each (family, block, step, layer) key seeds its
# own torch generator; bf16 conversion is round-to-nearest-even.
def _seed64(key) -> int:
    return int(np.random.SeedSequence([int(k) & 0xFFFFFFFF for k in key]).generate_state(1, np.uint64)[0] >> 1)


def normal_tokens_torch(n_tokens: int, cfg: PRSinkConfig, scale: float, device, *key):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(_seed64(key))
    x = torch.randn((n_tokens, cfg.n_heads, cfg.head_dim), generator=g, device=device,
                    dtype=torch.float32) * scale
    return x.to(torch.bfloat16 if cfg.dtype == DTYPE_BF16 else torch.float32)


def ref_kv_torch(cfg: PRSinkConfig, layer: int, seed: int, device):
    n = cfg.ref_tokens
    return (normal_tokens_torch(n, cfg, 0.5, device, seed, TAG_KREF, layer),
            normal_tokens_torch(n, cfg, 0.5, device, seed, TAG_VREF, layer))


def clean_kv_torch(cfg: PRSinkConfig, block: int, layer: int, seed: int, device):
    n = cfg.block_tokens
    return (normal_tokens_torch(n, cfg, 0.5, device, seed, TAG_KCLEAN, block, layer),
            normal_tokens_torch(n, cfg, 0.5, device, seed, TAG_VCLEAN, block, layer))


def step_qkv_torch(cfg: PRSinkConfig, block: int, step: int, layer: int, seed: int, device):
    n = cfg.block_tokens
    return (normal_tokens_torch(n, cfg, 1.0, device, seed, TAG_Q, block, step, layer),
            normal_tokens_torch(n, cfg, 0.5, device, seed, TAG_KCUR, block, step, layer),
            normal_tokens_torch(n, cfg, 0.5, device, seed, TAG_VCUR, block, step, layer))


# ----------------------------------------------------------------------------
# Pose fingerprints: raw 558-vectors, [3 frames][62 keypoints][x, y, conf].
# ----------------------------------------------------------------------------
N_KPTS = 62
N_FRAMES_FP = 3


def _prototypes(rng: np.random.Generator, n_protos: int) -> np.ndarray:
    xy = rng.uniform(0.0, 1.0, size=(n_protos, N_KPTS, 2))
    conf = rng.uniform(0.6, 1.0, size=(n_protos, N_KPTS, 1))
    return np.concatenate([xy, conf], axis=-1)  # [P][62][3]


def _walk(rng: np.random.Generator, n_blocks: int, n_protos: int) -> np.ndarray:
    idx = np.empty(n_blocks, dtype=np.int64)
    cur = int(rng.integers(n_protos))
    for b in range(n_blocks):
        idx[b] = cur
        u = rng.uniform()
        if u >= 0.5:
            cur = (cur + (1 if u < 0.75 else -1)) % n_protos
    return idx


def _motif_walk(rng: np.random.Generator, n_blocks: int, n_protos: int,
                n_motifs: int = 4, motif_len: int = 6) -> np.ndarray:
    motifs = [rng.integers(n_protos, size=motif_len) for _ in range(n_motifs)]
    out = []
    cur = int(rng.integers(n_protos))
    while len(out) < n_blocks:
        out.extend(int(i) for i in motifs[int(rng.integers(n_motifs))])
        cur = out[-1]
        for _ in range(int(rng.integers(0, 5))):
            u = rng.uniform()
            if u >= 0.5:
                cur = (cur + (1 if u < 0.75 else -1)) % n_protos
            out.append(cur)
    return np.asarray(out[:n_blocks], dtype=np.int64)


def pose_stream(n_blocks: int, n_protos: int = 8, seed: int = 3, motifs: bool = False,
                noise: float = 0.05, p_fail: float = 0.10) -> np.ndarray:
    """float32 [n_blocks][558] raw fingerprints from a prototype random walk."""
    rng = np.random.default_rng(seed)
    protos = _prototypes(rng, n_protos)
    walk = _motif_walk(rng, n_blocks, n_protos) if motifs else _walk(rng, n_blocks, n_protos)
    fps = np.empty((n_blocks, N_FRAMES_FP, N_KPTS, 3), dtype=np.float64)
    for b in range(n_blocks):
        for f in range(N_FRAMES_FP):
            fr = protos[walk[b]] + rng.normal(0.0, noise, size=(N_KPTS, 3))
            fr[:, 2] = np.clip(fr[:, 2], 0.0, 1.0)
            if rng.uniform() < p_fail:
                fr[:] = 0.0
            fps[b, f] = fr
    return fps.reshape(n_blocks, -1).astype(np.float32)
