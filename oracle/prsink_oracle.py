"""Plain fp64 CPU oracle of the PR-Sink hot path (LiveAnimate).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library or its Python binding, and it is never a fallback for it.

Everything here is written from the method's description on the pages and
follows their order:

* Block-causal attention over the bounded cache: the current block's queries
  attend, with scale 1/sqrt(d), over the Ref Sink, the cached history and the
  current block itself (LiveAnimate review on paper.rainbus.top, full-pipeline
  paragraph, attention formula and the prose next to it).
* The cache holds a Static Sink (first generated block, kept for good), one
  Dynamic Sink block recalled by pose retrieval, and a 3-slot rolling window
  made of the current block and the two before it (HF papers abstract;
  papers.ananclaw.com explainer, section "Pose-Retrieval Sink Attention";
  jiazhuangai.com article, section "three key breakthroughs").
* Keys are cached before RoPE and rotated at their current cache position on
  every attention call ("RoPE follow"; review, full-pipeline paragraph, and the
  novelty paragraph on position-consistent reuse).
* Pose fingerprint: 3 frames x 62 keypoints x 3 channels = 558 values,
  l2-normalised; retrieval is the argmax of the dot product over the memory
  bank, leaving out block b-1 (review, full-pipeline paragraph; novelty
  paragraph: cosine-similarity maximisation).
* Memory bank: M = 5 entries written over the first 20 blocks, then frozen
  (review, weaknesses and reproducibility paragraphs); replacement is an
  exhaustive search that minimises the mean in-bank similarity (review,
  novelty paragraph).
* Clean KV Update writes the clean K/V of the finished block into the rolling
  window (review, full-pipeline paragraph).

Readings where the pages are silent (all listed in the design notes):
segment temporal positions are fixed by slot order and start at ``t0``; empty
segments are skipped without shifting the others; the 3D RoPE splits head_dim
into (t, h, w) bands of adjacent pairs with frequency theta^(-2i/D_band); an
all-zero fingerprint normalises to zero; argmax ties go to the lowest bank
slot; "keep the bank unchanged" is one of the replacement options, evaluated
first, and a swap wins only on a strict decrease; the bank stores the clean
K/V of the block together with its driving fingerprint; every squared norm and
dot product of the fingerprint arithmetic is the plain sum of the rounded
products in index order (``seq_dot``), which fixes its bits.

Parity unpinned: the RoPE band split / pairing / frequency convention and the
Ref Sink's temporal slot are this oracle's reading; the pages fix neither.
They are pinned only to that stated reading (closed forms) and to invariants.

Bank-policy variants (review, weaknesses paragraph: the frozen M = 5 bank is
fragile; directions: continual writes with decaying weights, a bank refresh
gated by fingerprint distance, and, when pose detection fails, falling back to
the Static Sink + window).  The pages name the directions only; the readings,
each off by default (policy 0 is the method as described):

* ZERO_FALLBACK: a block whose fingerprint is all zero (every frame failed)
  attends no Dynamic Sink and is never written into the bank.
* CONTINUAL: an entry's weight halves every K = bank_stale_blocks blocks since
  it was last written or retrieved; after the fill phase the exhaustive
  replacement keeps running, but may only evict entries whose weight has
  reached 1/2 (unused for at least K blocks).
* GATED: after the fill phase, a block whose best dot product with the bank
  (all entries) is below tau = bank_refresh_tau triggers the full exhaustive
  replacement.
Insertion: while the bank has room, an update inserts into the next slot.
"""
from __future__ import annotations

import math

import numpy as np

SEG_REF, SEG_STATIC, SEG_DYNAMIC, SEG_WINDOW, SEG_CURRENT = (
    "ref", "static", "dynamic", "window", "current")

# bank-policy bits
POLICY_ZERO_FALLBACK, POLICY_CONTINUAL, POLICY_GATED = 1, 2, 4


# ----------------------------------------------------------------------------
# 3D rotary position embedding
# ----------------------------------------------------------------------------
def rope_frequencies(band_dim: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/D) for the D/2 pairs of one band."""
    i = np.arange(band_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / band_dim)


def rope_rotate(x: np.ndarray, pos: np.ndarray, rope_dims, theta: float) -> np.ndarray:
    """Rotate the feature pairs of ``x`` by their token's (t, h, w) angles.

    x:   [n, ..., d]  (any middle axes, e.g. heads)
    pos: [n, 3]       integer (t, h, w) position of each token
    Band a covers dims [o_a, o_a + D_a); pair i of it is (o_a+2i, o_a+2i+1) and
    turns by angle pos_a * omega_i, counter-clockwise.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    out = x.copy()
    extra = (1,) * (x.ndim - 2)
    off = 0
    for a, band in enumerate(rope_dims):
        ang = pos[:, a][:, None] * rope_frequencies(band, theta)[None, :]  # [n, D/2]
        c = np.cos(ang).reshape((ang.shape[0],) + extra + (ang.shape[1],))
        s = np.sin(ang).reshape(c.shape)
        x0 = x[..., off:off + band:2]
        x1 = x[..., off + 1:off + band:2]
        out[..., off:off + band:2] = x0 * c - x1 * s
        out[..., off + 1:off + band:2] = x0 * s + x1 * c
        off += band
    if off != x.shape[-1]:
        raise ValueError("rope band widths must sum to the head dim")
    return out


def frame_positions(n_frames: int, t_start: int, lat_h: int, lat_w: int) -> np.ndarray:
    """(t, h, w) of every token of ``n_frames`` latent frames, frame-major then row-major."""
    f, y, x = np.meshgrid(np.arange(n_frames), np.arange(lat_h), np.arange(lat_w),
                          indexing="ij")
    return np.stack([t_start + f.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.int64)


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              return_probs: bool = False):
    """softmax(Q K^T * scale) V per head.  q [Tq][H][d], k [Tk][H][d], v [Tk][H][dv]."""
    qh = np.asarray(q, np.float64).transpose(1, 0, 2)
    kh = np.asarray(k, np.float64).transpose(1, 0, 2)
    vh = np.asarray(v, np.float64).transpose(1, 0, 2)
    s = np.matmul(qh, kh.transpose(0, 2, 1)) * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    o = np.matmul(p, vh).transpose(1, 0, 2)
    return (o, p) if return_probs else o


# ----------------------------------------------------------------------------
# Fingerprint, retrieval and the diversity bank
# ----------------------------------------------------------------------------
def seq_dot(a, b) -> float:
    """sum_k a[k] * b[k] as written: k = 0, 1, 2, ... in order, every product and
    every partial sum rounded to fp64 (Python floats: no fused multiply-add, no
    pairwise or blocked summation).  Used for the squared norm of a fingerprint
    and for every fingerprint dot product, so that the result has one definition
    and any other implementation that adds in index order reproduces it bit for
    bit (review, full-pipeline paragraph: l2-normalised fingerprints compared by
    dot product)."""
    s = 0.0
    for x, y in zip(np.asarray(a, np.float64).ravel().tolist(),
                    np.asarray(b, np.float64).ravel().tolist()):
        s += x * y
    return s


def fingerprint(x_raw: np.ndarray) -> np.ndarray:
    """phi = x / ||x||_2 in fp64, ||x||_2 = sqrt of the index-order sum of x_k^2
    (correctly rounded square root, then one correctly rounded division per
    element); an all-zero fingerprint stays zero."""
    x = np.asarray(x_raw, dtype=np.float64).ravel()
    n = math.sqrt(seq_dot(x, x))
    return x / n if n > 0.0 else np.zeros_like(x)


def retrieval_scores(phi_b: np.ndarray, bank_phi) -> np.ndarray:
    """phi_b . phi_i for every bank entry, each an index-order sum."""
    return np.array([seq_dot(phi_b, p) for p in bank_phi], dtype=np.float64)


def retrieve(phi_b: np.ndarray, bank_ids, bank_phi, block: int):
    """r(b) = argmax_i phi_b . phi_i over bank entries whose block id is not b-1.

    Returns the bank slot, or None if no entry is eligible.  Ties go to the
    lowest slot.
    """
    best, best_s = None, -math.inf
    scores = retrieval_scores(phi_b, bank_phi)
    for slot, bid in enumerate(bank_ids):
        if bid == block - 1:
            continue
        if best is None or scores[slot] > best_s:
            best, best_s = slot, scores[slot]
    return best


def mean_pairwise_similarity(phis) -> float:
    """Mean of phi_i . phi_j over unordered pairs i < j, in slot order."""
    n = len(phis)
    tot, cnt = 0.0, 0
    for i in range(n):
        for j in range(i + 1, n):
            tot += seq_dot(phis[i], phis[j])
            cnt += 1
    return tot / cnt


def bank_decision(bank_phi, phi_b: np.ndarray, bank_size: int, evictable=None):
    """Diversity update of a bank that is being written.

    Returns ("insert", slot) while the bank has room, else ("keep", None) or
    ("swap", j): the option among [keep, swap 0, ..., swap M-1] with the
    smallest mean in-bank similarity, the first one winning ties.  With
    ``evictable`` (one flag per entry) only those entries may be swapped out.
    """
    if len(bank_phi) < bank_size:
        return ("insert", len(bank_phi))
    best, best_s = ("keep", None), mean_pairwise_similarity(bank_phi)
    for j in range(len(bank_phi)):
        if evictable is not None and not evictable[j]:
            continue
        cand = list(bank_phi)
        cand[j] = phi_b
        s = mean_pairwise_similarity(cand)
        if s < best_s:
            best, best_s = ("swap", j), s
    return best


# ----------------------------------------------------------------------------
# The bounded cache, tracked by block id
# ----------------------------------------------------------------------------
class PRSinkOracle:
    """Stream-level oracle.

    The cache is tracked by *which block's clean K/V* sits in each segment;
    the caller supplies the raw tensors on demand, so long streams need no
    fp64 copy of the whole cache.  Per block: ``open_block`` (fingerprint +
    retrieval), any number of ``attend`` calls, then ``close_block`` (clean
    write into the window, and the bank update while b < bank_fill_blocks).
    """

    def __init__(self, cfg):
        self.cfg = cfg
        self.next_block = 0
        self.is_open = False
        self.window = []          # ids of the closed blocks still in the window, oldest first
        self.static_id = None
        self.dynamic_id = None
        self.bank_ids = []
        self.bank_phi = []
        self.bank_last_used = []  # block at which each entry was last written or retrieved
        self.best_score = -math.inf  # the open block's best dot product with the bank
        self.phi_cur = None
        self.last_r = None
        self.last_decision = None

    # -- layout ------------------------------------------------------------
    def segment_layout(self):
        """Segments of the current block, in cache order.

        Each entry: (kind, block_id, t_start, n_frames, present).  Temporal
        starts are fixed by slot: Ref, Static, Dynamic, the W-1 previous window
        blocks (oldest first), then the current block, each one after the
        other from t0; an empty segment keeps its positions reserved.
        """
        c = self.cfg
        fr, fb = c.ref_frames, c.block_frames
        t = c.t0
        segs = [(SEG_REF, None, t, fr, True)]
        t += fr
        segs.append((SEG_STATIC, self.static_id, t, fb, self.static_id is not None))
        t += fb
        segs.append((SEG_DYNAMIC, self.dynamic_id, t, fb, self.dynamic_id is not None))
        t += fb
        n_prev = c.window_slots - 1
        prev = [self.current_block - n_prev + j for j in range(n_prev)]
        for pid in prev:
            segs.append((SEG_WINDOW, pid, t, fb, pid >= 0))
            t += fb
        segs.append((SEG_CURRENT, self.current_block, t, fb, True))
        return segs

    @property
    def current_block(self) -> int:
        if not self.is_open:
            raise RuntimeError("no block is open")
        return self.next_block

    # -- block open: fingerprint + retrieval --------------------------------
    def open_block(self, block: int, fp_raw: np.ndarray):
        if self.is_open or block != self.next_block:
            raise RuntimeError("blocks must be opened in order, one at a time")
        self.phi_cur = fingerprint(fp_raw)
        policy = getattr(self.cfg, "bank_policy", 0)
        scores = retrieval_scores(self.phi_cur, self.bank_phi)
        self.best_score = float(scores.max()) if len(scores) else -math.inf
        if policy & POLICY_ZERO_FALLBACK and not np.any(self.phi_cur):
            r = None  # no pose detected: Static Sink + window only
        else:
            r = retrieve(self.phi_cur, self.bank_ids, self.bank_phi, block)
        if r is None:
            self.dynamic_id = None
        else:
            self.dynamic_id = self.bank_ids[r]
            self.bank_last_used[r] = block
        self.last_r = r
        self.is_open = True
        return r

    # -- attention ------------------------------------------------------------
    def assemble(self, k_cur, v_cur, ref_kv, block_kv, heads=None):
        """Raw keys, values and their (t, h, w) positions in cache order.

        ``heads`` optionally keeps a subset of heads (sampled checks at full size).
        """
        c = self.cfg
        sel = (lambda x: np.asarray(x)[:, heads]) if heads is not None else np.asarray
        ks, vs, ps = [], [], []
        for kind, bid, t0, nf, present in self.segment_layout():
            if not present:
                continue
            if kind == SEG_REF:
                k, v = ref_kv
            elif kind == SEG_CURRENT:
                k, v = k_cur, v_cur
            else:
                k, v = block_kv(bid)
            ks.append(np.asarray(sel(k), np.float64))
            vs.append(np.asarray(sel(v), np.float64))
            ps.append(frame_positions(nf, t0, c.lat_h, c.lat_w))
        return np.concatenate(ks), np.concatenate(vs), np.concatenate(ps)

    def query_positions(self):
        c = self.cfg
        kind, _, t0, nf, _ = self.segment_layout()[-1]
        assert kind == SEG_CURRENT
        return frame_positions(nf, t0, c.lat_h, c.lat_w)

    def attend(self, q, k_cur, v_cur, ref_kv, block_kv, q_rows=None, heads=None):
        """Attention output of the current block for one layer and step.

        ref_kv:   (k, v) raw Ref Sink tensors of this layer
        block_kv: callable block_id -> (k, v) raw clean tensors of this layer
        q_rows / heads: optional subsets (sampled checks at full size)
        """
        c = self.cfg
        k, v, kpos = self.assemble(k_cur, v_cur, ref_kv, block_kv, heads)
        qpos = self.query_positions()
        q = np.asarray(q, np.float64)
        if q_rows is not None:
            q, qpos = q[q_rows], qpos[q_rows]
        if heads is not None:
            q = q[:, heads]
        qr = rope_rotate(q, qpos, c.rope_dims, c.rope_theta)
        kr = rope_rotate(k, kpos, c.rope_dims, c.rope_theta)
        return attention(qr, kr, v, 1.0 / math.sqrt(c.head_dim))

    # -- block close: clean write + bank update ---------------------------------
    def close_block(self, block: int):
        if not self.is_open or block != self.next_block:
            raise RuntimeError("close the open block")
        c = self.cfg
        self.window.append(block)
        self.window = self.window[-c.window_slots:]
        if block == 0:
            self.static_id = 0
        self.last_decision = None
        policy = getattr(c, "bank_policy", 0)
        filling = block < c.bank_fill_blocks
        if filling or policy & (POLICY_CONTINUAL | POLICY_GATED):
            if policy & POLICY_ZERO_FALLBACK and not np.any(self.phi_cur):
                kind, slot = "keep", None  # an undetected pose is never written
            elif filling or (policy & POLICY_GATED and self.best_score < c.bank_refresh_tau):
                kind, slot = bank_decision(self.bank_phi, self.phi_cur, c.bank_size)
            else:  # continual writes: only entries unused for K blocks may go
                K = c.bank_stale_blocks
                stale = [block - t >= K for t in self.bank_last_used] if policy & POLICY_CONTINUAL \
                    else [False] * len(self.bank_phi)
                kind, slot = bank_decision(self.bank_phi, self.phi_cur, c.bank_size, stale)
            if kind == "insert":
                self.bank_ids.append(block)
                self.bank_phi.append(self.phi_cur.copy())
                self.bank_last_used.append(block)
            elif kind == "swap":
                self.bank_ids[slot] = block
                self.bank_phi[slot] = self.phi_cur.copy()
                self.bank_last_used[slot] = block
            self.last_decision = (kind, slot)
        self.is_open = False
        self.next_block = block + 1
        return self.last_decision
