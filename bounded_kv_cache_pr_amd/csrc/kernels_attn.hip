// PR-Sink block-causal attention on gfx950.
//
// The current block's queries attend over [Ref; Static; Dynamic; window;
// current] with scale 1/sqrt(d) (LiveAnimate review on paper.rainbus.top,
// full-pipeline paragraph: the attention formula and the prose around it,
// which includes the current block).  Keys arrive already rotated at their
// segment's current position (RoPE follow runs when a block takes a place in
// the cache, in rope_follow); the queries are rotated here, at the current
// block's positions.
//
// bf16 kernel, one workgroup = 256 query rows of one head, 4 waves x 64 rows:
//   * S'^T = K_rot Q'^T on v_mfma_f32_32x32x16_bf16, with
//     Q' = bf16(Q_rot * log2(e) / sqrt(d)), so scores come out in base 2.  A
//     lane owns one query column and 16 key rows of each 32x32 block, so the
//     softmax needs no shuffles except one exchange with lane ^ 32.  Keys sit
//     in LDS with bits 2 and 3 of their row index swapped: the probabilities
//     a lane holds after QK^T are then exactly the B operand of the PV MFMA.
//   * O^T = V^T P^T accumulates in fp32.  V stays row-major in LDS; the V^T
//     operand comes from ds_read_b64_tr_b16.
//   * Softmax against a fixed reference: the first 64-key tile sets each row's
//     max m; every later score is accumulated as 2^(s' - m), with -m folded
//     into the accumulator the QK^T MFMA starts from.  Probabilities above 1
//     are harmless in fp32; if a row's sum ever leaves [0, 2^64] (a score more
//     than 64 powers of two above the first tile's max) the workgroup redoes
//     the whole row block with exact online softmax.
//   * Tiles move global -> LDS by DMA (buffer_load ... lds) into a 3-stage
//     ring, two tiles ahead.  Iteration j computes QK^T of tile j+1 and PV of
//     tile j, so the exp2 of one tile overlaps the MFMAs of its neighbours.
//   * Ragged tiles (the last of each segment) run afterwards through the exact
//     online-softmax step with masking; tile order does not change the result.
// The fp32 kernel is a plain one-query-per-lane loop for fp32 caches.
#include "prsink_device.h"

#include <type_traits>

namespace prsink {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;


// Fourth dword of a gfx9 raw buffer resource (32-bit data format).
constexpr int kBufferConfig = 0x00020000;
// A buffer offset beyond every range the kernels build (ranges stay < 2^31).
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ inline uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Row r of a 64-row key tile lives at LDS row key_perm(r): bits 2 and 3 swapped.
__device__ inline int key_perm(int r) { return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1); }

// XCD-aware work order: consecutive workgroup ids land on different XCDs
// (xcd = id % 8), and XCD x takes the heads h = x (mod 8), so the query tiles
// of a head share that XCD's L2 while they stream the same keys.  On each
// XCD, job jx (head x + 8 (jx / n_qtiles), query tile jx % n_qtiles): the
// first full_jobs run whole; the next tail_jobs run as `split` pieces each,
// piece-major, so the pieces running side by side cover the same key range.
struct Work {
  int head, qt, piece, n_pieces, job;  // job: index among the XCD-major split jobs
};
__device__ inline bool map_work(const AttnParams& p, Work& w) {
  const int wg = blockIdx.x;
  const int xcd = wg & 7, k = wg >> 3;
  int jx;
  if (k < p.full_jobs) {
    jx = k;
    w.piece = 0;
    w.n_pieces = 1;
    w.job = -1;
  } else {
    const int kk = k - p.full_jobs;
    const int jt = kk % p.tail_jobs;
    jx = p.full_jobs + jt;
    w.piece = kk / p.tail_jobs;
    w.n_pieces = p.split;
    w.job = xcd * p.tail_jobs + jt;
  }
  // uniform per workgroup; the divisions above run on the VALU, so pin the
  // results to SGPRs (buffer resources built from them must be scalar)
  w.head = __builtin_amdgcn_readfirstlane(xcd + 8 * (jx / p.n_qtiles));
  w.qt = __builtin_amdgcn_readfirstlane(jx % p.n_qtiles);
  w.piece = __builtin_amdgcn_readfirstlane(w.piece);
  w.job = __builtin_amdgcn_readfirstlane(w.job);
  return w.head < p.n_heads;
}

__device__ inline uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// 16 bytes per lane from a buffer resource into LDS: lane i writes
// M0 + 16 i; the global offset is voff + soff.  The load is invisible to the
// compiler's counters; callers wait on vmcnt themselves.  M0 is saved and
// restored around it, and the LDS DMA issues one wait state after the M0
// write (the gfx9 M0 -> LDS-DMA hazard).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff,
                                      uint32_t soff = 0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(r), "s"(soff)
      : "memory");
}

// The same inside a run of DMAs, with M0 = base + OFF set by one scalar add.
// The run's first DMA (save) keeps M0 in `saved`, its last (restore) puts it
// back; nothing between them reads M0.
template <int OFF>
__device__ __forceinline__ void dma16_imm(__amdgpu_buffer_rsrc_t r, uint32_t base, uint32_t voff,
                                          uint32_t soff) {
  asm volatile(
      "s_add_u32 m0, %0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(base), "v"(voff), "s"(r), "s"(soff), "i"(OFF)
      : "memory", "scc");
}
// k selects OFF = 4096 k (k is a constant once the caller's loop is unrolled).
__device__ __forceinline__ void dma16_run(__amdgpu_buffer_rsrc_t r, uint32_t base, int k, uint32_t voff,
                                          uint32_t soff, bool save, bool restore, uint32_t& saved) {
  if (save) asm volatile("s_mov_b32 %0, m0" : "=s"(saved));
  switch (k) {
    case 0: dma16_imm<0>(r, base, voff, soff); break;
    case 1: dma16_imm<4096>(r, base, voff, soff); break;
    case 2: dma16_imm<8192>(r, base, voff, soff); break;
    case 3: dma16_imm<12288>(r, base, voff, soff); break;
    case 4: dma16_imm<16384>(r, base, voff, soff); break;
    case 5: dma16_imm<20480>(r, base, voff, soff); break;
    case 6: dma16_imm<24576>(r, base, voff, soff); break;
    default: dma16_imm<28672>(r, base, voff, soff); break;
  }
  if (restore) asm volatile("s_mov_b32 m0, %0" : : "s"(saved));
}

// The same load as a compiler builtin, and its per-lane-address form (a
// gather), for the prologue and the packed tiles: the compiler sets M0, keeps
// the wait state after it, and counts the loads in its own vmcnt bookkeeping.
__device__ __forceinline__ void dma16_b(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, voff,
                                           soff, 0, 0);
}
__device__ __forceinline__ void dma16_flat_b(const void* gaddr, uint32_t lds) {
  __builtin_amdgcn_global_load_lds(gaddr, (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, 0, 0);
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x3f70 | (N & 15) | ((N >> 4) << 14));
}

// QK^T MFMAs of the steady-state loop, with the scores accumulating in VGPRs
// and the query operand read from AGPRs.  (The compiler gives every MFMA of a
// function one register form; the PV MFMAs keep O in AGPRs, and a VALU read
// of an AGPR next to running MFMAs costs several cycles, so the scores the
// softmax reads live in VGPRs.)  The loop reads a score no sooner than nine
// steps (18 MFMAs) after the MFMA that wrote it, well past the wait states an
// MFMA result needs before a VALU read; the accumulating MFMA has its source
// C tied to its destination, the case the hardware chains back to back.
__device__ __forceinline__ f32x16 mfma_qk_first(bf16x8 a, bf16x8 b, const f32x16& c) {
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
  return d;
}
__device__ __forceinline__ void mfma_qk_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// Walks the full 64-key tiles of one head, for K or V, in segment order: a
// buffer resource per segment whose range is this head's rows of the segment,
// and the byte offset of the next tile in it (the DMA's scalar offset).
// Moving to the next segment (the only scalar loads) happens a handful of
// times per workgroup.  Past the last tile the cursor stays on it, so loads
// issued beyond the end re-read real data into stages nobody reads.
struct SegCursor {
  __amdgpu_buffer_rsrc_t r;
  uint32_t off, step;
  int left, s;
  int dyn_r;  // bank entry of the Dynamic Sink (load_dyn_r)
  __device__ __forceinline__ void seek(const AttnParams& p, size_t head_off, uint32_t tok_bytes,
                                       uint32_t tile_bytes, bool is_k) {
    while (s < p.n_seg && seg_count(p, s, dyn_r) < kKeyTile) ++s;
    if (s < p.n_seg) {
      const char* base = seg_base(p, s, is_k, dyn_r) + head_off;
      const int nrec = (int)((size_t)seg_count(p, s, dyn_r) * tok_bytes - head_off);
      r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, nrec, 0x00020000);
      off = 0;
      step = tile_bytes;
      left = seg_count(p, s, dyn_r) / kKeyTile;
    } else {  // past the last tile: back onto it, and stay
      off -= step;
      step = 0;
      left = 1 << 30;
    }
  }
  // Full tile `start` of the head (counting across segments); the caller
  // guarantees it exists.
  __device__ __forceinline__ void first(const AttnParams& p, size_t head_off, uint32_t tok_bytes,
                                        uint32_t tile_bytes, bool is_k, int start, int dyn) {
    dyn_r = dyn;
    // the segment holding tile `start`, by an unrolled scan of every slot
    int acc = 0, sel = -1, skip = 0;
#pragma unroll
    for (int i = 0; i < kMaxSegments; ++i) {
      const int n = seg_count(p, i, dyn_r) / kKeyTile;
      if (sel < 0 && start < acc + n) {
        sel = i;
        skip = start - acc;
      }
      acc += n;
    }
    s = __builtin_amdgcn_readfirstlane(sel);  // uniform: keep the resource in SGPRs
    start = __builtin_amdgcn_readfirstlane(skip);
    off = step = 0;
    seek(p, head_off, tok_bytes, tile_bytes, is_k);
    off = (uint32_t)start * tile_bytes;
    left -= start;
  }
  __device__ __forceinline__ void next(const AttnParams& p, size_t head_off, uint32_t tok_bytes,
                                       uint32_t tile_bytes, bool is_k) {
    off += step;
    if (__builtin_expect(--left == 0, 0)) {
      ++s;
      seek(p, head_off, tok_bytes, tile_bytes, is_k);
    }
  }
};


template <int D>
struct Attn {
  static constexpr int KT = kKeyTile;    // keys per tile
  static constexpr int QT = 256;         // query rows per workgroup
  static constexpr int RB = D * 2;       // bytes per key row
  static constexpr int NS = RB / 16;     // 16-byte data units per row
  // Padded LDS row stride: 16 consecutive rows start 12 (d=128) or 36 (d=64)
  // banks apart, so the 16-byte operand reads of a 16-lane phase cover all 64
  // banks once.
  static constexpr int RBP = D == 128 ? RB + 48 : RB + 16;
  static constexpr int NU = RBP / 16;    // 16-byte units per padded row
  static constexpr int UNITS = KT * NU;  // 16-byte units of one LDS tile
  static constexpr int NDMA = (UNITS + 255) / 256;  // DMA instructions per wave, tile and tensor
  static constexpr int NBLK = UNITS / 64;           // 64-unit blocks of a tile (one DMA each)
  static constexpr int TILE = KT * RBP;  // bytes per tile buffer
  static constexpr int STAGES = 3;
  // K stages, V stages, the packed ragged K and V tile, DMA sink
  static constexpr int LDS_BYTES = 2 * STAGES * TILE + 2 * TILE + 1024;
  static_assert(UNITS % 64 == 0, "a DMA instruction never straddles the end of a tile");
  static_assert(4 * (NDMA - 1) >= NBLK - 4 && 4 * NDMA >= NBLK,
                "every block is covered and only the last instruction of a wave can fall past the tile");
  static constexpr int NC = D / 16;      // QK^T k-steps
  static constexpr int NDB = D / 32;     // dv blocks
  static constexpr float SUM_LIMIT = 18446744073709551616.0f;  // 2^64

  const AttnParams& p;
  char* smem;  // K stages then V stages
  int head, lane, wave, hh, l32;
  int dyn_r;  // bank entry of the Dynamic Sink
  uint32_t tok_bytes;

  uint32_t voff_k[NDMA], voff_v[NDMA];
  bool last_ok;  // this wave's last DMA instruction lands inside the tile

  bf16x8 qreg[2][NC];
  f32x16 o[2][NDB];
  float m_run[2], l_run[2];

  __device__ Attn(const AttnParams& p_, char* smem_, int head_) : p(p_), smem(smem_), head(head_) {
    dyn_r = load_dyn_r(p);
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    hh = lane >> 5;
    l32 = lane & 31;
    tok_bytes = (uint32_t)(p.n_heads * D * 2);
    // DMA instruction i of a wave moves unit block 4i + wave of a tile (only a
    // wave's last one can fall past the tile); unit u = 64 block + lane ->
    // (row, 16-byte slot)
    last_ok = 4 * (NDMA - 1) + wave < NBLK;
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int u = (4 * i + wave) * 64 + lane;
      const int r = u / NU, c = u - r * NU;
      const bool data = r < KT && c < NS;
      voff_k[i] = data ? (uint32_t)key_perm(r) * tok_bytes + c * 16 : kOutOfRange;
      voff_v[i] = data ? (uint32_t)r * tok_bytes + c * 16 : kOutOfRange;
    }
  }

  __device__ char* kbuf(int st) const { return smem + st * TILE; }
  __device__ char* vbuf(int st) const { return smem + (STAGES + st) * TILE; }
  __device__ char* pkbuf() const { return smem + 2 * STAGES * TILE; }
  __device__ char* pvbuf() const { return smem + (2 * STAGES + 1) * TILE; }

  // LDS destination of this wave's DMA instruction i into `tile`.  The four
  // waves issue NDMA instructions each; an instruction that falls wholly past
  // the tile (all its lanes are padding and load zeros) goes to a 1 KB sink.
  __device__ __forceinline__ uint32_t dma_lds(const char* tile, int i) const {
    return i < NDMA - 1 || last_ok ? lds_addr(tile) + (4 * i + wave) * 1024 : sink();
  }
  __device__ __forceinline__ uint32_t sink() const { return lds_addr(smem + (2 * STAGES + 2) * TILE); }

  // ---- packed ragged keys --------------------------------------------------
  // The last count % 64 keys of every segment, concatenated in segment order
  // (R of them), form packed tiles of 64 keys; with the keys already rotated,
  // attention does not care which segment a key came from.  Packed key kk of
  // this head: its K (or V) row.
  __device__ const char* packed_row(int kk, bool k) const {
    // unrolled over every segment slot (unused slots have count 0), with a
    // select per slot: kk differs between lanes
    int off = 0;
    const char* row = nullptr;
#pragma unroll
    for (int s = 0; s < kMaxSegments; ++s) {
      const int cnt = seg_count(p, s, dyn_r), r = cnt % KT;
      const char* base = seg_base(p, s, k, dyn_r);
      const char* cand = base + (size_t)head * D * 2 + (size_t)(cnt - r + kk - off) * tok_bytes;
      row = kk >= off && kk < off + r ? cand : row;
      off += r;
    }
    return row;
  }
  __device__ int ragged_keys() const {
    int r = 0;
#pragma unroll
    for (int s = 0; s < kMaxSegments; ++s) r += seg_count(p, s, dyn_r) % KT;
    return r;
  }

  // This wave's share of packed tile pt into kdst / vdst: a gather, one
  // 16-byte global load per lane (rows past R repeat packed key 0 and are
  // masked later; row padding loads the row's first 16 bytes, never read).
  // Lane L first finds the global rows of LDS row L of both tiles (K row L
  // holds packed key key_perm(L), V row L packed key L); each DMA lane then
  // takes the address of its row from that lane, so the segment search runs
  // twice per lane instead of twice per DMA instruction.
  __device__ __forceinline__ void dma_packed(int pt, int R, char* kdst, char* vdst) const {
    int kk = KT * pt + key_perm(lane), kv = KT * pt + lane;
    if (kk >= R) kk = 0;
    if (kv >= R) kv = 0;
    const uint64_t krow = reinterpret_cast<uint64_t>(packed_row(kk, true));
    const uint64_t vrow = reinterpret_cast<uint64_t>(packed_row(kv, false));
    const uint32_t k_lo = (uint32_t)krow, k_hi = (uint32_t)(krow >> 32);
    const uint32_t v_lo = (uint32_t)vrow, v_hi = (uint32_t)(vrow >> 32);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
      const int u = (4 * i + wave) * 64 + lane;
      const int r = u / NU, c = u - r * NU;
      const int cb = c < NS ? c * 16 : 0;
      const int src = r < KT ? r : 0;
      const uint64_t ka = ((uint64_t)(uint32_t)__shfl((int)k_hi, src, 64) << 32) | (uint32_t)__shfl((int)k_lo, src, 64);
      const uint64_t va = ((uint64_t)(uint32_t)__shfl((int)v_hi, src, 64) << 32) | (uint32_t)__shfl((int)v_lo, src, 64);
      dma16_flat_b(reinterpret_cast<const char*>(ka) + cb, dma_lds(kdst, i));
      dma16_flat_b(reinterpret_cast<const char*>(va) + cb, dma_lds(vdst, i));
    }
  }

  // Q' = bf16(rot(q) * log2(e)/sqrt(d)) as the QK^T B operand, in two
  // halves so that other loads can be issued between them: load_queries
  // issues the raw query chunks and the cos/sin of every pair the lane
  // holds, rotate_queries rotates, scales and packs them.
  struct QLoad {
    uint4 w[2][NC];
    float2 cs[2][NC][4];
  };
  __device__ __forceinline__ void load_queries(int qt, QLoad& L) const {
    const RopeGeom g = p.g;  // in registers: the lookups below must not reload it
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qrow = qt * QT + wave * 64 + qb * 32 + l32;
      const bool valid = qrow < p.n_q;
      int tq = 0, yq = 0, xq = 0;
      if (valid) token_pos(g, qrow, p.q_t_index, tq, yq, xq);
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((size_t)qrow * p.n_heads + head) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = 16 * c + 8 * hh;
        L.w[qb][c] = valid ? *reinterpret_cast<const uint4*>(qp + off) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) L.cs[qb][c][e] = rope_cs(g, off / 2 + e, tq, yq, xq);
      }
    }
  }
  __device__ __forceinline__ void rotate_queries(const QLoad& L) {
    const float sc = p.scale_log2;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t ws[4] = {L.w[qb][c].x, L.w[qb][c].y, L.w[qb][c].z, L.w[qb][c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 cs = L.cs[qb][c][e];
          const float x0 = __uint_as_float(ws[e] << 16), x1 = __uint_as_float(ws[e] & 0xffff0000u);
          ws[e] = pack_bf16((x0 * cs.x - x1 * cs.y) * sc, (x0 * cs.y + x1 * cs.x) * sc);
        }
        qreg[qb][c] = __builtin_bit_cast(bf16x8, make_uint4(ws[0], ws[1], ws[2], ws[3]));
      }
    reset_accumulators();
  }
  __device__ void init_queries(int qt) {
    QLoad L;
    load_queries(qt, L);
    rotate_queries(L);
  }

  __device__ void reset_accumulators() {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int i = 0; i < NDB; ++i) o[qb][i] = f32x16{};
      m_run[qb] = -INFINITY;
      l_run[qb] = 0.f;
    }
  }

  // Buffer resources of tile (s, n0) of this head: the range ends at the
  // segment's last token, so rows past it read as zero and nothing outside the
  // segment is touched.  valid == false gives an empty range (all zeros).
  __device__ __forceinline__ void rsrc(int s, int n0, bool valid, __amdgpu_buffer_rsrc_t& rk,
                                       __amdgpu_buffer_rsrc_t& rv) const {
    const int si = valid ? s : 0;
    const Segment& sg = p.seg[si];
    const size_t off = valid ? (size_t)head * sg.head * 2 + (size_t)n0 * tok_bytes : 0;
    const int nrec = valid ? (int)((size_t)(seg_count(p, si, dyn_r) - n0) * tok_bytes) : 0;
    rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(seg_base(p, si, true, dyn_r) + off), 0, nrec,
                                           kBufferConfig);
    rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(seg_base(p, si, false, dyn_r) + off), 0, nrec,
                                           kBufferConfig);
  }

  // This wave's share (NDMA instructions) of a K or V tile into LDS.
  __device__ __forceinline__ void dma_k(char* dst, __amdgpu_buffer_rsrc_t r) const {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma16(r, dma_lds(dst, i), voff_k[i]);
  }
  __device__ __forceinline__ void dma_v(char* dst, __amdgpu_buffer_rsrc_t r) const {
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma16(r, dma_lds(dst, i), voff_v[i]);
  }

  // S'^T of key block kb (32 keys) for both query blocks; the accumulators
  // start from c0[qb].
  __device__ __forceinline__ void qk_half(const char* kt, int kb, const f32x16 (&c0)[2],
                                          f32x16 (&sc)[2]) const {
    const char* kr = kt + (kb * 32 + l32) * RBP + hh * 16;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + c * 32);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][c], c == 0 ? c0[qb] : sc[qb], 0, 0, 0);
    }
  }

  // p = 2^s for the 16 scores of one (query block, key block), packed to bf16
  // as the PV B operands of k-steps 2kb and 2kb+1 (register r holds key
  // 16*(r/8) + 8hh + r%8 of the block); returns the lane's sum of the packed
  // values, so the normaliser sums the same rounded weights the PV uses.
  __device__ __forceinline__ void soft(const f32x16& s, bf16x8& p_lo, bf16x8& p_hi, float& acc) const {
    uint32_t pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pw[e] = pack_bf16(__builtin_amdgcn_exp2f(s[2 * e]), __builtin_amdgcn_exp2f(s[2 * e + 1]));
      acc += __uint_as_float(pw[e] << 16);
      acc += __uint_as_float(pw[e] & 0xffff0000u);
    }
    p_lo = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    p_hi = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
  }

  // O^T += V^T P^T over keys 32kb .. 32kb+31.  Lane (dv = 32db + l32, hh) needs
  // keys 16kc + 8hh + j, j = 0..7: two transpose reads; in each, lane 4e + q of
  // a 16-lane group points at row 16kc + 8hh + 4rd + e, dims
  // 32db + 16*(group&1) + 4q .. +3.
  __device__ __forceinline__ void pv_half(const char* vt, int kb, const bf16x8 (&pb)[2][4]) {
    const int grp = lane >> 4, i16 = lane & 15;
    const char* vl = vt + (8 * hh + (i16 >> 2)) * RBP + (16 * (grp & 1) + 4 * (i16 & 3)) * 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kc = 2 * kb; kc < 2 * kb + 2; ++kc) {
        i16x4 h[2];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd)
          h[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vl + (16 * kc + 4 * rd) * RBP + 64 * db));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][kc], o[qb][db], 0, 0, 0);
      }
  }

  // Any tile, exact online softmax: keys past `count` are masked, the running
  // max follows the tile max and O and the normaliser are rescaled.
  __device__ void step_exact(const char* kt, const char* vt, int n0, int count) {
    const f32x16 zero[2] = {f32x16{}, f32x16{}};
    f32x16 sc[2][2];  // [key block][query block]
    qk_half(kt, 0, zero, sc[0]);
    qk_half(kt, 1, zero, sc[1]);
    // register r of key block kb holds key kb*32 + 16*(r/8) + 8hh + r%8
    const int lim = count - n0 - hh * 8;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + (r >> 3) * 16 + (r & 7) >= lim) sc[kb][qb][r] = -INFINITY;
    bf16x8 pb[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float m = sc[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, sc[kb][qb][r]);
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      const float m_new = fmaxf(m_run[qb], m);  // finite: every tile has a valid key
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[qb][db] *= alpha;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 t = sc[kb][qb];
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] -= m_new;
        soft(t, pb[qb][2 * kb], pb[qb][2 * kb + 1], rs);
      }
      l_run[qb] = l_run[qb] * alpha + rs;
    }
    pv_half(vt, 0, pb);
    pv_half(vt, 1, pb);
  }

  // ---- steady-state schedule -------------------------------------------
  // One iteration (QK^T of the next tile, PV of the current one) is a fixed
  // sequence of NOPS steps in four groups: A = QK^T keys 0..31 (NC steps),
  // B = PV keys 0..31 (2*NDB steps), C = QK^T keys 32..63, D = PV keys 32..63.
  // Each step issues the LDS read of the operand three steps ahead, its two
  // MFMAs (one per query block) and PAIRS packed softmax pairs split between
  // the two MFMA shadows; steps are fenced, so this order is the issue order.
  static constexpr int GA = NC, GB = 2 * NDB;
  static constexpr int NOPS = 2 * GA + 2 * GB;
  static constexpr int PAIRS = 8 / GA;  // softmax pairs per step (GA == GB)
  static_assert(GA == GB, "groups of equal length");

  // MFMA A operand t of an iteration (t >= NOPS: the next iteration's first
  // operands, from the next K tile).
  __device__ __forceinline__ bf16x8 op(int t, const char* kt, const char* vt, const char* kn) const {
    if (t >= NOPS) return *reinterpret_cast<const bf16x8*>(kn + l32 * RBP + hh * 16 + (t - NOPS) * 32);
    const int g = t / GA, i = t % GA;
    if (g == 0 || g == 2) {  // K, key block g/2, k-step i
      return *reinterpret_cast<const bf16x8*>(kt + ((g / 2) * 32 + l32) * RBP + hh * 16 + i * 32);
    }
    // V^T, dv block i/2, k-step kc = 2*(g/2) + i%2
    const int db = i / 2, kc = 2 * (g / 2) + i % 2;
    const int grp = lane >> 4, i16 = lane & 15;
    const char* vl = vt + (8 * hh + (i16 >> 2)) * RBP + (16 * (grp & 1) + 4 * (i16 & 3)) * 2;
    i16x4 h[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
      h[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vl + (16 * kc + 4 * rd) * RBP + 64 * db));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
  }

  static __device__ __forceinline__ bf16x8 words(const uint32_t (&w)[4]) {
    return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }

  // ---- split jobs ------------------------------------------------------
  // A partial record holds this workgroup's unnormalised O (fp32, in the
  // MFMA lane layout: float4 (dv 32db+8g+4hh .. +3) of query block qb at
  // [((wave*2 + qb)*NDB + db)*4 + g][lane]) and (m, l) per lane at
  // [(wave*2 + qb)][lane] after it; the workgroups that read a record run
  // this same code, so the layout is the registers' own.  Records move with
  // system-coherent buffer accesses (sc0 sc1): they bypass the XCD's L2, so
  // handing one over needs no L2-wide write-back or invalidate, which would
  // evict the keys the other workgroups of the XCD are sharing.
  static constexpr int kCoherent = 1 | 16;  // sc0 | sc1
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t record(float* rec) {
    return __builtin_amdgcn_make_buffer_rsrc(rec, 0, (int)(partial_record_floats(D) * 4), kBufferConfig);
  }
  __device__ void store_partial(float* rec) const {
    const __amdgpu_buffer_rsrc_t r = record(rec);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 v = {__float_as_uint(o[qb][db][4 * g]), __float_as_uint(o[qb][db][4 * g + 1]),
                           __float_as_uint(o[qb][db][4 * g + 2]), __float_as_uint(o[qb][db][4 * g + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(v, r, ((((wave * 2 + qb) * NDB + db) * 4 + g) * 64 + lane) * 16,
                                                 0, kCoherent);
        }
      const u32x2 ml = {__float_as_uint(m_run[qb]), __float_as_uint(l_run[qb])};
      __builtin_amdgcn_raw_buffer_store_b64(ml, r, 256 * D * 4 + ((wave * 2 + qb) * 64 + lane) * 8, 0, kCoherent);
    }
  }
  // Folds another piece of the same job into the registers (first: replaces
  // them): both sides are rescaled to the larger reference max.  All of the
  // record's loads are issued before any is used (coherent loads are not
  // reordered, so waiting on each in turn would pay the memory latency once
  // per load).
  __device__ void merge_partial(float* rec, bool first) {
    const __amdgpu_buffer_rsrc_t r = record(rec);
    u32x2 ml[2];
    u32x4 v[2][NDB][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      ml[qb] = __builtin_amdgcn_raw_buffer_load_b64(r, 256 * D * 4 + ((wave * 2 + qb) * 64 + lane) * 8, 0, kCoherent);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          v[qb][db][g] = __builtin_amdgcn_raw_buffer_load_b128(
              r, ((((wave * 2 + qb) * NDB + db) * 4 + g) * 64 + lane) * 16, 0, kCoherent);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mq = __uint_as_float(ml[qb].x), lq = __uint_as_float(ml[qb].y);
      if (first) {
        m_run[qb] = mq;
        l_run[qb] = lq;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[qb][db][4 * g + e] = __uint_as_float(v[qb][db][g][e]);
        continue;
      }
      const float mx = fmaxf(m_run[qb], mq);
      const float al = __builtin_amdgcn_exp2f(m_run[qb] - mx), be = __builtin_amdgcn_exp2f(mq - mx);
      m_run[qb] = mx;
      l_run[qb] = l_run[qb] * al + lq * be;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[qb][db][4 * g + e] = o[qb][db][4 * g + e] * al + __uint_as_float(v[qb][db][g][e]) * be;
    }
  }

  __device__ void epilogue(int qt) {
    // The normalised bf16 rows go through this wave's own LDS region, so each
    // global store writes whole 256-byte rows (16 lanes a row) instead of 16
    // bytes in each of 32 rows.  Every wave has passed a barrier after its
    // last read of the ring and no DMA is in flight, so the region is free.
    // register 4g+e of dv block db is dv = 32db + 8g + 4hh + e
    constexpr int OS = RB + 16;  // LDS row stride (16-byte aligned rows)
    char* const ob = smem + wave * 64 * OS;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
      const float inv = 1.0f / l_tot;
      char* const orow = ob + (qb * 32 + l32) * OS + hh * 8;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(orow + db * 64 + g * 16) =
              make_uint2(pack_bf16(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv),
                         pack_bf16(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv));
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    constexpr int RPI = 64 / NS;  // rows per store instruction
    const int c = lane % NS;
    const int row0 = qt * QT + wave * 64 + lane / NS;
    char* const out0 = static_cast<char*>(p.out) + ((size_t)row0 * p.n_heads + head) * RB + c * 16;
    const size_t step = (size_t)RPI * p.n_heads * RB;
    const char* const in0 = ob + (lane / NS) * OS + c * 16;
    if (qt * QT + wave * 64 + 64 <= p.n_q) {  // every row of the wave is a query
#pragma unroll
      for (int i = 0; i < 64 / RPI; ++i)
        *reinterpret_cast<uint4*>(out0 + i * step) = *reinterpret_cast<const uint4*>(in0 + i * RPI * OS);
    } else {
#pragma unroll
      for (int i = 0; i < 64 / RPI; ++i)
        if (row0 + i * RPI < p.n_q)
          *reinterpret_cast<uint4*>(out0 + i * step) = *reinterpret_cast<const uint4*>(in0 + i * RPI * OS);
    }
  }
};

// Software-pipelined softmax of the steady-state loop (see the kernel).  Pair
// q (0..31) of an iteration is exponentiated at step q / PAIRS (stage 0) and
// packed to bf16 and summed one step later (stage 1), in the next iteration
// when that passes the end.  Exponentials move between the stages through a
// two-slot ring indexed by the parity of the stage-0 step (NOPS is even, so
// the parity survives the wrap).
template <class A>
struct SoftPipe {
  static constexpr int NOPS = A::NOPS, PAIRS = A::PAIRS, NSTAGE = 2;
  static_assert(NOPS % 2 == 0, "the stage ring is indexed by step parity");
  f32x16 s_hi[2];         // scores of keys 32..63 of the current tile, shifted by -m
  uint32_t pw[2][4][4];   // PV B operands [query block][k-step][word]
  uint32_t nw[2][2][4];   // words of the next tile's keys 0..31 made in this iteration
  float e[2][PAIRS][2];
  float acc[2][2];        // row sums [query block][even/odd element]

  __device__ void init(const bf16x8 (&pb)[2][4], float l0, float l1, const f32x16 (&sh)[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s_hi[qb] = sh[qb];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int w = 0; w < 4; ++w) pw[qb][kc][w] = __builtin_bit_cast(uint4, pb[qb][kc])[w];
    }
    acc[0][0] = l0;
    acc[1][0] = l1;
    acc[0][1] = acc[1][1] = 0.f;
  }

  // The packed word of pair q: pairs 0..15 feed k-steps 2..3 of this tile;
  // pairs 16..31 feed k-steps 0..1 of the next tile, held in nw while made
  // within their iteration and in pw once the next iteration has begun.
  __device__ __forceinline__ uint32_t& word(int q, bool next) {
    if (q < 16) return pw[q / 8][2 + (q % 8) / 4][q % 4];
    const int u = q - 16;
    return next ? pw[u / 8][(u % 8) / 4][u % 4] : nw[u / 8][(u % 8) / 4][u % 4];
  }

  // Stages due at step t.  FIRST: no earlier iteration (skip wrapped stages).
  // FLUSH: only the wrapped stages (the step after the last iteration).
  // Parts of a pair's work, so a step's work can be split between the
  // shadows of its two MFMAs.
  static constexpr int kExp0 = 1, kExp1 = 2, kPack = 4, kAdd0 = 8, kAdd1 = 16, kAll = 31;

  // Stages due at step t, the parts in `parts` only.  FIRST: no earlier
  // iteration (skip wrapped stages).  FLUSH: only the wrapped stages (the
  // step after the last iteration).
  template <bool FIRST, bool FLUSH>
  __device__ __forceinline__ void run(int t, const f32x16& n_lo0, const f32x16& n_lo1, int parts = kAll) {
#pragma unroll
    for (int k = NSTAGE - 1; k >= 0; --k) {
      const int s0 = t - k;
      const bool wrapped = s0 < 0;
      if ((wrapped && FIRST) || (!wrapped && FLUSH)) continue;
      const int sl = (s0 + NOPS) & 1;
#pragma unroll
      for (int pp = 0; pp < PAIRS; ++pp) {
        const int q = (wrapped ? s0 + NOPS : s0) * PAIRS + pp;
        const int qb = (q / 8) & 1;
        if (k == 0) {
          const f32x16& sv = q < 8 ? s_hi[0] : q < 16 ? s_hi[1] : q < 24 ? n_lo0 : n_lo1;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (parts & (kExp0 << h)) {
              e[sl][pp][h] = __builtin_amdgcn_exp2f(sv[2 * (q % 8) + h]);
              asm volatile("" : "+v"(e[sl][pp][h]));
            }
        } else {
          if (parts & kPack) {
            uint32_t& w = word(q, wrapped);
            w = pack_bf16(e[sl][pp][0], e[sl][pp][1]);
            asm volatile("" : "+v"(w));
          }
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (parts & (kAdd0 << h)) {
              acc[qb][h] += e[sl][pp][h];
              asm volatile("" : "+v"(acc[qb][h]));
            }
        }
      }
    }
  }

  template <bool FIRST>
  __device__ __forceinline__ void step(int t, int parts, const f32x16& n_lo0, const f32x16& n_lo1) {
    run<FIRST, false>(t, n_lo0, n_lo1, parts);
  }

  // Closes an iteration: the new keys 32..63 become s_hi, and the words made
  // within it move to their next-iteration place.
  __device__ __forceinline__ void end_iteration(const f32x16 (&n_hi)[2]) {
    s_hi[0] = n_hi[0];
    s_hi[1] = n_hi[1];
#pragma unroll
    for (int q = 16; q < 32; ++q)
      if (q / PAIRS + 1 < NOPS) word(q, true) = word(q, false);
  }

  // Runs the stages still pending after the last iteration.
  __device__ __forceinline__ void flush() {
#pragma unroll
    for (int t = 0; t < NSTAGE - 1; ++t) run<false, true>(t, s_hi[0], s_hi[1]);  // no reads
  }

  __device__ __forceinline__ float sum(int qb) const { return acc[qb][0] + acc[qb][1]; }
};

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_kernel(const AttnParams p) {
  using A = Attn<D>;
  __shared__ __align__(16) char smem[A::LDS_BYTES];
  __shared__ int bad_flag[4];
  __shared__ int last_piece;

  Work w;
  if (!map_work(p, w)) return;
  const int head = w.head, qt = w.qt;
  A a(p, smem, head);

  int n_tiles = 0;  // full tiles of the head (unused segment slots have count 0)
#pragma unroll
  for (int s = 0; s < kMaxSegments; ++s) n_tiles += seg_count(p, s, a.dyn_r) / A::KT;
  const int n_ragged = a.ragged_keys();
  // this piece's units [u0, u1): full tiles [f0, f0 + n_full), then packed
  // ragged tiles [pk0, pk1)
  const int u0 = p.units * w.piece / w.n_pieces, u1 = p.units * (w.piece + 1) / w.n_pieces;
  const int f0 = min(u0, n_tiles), n_full = min(u1, n_tiles) - f0;
  // (units counts the Dynamic segment as planned; a vanished one leaves fewer
  // tiles than planned, so both ranges are clamped to what exists)
  const int n_pk = (n_ragged + A::KT - 1) / A::KT;
  const int pk0 = min(max(u0, n_tiles) - n_tiles, n_pk), pk1 = min(max(u1, n_tiles) - n_tiles, n_pk);

  bool bad = false;
  if (n_full > 0) {
    // K and V of tile t go to stage t % 3.  The prologue issues the queries'
    // loads and their cos/sin lookups first, then K0, K1, V0, K2, V1 and the
    // gather of the first packed ragged tile, then rotates the queries while
    // the DMAs land; iteration j issues {K(j+3), V(j+2)} after its barrier,
    // which waits for every earlier group.  Tiles past the piece's last one
    // re-read real keys into stages nobody reads.
    typename A::QLoad ql;
    a.load_queries(qt, ql);
    __builtin_amdgcn_sched_barrier(0);
    const size_t head_off = (size_t)head * D * 2;
    const uint32_t tok_bytes = a.tok_bytes, tile_bytes = A::KT * tok_bytes;
    SegCursor ck, cv;  // next K tile to load, next V tile to load
    ck.first(p, head_off, tok_bytes, tile_bytes, true, f0, a.dyn_r);
    cv.first(p, head_off, tok_bytes, tile_bytes, false, f0, a.dyn_r);
    const uint32_t kbase = lds_addr(a.kbuf(0)), vbase = lds_addr(a.vbuf(0));
    auto load = [&](SegCursor& c, uint32_t stage, const uint32_t (&voff)[A::NDMA], bool is_k) {
#pragma unroll
      for (int i = 0; i < A::NDMA; ++i)
        dma16_b(c.r, i < A::NDMA - 1 || a.last_ok ? stage + (4 * i + a.wave) * 1024 : a.sink(), voff[i],
                c.off);
      c.next(p, head_off, tok_bytes, tile_bytes, is_k);
    };
    load(ck, kbase, a.voff_k, true);                 // K0
    load(ck, kbase + A::TILE, a.voff_k, true);       // K1
    load(cv, vbase, a.voff_v, false);                // V0
    load(ck, kbase + 2 * A::TILE, a.voff_k, true);   // K2
    load(cv, vbase + A::TILE, a.voff_v, false);      // V1
    if (pk1 > pk0) a.dma_packed(pk0, n_ragged, a.pkbuf(), a.pvbuf());
    __builtin_amdgcn_sched_barrier(0);
    a.rotate_queries(ql);
    wait_vm<0>();
    __syncthreads();

    // First tile, exact: sets each row's reference max m.
    const f32x16 zero[2] = {f32x16{}, f32x16{}};
    f32x16 s_lo[2], s_hi[2];  // [query block]: keys 0..31 / keys 32..63 of the tile
    a.qk_half(a.kbuf(0), 0, zero, s_lo);
    a.qk_half(a.kbuf(0), 1, zero, s_hi);
    f32x16 cm[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float m = s_lo[qb][0];
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(fmaxf(m, s_lo[qb][r]), s_hi[qb][r]);
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      a.m_run[qb] = m;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        cm[qb][r] = -m;
        s_lo[qb][r] -= m;
        s_hi[qb][r] -= m;
      }
    }
    bf16x8 pb[2][4];
    float l0 = 0.f, l1 = 0.f;
    a.soft(s_lo[0], pb[0][0], pb[0][1], l0);
    a.soft(s_lo[1], pb[1][0], pb[1][1], l1);

    // Steady state: iteration j = QK^T of tile j+1 and PV of tile j, in the
    // fixed step order of Attn::NOPS.  Entering it: pw[.][0..1] (P of keys
    // 0..31 of tile j), s_hi (scores of keys 32..63 of tile j, shifted by -m)
    // and the first three K operands of tile j+1 are ready.  The one barrier of
    // an iteration sits between groups B and C: it waits for the DMA group
    // issued an iteration earlier ({K(j+2), V(j+1)}), so the next tile's first
    // operands can be read before the iteration ends; then the group
    // {K(j+3), V(j+2)} is issued, one DMA per step of groups C and D.
    //
    // Softmax runs as a two-stage software pipeline over the 32 packed pairs
    // of an iteration (pairs 0..7: s_hi of query block 0, 8..15: s_hi of block
    // 1, 16..23 / 24..31: the new keys 0..31 of blocks 0 / 1): stage 0
    // exponentiates a pair's two scores, stage 1, one step later, packs them
    // to bf16 (the PV operand word) and adds the fp32 exponentials to the row
    // sums, so no instruction waits on a result issued in the same step and
    // the MFMAs keep issuing.  Stage 1 of an iteration's last pairs runs in
    // the next iteration's first step (or in the drain).
    using SP = SoftPipe<A>;
    SP sp;
    sp.init(pb, l0, l1, s_hi);
    // queries live in AGPRs from here on (the QK^T MFMAs read them there)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int c = 0; c < A::NC; ++c) asm volatile("" : "+a"(a.qreg[qb][c]));
    bf16x8 ring[4];
    {
      const char* kt = a.kbuf(1 % A::STAGES);
      ring[0] = a.op(A::NOPS, kt, kt, kt);
      ring[1] = a.op(A::NOPS + 1, kt, kt, kt);
      ring[2] = a.op(A::NOPS + 2, kt, kt, kt);
    }
    // LDS byte offsets of stages j % 3, (j + 1) % 3 and (j + 2) % 3 in
    // iteration j: QK^T reads K stage st1, PV reads V stage st0, the next
    // tile's first operands come from K stage st2; K(j+3) goes to K stage st0
    // and V(j+2) to V stage st2.
    uint32_t st0 = 0, st1 = A::TILE, st2 = 2 * A::TILE;
    const uint32_t wave_blk = a.wave * 1024;
    auto iteration = [&](auto first) {
      constexpr bool FIRST = decltype(first)::value;
      const char* kt = a.kbuf(0) + st1;
      const char* vt = a.vbuf(0) + st0;
      const char* kn = a.kbuf(0) + st2;
      f32x16 n_lo[2], n_hi[2];
      uint32_t kdst = 0, vdst = 0, klast = 0, vlast = 0, m0_saved = 0;
#pragma unroll
      for (int t = 0; t < A::NOPS; ++t) {
        const int g = t / A::GA, i = t % A::GA;
        if (t == 2 * A::GA) {  // between groups B and C
          wait_vm<0>();
          __syncthreads();
          kdst = kbase + st0 + wave_blk;
          vdst = vbase + st2 + wave_blk;
          klast = a.last_ok ? kdst + (A::NDMA - 1) * 4096 : a.sink();
          vlast = a.last_ok ? vdst + (A::NDMA - 1) * 4096 : a.sink();
          __builtin_amdgcn_sched_barrier(0);
        }
        ring[(t + 3) % 4] = a.op(t + 3, kt, vt, kn);
        const bf16x8 x = ring[t % 4];
        // MFMA of query block 0 with the exponentials and the packing in its
        // shadow, then MFMA of query block 1 with the row sums and the DMA in
        // its shadow.  (An MFMA issued right behind another holds the wave
        // until the first one drains, so work placed between two MFMAs is the
        // only work that overlaps the first.)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (qb == 1) {
            __builtin_amdgcn_sched_barrier(0);
            sp.template step<FIRST>(t, SP::kExp0 | SP::kExp1 | SP::kPack, n_lo[0], n_lo[1]);
            __builtin_amdgcn_sched_barrier(0);
          }
          if (g == 0) {
            if (i == 0) n_lo[qb] = mfma_qk_first(x, a.qreg[qb][i], cm[qb]);
            else mfma_qk_acc(n_lo[qb], x, a.qreg[qb][i]);
          }
          if (g == 2) {
            if (i == 0) n_hi[qb] = mfma_qk_first(x, a.qreg[qb][i], cm[qb]);
            else mfma_qk_acc(n_hi[qb], x, a.qreg[qb][i]);
          }
          if (g == 1 || g == 3) {
            const int db = i / 2, kc = 2 * (g / 2) + i % 2;
            a.o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, A::words(sp.pw[qb][kc]), a.o[qb][db], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        sp.template step<FIRST>(t, SP::kAdd0 | SP::kAdd1, n_lo[0], n_lo[1]);
        if ((g == 2 || g == 3) && i < A::NDMA) {
          const SegCursor& c = g == 2 ? ck : cv;
          const uint32_t vo = g == 2 ? a.voff_k[i] : a.voff_v[i];
          const bool save = t == 2 * A::GA, restore = t == 3 * A::GA + A::NDMA - 1;
          if (i == A::NDMA - 1)
            dma16_run(c.r, g == 2 ? klast : vlast, 0, vo, c.off, save, restore, m0_saved);
          else
            dma16_run(c.r, g == 2 ? kdst : vdst, i, vo, c.off, save, restore, m0_saved);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      ck.next(p, head_off, tok_bytes, tile_bytes, true);
      cv.next(p, head_off, tok_bytes, tile_bytes, false);
      sp.end_iteration(n_hi);
      const uint32_t t0 = st0;
      st0 = st1;
      st1 = st2;
      st2 = t0;
    };
    if (n_full > 1) iteration(std::true_type{});
    for (int j = 1; j + 1 < n_full; ++j) iteration(std::false_type{});
    // Drain: finish the pipeline, then PV of the last full tile (its V arrived
    // with an earlier group).
    if (n_full > 1) sp.flush();
    wait_vm<0>();
    __syncthreads();
    {
      const char* vt = a.vbuf((n_full - 1) % A::STAGES);
      float r0 = 0.f, r1 = 0.f;
      a.soft(sp.s_hi[0], pb[0][2], pb[0][3], r0);
      a.soft(sp.s_hi[1], pb[1][2], pb[1][3], r1);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) pb[qb][kc] = A::words(sp.pw[qb][kc]);
      a.pv_half(vt, 0, pb);
      a.pv_half(vt, 1, pb);
      l0 = sp.sum(0) + r0;
      l1 = sp.sum(1) + r1;
    }
    a.l_run[0] = l0;
    a.l_run[1] = l1;
    const bool mine = __any(!(l0 <= A::SUM_LIMIT) | !(l1 <= A::SUM_LIMIT));
    if (a.lane == 0) bad_flag[a.wave] = mine;
    wait_vm<0>();
    __syncthreads();  // every DMA done, flags visible, stages free
    bad = bad_flag[0] | bad_flag[1] | bad_flag[2] | bad_flag[3];
  } else {
    a.init_queries(qt);
  }

  // Exact, single-buffered passes: the packed ragged tiles (the first one is
  // already in LDS when the pipelined loop ran), and after an overflow every
  // full tile again.
  if (bad) {
    a.reset_accumulators();
    for (int s = 0, t = 0; s < p.n_seg; ++s) {
      const int cnt = seg_count(p, s, a.dyn_r);
      for (int n0 = 0; n0 + A::KT <= cnt; n0 += A::KT, ++t) {
        if (t < f0 || t >= f0 + n_full) continue;
        __amdgpu_buffer_rsrc_t rk, rv;
        a.rsrc(s, n0, true, rk, rv);
        a.dma_k(a.kbuf(0), rk);
        a.dma_v(a.vbuf(0), rv);
        wait_vm<0>();
        __syncthreads();
        a.step_exact(a.kbuf(0), a.vbuf(0), n0, cnt);
        __syncthreads();
      }
    }
  }
  for (int pt = pk0; pt < pk1; ++pt) {
    if (pt > pk0 || n_full == 0) {
      a.dma_packed(pt, n_ragged, a.pkbuf(), a.pvbuf());
      wait_vm<0>();
      __syncthreads();
    }
    a.step_exact(a.pkbuf(), a.pvbuf(), pt * A::KT, n_ragged);
    __syncthreads();
  }
  if (w.n_pieces > 1) {
    // Split job: publish this piece, and the last piece to arrive merges the
    // others (the counter wraps back to 0 on that arrival).
    const size_t rec = partial_record_floats(D);
    float* const base = p.part + (size_t)w.job * w.n_pieces * rec;
    // Ordering without cache-wide fences: every record access and the counter
    // are system-coherent, each thread's stores have completed (vmcnt 0)
    // before the barrier that precedes the counter update, and the other
    // records are read only after the update has returned.
    a.store_partial(base + (size_t)w.piece * rec);
    wait_vm<0>();
    __syncthreads();
    if (threadIdx.x == 0)
      last_piece = __builtin_amdgcn_atomic_inc32(p.cnt + w.job, (uint32_t)(w.n_pieces - 1), __ATOMIC_RELAXED,
                                                 "") == (uint32_t)(w.n_pieces - 1);
    __syncthreads();
    if (!last_piece) return;
    // rebuilt from every record in piece order, this one's included, so the
    // result does not depend on which piece arrived last
    for (int r = 0; r < w.n_pieces; ++r) a.merge_partial(base + (size_t)r * rec, r == 0);
  }
  a.epilogue(qt);
}

// ---------------------------------------------------------------------------
// fp32: one query row per lane, 64-key tiles staged in LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnParams p) {
  constexpr int KT = kKeyTile;
  __shared__ float Ks[KT][D + 1];
  __shared__ float Vs[KT][D + 1];
  const int head = blockIdx.y;
  const int lane = threadIdx.x;
  const int H = p.n_heads;
  const int qrow = blockIdx.x * KT + lane;
  const bool qvalid = qrow < p.n_q;

  float q[D];
  {
    int tq = 0, yq = 0, xq = 0;
    if (qvalid) token_pos(p.g, qrow, p.q_t_index, tq, yq, xq);
    const float* qp = static_cast<const float*>(p.q) + ((size_t)qrow * H + head) * D;
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      float x0 = 0.f, x1 = 0.f;
      if (qvalid) { x0 = qp[2 * i]; x1 = qp[2 * i + 1]; }
      const float2 cs = rope_cs(p.g, i, tq, yq, xq);
      q[2 * i] = x0 * cs.x - x1 * cs.y;
      q[2 * i + 1] = x0 * cs.y + x1 * cs.x;
    }
  }
  float o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int dyn_r = load_dyn_r(p);

  for (int s = 0; s < p.n_seg; ++s) {
    const Segment sg = p.seg[s];
    const int count = seg_count(p, s, dyn_r);
    const float* kbase = reinterpret_cast<const float*>(seg_base(p, s, true, dyn_r)) + (size_t)head * sg.head;
    const float* vbase = reinterpret_cast<const float*>(seg_base(p, s, false, dyn_r)) + (size_t)head * sg.head;
    for (int n0 = 0; n0 < count; n0 += KT) {
      for (int id = lane; id < KT * D; id += KT) {
        const int r = id / D, dv = id % D;
        const int n = n0 + r;
        Ks[r][dv] = n < count ? kbase[(size_t)n * sg.tok + dv] : 0.f;
        Vs[r][dv] = n < count ? vbase[(size_t)n * sg.tok + dv] : 0.f;
      }
      __syncthreads();
      const int nk = min(KT, count - n0);
      for (int j = 0; j < nk; ++j) {
        float sdot = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) sdot += q[i] * Ks[j][i];
        const float sv = sdot * p.scale_log2;
        const float m_new = fmaxf(m_run, sv);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        const float pj = __builtin_amdgcn_exp2f(sv - m_new);
        m_run = m_new;
        l_run = l_run * alpha + pj;
#pragma unroll
        for (int i = 0; i < D; ++i) o[i] = o[i] * alpha + pj * Vs[j][i];
      }
      __syncthreads();
    }
  }
  if (qvalid) {
    float* op = static_cast<float*>(p.out) + ((size_t)qrow * H + head) * D;
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int i = 0; i < D; ++i) op[i] = o[i] * inv;
  }
}

// Split plan of the bf16 kernel: per XCD, nj jobs on c CUs run as F = nj / c
// rounds of whole jobs and R = nj % c jobs cut into s key ranges, s chosen
// for the shortest estimated makespan.  A piece costs its share of a job plus
// a start-up of about 8 key units and 15 % of a job: the chip runs power
// limited, so a partly idle last round clocks higher and a split buys less
// than the idle CUs suggest (measured at 480x480: 40 heads x 11 query tiles
// on 256 CUs run fastest unsplit), while a handful of jobs on an otherwise
// idle chip still gains from it.
void plan_split(AttnParams& p, int n_cu) {
  int c = n_cu / 8;
  if (c < 1) c = 1;
  if (c > kMaxCuPerXcd) c = kMaxCuPerXcd;
  const int nj = (p.n_heads + 7) / 8 * p.n_qtiles;
  const int F = nj / c, R = nj - F * c;
  int best = 1;
  if (R > 0 && p.part != nullptr && !p.dyn_may_vanish) {
    const double o = 0.15 + 8.0 / p.units;
    double best_cost = 1e30;
    for (int sp = 1; sp <= kMaxSplit && sp <= p.units; ++sp) {
      const double cost = (double)((R * sp + c - 1) / c) * (1.0 / sp + o);
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = sp;
      }
    }
  }
  if (best == 1) {  // every job whole
    p.full_jobs = nj;
    p.tail_jobs = 0;
  } else {
    p.full_jobs = F * c;
    p.tail_jobs = R;
  }
  p.split = best;
}

}  // namespace

hipError_t launch_attention(const AttnParams& p_in, int dtype, int head_dim, int n_cu, hipStream_t s) {
  AttnParams p = p_in;
  if (dtype == 0) {  // bf16
    p.n_qtiles = (p.n_q + 255) / 256;
    int n_full = 0, n_rag = 0;
    for (int i = 0; i < p.n_seg; ++i) {
      n_full += p.seg[i].count / kKeyTile;
      n_rag += p.seg[i].count % kKeyTile;
    }
    p.units = n_full + (n_rag + kKeyTile - 1) / kKeyTile;
    plan_split(p, n_cu);
    const dim3 grid(8 * (p.full_jobs + p.tail_jobs * p.split));
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(256), 0, s, p);
  } else {
    p.n_qtiles = (p.n_q + kKeyTile - 1) / kKeyTile;
    const dim3 grid(p.n_qtiles, p.n_heads);
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace prsink
