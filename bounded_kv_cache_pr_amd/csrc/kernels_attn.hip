// PR-Sink block-causal attention with RoPE follow on gfx950.
//
// The current block's queries attend over [Ref; Static; Dynamic; window;
// current] with scale 1/sqrt(d) (LiveAnimate review on paper.rainbus.top,
// full-pipeline paragraph, attention formula and the prose around it: the
// current block is attended too).  Every key is read raw and rotated with 3D
// RoPE at its segment's *current* temporal slot and its latent (row, column)
// before use (same paragraph: raw keys re-rotated at the current cache
// position; novelty paragraph: reuse decoupled from the original timestamp).
//
// Common structure of the bf16 kernels:
//   * S^T = K_rot Q_rot^T on v_mfma_f32_32x32x16_bf16.  A lane owns one query
//     column and 16 key rows of each 32x32 block, so the softmax row max/sum
//     stay in-lane except for one exchange with lane ^ 32.  Keys sit in LDS
//     with bits 2 and 3 of their row index swapped, which makes the
//     probabilities a lane holds after QK^T exactly the B operand of the PV
//     MFMA, with no shuffles.
//   * O^T = V^T P^T accumulates in fp32; the online softmax runs in base 2
//     with the 1/sqrt(d) scale folded into one FMA per score.
// The fp32 kernel is a plain one-query-per-lane loop for fp32 caches.
#include "prsink_internal.h"

namespace prsink {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ constexpr bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};

// Fourth dword of a gfx9 raw buffer resource (32-bit data format).
constexpr int kBufferConfig = 0x00020000;
// A buffer offset beyond every range the kernels build (ranges stay < 2^31).
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ inline uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// One RoPE pair stored as two bf16 in a dword (element 0 in the low half).
__device__ inline uint32_t rotate_pair_bf16(uint32_t w, float2 cs) {
  const float x0 = __uint_as_float(w << 16);
  const float x1 = __uint_as_float(w & 0xffff0000u);
  return pack_bf16(x0 * cs.x - x1 * cs.y, x0 * cs.y + x1 * cs.x);
}

// n / d for the token ranges the host checked: multiply-high, or n itself when d == 1.
__device__ inline uint32_t div_magic(uint32_t n, uint32_t magic, uint32_t one) {
  return __umulhi(n, magic) + n * one;
}

// Where the cos/sin of RoPE pair `pair` live: band base offset, row stride
// (pairs per band) and which position component (0 t, 1 h, 2 w) indexes it.
struct PairTab {
  int base, stride, comp;
};

__device__ inline PairTab pair_tab(const AttnParams& p, int pair) {
  PairTab t;
  if (pair < p.np_t) {
    t.base = pair; t.stride = p.np_t; t.comp = 0;
  } else if (pair < p.np_t + p.np_h) {
    t.base = p.rope_h_off + pair - p.np_t; t.stride = p.np_h; t.comp = 1;
  } else {
    t.base = p.rope_w_off + pair - p.np_t - p.np_h; t.stride = p.np_w; t.comp = 2;
  }
  return t;
}

__device__ inline float2 pair_cs(const AttnParams& p, const PairTab& t, int tt, int y, int x) {
  const int pos = t.comp == 0 ? tt : (t.comp == 1 ? y : x);
  return p.rope[t.base + pos * t.stride];
}

__device__ inline void token_pos(const AttnParams& p, int n, int t_index, int& tt, int& y, int& x) {
  const int f = div_magic(n, p.magic_hw, p.one_hw), j = n - f * p.hw;
  y = div_magic(j, p.magic_w, p.one_w);
  x = j - y * p.lat_w;
  tt = t_index + f;
}

// Row r of a 64-row key tile lives at LDS row key_perm(r): bits 2 and 3 swapped.
__device__ inline int key_perm(int r) { return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Rotates 8 raw bf16 (4 pairs, starting at pair `pair0`) of one row at (tt, y, x).
__device__ inline bf16x8 rotate_chunk_generic(const AttnParams& p, uint4 w, int pair0, int tt,
                                              int y, int x) {
  uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) ws[e] = rotate_pair_bf16(ws[e], pair_cs(p, pair_tab(p, pair0 + e), tt, y, x));
  return __builtin_bit_cast(bf16x8, make_uint4(ws[0], ws[1], ws[2], ws[3]));
}

// XCD-aware tile order: consecutive workgroup ids land on different XCDs, so
// every XCD gets whole heads; the query tiles of a head then share that XCD's
// L2 while they stream the same keys.
__device__ inline bool map_workgroup(const AttnParams& p, int& head, int& qt) {
  const int wg = blockIdx.x;
  const int xcd = wg & 7, jx = wg >> 3;
  head = xcd + 8 * (jx / p.n_qtiles);
  qt = jx % p.n_qtiles;
  return head < p.n_heads;
}

// ---------------------------------------------------------------------------
// Generic bf16 kernel (any RoPE band split): 4 waves x 32 query rows, one
// 64-key tile staged per iteration through registers.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_bf16_generic(const AttnParams p) {
  constexpr int KT = kKeyTile;
  constexpr int QT = 128;
  constexpr int KS = D + 8;         // LDS K row stride (bf16 elements)
  constexpr int VS = KT + 8;        // LDS V^T row stride
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __align__(16) uint16_t Ks[KT * KS];
  __shared__ __align__(16) uint16_t Vs[D * VS];

  int head, qt;
  if (!map_workgroup(p, head, qt)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int H = p.n_heads;

  const int qrow = qt * QT + wave * 32 + l32;
  const bool qvalid = qrow < p.n_q;
  bf16x8 qreg[NC];
  {
    int tq = 0, yq = 0, xq = 0;
    if (qvalid) token_pos(p, qrow, p.q_t_index, tq, yq, xq);
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((size_t)qrow * H + head) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int off = 16 * c + 8 * hh;
      const uint4 w = qvalid ? *reinterpret_cast<const uint4*>(qp + off) : make_uint4(0, 0, 0, 0);
      qreg[c] = rotate_chunk_generic(p, w, off / 2, tq, yq, xq);
    }
  }

  constexpr int KCPR = D / 8;             // 16-byte chunks per key row
  constexpr int KROWS = 256 / KCPR;
  const int kcc = tid % KCPR;
  const int kr0 = tid / KCPR;

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  for (int s = 0; s < p.n_seg; ++s) {
    const Segment sg = p.seg[s];
    const int count = sg.count;
    const uint16_t* kbase = static_cast<const uint16_t*>(sg.k) + (size_t)head * sg.head;
    const uint16_t* vbase = static_cast<const uint16_t*>(sg.v) + (size_t)head * sg.head;
    for (int n0 = 0; n0 < count; n0 += KT) {
#pragma unroll
      for (int it = 0; it < KT / KROWS; ++it) {
        const int r = kr0 + it * KROWS;
        const int n = n0 + r;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (n < count) {
          int tt, y, x;
          token_pos(p, n, sg.t_index, tt, y, x);
          w = __builtin_bit_cast(uint4, rotate_chunk_generic(
              p, *reinterpret_cast<const uint4*>(kbase + (size_t)n * sg.tok + kcc * 8), kcc * 4, tt, y, x));
        }
        *reinterpret_cast<uint4*>(&Ks[key_perm(r) * KS + kcc * 8]) = w;
      }
      {  // V rows -> V^T in LDS
        const int key = tid % KT, cg = tid / KT;
        const int n = n0 + key;
#pragma unroll
        for (int it = 0; it < D / 32; ++it) {
          const int ch = cg + 4 * it;
          uint4 w = make_uint4(0, 0, 0, 0);
          if (n < count) w = *reinterpret_cast<const uint4*>(vbase + (size_t)n * sg.tok + ch * 8);
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            Vs[(ch * 8 + 2 * e) * VS + key] = (uint16_t)(ws[e] & 0xffffu);
            Vs[(ch * 8 + 2 * e + 1) * VS + key] = (uint16_t)(ws[e] >> 16);
          }
        }
      }
      __syncthreads();

      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb] = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + l32) * KS + c * 16 + hh * 8]);
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], sc[kb], 0, 0, 0);
        }
      }
      // register r of block kb holds key kb*32 + (r/8)*16 + hh*8 + r%8
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + kb * 32 + (r >> 3) * 16 + hh * 8 + (r & 7);
          const float v = key < count ? sc[kb][r] * sl2 : -INFINITY;
          sc[kb][r] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);  // finite: every tile has a valid key
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float rs = 0.f;
      bf16x8 pb[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        uint32_t pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(sc[kc >> 1][(kc & 1) * 8 + 2 * e] - m_new);
          const float p1 = __builtin_amdgcn_exp2f(sc[kc >> 1][(kc & 1) * 8 + 2 * e + 1] - m_new);
          rs += p0 + p1;
          pw[e] = pack_bf16(p0, p1);
        }
        pb[kc] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vs[(db * 32 + l32) * VS + kc * 16 + hh * 8]);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], o[db], 0, 0, 0);
        }
      __syncthreads();
    }
  }

  // register 4g+e of block db is dv = 32db + 8g + 4hh + e
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    uint16_t* op = static_cast<uint16_t*>(p.out) + ((size_t)qrow * H + head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint2 w = make_uint2(pack_bf16(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                   pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
        *reinterpret_cast<uint2*>(op + db * 32 + g * 8 + hh * 4) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// Fast bf16 kernel for the Wan-style band split (t = d - 4*floor(d/6), h = w =
// 2*floor(d/6)), the layout of every workload here.
//   * 4 waves x 64 query rows (two 32-row MFMA column blocks per wave): every
//     K and V operand read from LDS feeds two MFMAs.
//   * K and V tiles move global -> LDS by DMA (global_load_lds_dwordx4), no
//     registers in between.  LDS rows are padded (d=128: 304-byte stride, so
//     16 consecutive rows start 12 banks apart and the 16-byte operand reads
//     of a 16-lane phase cover all 64 banks once); every LDS address is then
//     a per-lane base plus an immediate.  DMA lanes that land in padding are
//     masked off.  The DMA for tile i+1 is issued before tile i is computed
//     (double-buffered LDS).
//   * Each wave rotates, in place, the 16 key rows its own DMA brought in
//     (RoPE follow), with cos/sin read from an LDS copy of the table.
//   * V stays row-major; the PV operand (V^T) comes from ds_read_b64_tr_b16,
//     which returns, within each 16-lane group, lane i element e = the value
//     lane 4e + i/4 points at, element i%4.
//   * Ragged tiles (the last of each segment) mask keys past the end in a
//     short uniform branch; the rest of the step is shared.
//   * Online softmax rescales lazily: the running max used for exp2 moves
//     only when a score exceeds it by more than 2^8, so probabilities stay
//     <= 256 and the O rescale is skipped on most tiles.
// ---------------------------------------------------------------------------
template <int D, int DT, int DH>
struct Bands {
  static constexpr int NPT = DT / 2, NPH = DH / 2, NPW = (D - DT - DH) / 2;
  static constexpr int band(int g) { return g < NPT ? 0 : (g < NPT + NPH ? 1 : 2); }
  static constexpr int start(int b) { return b == 0 ? 0 : (b == 1 ? NPT : NPT + NPH); }
};

template <int D, int DT, int DH>
struct FastAttn {
  using B = Bands<D, DT, DH>;
  static constexpr int KT = kKeyTile;    // keys per tile
  static constexpr int QT = 256;         // query rows per workgroup
  static constexpr int RB = D * 2;       // bytes per key row
  static constexpr int NS = RB / 16;     // 16-byte slots per row
  static constexpr int RBP = D == 128 ? RB + 48 : RB + 16;  // padded LDS row stride
  static constexpr int NU = RBP / 16;    // 16-byte units per padded row
  static constexpr int TILE = KT * RBP;  // bytes per K or V tile in LDS
  static constexpr int DMA_PER_WAVE = (16 * NU + 63) / 64;  // 1 KB DMA instructions per wave per tensor
  static constexpr int NC = D / 16;      // QK^T k-steps
  static constexpr int NDB = D / 32;     // dv blocks
  static constexpr int SPL = NS / 4;     // slots each lane rotates (a quarter of a row)
  static constexpr int PPL = SPL * 4;    // RoPE pairs each lane rotates
  // A tile whose partial row sum of probabilities exceeds this takes the slow
  // path (exact tile max, rescale).  Below it every probability is < 2^14.
  static constexpr float SUM_LIMIT = 16384.0f;

  const AttnParams& p;
  const char* tab;  // LDS: packed-bf16 rotation table
  int head, tid, lane, wave, hh, l32;
  float sl2;
  // rotation: this lane's row inside its wave's 16 rows, and the band pattern of its pairs
  int rot_row, rot_q, b0, b1, esplit, c0, c1;

  uint32_t voff_k[DMA_PER_WAVE], voff_v[DMA_PER_WAVE];

  bf16x8 qreg[2][NC];
  f32x16 o[2][NDB];
  float m_run[2], l_run[2];

  __device__ FastAttn(const AttnParams& p_, const char* tab_, int head_)
      : p(p_), tab(tab_), head(head_) {
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    hh = lane >> 5;
    l32 = lane & 31;
    sl2 = p.scale_log2;
    rot_row = wave * 16 + (lane >> 2);
    rot_q = lane & 3;
    const int g0 = rot_q * PPL;
    b0 = B::band(g0);
    b1 = B::band(g0 + PPL - 1);
    esplit = b0 == b1 ? PPL : B::start(b1) - g0;
    c0 = (g0 - B::start(b0)) * 8;
    c1 = (g0 - B::start(b1)) * 8;
    // DMA unit i*64 + lane of this wave's 16 padded rows -> (row, 16-byte slot)
    const uint32_t tok_bytes = (uint32_t)(p.n_heads * D * 2);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int u = i * 64 + lane;
      const int rr = u / NU, c = u - rr * NU;
      const int r = wave * 16 + rr;
      const bool data = rr < 16 && c < NS;
      voff_k[i] = data ? (uint32_t)key_perm(r) * tok_bytes + c * 16 : kOutOfRange;
      voff_v[i] = data ? (uint32_t)r * tok_bytes + c * 16 : kOutOfRange;
    }
  }

  __device__ void init_queries(int qt) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qrow = qt * QT + wave * 64 + qb * 32 + l32;
      const bool valid = qrow < p.n_q;
      int tq = 0, yq = 0, xq = 0;
      if (valid) token_pos(p, qrow, p.q_t_index, tq, yq, xq);
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((size_t)qrow * p.n_heads + head) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = 16 * c + 8 * hh;
        const uint4 w = valid ? *reinterpret_cast<const uint4*>(qp + off) : make_uint4(0, 0, 0, 0);
        qreg[qb][c] = rotate_chunk_generic(p, w, off / 2, tq, yq, xq);
      }
#pragma unroll
      for (int i = 0; i < NDB; ++i) o[qb][i] = f32x16{};
      m_run[qb] = -INFINITY;
      l_run[qb] = 0.f;
    }
  }

  // Queue the DMA of tile (s, n0) into LDS tiles kdst / vdst.  K row r holds
  // key n0 + key_perm(r), V row r holds key n0 + r; rows past the segment's
  // end repeat its last key (masked later, and always in bounds).  Wave w
  // fills exactly rows 16w .. 16w+15, the rows it rotates later, so its own
  // vmcnt wait covers every byte it reads back.
  //
  // The loads go through buffer resources whose range ends at the segment's
  // last token: rows past it read as zero, and no address outside a segment
  // is touched.  Per-lane byte offsets inside a tile are loop constants
  // (voff_k / voff_v); lanes that land in LDS row padding get an offset past
  // any range, so they write zeros there.
  __device__ __forceinline__ void dma_tile(char* kdst, char* vdst, int s, int n0) {
    const Segment& sg = p.seg[s];
    const size_t tok_bytes = (size_t)sg.tok * 2;
    const size_t off = (size_t)head * sg.head * 2 + (size_t)n0 * tok_bytes;
    const int nrec = (int)((size_t)(sg.count - n0) * tok_bytes);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(sg.k) + off), 0, nrec, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(sg.v) + off), 0, nrec, kBufferConfig);
    const int wbase = wave * 16 * RBP;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      if (i * 64 + 64 <= 16 * NU || i * 64 + lane < 16 * NU) {  // the wave's own 16 rows only
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(kdst + wbase + i * 1024),
                                                 16, voff_k[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(vdst + wbase + i * 1024),
                                                 16, voff_v[i], 0, 0, 0);
      }
    }
  }

  // Rotate, in place, the quarter-row of K this lane owns: for every pair,
  // (x0, x1) -> (x0 c - x1 s, x0 s + x1 c) as two v_dot2 with packed-bf16
  // (c, -s) and (s, c) from the LDS table.
  __device__ __forceinline__ void rotate_tile(char* kt, int s, int n0) {
    const Segment& sg = p.seg[s];
    const int n = min(n0 + key_perm(rot_row), sg.count - 1);
    int tt, y, x;
    token_pos(p, n, sg.t_index, tt, y, x);
    const int rt = tt * (B::NPT * 8);
    const int rh = p.rope_h_off * 8 + y * (B::NPH * 8);
    const int rw = p.rope_w_off * 8 + x * (B::NPW * 8);
    const int r0 = (b0 == 0 ? rt : (b0 == 1 ? rh : rw)) + c0;
    const int r1 = (b1 == 0 ? rt : (b1 == 1 ? rh : rw)) + c1;
    char* base = kt + rot_row * RBP + rot_q * SPL * 16;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const uint4 w = *reinterpret_cast<const uint4*>(base + 16 * i);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      uint32_t out[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pe = 4 * i + e;
        const uint2 cs = *reinterpret_cast<const uint2*>(tab + (pe < esplit ? r0 : r1) + 8 * pe);
        const bf16x2 xv = __builtin_bit_cast(bf16x2, ws[e]);
        const float y0 = __builtin_amdgcn_fdot2_f32_bf16(xv, __builtin_bit_cast(bf16x2, cs.x), 0.f, false);
        const float y1 = __builtin_amdgcn_fdot2_f32_bf16(xv, __builtin_bit_cast(bf16x2, cs.y), 0.f, false);
        out[e] = pack_bf16(y0, y1);
      }
      *reinterpret_cast<uint4*>(base + 16 * i) = make_uint4(out[0], out[1], out[2], out[3]);
    }
  }

  // S^T = K_rot Q_rot^T: [2 query blocks] x [2 key blocks] of 32x32
  __device__ __forceinline__ void qk(const char* kt, f32x16 (&sc)[2][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) { sc[qb][0] = f32x16{}; sc[qb][1] = f32x16{}; }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const char* kr = kt + l32 * RBP + hh * 16 + c * 32;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kr);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kr + 32 * RBP);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        sc[qb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[qb][c], sc[qb][0], 0, 0, 0);
        sc[qb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[qb][c], sc[qb][1], 0, 0, 0);
      }
    }
  }

  // Probabilities p = 2^(s*scale - m_run*scale) of query block qb packed to
  // bf16 (the PV B operand); returns this lane's partial sum of the packed
  // values, so the normaliser sums the same rounded weights the PV uses.
  __device__ __forceinline__ float probs(const f32x16 (&sq)[2], int qb, bf16x8 (&pq)[4]) {
    const float mb = m_run[qb] * sl2;
    float acc = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sq[kc >> 1][(kc & 1) * 8 + 2 * e], sl2, -mb));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sq[kc >> 1][(kc & 1) * 8 + 2 * e + 1], sl2, -mb));
        pw[e] = pack_bf16(p0, p1);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[e]), kOnes, acc, false);
      }
      pq[kc] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    }
    return acc;
  }

  // O^T += V^T P^T.  Lane (dv = 32db + l32, hh) needs keys 16kc + 8hh + j, j = 0..7:
  // two transpose reads; in each, lane 4e + q of a 16-lane group points at
  // row 16kc + 8hh + 4rd + e, dims 32db + 16*(group&1) + 4q .. +3.
  __device__ __forceinline__ void pv(const char* vt, const bf16x8 (&pb)[2][4]) {
    const int grp = lane >> 4, i16 = lane & 15;
    const char* vl = vt + (8 * hh + (i16 >> 2)) * RBP + (16 * (grp & 1) + 4 * (i16 & 3)) * 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
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

  // Full tile against the fixed running max, branch-free.  Returns true (for
  // the whole wave) when some probability reached SUM_LIMIT or is not finite;
  // the workgroup then recomputes everything with step_exact.
  __device__ __forceinline__ bool step_fast(const char* kt, const char* vt) {
    f32x16 sc[2][2];
    qk(kt, sc);
    bf16x8 pb[2][4];
    const float r0 = probs(sc[0], 0, pb[0]);
    const float r1 = probs(sc[1], 1, pb[1]);
    l_run[0] += r0;
    l_run[1] += r1;
    pv(vt, pb);
    return __any(!(r0 <= SUM_LIMIT) | !(r1 <= SUM_LIMIT));
  }

  // Any tile, exact online softmax: keys past `count` are masked, the running
  // max follows the tile max and O and the normaliser are rescaled.
  __device__ __forceinline__ void step_exact(const char* kt, const char* vt, int n0, int count) {
    f32x16 sc[2][2];
    qk(kt, sc);
    // register r of key block kb holds key kb*32 + (r/8)*16 + hh*8 + r%8
    const int lim = count - n0 - hh * 8;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + (r >> 3) * 16 + (r & 7) >= lim) sc[qb][kb][r] = -INFINITY;
    bf16x8 pb[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float m = sc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, sc[qb][kb][r]);
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      const float m_new = fmaxf(m_run[qb], m);  // finite: every tile has a valid key
      const float alpha = __builtin_amdgcn_exp2f((m_run[qb] - m_new) * sl2);
      m_run[qb] = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[qb][db] *= alpha;
      l_run[qb] = l_run[qb] * alpha + probs(sc[qb], qb, pb[qb]);
    }
    pv(vt, pb);
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

  __device__ void epilogue(int qt) {
    // register 4g+e of dv block db is dv = 32db + 8g + 4hh + e
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qrow = qt * QT + wave * 64 + qb * 32 + l32;
      const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
      const float inv = 1.0f / l_tot;
      if (qrow < p.n_q) {
        uint16_t* op = static_cast<uint16_t*>(p.out) + ((size_t)qrow * p.n_heads + head) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint2 w = make_uint2(pack_bf16(o[qb][db][4 * g] * inv, o[qb][db][4 * g + 1] * inv),
                                       pack_bf16(o[qb][db][4 * g + 2] * inv, o[qb][db][4 * g + 3] * inv));
            *reinterpret_cast<uint2*>(op + db * 32 + g * 8 + hh * 4) = w;
          }
      }
    }
  }
};

__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x3f70); }  // vmcnt(0)

// Next full 64-key tile after (s, n0); returns false past the last one.
__device__ inline bool next_full(const AttnParams& p, int& s, int& n0) {
  n0 += kKeyTile;
  if (n0 + kKeyTile > p.seg[s].count) {
    ++s;
    n0 = 0;
    while (s < p.n_seg && p.seg[s].count < kKeyTile) ++s;
  }
  return s < p.n_seg;
}

template <int D, int DT, int DH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_fast(const AttnParams p) {
  using F = FastAttn<D, DT, DH>;
  // Two K and two V tiles as distinct objects: the compiler can then tell the
  // DMA into one buffer from the reads of the other and does not wait on it.
  __shared__ __align__(16) char k0[F::TILE];
  __shared__ __align__(16) char k1[F::TILE];
  __shared__ __align__(16) char v0[F::TILE];
  __shared__ __align__(16) char v1[F::TILE];
  extern __shared__ __align__(16) char rope_lds[];

  int head, qt;
  if (!map_workgroup(p, head, qt)) return;

  // packed-bf16 rotation table -> LDS (read by the key rotation of every tile)
  {
    const int n16 = (p.rope_bytes + 15) >> 4;
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p.rope) + p.rope_bytes);
    for (int i = threadIdx.x; i < n16; i += 256) reinterpret_cast<uint4*>(rope_lds)[i] = src[i];
  }
  F a(p, rope_lds, head);
  // Full 64-key tiles go through the pipelined fast loop; the ragged last tile
  // of each segment (and, after an overflow, everything) through exact steps.
  // Tile order does not change the softmax result.
  __shared__ int ovf[2][4];  // per-wave overflow flags, one set per unrolled half
  int s = 0;
  while (s < p.n_seg && p.seg[s].count < F::KT) ++s;
  const bool have_full = s < p.n_seg;
  if (have_full) a.dma_tile(k0, v0, s, 0);
  a.init_queries(qt);
  wait_dma();
  __syncthreads();  // the table and the first tile are in LDS
  bool overflow = false;
  if (have_full) {
    a.rotate_tile(k0, s, 0);
    __syncthreads();
    int s1 = s, n1 = 0;
    bool more = next_full(p, s1, n1);
    if (more) a.dma_tile(k1, v1, s1, n1);
    a.step_exact(k0, v0, 0, p.seg[s].count);  // sets the running max
    if (more) {
      wait_dma();
      a.rotate_tile(k1, s1, n1);
      __syncthreads();
      more = next_full(p, s1, n1);
      while (true) {
        if (more) a.dma_tile(k0, v0, s1, n1);
        ovf[0][a.wave] = a.step_fast(k1, v1);
        if (more) {
          wait_dma();
          a.rotate_tile(k0, s1, n1);
        }
        __syncthreads();
        if (ovf[0][0] | ovf[0][1] | ovf[0][2] | ovf[0][3]) { overflow = true; break; }
        if (!more) break;
        more = next_full(p, s1, n1);

        if (more) a.dma_tile(k1, v1, s1, n1);
        ovf[1][a.wave] = a.step_fast(k0, v0);
        if (more) {
          wait_dma();
          a.rotate_tile(k1, s1, n1);
        }
        __syncthreads();
        if (ovf[1][0] | ovf[1][1] | ovf[1][2] | ovf[1][3]) { overflow = true; break; }
        if (!more) break;
        more = next_full(p, s1, n1);
      }
    }
    __syncthreads();
  }
  // Exact, single-buffered passes: the ragged tiles, or every tile again after
  // an overflow (rare: a score more than 14 powers of two above the first tile's max).
  if (overflow) a.reset_accumulators();
  for (int ss = 0; ss < p.n_seg; ++ss) {
    const int cnt = p.seg[ss].count;
    for (int nn = overflow ? 0 : cnt - cnt % F::KT; nn < cnt; nn += F::KT) {
      a.dma_tile(k0, v0, ss, nn);
      wait_dma();
      a.rotate_tile(k0, ss, nn);
      __syncthreads();
      a.step_exact(k0, v0, nn, cnt);
      __syncthreads();
    }
  }
  a.epilogue(qt);
}

// ---------------------------------------------------------------------------
// fp32: one query row per lane, 64-key tiles staged (rotated) in LDS.
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
    if (qvalid) token_pos(p, qrow, p.q_t_index, tq, yq, xq);
    const float* qp = static_cast<const float*>(p.q) + ((size_t)qrow * H + head) * D;
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      float x0 = 0.f, x1 = 0.f;
      if (qvalid) { x0 = qp[2 * i]; x1 = qp[2 * i + 1]; }
      const float2 cs = pair_cs(p, pair_tab(p, i), tq, yq, xq);
      q[2 * i] = x0 * cs.x - x1 * cs.y;
      q[2 * i + 1] = x0 * cs.y + x1 * cs.x;
    }
  }
  float o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int s = 0; s < p.n_seg; ++s) {
    const Segment sg = p.seg[s];
    const int count = sg.count;
    const float* kbase = static_cast<const float*>(sg.k) + (size_t)head * sg.head;
    const float* vbase = static_cast<const float*>(sg.v) + (size_t)head * sg.head;
    for (int n0 = 0; n0 < count; n0 += KT) {
      for (int id = lane; id < KT * (D / 2); id += KT) {
        const int r = id / (D / 2), pr = id % (D / 2);
        const int n = n0 + r;
        float y0 = 0.f, y1 = 0.f;
        if (n < count) {
          const float x0 = kbase[(size_t)n * sg.tok + 2 * pr];
          const float x1 = kbase[(size_t)n * sg.tok + 2 * pr + 1];
          int tt, y, x;
          token_pos(p, n, sg.t_index, tt, y, x);
          const float2 cs = pair_cs(p, pair_tab(p, pr), tt, y, x);
          y0 = x0 * cs.x - x1 * cs.y;
          y1 = x0 * cs.y + x1 * cs.x;
        }
        Ks[r][2 * pr] = y0;
        Ks[r][2 * pr + 1] = y1;
      }
      for (int id = lane; id < KT * D; id += KT) {
        const int r = id / D, dv = id % D;
        const int n = n0 + r;
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

}  // namespace

hipError_t launch_attention(const AttnParams& p_in, int dtype, int head_dim, hipStream_t s) {
  AttnParams p = p_in;
  const int heads_per_xcd = (p.n_heads + 7) / 8;
  if (dtype == 0) {  // bf16
    // the fast kernel's buffer ranges are 31-bit byte counts
    size_t max_seg_bytes = 0;
    for (int i = 0; i < p.n_seg; ++i) {
      const size_t b = (size_t)p.seg[i].count * p.seg[i].tok * 2;
      if (b > max_seg_bytes) max_seg_bytes = b;
    }
    const bool wan = p.np_h == p.np_w && p.np_h == head_dim / 6 && p.rope_bytes <= kMaxRopeLdsBytes &&
                     max_seg_bytes < (size_t)kOutOfRange;
    if (wan && (head_dim == 128 || head_dim == 64)) {
      p.n_qtiles = (p.n_q + 255) / 256;
      const dim3 grid(8 * heads_per_xcd * p.n_qtiles);
      const size_t lds = ((size_t)p.rope_bytes + 15) / 16 * 16;
      if (head_dim == 128)
        hipLaunchKernelGGL((attn_bf16_fast<128, 44, 42>), grid, dim3(256), lds, s, p);
      else
        hipLaunchKernelGGL((attn_bf16_fast<64, 24, 20>), grid, dim3(256), lds, s, p);
    } else {
      p.n_qtiles = (p.n_q + 127) / 128;
      const dim3 grid(8 * heads_per_xcd * p.n_qtiles);
      if (head_dim == 128)
        hipLaunchKernelGGL(attn_bf16_generic<128>, grid, dim3(256), 0, s, p);
      else
        hipLaunchKernelGGL(attn_bf16_generic<64>, grid, dim3(256), 0, s, p);
    }
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
