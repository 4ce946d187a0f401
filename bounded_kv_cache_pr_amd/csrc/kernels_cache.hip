// Cache-maintenance kernels of the PR-Sink path on gfx950:
//   kv_write     raw K/V [T][H][d] -> slot layout [t_pad][H][d] (contiguous copy)
//   clean_write  the same for a closing block's clean K/V, plus its keys
//                rotated at every window place they will take
//   rope_follow  raw keys -> keys rotated at a segment's current positions
//   slot_copy    the first bytes of a block slot (all layers) -> another slot;
//                source and destination come from device state, so no host
//                round trip
//   retrieve     fingerprint l2-normalisation + argmax over the bank (fp64)
//   bank_update  exhaustive diversity replacement (fp64)
#include "prsink_device.h"

namespace prsink {
namespace {

// Streaming 16-byte accesses (the nt bit) in the copies and the clean write:
// each byte is read or written once per launch, so none of them should evict
// from L2 the keys that attention running beside them streams; on copies much
// larger than the L2 they also moved more bytes per second than plain
// accesses, with one chunk per thread and loop iteration.  (rope_follow keeps
// plain accesses: the current keys it rotates are read right back by the
// attention kernel.)
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(uint4* p, uint4 w) {
  const u32x4_nt v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_nt*>(p));
}

// ---------------------------------------------------------------------------
// kv_write: raw K and V [T][H][d] -> slot layout [t_pad][H][d] (the same
// token-major order, so a contiguous copy), optionally to a second
// destination.  Rows past T (the slot's padding) are never written and stay
// zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint4* __restrict__ k_src, const uint4* __restrict__ v_src, uint4* __restrict__ k_dst0,
    uint4* __restrict__ v_dst0, uint4* __restrict__ k_dst1, uint4* __restrict__ v_dst1,
    size_t n_chunks) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_chunks; i += stride) {
    const uint4 kv = ld_nt(k_src + i), vv = ld_nt(v_src + i);
    st_nt(k_dst0 + i, kv);
    st_nt(v_dst0 + i, vv);
    if (k_dst1) {
      st_nt(k_dst1 + i, kv);
      st_nt(v_dst1 + i, vv);
    }
  }
}

// ---------------------------------------------------------------------------
// slot_copy: grid-stride 16-byte copy of copy_bytes at byte offset copy_off of
// one block slot to the same place in another.  Reads the (source,
// destination) pair from device state; a negative source means there is
// nothing to copy.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void slot_copy_kernel(uint8_t* __restrict__ base,
                                                        size_t slot_bytes, size_t copy_off, size_t copy_bytes,
                                                        const DevState* __restrict__ st) {
  const int src = st->copy_src, dst = st->copy_dst;
  if (src < 0 || src == dst) return;
  const uint4* __restrict__ s = reinterpret_cast<const uint4*>(base + (size_t)src * slot_bytes + copy_off);
  uint4* __restrict__ d = reinterpret_cast<uint4*>(base + (size_t)dst * slot_bytes + copy_off);
  const size_t n = copy_bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) st_nt(d + i, ld_nt(s + i));
}

// ---------------------------------------------------------------------------
// rope_follow: RoPE follow for cached keys.  The cache keeps each block's keys
// rotated at the positions of every place it takes, computed from the raw
// keys (kept for the Ref Sink and the window blocks, whose later rotations
// read them): this kernel rotates the Ref Sink at set-up, a bank entry at the
// Dynamic Sink's place when written, and the current block's keys at the
// current positions on every call (clean_write rotates the window and Static
// places) (review on
// paper.rainbus.top, full-pipeline paragraph: raw keys re-rotated at their
// current cache positions; novelty paragraph: position-consistent reuse).
// Pair (x0, x1) at angle a becomes (x0 cos a - x1 sin a, x0 sin a + x1 cos a),
// in fp32, rounded once to the cache dtype; cos a and sin a come from the
// place's [token][pair] table, one 32-byte (bf16) or 16-byte (fp32) read per
// 16-byte chunk.  Thread = one 16-byte chunk (4 bf16 pairs or 2 fp32 pairs) of
// one token and head; grid = (chunks, layer, job).
// ---------------------------------------------------------------------------
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Token of chunk i and the chunk's first RoPE pair within the head.
__device__ __forceinline__ void chunk_place(const ChunkDiv& d, uint32_t i, int elem, uint32_t& n, uint32_t& pair) {
  n = d.exact ? __umulhi(i, d.magic) : i / d.per_tok;
  const uint32_t per_head = (uint32_t)d.np * 4 / 16 * (elem == 2 ? 1 : 2);  // chunks per head row (a power of 2)
  pair = (i & (per_head - 1)) * (elem == 2 ? 4 : 2);
}

// Chunk w of a head row rotated with the table entries at cs (4 pairs in bf16,
// 2 in fp32).
__device__ __forceinline__ uint4 rotate_chunk(uint4 w, const float2* __restrict__ cs, int elem) {
  if (elem == 2) {
    const float4 c01 = *reinterpret_cast<const float4*>(cs), c23 = *reinterpret_cast<const float4*>(cs + 2);
    const float cx[4] = {c01.x, c01.z, c23.x, c23.z}, sx[4] = {c01.y, c01.w, c23.y, c23.w};
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf16_lo(ws[e]), x1 = bf16_hi(ws[e]);
      ws[e] = pack_bf16(x0 * cx[e] - x1 * sx[e], x0 * sx[e] + x1 * cx[e]);
    }
    return make_uint4(ws[0], ws[1], ws[2], ws[3]);
  }
  const float4 c01 = *reinterpret_cast<const float4*>(cs);
  const float cx[2] = {c01.x, c01.z}, sx[2] = {c01.y, c01.w};
  float f[4] = {__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w)};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float x0 = f[2 * e], x1 = f[2 * e + 1];
    f[2 * e] = x0 * cx[e] - x1 * sx[e];
    f[2 * e + 1] = x0 * sx[e] + x1 * cx[e];
  }
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

__global__ __launch_bounds__(256) void rope_follow_kernel(const RotParams p) {
  const RotJob& jb = p.job[blockIdx.z];
  const size_t lay = (size_t)blockIdx.y * p.layer_bytes;
  const char* __restrict__ src = jb.src + lay;
  char* __restrict__ dst;
  if (jb.from_state) {
    const int cs = p.st->copy_src, cd = p.st->copy_dst;
    if (cs < 0) return;
    dst = p.block_base + (size_t)cd * p.slot_bytes + jb.dst_off + lay;
  } else {
    dst = jb.dst + lay;
  }
  const uint32_t total = p.cd.per_tok * (uint32_t)p.n_tok;
  const uint32_t stride = gridDim.x * 256;
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const uint4 w = reinterpret_cast<const uint4*>(src)[i];
    uint32_t n, pair;
    chunk_place(p.cd, i, p.elem, n, pair);
    reinterpret_cast<uint4*>(dst)[i] = rotate_chunk(w, jb.cs + (size_t)n * p.cd.np + pair, p.elem);
  }
}

// ---------------------------------------------------------------------------
// clean_write: the clean K/V of one layer of the block being closed go to its
// window slot, raw, together with its keys rotated at every window place the
// block takes while it stays in the window (newest first); for block 0 the V
// also goes to the Static Sink, with the keys rotated at its place (a
// destination without k keeps no raw keys).
// One pass reads the clean keys once, and no key is rotated again when the
// window slides.  Thread = one 16-byte chunk of K and of V.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void clean_write_kernel(const CleanWrite p) {
  const uint32_t total = p.cd.per_tok * (uint32_t)p.n_tok;
  const uint32_t stride = gridDim.x * 256;
  const uint4* __restrict__ ks = reinterpret_cast<const uint4*>(p.k_src);
  const uint4* __restrict__ vs = reinterpret_cast<const uint4*>(p.v_src);
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const uint4 k = ld_nt(ks + i), v = ld_nt(vs + i);
    uint32_t n, pair;
    chunk_place(p.cd, i, p.elem, n, pair);
    const size_t e = (size_t)n * p.cd.np + pair;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const CleanDst& o = p.dst[d];
      if (!o.v) continue;
      if (o.k) st_nt(reinterpret_cast<uint4*>(o.k) + i, k);
      st_nt(reinterpret_cast<uint4*>(o.v) + i, v);
#pragma unroll
      for (int r = 0; r < kMaxRot; ++r) {
        if (r >= o.n_rot) break;
        st_nt(reinterpret_cast<uint4*>(o.k_rot[r]) + i, rotate_chunk(k, o.cs[r] + e, p.elem));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fingerprint arithmetic (fp64).  Every squared norm and dot product is the
// plain sum of the rounded products in index order, k = 0, 1, 2, ..., with no
// fused multiply-add: one lane per sum.  That is the definition itself, so any
// implementation that adds in the same order gets the same bits, and the
// retrieval and bank decisions never depend on how a reduction was split.
// ---------------------------------------------------------------------------
// The vectors stream through LDS in chunks of kChunk elements, staged by the
// whole wave, so each lane's sequential sum reads LDS rather than waiting on a
// global load per element; the order of the additions is unchanged.
constexpr int kChunk = 256;
constexpr int kPerLane = kChunk / 64;

// Rows [0, n_rows) of `rows` (row i at rows + i * n), elements [k0, k0+len),
// into lds (row i at lds + i * kChunk).  Every lane issues all its loads
// before its first LDS store, so the loads overlap.
__device__ __forceinline__ void stage_rows(double* __restrict__ lds, const double* __restrict__ rows, int n_rows,
                                           size_t n, int k0, int len, int lane) {
  double v[kMaxBank + 1][kPerLane];
#pragma unroll
  for (int i = 0; i < kMaxBank + 1; ++i)
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const int k = lane + 64 * e;
      v[i][e] = i < n_rows && k < len ? rows[(size_t)i * n + k0 + k] : 0.0;
    }
#pragma unroll
  for (int i = 0; i < kMaxBank + 1; ++i)
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) {
      const int k = lane + 64 * e;
      if (i < n_rows && k < len) lds[i * kChunk + k] = v[i][e];
    }
}

// acc + x[0] y[0] + x[1] y[1] + ... + x[len-1] y[len-1], added one by one in
// that order; eight elements are read (and multiplied) ahead of their adds.
__device__ __forceinline__ double seq_dot_acc(double acc, const double* __restrict__ x, const double* __restrict__ y,
                                              int len) {
#pragma clang fp contract(off)
  int k = 0;
  for (; k + 8 <= len; k += 8) {
    double pr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pr[j] = x[k + j] * y[k + j];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = acc + pr[j];
  }
  for (; k < len; ++k) acc = acc + x[k] * y[k];
  return acc;
}

// Fingerprint + retrieval, one wave64.  Entries fill the bank in slot order
// (id -1 = empty).
__global__ __launch_bounds__(64) void retrieve_kernel(const float* __restrict__ fp_raw,
                                                      double* __restrict__ phi_cur,
                                                      const double* __restrict__ bank_phi,
                                                      DevState* __restrict__ st, int fp_dim,
                                                      const BankRule rule, int block,
                                                      int32_t* slot_out) {
#pragma clang fp contract(off)
  __shared__ double lds[(kMaxBank + 1) * kChunk];
  __shared__ double score[kMaxBank];
  const int lane = threadIdx.x;
  const int M = rule.size;
  // ||x||^2 as an index-order sum (lane 0; the chunks go through LDS), the
  // correctly rounded square root, one correctly rounded division per
  // element; zero stays zero
  double ss = 0.0;
  for (int k0 = 0; k0 < fp_dim; k0 += kChunk) {
    const int len = min(kChunk, fp_dim - k0);
    float v[kPerLane];
#pragma unroll
    for (int e = 0; e < kPerLane; ++e) v[e] = lane + 64 * e < len ? fp_raw[k0 + lane + 64 * e] : 0.0f;
#pragma unroll
    for (int e = 0; e < kPerLane; ++e)
      if (lane + 64 * e < len) lds[lane + 64 * e] = (double)v[e];
    __syncthreads();
    if (lane == 0) ss = seq_dot_acc(ss, lds, lds, len);
    __syncthreads();
  }
  if (lane == 0) lds[0] = ss;
  __syncthreads();
  ss = lds[0];
  __syncthreads();
  const double nrm = sqrt(ss);
  for (int k = lane; k < fp_dim; k += 64) {
    const double x = (double)fp_raw[k];
    phi_cur[k] = nrm > 0.0 ? x / nrm : 0.0;
  }
  __syncthreads();  // phi_cur is read back below by other lanes
  // score of entry s by lane s: phi_cur . phi_s, in index order (phi_cur
  // staged as row M)
  const bool active = lane < M && st->ids[lane] >= 0;
  double acc = 0.0;
  for (int k0 = 0; k0 < fp_dim; k0 += kChunk) {
    const int len = min(kChunk, fp_dim - k0);
    stage_rows(lds, bank_phi, M, fp_dim, k0, len, lane);
    stage_rows(lds + M * kChunk, phi_cur, 1, fp_dim, k0, len, lane);
    __syncthreads();
    if (active) acc = seq_dot_acc(acc, lds + M * kChunk, lds + lane * kChunk, len);
    __syncthreads();
  }
  if (active) score[lane] = acc;
  __syncthreads();
  if (lane != 0) return;
  // r(b) = argmax over entries whose id != b-1; strict '>' keeps the lowest
  // slot on ties.  best: over every entry (the gated refresh's distance).
  const bool undetected = nrm == 0.0 && (rule.policy & kBankZeroFallback);
  int r = -1;
  double best_r = 0.0, best = -INFINITY;
  for (int s = 0; s < M; ++s) {
    if (st->ids[s] < 0) continue;
    const double sc = score[s];
    best = fmax(best, sc);
    if (st->ids[s] == block - 1 || undetected) continue;
    if (r < 0 || sc > best_r) { r = s; best_r = sc; }
  }
  // the Dynamic Sink of this block is bank entry r (none if r < 0)
  st->last_r = r;
  st->dyn_id = r >= 0 ? st->ids[r] : -1;
  if (r >= 0) st->last_used[r] = block;
  st->phi_zero = nrm == 0.0;
  st->best = best;
  if (slot_out) *slot_out = r;
}

// Diversity bank update, one wave64.  The fill phase (block < fill_blocks)
// inserts while there is room and then swaps by exhaustive search; later
// blocks update only under the CONTINUAL (stale entries may go) or GATED
// (far fingerprint: full search) policies.  A zero fingerprint under
// ZERO_FALLBACK is never written.
__global__ __launch_bounds__(64) void bank_update_kernel(const double* __restrict__ phi_cur,
                                                         double* __restrict__ bank_phi,
                                                         DevState* __restrict__ st, int fp_dim,
                                                         const BankRule rule, int block,
                                                         int win_slot, int bank_slot0) {
#pragma clang fp contract(off)
  __shared__ double lds[(kMaxBank + 1) * kChunk];
  __shared__ double G[kMaxBank][kMaxBank];  // pairwise dots of the bank, i < j
  __shared__ double g[kMaxBank];            // dots with the candidate
  const int lane = threadIdx.x;
  const int M = rule.size;
  int count = 0;
  while (count < M && st->ids[count] >= 0) ++count;
  const bool filling = block < rule.fill_blocks;
  const bool refresh = filling || ((rule.policy & kBankGated) && st->best < rule.refresh_tau);
  int dec;  // -1 keep, j = entry to write
  if (st->phi_zero && (rule.policy & kBankZeroFallback)) {
    dec = -1;
  } else if (count < M) {
    dec = count;
  } else {
    // one lane per dot product, each an index-order sum: lanes 0..M-1 the
    // candidate (row M of the staged rows) against entry i, the next
    // M(M-1)/2 lanes the pairs (i, j), i < j, in lexicographic order (at
    // most 8 + 28 < 64 lanes)
    int ia = 0, ib = 0;
    bool active = true;
    if (lane < M) {
      ia = M;
      ib = lane;
    } else {
      int t = lane - M;
      active = false;
      for (int i = 0; i < M; ++i)
        for (int j = i + 1; j < M; ++j, --t)
          if (t == 0) {
            ia = i;
            ib = j;
            active = true;
          }
    }
    double acc = 0.0;
    for (int k0 = 0; k0 < fp_dim; k0 += kChunk) {
      const int len = min(kChunk, fp_dim - k0);
      stage_rows(lds, bank_phi, M, fp_dim, k0, len, lane);
      stage_rows(lds + M * kChunk, phi_cur, 1, fp_dim, k0, len, lane);
      __syncthreads();
      if (active) acc = seq_dot_acc(acc, lds + ia * kChunk, lds + ib * kChunk, len);
      __syncthreads();
    }
    if (active) {
      if (lane < M) g[lane] = acc;
      else G[ia][ib] = acc;
    }
    __syncthreads();
    const double npairs = (double)(M * (M - 1) / 2);
    // mean pairwise similarity of an option, summed over pairs in slot order
    double tot = 0.0;
    for (int i = 0; i < M; ++i)
      for (int j = i + 1; j < M; ++j) tot = tot + G[i][j];
    double best = tot / npairs;
    dec = -1;
    for (int x = 0; x < M; ++x) {
      const bool evictable = refresh || ((rule.policy & kBankContinual) &&
                                         block - st->last_used[x] >= rule.stale_blocks);
      if (!evictable) continue;
      double t = 0.0;
      for (int i = 0; i < M; ++i)
        for (int j = i + 1; j < M; ++j) t = t + ((i == x) ? g[j] : (j == x) ? g[i] : G[i][j]);
      const double sx = t / npairs;
      if (sx < best) { best = sx; dec = x; }
    }
  }
  if (dec >= 0) {
    for (int k = lane; k < fp_dim; k += 64) bank_phi[(size_t)dec * fp_dim + k] = phi_cur[k];
  }
  if (lane == 0) {
    st->decision = dec;
    if (dec >= 0) {
      st->ids[dec] = block;
      st->last_used[dec] = block;
      st->copy_src = win_slot;
      st->copy_dst = bank_slot0 + dec;
    } else {
      st->copy_src = -1;
    }
  }
}

__global__ void state_init_kernel(DevState* st) {
  const int i = threadIdx.x;
  if (i < kMaxBank) {
    st->ids[i] = -1;
    st->last_used[i] = -1;
  }
  if (i == 0) {
    st->phi_zero = 0;
    st->best = -INFINITY;
    st->last_r = -1;
    st->dyn_id = -1;
    st->decision = -2;
    st->copy_src = -1;
    st->copy_dst = -1;
  }
}

}  // namespace

hipError_t launch_kv_write(const void* k_src, const void* v_src, void* k_dst0, void* v_dst0,
                           void* k_dst1, void* v_dst1, size_t bytes, hipStream_t s) {
  const size_t n_chunks = bytes / 16;
  size_t blocks = (n_chunks + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
                     static_cast<uint4*>(k_dst0), static_cast<uint4*>(v_dst0),
                     static_cast<uint4*>(k_dst1), static_cast<uint4*>(v_dst1), n_chunks);
  return hipGetLastError();
}

hipError_t launch_rope_follow(const RotParams& p, int n_layers, hipStream_t s) {
  const size_t total = (size_t)p.n_tok * p.n_heads * p.head_dim * p.elem / 16;
  size_t blocks = (total + 255) / 256;
  const size_t cap = n_layers * p.n_jobs > 8 ? 512 : 4096;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(rope_follow_kernel, dim3((unsigned)blocks, (unsigned)n_layers, (unsigned)p.n_jobs),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_clean_write(const CleanWrite& p, hipStream_t s) {
  const size_t total = (size_t)p.n_tok * p.n_heads * p.head_dim * p.elem / 16;
  size_t blocks = (total + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  hipLaunchKernelGGL(clean_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_slot_copy(char* block_base, size_t slot_bytes, size_t copy_off, size_t copy_bytes,
                            const DevState* st, hipStream_t s) {
  const size_t n16 = copy_bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 128) blocks = 256 * 128;
  hipLaunchKernelGGL(slot_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint8_t*>(block_base), slot_bytes, copy_off, copy_bytes, st);
  return hipGetLastError();
}

hipError_t launch_retrieve(const float* fp_raw, double* phi_cur, const double* bank_phi,
                           DevState* st, int fp_dim, const BankRule& rule, int block, int32_t* slot_out,
                           hipStream_t s) {
  hipLaunchKernelGGL(retrieve_kernel, dim3(1), dim3(64), 0, s, fp_raw, phi_cur, bank_phi, st,
                     fp_dim, rule, block, slot_out);
  return hipGetLastError();
}

hipError_t launch_bank_update(const double* phi_cur, double* bank_phi, DevState* st, int fp_dim,
                              const BankRule& rule, int block, int win_slot, int bank_slot0,
                              hipStream_t s) {
  hipLaunchKernelGGL(bank_update_kernel, dim3(1), dim3(64), 0, s, phi_cur, bank_phi, st, fp_dim,
                     rule, block, win_slot, bank_slot0);
  return hipGetLastError();
}

hipError_t launch_state_init(DevState* st, hipStream_t s) {
  hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(64), 0, s, st);
  return hipGetLastError();
}

}  // namespace prsink
