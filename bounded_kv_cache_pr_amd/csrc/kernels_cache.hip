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

// Streaming 16-byte accesses (the nt bit): what the clean write and the bank
// copy read is read once, and what they write is read back only blocks later,
// so neither should evict from L2 the keys that attention running beside them
// streams.
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
    const uint4 kv = k_src[i], vv = v_src[i];
    k_dst0[i] = kv;
    v_dst0[i] = vv;
    if (k_dst1) { k_dst1[i] = kv; v_dst1[i] = vv; }
  }
}

// ---------------------------------------------------------------------------
// slot_copy: grid-stride 16-byte copy of the first copy_bytes of one block
// slot to another.  Reads the (source, destination) pair from device state; a
// negative source means there is nothing to copy.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void slot_copy_kernel(uint8_t* __restrict__ base,
                                                        size_t slot_bytes, size_t copy_bytes,
                                                        const DevState* __restrict__ st) {
  const int src = st->copy_src, dst = st->copy_dst;
  if (src < 0 || src == dst) return;
  const uint4* __restrict__ s = reinterpret_cast<const uint4*>(base + (size_t)src * slot_bytes);
  uint4* __restrict__ d = reinterpret_cast<uint4*>(base + (size_t)dst * slot_bytes);
  const size_t n = copy_bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = ld_nt(s + i), b = ld_nt(s + i + stride), c = ld_nt(s + i + 2 * stride),
                e = ld_nt(s + i + 3 * stride);
    st_nt(d + i, a);
    st_nt(d + i + stride, b);
    st_nt(d + i + 2 * stride, c);
    st_nt(d + i + 3 * stride, e);
  }
  for (; i < n; i += stride) st_nt(d + i, ld_nt(s + i));
}

// ---------------------------------------------------------------------------
// rope_follow: RoPE follow for cached keys.  The cache keeps every key raw,
// and keeps a copy rotated at the positions of each place a block takes: this
// kernel rotates the Ref Sink at set-up, a bank entry at the Dynamic Sink's
// place when written, and the current block's keys at the current positions
// on every call (clean_write rotates the window and Static places) (review on
// paper.rainbus.top, full-pipeline paragraph: raw keys re-rotated at their
// current cache positions; novelty paragraph: position-consistent reuse).
// Pair (x0, x1) of a band at angle a becomes (x0 cos a - x1 sin a,
// x0 sin a + x1 cos a), in fp32, rounded once to the cache dtype.
// Thread = one 16-byte chunk (4 bf16 pairs or 2 fp32 pairs) of one token and
// head; grid = (chunks, layer, job).
// ---------------------------------------------------------------------------
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Chunk c (16 bytes: 4 bf16 pairs or 2 fp32 pairs) of one head row of a key
// at position (tt, y, x), rotated.
__device__ inline uint4 rotate_chunk(const RopeGeom& g, uint4 w, uint32_t c, int elem, int tt, int y, int x) {
  if (elem == 2) {
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 cs = rope_cs(g, (int)c * 4 + e, tt, y, x);
      const float x0 = bf16_lo(ws[e]), x1 = bf16_hi(ws[e]);
      ws[e] = pack_bf16(x0 * cs.x - x1 * cs.y, x0 * cs.y + x1 * cs.x);
    }
    return make_uint4(ws[0], ws[1], ws[2], ws[3]);
  }
  float f[4] = {__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w)};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float2 cs = rope_cs(g, (int)c * 2 + e, tt, y, x);
    const float x0 = f[2 * e], x1 = f[2 * e + 1];
    f[2 * e] = x0 * cs.x - x1 * cs.y;
    f[2 * e + 1] = x0 * cs.y + x1 * cs.x;
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
  const uint32_t per_head = (uint32_t)(p.head_dim * p.elem / 16);  // chunks per head row
  const uint32_t per_tok = per_head * (uint32_t)p.n_heads;
  const uint32_t total = per_tok * (uint32_t)p.n_tok;
  const uint32_t stride = gridDim.x * 256;
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const uint32_t n = i / per_tok;
    const uint32_t c = (i - n * per_tok) % per_head;
    int tt, y, x;
    token_pos(p.g, (int)n, jb.t_index, tt, y, x);
    reinterpret_cast<uint4*>(dst)[i] = rotate_chunk(p.g, reinterpret_cast<const uint4*>(src)[i], c, p.elem, tt, y, x);
  }
}

// ---------------------------------------------------------------------------
// clean_write: the clean K/V of one layer of the block being closed go to its
// window slot, raw, together with its keys rotated at every window place the
// block takes while it stays in the window (newest first); for block 0 the
// raw tensors also go to the Static Sink, with the keys rotated at its place.
// One pass reads the clean keys once, and no key is rotated again when the
// window slides.  Thread = one 16-byte chunk of K and of V.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void clean_write_kernel(const CleanWrite p) {
  const uint32_t per_head = (uint32_t)(p.head_dim * p.elem / 16);
  const uint32_t per_tok = per_head * (uint32_t)p.n_heads;
  const uint32_t total = per_tok * (uint32_t)p.n_tok;
  const uint32_t stride = gridDim.x * 256;
  const uint4* __restrict__ ks = reinterpret_cast<const uint4*>(p.k_src);
  const uint4* __restrict__ vs = reinterpret_cast<const uint4*>(p.v_src);
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const uint32_t n = i / per_tok;
    const uint32_t c = (i - n * per_tok) % per_head;
    const uint4 k = ld_nt(ks + i), v = ld_nt(vs + i);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const CleanDst& o = p.dst[d];
      if (!o.k) continue;
      st_nt(reinterpret_cast<uint4*>(o.k) + i, k);
      st_nt(reinterpret_cast<uint4*>(o.v) + i, v);
#pragma unroll
      for (int r = 0; r < kMaxRot; ++r) {
        if (r >= o.n_rot) break;
        int tt, y, x;
        token_pos(p.g, (int)n, o.t_index[r], tt, y, x);
        st_nt(reinterpret_cast<uint4*>(o.k_rot[r]) + i, rotate_chunk(p.g, k, c, p.elem, tt, y, x));
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
__device__ inline double seq_dot(const double* __restrict__ a, const double* __restrict__ b, int n) {
#pragma clang fp contract(off)
  double s = 0.0;
  for (int k = 0; k < n; ++k) s = s + a[k] * b[k];
  return s;
}

// Fingerprint + retrieval, one wave64.  Entries fill the bank in slot order
// (id -1 = empty).  lds: (kMaxBank + 1) doubles of scores, then fp_dim doubles
// of the raw fingerprint.
__global__ __launch_bounds__(64) void retrieve_kernel(const float* __restrict__ fp_raw,
                                                      double* __restrict__ phi_cur,
                                                      const double* __restrict__ bank_phi,
                                                      DevState* __restrict__ st, int fp_dim,
                                                      const BankRule rule, int block,
                                                      int32_t* slot_out) {
  extern __shared__ double lds[];
  double* const score = lds;
  double* const x = lds + kMaxBank + 1;
  const int lane = threadIdx.x;
  for (int k = lane; k < fp_dim; k += 64) x[k] = (double)fp_raw[k];
  __syncthreads();
  // ||x||^2 as an index-order sum (every lane computes the same value), the
  // correctly rounded square root, one correctly rounded division per
  // element; zero stays zero
  const double ss = seq_dot(x, x, fp_dim);
  const double nrm = sqrt(ss);
  for (int k = lane; k < fp_dim; k += 64) phi_cur[k] = nrm > 0.0 ? x[k] / nrm : 0.0;
  __syncthreads();  // phi_cur is read back below by other lanes
  // score of entry s by lane s
  if (lane < rule.size && st->ids[lane] >= 0) score[lane] = seq_dot(phi_cur, bank_phi + (size_t)lane * fp_dim, fp_dim);
  __syncthreads();
  if (lane != 0) return;
  // r(b) = argmax over entries whose id != b-1; strict '>' keeps the lowest
  // slot on ties.  best: over every entry (the gated refresh's distance).
  const bool undetected = nrm == 0.0 && (rule.policy & kBankZeroFallback);
  int r = -1;
  double best_r = 0.0, best = -INFINITY;
  for (int s = 0; s < rule.size; ++s) {
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
    __shared__ double G[kMaxBank][kMaxBank];  // pairwise dots of the bank, i < j
    __shared__ double g[kMaxBank];            // dots with the candidate
    // one lane per dot product: lanes 0..M-1 the candidate against entry i,
    // the next M(M-1)/2 lanes the pairs (i, j), i < j, in lexicographic order
    // (at most 8 + 28 < 64 lanes)
    if (lane < M) {
      g[lane] = seq_dot(phi_cur, bank_phi + (size_t)lane * fp_dim, fp_dim);
    } else {
      int t = lane - M;
      for (int i = 0; i < M; ++i)
        for (int j = i + 1; j < M; ++j, --t)
          if (t == 0) G[i][j] = seq_dot(bank_phi + (size_t)i * fp_dim, bank_phi + (size_t)j * fp_dim, fp_dim);
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
  if (blocks > 256 * 8) blocks = 256 * 8;
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
  if (blocks > 256 * 8) blocks = 256 * 8;
  hipLaunchKernelGGL(clean_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_slot_copy(char* block_base, size_t slot_bytes, size_t copy_bytes,
                            const DevState* st, hipStream_t s) {
  const size_t n16 = copy_bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  hipLaunchKernelGGL(slot_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<uint8_t*>(block_base), slot_bytes, copy_bytes, st);
  return hipGetLastError();
}

hipError_t launch_retrieve(const float* fp_raw, double* phi_cur, const double* bank_phi,
                           DevState* st, int fp_dim, const BankRule& rule, int block, int32_t* slot_out,
                           hipStream_t s) {
  const size_t lds = sizeof(double) * ((size_t)kMaxBank + 1 + (size_t)fp_dim);
  hipLaunchKernelGGL(retrieve_kernel, dim3(1), dim3(64), lds, s, fp_raw, phi_cur, bank_phi, st,
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
