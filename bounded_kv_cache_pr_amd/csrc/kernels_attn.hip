// PR-Sink block-causal attention with RoPE follow on gfx950.
//
// The current block's queries attend over [Ref; Static; Dynamic; window;
// current] with scale 1/sqrt(d) (LiveAnimate review on paper.rainbus.top,
// full-pipeline paragraph, attention formula).  Every key is read raw and
// rotated with 3D RoPE at its segment's *current* temporal slot and its
// latent (row, column) before use (same paragraph: raw keys re-rotated at the
// current cache position; novelty paragraph: reuse decoupled from the
// original timestamp).
//
// bf16 kernel (one workgroup = 4 wave64 = 128 query rows of one head):
//   * Q rows are rotated once in the prologue and kept in VGPRs as the MFMA
//     B operand.
//   * Per 64-key tile, the workgroup stages the keys into LDS rotated (each
//     key is rotated once per workgroup, in fp32, rounded to bf16) and V^T
//     (cached V is already stored transposed; the current block's V is
//     transposed while staging).
//   * S^T = K_rot Q_rot^T on v_mfma_f32_32x32x16_bf16: a lane owns one query
//     column and 16 key rows of each 32x32 block, so the softmax row max/sum
//     stay in-lane except for one exchange with lane ^ 32.  Keys are placed
//     in LDS with bits 2 and 3 of the row index swapped, which makes the
//     probabilities a lane holds after the QK^T MFMA exactly the B operand of
//     the PV MFMA, with no shuffles.
//   * O^T = V^T P^T accumulates in fp32; online softmax in base 2 with the
//     1/sqrt(d) scale folded in.
// fp32 kernel: a plain one-query-per-lane loop for the fp32 configuration.
#include "prsink_internal.h"

namespace prsink {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

// Row r of a 64-row key tile lives at LDS row key_perm(r): bits 2 and 3 swapped.
__device__ inline int key_perm(int r) { return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int D>
__global__ __launch_bounds__(256) void attn_bf16_kernel(const AttnParams p) {
  constexpr int KT = kKeyTile;      // keys per tile
  constexpr int QW = 32;            // query rows per wave
  constexpr int QT = 4 * QW;        // query rows per workgroup
  constexpr int KS = D + 8;         // LDS K row stride (bf16 elements)
  constexpr int VS = KT + 8;        // LDS V^T row stride
  constexpr int NC = D / 16;        // 16-wide d chunks (QK^T k-steps)
  constexpr int NDB = D / 32;       // 32-wide dv blocks of O^T
  __shared__ __align__(16) uint16_t Ks[KT * KS];
  __shared__ __align__(16) uint16_t Vs[D * VS];

  // XCD-aware tile order: consecutive workgroup ids land on different XCDs,
  // so give every XCD whole heads; the query tiles of a head then share that
  // XCD's L2 while they stream the same keys.
  const int wg = blockIdx.x;
  const int xcd = wg & 7, jx = wg >> 3;
  const int head = xcd + 8 * (jx / p.n_qtiles);
  const int qt = jx % p.n_qtiles;
  if (head >= p.n_heads) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int H = p.n_heads;

  // ---- prologue: rotate this lane's query row, keep it as the MFMA B operand
  const int qrow = qt * QT + wave * QW + l32;
  const bool qvalid = qrow < p.n_q;
  bf16x8 qreg[NC];
  {
    int tq = 0, yq = 0, xq = 0;
    if (qvalid) {
      const int f = qrow / p.hw, rem = qrow - f * p.hw;
      yq = rem / p.lat_w;
      xq = rem - yq * p.lat_w;
      tq = p.q_t_index + f;
    }
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((size_t)qrow * H + head) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int off = 16 * c + 8 * hh;
      uint4 w = make_uint4(0, 0, 0, 0);
      if (qvalid) w = *reinterpret_cast<const uint4*>(qp + off);
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const PairTab t = pair_tab(p, off / 2 + e);
        ws[e] = rotate_pair_bf16(ws[e], pair_cs(p, t, tq, yq, xq));
      }
      const uint4 r = make_uint4(ws[0], ws[1], ws[2], ws[3]);
      qreg[c] = __builtin_bit_cast(bf16x8, r);
    }
  }

  // ---- staging assignments (fixed per thread)
  constexpr int KCPR = D / 8;             // 16-byte chunks per key row
  constexpr int KROWS = 256 / KCPR;       // key rows per staging pass
  const int kcc = tid % KCPR;
  const int kr0 = tid / KCPR;
  PairTab ktab[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ktab[e] = pair_tab(p, kcc * 4 + e);

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  for (int s = 0; s < p.n_seg; ++s) {
    const Segment sg = p.seg[s];
    const int count = sg.count;
    const uint16_t* kbase = static_cast<const uint16_t*>(sg.k) + (size_t)head * sg.k_head;
    const uint16_t* vbase = static_cast<const uint16_t*>(sg.v) + (size_t)head * sg.v_head;
    for (int n0 = 0; n0 < count; n0 += KT) {
      // -- stage K (rotated at this segment's current positions)
#pragma unroll
      for (int it = 0; it < KT / KROWS; ++it) {
        const int r = kr0 + it * KROWS;
        const int n = n0 + r;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (n < count) {
          w = *reinterpret_cast<const uint4*>(kbase + (size_t)n * sg.k_tok + kcc * 8);
          const int f = n / p.hw, rem = n - f * p.hw;
          const int y = rem / p.lat_w, x = rem - y * p.lat_w;
          const int tt = sg.t_index + f;
          w.x = rotate_pair_bf16(w.x, pair_cs(p, ktab[0], tt, y, x));
          w.y = rotate_pair_bf16(w.y, pair_cs(p, ktab[1], tt, y, x));
          w.z = rotate_pair_bf16(w.z, pair_cs(p, ktab[2], tt, y, x));
          w.w = rotate_pair_bf16(w.w, pair_cs(p, ktab[3], tt, y, x));
        }
        *reinterpret_cast<uint4*>(&Ks[key_perm(r) * KS + kcc * 8]) = w;
      }
      // -- stage V^T
      if (sg.v_transposed) {
        constexpr int VCPR = KT / 8;        // chunks per V^T row
        constexpr int VROWS = 256 / VCPR;
        const int vc = tid % VCPR, vr0 = tid / VCPR;
#pragma unroll
        for (int it = 0; it < D / VROWS; ++it) {
          const int dv = vr0 + it * VROWS;
          // in bounds: the slot is padded to a multiple of KT with zeros
          const uint4 w =
              *reinterpret_cast<const uint4*>(vbase + (size_t)dv * sg.v_dim + n0 + vc * 8);
          *reinterpret_cast<uint4*>(&Vs[dv * VS + vc * 8]) = w;
        }
      } else {
        const int key = tid % KT, cg = tid / KT;
        const int n = n0 + key;
#pragma unroll
        for (int it = 0; it < D / 32; ++it) {
          const int ch = cg + 4 * it;
          uint4 w = make_uint4(0, 0, 0, 0);
          if (n < count) w = *reinterpret_cast<const uint4*>(vbase + (size_t)n * sg.v_tok + ch * 8);
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            Vs[(ch * 8 + 2 * e) * VS + key] = (uint16_t)(ws[e] & 0xffffu);
            Vs[(ch * 8 + 2 * e + 1) * VS + key] = (uint16_t)(ws[e] >> 16);
          }
        }
      }
      __syncthreads();

      // -- S^T = K_rot Q_rot^T for 64 keys x this wave's 32 queries
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
      // -- online softmax (base 2); register r of block kb holds key kb*32 + (r/8)*16 + hh*8 + r%8
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
        const uint4 u = make_uint4(pw[0], pw[1], pw[2], pw[3]);
        pb[kc] = __builtin_bit_cast(bf16x8, u);
      }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      // -- O^T += V^T P^T
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

  // ---- epilogue: O = O^T / rowsum; register 4g+e of block db is dv = 32db + 8g + 4hh + e
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
    if (qvalid) {
      const int f = qrow / p.hw, rem = qrow - f * p.hw;
      yq = rem / p.lat_w;
      xq = rem - yq * p.lat_w;
      tq = p.q_t_index + f;
    }
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
    const float* kbase = static_cast<const float*>(sg.k) + (size_t)head * sg.k_head;
    const float* vbase = static_cast<const float*>(sg.v) + (size_t)head * sg.v_head;
    for (int n0 = 0; n0 < count; n0 += KT) {
      for (int id = lane; id < KT * (D / 2); id += KT) {
        const int r = id / (D / 2), pr = id % (D / 2);
        const int n = n0 + r;
        float y0 = 0.f, y1 = 0.f;
        if (n < count) {
          const float x0 = kbase[(size_t)n * sg.k_tok + 2 * pr];
          const float x1 = kbase[(size_t)n * sg.k_tok + 2 * pr + 1];
          const int f = n / p.hw, rem = n - f * p.hw;
          const int y = rem / p.lat_w, x = rem - y * p.lat_w;
          const float2 cs = pair_cs(p, pair_tab(p, pr), sg.t_index + f, y, x);
          y0 = x0 * cs.x - x1 * cs.y;
          y1 = x0 * cs.y + x1 * cs.x;
        }
        Ks[r][2 * pr] = y0;
        Ks[r][2 * pr + 1] = y1;
      }
      for (int id = lane; id < KT * D; id += KT) {
        int r, dv;
        if (sg.v_transposed) { r = id % KT; dv = id / KT; }
        else { r = id / D; dv = id % D; }
        const int n = n0 + r;
        float v = 0.f;
        if (n < count)
          v = sg.v_transposed ? vbase[(size_t)dv * sg.v_dim + n] : vbase[(size_t)n * sg.v_tok + dv];
        Vs[r][dv] = v;
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
  if (dtype == 0) {  // bf16
    const int qt = 128;
    p.n_qtiles = (p.n_q + qt - 1) / qt;
    const int heads_per_xcd = (p.n_heads + 7) / 8;
    const dim3 grid(8 * heads_per_xcd * p.n_qtiles);
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
