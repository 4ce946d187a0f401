// Device-side helpers of the PR-Sink kernels (RoPE table lookups, token
// positions, segment addressing).  Included by the HIP sources only; the host
// side sees the plain types in prsink_internal.h.
#pragma once

#include "prsink_internal.h"

namespace prsink {

__device__ inline uint32_t div_magic(uint32_t n, uint32_t magic, uint32_t one) {
  return __umulhi(n, magic) + n * one;
}

// (temporal row, latent row, latent column) of token n of a segment whose
// first frame uses temporal row t_index.
__device__ inline void token_pos(const RopeGeom& g, int n, int t_index, int& tt, int& y, int& x) {
  const int f = div_magic(n, g.magic_hw, g.one_hw), j = n - f * g.hw;
  y = div_magic(j, g.magic_w, g.one_w);
  x = j - y * g.lat_w;
  tt = t_index + f;
}

// cos/sin of RoPE pair `pair` (adjacent elements 2*pair, 2*pair+1 of a head)
// at position (tt, y, x): the t band covers the first np_t pairs, then h, then w.
// The table index is chosen with selects, not branches: `pair` often differs
// between lanes, and a branch per lookup would serialise the loads.
__device__ inline int rope_index(const RopeGeom& g, int pair, int tt, int y, int x) {
  const int it = tt * g.np_t + pair;
  const int ih = g.rope_h_off + y * g.np_h + (pair - g.np_t);
  const int iw = g.rope_w_off + x * g.np_w + (pair - g.np_t - g.np_h);
  return pair < g.np_t ? it : pair < g.np_t + g.np_h ? ih : iw;
}
__device__ inline float2 rope_cs(const RopeGeom& g, int pair, int tt, int y, int x) {
  return g.rope[rope_index(g, pair, tt, y, x)];
}

// The bank entry the Dynamic Sink reads, loaded once per workgroup with a
// scalar load (the value then stays in SGPRs, so addresses built from it can
// feed buffer resources; the load waits for itself inside the asm).  -1 when
// the device found no entry; 0 when the block has no Dynamic segment.
__device__ inline int load_dyn_r(const AttnParams& p) {
  if (p.dyn_seg < 0) return 0;
  int r;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(r) : "s"(p.dyn_r) : "memory");
  return r;
}

// Keys of segment s: the Dynamic segment is empty when no entry was found.
__device__ inline int seg_count(const AttnParams& p, int s, int dyn_r) {
  const int c = p.seg[s].count;
  return s == p.dyn_seg && dyn_r < 0 ? 0 : c;
}

// K (is_k) or V base of segment s; dyn_r from load_dyn_r.  Written as a
// select of two computed bases: an early return here let the compiler treat
// the result as divergent and move it to VGPRs.
__device__ inline const char* seg_base(const AttnParams& p, int s, bool is_k, int dyn_r) {
  const char* dyn = (is_k ? p.dyn_k0 : p.dyn_v0) + (int64_t)(dyn_r > 0 ? dyn_r : 0) * p.dyn_stride;
  const char* seg = static_cast<const char*>(is_k ? p.seg[s].k : p.seg[s].v);
  return s == p.dyn_seg ? dyn : seg;
}

}  // namespace prsink
