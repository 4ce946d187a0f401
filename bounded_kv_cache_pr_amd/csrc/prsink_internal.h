// Internal types shared by the host side (prsink_host.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace prsink {

constexpr int kMaxSegments = 8;   // Ref, Static, Dynamic, <= 4 previous window blocks, current
constexpr int kMaxBank = 8;
constexpr int kKeyTile = 64;      // keys per attention tile; slot token counts pad to this
constexpr int kMaxRopeLdsBytes = 48 * 1024;  // cos/sin table size the fast kernel stages in LDS

// One attended segment of the cache as the attention kernel sees it.  K and V
// share one layout: element (token n, head h, dim i) is at n*tok + h*head + i.
struct Segment {
  const void* k;        // raw keys, head 0, token 0
  const void* v;        // values, head 0, token 0
  int64_t tok;          // elements between consecutive tokens of one head
  int64_t head;         // elements between heads
  int32_t count;        // tokens attended (0 = segment empty)
  int32_t t_index;      // temporal table row of the segment's first frame
};

struct AttnParams {
  Segment seg[kMaxSegments];
  const void* q;        // [T][H][d] raw queries of the current block
  void* out;            // [T][H][d]
  const float2* rope;   // cos/sin table: t band [n_t][np_t], then h [lat_h][np_h], then w [lat_w][np_w]
  int32_t n_seg;
  int32_t n_q;          // T
  int32_t n_heads;
  int32_t lat_w;
  int32_t hw;           // tokens per frame
  int32_t q_t_index;    // temporal table row of the current block's first frame
  int32_t np_t, np_h, np_w;   // RoPE pairs per band
  int32_t rope_h_off, rope_w_off;  // float2 offsets of the h and w tables
  int32_t rope_bytes;   // size of the whole cos/sin table
  int32_t n_qtiles;
  float scale_log2;     // log2(e) / sqrt(d)
  // n / hw == umulhi(n, magic_hw) + n * one_hw and j / lat_w == umulhi(j, magic_w) +
  // j * one_w over the token ranges used (checked on the host); a divisor of 1 has
  // magic 0 and one 1.
  uint32_t magic_hw, one_hw;
  uint32_t magic_w, one_w;
};

// Bank / retrieval state kept in device memory inside the arena.
struct DevState {
  int32_t ids[kMaxBank];   // block id per bank entry, -1 = empty
  int32_t last_r;          // last retrieved bank entry, -1 = none
  int32_t dyn_id;          // block id whose K/V sit in the Dynamic slot, -1 = none
  int32_t decision;        // last bank decision: -2 none, -1 keep, j = entry written
  int32_t copy_src;        // pending slot copy: source block-slot index, -1 = skip
  int32_t copy_dst;        // destination block-slot index
  int32_t pad_[3];
};

// Launchers (kernels_*.hip).  All return the launch status.
hipError_t launch_attention(const AttnParams& p, int dtype, int head_dim, hipStream_t s);
hipError_t launch_kv_write(const void* k_src, const void* v_src, void* k_dst0, void* v_dst0,
                           void* k_dst1, void* v_dst1, int n_tok, int n_heads, int head_dim,
                           int t_pad, int elem_bytes, hipStream_t s);
hipError_t launch_slot_copy(char* block_base, size_t slot_bytes, const DevState* st,
                            hipStream_t s);
hipError_t launch_retrieve(const float* fp_raw, double* phi_cur, const double* bank_phi,
                           DevState* st, int fp_dim, int bank_count, int block,
                           int dyn_slot, int bank_slot0, int32_t* slot_out, hipStream_t s);
hipError_t launch_bank_update(const double* phi_cur, double* bank_phi, DevState* st,
                              int fp_dim, int bank_size, int bank_count, int block,
                              int win_slot, int bank_slot0, hipStream_t s);
hipError_t launch_state_init(DevState* st, hipStream_t s);

}  // namespace prsink
