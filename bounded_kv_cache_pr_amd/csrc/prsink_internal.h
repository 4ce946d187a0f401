// Internal types shared by the host side (prsink_host.cpp) and the HIP
// kernels, and the kernel launchers.  Not part of the public ABI.  Device-only
// helpers live in prsink_device.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace prsink {

constexpr int kMaxSegments = 8;   // Ref, Static, Dynamic, <= 4 previous window blocks, current
constexpr int kMaxBank = 8;
// Bank-policy bits, the values of pr_sink_bank_policy.
constexpr int kBankZeroFallback = 1, kBankContinual = 2, kBankGated = 4;
constexpr int kKeyTile = 64;      // keys per attention tile; slot token counts pad to this
constexpr int kMaxRotJobs = 6;    // rotation jobs per rope_follow launch

// Geometry of the 3D RoPE tables and of the latent grid, shared by every
// kernel that rotates.  The cos/sin table holds float2 (cos, sin) entries:
// t band [n_t][np_t], then h band [lat_h][np_h] at rope_h_off, then w band
// [lat_w][np_w] at rope_w_off.  Token n of a segment sits in frame n / hw, row
// (n % hw) / lat_w, column n % lat_w; the divisions use multiply-high magic
// numbers the host checked to be exact over the token ranges in use
// (n / d == umulhi(n, magic) + n * one, and a divisor of 1 has magic 0, one 1).
struct RopeGeom {
  const float2* rope;
  int32_t np_t, np_h, np_w;
  int32_t rope_h_off, rope_w_off;
  int32_t lat_w, hw;
  uint32_t magic_hw, one_hw, magic_w, one_w;
};

// One attended segment of the cache as the attention kernel sees it.  K and V
// share one layout: element (token n, head h, dim i) is at n*tok + h*head + i.
struct Segment {
  const void* k;        // keys already rotated at this segment's current positions
  const void* v;        // values
  int64_t tok;          // elements between consecutive tokens of one head
  int64_t head;         // elements between heads
  int32_t count;        // tokens attended (0 = segment empty)
  int32_t t_index;      // temporal table row of the segment's first frame
};

struct AttnParams {
  Segment seg[kMaxSegments];
  const void* q;        // [T][H][d] raw queries of the current block
  void* out;            // [T][H][d]
  RopeGeom g;
  int32_t n_seg;
  int32_t n_q;          // T
  int32_t n_heads;
  int32_t q_t_index;    // temporal table row of the current block's first frame
  int32_t n_qtiles;
  float scale_log2;     // log2(e) / sqrt(d)
  // Work split of the bf16 kernel.  A job is one (head, 256-query tile); its
  // keys are `units` 64-key units (the full tiles, then the packed ragged
  // tiles).  Each XCD takes the heads h = xcd (mod 8): its first `full_jobs`
  // jobs run whole, the next `tail_jobs` are each cut into `split` key ranges
  // whose partial results (`part`) are merged by the last piece to arrive
  // (`cnt`, one self-resetting counter per split job).
  int32_t full_jobs;
  int32_t tail_jobs;
  int32_t split;
  int32_t units;
  float* part;
  uint32_t* cnt;
  // The Dynamic Sink is not a copy: segment dyn_seg (-1 = none) reads bank
  // entry r = *dyn_r, whose rotated K (dyn_k0) and V (dyn_v0) sit dyn_stride
  // bytes apart per entry.  r is read on the device, so the host never waits
  // for the retrieval.
  const int32_t* dyn_r;
  const char* dyn_k0;
  const char* dyn_v0;
  int64_t dyn_stride;
  int32_t dyn_seg;
  // the device may find no entry although the host planned a Dynamic segment
  // (an undetected pose under the zero-fingerprint fallback): the segment then
  // counts 0 keys, and the work is not split
  int32_t dyn_may_vanish;
};

// Largest split of a job's keys the partial-record workspace is sized for, and
// the most CUs per XCD the work split plans for.
constexpr int kMaxSplit = 4;
constexpr int kMaxCuPerXcd = 32;
// Floats of one partial record: 256 rows x d of O, then (m, l) per lane.
__host__ __device__ constexpr size_t partial_record_floats(int head_dim) { return 256 * (size_t)head_dim + 2 * 512; }

// Bank / retrieval state kept in device memory inside the arena.
struct DevState {
  int32_t ids[kMaxBank];   // block id per bank entry, -1 = empty
  int32_t last_r;          // last retrieved bank entry, -1 = none
  int32_t dyn_id;          // block id of the open block's Dynamic Sink (bank entry last_r), -1 = none
  int32_t decision;        // last bank decision: -2 none, -1 keep, j = entry written
  int32_t copy_src;        // pending slot copy: source block-slot index, -1 = skip
  int32_t copy_dst;        // destination block-slot index
  int32_t last_used[kMaxBank];  // block at which each entry was last written or retrieved
  int32_t phi_zero;        // the open block's fingerprint is all zero
  double best;             // the open block's best dot product with the bank (-inf: empty bank)
};

// cos/sin of one place in the cache (Ref, Static, Dynamic, a window place, the
// current block): float2 (cos, sin) [token][pair] for every token a block (or
// the Ref Sink) has at that place and every RoPE pair of a head, in head order
// (t band pairs, then h, then w).  The places are fixed by the config, so the
// host fills these tables once, from the same angles as the band table.
// Chunk c (16 bytes) of a head row at token n needs pairs [4c, 4c+4) (bf16) or
// [2c, 2c+2) (fp32): one 32- or 16-byte read at cs + n * np + pair.

// One RoPE-follow job: rotate raw keys [n_tok][H][d] of n_layers layers with
// the cos/sin table of the place they take.
struct RotJob {
  const char* src;      // raw K of layer 0
  char* dst;            // rotated K of layer 0; ignored when from_state
  int64_t dst_off;      // from_state: byte offset of layer 0's rotated K inside a block slot
  const float2* cs;     // cos/sin table of the place
  int32_t from_state;   // 1: destination slot = device state's copy_dst, skipped when copy_src < 0
};

// Chunk index -> token: n = i / per_tok by multiply-high when exact (the host
// checks it over the chunk range), else by division.
struct ChunkDiv {
  uint32_t per_tok, magic, exact;
  int32_t np;           // RoPE pairs per head (head_dim / 2)
};

struct RotParams {
  RotJob job[kMaxRotJobs];
  ChunkDiv cd;
  const DevState* st;
  char* block_base;     // first block slot (from_state jobs)
  int64_t slot_bytes;   // block slot size (from_state jobs)
  int64_t layer_bytes;  // distance between consecutive layers, source and destination
  int32_t n_jobs, n_tok, n_heads, head_dim, elem;
};

// Places a window block is attended at: one per previous-block slot of the
// window (at most kMaxSegments - 4 of them).
constexpr int kMaxRot = kMaxSegments - 4;

// One destination of a clean write: raw K (k == nullptr: not kept), V and
// n_rot copies of K, copy i rotated with the cos/sin table cs[i] of its place.
// v == nullptr: unused.
struct CleanDst {
  char* k;
  char* v;
  char* k_rot[kMaxRot];
  const float2* cs[kMaxRot];
  int32_t n_rot;
};
struct CleanWrite {
  const char* k_src;    // clean K of one layer, [n_tok][H][d]
  const char* v_src;
  CleanDst dst[2];      // the window slot; the Static Sink (block 0 only)
  ChunkDiv cd;
  int32_t n_tok, n_heads, head_dim, elem;
};

// Launchers (kernels_*.hip).  All return the launch status.
// n_cu: compute units of the device (sizes the work split of the bf16 kernel).
hipError_t launch_attention(const AttnParams& p, int dtype, int head_dim, int n_cu, hipStream_t s);
hipError_t launch_rope_follow(const RotParams& p, int n_layers, hipStream_t s);
hipError_t launch_kv_write(const void* k_src, const void* v_src, void* k_dst0, void* v_dst0,
                           void* k_dst1, void* v_dst1, size_t bytes, hipStream_t s);
hipError_t launch_clean_write(const CleanWrite& p, hipStream_t s);
hipError_t launch_slot_copy(char* block_base, size_t slot_bytes, size_t copy_off, size_t copy_bytes,
                            const DevState* st, hipStream_t s);
// Bank update rules of one cache (pr_sink_config's bank fields).
struct BankRule {
  int32_t size, fill_blocks, policy, stale_blocks;
  double refresh_tau;
};
hipError_t launch_retrieve(const float* fp_raw, double* phi_cur, const double* bank_phi,
                           DevState* st, int fp_dim, const BankRule& rule, int block,
                           int32_t* slot_out, hipStream_t s);
hipError_t launch_bank_update(const double* phi_cur, double* bank_phi, DevState* st,
                              int fp_dim, const BankRule& rule, int block,
                              int win_slot, int bank_slot0, hipStream_t s);
hipError_t launch_state_init(DevState* st, hipStream_t s);

// Per-call scratch of an attention call supplied by the caller of
// attend_with_workspace instead of the arena: cur_rot receives the current
// block's rotated keys (cur_rot_bytes available).  Such a call plans no
// split jobs, so it needs no partial records or counters.
struct AttendWorkspace {
  void* cur_rot;
  size_t cur_rot_bytes;
};

}  // namespace prsink

struct pr_sink_cache;
namespace prsink {
// True for a dry-run cache (no arena, no device).
bool cache_is_dry(const pr_sink_cache* c);
// Records a HIP failure as the calling thread's last error; returns PR_SINK_EHIP.
int report_hip_error(hipError_t e, const char* what);
// pr_sink_attend with its per-call scratch taken from ws (nullptr: the arena).
int attend_with_workspace(pr_sink_cache* c, int32_t layer, const void* q_raw, const void* k_cur_raw,
                          const void* v_cur_raw, void* out, void* stream, const AttendWorkspace* ws);

}  // namespace prsink
