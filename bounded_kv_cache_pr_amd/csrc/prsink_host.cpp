// Host side of the PR-Sink C ABI: config validation, arena layout, RoPE
// tables, the per-block state machine, and kernel launches.
//
// The cache follows the PR-Sink description: Ref Sink, Static Sink (first
// generated block), one Dynamic Sink recalled by pose retrieval, and a rolling
// window of W slots whose last slot is the current block (HF papers abstract
// of LiveAnimate; papers.ananclaw.com explainer, "Pose-Retrieval Sink
// Attention" section; paper.rainbus.top review, full-pipeline paragraph).
// Memory is one caller-owned arena whose size is a closed form of the config,
// so the footprint cannot grow with the stream (HF abstract: memory and
// per-block latency independent of stream length).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <new>
#include <string>
#include <vector>

#include "pr_sink.h"
#include "prsink_internal.h"

using namespace prsink;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define PRS_HIP(x)                                                                     \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) return fail(PR_SINK_EHIP, "%s: %s", #x, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 4096;
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int pad_tokens(int n) { return (n + kKeyTile - 1) / kKeyTile * kKeyTile; }

// Multiply-high divisor: n / d == umulhi(n, ceil(2^32 / d)) for every n with
// n * (ceil(2^32/d) * d - 2^32) < 2^32.  0 encodes d == 1.
uint32_t magic_for(uint32_t d) {
  if (d <= 1) return 0;
  return (uint32_t)(((1ull << 32) + d - 1) / d);
}

bool magic_exact(uint32_t d, uint32_t n_max) {
  if (d <= 1) return true;
  const unsigned long long m = magic_for(d);
  const unsigned long long e = m * d - (1ull << 32);
  return (unsigned long long)n_max * e < (1ull << 32);
}

// Arena layout (offsets in bytes from the arena base):
//   [state | fingerprints | rope table | current block's rotated K] [Ref slot] [block slots...]
// Block slots: Static, Dynamic, window 0..W-1, bank 0..M-1.  A slot holds three
// regions of n_layers tensors each, every tensor [t_pad][H][d] (token-major,
// like the tensors the caller passes, so every segment shares one row stride;
// rows past T stay zero): raw K, V, and K rotated at the positions of the
// slot's current place in the layout (a bank entry: the Dynamic Sink's place).
struct Layout {
  int elem, tpf, tb, tr, tb_pad, tr_pad;
  size_t kv_b, slot_b;   // block slot: one tensor of one layer, whole slot
  size_t kv_r, slot_r;   // Ref slot
  size_t off_state, off_phi_bank, off_phi_cur, off_rope, off_ptab, off_cur_rot, off_part, off_cnt, off_ref,
      off_blocks, off_wraw, off_wrot, total;
  size_t wrot_b;             // per window slot: its keys rotated at the older window places
  size_t n_part_rec, n_cnt;  // partial records and counters of split attention jobs
  int n_t, np_t, np_h, np_w, rope_h_off, rope_w_off, rope_entries;
  size_t ptab_entries;  // per-place cos/sin: Ref [tr][np], then W + 2 block places [tb][np] each
  int n_block_slots;
};

bool check_config(const pr_sink_config* c) {
  if (!c) return fail(PR_SINK_EINVAL, "config is NULL"), false;
  if (c->n_layers < 1 || c->n_layers > 4096) return fail(PR_SINK_EINVAL, "n_layers out of range"), false;
  if (c->n_heads < 1 || c->n_heads > 1024) return fail(PR_SINK_EINVAL, "n_heads out of range"), false;
  if (c->head_dim != 64 && c->head_dim != 128) return fail(PR_SINK_EINVAL, "head_dim must be 64 or 128"), false;
  int sum = 0;
  for (int a = 0; a < 3; ++a) {
    if (c->rope_dims[a] < 2 || c->rope_dims[a] % 2) return fail(PR_SINK_EINVAL, "rope band %d must be even and >= 2", a), false;
    sum += c->rope_dims[a];
  }
  if (sum != c->head_dim) return fail(PR_SINK_EINVAL, "rope bands sum to %d, head_dim is %d", sum, c->head_dim), false;
  if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta)) return fail(PR_SINK_EINVAL, "rope_theta must be > 0"), false;
  if (c->lat_h < 1 || c->lat_w < 1 || c->lat_h > 1024 || c->lat_w > 1024) return fail(PR_SINK_EINVAL, "latent size out of range"), false;
  if (c->ref_frames < 1 || c->block_frames < 1 || c->ref_frames > 64 || c->block_frames > 64) return fail(PR_SINK_EINVAL, "frame counts out of range"), false;
  if (c->window_slots < 1 || c->window_slots > kMaxSegments - 3) return fail(PR_SINK_EINVAL, "window_slots must be 1..%d", kMaxSegments - 3), false;
  if (c->bank_size < 2 || c->bank_size > kMaxBank) return fail(PR_SINK_EINVAL, "bank_size must be 2..%d", kMaxBank), false;
  if (c->bank_fill_blocks < 0) return fail(PR_SINK_EINVAL, "bank_fill_blocks must be >= 0"), false;
  if (c->fp_dim < 1 || c->fp_dim > 4096) return fail(PR_SINK_EINVAL, "fp_dim must be 1..4096"), false;
  if (c->dtype != PR_SINK_BF16 && c->dtype != PR_SINK_F32) return fail(PR_SINK_EINVAL, "unknown dtype"), false;
  if (c->t0 < 0 || c->t0 > (1 << 20)) return fail(PR_SINK_EINVAL, "t0 out of range"), false;
  if (c->bank_policy & ~7) return fail(PR_SINK_EINVAL, "unknown bank_policy bits"), false;
  if ((c->bank_policy & PR_SINK_BANK_CONTINUAL) && c->bank_stale_blocks < 1)
    return fail(PR_SINK_EINVAL, "bank_stale_blocks must be >= 1"), false;
  if ((c->bank_policy & PR_SINK_BANK_GATED) && !(c->bank_refresh_tau >= -1.0 && c->bank_refresh_tau <= 1.0))
    return fail(PR_SINK_EINVAL, "bank_refresh_tau must be in [-1, 1]"), false;
  const long long tpf = (long long)c->lat_h * c->lat_w;
  if (tpf * c->block_frames > (1 << 24) || tpf * c->ref_frames > (1 << 24)) return fail(PR_SINK_EINVAL, "block too large"), false;
  const uint32_t n_max = (uint32_t)(tpf * (c->block_frames > c->ref_frames ? c->block_frames : c->ref_frames));
  if (!magic_exact((uint32_t)tpf, n_max) || !magic_exact((uint32_t)c->lat_w, (uint32_t)tpf))
    return fail(PR_SINK_EINVAL, "latent frame %dx%d too large for 32-bit position division", c->lat_h, c->lat_w), false;
  // rotation kernels index 16-byte chunks of one block's keys with 32-bit ints;
  // attention buffer ranges (one segment of one layer) stay below 2^31 bytes
  const long long elem = c->dtype == PR_SINK_BF16 ? 2 : 4;
  const long long seg_bytes = (long long)n_max * c->n_heads * c->head_dim * elem;
  if (seg_bytes >= (1ll << 31)) return fail(PR_SINK_EINVAL, "one block of one layer must stay below 2 GiB"), false;
  return true;
}

Layout make_layout(const pr_sink_config* c) {
  Layout L{};
  L.elem = c->dtype == PR_SINK_BF16 ? 2 : 4;
  L.tpf = c->lat_h * c->lat_w;
  L.tb = L.tpf * c->block_frames;
  L.tr = L.tpf * c->ref_frames;
  L.tb_pad = pad_tokens(L.tb);
  L.tr_pad = pad_tokens(L.tr);
  const size_t hd = (size_t)c->n_heads * c->head_dim * L.elem;
  L.kv_b = align_up(hd * L.tb_pad, 256);
  // a block slot holds V and the keys rotated at the slot's place; the raw
  // keys of the window's blocks live in a ring-indexed area of their own
  L.slot_b = align_up(2 * L.kv_b * c->n_layers, kAlign);
  L.kv_r = align_up(hd * L.tr_pad, 256);
  L.slot_r = align_up(3 * L.kv_r * c->n_layers, kAlign);
  // Static, the window, the bank; the Dynamic Sink is a reference to a bank
  // entry and takes no slot of its own
  L.n_block_slots = 1 + c->window_slots + c->bank_size;
  // temporal positions: Ref, Static, Dynamic, W-1 previous blocks, current
  L.n_t = c->ref_frames + (c->window_slots + 2) * c->block_frames;
  L.np_t = c->rope_dims[0] / 2;
  L.np_h = c->rope_dims[1] / 2;
  L.np_w = c->rope_dims[2] / 2;
  L.rope_h_off = L.n_t * L.np_t;
  L.rope_w_off = L.rope_h_off + c->lat_h * L.np_h;
  L.rope_entries = L.rope_w_off + c->lat_w * L.np_w;
  size_t off = 0;
  L.off_state = off;
  off = align_up(off + sizeof(DevState), 256);
  L.off_phi_bank = off;
  off = align_up(off + sizeof(double) * c->bank_size * c->fp_dim, 256);
  L.off_phi_cur = off;
  off = align_up(off + sizeof(double) * c->fp_dim, 256);
  L.off_rope = off;  // fp32 (cos, sin) table
  off = align_up(off + 8 * (size_t)L.rope_entries, kAlign);
  // per-place tables for the rotation kernels: the Ref place, then the block
  // places Static, Dynamic, the W-1 window places and the current block
  L.off_ptab = off;
  L.ptab_entries = ((size_t)L.tr + (size_t)(c->window_slots + 2) * L.tb) * (c->head_dim / 2);
  off = align_up(off + 8 * L.ptab_entries, kAlign);
  L.off_cur_rot = off;
  off = align_up(off + L.kv_b, kAlign);
  // split attention jobs (bf16): per XCD fewer than kMaxCuPerXcd jobs are split,
  // into at most kMaxSplit pieces, each piece one partial record
  const bool split = c->dtype == PR_SINK_BF16;
  L.n_cnt = split ? 8 * (size_t)kMaxCuPerXcd : 0;
  L.n_part_rec = L.n_cnt * kMaxSplit;
  L.off_part = off;
  off = align_up(off + L.n_part_rec * partial_record_floats(c->head_dim) * sizeof(float), kAlign);
  L.off_cnt = off;
  off = align_up(off + L.n_cnt * sizeof(uint32_t), kAlign);
  L.off_ref = off;
  off += L.slot_r;
  L.off_blocks = off;
  off += L.slot_b * L.n_block_slots;
  L.off_wraw = off;  // raw keys of window slot j: W x n_layers tensors
  off += align_up((size_t)c->window_slots * c->n_layers * L.kv_b, kAlign);
  // a window block is attended at W-1 places; the block slot holds its keys
  // rotated at the newest one, this area the W-2 older ones
  L.off_wrot = off;
  L.wrot_b = c->window_slots >= 3 ? align_up((size_t)(c->window_slots - 2) * L.kv_b * c->n_layers, kAlign) : 0;
  off += L.wrot_b * c->window_slots;
  L.total = off;
  return L;
}

// cos/sin of every (band, position, pair), computed in double and stored as
// fp32 (cos, sin): the t band over the n_t temporal rows, then h, then w.  The
// angle of pair i of a band of D dims at position p is p * theta^(-2i/D).
std::vector<uint32_t> rope_table(const pr_sink_config* c, const Layout& L) {
  const size_t E = (size_t)L.rope_entries;
  std::vector<uint32_t> t(2 * E);
  auto fill = [&](int base, int npos, int pos0, int band_dim) {
    const int np = band_dim / 2;
    for (int ps = 0; ps < npos; ++ps)
      for (int i = 0; i < np; ++i) {
        const double w = std::pow(c->rope_theta, -2.0 * i / band_dim);
        const double a = (double)(pos0 + ps) * w;
        const float cs = (float)std::cos(a), sn = (float)std::sin(a);
        const size_t e = (size_t)(base + ps * np + i);
        std::memcpy(&t[2 * e], &cs, 4);
        std::memcpy(&t[2 * e + 1], &sn, 4);
      }
  };
  fill(0, L.n_t, c->t0, c->rope_dims[0]);
  fill(L.rope_h_off, c->lat_h, 0, c->rope_dims[1]);
  fill(L.rope_w_off, c->lat_w, 0, c->rope_dims[2]);
  return t;
}

// The per-place tables, gathered from the band table: for a place whose first
// frame has temporal row t_index, token n = (frame f, row y, column x) takes
// the t band at row t_index + f, the h band at y and the w band at x.
std::vector<uint32_t> place_tables(const pr_sink_config* c, const Layout& L, const std::vector<uint32_t>& band) {
  const int np = c->head_dim / 2;
  std::vector<uint32_t> t(2 * L.ptab_entries);
  size_t e = 0;
  auto place = [&](int t_index, int n_tok) {
    for (int n = 0; n < n_tok; ++n) {
      const int f = n / L.tpf, y = (n % L.tpf) / c->lat_w, x = n % c->lat_w;
      for (int pr = 0; pr < np; ++pr) {
        size_t b;
        if (pr < L.np_t) b = (size_t)(t_index + f) * L.np_t + pr;
        else if (pr < L.np_t + L.np_h) b = L.rope_h_off + (size_t)y * L.np_h + (pr - L.np_t);
        else b = L.rope_w_off + (size_t)x * L.np_w + (pr - L.np_t - L.np_h);
        t[2 * e] = band[2 * b];
        t[2 * e + 1] = band[2 * b + 1];
        ++e;
      }
    }
  };
  place(0, L.tr);
  for (int k = 0; k < c->window_slots + 2; ++k) place(c->ref_frames + k * c->block_frames, L.tb);
  return t;
}

}  // namespace

struct pr_sink_cache {
  pr_sink_config cfg;
  Layout lay;
  bool dry;
  char* arena;
  int next_block;     // block to open next
  bool open;
  int bank_count;     // entries filled so far (the first M blocks are inserted unconditionally)
  bool dyn_present;   // the open block attends the Dynamic Sink
  std::vector<uint8_t> ref_set, written;
  std::vector<uint8_t> win_raw;  // [window slot][layer]: the slot's raw keys were written
  int n_cu;           // compute units of the device

  // Cross-stream order.  Every call may use its own stream; an event marks
  // each producer, and a consumer's stream waits on it only when the
  // producer ran on another stream (same stream: queue order suffices).
  struct Mark {
    hipEvent_t ev = nullptr;
    hipStream_t st = nullptr;
    bool set = false;
    bool pending = false;         // marked but not recorded yet (see defer)
    bool waited = false;          // `seen` already waits for this recording
    hipStream_t seen = nullptr;   // (the null stream is a stream too)
  };
  std::vector<Mark> clean;  // per layer: the last clean write of that layer
  Mark clean_all;           // every clean write of block clean_all_block (all on one stream)
  int clean_all_block = -1;
  hipStream_t clean_stream = nullptr;  // the stream of this block's clean writes so far
  bool clean_one_stream = true;
  std::vector<Mark> ref;    // per layer: the last Ref Sink write of that layer
  Mark attn;                // the last attention call
  Mark retr;                // the last retrieval
  Mark dec;                 // the last bank decision (state only; entries may still be copying)
  Mark bank;                // the last bank update that wrote the bank, its copies included
  Mark done[2];             // block b's bank update complete, at [b & 1]
  hipEvent_t time_start = nullptr, time_stop = nullptr;  // caller's events around the attention kernel

  ~pr_sink_cache() {
    auto drop = [](Mark& m) { if (m.ev) (void)hipEventDestroy(m.ev); };
    for (Mark& m : clean) drop(m);
    for (Mark& m : ref) drop(m);
    drop(clean_all); drop(attn); drop(retr); drop(dec); drop(bank); drop(done[0]); drop(done[1]);
  }

  char* block_slot(int bs) const { return arena + lay.off_blocks + (size_t)bs * lay.slot_b; }
  char* ref_slot() const { return arena + lay.off_ref; }
  // Byte offsets of one layer's tensors inside a slot (tensors of kv_r or kv_b
  // bytes).  Ref slot: raw K, V and rotated K of layer l
  size_t ref_k(int l) const { return (size_t)l * lay.kv_r; }
  size_t ref_v(int l) const { return ((size_t)cfg.n_layers + l) * lay.kv_r; }
  size_t ref_r(int l) const { return (2 * (size_t)cfg.n_layers + l) * lay.kv_r; }
  // block slot: V and rotated K of layer l
  size_t blk_v(int l) const { return (size_t)l * lay.kv_b; }
  size_t blk_r(int l) const { return ((size_t)cfg.n_layers + l) * lay.kv_b; }
  // raw keys of the block in window slot j, layer l
  char* window_raw(int j, int l) const {
    return arena + lay.off_wraw + ((size_t)j * cfg.n_layers + l) * lay.kv_b;
  }
  DevState* state() const { return reinterpret_cast<DevState*>(arena + lay.off_state); }
  double* phi_bank() const { return reinterpret_cast<double*>(arena + lay.off_phi_bank); }
  double* phi_cur() const { return reinterpret_cast<double*>(arena + lay.off_phi_cur); }
  const float2* rope() const { return reinterpret_cast<const float2*>(arena + lay.off_rope); }
  // cos/sin table of the place whose first frame has temporal row t_index:
  // the Ref place (row 0) or block place k at row ref_frames + k block_frames
  const float2* place_cs(int t_index) const {
    const float2* base = reinterpret_cast<const float2*>(arena + lay.off_ptab);
    const size_t np = cfg.head_dim / 2;
    if (t_index == 0) return base;
    const int k = (t_index - cfg.ref_frames) / cfg.block_frames;
    return base + ((size_t)lay.tr + (size_t)k * lay.tb) * np;
  }
  int bs_static() const { return 0; }
  // Keys of window slot j rotated at window place p (0 = oldest, W-2 = newest)
  // for layer l.
  char* window_rot(int j, int p, int l) const {
    if (p == cfg.window_slots - 2) return block_slot(bs_window(j)) + blk_r(l);
    return arena + lay.off_wrot + (size_t)j * lay.wrot_b + ((size_t)p * cfg.n_layers + l) * lay.kv_b;
  }
  // First temporal row of window place p.
  int window_t(int p) const { return cfg.ref_frames + (2 + p) * cfg.block_frames; }
  int bs_window(int j) const { return 1 + j; }
  int bs_bank(int i) const { return 1 + cfg.window_slots + i; }
};

namespace {

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_layer(const pr_sink_cache* c, int layer) {
  if (!c) return fail(PR_SINK_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(PR_SINK_EINVAL, "layer %d out of range", layer);
  return PR_SINK_OK;
}

int check_tensor(const void* p, const char* name) {
  if (!p) return fail(PR_SINK_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(PR_SINK_EINVAL, "%s must be 16-byte aligned", name);
  return PR_SINK_OK;
}

// Segment token counts and temporal table rows for the open block.
void segment_table(const pr_sink_cache* c, int* tokens, int* t_index) {
  const pr_sink_config& g = c->cfg;
  const int b = c->next_block;
  const int fb = g.block_frames;
  int t = 0, s = 0;
  tokens[s] = c->lay.tr; t_index[s++] = t; t += g.ref_frames;
  tokens[s] = b >= 1 ? c->lay.tb : 0; t_index[s++] = t; t += fb;          // Static = block 0
  tokens[s] = c->dyn_present ? c->lay.tb : 0; t_index[s++] = t; t += fb;  // Dynamic
  for (int j = 0; j < g.window_slots - 1; ++j) {                           // blocks b-(W-1) .. b-1
    const int id = b - (g.window_slots - 1) + j;
    tokens[s] = id >= 0 ? c->lay.tb : 0; t_index[s++] = t; t += fb;
  }
  tokens[s] = c->lay.tb; t_index[s++] = t;                                 // current block
}

RopeGeom rope_geom(const pr_sink_cache* c) {
  const Layout& L = c->lay;
  RopeGeom g{};
  g.rope = c->rope();
  g.np_t = L.np_t;
  g.np_h = L.np_h;
  g.np_w = L.np_w;
  g.rope_h_off = L.rope_h_off;
  g.rope_w_off = L.rope_w_off;
  g.lat_w = c->cfg.lat_w;
  g.hw = L.tpf;
  g.magic_hw = magic_for((uint32_t)L.tpf);
  g.one_hw = L.tpf == 1;
  g.magic_w = magic_for((uint32_t)c->cfg.lat_w);
  g.one_w = c->cfg.lat_w == 1;
  return g;
}

// n = i / per_tok for chunk indices i < n_tok * per_tok.
ChunkDiv chunk_div(const pr_sink_cache* c, int n_tok) {
  ChunkDiv d{};
  d.per_tok = (uint32_t)(c->cfg.n_heads * c->cfg.head_dim * c->lay.elem / 16);
  d.magic = magic_for(d.per_tok);
  d.exact = magic_exact(d.per_tok, (uint32_t)((uint64_t)n_tok * d.per_tok));
  d.np = c->cfg.head_dim / 2;
  return d;
}

// Rotation launch over n_tok tokens per layer; consecutive layers of source
// and destination lie layer_bytes apart.
RotParams rot_params(const pr_sink_cache* c, int n_tok, size_t layer_bytes) {
  RotParams r{};
  r.cd = chunk_div(c, n_tok);
  r.st = c->state();
  r.block_base = c->block_slot(0);
  r.slot_bytes = (int64_t)c->lay.slot_b;
  r.layer_bytes = (int64_t)layer_bytes;
  r.n_tok = n_tok;
  r.n_heads = c->cfg.n_heads;
  r.head_dim = c->cfg.head_dim;
  r.elem = c->lay.elem;
  return r;
}

void add_job(const pr_sink_cache* c, RotParams& r, const void* src, void* dst, int t_index) {
  RotJob& j = r.job[r.n_jobs++];
  j.src = static_cast<const char*>(src);
  j.dst = static_cast<char*>(dst);
  j.dst_off = 0;
  j.cs = c->place_cs(t_index);
  j.from_state = 0;
}

BankRule bank_rule(const pr_sink_config& g) {
  return BankRule{g.bank_size, g.bank_fill_blocks, g.bank_policy, g.bank_stale_blocks, g.bank_refresh_tau};
}

size_t block_bytes(const pr_sink_cache* c, int n_tok) {
  return (size_t)n_tok * c->cfg.n_heads * c->cfg.head_dim * c->lay.elem;
}

// The bank is written during the fill phase, and later under the CONTINUAL
// and GATED policies (the device decides whether anything changes).
bool may_enter_bank(const pr_sink_config& g, int block) {
  return block < g.bank_fill_blocks || (g.bank_policy & (PR_SINK_BANK_CONTINUAL | PR_SINK_BANK_GATED));
}

// Stream s waits for producer m if m ran on another stream and s has not
// waited for this recording of m yet (a stream wait is a queue packet that
// costs microseconds between kernels; the three denoise steps of a layer
// would otherwise each wait for the same clean write).
hipError_t after(hipStream_t s, pr_sink_cache::Mark& m) {
  if (!m.set || m.st == s) return hipSuccess;
  if (m.pending) {
    // recorded now: the event then also covers work queued on m.st since the
    // mark, which only makes the wait longer, never too short
    if (hipError_t e = hipEventRecord(m.ev, m.st)) return e;
    m.pending = false;
    m.waited = false;
  }
  if (m.waited && m.seen == s) return hipSuccess;
  const hipError_t e = hipStreamWaitEvent(s, m.ev, 0);
  if (e == hipSuccess) {
    m.waited = true;
    m.seen = s;
  }
  return e;
}
// Marks the work queued so far on s as producer m.
hipError_t mark(hipStream_t s, pr_sink_cache::Mark& m) {
  m.st = s;
  m.set = true;
  m.pending = false;
  m.waited = false;
  return hipEventRecord(m.ev, s);
}
// mark() without the event record, which after() makes the first time a
// consumer on another stream waits.  For the attention calls: a record costs
// the queue a few microseconds between kernels, and their consumers (clean
// writes, bank updates, Ref writes) come after a whole block of them.  Work
// that other streams must see at a finer grain (the per-layer clean writes
// the next block's attention waits for) keeps mark().
void defer(hipStream_t s, pr_sink_cache::Mark& m) {
  m.st = s;
  m.set = true;
  m.pending = true;
  m.waited = false;
}

}  // namespace

extern "C" {

size_t pr_sink_arena_bytes(const pr_sink_config* cfg) {
  if (!check_config(cfg)) return 0;
  return make_layout(cfg).total;
}

namespace {
int cache_init(const pr_sink_config* cfg, void* arena_dev, size_t arena_bytes, void* stream,
               pr_sink_cache** out);
}  // namespace

// The only call that allocates host memory (the cos/sin table, per-layer
// state): an allocation failure returns an error instead of leaving the C ABI
// as an exception.
int pr_sink_cache_init(const pr_sink_config* cfg, void* arena_dev, size_t arena_bytes,
                       void* stream, pr_sink_cache** out) {
  try {
    return cache_init(cfg, arena_dev, arena_bytes, stream, out);
  } catch (const std::exception& e) {
    if (out) *out = nullptr;
    return fail(PR_SINK_EINVAL, "host allocation failed: %s", e.what());
  }
}

namespace {
int cache_init(const pr_sink_config* cfg, void* arena_dev, size_t arena_bytes, void* stream,
               pr_sink_cache** out) {
  if (!out) return fail(PR_SINK_EINVAL, "out is NULL");
  *out = nullptr;
  if (!check_config(cfg)) return PR_SINK_EINVAL;
  const Layout L = make_layout(cfg);
  const bool dry = arena_dev == nullptr && arena_bytes == 0;
  int n_cu = 0;
  if (!dry) {
    if (!arena_dev) return fail(PR_SINK_EINVAL, "arena is NULL");
    if (reinterpret_cast<uintptr_t>(arena_dev) & 255) return fail(PR_SINK_EINVAL, "arena must be 256-byte aligned");
    if (arena_bytes < L.total)
      return fail(PR_SINK_ENOSPACE, "arena has %zu bytes, config needs %zu", arena_bytes, L.total);
    int dev = 0;
    PRS_HIP(hipGetDevice(&dev));
    hipDeviceProp_t prop;
    PRS_HIP(hipGetDeviceProperties(&prop, dev));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return fail(PR_SINK_EHIP, "device %d is %s; this library is built for gfx950", dev, prop.gcnArchName);
    n_cu = prop.multiProcessorCount;
    hipStream_t s = as_stream(stream);
    char* a = static_cast<char*>(arena_dev);
    PRS_HIP(hipMemsetAsync(a, 0, L.total, s));  // zero padding keeps masked keys finite
    std::vector<uint32_t> tab = rope_table(cfg, L);
    PRS_HIP(hipMemcpyAsync(a + L.off_rope, tab.data(), tab.size() * sizeof(uint32_t),
                           hipMemcpyHostToDevice, s));
    std::vector<uint32_t> ptab = place_tables(cfg, L, tab);
    PRS_HIP(hipMemcpyAsync(a + L.off_ptab, ptab.data(), ptab.size() * sizeof(uint32_t),
                           hipMemcpyHostToDevice, s));
    PRS_HIP(launch_state_init(reinterpret_cast<DevState*>(a + L.off_state), s));
    PRS_HIP(hipStreamSynchronize(s));
  }
  pr_sink_cache* c = new (std::nothrow) pr_sink_cache();
  if (!c) return fail(PR_SINK_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->lay = L;
  c->dry = dry;
  c->arena = static_cast<char*>(arena_dev);
  c->next_block = 0;
  c->open = false;
  c->bank_count = 0;
  c->dyn_present = false;
  c->n_cu = n_cu;
  try {
    c->clean.resize(cfg->n_layers);
    c->ref.resize(cfg->n_layers);
  } catch (...) {
    delete c;
    throw;
  }
  if (!dry) {
    auto make = [](pr_sink_cache::Mark& m) { return hipEventCreateWithFlags(&m.ev, hipEventDisableTiming); };
    hipError_t e = hipSuccess;
    for (auto& m : c->clean) if (e == hipSuccess) e = make(m);
    for (auto& m : c->ref) if (e == hipSuccess) e = make(m);
    for (auto* m : {&c->clean_all, &c->attn, &c->retr, &c->dec, &c->bank, &c->done[0], &c->done[1]})
      if (e == hipSuccess) e = make(*m);
    if (e != hipSuccess) {
      delete c;
      return fail(PR_SINK_EHIP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
    }
  }
  try {
    c->ref_set.assign(cfg->n_layers, 0);
    c->written.assign(cfg->n_layers, 0);
    c->win_raw.assign((size_t)cfg->window_slots * cfg->n_layers, 0);
  } catch (...) {
    delete c;
    throw;
  }
  *out = c;
  g_err.clear();
  return PR_SINK_OK;
}
}  // namespace

int pr_sink_set_ref(pr_sink_cache* c, int32_t layer, const void* k_raw, const void* v_raw,
                    void* stream) {
  if (int e = check_layer(c, layer)) return e;
  if (int e = check_tensor(k_raw, "k_raw")) return e;
  if (int e = check_tensor(v_raw, "v_raw")) return e;
  if (c->open) return fail(PR_SINK_ESTATE, "set_ref while block %d is open", c->next_block);
  if (!c->dry) {
    const Layout& L = c->lay;
    hipStream_t s = as_stream(stream);
    char* ref = c->ref_slot();
    // earlier attention read the old Ref Sink; an earlier write of the same
    // layer, possibly on another stream, must land first (write after write)
    PRS_HIP(after(s, c->attn));
    PRS_HIP(after(s, c->ref[layer]));
    PRS_HIP(launch_kv_write(k_raw, v_raw, ref + c->ref_k(layer), ref + c->ref_v(layer),
                            nullptr, nullptr, block_bytes(c, L.tr), s));
    // the Ref Sink's place never moves: rotate its keys once
    RotParams r = rot_params(c, L.tr, L.kv_r);
    add_job(c, r, ref + c->ref_k(layer), ref + c->ref_r(layer), 0);
    PRS_HIP(launch_rope_follow(r, 1, s));
    PRS_HIP(mark(s, c->ref[layer]));
  }
  c->ref_set[layer] = 1;
  return PR_SINK_OK;
}

int pr_sink_retrieve(pr_sink_cache* c, int32_t block, const float* fp_raw_dev,
                     int32_t* slot_out_dev, void* stream) {
  if (!c) return fail(PR_SINK_EINVAL, "cache is NULL");
  if (!fp_raw_dev || (reinterpret_cast<uintptr_t>(fp_raw_dev) & 3)) return fail(PR_SINK_EINVAL, "fp_raw_dev must be a 4-byte aligned device pointer");
  if (slot_out_dev && (reinterpret_cast<uintptr_t>(slot_out_dev) & 3)) return fail(PR_SINK_EINVAL, "slot_out_dev must be 4-byte aligned");
  if (c->open) return fail(PR_SINK_ESTATE, "block %d is still open", c->next_block);
  if (block != c->next_block) return fail(PR_SINK_ESTATE, "expected block %d, got %d", c->next_block, block);
  for (int l = 0; l < c->cfg.n_layers; ++l)
    if (!c->ref_set[l]) return fail(PR_SINK_ESTATE, "Ref Sink of layer %d not set", l);
  // The host knows whether a candidate exists: every bank update inserts while
  // there is room, so a bank with one entry holds block 0, and a fuller bank
  // holds several distinct blocks of which at most one is block-1.  Under
  // ZERO_FALLBACK an undetected block is not inserted and retrieves nothing,
  // so bank_count is an upper bound and the attention kernels drop the
  // Dynamic segment themselves when the device found no entry.
  const bool candidate = c->bank_count >= 2 || (c->bank_count == 1 && block - 1 != 0);
  if (!c->dry) {
    const pr_sink_config& g = c->cfg;
    hipStream_t s = as_stream(stream);
    // the bank state of the last bank decision: not its entry copy, since the
    // entry it writes holds block-1, which this retrieval excludes (the other
    // entries were written by block-2's update at the latest); the whole update
    // of block-2 (entries this block may retrieve); the previous block's
    // attention, which read the state
    PRS_HIP(after(s, c->dec));
    if (block >= 2) PRS_HIP(after(s, c->done[block & 1]));
    PRS_HIP(after(s, c->attn));
    // r lands in the device state; attention reads bank entry r in place (its
    // K is kept rotated at the Dynamic Sink's place), so nothing is copied.
    // Nothing is rotated either: the window blocks' keys were rotated at every
    // window place when they were written, block 0's also at the Static
    // Sink's.
    PRS_HIP(launch_retrieve(fp_raw_dev, c->phi_cur(), c->phi_bank(), c->state(), g.fp_dim,
                            bank_rule(g), block, slot_out_dev, s));
    PRS_HIP(mark(s, c->retr));
  }
  c->dyn_present = candidate;
  c->open = true;
  std::fill(c->written.begin(), c->written.end(), 0);
  return PR_SINK_OK;
}

int pr_sink_attend(pr_sink_cache* c, int32_t layer, const void* q_raw, const void* k_cur_raw,
                   const void* v_cur_raw, void* out, void* stream) {
  return prsink::attend_with_workspace(c, layer, q_raw, k_cur_raw, v_cur_raw, out, stream, nullptr);
}

}  // extern "C"

bool prsink::cache_is_dry(const pr_sink_cache* c) { return c->dry; }

int prsink::report_hip_error(hipError_t e, const char* what) {
  return fail(PR_SINK_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// One attention call; ws == nullptr takes the per-call scratch from the arena.
int prsink::attend_with_workspace(pr_sink_cache* c, int32_t layer, const void* q_raw, const void* k_cur_raw,
                                  const void* v_cur_raw, void* out, void* stream, const AttendWorkspace* ws) {
  if (int e = check_layer(c, layer)) return e;
  if (int e = check_tensor(q_raw, "q_raw")) return e;
  if (int e = check_tensor(k_cur_raw, "k_cur_raw")) return e;
  if (int e = check_tensor(v_cur_raw, "v_cur_raw")) return e;
  if (int e = check_tensor(out, "out")) return e;
  if (out == q_raw || out == k_cur_raw || out == v_cur_raw) return fail(PR_SINK_EINVAL, "out aliases an input");
  if (!c->open) return fail(PR_SINK_ESTATE, "attend with no open block");
  if (ws && block_bytes(c, c->lay.tb) > ws->cur_rot_bytes)
    return fail(PR_SINK_EINVAL, "the current block's keys need %zu bytes of scratch, the workspace holds %zu",
                block_bytes(c, c->lay.tb), ws->cur_rot_bytes);
  if (c->dry) return PR_SINK_OK;
  const pr_sink_config& g = c->cfg;
  const Layout& L = c->lay;
  int tokens[kMaxSegments], t_index[kMaxSegments];
  segment_table(c, tokens, t_index);
  const int n_seg = g.window_slots + 3;
  hipStream_t st = as_stream(stream);
  // this layer's newest window block (the previous block's clean write; one
  // wait covers all layers when they went to one stream), the retrieval, this
  // layer's Ref Sink, and the previous call (attention calls share the
  // rotated-current-key scratch and the split-job records)
  PRS_HIP(after(st, c->clean_all_block == c->next_block - 1 ? c->clean_all : c->clean[layer]));
  PRS_HIP(after(st, c->retr));
  PRS_HIP(after(st, c->ref[layer]));
  PRS_HIP(after(st, c->attn));
  // the current block's keys, rotated at the current positions
  char* cur_rot = ws ? static_cast<char*>(ws->cur_rot) : c->arena + L.off_cur_rot;
  {
    RotParams r = rot_params(c, L.tb, 0);
    add_job(c, r, k_cur_raw, cur_rot, t_index[n_seg - 1]);
    PRS_HIP(launch_rope_follow(r, 1, st));
  }
  AttnParams p{};
  p.dyn_seg = -1;
  const int64_t D = g.head_dim;
  const int b = c->next_block;
  for (int s = 0; s < n_seg; ++s) {
    Segment& sg = p.seg[s];
    sg.count = tokens[s];
    sg.t_index = t_index[s];
    sg.tok = (int64_t)g.n_heads * D;
    sg.head = D;
    if (s == 0) {
      sg.k = c->ref_slot() + c->ref_r(layer);
      sg.v = c->ref_slot() + c->ref_v(layer);
    } else if (s == n_seg - 1) {  // current block: rotated copy, caller's V
      sg.k = cur_rot;
      sg.v = v_cur_raw;
    } else if (s == 2) {  // Dynamic Sink: bank entry r, resolved on the device
      sg.k = sg.v = nullptr;
      if (tokens[s] > 0) {
        p.dyn_seg = s;
        p.dyn_r = &c->state()->last_r;
        p.dyn_k0 = c->block_slot(c->bs_bank(0)) + c->blk_r(layer);
        p.dyn_v0 = c->block_slot(c->bs_bank(0)) + c->blk_v(layer);
        p.dyn_stride = (int64_t)L.slot_b;
      }
    } else if (s == 1) {  // Static Sink
      sg.k = c->block_slot(c->bs_static()) + c->blk_r(layer);
      sg.v = c->block_slot(c->bs_static()) + c->blk_v(layer);
    } else {  // window place s - 3: block b - (W-1) + (s-3)
      const int id = b - (g.window_slots - 1) + (s - 3);
      const int j = id >= 0 ? id % g.window_slots : 0;
      sg.k = c->window_rot(j, s - 3, layer);
      sg.v = c->block_slot(c->bs_window(j)) + c->blk_v(layer);
    }
  }
  p.q = q_raw;
  p.out = out;
  p.g = rope_geom(c);
  p.n_seg = n_seg;
  p.n_q = L.tb;
  p.n_heads = g.n_heads;
  p.q_t_index = t_index[n_seg - 1];
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)g.head_dim));
  p.dyn_may_vanish = (g.bank_policy & PR_SINK_BANK_ZERO_FALLBACK) != 0;
  // a caller-provided workspace carries no split-job records: every job runs whole
  p.part = L.n_part_rec && !ws ? reinterpret_cast<float*>(c->arena + L.off_part) : nullptr;
  p.cnt = L.n_cnt && !ws ? reinterpret_cast<uint32_t*>(c->arena + L.off_cnt) : nullptr;
  if (c->time_start) PRS_HIP(hipEventRecord(c->time_start, st));
  PRS_HIP(launch_attention(p, g.dtype, g.head_dim, c->n_cu, st));
  if (c->time_stop) PRS_HIP(hipEventRecord(c->time_stop, st));
  defer(st, c->attn);
  return PR_SINK_OK;
}

extern "C" {

int pr_sink_clean_kv_write(pr_sink_cache* c, int32_t layer, const void* k_raw, const void* v_raw,
                           void* stream) {
  if (int e = check_layer(c, layer)) return e;
  if (int e = check_tensor(k_raw, "k_raw")) return e;
  if (int e = check_tensor(v_raw, "v_raw")) return e;
  if (!c->open) return fail(PR_SINK_ESTATE, "clean_kv_write with no open block");
  if (c->written[layer]) return fail(PR_SINK_ESTATE, "layer %d already written for block %d", layer, c->next_block);
  if (!c->dry) {
    const Layout& L = c->lay;
    const int b = c->next_block;
    const pr_sink_config& g = c->cfg;
    char* w = c->block_slot(c->bs_window(b % g.window_slots));
    CleanWrite cw{};
    cw.k_src = static_cast<const char*>(k_raw);
    cw.v_src = static_cast<const char*>(v_raw);
    cw.cd = chunk_div(c, L.tb);
    cw.n_tok = L.tb;
    cw.n_heads = g.n_heads;
    cw.head_dim = g.head_dim;
    cw.elem = L.elem;
    // the window slot, with the keys rotated at each window place the block
    // takes from the next block on, newest first (none when the window holds
    // only the current block)
    const int j = b % g.window_slots;
    // raw keys only for a block that may enter the bank: the rotation of a new
    // bank entry at the Dynamic Sink's place is their only later reader
    const bool keep_raw = may_enter_bank(g, b);
    cw.dst[0].k = keep_raw ? c->window_raw(b % g.window_slots, layer) : nullptr;
    cw.dst[0].v = w + c->blk_v(layer);
    for (int p = g.window_slots - 2; p >= 0; --p) {
      CleanDst& d = cw.dst[0];
      d.k_rot[d.n_rot] = c->window_rot(j, p, layer);
      d.cs[d.n_rot++] = c->place_cs(c->window_t(p));
    }
    if (b == 0) {  // block 0 is also the Static Sink, from block 1 on
      char* st = c->block_slot(c->bs_static());
      CleanDst& d = cw.dst[1];
      d.k = nullptr;  // the Static Sink is attended rotated only: no raw keys
      d.v = st + c->blk_v(layer);
      d.k_rot[0] = st + c->blk_r(layer);
      d.cs[0] = c->place_cs(g.ref_frames);
      d.n_rot = 1;
    }
    // the window slot last held block b-W: its last reader was the previous
    // block's attention, which this block's retrieval waited for, and this
    // block's own attention reads other slots, so the write may overlap it.
    // Block b-W's bank copy also read the slot: with W >= 2 the retrieval's
    // wait for block b-2's update covers it, with W = 1 it is the last update,
    // so the write also waits for the last update's copies.
    // It also waits for the previous block's write of this layer (it may be on
    // another stream): an attention call of this block made after this write
    // waits on this layer's mark, which must then cover that write too.
    hipStream_t s = as_stream(stream);
    PRS_HIP(after(s, c->retr));
    PRS_HIP(after(s, c->bank));
    PRS_HIP(after(s, c->clean[layer]));
    PRS_HIP(launch_clean_write(cw, s));
    PRS_HIP(mark(s, c->clean[layer]));
    c->win_raw[(size_t)j * g.n_layers + layer] = keep_raw;
    const int n_written = (int)std::count(c->written.begin(), c->written.end(), (uint8_t)1);
    if (n_written == 0) {
      c->clean_stream = s;
      c->clean_one_stream = true;
    } else if (s != c->clean_stream) {
      c->clean_one_stream = false;
    }
    if (n_written + 1 == g.n_layers && c->clean_one_stream) {
      // the block's last clean write, and all of them on s: the next block's
      // attention waits once for them all
      PRS_HIP(mark(s, c->clean_all));
      c->clean_all_block = b;
    }
  }
  c->written[layer] = 1;
  return PR_SINK_OK;
}

int pr_sink_bank_update(pr_sink_cache* c, int32_t block, void* stream) {
  if (!c) return fail(PR_SINK_EINVAL, "cache is NULL");
  if (!c->open || block != c->next_block) return fail(PR_SINK_ESTATE, "bank_update(%d) but open block is %d", block, c->open ? c->next_block : -1);
  for (int l = 0; l < c->cfg.n_layers; ++l)
    if (!c->written[l]) return fail(PR_SINK_ESTATE, "clean K/V of layer %d not written for block %d", l, block);
  const pr_sink_config& g = c->cfg;
  hipStream_t s = as_stream(stream);
  const bool update = may_enter_bank(g, block);
  if (!c->dry) {
    // this block's retrieval (it wrote the fingerprint and the scores the
    // decision reads) and attention (it read bank entries as the Dynamic
    // Sink), and the previous update's copies (they read the copy plan the
    // decision below rewrites)
    PRS_HIP(after(s, c->retr));
    PRS_HIP(after(s, c->attn));
    PRS_HIP(after(s, c->bank));
  }
  // every clean write of this block: the bank copies the window slot, and the
  // block's completion mark covers them
  auto after_clean = [&]() -> hipError_t {
    for (auto& m : c->clean)
      if (hipError_t e = after(s, m)) return e;
    return hipSuccess;
  };
  if (update) {
    if (!c->dry) {
      const Layout& L = c->lay;
      const int ws = c->bs_window(block % g.window_slots);
      PRS_HIP(launch_bank_update(c->phi_cur(), c->phi_bank(), c->state(), g.fp_dim, bank_rule(g), block,
                                 ws, c->bs_bank(0), s));
      // the next retrieval needs the decision only (see pr_sink_retrieve)
      PRS_HIP(mark(s, c->dec));
      PRS_HIP(after_clean());
      // the written entry gets the block's V, and its K rotated at the
      // Dynamic Sink's place, the only place a bank entry is attended from
      // (rotated from the window slot's raw keys; an entry keeps no raw keys)
      PRS_HIP(launch_slot_copy(c->block_slot(0), L.slot_b, c->blk_v(0), L.kv_b * g.n_layers, c->state(), s));
      RotParams r = rot_params(c, L.tb, L.kv_b);
      add_job(c, r, c->window_raw(block % g.window_slots, 0), nullptr, g.ref_frames + g.block_frames);
      r.job[0].from_state = 1;
      r.job[0].dst_off = (int64_t)c->blk_r(0);
      PRS_HIP(launch_rope_follow(r, g.n_layers, s));
      PRS_HIP(mark(s, c->bank));
    }
    if (c->bank_count < g.bank_size) ++c->bank_count;
  }
  if (!c->dry) {
    PRS_HIP(after_clean());
    PRS_HIP(mark(s, c->done[block & 1]));
  }
  c->open = false;
  c->next_block = block + 1;
  return PR_SINK_OK;
}

int pr_sink_bank_state(pr_sink_cache* c, int32_t* ids_host, double* fp_host, int32_t* misc_host,
                       void* stream) {
  if (!c) return fail(PR_SINK_EINVAL, "cache is NULL");
  if (!ids_host) return fail(PR_SINK_EINVAL, "ids_host is NULL");
  if (c->dry) return fail(PR_SINK_EINVAL, "dry-run cache has no device state");
  hipStream_t s = as_stream(stream);
  // the state is written by retrievals and bank updates, possibly on other streams
  PRS_HIP(after(s, c->retr));
  PRS_HIP(after(s, c->bank));
  DevState st;
  PRS_HIP(hipMemcpyAsync(&st, c->state(), sizeof st, hipMemcpyDeviceToHost, s));
  if (fp_host)
    PRS_HIP(hipMemcpyAsync(fp_host, c->phi_bank(), sizeof(double) * c->cfg.bank_size * c->cfg.fp_dim,
                           hipMemcpyDeviceToHost, s));
  PRS_HIP(hipStreamSynchronize(s));
  for (int i = 0; i < c->cfg.bank_size; ++i) ids_host[i] = st.ids[i];
  if (misc_host) {
    misc_host[0] = st.last_r;
    misc_host[1] = st.dyn_id;
    misc_host[2] = st.decision;
  }
  return PR_SINK_OK;
}

int pr_sink_slot_view(const pr_sink_cache* c, int32_t slot, int32_t layer, void** k_dev,
                      void** v_dev, void** k_rot_dev, int32_t* t_pad_out) {
  if (int e = check_layer(c, layer)) return e;
  if (!k_dev || !v_dev || !t_pad_out) return fail(PR_SINK_EINVAL, "NULL output pointer");
  if (c->dry) return fail(PR_SINK_EINVAL, "dry-run cache has no arena");
  const Layout& L = c->lay;
  const int n_slots = 2 + L.n_block_slots;  // Ref, the Dynamic id, the block slots
  if (slot < 0 || slot >= n_slots) return fail(PR_SINK_EINVAL, "slot %d out of range", slot);
  if (slot == PR_SINK_SLOT_DYNAMIC)
    return fail(PR_SINK_EINVAL, "the Dynamic Sink is bank entry r (pr_sink_retrieve's slot_out), not a slot of its own; view that bank entry");
  if (slot == PR_SINK_SLOT_REF) {
    char* base = c->ref_slot();
    *t_pad_out = L.tr_pad;
    *k_dev = base + c->ref_k(layer);
    *v_dev = base + c->ref_v(layer);
    if (k_rot_dev) *k_rot_dev = base + c->ref_r(layer);
    return PR_SINK_OK;
  }
  // raw keys are kept for the window slots only
  const bool window = slot >= PR_SINK_SLOT_WINDOW0 && slot < PR_SINK_SLOT_WINDOW0 + c->cfg.window_slots;
  char* base = c->block_slot(slot == PR_SINK_SLOT_STATIC ? c->bs_static() : slot - PR_SINK_SLOT_WINDOW0 + 1);
  *t_pad_out = L.tb_pad;
  const int j = slot - PR_SINK_SLOT_WINDOW0;
  *k_dev = window && c->win_raw[(size_t)j * c->cfg.n_layers + layer] ? c->window_raw(j, layer) : nullptr;
  *v_dev = base + c->blk_v(layer);
  if (k_rot_dev) *k_rot_dev = base + c->blk_r(layer);
  const int W = c->cfg.window_slots;
  if (k_rot_dev && W >= 2 && slot >= PR_SINK_SLOT_WINDOW0 && slot < PR_SINK_SLOT_WINDOW0 + W) {
    // the copy at the place the slot's block holds in the window of the open
    // (else the next) block b: block b-W+d sits at place d-1; d = 0 is the
    // block written in block b, or the one that left the window (newest place)
    const int b = c->next_block;
    const int d = ((j - b) % W + W) % W;
    *k_rot_dev = c->window_rot(j, d == 0 ? W - 2 : d - 1, layer);
  }
  return PR_SINK_OK;
}

int pr_sink_segments(const pr_sink_cache* c, int32_t* tokens_out, int32_t* t_start_out,
                     int32_t* n_out) {
  if (!c) return fail(PR_SINK_EINVAL, "cache is NULL");
  if (!tokens_out || !t_start_out || !n_out) return fail(PR_SINK_EINVAL, "NULL output pointer");
  if (!c->open) return fail(PR_SINK_ESTATE, "no open block");
  int tokens[kMaxSegments], t_index[kMaxSegments];
  segment_table(c, tokens, t_index);
  const int n = c->cfg.window_slots + 3;
  for (int s = 0; s < n; ++s) {
    tokens_out[s] = tokens[s];
    t_start_out[s] = c->cfg.t0 + t_index[s];
  }
  *n_out = n;
  return PR_SINK_OK;
}

int pr_sink_set_attend_events(pr_sink_cache* c, void* ev_start, void* ev_stop) {
  if (!c) return fail(PR_SINK_EINVAL, "cache is NULL");
  if ((ev_start == nullptr) != (ev_stop == nullptr)) return fail(PR_SINK_EINVAL, "set both events or neither");
  c->time_start = static_cast<hipEvent_t>(ev_start);
  c->time_stop = static_cast<hipEvent_t>(ev_stop);
  return PR_SINK_OK;
}

int pr_sink_cache_destroy(pr_sink_cache* c) {
  delete c;
  return PR_SINK_OK;
}

const char* pr_sink_last_error(void) { return g_err.c_str(); }

}  // extern "C"
