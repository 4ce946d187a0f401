// Sanitizer driver for the host side of the PR-Sink C ABI (include/pr_sink.h).
//
// Built host-only with -fsanitize=address,undefined against hip_stub.cpp (no
// GPU, no HIP runtime): every call of the ABI runs its real validation, state
// machine, arena layout and launch-parameter code, the stubs check that each
// kernel would stay inside the arena or the caller's tensors, and the logged
// stream/event traffic is checked for the cross-stream order the header
// promises.  Exit status 0 and the line "abi_check: ALL OK" mean every check
// passed; each failure prints one line.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "hip_stub.h"
#include "pr_sink.h"

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                         \
  do {                                                           \
    if (!(cond)) {                                               \
      ++g_failures;                                              \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);  \
      std::fprintf(stderr, __VA_ARGS__);                         \
      std::fprintf(stderr, "\n");                                \
    }                                                            \
  } while (0)

pr_sink_config small_config(int dtype, int window, int bank) {
  pr_sink_config c;
  std::memset(&c, 0, sizeof c);
  c.n_layers = 2;
  c.n_heads = 3;
  c.head_dim = 64;
  c.rope_dims[0] = 24;
  c.rope_dims[1] = 20;
  c.rope_dims[2] = 20;
  c.rope_theta = 1e4;
  c.lat_h = 5;
  c.lat_w = 7;  // 35 tokens per frame: ragged against 64-key tiles
  c.ref_frames = 1;
  c.block_frames = 2;
  c.window_slots = window;
  c.bank_size = bank;
  c.bank_fill_blocks = 6;
  c.fp_dim = 558;
  c.dtype = dtype;
  c.t0 = 0;
  c.bank_policy = 0;
  c.bank_stale_blocks = 1;
  c.bank_refresh_tau = 0.0;
  return c;
}

// Host buffers standing in for device memory, registered with the stubs.
struct Buf {
  void* p = nullptr;
  size_t n = 0;
  Buf(size_t bytes, const char* name) : n(bytes) {
    const size_t r = (bytes + 4095) / 4096 * 4096;
    p = std::aligned_alloc(4096, r ? r : 4096);
    std::memset(p, 0, r ? r : 4096);
    stub::register_buffer(p, bytes, name);
  }
  ~Buf() { std::free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

// Launches logged during one ABI call.
struct Span {
  size_t begin, end;
  bool empty() const { return begin == end; }
};
template <class F>
Span logged(F&& f) {
  const size_t b = stub::launches().size();
  f();
  return Span{b, stub::launches().size()};
}
// Every launch of `a` is ordered before every launch of `b`.
bool ordered(const Span& a, const Span& b) {
  if (a.empty() || b.empty()) return true;
  const auto& L = stub::launches();
  return stub::happens_before(L[a.end - 1], L[b.begin]);
}

void* fake_stream(uintptr_t v) { return reinterpret_cast<void*>(v); }

// ---------------------------------------------------------------------------
void dry_run_checks() {
  pr_sink_config c = small_config(PR_SINK_BF16, 3, 5);
  CHECK(pr_sink_arena_bytes(&c) > 0, "arena bytes of a valid config");
  pr_sink_config bad = c;
  bad.head_dim = 96;
  CHECK(pr_sink_arena_bytes(&bad) == 0 && std::strlen(pr_sink_last_error()) > 0, "head_dim 96 rejected");
  bad = c;
  bad.rope_dims[2] = 18;
  CHECK(pr_sink_arena_bytes(&bad) == 0, "rope bands that do not sum to head_dim rejected");
  bad = c;
  bad.window_slots = 6;
  CHECK(pr_sink_arena_bytes(&bad) == 0, "window of 6 rejected");
  CHECK(pr_sink_arena_bytes(nullptr) == 0, "NULL config rejected");

  pr_sink_cache* h = nullptr;
  CHECK(pr_sink_cache_init(&c, nullptr, 0, nullptr, &h) == PR_SINK_OK && h, "dry-run init");
  alignas(16) static char fake[64];
  void* t = fake;
  void* mis = fake + 2;
  float fp[558] = {};
  CHECK(pr_sink_retrieve(h, 0, fp, nullptr, nullptr) == PR_SINK_ESTATE, "retrieve before the Ref Sink");
  for (int l = 0; l < c.n_layers; ++l) CHECK(pr_sink_set_ref(h, l, t, t, nullptr) == PR_SINK_OK, "set_ref");
  CHECK(pr_sink_set_ref(h, c.n_layers, t, t, nullptr) == PR_SINK_EINVAL, "set_ref layer out of range");
  CHECK(pr_sink_set_ref(h, 0, mis, t, nullptr) == PR_SINK_EINVAL, "misaligned k rejected");
  CHECK(pr_sink_attend(h, 0, t, t, t, fake + 16, nullptr) == PR_SINK_ESTATE, "attend with no open block");
  CHECK(pr_sink_retrieve(h, 1, fp, nullptr, nullptr) == PR_SINK_ESTATE, "block 1 before block 0");
  CHECK(pr_sink_retrieve(h, 0, fp, nullptr, nullptr) == PR_SINK_OK, "retrieve block 0");
  CHECK(pr_sink_set_ref(h, 0, t, t, nullptr) == PR_SINK_ESTATE, "set_ref while a block is open");
  CHECK(pr_sink_attend(h, 0, t, t, t, t, nullptr) == PR_SINK_EINVAL, "out aliasing q rejected");
  CHECK(pr_sink_attend(h, 0, t, t, t, fake + 16, nullptr) == PR_SINK_OK, "attend");
  CHECK(pr_sink_bank_update(h, 0, nullptr) == PR_SINK_ESTATE, "bank_update before the clean writes");
  CHECK(pr_sink_clean_kv_write(h, 0, t, t, nullptr) == PR_SINK_OK, "clean write layer 0");
  CHECK(pr_sink_clean_kv_write(h, 0, t, t, nullptr) == PR_SINK_ESTATE, "second clean write of a layer");
  CHECK(pr_sink_clean_kv_write(h, 1, t, t, nullptr) == PR_SINK_OK, "clean write layer 1");
  int32_t tok[8], ts[8], n = 0;
  CHECK(pr_sink_segments(h, tok, ts, &n) == PR_SINK_OK && n == c.window_slots + 3, "segments");
  CHECK(tok[0] == 35 && tok[1] == 0 && tok[2] == 0 && tok[n - 1] == 70, "segment token counts of block 0");
  CHECK(pr_sink_bank_update(h, 1, nullptr) == PR_SINK_ESTATE, "bank_update of the wrong block");
  CHECK(pr_sink_bank_update(h, 0, nullptr) == PR_SINK_OK, "bank_update");
  CHECK(pr_sink_segments(h, tok, ts, &n) == PR_SINK_ESTATE, "segments with no open block");
  void *k, *v, *r;
  int32_t tp;
  CHECK(pr_sink_slot_view(h, PR_SINK_SLOT_REF, 0, &k, &v, &r, &tp) == PR_SINK_EINVAL, "no view of a dry cache");
  int32_t ids[5];
  CHECK(pr_sink_bank_state(h, ids, nullptr, nullptr, nullptr) == PR_SINK_EINVAL, "no bank state of a dry cache");
  CHECK(pr_sink_set_attend_events(h, fake, nullptr) == PR_SINK_EINVAL, "one event without the other");
  CHECK(pr_sink_cache_destroy(h) == PR_SINK_OK, "destroy");
  // a config that is valid but an arena that is too small
  Buf tiny(4096, "tiny arena");
  CHECK(pr_sink_cache_init(&c, tiny.p, tiny.n, nullptr, &h) == PR_SINK_ENOSPACE && h == nullptr, "small arena");
}

// ---------------------------------------------------------------------------
// A stream of blocks on a host "arena": every launch bounds-checked, then the
// cross-stream order of the clean-KV path on a second stream.
struct Rig {
  pr_sink_config c;
  size_t row;
  int T, Tr;
  std::vector<Buf*> bufs;
  Buf* arena;
  pr_sink_cache* h = nullptr;
  void *q, *kc, *vc, *out, *kr, *vr;
  float* fp;
  int32_t* slot;

  explicit Rig(const pr_sink_config& cfg) : c(cfg) {
    const size_t elem = c.dtype == PR_SINK_BF16 ? 2 : 4;
    row = (size_t)c.n_heads * c.head_dim * elem;
    T = c.lat_h * c.lat_w * c.block_frames;
    Tr = c.lat_h * c.lat_w * c.ref_frames;
    arena = add(pr_sink_arena_bytes(&c), "arena");
    q = add(T * row, "q")->p;
    kc = add(T * row, "k")->p;
    vc = add(T * row, "v")->p;
    out = add(T * row, "out")->p;
    kr = add(Tr * row, "k_ref")->p;
    vr = add(Tr * row, "v_ref")->p;
    fp = static_cast<float*>(add(sizeof(float) * c.fp_dim, "fingerprint")->p);
    slot = static_cast<int32_t*>(add(4, "slot_out")->p);
    stub::bank_size_hint = c.bank_size;
    stub::block_slots_hint = 1 + c.window_slots + c.bank_size;
    CHECK(pr_sink_cache_init(&c, arena->p, arena->n, nullptr, &h) == PR_SINK_OK, "init: %s", pr_sink_last_error());
  }
  Buf* add(size_t n, const char* name) {
    bufs.push_back(new Buf(n, name));
    return bufs.back();
  }
  ~Rig() {
    pr_sink_cache_destroy(h);
    for (Buf* b : bufs) delete b;
  }
};

// mixed: attention calls alternate between the two streams, and in odd
// blocks the clean write of layer 0 goes to the attention stream, so the
// marks recorded on first use and the one-wait-per-block path for clean
// writes on one stream are crossed with their fallbacks.
void stream_checks(int dtype, int window, int bank, bool mixed) {
  stub::reset_log();
  Rig g(small_config(dtype, window, bank));
  const pr_sink_config& c = g.c;
  void* const A = fake_stream(0x1000);
  void* const B = fake_stream(0x2000);

  // Ref Sink writes for alternating layers on two streams, then layer 0 again
  // on the other stream: the rewrite is ordered after the first write of its
  // layer, and each layer's attention after that layer's last write.
  std::vector<Span> ref(c.n_layers);
  for (int l = 0; l < c.n_layers; ++l)
    ref[l] = logged([&] { CHECK(pr_sink_set_ref(g.h, l, g.kr, g.vr, l % 2 ? B : A) == PR_SINK_OK, "set_ref"); });
  const Span ref0_again = logged([&] { pr_sink_set_ref(g.h, 0, g.kr, g.vr, B); });
  CHECK(ordered(ref[0], ref0_again), "a second Ref write of layer 0 on another stream waits for the first");
  ref[0] = ref0_again;

  const int n_blocks = c.bank_fill_blocks + 4;
  std::vector<std::vector<Span>> attn(n_blocks), clean(n_blocks);
  std::vector<Span> retr(n_blocks), upd(n_blocks);
  for (int b = 0; b < n_blocks; ++b) {
    g.fp[b % c.fp_dim] = 1.0f;
    retr[b] = logged([&] { CHECK(pr_sink_retrieve(g.h, b, g.fp, g.slot, A) == PR_SINK_OK, "retrieve %d", b); });
    for (int s = 0; s < 3; ++s)
      for (int l = 0; l < c.n_layers; ++l)
        attn[b].push_back(logged([&] {
          void* const st = mixed && (s * c.n_layers + l) % 2 ? B : A;
          CHECK(pr_sink_attend(g.h, l, g.q, g.kc, g.vc, g.out, st) == PR_SINK_OK, "attend: %s", pr_sink_last_error());
        }));
    for (int l = 0; l < c.n_layers; ++l)
      clean[b].push_back(logged([&] {
        void* const st = mixed && b % 2 && l == 0 ? A : B;
        CHECK(pr_sink_clean_kv_write(g.h, l, g.kc, g.vc, st) == PR_SINK_OK, "clean");
      }));
    upd[b] = logged([&] { CHECK(pr_sink_bank_update(g.h, b, B) == PR_SINK_OK, "bank_update %d", b); });
  }
  for (int b = 0; b < n_blocks; ++b) {
    for (int i = 0; i < (int)attn[b].size(); ++i) {
      const int l = i % c.n_layers;
      if (b == 0) CHECK(ordered(ref[l], attn[b][i]), "attention of layer %d after its Ref Sink", l);
      CHECK(ordered(retr[b], attn[b][i]), "attention after the block's retrieval");
      if (b > 0) CHECK(ordered(clean[b - 1][l], attn[b][i]), "block %d attention of layer %d after the clean write", b, l);
      // attention calls share the rotated-current-key scratch and split records
      if (i > 0) CHECK(ordered(attn[b][i - 1], attn[b][i]), "block %d attention call %d after the previous one", b, i);
      if (i == 0 && b > 0) CHECK(ordered(attn[b - 1].back(), attn[b][i]), "block %d first attention after the last", b);
    }
    for (int l = 0; l < c.n_layers; ++l) {
      CHECK(ordered(retr[b], clean[b][l]), "clean write after its block's retrieval");
      // the slot it fills held block b-W, last read by block b-1's attention
      if (b > 0)
        for (const Span& a : attn[b - 1]) CHECK(ordered(a, clean[b][l]), "clean write %d after the previous block's attention", b);
      // the update's decision kernel reads only fingerprints; its copies read
      // the window slot the clean writes fill
      if (upd[b].end - upd[b].begin > 1)
        CHECK(ordered(clean[b][l], Span{upd[b].begin + 1, upd[b].end}), "bank copies after the block's clean writes");
    }
    for (const Span& a : attn[b]) CHECK(ordered(a, upd[b]), "bank update %d after the block's attention", b);
    if (b + 1 < n_blocks) CHECK(ordered(Span{upd[b].begin, upd[b].begin + (upd[b].empty() ? 0 : 1)}, retr[b + 1]),
                                "retrieval %d after the previous bank decision", b + 1);
    if (b + 2 < n_blocks) CHECK(ordered(upd[b], retr[b + 2]), "retrieval %d after the whole update of block %d", b + 2, b);
    CHECK(upd[b].empty() == (b >= c.bank_fill_blocks), "bank update launches only in the fill phase");
  }
  int32_t ids[8], misc[3];
  double phi[8 * 558];
  CHECK(pr_sink_bank_state(g.h, ids, phi, misc, A) == PR_SINK_OK, "bank_state");
  for (const std::string& e : stub::errors())
    CHECK(false, "dtype %d window %d bank %d mixed %d: %s", dtype, window, bank, (int)mixed, e.c_str());
}

// Attention calls interleaved with the clean writes of their block, over three
// streams: attention and retrieval on A, bank updates on B, clean writes on A,
// B or C.  In odd blocks each layer's clean K/V is written before the layer's
// first attention call, on A, so that call needs no wait for it: the call must
// still be ordered after the previous block's write of the layer, which went
// to B or C.
void interleaved_checks(int dtype, int window, int bank) {
  stub::reset_log();
  Rig g(small_config(dtype, window, bank));
  const pr_sink_config& c = g.c;
  void* const A = fake_stream(0x3000);
  void* const B = fake_stream(0x4000);
  void* const C = fake_stream(0x5000);
  for (int l = 0; l < c.n_layers; ++l)
    CHECK(pr_sink_set_ref(g.h, l, g.kr, g.vr, A) == PR_SINK_OK, "set_ref");
  const int n_blocks = c.bank_fill_blocks + 4;
  std::vector<std::vector<std::vector<Span>>> attn(n_blocks, std::vector<std::vector<Span>>(c.n_layers));
  std::vector<std::vector<Span>> clean(n_blocks, std::vector<Span>(c.n_layers));
  auto attend = [&](int b, int l) {
    attn[b][l].push_back(logged([&] { CHECK(pr_sink_attend(g.h, l, g.q, g.kc, g.vc, g.out, A) == PR_SINK_OK, "attend"); }));
  };
  for (int b = 0; b < n_blocks; ++b) {
    g.fp[(3 * b) % c.fp_dim] = 1.0f;
    CHECK(pr_sink_retrieve(g.h, b, g.fp, g.slot, A) == PR_SINK_OK, "retrieve %d", b);
    for (int l = 0; l < c.n_layers; ++l) {
      // odd blocks write each layer first, on A; even blocks attend first and
      // write on C (layer 0) or B
      const bool write_first = b % 2 == 1;
      if (!write_first) attend(b, l);
      clean[b][l] = logged([&] {
        void* const st = write_first ? A : (l == 0 ? C : B);
        CHECK(pr_sink_clean_kv_write(g.h, l, g.kc, g.vc, st) == PR_SINK_OK, "clean");
      });
      attend(b, l);
    }
    CHECK(pr_sink_bank_update(g.h, b, B) == PR_SINK_OK, "bank_update %d", b);
  }
  for (int b = 1; b < n_blocks; ++b)
    for (int l = 0; l < c.n_layers; ++l) {
      for (const Span& a : attn[b][l])
        CHECK(ordered(clean[b - 1][l], a), "interleaved: block %d attention of layer %d after the clean write", b, l);
      for (int l2 = 0; l2 < c.n_layers; ++l2)
        for (const Span& a : attn[b - 1][l2])
          CHECK(ordered(a, clean[b][l]), "interleaved: clean write %d after the previous block's attention", b);
    }
  for (const std::string& e : stub::errors())
    CHECK(false, "interleaved dtype %d window %d bank %d: %s", dtype, window, bank, e.c_str());
}

}  // namespace

int main() {
  dry_run_checks();
  for (int dtype : {PR_SINK_BF16, PR_SINK_F32})
    for (int w : {1, 2, 3, 5})
      for (bool mixed : {false, true}) stream_checks(dtype, w, w == 5 ? 8 : 5, mixed);
  for (int w : {1, 3}) interleaved_checks(PR_SINK_BF16, w, 5);
  CHECK(stub::live_events() == 0, "%d HIP events leaked", stub::live_events());
  if (g_failures) {
    std::printf("abi_check: %d failures\n", g_failures);
    return 1;
  }
  std::printf("abi_check: ALL OK\n");
  return 0;
}
