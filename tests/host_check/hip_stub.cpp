// Host-only stand-ins for the HIP runtime calls and the kernel launchers that
// prsink_host.cpp makes, for the sanitizer build of the C ABI (ASan + UBSan,
// no GPU).  They do two checks the real runtime cannot do on the CPU:
//
//   * bounds: every region a kernel would read or write (computed from its
//     launch parameters the way the kernel computes its addresses) must lie
//     inside one buffer the driver registered (the arena, or a caller tensor);
//     memset/memcpy on the "device" really run on host memory, so ASan sees
//     any overrun of the arena by the host code itself;
//   * order: each launch, event record and stream wait is logged against a
//     fake stream, and a vector clock per stream gives the happens-before
//     order of launches, so the driver can check that a consumer launched on
//     one stream is ordered after its producer on another.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "hip_stub.h"
#include "prsink_internal.h"

namespace stub {

namespace {
struct Range { const char* p; size_t n; std::string name; };
std::vector<Range> g_ranges;
std::vector<Launch> g_launches;
std::vector<std::string> g_errors;
int g_live_events = 0;

// Vector clock over the fake streams (keyed by handle value).
typedef std::map<const void*, long> Clock;
std::map<const void*, Clock> g_stream_clock;
std::map<const void*, long> g_stream_seq;

struct Event { Clock clock; bool recorded = false; };

void error(const std::string& msg) { g_errors.push_back(msg); }

void inside(const void* p, size_t n, const char* what) {
  if (n == 0) return;
  const char* c = static_cast<const char*>(p);
  for (const Range& r : g_ranges)
    if (c >= r.p && c + n <= r.p + r.n) return;
  char buf[256];
  snprintf(buf, sizeof buf, "%s: %zu bytes at %p lie outside every registered buffer", what, n, p);
  error(buf);
}

const void* key(hipStream_t s) { return reinterpret_cast<const void*>(s); }

void log_launch(const char* kind, hipStream_t s) {
  const void* k = key(s);
  const long seq = ++g_stream_seq[k];
  Clock& c = g_stream_clock[k];
  c[k] = seq;
  g_launches.push_back(Launch{kind, k, seq, c});
}
}  // namespace

void register_buffer(const void* p, size_t n, const char* name) {
  g_ranges.push_back(Range{static_cast<const char*>(p), n, name});
}
void reset_log() {
  g_launches.clear();
  g_errors.clear();
}
const std::vector<Launch>& launches() { return g_launches; }
const std::vector<std::string>& errors() { return g_errors; }
int live_events() { return g_live_events; }

bool happens_before(const Launch& a, const Launch& b) {
  auto it = b.clock.find(a.stream);
  return it != b.clock.end() && it->second >= a.seq;
}

}  // namespace stub

using stub::inside;

// ---- HIP runtime calls ------------------------------------------------------
hipError_t hipGetDevice(int* id) {
  *id = 0;
  return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int) {
  std::memset(prop, 0, sizeof *prop);
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  prop->multiProcessorCount = 256;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub error"; }
hipError_t hipMemsetAsync(void* dst, int value, size_t n, hipStream_t) {
  inside(dst, n, "hipMemsetAsync");
  std::memset(dst, value, n);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipEventCreateWithFlags(hipEvent_t* ev, unsigned) {
  *ev = reinterpret_cast<hipEvent_t>(new stub::Event());
  ++stub::g_live_events;
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t ev) {
  delete reinterpret_cast<stub::Event*>(ev);
  --stub::g_live_events;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t ev, hipStream_t s) {
  stub::Event* e = reinterpret_cast<stub::Event*>(ev);
  e->clock = stub::g_stream_clock[stub::key(s)];
  e->recorded = true;
  return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t ev, unsigned) {
  stub::Event* e = reinterpret_cast<stub::Event*>(ev);
  if (!e->recorded) stub::error("hipStreamWaitEvent on an event never recorded");
  stub::Clock& c = stub::g_stream_clock[stub::key(s)];
  for (const auto& kv : e->clock)
    if (c[kv.first] < kv.second) c[kv.first] = kv.second;
  return hipSuccess;
}

// ---- kernel launchers: bounds of every region, then a log entry ---------------
namespace prsink {

hipError_t launch_attention(const AttnParams& p, int dtype, int head_dim, int n_cu, hipStream_t s) {
  const size_t elem = dtype == 0 ? 2 : 4;
  if (n_cu != 256) stub::error("launch_attention: unexpected CU count");
  for (int i = 0; i < p.n_seg; ++i) {
    const Segment& g = p.seg[i];
    if (g.tok != (int64_t)p.n_heads * head_dim || g.head != head_dim) stub::error("attention: segment strides");
    const size_t n = (size_t)g.count * g.tok * elem;
    if (i == p.dyn_seg) {
      for (int r = 0; r < kMaxBank; ++r) {  // any entry the device may pick (checked up to the bank size by the driver)
        if (r >= stub::bank_size_hint) break;
        inside(p.dyn_k0 + (size_t)r * p.dyn_stride, n, "attention: Dynamic K");
        inside(p.dyn_v0 + (size_t)r * p.dyn_stride, n, "attention: Dynamic V");
      }
    } else if (g.count > 0) {
      inside(g.k, n, "attention: segment K");
      inside(g.v, n, "attention: segment V");
    }
  }
  const size_t qn = (size_t)p.n_q * p.n_heads * head_dim * elem;
  inside(p.q, qn, "attention: q");
  inside(p.out, qn, "attention: out");
  if (dtype == 0) {
    if (!p.part || !p.cnt) stub::error("attention: bf16 needs the split workspace");
  }
  stub::log_launch("attention", s);
  return hipSuccess;
}

hipError_t launch_rope_follow(const RotParams& p, int n_layers, hipStream_t s) {
  const size_t n = (size_t)p.n_tok * p.n_heads * p.head_dim * p.elem;
  for (int j = 0; j < p.n_jobs; ++j) {
    const RotJob& jb = p.job[j];
    inside(jb.cs, (size_t)p.n_tok * p.cd.np * 8, "rope_follow: cos/sin table of the place");
    if (p.cd.per_tok * 16 != (uint32_t)(p.n_heads * p.head_dim * p.elem)) stub::error("rope_follow: chunks per token");
    for (int l = 0; l < n_layers; ++l) {
      inside(jb.src + (size_t)l * p.layer_bytes, n, "rope_follow: source");
      if (jb.from_state) {
        for (int d = 0; d < stub::block_slots_hint; ++d)
          inside(p.block_base + (size_t)d * p.slot_bytes + jb.dst_off + (size_t)l * p.layer_bytes, n,
                 "rope_follow: destination from state");
      } else {
        inside(jb.dst + (size_t)l * p.layer_bytes, n, "rope_follow: destination");
      }
    }
  }
  stub::log_launch("rope_follow", s);
  return hipSuccess;
}

hipError_t launch_kv_write(const void* k_src, const void* v_src, void* k0, void* v0, void* k1, void* v1,
                           size_t bytes, hipStream_t s) {
  inside(k_src, bytes, "kv_write: k");
  inside(v_src, bytes, "kv_write: v");
  inside(k0, bytes, "kv_write: k destination");
  inside(v0, bytes, "kv_write: v destination");
  if (k1) inside(k1, bytes, "kv_write: k destination 2");
  if (v1) inside(v1, bytes, "kv_write: v destination 2");
  stub::log_launch("kv_write", s);
  return hipSuccess;
}

hipError_t launch_clean_write(const CleanWrite& p, hipStream_t s) {
  const size_t n = (size_t)p.n_tok * p.n_heads * p.head_dim * p.elem;
  inside(p.k_src, n, "clean_write: k");
  inside(p.v_src, n, "clean_write: v");
  for (const CleanDst& d : p.dst) {
    if (!d.v) continue;
    if (d.k) inside(d.k, n, "clean_write: raw K destination");
    inside(d.v, n, "clean_write: V destination");
    for (int r = 0; r < d.n_rot; ++r) {
      inside(d.k_rot[r], n, "clean_write: rotated K destination");
      inside(d.cs[r], (size_t)p.n_tok * p.cd.np * 8, "clean_write: cos/sin table of the place");
    }
  }
  stub::log_launch("clean_write", s);
  return hipSuccess;
}

hipError_t launch_slot_copy(char* base, size_t slot_bytes, size_t copy_off, size_t copy_bytes, const DevState* st,
                            hipStream_t s) {
  if (copy_off + copy_bytes > slot_bytes) stub::error("slot_copy: range past the slot");
  for (int d = 0; d < stub::block_slots_hint; ++d)
    inside(base + (size_t)d * slot_bytes + copy_off, copy_bytes, "slot_copy");
  inside(st, sizeof *st, "slot_copy: state");
  stub::log_launch("slot_copy", s);
  return hipSuccess;
}

hipError_t launch_retrieve(const float* fp_raw, double* phi_cur, const double* bank_phi, DevState* st,
                           int fp_dim, const BankRule& rule, int, int32_t* slot_out, hipStream_t s) {
  inside(fp_raw, sizeof(float) * fp_dim, "retrieve: fingerprint");
  inside(phi_cur, sizeof(double) * fp_dim, "retrieve: phi_cur");
  inside(bank_phi, sizeof(double) * fp_dim * rule.size, "retrieve: bank phi");
  inside(st, sizeof *st, "retrieve: state");
  if (slot_out) inside(slot_out, 4, "retrieve: slot_out");
  stub::log_launch("retrieve", s);
  return hipSuccess;
}

hipError_t launch_bank_update(const double* phi_cur, double* bank_phi, DevState* st, int fp_dim,
                              const BankRule& rule, int, int win_slot, int bank_slot0, hipStream_t s) {
  inside(phi_cur, sizeof(double) * fp_dim, "bank_update: phi_cur");
  inside(bank_phi, sizeof(double) * fp_dim * rule.size, "bank_update: bank phi");
  inside(st, sizeof *st, "bank_update: state");
  if (win_slot < 0 || bank_slot0 + rule.size > stub::block_slots_hint) stub::error("bank_update: slot indices");
  stub::log_launch("bank_update", s);
  return hipSuccess;
}

hipError_t launch_state_init(DevState* st, hipStream_t s) {
  inside(st, sizeof *st, "state_init");
  stub::log_launch("state_init", s);
  return hipSuccess;
}

}  // namespace prsink
