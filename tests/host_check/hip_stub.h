// Interface of the host-only HIP stand-ins (hip_stub.cpp) to the sanitizer
// driver (abi_check.cpp).
#pragma once

#include <map>
#include <string>
#include <vector>

namespace stub {

// One logged kernel launch: its kind, fake stream, position on that stream and
// the stream's vector clock at launch time.
struct Launch {
  std::string kind;
  const void* stream;
  long seq;
  std::map<const void*, long> clock;
};

// Buffers a kernel may touch: the arena and the caller's tensors.
void register_buffer(const void* p, size_t n, const char* name);
void reset_log();
const std::vector<Launch>& launches();
const std::vector<std::string>& errors();
int live_events();
// a is ordered before b (same stream, or through recorded events and waits).
bool happens_before(const Launch& a, const Launch& b);

// Set by the driver for the cache under test: the bank size and the number of
// block slots, the index ranges that device-resolved addresses can take.
inline int bank_size_hint = 0;
inline int block_slots_hint = 0;

}  // namespace stub
