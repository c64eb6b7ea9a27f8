// tls_api_internal.h -- shape derivation and error plumbing shared by the C ABI
// translation units (tls_api.cpp, offload.cpp). Internal.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tls.h"

namespace tls {

// Candidate tokens per pair the token stage handles (Kb'*bs): one 1024-thread
// workgroup keeps at most 16 keys per thread.

struct Derived {
  int B, Hq, Hkv, G, D, DV, row, v_off, bs, r, kb, kt, pairs;
  int64_t N, NB;    // tokens and blocks of every sequence
  int64_t Ns, NBs;  // allocated tokens and blocks per sequence (the strides)
  float sm;
};

int derive(const tls_shape_t* s, Derived* d);
int set_error(int code, const char* fmt, ...);
void clear_error();
int hip_error(hipError_t e, const char* what);
// Events registered with tls_profile_events for kernel `which` (NULL: none).
void profile_events(int which, hipEvent_t* start, hipEvent_t* end);
bool aligned(const void* p, size_t a);
size_t ws_bytes(const Derived& d, int which);

}  // namespace tls
