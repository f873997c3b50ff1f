// Internal interface between the host-side validation (pfa_api.cpp, plain C++) and the HIP
// launcher (pfa_kernel.hip). Not part of the public ABI.
#pragma once

#include <stdint.h>

namespace pfa {

// Everything one launch needs, already validated.
struct Launch {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* key_mask;  // may be null
  void* o;
  int batch, hq, hkv, group, lq, sk, d;
  float scale;
  int causal_offset;        // < 0: no causal term
  int window;               // > 0 only with the causal term
  unsigned flags;
  void* stream;
};

// Query rows handled by one workgroup of the prefill kernel.
int rows_per_block(int d);

// Number of workgroups the launch will use (64-bit; the caller checks it fits the grid).
long long grid_blocks(const Launch& p);

// Enqueue the prefill kernel. Returns PFA_OK or PFA_ERR_LAUNCH.
int launch_prefill(const Launch& p);

}  // namespace pfa
