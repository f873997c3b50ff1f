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
  int causal;               // causal term on
  int causal_offset;        // dense layout: row i sees keys j <= i + causal_offset (if causal)
  int window;               // > 0 only with the causal term
  unsigned flags;
  void* stream;
  // Packed variable-length layout (both null for the dense layout): batch is the number of
  // sequences, lq the largest query length the grid covers, cu_q / cu_k the device prefix sums
  // (batch + 1 entries each), total_q / total_k the packed row counts.
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int total_q = 0, total_k = 0;
};

// Query rows handled by one workgroup of the prefill kernel.
int rows_per_block(int d);

// Number of workgroups the launch will use (64-bit; the caller checks it fits the grid).
long long grid_blocks(const Launch& p);

// Enqueue the prefill kernel. Returns PFA_OK or PFA_ERR_LAUNCH.
int launch_prefill(const Launch& p);

}  // namespace pfa
