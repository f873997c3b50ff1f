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
  // Rotating cache (0 = off): K / V are [batch, hkv, ring, d], key position j in slot j mod ring.
  int ring = 0;
  // Logit soft-capping (0 = off): each scaled score s becomes softcap * tanh(s / softcap).
  float softcap = 0.0f;
  // Additive FP32 bias (null = none; dense layout only): element (b, h, i, j) at
  // bias + b*bias_sb + h*bias_sh + i*bias_sl + j; bias_nrec bytes per (b, h) base are in the call.
  const float* bias = nullptr;
  long long bias_sb = 0, bias_sh = 0;
  int bias_sl = 0;
  int bias_nrec = 0;
  // Attention sinks (null = none): fp32 [hq] logits, one extra normaliser term e^sink per row.
  const float* sinks = nullptr;
  // Block bitmap (null = none; dense layout only): key j visible to row i of (b, h) only if
  // sel[b*sel_sb + h*sel_sh + (i / sel_bq)*sel_sq + j / sel_bk] != 0; sel_bq % 32 == 0, sel_bk % 64 == 0.
  const uint8_t* sel = nullptr;
  int sel_bq = 0, sel_bk = 0;
  long long sel_sb = 0, sel_sh = 0, sel_sq = 0;
  // Key-split workspace (null = one workgroup per item): kSplitCounterBytes of counters, one per
  // item (zero on entry, left zero on return), then split_part_bytes(d) of FP32 partials. The
  // counters sit at a fixed place so that no call's partials, whatever its head size, land on them.
  void* workspace = nullptr;
};

// Workgroups of a key-split launch (one per compute unit of an MI355X).
constexpr int kSplitWorkgroups = 256;

// Counter region at the start of a key-split workspace: one 4-byte counter per item, and the split
// is taken with at most 3/4 * kSplitWorkgroups items.
constexpr long long kSplitCounterBytes = 1024;
static_assert(kSplitCounterBytes >= 4LL * (3 * kSplitWorkgroups / 4), "split counters");

// Bytes of FP32 partial slots a key-split launch uses (two per workgroup), before the counters.
long long split_part_bytes(int d);

// Whether launch_prefill runs the key split for this call: a workspace is given, the layout is the
// dense one without bias, block bitmap or rotating cache, and the call has at most 3/4 as many
// query blocks as the split has workgroups (with more, one workgroup per block is faster; the
// workspace size rule in pfa_api.cpp uses the same bound).
bool split_applies(const Launch& p);

// Query rows handled by one workgroup of the prefill kernel.
int rows_per_block(int d);

// Query heads of one KV group that share a workgroup of the per-item launch (1, 2 or 4).
int heads_per_block(const Launch& p);

// Number of workgroups the launch will use (64-bit; the caller checks it fits the grid).
long long grid_blocks(const Launch& p);

// Enqueue the prefill kernel. Returns PFA_OK or PFA_ERR_LAUNCH.
int launch_prefill(const Launch& p);

// Enqueue the rotating-cache append (K_new / V_new rows to slots (pos0 + i) mod ring).
int launch_ring_append(const void* k_new, const void* v_new, void* k_ring, void* v_ring, int B, int Hkv, int L,
                       int D, int ring, int pos0, void* stream);

// Work split of the short-query (decode) path, a pure function of the shape so that the
// workspace query and the launch agree: the rows of one KV head (G * L) in row groups of
// rows_per_group rows (32 when G * L <= 64, else 64), the keys in n_split ranges of
// tiles_per_split 32-key tiles, one partial per (b, kv head, row group, split).
struct DecodePlan {
  int n_rowgrp = 0;
  int rows_per_group = 0;
  int rows_cap = 0;  // rows stored per partial: min(G * L, rows_per_group)
  long long grid = 0;  // workgroups of the split kernel (32-row groups: padded, see decode_unit)
  int n_split = 0;
  int tiles_per_split = 0;
  long long n_partials = 0;
  long long workspace_bytes = 0;
};
DecodePlan decode_plan(int B, int Hq, int Hkv, int L, int S, int D);

// Enqueue the split kernel and the merge kernel. Returns PFA_OK or PFA_ERR_LAUNCH.
int launch_decode(const Launch& p, const DecodePlan& plan, void* workspace);

// Device address of the current device's copy of the library's decode scratch array
// (PFA_DECODE_SCRATCH_BYTES), looked up once per device. Returns PFA_OK or PFA_ERR_LAUNCH.
int decode_scratch(void** ptr);

}  // namespace pfa
