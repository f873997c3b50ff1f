// C-ABI entry points: argument validation (host only, before anything is enqueued) and dispatch
// to the HIP launcher. This file uses no HIP API, so its checks run without a GPU.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "../../include/pfa.h"
#include "pfa_internal.h"

namespace {

bool mul_fits(long long a, long long b, long long limit, long long* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > limit / a) return false;
  *out = a * b;
  return true;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int validate(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv, int L, int S,
             int D, float scale, int causal_offset, int window, const uint8_t* key_mask,
             void* O, unsigned flags) {
  if (!Q || !K || !V || !O) return PFA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || S < 1 || D < 1) return PFA_ERR_SIZE;
  // The kernel indexes rows and keys with 32-bit integers (with headroom for tile rounding).
  if (L > PFA_MAX_LEN || S > PFA_MAX_LEN) return PFA_ERR_SIZE;
  // Element counts must fit comfortably in 64 bits; byte offsets are formed in 64 bits.
  const long long lim = LLONG_MAX / 4;
  long long q_elems, kv_elems, t;
  if (!mul_fits(B, Hq, lim, &t) || !mul_fits(t, L, lim, &t) || !mul_fits(t, D, lim, &q_elems))
    return PFA_ERR_SIZE;
  if (!mul_fits(B, Hkv, lim, &t) || !mul_fits(t, S, lim, &t) || !mul_fits(t, D, lim, &kv_elems))
    return PFA_ERR_SIZE;
  // Row/key coordinates are compared as i + causal_offset in 64-bit, so any int is fine there.
  if (Hq % Hkv != 0) return PFA_ERR_GQA;
  if (D != 64 && D != 128) return PFA_ERR_HEAD_DIM;
  if (window > 0 && causal_offset < 0) return PFA_ERR_MASK_ARGS;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return PFA_ERR_SCALE;
  const uintptr_t a16 = 15;
  if ((reinterpret_cast<uintptr_t>(Q) & a16) || (reinterpret_cast<uintptr_t>(K) & a16) ||
      (reinterpret_cast<uintptr_t>(V) & a16) || (reinterpret_cast<uintptr_t>(O) & a16))
    return PFA_ERR_ALIGN;
  const Range o{reinterpret_cast<uintptr_t>(O),
                reinterpret_cast<uintptr_t>(O) + static_cast<uintptr_t>(q_elems) * 2u};
  const Range rq{reinterpret_cast<uintptr_t>(Q),
                 reinterpret_cast<uintptr_t>(Q) + static_cast<uintptr_t>(q_elems) * 2u};
  const Range rk{reinterpret_cast<uintptr_t>(K),
                 reinterpret_cast<uintptr_t>(K) + static_cast<uintptr_t>(kv_elems) * 2u};
  const Range rv{reinterpret_cast<uintptr_t>(V),
                 reinterpret_cast<uintptr_t>(V) + static_cast<uintptr_t>(kv_elems) * 2u};
  if (overlaps(o, rq) || overlaps(o, rk) || overlaps(o, rv)) return PFA_ERR_ALIAS;
  if (key_mask) {
    const Range rm{reinterpret_cast<uintptr_t>(key_mask),
                   reinterpret_cast<uintptr_t>(key_mask) +
                       static_cast<uintptr_t>(B) * static_cast<uintptr_t>(S)};
    if (overlaps(o, rm)) return PFA_ERR_ALIAS;
  }
  if (flags & ~PFA_FLAG_NO_SKIP) return PFA_ERR_FLAGS;
  return PFA_OK;
}

// Sink logits: fp32 [Hq], 4-byte aligned, not overlapping the output.
int check_sinks(const pfa_options* opts, int Hq, Range out) {
  const float* sinks = opts ? opts->sinks : nullptr;
  if (!sinks) return PFA_OK;
  if (reinterpret_cast<uintptr_t>(sinks) & 3u) return PFA_ERR_ALIGN;
  const Range rs{reinterpret_cast<uintptr_t>(sinks),
                 reinterpret_cast<uintptr_t>(sinks) + static_cast<uintptr_t>(Hq) * 4u};
  if (overlaps(out, rs)) return PFA_ERR_ALIAS;
  return PFA_OK;
}

}  // namespace

extern "C" {

// Workspace of the key-split prefill for this shape: the counter region (one counter per item,
// i.e. query block of a query head and batch element), then the FP32 partial slots. A shape with
// more items than the split takes (pfa::split_applies) runs one workgroup per item and touches no
// workspace: 16 bytes then, so that one valid, aligned buffer still satisfies the call.
static long long prefill_workspace_bytes(int B, int Hq, int L, int D) {
  const long long items = static_cast<long long>(B) * Hq * ((static_cast<long long>(L) + pfa::rows_per_block(D) - 1) /
                                                            pfa::rows_per_block(D));
  if (items * 4 > 3LL * pfa::kSplitWorkgroups) return 16;
  return pfa::kSplitCounterBytes + pfa::split_part_bytes(D);
}

// prefill_attn_gqa_opt (workspace == nullptr, use_ws false) or prefill_attn_gqa_ws.
static int prefill_call(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv, int L, int S, int D,
                        float scale, int causal_offset, int window, const uint8_t* key_mask, void* O, void* stream,
                        const pfa_options* opts, bool use_ws, void* workspace, int64_t workspace_bytes) {
  const unsigned flags = opts ? opts->flags : 0u;
  const float softcap = opts ? opts->softcap : 0.0f;
  int rc = validate(Q, K, V, B, Hq, Hkv, L, S, D, scale, causal_offset, window, key_mask, O,
                    flags);
  if (rc != PFA_OK) return rc;
  if (!std::isfinite(softcap) || softcap < 0.0f) return PFA_ERR_SCALE;
  const long long q_elems_o = static_cast<long long>(B) * Hq * L * D;
  const Range ro{reinterpret_cast<uintptr_t>(O), reinterpret_cast<uintptr_t>(O) + static_cast<uintptr_t>(q_elems_o) * 2u};
  rc = check_sinks(opts, Hq, ro);
  if (rc != PFA_OK) return rc;
  const float* bias = opts ? opts->bias : nullptr;
  long long bias_nrec = 0;
  if (bias) {
    const long long sb = opts->bias_stride_b, sh = opts->bias_stride_h, sl = opts->bias_stride_l;
    if (key_mask) return PFA_ERR_MASK_ARGS;
    if (sb < 0 || sh < 0 || sl < 0 || sb > (1LL << 40) || sh > (1LL << 40) || sl > (1LL << 29)) return PFA_ERR_SIZE;
    const long long block = (static_cast<long long>(L) - 1) * sl + S;  // elements of one (b, h) block
    if (block >= (1LL << 29)) return PFA_ERR_SIZE;
    if ((reinterpret_cast<uintptr_t>(bias) & 15u) || (sb & 3) || (sh & 3) || (sl & 3)) return PFA_ERR_ALIGN;
    bias_nrec = block * 4;
    const long long last = (static_cast<long long>(B) - 1) * sb + (static_cast<long long>(Hq) - 1) * sh + block;
    const Range rb{reinterpret_cast<uintptr_t>(bias),
                   reinterpret_cast<uintptr_t>(bias) + static_cast<uintptr_t>(last) * 4u};
    if (overlaps(ro, rb)) return PFA_ERR_ALIAS;
  }
  const uint8_t* sel = opts ? opts->block_sel : nullptr;
  if (sel) {
    if (key_mask || bias) return PFA_ERR_MASK_ARGS;
    const int bq = opts->block_q, bk = opts->block_k;
    const long long sb = opts->sel_stride_b, sh = opts->sel_stride_h, sq = opts->sel_stride_q;
    if (bq < 32 || bq % 32 != 0 || bk < 64 || bk % 64 != 0) return PFA_ERR_SIZE;
    const long long lim = LLONG_MAX / 4;
    const long long nqb = (static_cast<long long>(L) + bq - 1) / bq, nkb = (static_cast<long long>(S) + bk - 1) / bk;
    long long eb, eh, eq;
    if (sb < 0 || sh < 0 || sq < 0 || !mul_fits(B - 1, sb, lim, &eb) || !mul_fits(Hq - 1, sh, lim, &eh) ||
        !mul_fits(nqb - 1, sq, lim, &eq))
      return PFA_ERR_SIZE;
    const long long last = eb + eh + eq + nkb;  // one past the last byte read
    const Range rs{reinterpret_cast<uintptr_t>(sel), reinterpret_cast<uintptr_t>(sel) + static_cast<uintptr_t>(last)};
    if (overlaps(ro, rs)) return PFA_ERR_ALIAS;
  }
  if (use_ws) {
    if (!workspace) return PFA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return PFA_ERR_ALIGN;
    const long long need = prefill_workspace_bytes(B, Hq, L, D);
    if (workspace_bytes < need) return PFA_ERR_WORKSPACE;
    const auto at = [](const void* ptr, uintptr_t n) {
      return Range{reinterpret_cast<uintptr_t>(ptr), reinterpret_cast<uintptr_t>(ptr) + n};
    };
    const Range ws = at(workspace, static_cast<uintptr_t>(need));
    const uintptr_t kv_bytes = static_cast<uintptr_t>(B) * Hkv * static_cast<uintptr_t>(S) * D * 2u;
    if (overlaps(ws, at(Q, static_cast<uintptr_t>(q_elems_o) * 2u)) || overlaps(ws, at(K, kv_bytes)) ||
        overlaps(ws, at(V, kv_bytes)) || overlaps(ws, ro) ||
        (key_mask && overlaps(ws, at(key_mask, static_cast<uintptr_t>(B) * static_cast<uintptr_t>(S)))) ||
        (opts && opts->sinks && overlaps(ws, at(opts->sinks, static_cast<uintptr_t>(Hq) * 4u))))
      return PFA_ERR_ALIAS;
  }
  pfa::Launch p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.key_mask = key_mask;
  p.o = O;
  p.batch = B;
  p.hq = Hq;
  p.hkv = Hkv;
  p.group = Hq / Hkv;
  p.lq = L;
  p.sk = S;
  p.d = D;
  p.scale = scale;
  p.causal = causal_offset >= 0 ? 1 : 0;
  p.causal_offset = causal_offset < 0 ? PFA_NO_CAUSAL : causal_offset;
  p.window = (causal_offset >= 0 && window > 0) ? window : 0;
  p.flags = flags;
  p.stream = stream;
  p.softcap = softcap;
  p.workspace = use_ws ? workspace : nullptr;
  if (bias) {
    p.bias = bias;
    p.bias_sb = opts->bias_stride_b;
    p.bias_sh = opts->bias_stride_h;
    p.bias_sl = static_cast<int>(opts->bias_stride_l);
    p.bias_nrec = static_cast<int>(bias_nrec);
  }
  p.sinks = opts ? opts->sinks : nullptr;
  if (sel) {
    p.sel = sel;
    p.sel_bq = opts->block_q;
    p.sel_bk = opts->block_k;
    p.sel_sb = opts->sel_stride_b;
    p.sel_sh = opts->sel_stride_h;
    p.sel_sq = opts->sel_stride_q;
  }
  if (pfa::grid_blocks(p) > INT_MAX) return PFA_ERR_SIZE;
  return pfa::launch_prefill(p);
}

int prefill_attn_gqa_opt(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv,
                         int L, int S, int D, float scale, int causal_offset, int window,
                         const uint8_t* key_mask, void* O, void* stream, const pfa_options* opts) {
  return prefill_call(Q, K, V, B, Hq, Hkv, L, S, D, scale, causal_offset, window, key_mask, O, stream, opts, false,
                      nullptr, 0);
}

int prefill_attn_gqa_ws(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv, int L, int S, int D,
                        float scale, int causal_offset, int window, const uint8_t* key_mask, void* O,
                        void* workspace, int64_t workspace_bytes, void* stream, const pfa_options* opts) {
  return prefill_call(Q, K, V, B, Hq, Hkv, L, S, D, scale, causal_offset, window, key_mask, O, stream, opts, true,
                      workspace, workspace_bytes);
}

int64_t pfa_prefill_workspace_bytes(int B, int Hq, int Hkv, int L, int S, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || S < 1 || Hq % Hkv != 0 || (D != 64 && D != 128) || L > PFA_MAX_LEN ||
      S > PFA_MAX_LEN || B > (1 << 20) || Hq > (1 << 20))
    return -1;
  return prefill_workspace_bytes(B, Hq, L, D);
}

int prefill_attn_gqa_ex(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv,
                        int L, int S, int D, float scale, int causal_offset, int window,
                        const uint8_t* key_mask, void* O, void* stream, unsigned flags) {
  pfa_options o{};
  o.flags = flags;
  return prefill_attn_gqa_opt(Q, K, V, B, Hq, Hkv, L, S, D, scale, causal_offset, window, key_mask, O,
                              stream, &o);
}

int prefill_attn_gqa(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv, int L,
                     int S, int D, float scale, int causal_offset, int window,
                     const uint8_t* key_mask, void* O, void* stream) {
  return prefill_attn_gqa_ex(Q, K, V, B, Hq, Hkv, L, S, D, scale, causal_offset, window,
                             key_mask, O, stream, 0u);
}

int prefill_attn_gqa_varlen_opt(const void* Q, const void* K, const void* V,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seq,
                                int max_seqlen_q, int total_q, int total_k, int Hq, int Hkv, int D,
                                float scale, int causal, int window, void* O, void* stream,
                                const pfa_options* opts) {
  if (!Q || !K || !V || !O || !cu_seqlens_q || !cu_seqlens_k) return PFA_ERR_NULL;
  if (n_seq < 1 || max_seqlen_q < 1 || total_q < 1 || total_k < 1 || Hq < 1 || Hkv < 1 || D < 1)
    return PFA_ERR_SIZE;
  if (max_seqlen_q > PFA_MAX_LEN || n_seq == INT_MAX) return PFA_ERR_SIZE;
  // packed row strides (Hq * D, Hkv * D elements) and a 64-key tile's byte extent stay in 31 bits
  if (Hq >= (1 << 24) / 128 || Hkv >= (1 << 24) / 128) return PFA_ERR_SIZE;
  const long long lim = LLONG_MAX / 4;
  long long q_elems, kv_elems, t;
  if (!mul_fits(total_q, Hq, lim, &t) || !mul_fits(t, D, lim, &q_elems)) return PFA_ERR_SIZE;
  if (!mul_fits(total_k, Hkv, lim, &t) || !mul_fits(t, D, lim, &kv_elems)) return PFA_ERR_SIZE;
  if (Hq % Hkv != 0) return PFA_ERR_GQA;
  if (D != 64 && D != 128) return PFA_ERR_HEAD_DIM;
  if (window > 0 && !causal) return PFA_ERR_MASK_ARGS;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return PFA_ERR_SCALE;
  const uintptr_t a16 = 15, a4 = 3;
  if ((reinterpret_cast<uintptr_t>(Q) & a16) || (reinterpret_cast<uintptr_t>(K) & a16) ||
      (reinterpret_cast<uintptr_t>(V) & a16) || (reinterpret_cast<uintptr_t>(O) & a16) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & a4) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & a4))
    return PFA_ERR_ALIGN;
  const auto range = [](const void* p, long long bytes) {
    return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + static_cast<uintptr_t>(bytes)};
  };
  const Range o = range(O, q_elems * 2);
  const long long cu_bytes = (static_cast<long long>(n_seq) + 1) * 4;
  if (overlaps(o, range(Q, q_elems * 2)) || overlaps(o, range(K, kv_elems * 2)) ||
      overlaps(o, range(V, kv_elems * 2)) || overlaps(o, range(cu_seqlens_q, cu_bytes)) ||
      overlaps(o, range(cu_seqlens_k, cu_bytes)))
    return PFA_ERR_ALIAS;
  const unsigned flags = opts ? opts->flags : 0u;
  const float softcap = opts ? opts->softcap : 0.0f;
  if (flags & ~PFA_FLAG_NO_SKIP) return PFA_ERR_FLAGS;
  if (!std::isfinite(softcap) || softcap < 0.0f) return PFA_ERR_SCALE;
  // the packed layout takes no additive bias and no block bitmap (both are laid out per dense row)
  if (opts && (opts->bias || opts->block_sel)) return PFA_ERR_MASK_ARGS;
  const int rc = check_sinks(opts, Hq, o);
  if (rc != PFA_OK) return rc;
  pfa::Launch p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.key_mask = nullptr;
  p.o = O;
  p.batch = n_seq;
  p.hq = Hq;
  p.hkv = Hkv;
  p.group = Hq / Hkv;
  p.lq = max_seqlen_q;
  p.sk = 0;
  p.d = D;
  p.scale = scale;
  p.causal = causal ? 1 : 0;
  p.causal_offset = 0;  // per sequence: Lk - Lq
  p.window = (causal && window > 0) ? window : 0;
  p.flags = flags;
  p.stream = stream;
  p.softcap = softcap;
  p.sinks = opts ? opts->sinks : nullptr;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  if (pfa::grid_blocks(p) > INT_MAX) return PFA_ERR_SIZE;
  return pfa::launch_prefill(p);
}

int prefill_attn_gqa_varlen(const void* Q, const void* K, const void* V,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int n_seq,
                            int max_seqlen_q, int total_q, int total_k, int Hq, int Hkv, int D,
                            float scale, int causal, int window, void* O, void* stream) {
  return prefill_attn_gqa_varlen_opt(Q, K, V, cu_seqlens_q, cu_seqlens_k, n_seq, max_seqlen_q, total_q, total_k,
                                     Hq, Hkv, D, scale, causal, window, O, stream, nullptr);
}

}  // extern "C"

namespace pfa {

DecodePlan decode_plan(int B, int Hq, int Hkv, int L, int S, int D) {
  // one round of single-wave workgroups (five fit a compute unit's LDS, 256 units), at least
  // four 32-key tiles per split; with one 32-row group per KV head (the register-K kernel, whose
  // waves stream the keys fastest) at least twelve, which halves the partials the merge reads and
  // still leaves about 700 workgroups for one-token decode on a 32K cache (15 % faster per call
  // than four; the 64-row kernel needs the smaller splits to fill the chip); with two 32-row groups
  // per KV head at least nine, a multiple of the kernel's three-tile step (measured on 56 rows of
  // 8K keys per KV head: 18.2 us per call against 18.9 with eight, 19.3 with six and 19.8 with
  // twelve)
  constexpr long long kTargetGroups = 1280;
  constexpr long long kMinTilesPerSplit = 4;
  constexpr long long kMinTilesPerSplitFewRows = 12;
  constexpr long long kMinTilesPerSplitTwoGroups = 9;
  DecodePlan pl;
  const long long R = static_cast<long long>(Hq / Hkv) * L;
  // up to 64 rows per KV head go in groups of 32 (the one-block kernels, the register-K one
  // without a key mask), each group streaming the keys itself; more in groups of 64 (two blocks)
  pl.rows_per_group = R <= 64 ? 32 : 64;
  pl.n_rowgrp = static_cast<int>((R + pl.rows_per_group - 1) / pl.rows_per_group);
  pl.rows_cap = static_cast<int>(R < pl.rows_per_group ? R : pl.rows_per_group);
  const long long tiles = (static_cast<long long>(S) + 31) / 32;
  const long long units = static_cast<long long>(B) * Hkv * pl.n_rowgrp;
  long long n_split = (kTargetGroups + units - 1) / units;
  if (n_split > tiles) n_split = tiles;
  if (n_split < 1) n_split = 1;
  long long tps = (tiles + n_split - 1) / n_split;
  if (tps < kMinTilesPerSplit) tps = kMinTilesPerSplit;
  if (pl.rows_per_group == 32) {
    const long long few = pl.n_rowgrp == 1 ? kMinTilesPerSplitFewRows : kMinTilesPerSplitTwoGroups;
    if (tps < few) tps = few;
  }
  n_split = (tiles + tps - 1) / tps;
  pl.n_split = static_cast<int>(n_split);
  pl.tiles_per_split = static_cast<int>(tps);
  pl.n_partials = units * n_split;
  pl.grid = pl.rows_per_group == 32 ? (units / pl.n_rowgrp * n_split + 7) / 8 * 8 * pl.n_rowgrp : pl.n_partials;
  pl.workspace_bytes = pl.n_partials * pl.rows_cap * (static_cast<long long>(D) + 2) * 4;
  return pl;
}

}  // namespace pfa

extern "C" {

int prefill_attn_gqa_ring_opt(const void* Q, const void* K_new, const void* V_new, void* K_ring, void* V_ring,
                              int B, int Hq, int Hkv, int L, int pos0, int ring, int D, float scale, int window,
                              void* O, void* stream, const pfa_options* opts) {
  if (!Q || !K_new || !V_new || !K_ring || !V_ring || !O) return PFA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || D < 1 || pos0 < 0 || ring < 1) return PFA_ERR_SIZE;
  if (static_cast<long long>(pos0) + L > PFA_MAX_LEN || ring > PFA_MAX_LEN) return PFA_ERR_SIZE;
  // one (b, KV head) ring is addressed with 32-bit byte offsets (the tile descriptor's size and each
  // row's slot offset), so it must stay under 2 GiB
  if (static_cast<long long>(ring) * D * 2 >= (1LL << 31)) return PFA_ERR_SIZE;
  const long long lim = LLONG_MAX / 4;
  long long q_elems, new_elems, ring_elems, t;
  if (!mul_fits(B, Hq, lim, &t) || !mul_fits(t, L, lim, &t) || !mul_fits(t, D, lim, &q_elems)) return PFA_ERR_SIZE;
  if (!mul_fits(B, Hkv, lim, &t) || !mul_fits(t, L, lim, &t) || !mul_fits(t, D, lim, &new_elems)) return PFA_ERR_SIZE;
  if (!mul_fits(B, Hkv, lim, &t) || !mul_fits(t, ring, lim, &t) || !mul_fits(t, D, lim, &ring_elems))
    return PFA_ERR_SIZE;
  if (Hq % Hkv != 0) return PFA_ERR_GQA;
  if (D != 64 && D != 128) return PFA_ERR_HEAD_DIM;
  if (!std::isfinite(scale) || !(scale > 0.0f)) return PFA_ERR_SCALE;
  // the ring must hold every key some row of the chunk sees, after the chunk is appended
  const long long all = static_cast<long long>(pos0) + L;
  const long long need = window > 0 ? std::min(static_cast<long long>(window) - 1 + L, all) : all;
  if (ring < 64 || ring < need) return PFA_ERR_RING;
  const uintptr_t a16 = 15;
  for (const void* ptr : {Q, static_cast<const void*>(K_new), static_cast<const void*>(V_new),
                          static_cast<const void*>(K_ring), static_cast<const void*>(V_ring),
                          static_cast<const void*>(O)})
    if (reinterpret_cast<uintptr_t>(ptr) & a16) return PFA_ERR_ALIGN;
  const auto at = [](const void* p, long long elems) {
    return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + static_cast<uintptr_t>(elems) * 2u};
  };
  const Range ro = at(O, q_elems), rq = at(Q, q_elems), rkn = at(K_new, new_elems), rvn = at(V_new, new_elems);
  const Range rkr = at(K_ring, ring_elems), rvr = at(V_ring, ring_elems);
  // O and the two rings are written; none may overlap another buffer of the call
  if (overlaps(ro, rq) || overlaps(ro, rkn) || overlaps(ro, rvn) || overlaps(ro, rkr) || overlaps(ro, rvr) ||
      overlaps(rkr, rq) || overlaps(rkr, rkn) || overlaps(rkr, rvn) || overlaps(rkr, rvr) ||
      overlaps(rvr, rq) || overlaps(rvr, rkn) || overlaps(rvr, rvn))
    return PFA_ERR_ALIAS;
  const unsigned flags = opts ? opts->flags : 0u;
  const float softcap = opts ? opts->softcap : 0.0f;
  if (flags & ~PFA_FLAG_NO_SKIP) return PFA_ERR_FLAGS;
  if (!std::isfinite(softcap) || softcap < 0.0f) return PFA_ERR_SCALE;
  // no additive bias and no block bitmap through the rotating cache
  if (opts && (opts->bias || opts->block_sel)) return PFA_ERR_MASK_ARGS;
  // the rings are written before the sink logits are read: they must not overlap (4 bytes = 2 elements per head)
  if (opts && opts->sinks && (overlaps(rkr, at(opts->sinks, 2LL * Hq)) || overlaps(rvr, at(opts->sinks, 2LL * Hq))))
    return PFA_ERR_ALIAS;
  int rc = check_sinks(opts, Hq, ro);
  if (rc != PFA_OK) return rc;
  pfa::Launch p;
  p.q = Q;
  p.k = K_ring;
  p.v = V_ring;
  p.key_mask = nullptr;
  p.o = O;
  p.batch = B;
  p.hq = Hq;
  p.hkv = Hkv;
  p.group = Hq / Hkv;
  p.lq = L;
  p.sk = pos0 + L;  // positions 0 .. pos0 + L - 1, read through the ring
  p.d = D;
  p.scale = scale;
  p.causal = 1;
  p.causal_offset = pos0;
  p.window = window > 0 ? window : 0;
  p.flags = flags;
  p.stream = stream;
  p.ring = ring;
  p.softcap = softcap;
  p.sinks = opts ? opts->sinks : nullptr;
  if (pfa::grid_blocks(p) > INT_MAX) return PFA_ERR_SIZE;  // checked before anything is enqueued
  rc = pfa::launch_ring_append(K_new, V_new, K_ring, V_ring, B, Hkv, L, D, ring, pos0, stream);
  if (rc != PFA_OK) return rc;
  return pfa::launch_prefill(p);
}

int prefill_attn_gqa_ring(const void* Q, const void* K_new, const void* V_new, void* K_ring, void* V_ring, int B,
                          int Hq, int Hkv, int L, int pos0, int ring, int D, float scale, int window, void* O,
                          void* stream) {
  return prefill_attn_gqa_ring_opt(Q, K_new, V_new, K_ring, V_ring, B, Hq, Hkv, L, pos0, ring, D, scale, window, O,
                                   stream, nullptr);
}

int64_t pfa_decode_workspace_bytes(int B, int Hq, int Hkv, int L, int S, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || S < 1 || Hq % Hkv != 0 || (D != 64 && D != 128) ||
      L > PFA_DECODE_MAX_L || S > PFA_MAX_LEN || B > (1 << 20) || Hq > (1 << 20))
    return -1;
  return pfa::decode_plan(B, Hq, Hkv, L, S, D).workspace_bytes;
}

// The decode call with a caller workspace (workspace != nullptr) or, for the allocation-free entry
// point (workspace == nullptr), with the library's own device scratch array.
static int decode_call(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv, int L, int S, int D,
                       float scale, int causal_offset, int window, const uint8_t* key_mask, void* O,
                       void* workspace, int64_t workspace_bytes, bool library_scratch, void* stream,
                       const pfa_options* opts) {
  const unsigned flags = opts ? opts->flags : 0u;
  const float softcap = opts ? opts->softcap : 0.0f;
  int rc = validate(Q, K, V, B, Hq, Hkv, L, S, D, scale, causal_offset, window, key_mask, O, flags);
  if (rc != PFA_OK) return rc;
  if (flags != 0u) return PFA_ERR_FLAGS;
  if (!std::isfinite(softcap) || softcap < 0.0f) return PFA_ERR_SCALE;
  // the decode path takes no additive bias and no block bitmap
  if (opts && (opts->bias || opts->block_sel)) return PFA_ERR_MASK_ARGS;
  if (!library_scratch && !workspace) return PFA_ERR_NULL;
  if (L > PFA_DECODE_MAX_L || B > (1 << 20) || Hq > (1 << 20)) return PFA_ERR_SIZE;
  const pfa::DecodePlan plan = pfa::decode_plan(B, Hq, Hkv, L, S, D);
  if (plan.grid > INT_MAX || static_cast<long long>(B) * Hq * L > INT_MAX) return PFA_ERR_SIZE;
  const auto bytes = [](long long a, long long b, long long c, long long d) {
    return static_cast<uintptr_t>(a) * static_cast<uintptr_t>(b) * static_cast<uintptr_t>(c) *
           static_cast<uintptr_t>(d) * 2u;
  };
  const auto at = [](const void* p, uintptr_t n) {
    return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + n};
  };
  if (library_scratch) {
    if (plan.workspace_bytes > PFA_DECODE_SCRATCH_BYTES) return PFA_ERR_WORKSPACE;
  } else {
    if (reinterpret_cast<uintptr_t>(workspace) & 15u) return PFA_ERR_ALIGN;
    if (workspace_bytes < plan.workspace_bytes) return PFA_ERR_WORKSPACE;
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace);
    const Range ws{w0, w0 + static_cast<uintptr_t>(plan.workspace_bytes)};
    if (overlaps(ws, at(Q, bytes(B, Hq, L, D))) || overlaps(ws, at(K, bytes(B, Hkv, S, D))) ||
        overlaps(ws, at(V, bytes(B, Hkv, S, D))) || overlaps(ws, at(O, bytes(B, Hq, L, D))) ||
        (key_mask && overlaps(ws, at(key_mask, static_cast<uintptr_t>(B) * static_cast<uintptr_t>(S)))) ||
        (opts && opts->sinks && overlaps(ws, at(opts->sinks, static_cast<uintptr_t>(Hq) * 4u))))
      return PFA_ERR_ALIAS;
  }
  rc = check_sinks(opts, Hq, at(O, bytes(B, Hq, L, D)));
  if (rc != PFA_OK) return rc;
  if (library_scratch) {
    rc = pfa::decode_scratch(&workspace);  // the current device's copy of the library array
    if (rc != PFA_OK) return rc;
  }
  pfa::Launch p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.key_mask = key_mask;
  p.o = O;
  p.batch = B;
  p.hq = Hq;
  p.hkv = Hkv;
  p.group = Hq / Hkv;
  p.lq = L;
  p.sk = S;
  p.d = D;
  p.scale = scale;
  p.causal = causal_offset >= 0 ? 1 : 0;
  p.causal_offset = causal_offset < 0 ? PFA_NO_CAUSAL : causal_offset;
  p.window = (causal_offset >= 0 && window > 0) ? window : 0;
  p.flags = 0;
  p.stream = stream;
  p.softcap = softcap;
  p.sinks = opts ? opts->sinks : nullptr;
  return pfa::launch_decode(p, plan, workspace);
}

int prefill_attn_gqa_decode_opt(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv, int L,
                                int S, int D, float scale, int causal_offset, int window,
                                const uint8_t* key_mask, void* O, void* workspace, int64_t workspace_bytes,
                                void* stream, const pfa_options* opts) {
  return decode_call(Q, K, V, B, Hq, Hkv, L, S, D, scale, causal_offset, window, key_mask, O, workspace,
                     workspace_bytes, false, stream, opts);
}

int prefill_attn_gqa_decode_noalloc(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv, int L,
                                    int S, int D, float scale, int causal_offset, int window,
                                    const uint8_t* key_mask, void* O, void* stream, const pfa_options* opts) {
  return decode_call(Q, K, V, B, Hq, Hkv, L, S, D, scale, causal_offset, window, key_mask, O, nullptr, 0, true,
                     stream, opts);
}

int prefill_attn_gqa_decode(const void* Q, const void* K, const void* V, int B, int Hq, int Hkv, int L,
                            int S, int D, float scale, int causal_offset, int window,
                            const uint8_t* key_mask, void* O, void* workspace, int64_t workspace_bytes,
                            void* stream) {
  return prefill_attn_gqa_decode_opt(Q, K, V, B, Hq, Hkv, L, S, D, scale, causal_offset, window, key_mask, O,
                                     workspace, workspace_bytes, stream, nullptr);
}

const char* pfa_status_str(int status) {
  switch (status) {
    case PFA_OK: return "ok";
    case PFA_ERR_NULL: return "null pointer (every tensor of the call; varlen prefix sums; the decode workspace)";
    case PFA_ERR_SIZE: return "invalid size: B, Hq, Hkv, L, S, D must be >= 1 and fit the launch (block bitmap: block_q a multiple of 32, block_k of 64, strides >= 0)";
    case PFA_ERR_GQA: return "Hq must be a multiple of Hkv";
    case PFA_ERR_HEAD_DIM: return "head dimension D must be 64 or 128";
    case PFA_ERR_MASK_ARGS: return "invalid mask combination: a sliding window (window > 0) requires causal_offset >= 0; a bias or block bitmap takes no key mask, a block bitmap no bias, and the decode path neither";
    case PFA_ERR_SCALE: return "scale must be finite and > 0";
    case PFA_ERR_ALIGN: return "Q, K, V and O must be 16-byte aligned";
    case PFA_ERR_ALIAS: return "O must not overlap Q, K, V or key_mask";
    case PFA_ERR_FLAGS: return "unknown flag bit";
    case PFA_ERR_LAUNCH: return "HIP kernel launch failed (is a gfx950 device current?)";
    case PFA_ERR_WORKSPACE: return "workspace smaller than pfa_decode_workspace_bytes() / pfa_prefill_workspace_bytes() for this shape (or, for the allocation-free decode call, than the library's scratch array)";
    case PFA_ERR_RING: return "ring cache must have >= 64 slots and hold every visible key (window - 1 + L, or pos0 + L without a window)";
    default: return "unknown status";
  }
}

int pfa_version(void) { return PFA_VERSION; }

}  // extern "C"
