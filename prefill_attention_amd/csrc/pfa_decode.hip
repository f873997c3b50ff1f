// Short-query (decode) attention for gfx950: L <= 64 query rows per head against a long cache,
// with the key range split across workgroups and a deterministic merge.
//
// What is computed is exactly the operation of the prefill kernel (same masks and head map;
// tiny-llm, Week 2 Day 5 "Tiled Dense Prefill Attention", Tasks 1 and 2). The pages send one-token
// decode and L <= 8 to a separate path (tiny-llm Task 2) and run decode against a partially filled
// cache (brotensor flash_attention_decode). Work here is bound by HBM bandwidth: each KV head's
// keys are read once for all G * L query rows of its group (no per-head re-read), and the keys
// are split into ranges processed by different single-wave workgroups so that the whole chip
// streams the cache. Each range yields a partial (m, l, a) per row; a second kernel combines the
// partials in a fixed order with the merge equations (tiny-llm Task 1: m' = max(m, m_b),
// l' = e^(m - m') l + e^(m_b - m') l_b, a' likewise), so the result is deterministic.
//
// Decode-split kernel, one wave per workgroup:
//  * rows: the G * L (query head, row) pairs of one KV head, packed 32 per MFMA block (up to 64
//    per workgroup; more rows take more row groups);
//  * keys: 32-key tiles of the split's range, fetched by buffer-load DMA into one of two LDS
//    stages (the next tile lands while the current one is used);
//  * scores transposed, S^T = K . Q^T (v_mfma_f32_32x32x16_bf16), so a lane owns one row;
//    O^T = V^T . P^T with V^T read by ds_read_b64_tr_b16 and P from the score registers;
//  * exact online softmax per tile in the base-2 domain (scores times scale * log2 e).
#include <hip/hip_runtime.h>
#include <mutex>
#include <stdint.h>

#include "../../include/pfa.h"
#include "pfa_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kTk = 32;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr int kBufferFlags = 0x00020000;  // raw buffer descriptor dword 3: 32-bit format, per-byte bounds

template <int D>
struct DGeo {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kTileBytes = kTk * kRowBytes;  // one K or V tile
  static constexpr int kStageBytes = 2 * kTileBytes;  // K then V
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kRowsPerDma = 1024 / kRowBytes;
  static constexpr int kDmaPerTile = kTileBytes / 1024;  // DMA instructions per matrix
  static constexpr int KQ = D / 16;
  static constexpr int DB = D / 32;
  __device__ static int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

struct DParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* key_mask;
  float* ws;  // partials: [n_partials][rows_cap][D] accumulators, then [n_partials][rows_cap][2] (m, l)
  int hq, hkv, group, lq, sk;
  float c;
  int causal, causal_offset, window;
  float sc_inv, sc_cap_l2;  // logit soft-capping: scale / cap and cap * log2(e)
  const float* sinks;       // null, or fp32 [hq] sink logits (an extra normaliser term per row)
  int n_rowgrp, rows_cap, n_split, tiles_per_split;
  int rows_per_group;  // 32 (one MFMA block per wave) or 64 (two)
  int xcd_pairs;       // workgroup order of the 32-row kernels (decode_unit)
  long long n_partials;
};

// Workgroup -> (b, kv head, row group, split) and its partial index ((b * hkv + hk) * n_rowgrp +
// rg) * n_split + split, the numbering the merge kernel reads. The 64-row kernel numbers the
// workgroups like its partials (splits of one row group adjacent). The 32-row kernels deal the
// row groups of one (b, kv head, split) 8 workgroups apart: the hardware deals workgroups to the 8
// XCDs round-robin, so they run on one XCD at about the same time and the later ones find the K / V
// tiles in its L2. That grid is padded to a multiple of 8 per row group; padding workgroups get
// valid = false.
struct DecodeUnit {
  int b, hk, rg, split;
  long long part;
  bool valid;
};
__device__ __forceinline__ DecodeUnit decode_unit(const DParams& p) {
  DecodeUnit u;
  long long id = blockIdx.x;
  u.valid = true;
  if (p.xcd_pairs) {
    const int lane8 = (int)(id % 8);
    id /= 8;
    u.rg = (int)(id % p.n_rowgrp);
    id = id / p.n_rowgrp * 8 + lane8;  // the (b, kv head, split) unit, split fastest
    u.valid = id < p.n_partials / p.n_rowgrp;
    u.split = (int)(id % p.n_split);
    id /= p.n_split;
  } else {
    u.split = (int)(id % p.n_split);
    id /= p.n_split;
    u.rg = (int)(id % p.n_rowgrp);
    id /= p.n_rowgrp;
  }
  u.hk = (int)(id % p.hkv);
  u.b = (int)(id / p.hkv);
  u.part = (((long long)u.b * p.hkv + u.hk) * p.n_rowgrp + u.rg) * p.n_split + u.split;
  return u;
}

__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max(x, x of lane l^32) with one v_permlane32_swap_b32 (inline asm: the builtin returns its first
// result for both outputs when given equal inputs; the nops cover the VALU -> permlane hazard)
__device__ __forceinline__ float max_with_partner_half(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// N DMA instructions from a buffer of nrec bytes at base (wave-uniform) into LDS: instruction j
// writes lane l's 16 bytes, read from byte offset off[j], to LDS address dst + 1024 j + 16 l.
// Reads at or past nrec return zeros.
// log2(e) * cap * tanh(s * scale / cap) (inv = scale / cap, cap_l2 = cap * log2(e)) from
// tanh(y) = sign(y) (1 - t) / (1 + t), t = e^(-2|y|) in (0, 1]
__device__ __forceinline__ float softcap_l2(float s, float inv, float cap_l2) {
  const float y = s * inv;
  const float t = __builtin_amdgcn_exp2f(-2.0f * kLog2e * __builtin_fabsf(y));
  const float th = (1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t);
  return __builtin_copysignf(th, y) * cap_l2;
}

template <int N>
__device__ __forceinline__ void dma_rows(const void* base, int nrec, lds_char* dst, const unsigned* off) {
  __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nrec, kBufferFlags);
#pragma unroll
  for (int j = 0; j < N; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + 1024 * j), 16,
                                             off[j], 0, 0, 0);
}

template <int D, int RB, bool KMASK, bool SOFTCAP>
__global__ __launch_bounds__(64, (RB == 1 ? 2 : 1)) void pfa_decode_split_kernel(DParams p) {
  using G = DGeo<D>;
  constexpr int KQ = G::KQ;
  constexpr int DB = G::DB;
  __shared__ __attribute__((aligned(1024))) char lds_raw[2 * G::kStageBytes];

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- workgroup -> (b, kv head, row group, split) ----
  const DecodeUnit u = decode_unit(p);
  if (!u.valid) return;
  const int split = u.split, rg = u.rg, hk = u.hk, b = u.b;
  const long long part = u.part;
  const int L = p.lq, S = p.sk;
  const int R = p.group * L;  // rows of this KV head: (g, i) -> g * L + i

  // ---- this lane's rows (one per MFMA block) and their visible key interval [lo, hi] ----
  bf16x8 qreg[RB][KQ];
  int row_lo[RB], row_hi[RB];
  int grp_lo = S, grp_hi = -1;  // union over the workgroup's real rows (wave-uniform after reduction)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rg * p.rows_per_group + rb * 32 + l32;
    int lo = S, hi = -1;  // empty
    if (r < R) {
      const int g = r / L, i = r % L;
      const uint16_t* qrow = p.q + (((long long)b * p.hq + hk * p.group + g) * L + i) * (long long)D;
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) qreg[rb][kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk + 8 * hh);
      lo = 0;
      hi = S - 1;
      if (p.causal) {
        const long long pos = (long long)i + p.causal_offset;
        hi = (int)(pos < hi ? pos : hi);
        if (p.window > 0) {
          const long long w0 = pos - p.window + 1;
          lo = (int)(w0 > 0 ? w0 : 0);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk)
#pragma unroll
        for (int t = 0; t < 8; ++t) qreg[rb][kk][t] = (__bf16)0.0f;
    }
    row_lo[rb] = lo;
    row_hi[rb] = hi;
    if (lo <= hi) {
      grp_lo = min(grp_lo, lo);
      grp_hi = max(grp_hi, hi);
    }
  }
  // wave-wide union of the rows' intervals
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    grp_lo = min(grp_lo, __shfl_xor(grp_lo, o));
    grp_hi = max(grp_hi, __shfl_xor(grp_hi, o));
  }

  // ---- the split's tiles, clipped to the keys some row can see ----
  const int n_tiles = (S + kTk - 1) / kTk;
  int t_begin = split * p.tiles_per_split;
  int t_end = min(t_begin + p.tiles_per_split, n_tiles);
  if (grp_hi < grp_lo) {
    t_end = t_begin;  // no row sees anything
  } else {
    t_begin = max(t_begin, grp_lo / kTk);
    t_end = min(t_end, grp_hi / kTk + 1);
  }
  // visible iff tile key jj: lo <= key <= hi (and the key-mask byte is nonzero)
  const uint16_t* kg = p.k + ((long long)b * p.hkv + hk) * (long long)S * D;
  const uint16_t* vg = p.v + ((long long)b * p.hkv + hk) * (long long)S * D;
  const uint8_t* mrow = KMASK ? p.key_mask + (long long)b * S : nullptr;

  // DMA offsets (K and V rows of a tile; fixed per lane)
  unsigned off_k[G::kDmaPerTile], off_v[G::kDmaPerTile];
#pragma unroll
  for (int j = 0; j < G::kDmaPerTile; ++j) {
    const int row = j * G::kRowsPerDma + lane / G::kChunksPerRow;
    const int pch = lane % G::kChunksPerRow;
    off_k[j] = (unsigned)(row * G::kRowBytes + 16 * (pch ^ G::swz_k(row)));
    off_v[j] = (unsigned)(row * G::kRowBytes + 16 * (pch ^ G::swz_v(row)));
  }
  auto uniform_ptr = [&](const void* ptr) __attribute__((always_inline)) -> const void* {
    const uintptr_t a = reinterpret_cast<uintptr_t>(ptr);
    // readfirstlane returns int: go through unsigned so the low word is not sign-extended
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
    return reinterpret_cast<const void*>(((uintptr_t)hi << 32) | (uintptr_t)lo);
  };
  auto issue = [&](int t, char* stage) __attribute__((always_inline)) {
    const long long key0 = (long long)t * kTk;
    const long long rows = (long long)S - key0;
    const int nrec = __builtin_amdgcn_readfirstlane((rows < kTk ? (int)rows : kTk) * G::kRowBytes);
    dma_rows<G::kDmaPerTile>(uniform_ptr(kg + key0 * D), nrec, (lds_char*)stage, off_k);
    dma_rows<G::kDmaPerTile>(uniform_ptr(vg + key0 * D), nrec, (lds_char*)stage + G::kTileBytes, off_v);
  };

  // LDS read addresses inside a stage (as in the prefill kernel, with one 32-key block)
  int a_k, a_v;
  {
    const int x = G::swz_k(l32);
    a_k = l32 * G::kRowBytes + 16 * (hh ^ (x & 1)) + 32 * (x >> 1);
    const int g16 = lane >> 4, loc = lane & 15, r4 = loc >> 2, cc = loc & 3;
    const int row = 4 * (g16 >> 1) + r4;
    a_v = G::kTileBytes + row * G::kRowBytes + 64 * (G::swz_v(row) >> 2) + 32 * (g16 & 1) + 8 * cc;
  }

  f32x16 acc[RB][DB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][db][v] = 0.0f;
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.0f;
  }
  // with soft-capping the scores are turned into the base-2 exponent domain up front
  const float c = SOFTCAP ? 1.0f : p.c;

  if (t_begin < t_end) issue(t_begin, lds_raw);
  // One step: tile t is in `cur`, tile t+1 is fetched into `nxt`. The stages are restrict
  // pointers: the fetch into `nxt` is never read in the step, which lets the compiler keep it in
  // flight across the step's LDS reads (it is waited for at the top of the next step).
  auto step = [&](int t, char* __restrict__ cur, char* __restrict__ nxt) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile t has landed (one wave: no barrier)
    // the other stage's reads (previous tile) all completed before their MFMAs; refill it
    if (t + 1 < t_end) issue(t + 1, nxt);
    const lds_char* base = (const lds_char*)cur;
    // scores
    f32x16 s[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[rb][v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const bf16x8 a = *(const lds_bf16x8*)(base + (a_k ^ (32 * kk)));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[rb][kk], s[rb], 0, 0, 0);
    }
    if constexpr (SOFTCAP) {
      // logit soft-capping before the masks (brotensor flash_attention_decode, attn_softcap)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[rb][v] = softcap_l2(s[rb][v], p.sc_inv, p.sc_cap_l2);
    }
    // mask: lane row's interval and the key bytes
    const int key0 = t * kTk;
    uint32_t mb[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    if (KMASK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 8 * j + 4 * hh + i;
          const uint32_t byte = key < S ? (uint32_t)mrow[key] : 0u;
          w |= (byte != 0u ? 0xFFu : 0u) << (8 * i);
        }
        mb[j] = w;
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // key visible iff 0 <= key - lo <= span (one unsigned compare); an empty row gets lo = -1
      // and span 0, which only key -1 would pass: no key of any tile is visible to it
      const bool empty = row_hi[rb] < row_lo[rb];
      const unsigned span = empty ? 0u : (unsigned)(row_hi[rb] - row_lo[rb]);
      const int lo = empty ? -1 : row_lo[rb];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 8 * j + 4 * hh + i;
          const bool vis = ((unsigned)(key - lo) <= span) & (((mb[j] >> (8 * i)) & 0xFFu) != 0u);
          s[rb][4 * j + i] = vis ? s[rb][4 * j + i] : -INFINITY;
        }
    }
    // exact online softmax per row, P in bf16 pairs, row sums of the rounded P
    unsigned pw[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = s[rb][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = max2(mx, s[rb][v]);
      mx = max_with_partner_half(mx) * c;
      const float mnew = max2(m[rb], mx);
      const float msub = (mnew == -INFINITY) ? 0.0f : mnew;
      const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m[rb] - mnew);
      float ls[2] = {0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][2 * w], c, -msub));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][2 * w + 1], c, -msub));
        const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
        ls[w & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, ls[w & 1], false);
        pw[rb][w] = __builtin_bit_cast(unsigned, pr);
      }
      l[rb] = l[rb] * alpha + (ls[0] + ls[1]);
      m[rb] = mnew;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[rb][db][v] *= alpha;
    }
    // O^T += V^T . P^T over the tile's two 16-key steps
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const lds_char* pr = base + 16 * c2 * G::kRowBytes + (a_v ^ (64 * db));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pr);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pr + 8 * G::kRowBytes));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const u32x4 w = {pw[rb][4 * c2], pw[rb][4 * c2 + 1], pw[rb][4 * c2 + 2], pw[rb][4 * c2 + 3]};
          acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, w), acc[rb][db], 0, 0, 0);
        }
      }
  };
  for (int t = t_begin; t < t_end; ++t) {
    if (((t - t_begin) & 1) == 0)
      step(t, lds_raw, lds_raw + G::kStageBytes);
    else
      step(t, lds_raw + G::kStageBytes, lds_raw);
  }

  // ---- the partial of this workgroup: acc (unnormalised), m (base-2 domain), l ----
  const int rows_cap = p.rows_cap;
  float* ws_acc = p.ws + (size_t)part * rows_cap * D;
  float* ws_ml = p.ws + (size_t)p.n_partials * rows_cap * D + (size_t)part * rows_cap * 2;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rr = rb * 32 + l32;  // row within the group
    const float lt = l[rb] + __shfl_xor(l[rb], 32);
    if (rr < rows_cap) {
      float* dst = ws_acc + (size_t)rr * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 o4 = {acc[rb][db][4 * j], acc[rb][db][4 * j + 1], acc[rb][db][4 * j + 2], acc[rb][db][4 * j + 3]};
          *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * j + 4 * hh) = o4;
        }
      if (hh == 0) {
        ws_ml[2 * rr] = m[rb];
        ws_ml[2 * rr + 1] = lt;
      }
    }
  }
}

// Decode-split kernel for 32-row groups (up to 64 rows per KV head, as one or two groups) and no
// key mask (one-token decode and short chunks of small groups): K goes from memory straight into the registers of the GEMM1 operand
// (lane l: key l % 32, 16 bytes of dimensions per MFMA step, read by buffer loads whose descriptor
// ends at the last key), only V is staged in LDS (three 32-key stages, for the transpose reads),
// and while tile t is used tiles t+1 and t+2 are in flight: twice the bytes in flight per
// workgroup of the kernel above, in a quarter of its LDS. Same partials and arithmetic per tile.
template <int D, bool SOFTCAP>
__global__ __launch_bounds__(64, 2) void pfa_decode_kreg_kernel(DParams p) {
  using G = DGeo<D>;
  constexpr int KQ = G::KQ;
  constexpr int DB = G::DB;
  constexpr int kPerTile = KQ + G::kDmaPerTile;  // memory instructions per tile (K loads, V DMA)
  __shared__ __attribute__((aligned(1024))) char lds_raw[3 * G::kTileBytes];

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- workgroup -> (b, kv head, row group of 32 rows, split) ----
  const DecodeUnit u = decode_unit(p);
  if (!u.valid) return;
  const int split = u.split, hk = u.hk, b = u.b;
  const long long part = u.part;
  const int L = p.lq, S = p.sk;
  const int R = p.group * L;

  // ---- this lane's row and its visible key interval [lo, hi] ----
  bf16x8 qreg[KQ];
  int lo = S, hi = -1;  // empty
  const int r = u.rg * 32 + l32;
  if (r < R) {
    const int g = r / L, i = r % L;
    const uint16_t* qrow = p.q + (((long long)b * p.hq + hk * p.group + g) * L + i) * (long long)D;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk + 8 * hh);
    lo = 0;
    hi = S - 1;
    if (p.causal) {
      const long long pos = (long long)i + p.causal_offset;
      hi = (int)(pos < hi ? pos : hi);
      if (p.window > 0) {
        const long long w0 = pos - p.window + 1;
        lo = (int)(w0 > 0 ? w0 : 0);
      }
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
#pragma unroll
      for (int t = 0; t < 8; ++t) qreg[kk][t] = (__bf16)0.0f;
  }
  int grp_lo = lo <= hi ? lo : S, grp_hi = lo <= hi ? hi : -1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    grp_lo = min(grp_lo, __shfl_xor(grp_lo, o));
    grp_hi = max(grp_hi, __shfl_xor(grp_hi, o));
  }
  const int n_tiles = (S + kTk - 1) / kTk;
  int t_begin = split * p.tiles_per_split;
  int t_end = min(t_begin + p.tiles_per_split, n_tiles);
  if (grp_hi < grp_lo) {
    t_end = t_begin;
  } else {
    t_begin = max(t_begin, grp_lo / kTk);
    t_end = min(t_end, grp_hi / kTk + 1);
  }
  const uint16_t* kg = p.k + ((long long)b * p.hkv + hk) * (long long)S * D;
  const uint16_t* vg = p.v + ((long long)b * p.hkv + hk) * (long long)S * D;

  // DMA instruction j of a V tile: lane offset off_v0 + 1024 j (row j * kRowsPerDma + lane / CPR;
  // the swizzle of those rows does not depend on j)
  unsigned off_v0;
  {
    const int row = lane / G::kChunksPerRow;
    const int pch = lane % G::kChunksPerRow;
    off_v0 = (unsigned)(row * G::kRowBytes + 16 * (pch ^ G::swz_v(row)));
  }
  const unsigned off_k = (unsigned)(l32 * G::kRowBytes + 16 * hh);  // + 32 kk
  auto uniform_ptr = [&](const void* ptr) __attribute__((always_inline)) -> const void* {
    const uintptr_t a = reinterpret_cast<uintptr_t>(ptr);
    const unsigned ahi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
    const unsigned alo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
    return reinterpret_cast<const void*>(((uintptr_t)ahi << 32) | (uintptr_t)alo);
  };
  bf16x8 kreg[3][KQ];
  // K of tile t into kreg[buf], V of tile t into `stage`; keys past S, and every key of a tile at
  // or past t_end (the padding steps below), read as zeros
  auto issue = [&](int t, bf16x8* kr, char* stage) __attribute__((always_inline)) {
    const long long key0 = (long long)t * kTk;
    long long rows = t < t_end ? (long long)S - key0 : 0;
    rows = rows < 0 ? 0 : (rows > kTk ? kTk : rows);
    const int nrec = __builtin_amdgcn_readfirstlane((int)rows * G::kRowBytes);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform_ptr(kg + key0 * D)), 0, nrec, kBufferFlags);
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
      kr[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off_k + 32 * kk, 0, 0));
    unsigned off_v[G::kDmaPerTile];
#pragma unroll
    for (int j = 0; j < G::kDmaPerTile; ++j) off_v[j] = off_v0 + 1024u * j;
    dma_rows<G::kDmaPerTile>(uniform_ptr(vg + key0 * D), nrec, (lds_char*)stage, off_v);
  };
  int a_v;
  {
    const int g16 = lane >> 4, loc = lane & 15, r4 = loc >> 2, cc = loc & 3;
    const int row = 4 * (g16 >> 1) + r4;
    a_v = row * G::kRowBytes + 64 * (G::swz_v(row) >> 2) + 32 * (g16 & 1) + 8 * cc;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const float c = SOFTCAP ? 1.0f : p.c;
  // the row's keys within this split: [lo, min(hi, last key of tile t_end - 1)]. A row with no
  // key here gets lo_eff = -1 and span 0, which no key passes: the padding steps past t_end visit
  // keys up to S + 95, so a sentinel past S could coincide with one of them.
  const int hi_split = min(hi, t_end * kTk - 1);
  const bool empty = hi_split < lo;
  const unsigned span = empty ? 0u : (unsigned)(hi_split - lo);
  const int lo_eff = empty ? -1 : lo;

  // One step on tile t (K in kr, V in `cur`): wait for it (the next tile may stay in flight), the
  // scores, then tile t+2 to the buffers tile t-1 used (`nxt2`, kr2), softmax and P.V. The stages
  // are restrict pointers: the fetch into `nxt2` is never read in the step, so the compiler keeps
  // it in flight across the step's LDS reads.
  auto step = [&](int t, const bf16x8* kr, bf16x8* kr2, char* __restrict__ cur, char* __restrict__ nxt2)
                  __attribute__((always_inline)) {
    // vmcnt(kPerTile): only tile t+1's instructions may still be outstanding
    __builtin_amdgcn_s_waitcnt(0x0F70 | (kPerTile & 15) | ((kPerTile >> 4) << 14));
    const lds_char* base = (const lds_char*)cur;
    f32x16 s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[kk], qreg[kk], s, 0, 0, 0);
    // tile t+2 goes out once this tile's K registers have been read
    issue(t + 2, kr2, nxt2);
    if constexpr (SOFTCAP) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = softcap_l2(s[v], p.sc_inv, p.sc_cap_l2);
    }
    const int key0 = t * kTk;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 8 * j + 4 * hh + i;
        s[4 * j + i] = ((unsigned)(key - lo_eff) <= span) ? s[4 * j + i] : -INFINITY;
      }
    unsigned pw[8];
    {
      float mx = s[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = max2(mx, s[v]);
      mx = max_with_partner_half(mx) * c;
      const float mnew = max2(m, mx);
      const float msub = (mnew == -INFINITY) ? 0.0f : mnew;
      const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);
      float ls[2] = {0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w], c, -msub));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * w + 1], c, -msub));
        const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
        ls[w & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, ls[w & 1], false);
        pw[w] = __builtin_bit_cast(unsigned, pr);
      }
      l = l * alpha + (ls[0] + ls[1]);
      m = mnew;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
    }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const lds_char* pr = base + 16 * c2 * G::kRowBytes + (a_v ^ (64 * db));
        const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pr);
        const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pr + 8 * G::kRowBytes));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        const u32x4 w = {pw[4 * c2], pw[4 * c2 + 1], pw[4 * c2 + 2], pw[4 * c2 + 3]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, w), acc[db], 0, 0, 0);
      }
  };
  char* st0 = lds_raw;
  char* st1 = lds_raw + G::kTileBytes;
  char* st2 = lds_raw + 2 * G::kTileBytes;
  // The steps run in threes (the registers of a tile rotate with the step) over the tile range
  // padded to a multiple of three; a padding step fetches zeros and masks every key (its keys are
  // past hi_split), which leaves m, l and the accumulator exactly as they were. Every step issues
  // and waits alike, so the compiler sees one regular pattern and adds no waits of its own.
  issue(t_begin, kreg[0], st0);
  issue(t_begin + 1, kreg[1], st1);
  const int t_pad = t_begin + (t_end - t_begin + 2) / 3 * 3;
  for (int t = t_begin; t < t_pad; t += 3) {
    step(t, kreg[0], kreg[2], st0, st2);
    step(t + 1, kreg[1], kreg[0], st1, st0);
    step(t + 2, kreg[2], kreg[1], st2, st1);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the last padding fetches have landed before the wave ends

  // ---- the partial of this workgroup (same layout as the kernel above) ----
  const int rows_cap = p.rows_cap;
  float* ws_acc = p.ws + (size_t)part * rows_cap * D;
  float* ws_ml = p.ws + (size_t)p.n_partials * rows_cap * D + (size_t)part * rows_cap * 2;
  const float lt = l + __shfl_xor(l, 32);
  if (l32 < rows_cap) {
    float* dst = ws_acc + (size_t)l32 * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 o4 = {acc[db][4 * j], acc[db][4 * j + 1], acc[db][4 * j + 2], acc[db][4 * j + 3]};
        *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * j + 4 * hh) = o4;
      }
    if (hh == 0) {
      ws_ml[2 * l32] = m;
      ws_ml[2 * l32 + 1] = lt;
    }
  }
}

// One workgroup per output row (b, h, i): combine the row's n_split partials with the merge
// equations and write O = a / l in BF16 (0 when no key was visible). Thread t owns four columns
// (d4 = t % (D/4)) of the splits s = j, j + P, ... (j = t / (D/4), P = kMergeThreads / (D/4)): it
// loads four of them at a time and merges them locally, then the P partial triples (m, l, a) are
// combined by a fixed tree over j with the same equations, so the result does not depend on
// timing. Calls with many rows use 256 threads per row (fewer tree levels and barriers, more
// splits per thread), calls with few rows 1024.
template <int D, int kMergeThreads>
__global__ __launch_bounds__(kMergeThreads) void pfa_decode_merge_kernel(DParams p, uint16_t* o) {
  constexpr int C4 = D / 4;              // float4 columns
  constexpr int P = kMergeThreads / C4;  // split lanes
  __shared__ f32x4 red[kMergeThreads];
  __shared__ float red_m[P], red_l[P];
  const int t = threadIdx.x;
  const int d4 = t % C4, j = t / C4;
  long long id = blockIdx.x;  // (b, h, i)
  const int i = (int)(id % p.lq);
  id /= p.lq;
  const int h = (int)(id % p.hq);
  const int b = (int)(id / p.hq);
  const int hk = h / p.group, g = h % p.group;
  const int r = g * p.lq + i;
  const int rg = r / p.rows_per_group, rr = r % p.rows_per_group;
  const long long part0 = (((long long)b * p.hkv + hk) * p.n_rowgrp + rg) * p.n_split;
  const float* ws_ml = p.ws + (size_t)p.n_partials * p.rows_cap * D;
  // local merge of this thread's splits (empty splits have m = -inf and l = a = 0)
  float mloc = -INFINITY, lloc = 0.0f;
  f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = j; s0 < p.n_split; s0 += 4 * P) {
    float ms[4], ls[4];
    f32x4 vs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // four splits' loads in flight before any use
      const int sp = s0 + u * P;
      if (sp < p.n_split) {
        const size_t q = (size_t)(part0 + sp);
        ms[u] = ws_ml[q * p.rows_cap * 2 + 2 * rr];
        ls[u] = ws_ml[q * p.rows_cap * 2 + 2 * rr + 1];
        vs[u] = *reinterpret_cast<const f32x4*>(p.ws + (q * p.rows_cap + rr) * D + 4 * d4);
      } else {
        ms[u] = -INFINITY;
        ls[u] = 0.0f;
        vs[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float mn = max2(mloc, ms[u]);
      if (mn != -INFINITY) {
        const float w0 = __builtin_amdgcn_exp2f(mloc - mn), w1 = __builtin_amdgcn_exp2f(ms[u] - mn);
        lloc = lloc * w0 + ls[u] * w1;
        a = a * w0 + vs[u] * w1;
        mloc = mn;
      }
    }
  }
  red[t] = a;
  if (d4 == 0) {
    red_m[j] = mloc;
    red_l[j] = lloc;
  }
  __syncthreads();
  // fixed tree over the split lanes j (red[j * C4 + d4])
  for (int w = P / 2; w > 0; w >>= 1) {
    float m1 = 0.0f, m2 = 0.0f, mn = 0.0f;
    if (j < w) {
      m1 = red_m[j];
      m2 = red_m[j + w];
      mn = max2(m1, m2);
      if (mn != -INFINITY) {
        const float w0 = __builtin_amdgcn_exp2f(m1 - mn), w1 = __builtin_amdgcn_exp2f(m2 - mn);
        red[t] = red[t] * w0 + red[t + w * C4] * w1;
        if (d4 == 0) red_l[j] = red_l[j] * w0 + red_l[j + w] * w1;
      }
    }
    __syncthreads();
    if (j < w && d4 == 0) red_m[j] = mn;
    __syncthreads();
  }
  if (j == 0) {
    float lt = red_l[0];
    // an attention sink adds e^sink to the normaliser, relative to the merged maximum
    if (p.sinks != nullptr && lt > 0.0f) lt += __builtin_amdgcn_exp2f(__builtin_fmaf(p.sinks[h], kLog2e, -red_m[0]));
    const f32x4 at = red[d4];
    uint16_t* orow = o + (((long long)b * p.hq + h) * p.lq + i) * D + 4 * d4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float out = lt > 0.0f ? at[k] / lt : 0.0f;
      const __bf16 ob = (__bf16)out;
      orow[k] = __builtin_bit_cast(uint16_t, ob);
    }
  }
}

template <int D, int RB>
int launch_decode_variant(const pfa::Launch& L, const pfa::DecodePlan& plan, void* ws) {
  DParams p;
  p.q = static_cast<const uint16_t*>(L.q);
  p.k = static_cast<const uint16_t*>(L.k);
  p.v = static_cast<const uint16_t*>(L.v);
  p.key_mask = L.key_mask;
  p.ws = static_cast<float*>(ws);
  p.hq = L.hq;
  p.hkv = L.hkv;
  p.group = L.group;
  p.lq = L.lq;
  p.sk = L.sk;
  p.c = L.scale * kLog2e;
  p.causal = L.causal;
  p.causal_offset = L.causal_offset;
  p.window = L.window;
  const bool sc = L.softcap > 0.0f;
  p.sc_inv = sc ? L.scale / L.softcap : 0.0f;
  p.sc_cap_l2 = sc ? L.softcap * kLog2e : 0.0f;
  p.sinks = L.sinks;
  p.n_rowgrp = plan.n_rowgrp;
  p.rows_cap = plan.rows_cap;
  p.n_split = plan.n_split;
  p.tiles_per_split = plan.tiles_per_split;
  p.n_partials = plan.n_partials;
  p.rows_per_group = plan.rows_per_group;
  p.xcd_pairs = plan.rows_per_group == 32 ? 1 : 0;
  hipStream_t stream = static_cast<hipStream_t>(L.stream);
  void* args[] = {&p};
  const void* fn =
      (RB == 1 && !L.key_mask)
          ? (sc ? reinterpret_cast<const void*>(&pfa_decode_kreg_kernel<D, true>)
                : reinterpret_cast<const void*>(&pfa_decode_kreg_kernel<D, false>))
      : L.key_mask ? (sc ? reinterpret_cast<const void*>(&pfa_decode_split_kernel<D, RB, true, true>)
                       : reinterpret_cast<const void*>(&pfa_decode_split_kernel<D, RB, true, false>))
                 : (sc ? reinterpret_cast<const void*>(&pfa_decode_split_kernel<D, RB, false, true>)
                       : reinterpret_cast<const void*>(&pfa_decode_split_kernel<D, RB, false, false>));
  if (hipLaunchKernel(fn, dim3((unsigned)plan.grid), dim3(64), args, 0, stream) != hipSuccess)
    return PFA_ERR_LAUNCH;
  uint16_t* o = static_cast<uint16_t*>(L.o);
  void* margs[] = {&p, &o};
  const long long rows = (long long)L.batch * L.hq * L.lq;
  // 256 rows or more: 256 threads per row (448 rows of 32 splits: 6.7 -> 5.2 us per merge)
  const bool many = rows >= 256;
  const void* mfn = many ? reinterpret_cast<const void*>(&pfa_decode_merge_kernel<D, 256>)
                         : reinterpret_cast<const void*>(&pfa_decode_merge_kernel<D, 1024>);
  if (hipLaunchKernel(mfn, dim3((unsigned)rows), dim3(many ? 256 : 1024), margs, 0, stream) != hipSuccess)
    return PFA_ERR_LAUNCH;
  return PFA_OK;
}

// ---- the allocation-free variant's scratch: the partials live in a library-held device array ----
// One copy per GPU (the module's device globals are instantiated on every device it is loaded on),
// held until the process ends. Host code never passes `decode_scratch_array` itself to a kernel (on
// the host it names a host-side stand-in): its device address is looked up per device with
// hipGetSymbolAddress and kept in g_scratch_ptr.
static __device__ __align__(256) char decode_scratch_array[PFA_DECODE_SCRATCH_BYTES];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace pfa {

int decode_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PFA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(decode_scratch_array)) != hipSuccess || a == nullptr)
      return PFA_ERR_LAUNCH;
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return PFA_OK;
}

int launch_decode(const Launch& p, const DecodePlan& plan, void* workspace) {
  const bool two = plan.rows_cap > 32;
  if (p.d == 128) return two ? launch_decode_variant<128, 2>(p, plan, workspace) : launch_decode_variant<128, 1>(p, plan, workspace);
  return two ? launch_decode_variant<64, 2>(p, plan, workspace) : launch_decode_variant<64, 1>(p, plan, workspace);
}

}  // namespace pfa
