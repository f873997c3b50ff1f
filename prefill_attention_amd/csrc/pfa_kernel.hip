// Grouped-query flash prefill attention for gfx950 (MI355X / CDNA4).
//
// What is computed (tiny-llm, Week 2 Day 5 "Tiled Dense Prefill Attention", Tasks 1 and 2):
// for each query row an FP32 running maximum m, running sum l and accumulator a are merged key
// tile by key tile (the merge equations: m' = max(m, m_b), l' = e^(m-m') l + sum_b, a' likewise),
// and the output a / l is rounded to BF16 only at the end. Fully masked key tiles are skipped
// before their K/V tile is loaded (brotensor flash_attention_decode_masked; mlx-lm PR "Skip fully
// masked key tiles ...") on a fixed grid of 64-key tiles, so skipping is bit-identical to
// visiting every tile.
//
// gfx950 design:
//  * One workgroup = 8 waves; each wave owns 32 query rows of one query head; the workgroup
//    covers 256 consecutive rows. Waves w and w+4 share a SIMD.
//  * Scores are computed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16. In the MFMA
//    result lane l holds key rows 8j+4h+i (h = l/32) of query column l%32, so every lane owns one
//    query row: row max and row sum are in-lane plus one exchange between the two lane halves.
//  * The output is accumulated transposed too, O^T = V^T . P^T. The S^T result registers
//    (exponentiated, rounded to BF16) are directly the B operand of that MFMA: the key order they
//    imply is matched by reading V^T from LDS with ds_read_b64_tr_b16, which hands each lane four
//    consecutive keys of one column. P never goes through LDS and V is never transposed by VALU.
//  * Software pipeline and ping-pong: a wave's work on tile t is GEMM1(t) (scores), SOFTMAX(t)
//    and GEMM2(t) (P.V). A wave runs "GEMM1(t) + GEMM2(t-1)" as one MFMA phase and SOFTMAX(t) as
//    one VALU phase. Waves 0-3 and 4-7 run these phases in opposite halves of each iteration
//    (a barrier closes each iteration; one between the halves at D = 64 and with a bias), so on
//    every SIMD one wave feeds the matrix core while the other runs the exponentials. In the MFMA
//    phase each LDS operand is read three MFMAs ahead, at an immediate offset: the loop is unrolled
//    once per LDS stage.
//  * K/V tiles (64 keys x D) go from HBM straight into LDS with buffer_load_dwordx4 ... lds (each
//    instruction writes 1 KB of consecutive LDS; waves 0-3 fetch K, waves 4-7 fetch V), into one
//    of three stages: tile t+1 lands while tile t's K and tile t-1's V are read. Rows are
//    unpadded; 16-byte chunks are XOR-swizzled per row so both the K reads (ds_read_b128, one row
//    per lane) and the V transpose reads (four rows per 16 lanes) are free of bank conflicts.
//  * Scores are scaled by scale*log2(e) inside the exp2 argument (one FMA per score), in FP32:
//    folding the scale into Q instead rounds q*scale*log2(e) to BF16, an error proportional to the
//    logit, which breaks the accuracy bound once logits reach tens of units.
//  * The tile range of a workgroup is bounded by the causal and window edges; with a key mask a
//    per-tile "any valid" bitmap (64 tiles per ballot) lets the loop jump over empty tiles; waves
//    whose own rows see nothing of a tile skip its arithmetic. Elementwise masks run only on
//    tiles that straddle an edge.
//  * Workgroups are ordered so that those sharing a KV head land on the same XCD (the hardware
//    deals workgroups to the 8 XCDs round-robin), heaviest causal blocks first.
#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "../../include/pfa.h"
#include "pfa_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kBN = 64;  // keys per tile
constexpr int kWaveRows = 32;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * kWaveRows;  // query rows per workgroup
constexpr int kStages = 3;
constexpr int kXcds = 8;
constexpr int kRing = 4;  // LDS operands in flight in the MFMA phase
constexpr float kLog2e = 1.4426950408889634f;
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr float kLazyLog2 = 8.0f;  // reference-max slack of the lazy rescale (P <= 2^8)
// dword 3 of a raw buffer descriptor (32-bit data format, no swizzle, bounds checked per byte)
constexpr int kBufferFlags = 0x00020000;

// sched_group_barrier masks
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

template <int D>
struct Geo {
  static constexpr int kRowBytes = 2 * D;              // unpadded K / V row in LDS
  static constexpr int kTileBytes = kBN * kRowBytes;   // one K or V tile
  static constexpr int kStageBytes = 2 * kTileBytes;   // one K and one V tile
  // LDS: the K tiles of the stages first, then their V tiles, so that every operand read of an
  // iteration with a known stage is one lane address plus an immediate offset below 64 KB
  static constexpr int kVRegion = kStages * kTileBytes;
  // part of the V region's offset held in the lane's V^T read addresses rather than in the
  // immediate offsets (those of stage 2 would pass 64 KB at D = 128)
  static constexpr int kVHeld = D == 128 ? 32768 : 0;
  static constexpr int kChunksPerRow = D / 8;          // 16-byte chunks per row
  static constexpr int kRowsPerDma = 1024 / kRowBytes;  // rows written by one DMA instruction
  static constexpr int kDmaPerTile = kTileBytes / 1024;
  static constexpr int kDmaPerWave = kDmaPerTile / 4;  // per wave of the group fetching a matrix
  static constexpr int KQ = D / 16;  // MFMA k-steps over the head dimension
  static constexpr int DB = D / 32;  // 32-wide output blocks
  // Physical chunk of logical chunk c in row r is c ^ swz(r).
  __device__ static int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* key_mask;
  uint16_t* o;
  int hq, hkv, group, lq, sk;
  float c;  // scale * log2(e)
  int causal;         // causal term on
  int causal_offset, window;
  // Packed variable-length batches (null for the dense layout): sequence b owns query rows
  // [cu_q[b], cu_q[b+1]) of the packed [total_q, Hq, D] Q / O and keys [cu_k[b], cu_k[b+1]) of
  // the packed [total_k, Hkv, D] K / V; the causal offset is taken per sequence (Lk - Lq).
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  // Rotating (ring) cache, dense layout only (0 = off): K / V are [B, Hkv, ring, D] and key
  // position j lives in slot j mod ring.
  int ring;
  float sc_inv, sc_cap_l2;  // soft-capping: scale / cap and cap * log2(e)
  // Additive FP32 bias (dense layout): element (b, h, i, j) at bias + b*sb + h*sh + i*sl + j;
  // bias_nrec = bytes from the (b, h) base that belong to the call (reads past it return 0).
  const float* bias;
  long long bias_sb, bias_sh;
  int bias_sl;
  int bias_nrec;
  // Attention sinks (null = none): fp32 [hq] logits, each an extra normaliser term of its head.
  const float* sinks;
  // Block bitmap (dense layout): key j visible to row i of (b, h) only if
  // sel[b*sel_sb + h*sel_sh + (i / sel_bq)*sel_sq + j / sel_bk] != 0 (sel_bq % 32 == 0,
  // sel_bk % 64 == 0, so a wave's rows share one query block and a tile's keys one key block).
  const uint8_t* sel;
  int sel_bq, sel_bk;
  long long sel_sb, sel_sh, sel_sq;
  int no_skip;
  // Key-split (stream) launch: nullptr = one workgroup per item. Otherwise gridDim.x workgroups
  // each take an equal share of the linear (item, key tile) space; a part of an item leaves its
  // FP32 partial in ws_part and the last part to finish merges them (ws_cnt: per-item counters,
  // zero between calls).
  float* ws_part;
  unsigned* ws_cnt;
  int batch;
  int n_qblk;
  // Query heads of one KV group that share a workgroup (1, 2 or 4; 1 with a bias, a bitmap or the
  // key split): wave w takes head (w mod hpw) of the item's head set and rows 32 (w / hpw) of the
  // item's block of 256 / hpw rows. Every head of the set reads the same K / V tiles, and the
  // block's key range (causal and window edges) narrows with its height.
  int hpw;
  int n_hset;  // group / hpw head sets per KV head
  int n_wg;
  int xcd_remap;
};

// N DMA instructions of one wave from a buffer of `nrec` bytes at `base` (wave-uniform) into LDS:
// instruction j writes lane l's 16 bytes, read from byte offset off[j] of the buffer, to LDS
// address dst + 1024 j + 16 l. Reads at or past nrec return zeros.
template <int N>
__device__ __forceinline__ void dma_rows(const void* base, int nrec, lds_char* dst, const unsigned* off) {
  __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nrec, kBufferFlags);
#pragma unroll
  for (int j = 0; j < N; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + 1024 * j), 16,
                                             off[j], 0, 0, 0);
}

// Workgroup barrier that waits only for this wave's LDS instructions, not for its DMA still in
// flight; the memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Maxima of scores with the IEEE 754-2019 maximum (NaN-propagating), which maps to
// v_maximum3_f32 with no input quieting; fmaxf would first canonicalize every MFMA result.
// Scores are never NaN here (finite inputs, -inf for masked keys).
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3(float a, float b, float c) { return max2(max2(a, b), c); }

// max(x, x of lane l^32) with one v_permlane32_swap_b32 (a VALU lane exchange, no memory
// access): swapping lanes 32-63 of one copy with lanes 0-31 of another leaves [lo, lo] and
// [hi, hi]. It is written as inline asm because the compiler builtin, given two equal inputs,
// returns its first result for both; the s_nop pads cover the VALU-write -> permlane hazard.
__device__ __forceinline__ float max_with_partner_half(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return max2(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// log2(e) * cap * tanh(s * scale / cap), with inv = scale / cap and cap_l2 = cap * log2(e):
// tanh(y) = sign(y) (1 - t) / (1 + t), t = e^(-2|y|) in (0, 1], so nothing overflows and the
// absolute error stays a few ulp of cap (the softmax needs the exponent to absolute accuracy).
__device__ __forceinline__ float softcap_l2(float s, float inv, float cap_l2) {
  const float y = s * inv;
  const float t = __builtin_amdgcn_exp2f(-2.0f * kLog2e * __builtin_fabsf(y));
  const float th = (1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t);
  return __builtin_copysignf(th, y) * cap_l2;
}

// 16 bytes of an FP32 buffer at byte offset `off` (reads at or past the descriptor's end are 0)
__device__ __forceinline__ f32x4 buffer_load_f32x4(__amdgpu_buffer_rsrc_t rsrc, unsigned off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
}

__device__ __forceinline__ bool any_zero_byte(uint32_t x) {
  return ((x - 0x01010101u) & ~x & 0x80808080u) != 0u;
}

// Per-wave key-mask summary for 64 consecutive tiles starting at tile t0: bit i of `any` is set
// when tile t0+i has a valid key, bit i of `all` when every key < S of that tile is valid.
__device__ void key_mask_chunk(const uint8_t* mrow, int S, int t0, int lane, uint64_t* any,
                               uint64_t* all) {
  const long long key0 = (long long)(t0 + lane) * kBN;
  bool a = false, al = false;
  if (key0 < S) {
    const int n = (S - key0) < kBN ? (int)(S - key0) : kBN;
    const uint8_t* p = mrow + key0;
    if (n == kBN && (reinterpret_cast<uintptr_t>(p) & 15u) == 0u) {
      const uint4* p4 = reinterpret_cast<const uint4*>(p);
      bool nz = false, z = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint4 w = p4[r];
        nz |= (w.x | w.y | w.z | w.w) != 0u;
        z = z || any_zero_byte(w.x) || any_zero_byte(w.y) || any_zero_byte(w.z) ||
            any_zero_byte(w.w);
      }
      a = nz;
      al = !z;
    } else {
      bool nz = false, z = false;
      for (int i = 0; i < n; ++i) {
        bool valid = p[i] != 0;
        nz |= valid;
        z |= !valid;
      }
      a = nz;
      al = !z;
    }
  }
  *any = __ballot(a);
  *all = __ballot(al);
}

// Per-wave block-bitmap summary for 64 consecutive tiles starting at tile t0: bit i of `any` is
// set when key block of tile t0+i is selected for some query block in [qb_lo, qb_hi] (the
// workgroup's rows), bit i of `own` when it is selected for query block qb_own (the wave's rows;
// -1 for a wave without rows).
__device__ void sel_chunk(const uint8_t* sel_bh, long long sq, int bk, int qb_lo, int qb_hi, int qb_own,
                          int n_tiles, int t0, int lane, uint64_t* any, uint64_t* own) {
  const int t = t0 + lane;
  bool a = false, o = false;
  if (t < n_tiles) {
    const long long kb = (long long)t * kBN / bk;
    for (int qb = qb_lo; qb <= qb_hi; ++qb) {
      const bool on = sel_bh[(long long)qb * sq + kb] != 0;
      a |= on;
      o |= on & (qb == qb_own);
    }
  }
  *any = __ballot(a);
  *own = __ballot(o);
}

// Kernel variants (template MODE bits): a key mask, a rotating cache, logit soft-capping, an
// additive bias, a block bitmap.
constexpr int kModeKeyMask = 1;
constexpr int kModeRing = 2;
constexpr int kModeSoftcap = 4;
constexpr int kModeBias = 8;
constexpr int kModeSel = 16;

// Key tiles [lo, hi) that query rows [q0, q1) can see (dense layout, skipping on): the causal edge
// bounds hi, the window edge lo.
struct TileRange {
  int lo, hi;
};
__device__ __forceinline__ TileRange skip_range(int q0, int q1, int S, int causal, int causal_offset, int W) {
  const int n_tiles = (S + kBN - 1) / kBN;
  TileRange r{0, n_tiles};
  if (causal) {
    long long hi_key = (long long)q1 + causal_offset;  // exclusive
    if (hi_key > S) hi_key = S;
    if (hi_key < 0) hi_key = 0;
    r.hi = (int)((hi_key + kBN - 1) / kBN);
    if (W > 0) {
      long long lo_key = (long long)q0 + causal_offset - W + 1;
      if (lo_key < 0) lo_key = 0;
      const long long t = lo_key / kBN;
      r.lo = (int)(t < n_tiles ? t : n_tiles);
    }
  }
  return r;
}

// One piece of work of a workgroup: an item (kv head, query block, batch element, head in group)
// and the part [t_from, t_to) of its n key tiles (counted from the item's first tile with skipping
// on). A piece that is not the whole item writes an FP32 partial to workspace slot `slot`; the
// item's parts are the consecutive workgroups v_first .. v_first + n_parts - 1 of the key split.
struct Piece {
  int item;
  int t_from, t_to, n;
  bool whole;
  int slot;
  int v_first, n_parts;
};

// Workspace slot of a part: two per workgroup v of the split, 2v for a part that continues an item
// (it starts inside it), 2v + 1 for a part that starts an item and ends inside it.
__device__ __forceinline__ int part_slot(int v, bool starts_item) { return 2 * v + (starts_item ? 1 : 0); }

// Device-coherent FP32 accesses to the key split's partials: buffer loads and stores with the SC1
// cache-policy bit (agent scope), which go through to the memory side past the per-XCD L2s. They
// are ordinary (non-atomic) accesses, so many are in flight at once.
constexpr int kCoherent = 16;  // SC1
__device__ __forceinline__ void part_store(__amdgpu_buffer_rsrc_t r, unsigned off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, off, 0, kCoherent);
}
__device__ __forceinline__ float part_load(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoherent));
}

template <int D>
struct Slot {
  static constexpr int kRegs = 16 * (D / 32) + 2;   // accumulator registers, reference max, sum
  static constexpr int kFloats = kWaves * 64 * kRegs;
};

template <int D, int MODE>
__device__ __forceinline__ void prefill_piece(const Params& p, const Piece& pc, const int tid) {
  constexpr bool KMASK = (MODE & kModeKeyMask) != 0;
  constexpr bool RING = (MODE & kModeRing) != 0;
  constexpr bool SOFTCAP = (MODE & kModeSoftcap) != 0;
  constexpr bool BIAS = (MODE & kModeBias) != 0;
  constexpr bool SEL = (MODE & kModeSel) != 0;
  // Soft-cap without a bias: the row maximum is taken on the raw scores (the cap is increasing),
  // and each score's exponent is cap log2(e) tanh(y) - reference with y = scale * s / cap, as
  // (cap_l2 - reference) - 2 cap_l2 / (1 + 2^z), z = 2 log2(e) y, all in FP32: one FMA folds the
  // reference in and no sign handling is needed.
  constexpr bool CAPFAST = SOFTCAP && !BIAS;
  using G = Geo<D>;
  constexpr int KQ = G::KQ;
  constexpr int DB = G::DB;
  constexpr int NG1 = 2 * KQ;  // GEMM1 MFMAs per tile
  constexpr int NG2 = 4 * DB;  // GEMM2 MFMAs per tile

  __shared__ __attribute__((aligned(1024))) char lds_raw[kStages * G::kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t m_lds[kStages][kBN];

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const bool group_a = wave < 4;  // waves w and w+4 share a SIMD and take opposite phases

  // ---- workgroup -> (kv head, query-block rank, b, head in group) ----
  // Items are numbered with the KV head slowest, so that (when the hardware deals workgroups to
  // the 8 XCDs round-robin and blockIdx is remapped accordingly) every XCD holds whole KV heads of
  // every batch element: the workgroups that share a K/V tile share an L2, and sequences of
  // different lengths spread over all XCDs. With the causal term the rank comes next (rank 0 is
  // each sequence's heaviest block, so the heaviest blocks start first); without it every block of
  // a sequence has the same work, and the batch element comes next instead, so that the
  // workgroups running together on an XCD share one sequence's K / V (8 sequences of 4096 keys:
  // 1414 -> 1343 us per launch).
  int item = pc.item;
  const bool causal = p.causal != 0;
  // a bias or a bitmap is laid out per head and row block: one head per workgroup there
  const int hpw = (BIAS || SEL) ? 1 : p.hpw;
  const int bm = kBM / hpw;  // query rows of the item
  const int hset = item % p.n_hset;
  item /= p.n_hset;
  int b, qrank;
  if (causal) {
    b = item % p.batch;
    item /= p.batch;
    qrank = item % p.n_qblk;
    item /= p.n_qblk;
  } else {
    qrank = item % p.n_qblk;
    item /= p.n_qblk;
    b = item % p.batch;
    item /= p.batch;
  }
  const int hk = item;
  // the wave's head and row chunk, made scalar explicitly (the compiler cannot see that tid >> 6 is
  // wave-uniform): every per-wave quantity derived from them, such as the tile views, then lives in
  // SGPRs (not with a block bitmap: its per-wave bitmap state then overflowed the scalar registers,
  // and their spills into vector registers spilled those in turn)
  const int wv = SEL ? wave : __builtin_amdgcn_readfirstlane(wave);
  const int h = hk * p.group + hset * hpw + wv % hpw;
  // Rows and keys of this workgroup's sequence, their base elements and strides. Dense layout:
  // [B, H, L|S, D] (row stride D). Packed layout: [total, H, D] (row stride H * D), with the
  // sequence bounds clamped to the packed extents so that malformed prefix sums stay in bounds.
  int L, S, causal_offset;
  long long q_base, kv_base;
  int q_stride, kv_stride;
  if (p.cu_q == nullptr) {
    L = p.lq;
    S = p.sk;
    causal_offset = p.causal_offset;
    q_base = ((long long)b * p.hq + h) * (long long)L * D;
    kv_base = ((long long)b * p.hkv + hk) * (long long)(RING ? p.ring : S) * D;
    q_stride = D;
    kv_stride = D;
  } else {
    const int qs = min(max(p.cu_q[b], 0), p.total_q);
    const int qe = min(max(p.cu_q[b + 1], qs), p.total_q);
    const int ks = min(max(p.cu_k[b], 0), p.total_k);
    const int ke = min(max(p.cu_k[b + 1], ks), p.total_k);
    L = min(qe - qs, p.lq);  // p.lq holds the largest sequence length the grid covers
    S = ke - ks;
    causal_offset = S - L;
    q_base = ((long long)qs * p.hq + h) * D;
    kv_base = ((long long)ks * p.hkv + hk) * D;
    q_stride = p.hq * D;
    kv_stride = p.hkv * D;
  }
  const int W = p.window;
  const int nb = (L + bm - 1) / bm;  // query blocks of this sequence
  if (qrank >= nb) return;  // past the end of a shorter sequence: the whole workgroup leaves
  const int qblk = causal ? (nb - 1 - qrank) : qrank;
  const int q0 = qblk * bm;
  const int q1 = (q0 + bm) < L ? (q0 + bm) : L;

  const uint16_t* kg = p.k + kv_base;
  const uint16_t* vg = p.v + kv_base;
  const uint8_t* mrow = KMASK ? p.key_mask + (long long)b * S : nullptr;
  constexpr bool kmask = KMASK;

  // ---- key-tile range of the piece ----
  // Skipping on: the tiles the block's rows can see, or the piece's part of them. Under NO_SKIP
  // the first part of an item starts at tile 0 and the last one ends at the last tile, so both
  // runs split an item at the same tiles and the extra tiles (fully masked) leave every partial
  // bit for bit as it was.
  const int n_tiles = (S + kBN - 1) / kBN;
  const TileRange sr = skip_range(q0, q1, S, causal, causal_offset, W);
  int kt_lo = pc.whole ? sr.lo : sr.lo + pc.t_from;
  int kt_hi = pc.whole ? sr.hi : sr.lo + pc.t_to;
  if (p.no_skip) {
    if (pc.whole || pc.t_from == 0) kt_lo = 0;
    if (pc.whole || pc.t_to == pc.n) kt_hi = n_tiles;
  }

  // ---- per-wave row state ----
  const int qw0 = q0 + (wv / hpw) * kWaveRows;  // the wave's first row
  const bool wave_active = qw0 < L;
  const int ii_last = wave_active ? ((L - 1 - qw0) < 31 ? (L - 1 - qw0) : 31) : 0;

  bf16x8 qreg[KQ];
  {
    const int row = qw0 + l32;
    if (row < L) {
      const uint16_t* qrow = p.q + q_base + (long long)row * q_stride;
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk)
        qreg[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk + 8 * hh);
    } else {
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk)
#pragma unroll
        for (int t = 0; t < 8; ++t) qreg[kk][t] = (__bf16)0.0f;
    }
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.0f;
  // Running state of the lane's query row: mref is the reference maximum the exponentials are
  // taken against, in the base-2 exponent domain (scores times c; -inf before the row has seen a
  // key), l_run this lane's half of the row sum of P.
  float mref = -INFINITY;
  float l_run = 0.0f;
  // with soft-capping or a bias the scores are turned into the base-2 exponent domain up front
  const float c = (SOFTCAP || BIAS) ? 1.0f : p.c;

  // ---- additive bias: this lane's row of the (b, h) bias, fetched one phase ahead ----
  // Each wave fetches the 32 bias values of its next softmax tile (8 loads of 4 keys) right before
  // its MFMA phase, so the loads land while the matrix core works.
  f32x4 bpre[8];
  const float* bias_base = nullptr;  // wave-uniform (b, h) base of the bias
  unsigned bias_row_off = 0;
  if constexpr (BIAS) {
    const float* bb = p.bias + (long long)b * p.bias_sb + (long long)h * p.bias_sh;
    const uintptr_t a = reinterpret_cast<uintptr_t>(bb);
    const unsigned ahi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
    const unsigned alo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
    bias_base = reinterpret_cast<const float*>(((uintptr_t)ahi << 32) | (uintptr_t)alo);
    bias_row_off = (unsigned)(qw0 + l32) * (unsigned)p.bias_sl * 4u;
#pragma unroll
    for (int i = 0; i < 8; ++i) bpre[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  auto bias_fetch = [&](int kt) __attribute__((always_inline)) {
    if constexpr (BIAS) {
      if (kt < kt_hi) {
        const __amdgpu_buffer_rsrc_t bias_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(bias_base), 0, p.bias_nrec, kBufferFlags);
        const unsigned k0 = (unsigned)kt * kBN;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            bpre[4 * kb + j] = buffer_load_f32x4(bias_rsrc, bias_row_off + (k0 + 32 * kb + 8 * j + 4 * hh) * 4u);
      }
    }
  };

  // ---- key-mask or block-bitmap summary (per wave, 64 tiles per chunk) ----
  // Key mask: m_any = tiles with a valid key, m_all = tiles whose keys are all valid. Block
  // bitmap: m_any = tiles some wave of the workgroup selects, m_all = tiles this wave selects.
  int mchunk = -1;
  uint64_t m_any = 0, m_all = 0;
  const uint8_t* sel_bh = nullptr;
  int qb_lo = 0, qb_hi = -1, qb_own = -1;
  if constexpr (SEL) {
    sel_bh = p.sel + (long long)b * p.sel_sb + (long long)h * p.sel_sh;
    qb_lo = q0 / p.sel_bq;
    qb_hi = (q1 - 1) / p.sel_bq;
    qb_own = wave_active ? qw0 / p.sel_bq : -1;
  }
  auto ensure_chunk = [&](int kt) __attribute__((always_inline)) {
    const int ch = kt >> 6;
    if (ch != mchunk) {
      if constexpr (SEL)
        sel_chunk(sel_bh, p.sel_sq, p.sel_bk, qb_lo, qb_hi, qb_own, n_tiles, ch << 6, lane, &m_any, &m_all);
      else
        key_mask_chunk(mrow, S, ch << 6, lane, &m_any, &m_all);
      mchunk = ch;
    }
  };
  // Next tile >= k (and < kt_hi) to visit, or kt_hi, packed as (tile << 1) | bit. With a key mask
  // or a block bitmap and skipping on, tiles without a valid (selected) key are passed over. The
  // bit is m_all's: whether every key of the returned tile is valid (no elementwise key masking
  // needed), or whether this wave's query block selects the tile.
  auto next_tile = [&](int k) __attribute__((always_inline)) -> int {
    // without a key mask or bitmap every tile of the range is visited; a k >= kt_hi (the end, or an
    // empty range) is treated by every caller like kt_hi
    if (!kmask && !SEL) return (k << 1) | 1;
    if (k >= kt_hi) return (kt_hi << 1) | 1;
    while (k < kt_hi) {
      ensure_chunk(k);
      if (p.no_skip) return (k << 1) | (int)((m_all >> (k & 63)) & 1ull);
      const uint64_t bits = m_any >> (k & 63);
      if (bits) {
        const int t = k + __builtin_ctzll(bits);
        if (t >= kt_hi) return (kt_hi << 1) | 1;
        return (t << 1) | (int)((m_all >> (t & 63)) & 1ull);
      }
      k = (k | 63) + 1;
    }
    return (kt_hi << 1) | 1;
  };

  // ---- tile staging: HBM -> LDS stage by DMA; the key-mask bytes through registers ----
  // Waves 0-3 fetch K, waves 4-7 fetch V, each right after its own MFMA phase. A fetch is a
  // buffer load with the LDS as destination: the buffer descriptor starts at the tile's first key
  // and covers only keys < S, so rows past the end of the cache come back as zeros without any
  // per-lane test. DMA instruction i of a matrix writes LDS bytes [1024 i, 1024 (i+1)) of the
  // tile: lane l lands at row i*RPI + l/CPR, physical chunk l%CPR, and fetches the logical chunk
  // that belongs there (byte offset dma_off[j] within the tile). The table is fixed per wave.
  unsigned dma_off[G::kDmaPerWave];
  const int w4 = wave & 3;
#pragma unroll
  for (int j = 0; j < G::kDmaPerWave; ++j) {
    const int i = w4 * G::kDmaPerWave + j;
    const int row = i * G::kRowsPerDma + lane / G::kChunksPerRow;
    const int pch = lane % G::kChunksPerRow;
    const int sw = group_a ? G::swz_k(row) : G::swz_v(row);
    dma_off[j] = (unsigned)(row * 2 * kv_stride + 16 * (pch ^ sw));
  }
  // wave-uniform values, made scalar explicitly (the compiler cannot see that tid >> 6 is), so
  // that a fetch's address arithmetic is scalar only: with the source pointer in vector registers
  // it went through a vector add and two readfirstlanes, and each fetch cost a few hundred cycles
  // after the MFMA phase
  const int dma_lds = __builtin_amdgcn_readfirstlane((group_a ? 0 : G::kVRegion) + w4 * G::kDmaPerWave * 1024);
  unsigned long long dma_src;
  {
    // readfirstlane returns int: go through unsigned so the low word is not sign-extended
    const uintptr_t a = reinterpret_cast<uintptr_t>(group_a ? kg : vg);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
    dma_src = ((unsigned long long)hi << 32) | lo;
  }
  const int tile_bytes = kBN * 2 * kv_stride;  // < 2^31: kv_stride < 2^24
  uint8_t mreg = 0;
  // this wave's share of matrix (K for waves 0-3, V for 4-7) of tile kt into stage st
  auto issue = [&](int kt, int st) __attribute__((always_inline)) {
    const int key0 = kt * kBN;  // kt * 64 <= S + 63 < 2^31
    const int rows = S - key0;
    constexpr bool ring = RING;  // rotating cache (p.ring slots)
    // ring cache: the descriptor covers the whole ring
    const int nrec = ring ? p.ring * G::kRowBytes : (rows < kBN ? rows : kBN) * 2 * kv_stride;
    const uintptr_t base_u = ring ? dma_src : dma_src + (unsigned long long)(unsigned)kt * (unsigned)tile_bytes;
    lds_char* dst = (lds_char*)lds_raw + st * G::kTileBytes + dma_lds;
    if constexpr (!ring) {
      dma_rows<G::kDmaPerWave>(reinterpret_cast<const void*>(base_u), __builtin_amdgcn_readfirstlane(nrec),
                               dst, dma_off);
    } else {
      // row r of the tile (position key0 + r) is slot (key0 mod ring) + r, wrapped once
      // (ring >= 64 > r); rows at positions past S read as zeros (offset at the descriptor's end)
      const int slot0 = (int)(key0 % p.ring);
      unsigned off[G::kDmaPerWave];
#pragma unroll
      for (int j = 0; j < G::kDmaPerWave; ++j) {
        const int row = (w4 * G::kDmaPerWave + j) * G::kRowsPerDma + lane / G::kChunksPerRow;
        int slot = slot0 + row;
        if (slot >= p.ring) slot -= p.ring;
        const unsigned in_row = dma_off[j] - (unsigned)(row * G::kRowBytes);
        off[j] = (row < rows) ? (unsigned)(slot * G::kRowBytes) + in_row : (unsigned)nrec;
      }
      dma_rows<G::kDmaPerWave>(reinterpret_cast<const void*>(base_u), __builtin_amdgcn_readfirstlane(nrec),
                               dst, off);
    }
    if (kmask && tid < kBN) mreg = (key0 + tid < S) ? mrow[key0 + tid] : (uint8_t)0;
  };
  // wait for this wave's fetches; waves 0-3 also publish the tile's mask bytes
  auto finish = [&](int st) __attribute__((always_inline)) {
    if (kmask && tid < kBN) m_lds[st][tid] = mreg;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };

  // ---- per-lane LDS read addresses (byte offsets inside a K or V tile) ----
  // K (GEMM1 A operand): row l32 (+32 kb), logical chunk 2kk+hh -> address a_k ^ (32 kk).
  int a_k;
  {
    const int x = G::swz_k(l32);
    a_k = l32 * G::kRowBytes + 16 * (hh ^ (x & 1)) + 32 * (x >> 1);
  }
  // V^T (GEMM2 A operand, transpose reads): 16-lane group g16 reads rows 4(g16>>1)+r4 of a
  // 16-key step, columns 32db + 16(g16&1) + 4cc -> address a_v ^ (64 db).
  int a_v;
  {
    const int g16 = lane >> 4, loc = lane & 15, r4 = loc >> 2, cc = loc & 3;
    const int row = 4 * (g16 >> 1) + r4;
    const int sv = G::swz_v(row) >> 2;  // swizzle of the 64-byte column block
    a_v = row * G::kRowBytes + 64 * sv + 32 * (g16 & 1) + 8 * cc;
  }
  // the four V^T read addresses of the lane, with kVHeld added; the empty asm hides the addition
  // from the compiler, which would otherwise fold it back into (too large) immediate offsets
  int a_vh[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db) {
    a_vh[db] = (a_v ^ (64 * db)) + G::kVHeld;
    asm volatile("" : "+v"(a_vh[db]));
  }

  // ---- per-wave view of one tile: mask thresholds, skip and mask decisions ----
  struct TileView {
    int lim_tail, dc, dw;
    bool live;       // some real row of this wave sees some key of the tile
    bool need_mask;  // the tile straddles an edge for this wave
  };
  // Row ii of the wave sees tile key jj iff dw <= jj - ii <= dc and jj < lim_tail. The causal
  // and window bounds relative to key 0 are precomputed per wave and saturated (keys and rows fit
  // in 31 bits), so the per-tile view is a few branch-free integer operations; with no causal
  // term dc is pinned at +256 and with no window dw at -256, i.e. no bound inside a tile.
  const int cbase = [&] {
    if (!causal) return S + 512;
    const long long t = (long long)causal_offset + qw0;
    return (int)(t < -512 ? -512 : (t > (long long)S + 512 ? (long long)S + 512 : t));
  }();
  const int wbase = [&] {
    if (!causal || W <= 0) return -512;
    const long long t = (long long)causal_offset - W + 1 + qw0;
    return (int)(t < -512 ? -512 : (t > (long long)S + 512 ? (long long)S + 512 : t));
  }();
  // Tiles that every row of the wave sees whole -- no causal, window or tail edge inside them, i.e.
  // dc >= 63, dw <= -31 and lim_tail == 64 below -- are kt in [t_int_lo, t_int_hi]; with every key
  // valid (or, with a block bitmap, the tile selected) their view is constant.
  const int t_int_lo = (wbase + 31 + (kBN - 1)) >> 6;                 // ceil((wbase + 31) / 64)
  const int t_int_hi = min((cbase - (kBN - 1)) >> 6, (S >> 6) - 1);  // floor((cbase - 63) / 64)
  auto view_of = [&](int kt, bool tile_bit) __attribute__((always_inline)) -> TileView {
    TileView tv;
    if ((kt >= t_int_lo) & (kt <= t_int_hi) & tile_bit) {
      tv.lim_tail = kBN;
      tv.dc = 256;
      tv.dw = -256;
      tv.live = wave_active;
      tv.need_mask = false;
      return tv;
    }
    const int key0 = kt * kBN;
    // a tile the wave's query block does not select is a tile without keys (lim_tail = 0)
    const bool selected = SEL ? tile_bit : true;
    const bool tile_all_valid = SEL ? true : tile_bit;
    tv.lim_tail = selected ? min(S - key0, kBN) : 0;
    tv.dc = max(min(cbase - key0, 256), -256);
    tv.dw = max(min(wbase - key0, 256), -256);
    const int lo = max(tv.dw, -ii_last);
    const int hi = min(tv.dc, tv.lim_tail - 1);
    tv.live = wave_active & ((p.no_skip != 0) | ((lo <= hi) & selected));
    tv.need_mask = (tv.lim_tail < kBN) | (tv.dc < kBN - 1) | (tv.dw > -31) | !tile_all_valid;
    return tv;
  };

  // ---- the MFMA phase: GEMM1 of one tile and/or GEMM2 of the previous one ----
  f32x16 s[2];   // scores of a tile between GEMM1 and SOFTMAX
  bf16x8 pb[4];  // probabilities of a tile between SOFTMAX and GEMM2

  // GEMM1 of the current tile and GEMM2 of the previous one, steps alternating. Both always run:
  // a wave with no scores to make runs GEMM1 for nothing, and a wave with no probabilities runs
  // GEMM2 on pb = 0, which adds exact zeros to the accumulator (it starts at +0 and sums
  // non-negative weights, so it is never -0 and acc + 0 == acc bit for bit).
  auto mfma_run = [&](int st1, int st2, auto do_g1, auto do_g2) __attribute__((always_inline)) {
    constexpr bool DO1 = decltype(do_g1)::value;
    constexpr bool DO2 = decltype(do_g2)::value;
    const lds_char* base1 = (const lds_char*)lds_raw + st1 * G::kTileBytes;
    const lds_char* base2 = (const lds_char*)lds_raw + (G::kVRegion - G::kVHeld) + st2 * G::kTileBytes;
    auto load_g1 = [&](int j) __attribute__((always_inline)) -> bf16x8 {
      const int kb = j / KQ, kk = j % KQ;
      return *(const lds_bf16x8*)(base1 + kb * 32 * G::kRowBytes + (a_k ^ (32 * kk)));
    };
    auto load_g2 = [&](int j) __attribute__((always_inline)) -> bf16x8 {
      const int kb = j / (2 * DB), c2 = (j / DB) & 1, db = j % DB;
      const lds_char* pr = base2 + (kb * 32 + 16 * c2) * G::kRowBytes + a_vh[db];
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pr);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pr + 8 * G::kRowBytes));
      // Join the two reads as one integer vector and reinterpret it whole: assembling the bf16
      // operand element by element from 16-bit integers is mis-lowered by the compiler.
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto mma_g1 = [&](int j, const bf16x8& a) __attribute__((always_inline)) {
      const int kb = j / KQ, kk = j % KQ;
      if (kk == 0) {
        f32x16 z;
#pragma unroll
        for (int v = 0; v < 16; ++v) z[v] = 0.0f;
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[0], z, 0, 0, 0);
      } else {
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s[kb], 0, 0, 0);
      }
    };
    auto mma_g2 = [&](int j, const bf16x8& a) __attribute__((always_inline)) {
      const int kb = j / (2 * DB), c2 = (j / DB) & 1, db = j % DB;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[2 * kb + c2], acc[db], 0, 0, 0);
    };
    bf16x8 ring[kRing];
    // both: even steps GEMM1, odd steps GEMM2 (NG1 == NG2); otherwise the one GEMM alone
    constexpr int NS = (DO1 ? NG1 : 0) + (DO2 ? NG2 : 0);
    auto is_g2 = [](int m) { return DO1 && DO2 ? (m & 1) != 0 : DO2; };
    auto index = [](int m) { return DO1 && DO2 ? (m >> 1) : m; };
#pragma unroll
    for (int m = 0; m < NS + kRing - 1; ++m) {
      if (m < NS) {
        if (is_g2(m)) {
          ring[m % kRing] = load_g2(index(m));
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        } else {
          ring[m % kRing] = load_g1(index(m));
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
      }
      const int u = m - (kRing - 1);
      if (u >= 0) {
        if (is_g2(u)) mma_g2(index(u), ring[u % kRing]);
        else mma_g1(index(u), ring[u % kRing]);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      }
    }
  };
  // g1 / g2 (constants): whether the iteration has a current tile (GEMM1) and a previous one
  // (GEMM2); the first iteration of a piece has no previous tile (P would be zero) and the last no
  // current one (its scores would never be used), so they leave that GEMM out. With a block bitmap
  // a wave often has no keys in the tile (its query block did not select it) while the workgroup
  // visits it for the other waves: then its GEMM1 (scores never used) and its GEMM2 of a tile
  // without keys (P = 0, adding exact zeros) are left out as well.
  auto mfma_phase = [&](int st1, int st2, bool live1, bool live2, auto g1, auto g2) __attribute__((always_inline)) {
    using T = std::true_type;
    using F = std::false_type;
    constexpr bool G1 = decltype(g1)::value;
    constexpr bool G2 = decltype(g2)::value;
    if constexpr (SEL) {
      const bool l1 = G1 && live1, l2 = G2 && live2;
      if (l1 && l2) mfma_run(st1, st2, T{}, T{});
      else if (l1) mfma_run(st1, st2, T{}, F{});
      else if (l2) mfma_run(st1, st2, F{}, T{});
    } else {
      mfma_run(st1, st2, g1, g2);
    }
  };

  // ---- the VALU phase: mask, online softmax, P in bf16, accumulator rescale ----
  auto softmax = [&](const TileView& tv, int st) __attribute__((always_inline)) {
    if constexpr (SOFTCAP && !CAPFAST) {
      // logit soft-capping before the masks and the softmax (brotensor flash_attention_decode,
      // attn_softcap): x = log2(e) * cap * tanh(scale * s / cap)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = softcap_l2(s[kb][v], p.sc_inv, p.sc_cap_l2);
    }
    if constexpr (BIAS) {
      // x = c s + log2(e) bias (after the soft-cap, which already is in the base-2 domain), before
      // the masks (tiny-llm Task 2: the additive mask is applied before the online-softmax update)
      const float c0 = SOFTCAP ? 1.0f : p.c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            s[kb][4 * j + i] = __builtin_fmaf(s[kb][4 * j + i], c0, bpre[4 * kb + j][i] * kLog2e);
    }
    // masked scores become -inf (run on tiles that cross an edge)
    auto apply_mask = [&]() __attribute__((always_inline)) {
      // Row ii = l32 sees tile keys jj in [lo, lo + span] (causal, window and tail bounds),
      // tested as one unsigned compare per score; span < 0 means the row sees nothing.
      const int ii = l32;
      int lo = ii + tv.dw;
      if (lo < 0) lo = 0;
      int hi = ii + tv.dc;
      if (hi > tv.lim_tail - 1) hi = tv.lim_tail - 1;
      unsigned span = (unsigned)(hi - lo);
      if (hi < lo) {
        lo = kBN;  // every jj - lo is then negative, i.e. a huge unsigned value
        span = 0;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t mb =
              kmask ? *reinterpret_cast<const uint32_t*>(&m_lds[st][kb * 32 + 8 * j + 4 * hh])
                    : 0xFFFFFFFFu;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jj = kb * 32 + 8 * j + 4 * hh + i;
            const bool vis = ((unsigned)(jj - lo) <= span) & (((mb >> (8 * i)) & 0xFFu) != 0u);
            s[kb][4 * j + i] = vis ? s[kb][4 * j + i] : -INFINITY;
          }
        }
      }
    };
    if (tv.need_mask) apply_mask();
    // per lane: one query row, 32 of the tile's 64 keys. Short dependency chains: a tree of
    // 3-input maxima, the cross-half exchange as a VALU lane swap, independent exponentials and
    // four partial sums.
    float r[32];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      r[v] = s[0][v];
      r[16 + v] = s[1][v];
    }
    float t1[12];
#pragma unroll
    for (int i = 0; i < 10; ++i) t1[i] = max3(r[3 * i], r[3 * i + 1], r[3 * i + 2]);
    t1[10] = r[30];
    t1[11] = r[31];
    const float t2a = max3(t1[0], t1[1], t1[2]);
    const float t2b = max3(t1[3], t1[4], t1[5]);
    const float t2c = max3(t1[6], t1[7], t1[8]);
    const float t2d = max3(t1[9], t1[10], t1[11]);
    const float mtile = max_with_partner_half(max3(t2a, t2b, max2(t2c, t2d)));
    // z = 2 log2(e) scale s / cap (soft-cap only)
    const float zk = CAPFAST ? 2.0f * kLog2e * p.sc_inv : 0.0f;
    float mx;
    if constexpr (CAPFAST) {
      // the tile maximum of the capped exponents, from the largest raw score (-inf: none seen)
      mx = (mtile == -INFINITY)
               ? -INFINITY
               : __builtin_fmaf(__builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(mtile * zk)), -2.0f * p.sc_cap_l2,
                                p.sc_cap_l2);
    } else {
      mx = mtile * c;
    }
    // Lazy rescaling: the reference is raised (and the accumulators rescaled) only when some
    // row's tile maximum exceeds it by more than 2^8 in probability, or a row meets its first
    // visible key (mx - mref = +inf); otherwise P <= 256, exact arithmetic on both sides of the
    // final a / l. A row that has seen nothing yet and sees nothing here gives -inf - -inf = NaN,
    // which compares false: a fully masked tile never raises, so visiting it changes nothing.
    const bool raise = __any((mx - mref) > kLazyLog2);
    const float mnew = raise ? max2(mref, mx) : mref;
    const float msub_new = (mnew == -INFINITY) ? 0.0f : mnew;
    if (raise) {
      // rescale the accumulator and the sum to the raised reference before this tile's terms
      // (a row still without keys keeps alpha = 1: its accumulator and sum are zero)
      const float alpha = (mnew == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(mref - mnew);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
      l_run *= alpha;
    }
    mref = mnew;
    if constexpr (CAPFAST) {
      const float k0 = p.sc_cap_l2 - msub_new;
#pragma unroll
      for (int v = 0; v < 32; ++v)
        r[v] = __builtin_fmaf(__builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(r[v] * zk)), -2.0f * p.sc_cap_l2, k0);
      if (tv.need_mask) {
        // a masked score caps to a finite value: mask the exponents themselves
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          r[v] = (s[0][v] == -INFINITY) ? -INFINITY : r[v];
          r[16 + v] = (s[1][v] == -INFINITY) ? -INFINITY : r[16 + v];
        }
      }
    }
    // P in bf16 pairs; the row sum is taken over the rounded values (the weights that multiply
    // V), one dot product with (1, 1) per pair in four independent chains, the first seeded with
    // the running sum. The operand is assembled from whole 32-bit pairs: extracting pairs back
    // out of the bf16x8 vector is mis-lowered by the compiler.
    float ls[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = CAPFAST ? __builtin_amdgcn_exp2f(r[8 * q4 + 2 * i])
                                 : __builtin_amdgcn_exp2f(__builtin_fmaf(r[8 * q4 + 2 * i], c, -msub_new));
        const float e1 = CAPFAST ? __builtin_amdgcn_exp2f(r[8 * q4 + 2 * i + 1])
                                 : __builtin_amdgcn_exp2f(__builtin_fmaf(r[8 * q4 + 2 * i + 1], c, -msub_new));
        const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
        const float seed = q4 > 0 ? ls[i] : (i == 0 ? l_run : 0.0f);
        ls[i] = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, seed, false);
        w[i] = __builtin_bit_cast(unsigned, pr);
      }
      pb[q4] = __builtin_bit_cast(bf16x8, w);
    }
    l_run = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  // ---- main loop ----
  // An iteration works on tile `cur` (its K in stage st_cur), tile `prv` (its V in stage st_prv)
  // and fetches tile `nxt` into the third stage. A wave runs its MFMA phase in one half of the
  // iteration and its softmax phase in the other (group A: MFMA first); the iteration ends with a
  // barrier (and, at D = 64 or with a bias, its halves are separated by one). Group A issues the
  // fetch of `nxt` right after its MFMA phase; it lands during the second half and is waited for
  // before the closing barrier.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) pb[i][t] = (__bf16)0.0f;
  int packed = next_tile(kt_lo);
  int cur = packed >> 1;
  bool all_cur = packed & 1;
  // The first tile goes to stage 0 (every byte of it written by the fetch, keys past S as zeros).
  // No GEMM ever reads a stage before its tile has landed: GEMM1 of an iteration reads the K of
  // the tile fetched before it, GEMM2 the V of the tile fetched two halves earlier, and the first
  // iteration of a piece runs no GEMM2. So the other stages need no initial contents (uninitialised
  // LDS could hold non-finite bit patterns, which times P = 0 would still give NaN: the peeled
  // first iteration is what keeps them out of the accumulators).
  // (a later piece of the workgroup reuses the stages: every wave has left the previous piece's
  // loop, whose last barrier follows its last LDS read, before any wave gets here)
  if (cur < kt_hi) issue(cur, 0);
  if (cur < kt_hi) finish(0);
  __syncthreads();
  TileView tv_cur{}, tv_prv{};
  tv_prv.live = false;
  auto softmax_phase = [&](const TileView& tv, int st) __attribute__((always_inline)) {
    if (__builtin_amdgcn_readfirstlane((int)tv.live)) {  // wave-uniform: a scalar branch
      softmax(tv, st);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t) pb[i][t] = (__bf16)0.0f;
    }
  };
  // `group` is the wave's group: a runtime flag (one loop for both groups, their phases selected
  // under the execution mask) or, with a bias, a constant (the two groups run separate copies of
  // the loop behind a branch on a wave-uniform value, so the compiler sees each group's own tile
  // fetches only and does not make one group's LDS reads wait for the loads of the other: its
  // bias loads. Without a bias the shared loop is the faster one.)
  // One iteration; g1 / g2 (constants) say whether it has a current and a previous tile: the loop
  // runs one iteration without a previous tile, then full ones, then one without a current tile.
  // stage: the stage of the current tile (iteration k of a piece uses stage k mod 3), a constant in
  // all but the last iteration (without a bias), so that the LDS addresses of the operand reads are
  // constant offsets from the lane's read addresses.
  auto iteration = [&](auto group, auto g1, auto g2, auto stage) __attribute__((always_inline)) {
    constexpr bool G1 = decltype(g1)::value;
    constexpr bool G2 = decltype(g2)::value;
    const bool GA = group;
    const int st_cur = stage;
    const int st_prv = st_cur == 0 ? kStages - 1 : st_cur - 1;
    const int st_nxt = st_cur + 1 == kStages ? 0 : st_cur + 1;
    const int packed_nxt = next_tile(cur + 1 <= kt_hi ? cur + 1 : kt_hi);
    const int nxt = packed_nxt >> 1;
    const bool all_nxt = packed_nxt & 1;
    if constexpr (G1) {
      tv_cur = view_of(cur, all_cur);
    } else {
      tv_cur.live = false;
    }
    // first half
    if (GA) {
      if constexpr (G1) bias_fetch(cur);  // for this iteration's softmax (second half)
      mfma_phase(st_cur, st_prv, tv_cur.live, tv_prv.live, g1, g2);
      if (nxt < kt_hi) issue(nxt, st_nxt);  // K of tile nxt
    } else {
      // With a bias, V of tile cur is fetched here rather than at the end of the previous
      // iteration: no tile fetch is then in flight across the loop edge, so the MFMA phase's
      // LDS reads need not wait for the bias loads issued just before it. (Tile cur of the first
      // iteration was fetched whole by the prologue.)
      if constexpr (BIAS && G1 && G2) issue(cur, st_cur);
      if constexpr (G2) softmax_phase(tv_prv, st_prv);  // (first iteration: P is still zero)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // V of tile cur has landed
    }
    // Nothing stored to LDS in the first half is read in the second (the K in flight targets
    // the stage nobody reads this iteration), so the middle barrier only aligns the phases. At
    // D = 128 without a bias the phases stay aligned by themselves and the iteration is faster
    // without it; at D = 64 (a softmax phase much longer than the MFMA phase) it is faster with.
    if constexpr (D != 128 || BIAS) __builtin_amdgcn_s_barrier();
    // second half
    if (GA) {
      if constexpr (G1) softmax_phase(tv_cur, st_cur);
      if (nxt < kt_hi) finish(st_nxt);
      // with a bias, also wait where no fetch was issued, so that no path leaves one in flight
      if constexpr (BIAS) __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
      bias_fetch(cur);  // for the next iteration's softmax (first half), whose tile is this cur
      mfma_phase(st_cur, st_prv, tv_cur.live, tv_prv.live, g1, g2);
      if constexpr (!BIAS) {
        if (nxt < kt_hi) issue(nxt, st_nxt);  // V of tile nxt: first read one iteration later
      }
    }
    lds_barrier();
    tv_prv = tv_cur;
    cur = nxt;
    all_cur = all_nxt;
  };
  auto main_loop = [&](auto group) __attribute__((always_inline)) {
    using T = std::true_type;
    using F = std::false_type;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    static_assert(kStages == 3, "the loop is unrolled over three stages");
    if (cur < kt_hi) {
      iteration(group, T{}, F{}, S0{});
      int st_last = 1;
      if constexpr (!BIAS) {
        for (;;) {
          if (cur >= kt_hi) { st_last = 1; break; }
          iteration(group, T{}, T{}, S1{});
          if (cur >= kt_hi) { st_last = 2; break; }
          iteration(group, T{}, T{}, S2{});
          if (cur >= kt_hi) { st_last = 0; break; }
          iteration(group, T{}, T{}, S0{});
        }
      } else {
        // the bias mode runs a separate loop per wave group; unrolled, its bias loads in flight
        // no longer fit the registers
        while (cur < kt_hi) {
          iteration(group, T{}, T{}, st_last);
          st_last = st_last + 1 == kStages ? 0 : st_last + 1;
        }
      }
      iteration(group, F{}, T{}, st_last);
    }
  };
  if constexpr (BIAS) {
    if (__builtin_amdgcn_readfirstlane(wave) < 4)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
  } else {
    main_loop(group_a);
  }

  // ---- a part of an item: its partial to the workspace; the last part to finish merges ----
  if (!pc.whole) {
    using SL = Slot<D>;
    __shared__ int s_last;
    // the partial slots: 2 per workgroup of the split, each lane's values 64 floats apart
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        p.ws_part, 0, 2 * pfa::kSplitWorkgroups * SL::kFloats * 4, kBufferFlags);
    auto part_base = [&](int slot) -> unsigned {
      return ((unsigned)slot * SL::kFloats + (unsigned)(wave * SL::kRegs * 64 + lane)) * 4u;
    };
    const unsigned mine = part_base(pc.slot);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) part_store(rs, mine + (16 * db + v) * 256, acc[db][v]);
    part_store(rs, mine + (16 * DB) * 256, mref);
    part_store(rs, mine + (16 * DB + 1) * 256, l_run);
    // Partials are written and read with device-coherent accesses instead of a device-wide fence
    // (which writes back and invalidates this XCD's whole L2, where the other workgroups stream
    // K / V). Every store has completed before the count is raised (the asm also keeps the
    // compiler from moving a store past it), and the last part's loads are issued only after its
    // count has returned.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&p.ws_cnt[pc.item], 1u) + 1u == (unsigned)pc.n_parts;
    __syncthreads();
    if (!s_last) return;
    // merge the parts in their key order, whichever finished last: the merge equations (tiny-llm
    // Task 1) on (reference max, sum, accumulator) in the base-2 domain, taken against the largest
    // reference of the parts; a part without visible keys (reference -inf, sum 0, zero
    // accumulator) gets weight 0
    float mm = -INFINITY;
    for (int k = 0; k < pc.n_parts; ++k)
      mm = max2(mm, part_load(rs, part_base(part_slot(pc.v_first + k, k == 0)) + (16 * DB) * 256));
    l_run = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[db][v] = 0.0f;
    for (int k = 0; k < pc.n_parts; ++k) {
      const unsigned src = part_base(part_slot(pc.v_first + k, k == 0));
      // all of a part's loads are issued before the first is used (the scheduling barrier keeps
      // the compiler from waiting for each load before issuing the next, which it did in the
      // key-mask instantiations and which made a 16-part merge hundreds of microseconds long)
      float x[16 * DB + 2];
#pragma unroll
      for (int i = 0; i < 16 * DB + 2; ++i) x[i] = part_load(rs, src + i * 256);
      __builtin_amdgcn_sched_barrier(0);
      const float mk = x[16 * DB];
      const float w = (mk == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mk - mm);
      l_run = __builtin_fmaf(x[16 * DB + 1], w, l_run);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = __builtin_fmaf(x[16 * db + v], w, acc[db][v]);
    }
    mref = mm;
    if (tid == 0) __hip_atomic_store(&p.ws_cnt[pc.item], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next call
  }

  // ---- epilogue: O = acc / l, rows without visible keys -> 0 ----
  if (!wave_active) return;
  float lt = l_run + __shfl_xor(l_run, 32);
  // an attention sink adds e^sink to the normaliser, relative to the row's reference maximum
  // (overflow to +inf gives O = 0, the limit; a -inf sink adds 0)
  if (p.sinks != nullptr && lt > 0.0f) lt += __builtin_amdgcn_exp2f(__builtin_fmaf(p.sinks[h], kLog2e, -mref));
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  // The lane holds 8-byte pieces of its row; stored as they are, every store instruction would
  // touch 32 rows with 16 bytes each. They go through the wave's own 32 rows of LDS instead (the
  // stages are free: the loop's last barrier follows every wave's last read of them, and no fetch
  // is in flight), 16-byte chunks XOR-swizzled by row, and leave as whole rows: 16-byte stores,
  // consecutive lanes on consecutive chunks.
  constexpr int kChunks = G::kRowBytes / 16;  // 16-byte chunks per row
  lds_char* obuf = (lds_char*)lds_raw + wave * (kWaveRows * G::kRowBytes);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc[db][4 * j + i] * inv);
      const int c = (4 * db + j) ^ (l32 & (kChunks - 1));
      *(__attribute__((address_space(3))) bf16x4*)(obuf + l32 * G::kRowBytes + 16 * c + 8 * hh) = ov;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the writes of the other lanes are in LDS
  constexpr int kRowsPerStore = 64 / kChunks;
  const int cl = lane % kChunks;
#pragma unroll
  for (int i = 0; i < kWaveRows / kRowsPerStore; ++i) {
    const int r = i * kRowsPerStore + lane / kChunks;
    const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(obuf + r * G::kRowBytes +
                                                                         16 * (cl ^ (r & (kChunks - 1))));
    if (qw0 + r < L) *reinterpret_cast<u32x4*>(p.o + q_base + (long long)(qw0 + r) * q_stride + 8 * cl) = v;
  }
}

// The key split's walk over its linear (item, key tile) space: items in the order of the per-item
// grid (KV head slowest, then query-block rank, batch element, head in group; without the causal
// term the item decodes batch element before rank, which changes nothing here since every rank
// then has the same tiles), each with the tiles of its query block; the tile count depends on the
// rank only. Workgroup v of Pe takes tiles
// [T v / Pe, T (v + 1) / Pe). One thread keeps the walk in LDS and advances it between pieces, so
// nothing of it is held in registers across a piece.
struct SplitWalk {
  long long T, T_head, per_block;  // tiles in all, tiles of one KV head, items per (KV head, rank)
  long long base;                  // linear start of the current (KV head, rank) block
  long long in_block;              // item within that block
  long long pos, r1;               // next tile of the share, end of the share
  int hk, qrank, n, nb, Pe, v;
  int done;
  int zero;  // 0, read again for every piece (see the piece loop)
  Piece pc;
};

// Tiles of query-block rank qrank (skipping on). A block whose rows see no key (a window past the
// last key) weighs one tile: it is then always a whole piece of some workgroup, which runs its
// true (empty) range and writes zeros.
__device__ __forceinline__ int split_tiles_of(const Params& p, int qrank, int nb) {
  const int qblk = p.causal ? (nb - 1 - qrank) : qrank;
  const int q0 = qblk * kBM;
  const int q1 = (q0 + kBM) < p.lq ? (q0 + kBM) : p.lq;
  const TileRange r = skip_range(q0, q1, p.sk, p.causal, p.causal_offset, p.window);
  return r.hi - r.lo > 1 ? r.hi - r.lo : 1;
}

// Workgroup of the split whose share holds linear tile t.
__device__ __forceinline__ int split_wg_of(const SplitWalk& w, long long t) {
  auto start_of = [&](int k) -> long long { return w.T * k / w.Pe; };
  int k = (int)(t * w.Pe / w.T);
  while (k + 1 < w.Pe && start_of(k + 1) <= t) ++k;
  while (k > 0 && start_of(k) > t) --k;
  return k;
}

// The piece at w.pos (w.pos < w.r1), or done.
__device__ __forceinline__ void split_piece(SplitWalk& w) {
  if (w.pos >= w.r1) {
    w.done = 1;
    return;
  }
  const long long I = w.base + w.in_block * w.n;  // the item's first linear tile
  Piece& pc = w.pc;
  pc.item = (int)(((long long)w.hk * w.nb + w.qrank) * w.per_block + w.in_block);
  pc.n = w.n;
  pc.t_from = (int)(w.pos - I);
  pc.t_to = (int)((w.r1 - I) < w.n ? (w.r1 - I) : w.n);
  pc.whole = pc.t_from == 0 && pc.t_to == w.n;
  pc.slot = part_slot(w.v, pc.t_from == 0);
  pc.v_first = pc.whole ? w.v : split_wg_of(w, I);
  pc.n_parts = pc.whole ? 1 : split_wg_of(w, I + w.n - 1) - pc.v_first + 1;
  w.pos = I + pc.t_to;
}

__device__ __forceinline__ void split_init(const Params& p, SplitWalk& w) {
  const int P = gridDim.x;  // a multiple of kXcds
  // v follows the hardware's round-robin over the 8 XCDs, so each XCD takes a contiguous eighth of
  // the space (whole KV heads, when the heads divide evenly)
  w.v = (blockIdx.x % kXcds) * (P / kXcds) + blockIdx.x / kXcds;
  w.nb = (p.lq + kBM - 1) / kBM;
  w.per_block = (long long)p.batch * p.group;
  w.T_head = 0;
  for (int r = 0; r < w.nb; ++r) w.T_head += w.per_block * split_tiles_of(p, r, w.nb);
  w.T = w.T_head * p.hkv;
  // with fewer tiles than workgroups only the first T take a share, so every share is non-empty
  // and the parts of an item are consecutive workgroups
  w.Pe = (int)(w.T < P ? w.T : P);
  w.done = 0;
  w.zero = 0;
  if (w.v >= w.Pe) {
    w.done = 1;
    return;
  }
  const long long r0 = w.T * w.v / w.Pe;
  w.r1 = w.T * (w.v + 1) / w.Pe;
  // locate r0: KV head, rank, item within the (head, rank) block
  w.hk = (int)(r0 / w.T_head);
  long long rem = r0 - w.hk * w.T_head;
  w.base = w.hk * w.T_head;
  w.qrank = 0;
  w.n = split_tiles_of(p, 0, w.nb);
  while (rem >= w.per_block * w.n) {
    rem -= w.per_block * w.n;
    w.base += w.per_block * w.n;
    ++w.qrank;
    w.n = split_tiles_of(p, w.qrank, w.nb);
  }
  w.in_block = rem / w.n;
  w.pos = r0;
  split_piece(w);
}

__device__ __forceinline__ void split_next(const Params& p, SplitWalk& w) {
  if (++w.in_block == w.per_block) {
    w.in_block = 0;
    w.base += w.per_block * w.n;
    if (++w.qrank == w.nb) {
      w.qrank = 0;
      ++w.hk;
    }
    w.n = split_tiles_of(p, w.qrank, w.nb);
  }
  split_piece(w);
}

template <int D, int MODE, bool SPLIT>
__global__ __launch_bounds__(kThreads) void pfa_prefill_kernel(Params p) {
  if constexpr (!SPLIT) {
    // one workgroup per item
    int item = blockIdx.x;
    if (p.xcd_remap) item = (blockIdx.x % kXcds) * (p.n_wg / kXcds) + blockIdx.x / kXcds;
    Piece pc{};
    pc.item = item;
    pc.whole = true;
    prefill_piece<D, MODE>(p, pc, (int)threadIdx.x);
  } else {
    // key split (dense layout): a fixed grid, each workgroup its share of the linear space
    __shared__ SplitWalk walk;
    if (threadIdx.x == 0) split_init(p, walk);
    __syncthreads();
    for (;;) {
      if (__builtin_amdgcn_readfirstlane(walk.done)) break;
      Piece pc;
      pc.item = __builtin_amdgcn_readfirstlane(walk.pc.item);
      pc.t_from = __builtin_amdgcn_readfirstlane(walk.pc.t_from);
      pc.t_to = __builtin_amdgcn_readfirstlane(walk.pc.t_to);
      pc.n = __builtin_amdgcn_readfirstlane(walk.pc.n);
      pc.whole = __builtin_amdgcn_readfirstlane((int)walk.pc.whole) != 0;
      pc.slot = __builtin_amdgcn_readfirstlane(walk.pc.slot);
      pc.v_first = __builtin_amdgcn_readfirstlane(walk.pc.v_first);
      pc.n_parts = __builtin_amdgcn_readfirstlane(walk.pc.n_parts);
      // the thread index plus a zero the compiler cannot see through: everything a piece derives
      // from the lane (LDS and global addresses) is then computed per piece instead of being
      // hoisted out of this loop, where it would stay live through every piece's merge
      prefill_piece<D, MODE>(p, pc, (int)threadIdx.x + walk.zero);
      __syncthreads();  // every wave is done with the piece (and with reading the walk)
      if (threadIdx.x == 0) split_next(p, walk);
      __syncthreads();
    }
  }
}

template <int D>
int launch_variant(const pfa::Launch& L) {
  Params p;
  p.q = static_cast<const uint16_t*>(L.q);
  p.k = static_cast<const uint16_t*>(L.k);
  p.v = static_cast<const uint16_t*>(L.v);
  p.key_mask = L.key_mask;
  p.o = static_cast<uint16_t*>(L.o);
  p.hq = L.hq;
  p.hkv = L.hkv;
  p.group = L.group;
  p.lq = L.lq;
  p.sk = L.sk;
  p.c = L.scale * kLog2e;
  p.causal = L.causal;
  p.causal_offset = L.causal_offset;
  p.cu_q = L.cu_q;
  p.cu_k = L.cu_k;
  p.total_q = L.total_q;
  p.total_k = L.total_k;
  p.window = L.window;
  p.no_skip = (L.flags & PFA_FLAG_NO_SKIP) ? 1 : 0;
  p.ws_part = nullptr;
  p.ws_cnt = nullptr;
  p.ring = L.ring;
  p.batch = L.batch;
  const bool split = pfa::split_applies(L);
  p.hpw = split ? 1 : pfa::heads_per_block(L);
  p.n_hset = L.group / p.hpw;
  p.n_qblk = (L.lq + kBM / p.hpw - 1) / (kBM / p.hpw);
  const long long n = (long long)L.batch * (L.hq / p.hpw) * p.n_qblk;
  p.n_wg = (int)n;
  p.xcd_remap = (n % kXcds) == 0 ? 1 : 0;
  void* args[] = {&p};
  const bool sc = L.softcap > 0.0f;
  p.sc_inv = sc ? L.scale / L.softcap : 0.0f;
  p.sc_cap_l2 = sc ? L.softcap * kLog2e : 0.0f;
  p.bias = L.bias;
  p.bias_sb = L.bias_sb;
  p.bias_sh = L.bias_sh;
  p.bias_sl = L.bias_sl;
  p.bias_nrec = L.bias_nrec;
  p.sinks = L.sinks;
  p.sel = L.sel;
  p.sel_bq = L.sel_bq;
  p.sel_bk = L.sel_bk;
  p.sel_sb = L.sel_sb;
  p.sel_sh = L.sel_sh;
  p.sel_sq = L.sel_sq;
  const void* fn;
  if (split) {
    // key split over a fixed set of workgroups (one per compute unit of an MI355X)
    p.ws_cnt = static_cast<unsigned*>(L.workspace);
    p.ws_part = reinterpret_cast<float*>(static_cast<char*>(L.workspace) + pfa::kSplitCounterBytes);
    if (L.key_mask)
      fn = sc ? reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeKeyMask | kModeSoftcap, true>)
              : reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeKeyMask, true>);
    else
      fn = sc ? reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeSoftcap, true>)
              : reinterpret_cast<const void*>(&pfa_prefill_kernel<D, 0, true>);
  } else if (L.bias) {
    fn = sc ? reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeBias | kModeSoftcap, false>)
            : reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeBias, false>);
  } else if (L.ring) {
    fn = sc ? reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeRing | kModeSoftcap, false>)
            : reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeRing, false>);
  } else if (L.key_mask) {
    fn = sc ? reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeKeyMask | kModeSoftcap, false>)
            : reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeKeyMask, false>);
  } else if (L.sel) {
    fn = sc ? reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeSel | kModeSoftcap, false>)
            : reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeSel, false>);
  } else {
    fn = sc ? reinterpret_cast<const void*>(&pfa_prefill_kernel<D, kModeSoftcap, false>)
            : reinterpret_cast<const void*>(&pfa_prefill_kernel<D, 0, false>);
  }
  const unsigned grid = split ? (unsigned)pfa::kSplitWorkgroups : (unsigned)n;
  hipError_t e = hipLaunchKernel(fn,
                                 dim3(grid), dim3(kThreads), args, 0,
                                 static_cast<hipStream_t>(L.stream));
  return e == hipSuccess ? PFA_OK : PFA_ERR_LAUNCH;
}

// Rotating-cache append: row i of K_new / V_new [B, Hkv, L, D] (position pos0 + i) goes to slot
// (pos0 + i) mod ring of K_ring / V_ring [B, Hkv, ring, D]. One thread per 16 bytes; blockIdx.y
// (striding by gridDim.y) is the (b, kv head) pair, x the 16-byte chunk within its L rows. The
// slot is p0 + i with p0 = pos0 mod ring, wrapped once (the ring holds at least L slots).
__global__ __launch_bounds__(256) void pfa_ring_append_kernel(const uint4* __restrict__ kn, const uint4* __restrict__ vn,
                                                              uint4* __restrict__ kr, uint4* __restrict__ vr,
                                                              long long n_bh, int L, int ring, int p0,
                                                              int cpr_log2) {
  const long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // chunk within one (b, hk)
  const long long per_bh = (long long)L << cpr_log2;
  if (j >= per_bh) return;
  const int i = (int)(j >> cpr_log2);
  const long long c = j & ((1 << cpr_log2) - 1);
  int slot = p0 + i;
  if (slot >= ring) slot -= ring;
  for (long long bh = blockIdx.y; bh < n_bh; bh += gridDim.y) {
    const long long src = bh * per_bh + j;
    const long long dst = ((bh * ring + slot) << cpr_log2) + c;
    kr[dst] = kn[src];
    vr[dst] = vn[src];
  }
}

}  // namespace

namespace pfa {

int launch_ring_append(const void* k_new, const void* v_new, void* k_ring, void* v_ring, int B, int Hkv, int L,
                       int D, int ring, int pos0, void* stream) {
  const int cpr_log2 = D == 128 ? 4 : 3;  // 16-byte chunks per row: D / 8
  const long long per_bh = (long long)L << cpr_log2;
  const long long n_bh = (long long)B * Hkv;
  const long long bx = (per_bh + 255) / 256;
  const unsigned by = (unsigned)(n_bh < 65535 ? n_bh : 65535);
  hipLaunchKernelGGL(pfa_ring_append_kernel, dim3((unsigned)bx, by), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), static_cast<uint4*>(k_ring),
                     static_cast<uint4*>(v_ring), n_bh, L, ring, pos0 % ring, cpr_log2);
  return hipGetLastError() == hipSuccess ? PFA_OK : PFA_ERR_LAUNCH;
}

int rows_per_block(int) { return kBM; }

// The band of a windowed call narrows with the block's height: 256 rows of one head see W + 255
// keys, 64 rows of each of four heads W + 63, for the same work (sliding window W = 1024 on 2048
// rows, 32 query heads on 8 KV heads: 44.0 -> 39.3 us per launch; the same through the rotating
// cache: 52.4 -> 47.5 us). Measured slower, and kept at one head per workgroup: packed batches of
// causal prompts (8 prompts of 1024-4096 rows: 396 -> 460 us without a window, 307 -> 324 us with
// W = 1024); dense causal and bidirectional calls gain nothing (within 0.3 %).
int heads_per_block(const Launch& p) {
  if (p.bias != nullptr || p.sel != nullptr || p.cu_q != nullptr || p.window <= 0) return 1;
  if (p.group % 4 == 0) return 4;
  if (p.group % 2 == 0) return 2;
  return 1;
}

long long split_part_bytes(int d) {
  const long long floats = d == 128 ? Slot<128>::kFloats : Slot<64>::kFloats;
  return 2LL * kSplitWorkgroups * floats * 4;
}

bool split_applies(const Launch& p) {
  const long long items = (long long)p.batch * p.hq * ((p.lq + kBM - 1) / kBM);  // one head per item
  return p.workspace != nullptr && p.cu_q == nullptr && p.ring == 0 && p.bias == nullptr && p.sel == nullptr &&
         items * 4 <= 3LL * kSplitWorkgroups;
}

long long grid_blocks(const Launch& p) {
  if (split_applies(p)) return kSplitWorkgroups;
  const long long hpw = heads_per_block(p);
  const long long bm = kBM / hpw;
  return (long long)p.batch * (p.hq / hpw) * ((p.lq + bm - 1) / bm);
}

int launch_prefill(const Launch& p) {
  if (p.d == 128) return launch_variant<128>(p);
  return launch_variant<64>(p);
}

}  // namespace pfa
