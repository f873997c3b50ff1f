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
//  * One workgroup = NW waves; each wave owns 32 query rows of one query head; the workgroup
//    covers 32*NW consecutive rows.
//  * Scores are computed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16. In the MFMA
//    result lane l holds key rows 8j+4h+i (h = l/32) of query column l%32, so every lane owns one
//    query row: row max and row sum are in-lane plus one exchange between the two lane halves.
//  * The output is accumulated transposed too, O^T = V^T . P^T. The S^T result registers
//    (exponentiated, rounded to BF16) are directly the B operand of that MFMA: the key order they
//    imply is matched by reading V^T from LDS with ds_read_b64_tr_b16, which hands each lane four
//    consecutive keys of one column. P never goes through LDS and V is never transposed by VALU.
//  * K and V tiles (64 keys x D) are loaded with coalesced 16-byte global loads into registers one
//    tile ahead, then written to a double-buffered LDS tile; one barrier per tile.
//  * Scores are scaled by scale*log2(e) inside the exp2 argument (one FMA per score).
//  * The tile range of a workgroup is bounded by the causal and window edges; with a key mask a
//    per-tile "any valid" bitmap (64 tiles per ballot) lets the loop jump over empty tiles; waves
//    whose own rows see nothing of a tile skip its arithmetic. Elementwise masks run only on
//    tiles that straddle an edge.
//  * Workgroups are ordered so that those sharing a KV head land on the same XCD (the hardware
//    deals workgroups to the 8 XCDs round-robin), heaviest causal blocks first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pfa.h"
#include "pfa_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kBN = 64;      // keys per tile
constexpr int kWaveRows = 32;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Geo {
  static constexpr int kStride = D + 8;   // K row pitch in LDS (bf16): 16-byte pad
  // V row pitch: 320 B (D=128) / 192 B (D=64). The four rows of one 16-lane transpose read then
  // start 64 B apart modulo 256 B, so the eight 32-byte pieces a half-wave reads hit distinct banks.
  static constexpr int vStride = D + 32;
  static constexpr int kTile = kBN * kStride;
  static constexpr int vTile = kBN * vStride;
  static constexpr int kChunksPerRow = D / 8;  // 16-byte chunks
  static constexpr int kChunks = kBN * kChunksPerRow;
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint8_t* key_mask;
  uint16_t* o;
  int hq, hkv, group, lq, sk;
  float c;  // scale * log2(e)
  int causal_offset, window;
  int no_skip;
  int n_qblk;
  int n_wg;
  int xcd_remap;
};

__device__ __forceinline__ float wave_max_halves(float x) {
  return fmaxf(x, __shfl_xor(x, 32));
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

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void pfa_prefill_kernel(Params p) {
  using G = Geo<D>;
  constexpr int NT = NW * 64;
  constexpr int BM = NW * kWaveRows;
  constexpr int CPT = G::kChunks / NT;  // 16-byte chunks per thread per tile, for K and for V
  static_assert(G::kChunks % NT == 0, "tile chunks must divide evenly");
  constexpr int KQ = D / 16;  // MFMA k-steps over the head dimension
  constexpr int DB = D / 32;  // 32-wide output blocks

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][G::kTile];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][G::vTile];
  __shared__ __attribute__((aligned(16))) uint8_t m_lds[2][kBN];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- workgroup -> (b, kv head, query block, head in group) ----
  long long item = blockIdx.x;
  if (p.xcd_remap) {
    const int per = p.n_wg / kXcds;
    item = (long long)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  }
  const int g = (int)(item % p.group);
  item /= p.group;
  const int qrank = (int)(item % p.n_qblk);
  item /= p.n_qblk;
  const int hk = (int)(item % p.hkv);
  const int b = (int)(item / p.hkv);
  const bool causal = p.causal_offset >= 0;
  const int qblk = causal ? (p.n_qblk - 1 - qrank) : qrank;
  const int h = hk * p.group + g;
  const int L = p.lq, S = p.sk;
  const long long off = p.causal_offset;
  const int W = p.window;
  const int q0 = qblk * BM;
  const int q1 = (q0 + BM) < L ? (q0 + BM) : L;

  const uint16_t* kg = p.k + ((long long)b * p.hkv + hk) * (long long)S * D;
  const uint16_t* vg = p.v + ((long long)b * p.hkv + hk) * (long long)S * D;
  const uint8_t* mrow = p.key_mask ? p.key_mask + (long long)b * S : nullptr;
  const bool kmask = mrow != nullptr;

  // ---- key-tile range of the workgroup ----
  const int n_tiles = (S + kBN - 1) / kBN;
  int kt_lo = 0, kt_hi = n_tiles;
  if (!p.no_skip && causal) {
    long long hi_key = (long long)q1 + off;  // exclusive
    if (hi_key > S) hi_key = S;
    kt_hi = (int)((hi_key + kBN - 1) / kBN);
    if (W > 0) {
      long long lo_key = (long long)q0 + off - W + 1;
      if (lo_key < 0) lo_key = 0;
      long long t = lo_key / kBN;
      kt_lo = (int)(t < n_tiles ? t : n_tiles);
    }
  }

  // ---- per-wave row state ----
  const int qw0 = q0 + wave * kWaveRows;
  const bool wave_active = qw0 < L;
  const int ii_last = wave_active ? ((L - 1 - qw0) < 31 ? (L - 1 - qw0) : 31) : 0;

  bf16x8 qreg[KQ];
  {
    const int row = qw0 + l32;
    if (row < L) {
      const uint16_t* qrow = p.q + (((long long)b * p.hq + h) * L + row) * (long long)D;
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
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float c = p.c;

  // ---- key-mask bitmap (per wave, 64 tiles per chunk) ----
  int mchunk = -1;
  uint64_t m_any = 0, m_all = 0;
  auto ensure_chunk = [&](int kt) {
    const int ch = kt >> 6;
    if (ch != mchunk) {
      key_mask_chunk(mrow, S, ch << 6, lane, &m_any, &m_all);
      mchunk = ch;
    }
  };
  // Next tile >= k (and < kt_hi) to visit, or kt_hi. With a key mask and skipping on, tiles
  // without a valid key are passed over; *all_valid tells whether every key of the returned tile
  // is valid (no elementwise key masking needed).
  auto next_tile = [&](int k, bool* all_valid) -> int {
    *all_valid = true;
    if (!kmask) return k < kt_hi ? k : kt_hi;
    while (k < kt_hi) {
      ensure_chunk(k);
      if (p.no_skip) {
        *all_valid = (m_all >> (k & 63)) & 1ull;
        return k;
      }
      const uint64_t bits = m_any >> (k & 63);
      if (bits) {
        const int t = k + __builtin_ctzll(bits);
        if (t >= kt_hi) return kt_hi;
        *all_valid = (m_all >> (t & 63)) & 1ull;
        return t;
      }
      k = (k | 63) + 1;
    }
    return kt_hi;
  };

  // ---- tile staging ----
  uint4 kreg[CPT], vreg[CPT];
  uint8_t mreg = 0;
  auto load_tile = [&](int kt) {
    const long long key0 = (long long)kt * kBN;
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int ch = tid + r * NT;
      const int row = ch / G::kChunksPerRow;
      const int col = (ch % G::kChunksPerRow) * 8;
      const long long key = key0 + row;
      if (key < S) {
        const long long o = key * D + col;
        kreg[r] = *reinterpret_cast<const uint4*>(kg + o);
        vreg[r] = *reinterpret_cast<const uint4*>(vg + o);
      } else {
        kreg[r] = make_uint4(0, 0, 0, 0);
        vreg[r] = make_uint4(0, 0, 0, 0);
      }
    }
    if (kmask && tid < kBN) mreg = (key0 + tid < S) ? mrow[key0 + tid] : (uint8_t)0;
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int ch = tid + r * NT;
      const int row = ch / G::kChunksPerRow;
      const int col = (ch % G::kChunksPerRow) * 8;
      *reinterpret_cast<uint4*>(&k_lds[buf][row * G::kStride + col]) = kreg[r];
      *reinterpret_cast<uint4*>(&v_lds[buf][row * G::vStride + col]) = vreg[r];
    }
    if (kmask && tid < kBN) m_lds[buf][tid] = mreg;
  };

  // ---- one tile of arithmetic for this wave ----
  auto compute_tile = [&](int kt, int buf, bool tile_all_valid) {
    const long long key0 = (long long)kt * kBN;
    // relative mask thresholds: row i = qw0 + ii, key j = key0 + jj
    long long lim_tail_l = (long long)S - key0;
    const int lim_tail = lim_tail_l < kBN ? (int)lim_tail_l : kBN;
    int dc = 1 << 20, dw = -(1 << 20);
    if (causal) {
      long long t = off + qw0 - key0;  // visible iff jj - ii <= dc
      dc = t > 256 ? 256 : (t < -256 ? -256 : (int)t);
      if (W > 0) {
        long long u = off - W + 1 + qw0 - key0;  // visible iff jj - ii >= dw
        dw = u > 256 ? 256 : (u < -256 ? -256 : (int)u);
      }
    }
    // Does the tile hold any visible cell for this wave's real rows?
    if (!p.no_skip) {
      int lo = dw > -ii_last ? dw : -ii_last;
      int hi = dc < lim_tail - 1 ? dc : lim_tail - 1;
      if (lo > hi) return;
    }
    const bool need_mask = lim_tail < kBN || (causal && (kBN - 1) > dc) ||
                           (causal && W > 0 && -31 < dw) || !tile_all_valid;

    // S^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.0f;
      const uint16_t* kb_ptr = &k_lds[buf][(kb * 32 + l32) * G::kStride + 8 * hh];
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb_ptr + 16 * kk);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], s[kb], 0, 0, 0);
      }
    }

    if (need_mask) {
      const int ii = l32;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t mb = 0xFFFFFFFFu;
          if (kmask)
            mb = *reinterpret_cast<const uint32_t*>(&m_lds[buf][kb * 32 + 8 * j + 4 * hh]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jj = kb * 32 + 8 * j + 4 * hh + i;
            const int rel = jj - ii;
            bool vis = jj < lim_tail && rel <= dc && rel >= dw && ((mb >> (8 * i)) & 0xFFu) != 0u;
            if (!vis) s[kb][4 * j + i] = -INFINITY;
          }
        }
      }
    }

    // online softmax (per lane: one query row, 32 of the tile's 64 keys)
    float mx = s[0][0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[0][v]);
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[1][v]);
    mx = wave_max_halves(mx);
    const float m_new = fmaxf(m_run, mx);
    const float ms_new = (m_new == -INFINITY) ? 0.0f : m_new * c;
    const float ms_old = (m_run == -INFINITY) ? -INFINITY : m_run * c;
    const float alpha = __builtin_amdgcn_exp2f(ms_old - ms_new);
    m_run = m_new;

    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][v], c, -ms_new));
        s[kb][v] = e;
        lsum += e;
      }
    l_run = alpha * l_run + lsum;
    if (!__all(alpha == 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
    }

    // O^T += V^T . P^T
    const int g16 = lane >> 4;
    const int loc = lane & 15;
    const int r4 = loc >> 2;
    const int cc = loc & 3;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        bf16x8 pb;
#pragma unroll
        for (int t = 0; t < 8; ++t) pb[t] = (__bf16)s[kb][8 * c2 + t];
        const int key_row = kb * 32 + 16 * c2 + 4 * (g16 >> 1) + r4;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = 32 * db + 16 * (g16 & 1) + 4 * cc;
          lds_u16* base = (lds_u16*)(&v_lds[buf][0]);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(base + key_row * G::vStride + col));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(base + (key_row + 8) * G::vStride + col));
          // Join the two reads as one integer vector and reinterpret it whole: assembling the
          // bf16 operand element by element from 16-bit integers is mis-lowered by the compiler.
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[db], 0, 0, 0);
        }
      }
    }
  };

  // ---- main loop over key tiles ----
  bool all_cur = true;
  int kt = next_tile(kt_lo, &all_cur);
  if (kt < kt_hi) {
    load_tile(kt);
    store_tile(0);
  }
  __syncthreads();
  int buf = 0;
  while (kt < kt_hi) {
    bool all_nxt = true;
    const int nk = next_tile(kt + 1, &all_nxt);
    if (nk < kt_hi) load_tile(nk);
    if (wave_active) compute_tile(kt, buf, all_cur);
    if (nk < kt_hi) store_tile(buf ^ 1);
    __syncthreads();
    kt = nk;
    all_cur = all_nxt;
    buf ^= 1;
  }

  // ---- epilogue: O = acc / l, rows without visible keys -> 0 ----
  if (!wave_active) return;
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  const int row = qw0 + l32;
  if (row >= L) return;
  uint16_t* orow = p.o + (((long long)b * p.hq + h) * L + row) * (long long)D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = (__bf16)(acc[db][4 * j + i] * inv);
      *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * j + 4 * hh) = ov;
    }
  }
}

template <int D, int NW>
int launch_variant(const pfa::Launch& L) {
  constexpr int BM = NW * kWaveRows;
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
  p.causal_offset = L.causal_offset;
  p.window = L.window;
  p.no_skip = (L.flags & PFA_FLAG_NO_SKIP) ? 1 : 0;
  p.n_qblk = (L.lq + BM - 1) / BM;
  const long long n = (long long)L.batch * L.hq * p.n_qblk;
  p.n_wg = (int)n;
  p.xcd_remap = (n % kXcds) == 0 ? 1 : 0;
  void* args[] = {&p};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&pfa_prefill_kernel<D, NW>),
                                 dim3((unsigned)n), dim3(NW * 64), args, 0,
                                 static_cast<hipStream_t>(L.stream));
  return e == hipSuccess ? PFA_OK : PFA_ERR_LAUNCH;
}

constexpr int kWaves = 8;

}  // namespace

namespace pfa {

int rows_per_block(int) { return kWaves * kWaveRows; }

long long grid_blocks(const Launch& p) {
  const long long bm = rows_per_block(p.d);
  return (long long)p.batch * p.hq * ((p.lq + bm - 1) / bm);
}

int launch_prefill(const Launch& p) {
  if (p.d == 128) return launch_variant<128, kWaves>(p);
  return launch_variant<64, kWaves>(p);
}

}  // namespace pfa
