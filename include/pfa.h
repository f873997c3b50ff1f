/*
 * pfa.h -- C ABI of the gfx950 (MI355X) grouped-query flash prefill attention library.
 *
 * One operation: masked scaled-dot-product attention for a prefill chunk of L new query rows
 * against S keys that include a cached prefix, with grouped-query heads.
 *
 *   O[b,h,i,:] = sum_j softmax_j( scale * Q[b,h,i,:] . K[b,hk,j,:] + A[b,i,j] ) * V[b,hk,j,:]
 *   hk = floor(h / (Hq / Hkv))
 *
 * Sources for the definition (page titles and sections):
 *  - tiny-llm, Week 2 Day 5 "Tiled Dense Prefill Attention", Task 1: the layout contract
 *    Q [B,Hq,L,D], K/V [B,Hkv,S,D], output [B,Hq,L,D]; Hq % Hkv == 0; query head h reads KV head
 *    floor(h / (Hq/Hkv)) without copying K/V into Hq heads; FP32 running max / sum / accumulator
 *    merged tile by tile (the merge equations); BF16 only after the final FP32 normalisation.
 *  - same page, Task 2: causality aligned to the end of the cached prefix (row i sees keys through
 *    S - L + i); a row with no visible key returns finite zeros; tiles with no valid score skipped.
 *  - tinygrad "symbolic llm with prefill": the prefill mask is the lower-right triangle
 *    full(-inf).triu(start_pos + 1), not the upper-left one of is_causal.
 *  - TensorFold PR "Spark2.5's and Llama's prompt attention from one source", "What changes": the
 *    sliding-window mask term col < row - WINDOW + 1 and the window's first key block.
 *  - brotensor flash_attention.h: flash_attention_windowed_forward (query at absolute position
 *    pos sees keys [max(0, pos - window + 1), pos]; window <= 0 unbounded),
 *    flash_attention_gqa_forward (causal or bidirectional, length-Lk key mask), and
 *    flash_attention_decode_masked (fully masked key tiles skipped without touching K/V, result
 *    bit-identical to the unmasked call).
 *  - mlx-lm PR "Skip fully masked key tiles in Flint sliding-window prefill": skipping must keep
 *    the kernel's key-tile grid, so the result is bit-identical to visiting every tile; the
 *    window is an explicit argument, never inferred from a mask.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device, contiguous, row-major,
 *    owned by the caller. The library never allocates, frees or copies device memory and keeps no
 *    global mutable state; calls are thread-safe.
 *  - Arguments are validated on the host before anything is enqueued; on any error nothing is
 *    launched and O is left untouched.
 *  - Success means the kernel was enqueued on `stream` (asynchronous; no host synchronisation).
 */
#ifndef PFA_H
#define PFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PFA_VERSION 10800 /* 1.8.0 */

/* causal_offset < 0 selects bidirectional attention (no causal term). */
#define PFA_NO_CAUSAL (-1)

/* Largest L and S accepted: rows and keys are indexed with 32-bit integers in the kernel. */
#define PFA_MAX_LEN 1073741824 /* 2^30 */

/* Visit every key tile of the grid and mask elementwise instead of skipping fully masked tiles.
 * Exists for the bit-identity check: the result must equal the default (skipping) call bit for
 * bit. */
#define PFA_FLAG_NO_SKIP 1u

/* Largest L accepted by the short-query (decode) entry point. */
#define PFA_DECODE_MAX_L 64

/* Status codes. Codes 0-8 are the base set in their base order; 9-12 were added for the flags,
 * the scale check, the decode workspace and the rotating cache. Validation runs in the order
 * NULL, SIZE, GQA, HEAD_DIM, MASK_ARGS, SCALE, ALIGN, ALIAS, FLAGS (the first failing check is
 * returned); LAUNCH can only follow a call that passed all of them. */
enum pfa_status {
  PFA_OK = 0,
  PFA_ERR_NULL = 1,      /* Q, K, V, O, a varlen prefix-sum buffer or the decode workspace NULL */
  PFA_ERR_SIZE = 2,      /* a size < 1, L or S > PFA_MAX_LEN, a size product / grid too big, or */
                         /* one (b, KV head) ring of the rotating cache >= 2^31 bytes           */
  PFA_ERR_GQA = 3,       /* Hq is not a multiple of Hkv                                         */
  PFA_ERR_HEAD_DIM = 4,  /* D is not 64 or 128                                                  */
  PFA_ERR_MASK_ARGS = 5, /* window > 0 without the causal term; an unsupported mask combination */
  PFA_ERR_ALIGN = 6,     /* Q, K, V or O not 16-byte aligned (prefix sums: not 4-byte aligned)  */
  PFA_ERR_ALIAS = 7,     /* O (or the decode workspace) overlaps another buffer of the call     */
  PFA_ERR_LAUNCH = 8,    /* the HIP launch failed (e.g. no gfx950 device is current)            */
  PFA_ERR_FLAGS = 9,     /* unknown bit in flags                                                */
  PFA_ERR_SCALE = 10,    /* scale not finite or not > 0; softcap not finite or < 0              */
  PFA_ERR_WORKSPACE = 11, /* workspace smaller than pfa_{decode,prefill}_workspace_bytes()    */
  PFA_ERR_RING = 12       /* ring cache smaller than 64 slots or than the keys the chunk sees   */
};

/*
 * prefill_attn_gqa -- grouped-query flash prefill attention, BF16 in / BF16 out, FP32 softmax.
 *
 *   Q            bf16 [B, Hq,  L, D]   queries of the new chunk
 *   K, V         bf16 [B, Hkv, S, D]   keys / values, S includes the cached prefix
 *   B            batch size (>= 1)
 *   Hq, Hkv      query heads and KV heads (>= 1, Hq % Hkv == 0; Hq == Hkv is plain MHA)
 *   L, S         query rows and keys (>= 1; any combination, L > S allowed)
 *   D            head dimension, 64 or 128
 *   scale        score scale, finite and > 0 (usually 1/sqrt(D)); applied to Q.K^T in FP32
 *   causal_offset  >= 0: row i sees keys j <= i + causal_offset (S - L for a prefill chunk);
 *                  < 0 (PFA_NO_CAUSAL): no causal term (bidirectional)
 *   window       > 0: row i also needs j >= i + causal_offset - window + 1 (window keys including
 *                its own position); requires causal_offset >= 0. <= 0: no window term
 *   key_mask     NULL, or uint8 [B, S]: nonzero = key valid, 0 = key dropped for every row of that
 *                batch element. No alignment requirement
 *   O            bf16 [B, Hq, L, D], fully overwritten; rows with no visible key are set to 0
 *   stream       hipStream_t to enqueue on; NULL = the default stream
 *
 * Keys are always limited to j < S. Fully masked key tiles are skipped before their K/V tile is
 * loaded; the result is bit-identical to prefill_attn_gqa_ex(..., PFA_FLAG_NO_SKIP).
 * Returns a pfa_status code.
 */
int prefill_attn_gqa(const void* Q, const void* K, const void* V,
                     int B, int Hq, int Hkv, int L, int S, int D,
                     float scale, int causal_offset, int window,
                     const uint8_t* key_mask, void* O, void* stream);

/* As prefill_attn_gqa, with a flags word (0 or PFA_FLAG_NO_SKIP).
 * prefill_attn_gqa(...) == prefill_attn_gqa_ex(..., 0). */
int prefill_attn_gqa_ex(const void* Q, const void* K, const void* V,
                        int B, int Hq, int Hkv, int L, int S, int D,
                        float scale, int causal_offset, int window,
                        const uint8_t* key_mask, void* O, void* stream,
                        unsigned flags);

/*
 * Options of prefill_attn_gqa_opt / prefill_attn_gqa_decode_opt. A zero-filled struct (or a NULL
 * pointer) is the plain call.
 *
 *   flags    0 or PFA_FLAG_NO_SKIP (prefill only; the decode path rejects it with PFA_ERR_FLAGS)
 *   softcap  > 0: logit soft-capping (brotensor flash_attention_decode, attn_softcap, the Gemma-2
 *            extension): after the scale and before the masks and the softmax, every score s
 *            becomes softcap * tanh(s / softcap). 0 = off. Must be finite and >= 0
 *            (PFA_ERR_SCALE otherwise).
 *   bias     NULL, or an additive FP32 bias (tiny-llm Week 2 Day 5 Task 2: a broadcastable
 *            additive array mask, applied before the online-softmax update): element
 *            bias[b * bias_stride_b + h * bias_stride_h + i * bias_stride_l + j] is added to the
 *            (soft-capped) scaled score of query head h, row i, key j; keys are contiguous and a
 *            zero stride broadcasts (e.g. strides 0, 0, S for one [L, S] mask). Values are finite
 *            or -inf. Prefill entry point only, not with a key mask (PFA_ERR_MASK_ARGS); the
 *            pointer and the strides must be multiples of 16 bytes / 4 elements (PFA_ERR_ALIGN);
 *            one (b, h) block, (L - 1) * bias_stride_l + S elements, must stay under 2^29
 *            elements (PFA_ERR_SIZE); it must not overlap O (PFA_ERR_ALIAS).
 *   sinks    NULL, or DEVICE fp32 [Hq]: one attention-sink logit per query head (mlx-lm
 *            sliding-window prefill PR, "Correctness", lists attention sinks among the cases; the
 *            pages give no formula, and the reading taken is the usual one): every row's softmax
 *            gets one more term, e^sinks[h], in its normaliser, with no value, i.e.
 *            O[i] = sum_j e^(s_ij) V_j / (sum_j e^(s_ij) + e^sinks[h]) over the visible keys j,
 *            s_ij the final (scaled, soft-capped, biased) score. The sink is used as given (not
 *            scaled). Values finite or -inf (-inf = no sink for that head). A row without a
 *            visible key still gives zeros. Prefill (dense, packed, ring) and decode entry points.
 *   block_sel  NULL, or a DEVICE uint8 block bitmap (TensorFold PR "What changes": MiniMax-M3's
 *            prompt attention adds a block bitmap, SEL; the pages give no layout, and the reading
 *            taken is: with query blocks of block_q rows and key blocks of block_k keys, key j is
 *            visible to row i of (b, h) only if
 *              block_sel[b * sel_stride_b + h * sel_stride_h + (i / block_q) * sel_stride_q + j / block_k]
 *            is nonzero, on top of every other mask term). Key blocks whose byte is zero are
 *            skipped whole (never fetched) unless PFA_FLAG_NO_SKIP is set. block_q must be a
 *            positive multiple of 32 and block_k of 64 (PFA_ERR_SIZE); strides >= 0 (0
 *            broadcasts); the bitmap must not overlap O (PFA_ERR_ALIAS). Prefill entry point
 *            only, and not with a key mask or an additive bias (PFA_ERR_MASK_ARGS).
 */
typedef struct pfa_options {
  unsigned flags;
  float softcap;
  const float* bias;
  int64_t bias_stride_b, bias_stride_h, bias_stride_l;
  const float* sinks;
  const uint8_t* block_sel;
  int32_t block_q, block_k;
  int64_t sel_stride_b, sel_stride_h, sel_stride_q;
} pfa_options;

/* prefill_attn_gqa_ex with options (see pfa_options). */
int prefill_attn_gqa_opt(const void* Q, const void* K, const void* V,
                         int B, int Hq, int Hkv, int L, int S, int D,
                         float scale, int causal_offset, int window,
                         const uint8_t* key_mask, void* O, void* stream,
                         const pfa_options* opts);

/*
 * prefill_attn_gqa_ws -- prefill_attn_gqa_opt with a caller workspace that lets the call split the
 * key range of a query block over several workgroups. prefill_attn_gqa runs one workgroup per query
 * block (256 rows of one query head and batch element), so a call with fewer blocks than the
 * chip's 256 compute units leaves units idle for its whole length (8 query heads, 2048 rows and 32K
 * cached keys: 64 blocks). Here a fixed grid of 256 workgroups takes equal shares of the (query
 * block, key tile) space; a block split between workgroups leaves one FP32 partial (running max,
 * sum, accumulator) per part in the workspace, and the part that finishes last merges them in key
 * order with the merge equations (tiny-llm Week 2 Day 5, Task 1) and writes O. The merge order is
 * fixed, so results are run-to-run deterministic, and skipping is bit-identical to
 * PFA_FLAG_NO_SKIP; they may differ in the last bits from prefill_attn_gqa (other summation
 * boundaries). Both meet the same tolerance.
 *
 * The split is taken only where it pays, when B * Hq * ceil(L / 256) <= 192 (three quarters of
 * the grid). With more blocks, and with an additive bias or a block bitmap, the call runs exactly as
 * prefill_attn_gqa_opt (bit-identical results) and leaves the workspace untouched: one workgroup
 * per block is then faster, since those workgroups start together at the first key tile and walk
 * the keys in step (each K / V tile of a KV head is fetched once per L2), while the shares of a
 * split start at scattered key tiles.
 *
 * Same arguments as prefill_attn_gqa_opt, plus a DEVICE workspace of at least
 * pfa_prefill_workspace_bytes(B, Hq, Hkv, L, S, D) bytes, 16-byte aligned, not overlapping any
 * other buffer of the call, ZERO-FILLED before its first use (it holds one counter per query block,
 * and every call leaves the counters zero again). Calls that share a workspace must be ordered on
 * one stream. Returns a pfa_status code (PFA_ERR_WORKSPACE if the workspace is too small, checked
 * whether or not the split is taken).
 */
int prefill_attn_gqa_ws(const void* Q, const void* K, const void* V,
                        int B, int Hq, int Hkv, int L, int S, int D,
                        float scale, int causal_offset, int window,
                        const uint8_t* key_mask, void* O,
                        void* workspace, int64_t workspace_bytes, void* stream,
                        const pfa_options* opts);

/* Workspace bytes prefill_attn_gqa_ws needs for this shape (a pure function of the arguments),
 * or -1 if the shape is invalid for it: 1 KiB of counters (one per query block) followed by about
 * 69 MB at D = 128 (35 MB at D = 64) of FP32 partial slots when the call can take the split (at
 * most 192 query blocks), else 16 (the workspace is then not touched). The counters come first at
 * a fixed place, so one zero-filled workspace serves calls of any shape and head size it is large
 * enough for. */
int64_t pfa_prefill_workspace_bytes(int B, int Hq, int Hkv, int L, int S, int D);

/*
 * prefill_attn_gqa_varlen -- the same attention over a packed batch of variable-length sequences
 * (brotensor flash_attention.h, flash_attention_varlen_forward: all sequences live back to back
 * in one packed tensor, sequence boundaries come from INT32 prefix-sum buffers of n_seq + 1
 * entries, and no query attends to a key of another sequence).
 *
 *   Q, O          bf16 [total_q, Hq, D]   token-major: the rows of all sequences back to back,
 *                                        the Hq heads of one row contiguous
 *   K, V          bf16 [total_k, Hkv, D]  same packing for the keys (grouped-query heads as in
 *                                        prefill_attn_gqa: query head h reads KV head h / (Hq/Hkv))
 *   cu_seqlens_q  DEVICE int32 [n_seq + 1]: sequence b owns query rows
 *                 [cu_seqlens_q[b], cu_seqlens_q[b+1])
 *   cu_seqlens_k  DEVICE int32 [n_seq + 1]: sequence b owns keys [cu_seqlens_k[b], cu_seqlens_k[b+1])
 *                 Both must start at 0, be non-decreasing and end at total_q / total_k. They are
 *                 read only by the kernel (the host never dereferences them); every bound is
 *                 clamped into [0, total], so malformed sums cannot cause an out-of-bounds access
 *                 (the result is then unspecified).
 *   n_seq         number of sequences (>= 1); a sequence may have no rows or no keys
 *   max_seqlen_q  largest per-sequence query length (>= 1, <= PFA_MAX_LEN); the grid covers this
 *                 many rows per sequence, rows past it are not computed
 *   total_q, total_k  packed row counts (>= 1)
 *   Hq, Hkv, D, scale  as in prefill_attn_gqa
 *   causal        nonzero: local row i of sequence b sees local keys j <= i + (Lk_b - Lq_b), the
 *                 lower-right alignment of a chunk that follows its cached keys; for Lq_b == Lk_b
 *                 this is the page's rule j <= i. A row with no visible key gets zeros.
 *   window        > 0: also j >= i + (Lk_b - Lq_b) - window + 1; requires causal
 *   O             fully overwritten for well-formed prefix sums
 *   stream        hipStream_t to enqueue on; NULL = the default stream
 *
 * Each sequence is computed exactly as prefill_attn_gqa computes it alone (same key-tile grid
 * anchored at the sequence's first key), so the result for a sequence is bit-identical to the
 * dense call on that sequence. Returns a pfa_status code.
 */
int prefill_attn_gqa_varlen(const void* Q, const void* K, const void* V,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int n_seq, int max_seqlen_q, int total_q, int total_k,
                            int Hq, int Hkv, int D, float scale, int causal, int window,
                            void* O, void* stream);

/* prefill_attn_gqa_varlen with options (see pfa_options): flags, softcap and sinks apply as in
 * prefill_attn_gqa_opt (sinks indexed by query head); bias and block_sel are per dense row and are
 * rejected here (PFA_ERR_MASK_ARGS). */
int prefill_attn_gqa_varlen_opt(const void* Q, const void* K, const void* V,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int n_seq, int max_seqlen_q, int total_q, int total_k,
                                int Hq, int Hkv, int D, float scale, int causal, int window,
                                void* O, void* stream, const pfa_options* opts);

/*
 * prefill_attn_gqa_ring -- causal (optionally sliding-window) prefill of a chunk against a rotating
 * KV cache, with the chunk's own keys appended to the cache by the same call.
 *
 * TensorFold PR "Spark2.5's and Llama's prompt attention from one source", "What changes": the
 * sliding layer reads each key and value row from its ring slot (RING = WINDOW + 64 there); the
 * brotensor kv_cache_append comment: the new rows are copied into the cache at the current length.
 *
 *   Q             bf16 [B, Hq, L, D]    the chunk's queries, at positions pos0 .. pos0 + L - 1
 *   K_new, V_new  bf16 [B, Hkv, L, D]   the chunk's keys / values (positions pos0 .. pos0 + L - 1)
 *   K_ring, V_ring bf16 [B, Hkv, ring, D]  the rotating cache: key position j lives in slot
 *                 j mod ring. On entry it must hold every position the chunk's rows see before
 *                 pos0; on return the chunk's rows have been written to their slots (the cache
 *                 then holds positions up to pos0 + L - 1). Written by the call.
 *   pos0          position of the chunk's first row (>= 0)
 *   ring          slots of the cache; >= 64 and >= min(window - 1 + L, pos0 + L) (with a window)
 *                 or >= pos0 + L (without one), so that appending the chunk overwrites no key a
 *                 row still sees (PFA_ERR_RING otherwise); ring * D * 2 < 2^31, i.e. one
 *                 (b, KV head) ring under 2 GiB (PFA_ERR_SIZE otherwise: slot offsets are 32-bit)
 *   window        > 0: row at position p sees keys [max(0, p - window + 1), p]; <= 0: all of [0, p]
 *   O             bf16 [B, Hq, L, D], fully overwritten
 *
 * The append runs first and the attention then reads every key through the slot map (no gather
 * copy); both are enqueued on `stream` in that order. The result is bit-identical to
 * prefill_attn_gqa on the logical keys (history followed by K_new) with causal_offset = pos0.
 * Returns a pfa_status code (PFA_ERR_RING if the ring is too small; on error nothing is enqueued
 * and neither O nor the cache is touched).
 */
int prefill_attn_gqa_ring(const void* Q, const void* K_new, const void* V_new,
                          void* K_ring, void* V_ring,
                          int B, int Hq, int Hkv, int L, int pos0, int ring, int D,
                          float scale, int window, void* O, void* stream);

/* prefill_attn_gqa_ring with options (see pfa_options): flags, softcap and sinks apply as in
 * prefill_attn_gqa_opt; bias and block_sel are rejected (PFA_ERR_MASK_ARGS); the sink logits must
 * not overlap O or the rings (PFA_ERR_ALIAS). On any error nothing is enqueued. */
int prefill_attn_gqa_ring_opt(const void* Q, const void* K_new, const void* V_new,
                              void* K_ring, void* V_ring,
                              int B, int Hq, int Hkv, int L, int pos0, int ring, int D,
                              float scale, int window, void* O, void* stream,
                              const pfa_options* opts);

/*
 * prefill_attn_gqa_decode -- the operation of prefill_attn_gqa for a short query chunk (one-token
 * decode up to PFA_DECODE_MAX_L rows) against a long cache. tiny-llm Week 2 Day 5 Task 2 routes
 * one-token decode and L <= 8 to a separate path; brotensor flash_attention_decode runs decode
 * against a partially filled cache with query position valid_len - L_q + i, which is
 * causal_offset = S - L here.
 *
 * Same arguments, layouts, masks and result as prefill_attn_gqa (1 <= L <= PFA_DECODE_MAX_L),
 * plus a caller-owned DEVICE workspace of at least pfa_decode_workspace_bytes(B,Hq,Hkv,L,S,D)
 * bytes, 16-byte aligned, not overlapping any other buffer of the call. The keys are split into
 * ranges processed in parallel; each range leaves a partial (running max, sum, accumulator) per
 * query row in the workspace, and a second kernel on the same stream merges the partials in a
 * fixed order with the merge equations (tiny-llm Task 1), so the result is deterministic (run to
 * run bit-identical) but not bit-identical to prefill_attn_gqa (another summation order). The
 * workspace holds no state between calls; calls that share a workspace must be ordered (same
 * stream). Returns a pfa_status code (PFA_ERR_WORKSPACE if the workspace is too small).
 */
int prefill_attn_gqa_decode(const void* Q, const void* K, const void* V,
                            int B, int Hq, int Hkv, int L, int S, int D,
                            float scale, int causal_offset, int window,
                            const uint8_t* key_mask, void* O,
                            void* workspace, int64_t workspace_bytes, void* stream);

/* prefill_attn_gqa_decode with options (see pfa_options; flags must be 0). */
int prefill_attn_gqa_decode_opt(const void* Q, const void* K, const void* V,
                                int B, int Hq, int Hkv, int L, int S, int D,
                                float scale, int causal_offset, int window,
                                const uint8_t* key_mask, void* O,
                                void* workspace, int64_t workspace_bytes, void* stream,
                                const pfa_options* opts);

/* Workspace bytes prefill_attn_gqa_decode needs for this shape (a pure function of the
 * arguments), or -1 if the shape is invalid for it. */
int64_t pfa_decode_workspace_bytes(int B, int Hq, int Hkv, int L, int S, int D);

/* Size of the library's own decode scratch array (64 MiB), the most that
 * prefill_attn_gqa_decode_noalloc can use. */
#define PFA_DECODE_SCRATCH_BYTES 67108864

/*
 * prefill_attn_gqa_decode_noalloc -- prefill_attn_gqa_decode_opt for callers that cannot allocate
 * device memory or hand in a workspace (code under HIP graph capture, tight serving loops, runtimes
 * that forbid allocation): the same arguments without the workspace, the same kernels and the same
 * result bit for bit, with the partials kept in a device array that the library owns instead.
 *
 * The array holds PFA_DECODE_SCRATCH_BYTES; a shape whose pfa_decode_workspace_bytes() exceeds it is
 * rejected with PFA_ERR_WORKSPACE (use prefill_attn_gqa_decode with a workspace then). Each GPU the
 * library runs on holds one copy of the array from the module's load until the process ends; the
 * call itself allocates nothing (no hipMalloc, no allocating library routine). Every call on a GPU
 * shares that GPU's copy, so calls that overlap in time on one GPU (different streams or host
 * threads without ordering) race on it and give undefined results; calls ordered on one stream are
 * safe. No state is carried from one call to the next (every partial is rewritten before it is
 * read). Returns a pfa_status code; PFA_ERR_LAUNCH also if the array's device address cannot be
 * obtained on the current device.
 */
int prefill_attn_gqa_decode_noalloc(const void* Q, const void* K, const void* V,
                                    int B, int Hq, int Hkv, int L, int S, int D,
                                    float scale, int causal_offset, int window,
                                    const uint8_t* key_mask, void* O, void* stream,
                                    const pfa_options* opts);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* pfa_status_str(int status);

/* PFA_VERSION of the built library. */
int pfa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PFA_H */
