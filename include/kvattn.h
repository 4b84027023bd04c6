/*
 * kvattn.h — C ABI of libkvattn.so: softmax attention of a few query tokens,
 * or of a prefill chunk, over a long paged KV cache whose keys are stored as
 * Q8_0 and values as Q4_0 in 128-token pages, with log-sum-exp (LSE) merging
 * of partial results and KVMem-style top-k block selection.
 *
 * Sources (the method is described, not specified, by these pages):
 *  [KVMEM]  lcz.me topic 1972, KVMem reproduction report on one RX 7900 XTX:
 *           section "長上下文實測結果（主矩陣）/ 測試口徑" (the server flags
 *           --kvmem-budget 32768, --kvmem-gen-reserve 16384,
 *           --kvmem-block-tokens 128, --kv-dtype q8_0), section
 *           "Recall 測試" (256 of 485 blocks kept at budget 32768) and section
 *           "Full-KV 對照" (attention runs only over the ~48K-token working set).
 *  [STREAM] alphalab.site, "Adaptive KV Streaming 是什麼？AMD 16GB 長 Context
 *           六步驗收", step ④ (flags -ctk q8_0 -ctv q4_0, -ub 512; the stream
 *           path needs flash attention with Q8_0 K / Q4_0 V).
 *  [RDNA4]  wqu.guru, "Qwen 27B (IQ4_XS, Q8/Q4 KV) at full 262k context on a
 *           16GB RX 9070 XT: 80+ t/s decode with Adaptive KV Streaming",
 *           bullets "Online Log-Sum-Exp prefill & pipelined prefetch" and
 *           "Stream-optimized speculative decoding" (paged decode attention
 *           extended to verify batches).
 *  [VULKAN] lcz.me topic 1398, "單張 RX 7900 XTX 24GB 把 Qwen3.8-27B 推到
 *           124 t/s —— Vulkan 路線實測報告": section "模型結構" (16
 *           full-attention layers x 4 KV heads x 256 = 16384 elements per token
 *           for K and for V), section "坑 2" (q4_0 K+V = 18 KiB per token),
 *           section "坑 3" (only the legacy block types are KV types) and the
 *           closing remark that q8_0 K carries 8.5 bits per element.
 * None of the pages defines the bit layout, scale rule or rounding of Q8_0 and
 * Q4_0, the block-scoring function, or a page layout; the definitions below
 * are this library's, and the CPU oracle implements the same definitions
 * independently.
 *
 * Conventions shared by every entry point
 *  - Every pointer argument except `geom`, `workspace_bytes` and the status
 *    out-parameters is a DEVICE pointer on the current HIP device. The caller
 *    owns every buffer; the library never allocates, frees or synchronises.
 *    Work is only enqueued on `stream` (a hipStream_t; NULL = null stream).
 *  - Float arrays must be 16-byte aligned; pools 256-byte aligned.
 *  - All validation happens on the host before anything is enqueued; on any
 *    error nothing is enqueued and no output is touched.
 *  - Status codes: KVATTN_OK; KVATTN_E_INVALID (bad pointer, size, range or
 *    alignment); KVATTN_E_UNSUPPORTED (head_dim != 256, page_tokens != 128,
 *    too many query rows, or a device that is not gfx950); KVATTN_E_WORKSPACE
 *    (workspace smaller than required); KVATTN_E_DEVICE (a HIP runtime error
 *    while querying the device or launching). No exceptions cross the ABI and
 *    nothing is printed. There is no CPU fallback.
 *  - Workspace protocol: when `workspace` is NULL the function stores the
 *    required byte count in *workspace_bytes, returns KVATTN_OK and enqueues
 *    nothing. Otherwise *workspace_bytes is the size of `workspace`.
 *  - The first KVATTN_WORKSPACE_SYNC_BYTES bytes of every workspace are
 *    counters through which a launch's workgroups coordinate. They must be
 *    zero when a workspace is first used (allocate it zeroed), and every
 *    call leaves them zero, so one workspace serves every entry point and
 *    any number of calls; the partials and scores follow them. Bytes 0..3
 *    are an error word: bit 0 is set by a prefill launch in which a
 *    wavefront's bounded wait on the others of its workgroup gave up (never
 *    expected; that call's output is unspecified). Concurrent calls must not
 *    share a workspace.
 *  - Calls that overlap on one stream are ordered by the stream; concurrent
 *    calls on different streams must not share outputs or workspace.
 *
 * Pool byte layout (part of the ABI; page quantisation is bit-exact)
 *  A layer's pool is two arrays of records, k_pool and v_pool, indexed by
 *  (physical page P, KV head h): record (P * n_kv_heads + h). Token position
 *  `pos` lives in logical page pos / 128, slot t = pos % 128; the page table
 *  maps logical page -> physical page.
 *  K record, KVATTN_K_RECORD_BYTES = 34816:
 *   [0, 32768)      int8 Q8_0 code of (slot t, dim n) at byte t*256 + n.
 *   [32768, 34816)  IEEE binary16 scale of (slot t, 32-dim block b = n/32) at
 *                   byte 32768 + 2*(t*8 + b), little endian.
 *  V record, KVATTN_V_RECORD_BYTES = 18432:
 *   [0, 16384)      4096 little-endian 32-bit words of 4-bit Q4_0 codes. For
 *                   c in [0,4), q in [0,4), g in [0,4), d in [0,16),
 *                   e in [0,4), word w = (((c*4 + q)*4 + g)*16 + d)*4 + e
 *                   holds the codes of dim n = 16*(4*q + e) + d for the eight
 *                   slots t(c,g,j) = 32*c + 16*(j/4) + 4*g + (j%4), j = 0..7;
 *                   slot j's code sits at bit 4*(j/2) + 16*(j%2).
 *   [16384, 18432)  binary16 scale of (slot t(c,g,j), block b) at byte
 *                   16384 + 2*(((c*8 + b)*4 + g)*8 + j).
 *  The V word order places, for each group of 32 slots, the eight slots that
 *  one lane of a 16x16x32 matrix-core tile consumes in one 32-bit word, so a
 *  lane turns a word into four f16 pairs with one shift and one mask each.
 *  Q8_0 V record (v_type KVATTN_V_Q8_0), KVATTN_V8_RECORD_BYTES = 34816:
 *   [0, 32768)      int8 codes. For c in [0,4), q in [0,8), g in [0,4),
 *                   r in [0,16), half in [0,2), j in [0,8), byte
 *                   c*8192 + q*1024 + (16*g + r)*16 + 8*half + j holds the
 *                   code of dim n = 32*q + 16*half + r for slot t(c,g,j)
 *                   (t as above): each 16 bytes are what one lane of a
 *                   16x16x32 tile reads for two 16-dim tiles of one block.
 *   [32768, 34816)  binary16 scale of (slot t(c,g,j), block b) at byte
 *                   32768 + 2*(((c*8 + b)*4 + g)*8 + j).
 *  Q4_0 K record (k_type KVATTN_K_Q4_0), KVATTN_K4_RECORD_BYTES = 18432:
 *   [0, 16384)      4-bit codes, slot t's row of 32 little-endian 32-bit
 *                   words at byte t*128; word w holds dims 8w..8w+7, dim
 *                   8w + k at bit 4*(k/2) + 16*(k%2) (the V word nibble
 *                   order), so a lane turns a word into the f16 values of
 *                   eight consecutive dims with one shift and mask per pair.
 *   [16384, 18432)  binary16 scale of (slot t, block b) at 16384 + 2*(t*8 + b).
 *  Q5_1 K record (k_type KVATTN_K_Q5_1), KVATTN_K5_RECORD_BYTES = 24576:
 *   [0, 16384)      the low 4 bits of each 5-bit code, as in a Q4_0 K record.
 *   [16384, 20480)  fifth bits: byte 16384 + t*32 + w holds those of dims
 *                   8w..8w+7 of slot t, dim 8w + 2p at bit p and dim
 *                   8w + 2p + 1 at bit 4 + p (p = 0..3).
 *   [20480, 22528)  binary16 scale d of (slot t, block b) at 20480 + 2*(t*8 + b).
 *   [22528, 24576)  binary16 minimum m of (slot t, block b) at 22528 + 2*(t*8 + b).
 *
 * Quantisation (per token, per KV head, per 32-dim block x[0..31]; RN32 and
 * RN16 are IEEE round-to-nearest-even to binary32 / binary16, rint rounds
 * half to even):
 *  Q8_0 (keys): amax = max|x_i|; d = RN16(RN32(amax / 127)). If d == 0 every
 *   code is 0 and the stored scale is +0. Otherwise inv = RN32(1 / d) and
 *   code_i = clamp(rint(RN32(x_i * inv)), -127, 127). Dequantised: d * code.
 *   34 bytes per 32 elements = 8.5 bits per element ([VULKAN] closing remark).
 *  Q8_0 values (v_type KVATTN_V_Q8_0) follow the key rule above.
 *  Q4_0 keys (k_type KVATTN_K_Q4_0) follow the Q4_0 value rule below.
 *  Q5_1 (keys, k_type KVATTN_K_Q5_1): mn = min x_i, mx = max x_i;
 *   d = RN16(RN32((mx - mn) / 31)), m = RN16(mn). If d == 0 every code is 0
 *   and the stored scale is +0. Otherwise inv = RN32(1 / d) and
 *   code_i = clamp(rint(RN32(RN32(x_i - m) * inv)), 0, 31). Dequantised:
 *   d * code + m. 24 bytes per 32 elements (6 bits per element).
 *  Q4_0 (values): j* = lowest index with |x_j*| = amax; m = x_j* (signed);
 *   d = RN16(RN32(-m / 8)). If amax == 0 or d == 0, the stored scale is +0
 *   and every code is 8. Otherwise inv = RN32(1 / d) and
 *   code_i = clamp(rint(RN32(x_i * inv)), -8, 7) + 8. Dequantised:
 *   d * (code - 8). 18 bytes per 32 elements; K (Q8_0) + V (Q4_0) is 26 KiB
 *   per token at 16 layers x 4 KV heads x 256 ([VULKAN] "模型結構", "坑 2").
 *  Block summary (KVMem scoring input): for a full logical page p and head h,
 *   summary[h][p][n] = RN32((sum over t = 0..127, ascending, in binary64, of
 *   dequantised K[t][n]) / 128), i.e. the mean dequantised key of the block.
 */
#ifndef KVATTN_H
#define KVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvattn_status;
#define KVATTN_OK 0
#define KVATTN_E_INVALID 1
#define KVATTN_E_UNSUPPORTED 2
#define KVATTN_E_WORKSPACE 3
#define KVATTN_E_DEVICE 4

#define KVATTN_HEAD_DIM 256
#define KVATTN_PAGE_TOKENS 128
#define KVATTN_K_RECORD_BYTES 34816
#define KVATTN_V_RECORD_BYTES 18432
#define KVATTN_V8_RECORD_BYTES 34816 /* Q8_0 values (v_type KVATTN_V_Q8_0) */
#define KVATTN_V_Q4_0 0 /* value cache type: Q4_0 (the default) */
#define KVATTN_V_Q8_0 1 /* value cache type: Q8_0 (the q8_0/q8_0 pair) */
#define KVATTN_K4_RECORD_BYTES 18432 /* Q4_0 keys (k_type KVATTN_K_Q4_0) */
#define KVATTN_K_Q8_0 0 /* key cache type: Q8_0 (the default) */
#define KVATTN_K_Q4_0 1 /* key cache type: Q4_0 (the q4_0/q4_0 pair) */
#define KVATTN_K5_RECORD_BYTES 24576 /* Q5_1 keys (k_type KVATTN_K_Q5_1) */
#define KVATTN_K_Q5_1 2 /* key cache type: Q5_1 (the q5_1/q4_0 pair) */
#define KVATTN_MAX_QUERY_ROWS 32 /* n_q_tok * gqa per KV head in decode */
#define KVATTN_WORKSPACE_SYNC_BYTES 2048 /* counters at the start of a workspace */
#define KVATTN_MAX_APPEND_TOKENS 32 /* n_new of kvattn_append_decode */
#define KVATTN_NOALLOC_SCRATCH_BYTES 16777216 /* kvattn_append_decode_noalloc */

/* Geometry of one layer's pool. head_dim must be 256 and page_tokens 128
 * (the pages' shape: [VULKAN] "模型結構"; [KVMEM] --kvmem-block-tokens 128).
 * Query head hq uses KV head hq / gqa (grouped-query attention). v_type picks
 * the value type: KVATTN_V_Q4_0 (the [STREAM] -ctk q8_0 -ctv q4_0 pair) or
 * KVATTN_V_Q8_0 (KVMem's q8_0/q8_0, [KVMEM] 測試口徑 --kv-dtype q8_0), and
 * k_type the key type: KVATTN_K_Q8_0, KVATTN_K_Q4_0 (the q4_0/q4_0 pair,
 * [VULKAN] 坑 2) or KVATTN_K_Q5_1 (the q5_1/q4_0 pair of [VULKAN] 坑 3's
 * allowed list); each sets its record size. */
typedef struct kvattn_geom {
  int32_t n_kv_heads;   /* >= 1 */
  int32_t gqa;          /* query heads per KV head, >= 1 */
  int32_t head_dim;     /* 256 */
  int32_t page_tokens;  /* 128 */
  int32_t n_phys_pages; /* physical pages in k_pool / v_pool, >= 1;
                          n_phys_pages * n_kv_heads <= INT32_MAX */
  int32_t v_type;       /* KVATTN_V_Q4_0 or KVATTN_V_Q8_0 */
  int32_t k_type;       /* KVATTN_K_Q8_0, KVATTN_K_Q4_0 or KVATTN_K_Q5_1 */
} kvattn_geom;

/* Human-readable name of a status code (static storage, never NULL). */
const char *kvattn_status_string(kvattn_status s);

/* Number of blocks kvattn_select_blocks writes per KV head:
 * min(k_top, n_blocks - min(n_recent, n_blocks)) + min(n_recent, n_blocks);
 * -1 if an argument is negative or n_blocks < 1. Host-only, no device use. */
int32_t kvattn_select_count(int32_t n_blocks, int32_t n_recent, int32_t k_top);

/* a1 — quantise tokens into pages, and summarise completed pages.
 * Writes the Q8_0 keys and Q4_0 values of positions pos0 .. pos0+n_tok-1 into
 * their slots (layout and rounding above); every other byte of the pools is
 * left as it was ([STREAM] step ④: -ctk q8_0 -ctv q4_0; [KVMEM] 128-token
 * blocks). When k_summary is not NULL, the summary of every logical page p
 * that this call writes into and that is full afterwards
 * ((p+1)*128 <= pos0+n_tok; positions are assumed written in order) is
 * recomputed from the pool; other summaries are untouched.
 *  k, v        fp32 [n_tok][n_kv_heads][256], read only.
 *  page_table  int32 [n_logical_pages], values in [0, n_phys_pages).
 *              Requires pos0 >= 0, n_tok >= 1 and
 *              pos0 + n_tok <= n_logical_pages * 128.
 *  k_pool      n_phys_pages * n_kv_heads * the key record size (34816 bytes
 *              for Q8_0 keys, 18432 for Q4_0, 24576 for Q5_1).
 *  v_pool      n_phys_pages * n_kv_heads * the value record size (18432 bytes
 *              for Q4_0 values, 34816 for Q8_0).
 *  k_summary   fp32 [n_kv_heads][n_logical_pages][256] or NULL.
 * Logical pages that map to the same physical page race. A page-table entry
 * outside [0, n_phys_pages) makes the kernel skip that page's writes. */
kvattn_status kvattn_quantize_pages(const kvattn_geom *geom, const float *k,
                                    const float *v, int64_t pos0, int32_t n_tok,
                                    const int32_t *page_table,
                                    int32_t n_logical_pages, uint8_t *k_pool,
                                    uint8_t *v_pool, float *k_summary,
                                    void *stream);

/* a2 — KVMem block scoring and top-k selection ([KVMEM] 測試口徑 and
 * "Recall 測試": keep budget/128 history blocks plus a reserved recent window
 * on the GPU; attention then runs over that working set only). Per KV head h:
 *  q_sel[n] = RN32(sum over g = 0..gqa-1, ascending, in binary64, of
 *             q[h*gqa + g][n]);
 *  score[b] = sum over n = 0..255, ascending, in binary64, of
 *             q_sel[n] * summary[h][b][n], for candidates b in [0, NB - R),
 *  with R = min(n_recent, n_blocks) and NB = n_blocks. Candidates are ranked
 *  by (score descending, b ascending; -0 equals +0) and the first
 *  min(k_top, NB - R) are kept. out_blocks[h][...] receives the kept blocks
 *  together with the recent blocks NB-R .. NB-1, in ascending order;
 *  kvattn_select_count() gives the count per head.
 *  q           fp32 [n_kv_heads*gqa][256], one query token.
 *  k_summary   fp32 [n_kv_heads][n_logical_pages][256]; candidate blocks must
 *              be full pages whose summary has been written.
 *  n_blocks    1 <= n_blocks <= n_logical_pages. n_recent, k_top >= 0.
 *  out_blocks  int32 [n_kv_heads][kvattn_select_count(...)].
 *  workspace   2048 + 8 * n_kv_heads * (NB - R) bytes, rounded up; query
 *              with workspace == NULL. When 0 < k_top < NB - R the call
 *              leaves the scores there: binary64 [n_kv_heads][NB - R] from
 *              byte 2048. */
kvattn_status kvattn_select_blocks(const kvattn_geom *geom, const float *q,
                                   const float *k_summary,
                                   int32_t n_logical_pages, int32_t n_blocks,
                                   int32_t n_recent, int32_t k_top,
                                   int32_t *out_blocks, void *workspace,
                                   size_t *workspace_bytes, void *stream);

/* a3/a5 — decode and verify attention over the paged cache, split over pages
 * with an LSE merge ([RDNA4] paged decode attention extended to verify
 * batches; [STREAM] step ④). Query token t (0 <= t < n_q_tok) sits at
 * position p_t = kv_len - n_q_tok + t and sees keys at positions <= p_t.
 * For query head hq = h*gqa + g and its key set J:
 *  s_j = scale * dot(q[t][hq], Khat_j), m = max s_j, l = sum exp(s_j - m),
 *  out[t][hq] = sum exp(s_j - m) * Vhat_j / l, lse[t][hq] = m + ln l (natural
 *  log); an empty key set gives out = 0 and lse = -inf.
 *  Dense (blocks == NULL): J = positions 0 .. kv_len-1 through logical pages
 *   0 .. ceil(kv_len/128)-1. Sparse: J = the tokens (< kv_len) of the logical
 *   pages listed in blocks[h][0 .. n_blk-1] (the output of
 *   kvattn_select_blocks); entries should be distinct — a repeated entry is
 *   attended as often as it appears; an entry outside [0, n_logical_pages),
 *   or mapping to a physical page outside [0, n_phys_pages), contributes
 *   nothing.
 *  q        fp32 [n_q_tok][n_kv_heads*gqa][256]; n_q_tok >= 1 and
 *           n_q_tok*gqa <= 32 (else KVATTN_E_UNSUPPORTED).
 *  kv_len   n_q_tok <= kv_len <= n_logical_pages*128.
 *  out      fp32 [n_q_tok][n_kv_heads*gqa][256]; lse fp32 [n_q_tok][..].
 *  n_splits work splits per KV head, 0 = chosen by the library.
 *  workspace holds the split partials; query its size with workspace==NULL
 *           (the size depends on every argument above, including n_splits).
 *           The result is kvattn_decode_partials + kvattn_merge_lse of the
 *           same splits, bit for bit.
 * Arithmetic: f16 matrix-core products with fp32 accumulation; the result is
 * within 2e-3 (max-abs) of exact attention over the dequantised pages for
 * keys and values with |x| <= 65504 (the binary16 range the dequantised keys
 * and the scaled probabilities are formed in). */
kvattn_status kvattn_decode(const kvattn_geom *geom, const float *q,
                            int32_t n_q_tok, const uint8_t *k_pool,
                            const uint8_t *v_pool, const int32_t *page_table,
                            int32_t n_logical_pages, const int32_t *blocks,
                            int32_t n_blk, int64_t kv_len, float scale,
                            float *out, float *lse, int32_t n_splits,
                            void *workspace, size_t *workspace_bytes,
                            void *stream);

/* a1 + a3/a5 in one launch — append, then decode: the step of a decode or
 * verify pass that first writes the new tokens' keys and values into the
 * cache ([STREAM] step ④ quantised KV cache; [RDNA4] verify batches through
 * paged decode) and then attends over it. Equivalent to
 *   kvattn_quantize_pages(geom, k_new, v_new, kv_len - n_new, n_new,
 *                         page_table, n_logical_pages, k_pool, v_pool,
 *                         k_summary, stream)
 * followed by kvattn_decode with the other arguments: the pool bytes,
 * summaries, out and lse are identical bit for bit. The decode kernel itself
 * quantises the tokens: the wavefront that streams the tile holding them
 * writes them before it reads that tile, so no separate quantisation launch
 * is made. When k_summary is not NULL, the summary of the page the append
 * completes (the new positions complete at most one page) is written by the
 * same launch: the workgroup that streams that page sums it once its new
 * tokens are written, so in the sparse form the page must be listed (as the
 * rule below already requires).
 *  k_new, v_new  fp32 [n_new][n_kv_heads][256], finite; the keys and values
 *                of positions kv_len - n_new .. kv_len - 1.
 *  n_new         1 <= n_new <= min(KVATTN_MAX_APPEND_TOKENS, kv_len).
 *  k_pool, v_pool  written (the new tokens' slots) and read.
 *  Sparse form: every logical page that holds a new token must appear in
 *                blocks[h] of every KV head h (kvattn_select_blocks' recent
 *                window does); the tokens of a page that is not listed are
 *                not written. If a list repeats such a page, each listing
 *                writes the same bytes and a repeat may read them while they
 *                are written (before or after the new tokens land: its share
 *                of the result is then unspecified); list it once.
 * Other arguments, the workspace protocol and errors as kvattn_decode
 * (KVATTN_E_INVALID also for bad k_new, v_new or n_new). */
kvattn_status kvattn_append_decode(const kvattn_geom *geom, const float *k_new,
                                   const float *v_new, int32_t n_new,
                                   const float *q, int32_t n_q_tok,
                                   uint8_t *k_pool, uint8_t *v_pool,
                                   const int32_t *page_table,
                                   int32_t n_logical_pages,
                                   const int32_t *blocks, int32_t n_blk,
                                   int64_t kv_len, float scale,
                                   float *k_summary, float *out, float *lse,
                                   int32_t n_splits, void *workspace,
                                   size_t *workspace_bytes, void *stream);

/* kvattn_append_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, result and errors as kvattn_append_decode
 * without the workspace: the split-K partials go to a static array of
 * KVATTN_NOALLOC_SCRATCH_BYTES in the library, one per GPU (reserved when the
 * library's code is loaded on that GPU, kept until the process ends), looked
 * up on the first call on each device. The call allocates nothing, and its
 * out, lse, pool bytes and summaries equal kvattn_append_decode's bit for
 * bit. The partials take splits * n_q_tok * n_kv_heads * gqa * 1028 bytes
 * (each of the two arrays rounded up to 256): 6.3 MB for 4 KV heads x 24
 * rows per KV head at the default 64 splits. A call that needs more returns
 * KVATTN_E_WORKSPACE and enqueues nothing. Every call on one GPU uses that
 * GPU's one array: calls on one stream are ordered, but calls that overlap
 * on one GPU (other streams, other threads) race and their results are
 * unspecified. */
kvattn_status kvattn_append_decode_noalloc(const kvattn_geom *geom, const float *k_new,
                                           const float *v_new, int32_t n_new,
                                           const float *q, int32_t n_q_tok,
                                           uint8_t *k_pool, uint8_t *v_pool,
                                           const int32_t *page_table,
                                           int32_t n_logical_pages,
                                           const int32_t *blocks, int32_t n_blk,
                                           int64_t kv_len, float scale,
                                           float *k_summary, float *out, float *lse,
                                           int32_t n_splits, void *stream);

/* a3 alone — the split-K partials of kvattn_decode, without the merge, for
 * callers that combine them with partials computed elsewhere (other pages,
 * another device) through kvattn_merge_lse ([RDNA4] "Online Log-Sum-Exp":
 * partial results over streamed pages combined by online LSE). Arguments as
 * kvattn_decode, except:
 *  n_splits  >= 1. Split s covers units [n_units*s/n_splits,
 *            n_units*(s+1)/n_splits) of the unit list, where the units are
 *            logical pages 0 .. ceil(kv_len/128)-1 (dense) or blocks[h][..]
 *            (sparse), n_units their count.
 *  o_part    fp32 [n_splits][n_q_tok*n_kv_heads*gqa][256], 16-byte aligned;
 *            lse_part fp32 [n_splits][n_q_tok*n_kv_heads*gqa]. For split s
 *            and row r over the split's key set J_s: lse_part = ln sum
 *            exp(s_j), o_part = sum exp(s_j - lse_part) Vhat_j; an empty J_s
 *            gives o_part = 0, lse_part = -inf. kvattn_merge_lse of all
 *            splits is kvattn_decode's result.
 * No workspace; nothing but o_part and lse_part is written. */
kvattn_status kvattn_decode_partials(const kvattn_geom *geom, const float *q,
                                     int32_t n_q_tok, const uint8_t *k_pool,
                                     const uint8_t *v_pool,
                                     const int32_t *page_table,
                                     int32_t n_logical_pages,
                                     const int32_t *blocks, int32_t n_blk,
                                     int64_t kv_len, float scale,
                                     int32_t n_splits, float *o_part,
                                     float *lse_part, void *stream);

/* a1 + a3 — kvattn_append_decode's append with kvattn_decode_partials'
 * partials, without the merge: the new tokens (and the summary of a page they
 * complete) are written exactly as kvattn_append_decode writes them, and
 * o_part / lse_part receive the n_splits partials of the key set after the
 * append, exactly as kvattn_decode_partials writes them, so
 * kvattn_merge_lse of them is kvattn_append_decode's out and lse bit for bit
 * at the same n_splits (1 <= n_splits <= the unit count, which
 * kvattn_append_decode never exceeds). The partials of the key set that holds the new
 * tokens can then meet the partials of other key sets (pages streamed from
 * the host, another device's pages) in a single merge ([RDNA4] "Online
 * Log-Sum-Exp": partial results over streamed pages combined by LSE).
 * Arguments as kvattn_append_decode, with n_splits, o_part and lse_part as
 * kvattn_decode_partials; no workspace. */
kvattn_status kvattn_append_decode_partials(const kvattn_geom *geom, const float *k_new,
                                            const float *v_new, int32_t n_new,
                                            const float *q, int32_t n_q_tok,
                                            uint8_t *k_pool, uint8_t *v_pool,
                                            const int32_t *page_table,
                                            int32_t n_logical_pages,
                                            const int32_t *blocks, int32_t n_blk,
                                            int64_t kv_len, float scale,
                                            float *k_summary, int32_t n_splits,
                                            float *o_part, float *lse_part,
                                            void *stream);

/* The split count kvattn_decode chooses (n_splits = 0) for n_units units on
 * the current device; 0 if geom is invalid or n_units < 1. */
int32_t kvattn_decode_splits(const kvattn_geom *geom, int32_t n_units);


/* a6 — chunked prefill attention ([RDNA4] "Online Log-Sum-Exp prefill":
 * chunked prefill across pages with online LSE accumulation; [STREAM] step ④
 * -ub 512). Query token t (0 <= t < chunk) sits at position pos0 + t and sees
 * keys at positions <= pos0 + t, read through logical pages
 * 0 .. ceil((pos0+chunk)/128)-1; the chunk's own keys and values must already
 * be in the pool (kvattn_quantize_pages). Output definition as kvattn_decode.
 *  q        fp32 [chunk][n_kv_heads*gqa][256]; chunk >= 1; pos0 >= 0;
 *           pos0 + chunk <= n_logical_pages*128.
 *  out      fp32 [chunk][n_kv_heads*gqa][256]; lse fp32 [chunk][..].
 *  n_groups page groups per (KV head, query tile) merged by LSE; 0 = chosen
 *           by the library.
 *  workspace holds the group partials after the counter area; query its
 *           size with workspace == NULL. Bit 0 of its error word is set if a
 *           wavefront's bounded wait on the others of its workgroup gave up
 *           (never expected; the output is then unspecified).
 * Arithmetic: K/V tiles dequantised to f16 in LDS, f16 matrix-core products,
 * fp32 accumulation; within 1e-2 (max-abs) of exact attention. q and the
 * pool's scales must be finite: the kernel is compiled assuming no NaN
 * operands, so a NaN input gives unspecified (not necessarily NaN) output. */
kvattn_status kvattn_prefill_chunk(const kvattn_geom *geom, const float *q,
                                   int32_t chunk, const uint8_t *k_pool,
                                   const uint8_t *v_pool,
                                   const int32_t *page_table,
                                   int32_t n_logical_pages, int64_t pos0,
                                   float scale, float *out, float *lse,
                                   int32_t n_groups, void *workspace,
                                   size_t *workspace_bytes, void *stream);

/* a6 alone — the per-group partials of kvattn_prefill_chunk, without the
 * merge. Arguments as kvattn_prefill_chunk, except:
 *  n_groups  >= 1. Group gi covers logical pages [n_pages*gi/n_groups,
 *            n_pages*(gi+1)/n_groups), n_pages = ceil((pos0+chunk)/128).
 *  o_part    fp32 [n_groups][chunk*n_kv_heads*gqa][256], 16-byte aligned;
 *            lse_part fp32 [n_groups][chunk*n_kv_heads*gqa]; per group and
 *            row as kvattn_decode_partials (row order as out).
 * No workspace; nothing but o_part and lse_part is written. */
kvattn_status kvattn_prefill_partials(const kvattn_geom *geom, const float *q,
                                      int32_t chunk, const uint8_t *k_pool,
                                      const uint8_t *v_pool,
                                      const int32_t *page_table,
                                      int32_t n_logical_pages, int64_t pos0,
                                      float scale, int32_t n_groups,
                                      float *o_part, float *lse_part,
                                      void *stream);

/* a6 over a page range — the partials of kvattn_prefill_partials restricted
 * to the keys of logical pages [page_begin, page_end): the groups split that
 * range (group gi covers [b + (e-b)*gi/n_groups, b + (e-b)*(gi+1)/n_groups),
 * b = page_begin, e = page_end), and no key outside it is read, so the pool
 * and page table need to hold only those pages (entries outside the range are
 * never looked up). Partials of ranges that tile [0, ceil((pos0+chunk)/128))
 * merged by kvattn_merge_lse give the chunk's prefill ([RDNA4] "Online
 * Log-Sum-Exp prefill & pipelined prefetch": partial results over streamed
 * page ranges combine by LSE; the Adaptive KV Streaming guide's bounded
 * prefill working set, step ④ --kv-resident-mib 450). A group whose keys are
 * all masked for a row writes o = 0 and lse = -inf for it.
 *  0 <= page_begin < page_end <= ceil((pos0+chunk)/128); n_groups >= 1;
 *  other arguments and errors as kvattn_prefill_partials. */
kvattn_status kvattn_prefill_range_partials(const kvattn_geom *geom, const float *q,
                                            int32_t chunk, const uint8_t *k_pool,
                                            const uint8_t *v_pool,
                                            const int32_t *page_table,
                                            int32_t n_logical_pages, int64_t pos0,
                                            float scale, int32_t page_begin,
                                            int32_t page_end, int32_t n_groups,
                                            float *o_part, float *lse_part,
                                            void *stream);

/* The group count kvattn_prefill_chunk chooses (n_groups = 0) on the current
 * device; 0 if geom is invalid, chunk < 1 or pos0 < 0. */
int32_t kvattn_prefill_groups(const kvattn_geom *geom, int32_t chunk,
                              int64_t pos0);

/* a4 — merge partial attention results by log-sum-exp ([RDNA4] "Online
 * Log-Sum-Exp prefill"). For each row r:
 *  M = max_s lse_parts[s][r]; L = M + ln sum_s exp(lse_parts[s][r] - M);
 *  out[r] = sum_s exp(lse_parts[s][r] - L) * o_parts[s][r]; lse[r] = L.
 *  A part with lse = -inf contributes nothing; if every part is -inf the row
 *  is out = 0, lse = -inf. fp32 throughout; sums are taken in a fixed order,
 *  so results are deterministic.
 *  o_parts fp32 [n_parts][rows][head_dim]; lse_parts fp32 [n_parts][rows];
 *  out fp32 [rows][head_dim]; lse fp32 [rows]. n_parts >= 1, rows >= 1,
 *  head_dim >= 1. out must not alias o_parts. */
kvattn_status kvattn_merge_lse(int32_t n_parts, int64_t rows, int32_t head_dim,
                               const float *o_parts, const float *lse_parts,
                               float *out, float *lse, void *stream);

/* Hadamard rotation of 256-dim rows, in place ([VULKAN] section
 * "沒踩到的坑：注意力旋轉": the attention rotation raises the precision of a
 * quantised KV cache and stays on with q8_0 / q5_1 / q4_0 caches). Each row
 * x[r][0..255] becomes H_256 x / 16, H the Sylvester-ordered Hadamard matrix
 * (orthonormal after the 1/16), computed in binary32 by the fast
 * Walsh-Hadamard butterflies with half-widths 1, 2, 4, ..., 128 in that
 * order (pair (i, i + h), bit h of i clear, becomes x[i] + x[i+h],
 * x[i] - x[i+h], each rounded), then the exact multiplication by 1/16; the
 * result is reproducible bit for bit. Rotating the key rows before
 * kvattn_quantize_pages / kvattn_append_decode and the query rows before
 * attention or selection leaves q . k unchanged in exact arithmetic and
 * spreads a key's outlier channels over all dims, which lowers the Q8_0
 * error where a few channels dominate. Values may be rotated as well before
 * quantisation: H / 16 is symmetric and orthonormal, so rotating the
 * attention output rows once more returns the attention over the unrotated
 * values (this lowers the Q4_0 error in the same way).
 *  x       fp32 [n_rows][256], device, 16-byte aligned; n_rows >= 0
 *          (0: nothing is done). */
kvattn_status kvattn_rotate_rows(float *x, int64_t n_rows, void *stream);

/* KVMem host tier — the GPU pulls the blocks a selection kept from a pool
 * that may live in pinned host memory ([KVMEM] 測試口徑 and "Recall 測試":
 * history blocks in host RAM, budget/128 of them brought to the GPU next to a
 * reserved recent window). For every KV head h and rank i < n_sel, copies
 * the key and value records of logical page blocks[h][i] (physical page
 * page_table[blocks[h][i]]) into record (i * n_kv_heads + h) of the dst pools
 * and sets dst_blocks[h][i] = i; an entry outside [0, n_logical_pages), or
 * mapping to a physical page outside [0, n_phys_pages), copies nothing and
 * sets dst_blocks[h][i] = -1. A kernel does the copy, reading the block list
 * on the device, so a selection (kvattn_select_blocks, whose first k_top
 * entries per head are the kept history) feeds it with no host round trip.
 * kvattn_decode_partials over the dst pools with page_table = identity on
 * [0, n_sel) (and -1 beyond), blocks = dst_blocks attends exactly the
 * gathered blocks.
 *  geom        geometry of the src pools (n_phys_pages, n_kv_heads).
 *  src_k_pool, src_v_pool  device memory or pinned host memory
 *              (hipHostMalloc); the kernel reads host memory over the host
 *              link through its device mapping. Other host memory is
 *              rejected (E_INVALID).
 *  page_table  DEVICE int32 [n_logical_pages].
 *  blocks      DEVICE int32 [n_kv_heads][n_blk]; the first n_sel entries of
 *              each row are gathered; 0 <= n_sel <= n_blk.
 *  dst_k_pool, dst_v_pool  DEVICE pools of n_sel * n_kv_heads records.
 *  dst_blocks  DEVICE int32 [n_kv_heads][n_sel].
 * Pools 256-byte aligned. */
kvattn_status kvattn_gather_blocks(const kvattn_geom *geom,
                                   const uint8_t *src_k_pool,
                                   const uint8_t *src_v_pool,
                                   const int32_t *page_table,
                                   int32_t n_logical_pages,
                                   const int32_t *blocks, int32_t n_blk,
                                   int32_t n_sel, uint8_t *dst_k_pool,
                                   uint8_t *dst_v_pool, int32_t *dst_blocks,
                                   void *stream);

/* a7 — page prefetch for a host-resident pool ([RDNA4] "Online Log-Sum-Exp
 * prefill & pipelined prefetch": pages stream in ahead of the layer that
 * needs them; [STREAM] the Adaptive KV Streaming path keeps history in host
 * memory). Copies the records of physical pages pages[0 .. n_pages-1] (all
 * KV heads of each page) from the src pools to the same physical slots of the
 * dst pools, asynchronously on `stream` (hipMemcpyAsync; runs of consecutive
 * page indices go as one copy per pool). The typical use keeps the src pools
 * in pinned host memory (hipHostMalloc) and the dst pools on the device, and
 * issues layer L+1's pages on a copy stream while layer L computes; the
 * caller orders the streams with events.
 *  src_k_pool, src_v_pool, dst_k_pool, dst_v_pool: pools of geom's size
 *    (host or device memory, any combination hipMemcpyAsync accepts;
 *    pinned host memory for the copy to be asynchronous).
 *  pages  HOST array of n_pages physical page indices in [0, n_phys_pages);
 *         read before the call returns. n_pages >= 0 (0: nothing is done).
 * Errors: E_INVALID for a null pool, n_pages < 0, pages NULL with
 * n_pages > 0, or an index out of range (checked before any copy is
 * enqueued); E_DEVICE if a copy cannot be enqueued (copies enqueued before it
 * stay enqueued). */
kvattn_status kvattn_prefetch_pages(const kvattn_geom *geom,
                                    const uint8_t *src_k_pool,
                                    const uint8_t *src_v_pool,
                                    uint8_t *dst_k_pool, uint8_t *dst_v_pool,
                                    const int32_t *pages, int32_t n_pages,
                                    void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KVATTN_H */
