/*
 * kvc.h - single-token decode attention over a KV cache, for AMD MI355X
 * (gfx950).  C ABI: plain pointers and sizes only.
 *
 * What the calls compute (sources are the pages' titles and sections):
 *
 *  - "KV cache" guide (this.guide), "A cache you keep because attention
 *    looks backwards": at each generation step the new token's query attends
 *    to the key and value of every earlier position and of itself; keys and
 *    values are cached because they never change once produced.
 *  - Same guide, "Two tensors per layer": per layer and sequence the cache is
 *    a key tensor and a value tensor, each [n_kv, L, d_h].  Here a batch is
 *    stored as [B, n_kv, L_max, d_h] (a contiguous reservation at the maximum
 *    length, as in the guide's "The allocator, not the algorithm") with a
 *    per-sequence length seq_lens[b].
 *  - Same guide, "Fewer KV heads": grouped-query attention; n_h query heads
 *    in n_kv contiguous groups of G = n_h / n_kv, query head i reading KV
 *    head i / G.  G = 1 is multi-head attention, n_kv = 1 multi-query.
 *  - Same guide, "Caching a compressed latent" and the memory footnote: a
 *    latent cache row is a 512-wide latent c plus a 64-wide shared rotary
 *    key; with the key up-projection folded into the query, scores are taken
 *    directly against the cached row and the output is the weighted sum of
 *    the latents.
 *  - Podcast transcript (my-weird-prompts 640482), DeepSeek Sparse Attention
 *    passage: a top-k list of stored positions is read instead of all of them.
 *  - Same transcript, the decode walk-through: each new token's key and value
 *    are appended to the cache, one entry per layer per token.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous, owned
 *    by the caller.  The library allocates no memory and keeps no state
 *    between calls (the one exception is the test hook
 *    kvc_set_split_override, which stays at 0 unless a test sets it).  q/k/v/out pointers must be 16-byte aligned; seq_lens, idx, lse
 *    and flag 4-byte aligned.
 *  - dtype is KVC_F32 or KVC_BF16 and applies to q, caches, new rows and out.
 *    Arithmetic is float32 (exp, sums, products accumulate in float32); bf16
 *    outputs are rounded to nearest even.  lse is float32, natural log.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Calls are asynchronous and ordered on that stream.
 *  - Errors found on the host are returned synchronously before anything is
 *    enqueued (and before any HIP runtime call): KVC_ERR_* below.  KVC_ERR_HIP
 *    means a launch failed.
 *  - Conditions only the device can see are reported through an optional
 *    device int32 `flag` (bits OR-ed in, never cleared by the library):
 *    KVC_FLAG_CACHE_FULL and KVC_FLAG_BAD_INDEX.
 *  - A sequence with nothing to attend gives an output row of zeros and
 *    lse = -inf.
 *  - Workspace: decode calls that split the positions of a sequence across
 *    workgroups need a device workspace of the size the matching *_workspace
 *    _size call returns (0 means none).  It must be zero-filled before its
 *    first use; every call returns the counters it holds to zero (the rest is
 *    scratch that each call writes before reading), so a workspace is reused
 *    without clearing by calls with the same shape arguments (and the same
 *    split override).  Where the counters sit depends on those arguments:
 *    before a call with other ones, zero-fill the workspace again (a stale
 *    counter gives wrong results for that call, not an access outside the
 *    buffers).  Calls that may run at the same time need separate
 *    workspaces.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, caches, new rows and out (an int-sized enum). */
#ifdef __cplusplus
typedef enum kvc_dtype : int { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;
#else
typedef enum kvc_dtype { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;
#endif

/* status codes */
#define KVC_OK 0
#define KVC_ERR_NULL_PTR (-1)    /* a required pointer is NULL */
#define KVC_ERR_BAD_SHAPE (-2)   /* non-positive size, n_h % n_kv != 0, K > L_max, offsets beyond 2^31 */
#define KVC_ERR_BAD_DTYPE (-3)   /* dtype is not KVC_F32 or KVC_BF16 */
#define KVC_ERR_UNSUPPORTED (-4) /* a shape this build has no kernel for */
#define KVC_ERR_WORKSPACE (-5)   /* workspace smaller than required */
#define KVC_ERR_MISALIGNED (-6)  /* pointer alignment rule broken */
#define KVC_ERR_HIP (-7)         /* HIP launch error */
#define KVC_ERR_BAD_ARG (-8)     /* non-finite scale, negative split override, ... */
#define KVC_ERR_SCRATCH (-9)     /* the call does not fit the library's static scratch */

/* device-side condition bits */
#define KVC_FLAG_CACHE_FULL 1 /* append found seq_lens[b] outside [0, L_max) */
#define KVC_FLAG_BAD_INDEX 2  /* a top-k index outside [0, seq_lens[b]) */

/*
 * kvc_append - write the new token's key and value into the cache.
 * (Podcast transcript, decode walk-through; guide "Two tensors per layer".)
 *
 * For each b with n = seq_lens[b] in [0, L_max):
 *     k_cache[b, :, n, :] = k_new[b]; v_cache[b, :, n, :] = v_new[b];
 *     seq_lens[b] = n + 1.
 * Otherwise nothing is written for b and KVC_FLAG_CACHE_FULL is OR-ed into
 * *flag (when flag is not NULL).  The copy is bit-exact.
 *
 *   k_cache, v_cache  [B, n_kv, L_max, d]; v_cache NULL means a single-tensor
 *                     cache (the latent cache: n_kv = 1, d = d_c + d_r) and
 *                     then v_new must be NULL too.
 *   seq_lens          [B] int32, read and incremented on the device.
 *   k_new, v_new      [B, n_kv, d].
 *   d                 any positive width.
 */
int kvc_append(void* k_cache, void* v_cache, int32_t* seq_lens,
               const void* k_new, const void* v_new,
               int B, int n_kv, int L_max, int d, kvc_dtype dtype,
               int32_t* flag, void* stream);

/*
 * kvc_decode_attn - dense decode attention (MHA, GQA, MQA).
 * (Guide, first section and "Fewer KV heads".)
 *
 * For each b and query head i, with j = i / (n_h / n_kv), n = seq_lens[b]:
 *     s_t = scale * <q[b,i,:], k_cache[b,j,t,:]>   for t < n
 *     out[b,i,:] = sum_t softmax(s)_t * v_cache[b,j,t,:]
 *     lse[b,i]   = log(sum_t exp(s_t))
 * Positions t >= n are never read.  seq_lens must already count the token
 * appended this step (append first, then attend).
 *
 *   q      [B, n_h, d]          k_cache, v_cache [B, n_kv, L_max, d]
 *   out    [B, n_h, d]          lse [B, n_h] float32 or NULL
 *   d in {64, 128}; n_h / n_kv <= 16; L_max * d * elem_bytes < 2^31.
 */
size_t kvc_decode_attn_workspace_size(int B, int n_h, int n_kv, int L_max,
                                      int d, kvc_dtype dtype);
int kvc_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* seq_lens, void* out, float* lse,
                    int B, int n_h, int n_kv, int L_max, int d, float scale,
                    kvc_dtype dtype, void* workspace, size_t ws_bytes, void* stream);

/*
 * kvc_append_decode_attn - kvc_append followed by kvc_decode_attn, in one
 * kernel launch.  (Podcast transcript, decode walk-through: the new token's
 * pair is appended and the token attends over the cache including it.)
 *
 * For each b with n = seq_lens[b] in [0, L_max): k_new[b]/v_new[b] are
 * written at slot n, every query head attends over [0, n + 1), and
 * seq_lens[b] becomes n + 1.  If n is outside [0, L_max) nothing is written,
 * the head attends over [0, clamp(n, 0, L_max)) and KVC_FLAG_CACHE_FULL is
 * set.  Results are those of the two separate calls (bit-identical cache and
 * lengths; outputs equal up to rounding order).
 *
 * Arguments as for kvc_append and kvc_decode_attn; the workspace comes from
 * kvc_append_decode_attn_workspace_size (never 0: it holds one arrival
 * counter per sequence) and follows the same zero-fill rule.
 */
size_t kvc_append_decode_attn_workspace_size(int B, int n_h, int n_kv,
                                             int L_max, int d, kvc_dtype dtype);
int kvc_append_decode_attn(const void* q, void* k_cache, void* v_cache,
                           int32_t* seq_lens, const void* k_new,
                           const void* v_new, void* out, float* lse,
                           int B, int n_h, int n_kv, int L_max, int d,
                           float scale, kvc_dtype dtype, int32_t* flag,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * kvc_append_decode_attn_noalloc - kvc_append_decode_attn without a
 * workspace argument and without any allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The split counters and partials live in a
 * scratch array the library holds in device memory, one copy per GPU (32 MiB,
 * kept until the process ends).  Each call clears the counters it uses on
 * `stream` (a small kernel launch before the attention kernel; no memset, so
 * the call can be captured in a graph) and then runs exactly the kernels of
 * kvc_append_decode_attn, with the same results.
 *
 * Limits: B * n_kv <= 16384, and the split partials (B * n_h * splits
 * values of lse and of d floats of output, splits as the workspace query
 * of kvc_append_decode_attn would plan them) within 32 MiB less 192 KiB:
 * e.g. 32 sequences of 64 query heads, d = 128, up to 32768 positions.
 * A call beyond them returns KVC_ERR_SCRATCH before anything is enqueued.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap
 * on one GPU (on different streams, or from different threads) race and
 * must be serialised by the caller.  Arguments otherwise as for
 * kvc_append_decode_attn.
 */
int kvc_append_decode_attn_noalloc(const void* q, void* k_cache, void* v_cache,
                                   int32_t* seq_lens, const void* k_new, const void* v_new,
                                   void* out, float* lse, int B, int n_h, int n_kv, int L_max,
                                   int d, float scale, kvc_dtype dtype, int32_t* flag,
                                   void* stream);

/*
 * Paged cache (guide, "The allocator, not the algorithm": fixed-size blocks
 * in a shared pool, mapped per sequence by a block table, so a sequence
 * wastes at most block_size - 1 slots).
 *
 * Layout: k_pool, v_pool [num_blocks, n_kv, block_size, d]; block_table
 * [B, max_blocks] int32 device: position t of sequence b is row t % block_size
 * of block block_table[b][t / block_size].  A table entry outside
 * [0, num_blocks) is invalid.  block_size is a power of two in [8, 4096];
 * each pool is at most 2^31 bytes; max_blocks * block_size < 2^31.
 *
 * kvc_append_paged - kvc_append into slot n = seq_lens[b]: n at or past
 * max_blocks * block_size sets KVC_FLAG_CACHE_FULL, an invalid block at the
 * slot sets KVC_FLAG_BAD_INDEX; in both cases nothing is written and the
 * length stays.  dtype KVC_F32 or KVC_BF16, d * element size a multiple of 16.
 *
 * kvc_decode_attn_paged - kvc_decode_attn over positions [0, seq_lens[b])
 * read through the block table (seq_lens clamped to max_blocks *
 * block_size).  Positions in an invalid block are skipped and set
 * KVC_FLAG_BAD_INDEX.  This build supports dtype KVC_BF16 with d = 128.
 * The workspace query takes the table geometry.
 */
int kvc_append_paged(void* k_pool, void* v_pool, const int32_t* block_table,
                     int max_blocks, int32_t* seq_lens, const void* k_new,
                     const void* v_new, int B, int n_kv, int num_blocks,
                     int block_size, int d, kvc_dtype dtype, int32_t* flag, void* stream);
size_t kvc_decode_attn_paged_workspace_size(int B, int n_h, int n_kv, int max_blocks,
                                            int block_size, int d, kvc_dtype dtype);
int kvc_decode_attn_paged(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, int max_blocks,
                          const int32_t* seq_lens, void* out, float* lse, int B,
                          int n_h, int n_kv, int num_blocks, int block_size, int d,
                          float scale, kvc_dtype dtype, int32_t* flag, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * kvc_decode_attn_window - kvc_decode_attn over a sliding window of the
 * newest positions.  ("890 bytes a token", SWA bounded replay passage: for a
 * replay starting at position s, the query at position i attends to keys
 * [max(s, i - W + 1), i]; guide, "Keeping fewer tokens".)
 *
 * For each b with n = seq_lens[b] (the newest query is position n - 1):
 *     lo = clamp(max(s_b, n - window), 0, n), s_b = win_start[b] or 0,
 * and every head attends over [lo, n) exactly as kvc_decode_attn does over
 * [0, n).  Positions below lo are never read.  lo == n gives a zero row and
 * lse = -inf.
 *   window      >= 1, else KVC_ERR_BAD_ARG.
 *   win_start   [B] int32 device array or NULL (all 0).
 *   Other arguments, dtypes, shapes and workspace rules as kvc_decode_attn
 *   (the workspace query takes the window: a window shorter than L_max needs
 *   less).
 */
size_t kvc_decode_attn_window_workspace_size(int B, int n_h, int n_kv, int L_max,
                                             int d, kvc_dtype dtype, int window);
int kvc_decode_attn_window(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* seq_lens, const int32_t* win_start,
                           int window, void* out, float* lse, int B, int n_h,
                           int n_kv, int L_max, int d, float scale, kvc_dtype dtype,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * FP8 E4M3 cache (guide, "Fewer bits per number": the byte width b is a plain
 * multiplier of the cache size, and fp8 is the usual serving default; podcast
 * transcript, KV quantization passage).  Each cached number is one byte, an
 * OCP E4M3 code (finite-only variant: 4 exponent bits with bias 7, 3 mantissa
 * bits, largest finite value 448, codes 0x7F and 0xFF are NaN), and one
 * float32 scale per tensor: stored value = decode(code) * scale.
 *
 * kvc_append_fp8 - as kvc_append with dtype bf16 new rows and E4M3 caches.
 * Each new number x becomes the code nearest to float32(x) * inv in float32
 * arithmetic, where inv = (float)(1.0 / (double)scale), ties to the even
 * code, magnitudes beyond 448 saturating to +-448 and NaN giving 0x7F.
 *   k_cache, v_cache  [B, n_kv, L_max, d] uint8 (both required)
 *   k_new, v_new      [B, n_kv, d] bf16;  d a multiple of 16.
 *   k_scale, v_scale  finite and > 0, else KVC_ERR_BAD_ARG.
 */
int kvc_append_fp8(void* k_cache, void* v_cache, int32_t* seq_lens,
                   const void* k_new, const void* v_new,
                   int B, int n_kv, int L_max, int d,
                   float k_scale, float v_scale, int32_t* flag, void* stream);

/*
 * kvc_decode_attn_fp8 - kvc_decode_attn over E4M3 caches written by
 * kvc_append_fp8: keys are decode(code) * k_scale and values
 * decode(code) * v_scale (the scales are folded into the score scale and the
 * output; the codes are widened to bf16, which holds every E4M3 value
 * exactly).  q and out are bf16, lse float32 or NULL.
 *   q [B, n_h, d]   k_cache, v_cache [B, n_kv, L_max, d] uint8   d = 128;
 *   n_h / n_kv <= 16.  Workspace rules as for kvc_decode_attn.
 */
size_t kvc_decode_attn_fp8_workspace_size(int B, int n_h, int n_kv, int L_max,
                                          int d);
int kvc_decode_attn_fp8(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, void* out, float* lse,
                        int B, int n_h, int n_kv, int L_max, int d, float scale,
                        float k_scale, float v_scale, void* workspace,
                        size_t ws_bytes, void* stream);

/*
 * FP4 cache (podcast transcript, the 890-byte passage; DeepSeek KV cache
 * article, section 6): each number is a 4-bit E2M1 code (sign, 2 exponent
 * bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6)
 * and every 16 consecutive channels of a row share one E4M3 scale byte; no
 * second-level scale.  Stored value = E2M1(code) * E4M3(scale), at most
 * 448 * 6 = 2688 in magnitude.  Two codes per byte, channel 2i in the low
 * nibble of byte i.  Layout per tensor (keys, values):
 *   codes  [B, n_kv, L_max, d/2] uint8     scales [B, n_kv, L_max, d/16] uint8
 *
 * kvc_append_fp4 - quantise the new bf16 rows k_new, v_new [B, n_kv, d] into
 * slot n = seq_lens[b], then bump it (full cache: flag bit 0, nothing
 * written).  Per 16-channel block: scale = the E4M3 value nearest
 * float32(amax / 6) (ties to even, saturating at 448); each number x becomes
 * the E2M1 code nearest float32(x / scale) (ties to the even code, magnitudes
 * past 6 saturating, sign bit from the quotient's sign); a block whose scale
 * is zero stores zero codes.  NaN or infinite inputs are outside the
 * contract.  d a multiple of 16; codes 8-byte aligned, new rows 16-byte
 * aligned.
 */
int kvc_append_fp4(void* k_codes, void* k_scales, void* v_codes, void* v_scales,
                   int32_t* seq_lens, const void* k_new, const void* v_new, int B, int n_kv,
                   int L_max, int d, int32_t* flag, void* stream);

/*
 * kvc_decode_attn_fp4 - kvc_decode_attn over an FP4 cache written by
 * kvc_append_fp4: keys and values are dequantised exactly (to f16: every
 * E2M1 value times an E4M3 scale is an f16 number) and both products run
 * in f16 with float32 accumulation; each head's query is taken to f16
 * times a power of two (exact for every component within 2^29 of the
 * head's largest), the softmax weights are rounded to f16.  q and out are
 * bf16, lse float32 or NULL.  d = 128, n_h / n_kv <= 16; scale arrays
 * 8-byte aligned; scale bytes are finite E4M3 values (as kvc_append_fp4
 * writes them).  Workspace rules as for kvc_decode_attn.
 */
size_t kvc_decode_attn_fp4_workspace_size(int B, int n_h, int n_kv, int L_max, int d);
int kvc_decode_attn_fp4(const void* q, const void* k_codes, const void* k_scales,
                        const void* v_codes, const void* v_scales, const int32_t* seq_lens,
                        void* out, float* lse, int B, int n_h, int n_kv, int L_max, int d,
                        float scale, void* workspace, size_t ws_bytes, void* stream);

/*
 * kvc_decode_attn_mla - decode attention over a latent (MLA) cache.
 * (Guide, "Caching a compressed latent" and the memory footnote.)
 *
 * For each b and head i, n = seq_lens[b]:
 *     s_t = scale * (<q_lat[b,i], c[b,t]> + <q_rope[b,i], k_rope[b,t]>)
 *     out[b,i,:] = sum_t softmax(s)_t * c[b,t,:]        (d_c wide)
 * where q[b,i] = q_lat (d_c) followed by q_rope (d_r), and
 * ckv[b,t] = c (d_c) followed by k_rope (d_r).  Queries are the absorbed
 * ones; the up-projections are outside this call.
 *
 *   q [B, n_h, d_c + d_r]   ckv [B, L_max, d_c + d_r]   out [B, n_h, d_c]
 *   This build supports dtype KVC_BF16, d_c = 512, d_r = 64, n_h % 64 == 0.
 */
size_t kvc_decode_attn_mla_workspace_size(int B, int n_h, int L_max, int d_c,
                                          int d_r);
int kvc_decode_attn_mla(const void* q, const void* ckv,
                        const int32_t* seq_lens, void* out, float* lse,
                        int B, int n_h, int L_max, int d_c, int d_r,
                        float scale, kvc_dtype dtype, void* workspace,
                        size_t ws_bytes, void* stream);

/*
 * kvc_decode_attn_topk - decode attention over listed positions only.
 * (Podcast, DeepSeek Sparse Attention passage.)
 *
 * As kvc_decode_attn, but query heads of KV head j attend only over the
 * positions idx[b, j, 0..K-1] (gather, then attend; a position listed twice
 * counts twice).  An index outside [0, seq_lens[b]) is skipped and sets
 * KVC_FLAG_BAD_INDEX.
 *
 *   idx [B, n_kv, K] int32 device.   1 <= K <= L_max.
 */
size_t kvc_decode_attn_topk_workspace_size(int B, int n_h, int n_kv, int K,
                                           int d, kvc_dtype dtype);
int kvc_decode_attn_topk(const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* seq_lens,
                         const int32_t* idx, int K, void* out, float* lse,
                         int B, int n_h, int n_kv, int L_max, int d,
                         float scale, kvc_dtype dtype, int32_t* flag,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * kvc_topk_select - which positions the sparse decode reads.  (Podcast
 * transcript, DeepSeek Sparse Attention passage: an indexer scores the
 * prefix and keeps a top-k subset, k = 2048 in the released code; "A Hundred
 * Messages" blog, section 4: a deeper indexer picks its top-512 only from a
 * candidate pool of 8-position blocks, at most 2,048 of them.)
 *
 * For each row r = (b, j) of scores [B, R, L_max] float32: the K positions
 * t < clamp(seq_lens[b], 0, L_max) with the highest scores, equal scores
 * taken by lower position first, written to idx_out[b, j, :] in ascending
 * position order (the layout kvc_decode_attn_topk reads); if fewer than K
 * positions qualify, the rest of the row is -1.  With pool != NULL
 * ([B, R, P] int32 block ids), only positions t with t / pool_block among
 * the row's pool entries qualify (entries outside [0, ceil(L_max /
 * pool_block)) are ignored).  Scores are compared exactly (-0 equals +0);
 * NaN scores are outside the contract.  The result is deterministic.
 *   K >= 1; L_max < 2^29 (else KVC_ERR_UNSUPPORTED); pool mode: P >= 1,
 *   pool_block >= 1, ceil(L_max / pool_block) <= 393216 (else
 *   KVC_ERR_UNSUPPORTED).
 * Workspace (optional, same rules as the decode calls): with workspace !=
 * NULL, no pool and a non-zero kvc_topk_select_workspace_size, each row is
 * cut into segments spread over the compute units (a workspace smaller than
 * the queried size is KVC_ERR_WORKSPACE, one not 256-byte aligned
 * KVC_ERR_MISALIGNED); with workspace == NULL, in pool mode, or when the
 * query returns 0 (rows longer than 2^18 positions, or enough rows to fill
 * the device), one workgroup takes each row.  The result is the same either
 * way.
 */
size_t kvc_topk_select_workspace_size(int B, int R, int L_max, int K);
int kvc_topk_select(const float* scores, const int32_t* seq_lens, const int32_t* pool,
                    int P, int pool_block, int32_t* idx_out, int B, int R, int L_max,
                    int K, void* workspace, size_t ws_bytes, void* stream);

/* Text for a status code (static storage). */
const char* kvc_status_string(int status);

/*
 * Test and tuning hook, not part of the attention interface: the positions
 * one workgroup handles before results are merged across workgroups.  0 (the
 * initial value) restores the built-in policy; other values are rounded up
 * to the kernel granularity.  This is the library's only state: it is
 * process-wide and applies to every later workspace query and decode call,
 * so a query and the call that uses its workspace must see the same
 * setting.  Do not change it while decode calls may be enqueued from other
 * threads.  Returns KVC_ERR_BAD_ARG if negative.
 */
int kvc_set_split_override(int positions);

/* Positions per workgroup the policy would pick (after any override). */
int kvc_split_positions(int kind, int B, int units, int n_max);
#define KVC_KIND_DENSE 0
#define KVC_KIND_TOPK 1
#define KVC_KIND_MLA 2

/*
 * Diagnostics for bandwidth measurement (not part of the attention path).
 * kvc_stream_read reads `bytes` (multiple of 16) from src the way the decode
 * kernels read cache rows (each workgroup one contiguous slab, 16-byte
 * buffer loads with the non-temporal policy) and writes one float per
 * workgroup to sink (so the loads are kept); sink needs
 * kvc_stream_read_sink_floats(bytes) floats.
 * kvc_copy copies `bytes` (multiple of 16) from src to dst.
 */
size_t kvc_stream_read_sink_floats(size_t bytes);
int kvc_stream_read(const void* src, size_t bytes, float* sink, void* stream);
int kvc_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
