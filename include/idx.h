/* idx.h - C ABI of libidx.so, an MI355X (gfx950) implementation of the DeepSeek Sparse
 * Attention lightning indexer and two of its published accelerations.
 *
 * The indexer scores, for every query t, each key s of its causal prefix with
 *     I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s])
 * (H indexer heads, one shared indexer key per token, fp32 head weights) and keeps the k
 * best-scoring tokens of each query. All five source pages build on this indexer ("ADIndex:
 * Layer-Adaptive Sparse Attention Indexing via Group-Level Distillation", abstract; "Multi-layer
 * Indexer ...", authors' abstract, k = 2048; "PIVOT: Efficient Query-Group Indexing for
 * Token-Level Sparse Attention", abstract; "HISA: Efficient Hierarchical Indexing for
 * Fine-Grained Sparse Attention", abstract; "LatentIndex: Cross-Layer Sharing with
 * Layer-Specific Selection for Sparse Attention", abstract).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers (HIP device memory of the current device) unless stated.
 *     `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call only
 *     enqueues work on `stream` and returns; it never allocates, frees or synchronises.
 *   - The caller owns all buffers. Scratch memory is the caller's `ws` buffer of `ws_bytes`
 *     bytes, at least idx_workspace_bytes(...) for the same arguments.
 *   - Output rows hold a SET of token indices: the first n = min(k, visible candidates) entries
 *     are distinct token indices (within the sequence, 0..N-1) in unspecified order, the rest
 *     are -1; out_score (optional, may be NULL) holds the fp32 score of each index and -inf for
 *     the padding. When several tokens tie with the k-th best score, the lowest indices are kept,
 *     so the set is deterministic.
 *   - Return value: IDX_OK or a negative IDX_ERR_* code. Argument errors are detected before
 *     anything is enqueued. Device-array contents are preconditions and are not checked:
 *     0 <= k_len[b] <= N, keys and queries finite, fp8 scales >= 0 and finite.
 *   - Thread safety: calls are reentrant; calls that share a workspace on different streams race.
 */
#ifndef IDX_H_
#define IDX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element formats */
enum {
  IDX_F32 = 0,       /* IEEE binary32 */
  IDX_BF16 = 1,      /* bfloat16 (upper half of binary32) */
  IDX_FP8_E4M3 = 2   /* OCP FP8 E4M3FN with fp32 scales: key = decode(byte) * k_scale[token],
                        query = decode(byte) * q_scale[query, head] */
};

/* status codes */
enum {
  IDX_OK = 0,
  IDX_ERR_INVALID_ARG = -1,  /* null required pointer, size <= 0, k <= 0, bad group/block args */
  IDX_ERR_UNSUPPORTED = -2,  /* dtype / H / D / size combination not built (see below)        */
  IDX_ERR_ALIGN = -3,        /* q, k or w not 16-byte aligned, or k_scale/q_pos/k_len not 4    */
  IDX_ERR_WORKSPACE = -4,    /* ws NULL or ws_bytes < idx_workspace_bytes(...)                 */
  IDX_ERR_HIP = -5,          /* a HIP launch reported an error                                  */
  IDX_ERR_INTERNAL = -6      /* unexpected internal failure (no exception crosses the ABI)     */
};

/* operation ids for idx_workspace_bytes */
enum { IDX_OP_SCORE_TOPK = 0, IDX_OP_GROUP = 1, IDX_OP_BLOCK = 2, IDX_OP_REFINE = 3, IDX_OP_REUSE = 4 };

/* The indexer's inputs. Layouts are dense and row-major.
 *   q       [B, T, H, D]  q_dtype IDX_F32, IDX_BF16, or IDX_FP8_E4M3 (dense entry points only,
 *                         with FP8 keys and D in {64, 128}: both operands on the FP8 matrix cores)
 *   k       [B, N, D]     k_dtype IDX_F32, IDX_BF16 or IDX_FP8_E4M3 (the per-layer key cache)
 *   k_scale [B, N] fp32   required iff k_dtype == IDX_FP8_E4M3, else ignored
 *   w       [B, T, H] fp32 head weights, any sign
 *   q_pos   [B, T] int32  position of each query: key s is visible to query (b,t) iff
 *                         s <= q_pos[b,t] and s < k_len[b] (the query's own token is visible);
 *                         q_pos < 0 means an empty prefix
 *   k_len   [B] int32     keys present in each sequence's cache, or NULL for N
 *   q_scale [B, T, H] fp32 required iff q_dtype == IDX_FP8_E4M3, else ignored; scales >= 0 and
 *                         finite (a precondition, like k_scale)
 * Built shapes: H in 1..128, D in {32, 64, 128}. Prefill (T large) and decode (T = 1..4 multi-token
 * prediction queries against a long cache) use the same call; decode-shaped problems (bf16
 * queries, FP8 or bf16 keys, H <= 64, D in {64, 128}, T <= 4, N >= 2048) take a streaming path
 * whose workspace differs, so size it with idx_workspace_bytes for the same shape. */
typedef struct idx_problem {
  int32_t B, T, H, D, N;
  int32_t q_dtype, k_dtype;
  const void* q;
  const void* k;
  const float* k_scale;
  const float* w;
  const int32_t* q_pos;
  const int32_t* k_len;
  const float* q_scale;
} idx_problem;

/* Dense lightning indexer: score every visible key of every query and keep the top k.
 *   out_idx   [B, T, k] int32 (required), out_score [B, T, k] fp32 (optional).
 * FP8 queries with FP8 keys run the q.k contraction on FP8 x FP8 matrix cores: the dot product
 * of the stored bytes is accumulated in fp32, then each head's weight times its query scale and
 * the key's scale are applied (both scales >= 0 factor out of the ReLU). The other entry points
 * take F32 or BF16 queries (IDX_ERR_UNSUPPORTED for FP8 queries).
 * Source: the indexer itself ("Multi-layer Indexer ...", authors' abstract: every layer's indexer
 * scores the whole cache and keeps the k = 2048 best tokens; "PIVOT ...", abstract: the scan over
 * every preceding token costs O(L^2) per layer); its scoring on FP8 matrix cores follows the
 * LatentIndex page's ("LatentIndex: Cross-Layer Sharing ...", abstract) aim of a cheaper indexer
 * scan. */
int idx_score_topk(const idx_problem* p, int32_t k, int32_t* out_idx, float* out_score,
                   void* ws, size_t ws_bytes, void* stream);

/* idx_score_topk without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and errors as idx_score_topk, except that the
 * scratch is the library's own static device array of 256 MiB per device (held from the
 * library's first call on a device until the process ends; its address is looked up once per
 * device). Prefill-shaped problems hold their score rows in chunks that fit it; decode-shaped
 * problems need B*T*N*16 bytes plus a little, so decode calls up to about 16M cached (query,
 * key) slots fit (e.g. 32 sequences x 2 MTP queries x 131072 keys). A problem whose plan does
 * not fit (a single prefill row of more than about 64M keys, or a larger decode batch) returns
 * IDX_ERR_WORKSPACE before anything is enqueued. Every call on a device shares that device's
 * array: calls that overlap on one device (different streams, or several host threads) race and
 * must be serialised by the caller. The array's contents persist between calls; the kernels
 * read nothing from it that the same call did not write first. */
int idx_score_topk_noalloc(const idx_problem* p, int32_t k, int32_t* out_idx, float* out_score,
                           void* stream);

/* Group-shared scan with per-query refine ("PIVOT ...", abstract; PIVOT-Refine).
 * Queries are cut into groups of `group_size` consecutive queries (the last group may be
 * shorter). Each group is reduced to one proxy query: the element-wise mean of its queries and
 * of their head weights (fp32 sum in ascending query order, one fp32 division, rounded to bf16
 * nearest-even for bf16 queries), positioned at the largest member position. The proxy scores its
 * prefix once and keeps its n_cand best tokens (the candidate set, min(n_cand, prefix) entries).
 * Every member then scores the candidates inside its own prefix with its own query and weights
 * and keeps its top k.
 *   out_idx [B, T, k] int32 (required), out_score [B, T, k] fp32 (optional),
 *   out_cand [B, ceil(T/group_size), n_cand] int32 (optional): each group's candidates in
 *            ascending token order, -1 padded.
 * A proxy keeps min(n_cand, its prefix length) candidates, so any n_cand >= 1 is valid; with
 * n_cand >= the prefix length the result equals idx_score_topk's.
 * In decode, a group is the queries decoded together in one multi-token-prediction step (same
 * abstract): pass group_size = T, the number of MTP queries per sequence. */
int idx_group_proxy_refine(const idx_problem* p, int32_t k, int32_t group_size, int32_t n_cand,
                           int32_t* out_idx, float* out_score, int32_t* out_cand,
                           void* ws, size_t ws_bytes, void* stream);

/* Hierarchical block-coarse / token-refine indexer ("HISA ...", abstract).
 * The key cache is cut into blocks of `block_size` consecutive tokens; each block present in the
 * cache is pooled into one key (mean of its tokens: fp32 sum in ascending token order, one fp32
 * division, rounded to bf16 nearest-even for bf16 keys). A query scores the pooled blocks whose
 * first token is in its prefix (same score formula), keeps its n_blocks_keep best blocks, then
 * scores the tokens of the kept blocks inside its prefix and keeps its top k.
 *   out_idx [B, T, k] int32 (required), out_score [B, T, k] fp32 (optional),
 *   out_blocks [B, T, n_blocks_keep] int32 (optional): kept block ids in ascending order, -1
 *              padded.
 * Keys may be IDX_BF16, IDX_F32 or IDX_FP8_E4M3: an FP8 key enters its block's mean as its fp32
 * value decode(byte) * k_scale (one fp32 multiply), and the pooled keys are bf16 (fp32 for fp32
 * keys); the token refine scores the FP8 keys themselves. Requires ceil(N / block_size) <= 65536
 * and n_blocks_keep <= 32767. With n_blocks_keep >= the number of eligible blocks the result
 * equals idx_score_topk's. */
int idx_block_coarse_refine(const idx_problem* p, int32_t k, int32_t block_size,
                            int32_t n_blocks_keep, int32_t* out_idx, float* out_score,
                            int32_t* out_blocks, void* ws, size_t ws_bytes, void* stream);

/* The pooled block keys of idx_block_coarse_refine for the whole cache, written to `pooled`
 * [B, ceil(N / block_size), D]: bf16 for IDX_BF16 and IDX_FP8_E4M3 keys, fp32 for IDX_F32 keys (a
 * block past k_len[b] is written as zeros and never scored). Only the key fields of *p (B, N, D,
 * k_dtype, k, k_scale, k_len) are read. A caller that keeps the pooled keys beside its key cache
 * (a decoding server pools a block once it is complete) passes them to the *_pooled entry points
 * below instead of pooling the whole cache on every call ("HISA ...", abstract: block-level
 * pooled representations of the cache). Errors: IDX_ERR_INVALID_ARG (null k, pooled or
 * required k_scale, block_size < 1), IDX_ERR_UNSUPPORTED (D not 32, 64 or 128),
 * IDX_ERR_ALIGN (k or pooled not 16-byte aligned). */
int idx_block_pool(const idx_problem* p, int32_t block_size, void* pooled, void* stream);

/* Absorbed queries for a layer that scores a shared latent cache ("LatentIndex: Cross-Layer
 * Sharing with Layer-Specific Selection for Sparse Attention", abstract: a layer group shares one
 * latent cache, and each layer scores it by absorbing its key decoder into its queries instead of
 * rebuilding its own keys). With the layer's key k[s] = latent[s] . wk (decoder wk [Dc, D]),
 * q . k[s] = (wk q) . latent[s], so
 *   q_lat[r, h, j] = bf16 nearest-even of sum_d q[r, h, d] * wk[j, d]   (fp32 accumulation)
 * for rows r < rows (B * T), heads h < H, j < Dc. q: bf16 [rows, H, D]; wk: bf16 [Dc, D];
 * q_lat: bf16 [rows, H, Dc], caller-owned device memory. The absorbed queries then go to any
 * entry point of this library as its queries, with the latent cache [B, N, Dc] (bf16, fp32 or FP8
 * with per-token scales) as its keys and D = Dc. Errors: IDX_ERR_INVALID_ARG (null pointer,
 * rows or H < 1), IDX_ERR_UNSUPPORTED (D or Dc not 32, 64 or 128), IDX_ERR_ALIGN (a pointer not
 * 16-byte aligned). */
int idx_absorb_queries(const void* q, int32_t rows, int32_t H, int32_t D, const void* wk, int32_t Dc,
                       void* q_lat, void* stream);

/* idx_block_coarse_refine with the caller's pooled keys (as idx_block_pool writes them) in place
 * of pooling inside the call; `pooled` is required and 16-byte aligned. Same results. */
int idx_block_coarse_refine_pooled(const idx_problem* p, int32_t k, int32_t block_size,
                                   int32_t n_blocks_keep, const void* pooled, int32_t* out_idx,
                                   float* out_score, int32_t* out_blocks, void* ws, size_t ws_bytes,
                                   void* stream);

/* Group-shared scan without refine ("PIVOT ...", abstract; PIVOT-Reuse: the proxy's top-k is
 * shared across the group). Groups and proxies are those of idx_group_proxy_refine. The proxy
 * scores its prefix once and keeps its k best tokens (ties to the lower token); every member
 * takes those of them inside its own prefix, with the proxy's scores, and nothing is re-scored.
 * The member with the largest position receives the whole proxy top-k; group_size = 1 gives
 * idx_score_topk's result. In decode, group_size = T groups one step's MTP queries.
 *   out_idx [B, T, k] int32 (required), out_score [B, T, k] fp32 (optional): the member's part
 *           of the proxy top-k (order unspecified), then -1 / -inf. */
int idx_group_proxy_reuse(const idx_problem* p, int32_t k, int32_t group_size, int32_t* out_idx,
                          float* out_score, void* ws, size_t ws_bytes, void* stream);

/* Block-filtered group proxy: the group proxy of idx_group_proxy_refine ("PIVOT ...", abstract)
 * scores the pooled blocks of idx_block_coarse_refine ("HISA ...", abstract) instead of every
 * token of its prefix. Each group's proxy scores the pooled blocks whose first token is in its
 * prefix and keeps its n_blocks_keep best (ties to the lower block); every member then scores
 * the tokens of the kept blocks inside its own prefix with its own query and weights and keeps
 * its top k.
 *   out_idx [B, T, k] int32 (required), out_score [B, T, k] fp32 (optional),
 *   out_blocks [B, ceil(T/group_size), n_blocks_keep] int32 (optional): each group's kept blocks
 *              in ascending order, -1 padded.
 * Keys may be IDX_BF16, IDX_F32 or IDX_FP8_E4M3 (pooled as in idx_block_coarse_refine). Requires
 * ceil(N / block_size) <= 65536 and n_blocks_keep <= 32767. group_size = 1 gives
 * idx_block_coarse_refine's result; keeping every block gives idx_score_topk's. In decode,
 * group_size = T filters the cache once for the queries of one multi-token-prediction step. Its
 * workspace size is idx_group_block_workspace_bytes(...). */
int idx_group_block_refine(const idx_problem* p, int32_t k, int32_t group_size, int32_t block_size,
                           int32_t n_blocks_keep, int32_t* out_idx, float* out_score,
                           int32_t* out_blocks, void* ws, size_t ws_bytes, void* stream);

/* idx_group_block_refine with the caller's pooled keys (as idx_block_pool writes them) in place
 * of pooling inside the call; `pooled` is required and 16-byte aligned. Same results. */
int idx_group_block_refine_pooled(const idx_problem* p, int32_t k, int32_t group_size,
                                  int32_t block_size, int32_t n_blocks_keep, const void* pooled,
                                  int32_t* out_idx, float* out_score, int32_t* out_blocks, void* ws,
                                  size_t ws_bytes, void* stream);

/* Workspace bytes of idx_group_block_refine (and of its _pooled form) for the same arguments
 * (only the shape fields of *p are read); 0 for invalid arguments. */
size_t idx_group_block_workspace_bytes(const idx_problem* p, int32_t k, int32_t group_size,
                                       int32_t block_size, int32_t n_blocks_keep);

/* Per-query refine over candidate sets the caller supplies: a token bank shared by a group of
 * queries and refined by each of them ("ADIndex: Layer-Adaptive Sparse Attention Indexing via
 * Group-Level Distillation", abstract), or the candidate set an anchor layer proposes and a
 * follower layer refines ("LatentIndex: Cross-Layer Sharing with Layer-Specific Selection for
 * Sparse Attention", abstract, hierarchical selection).
 * Queries are cut into groups of `group_size` consecutive queries (the last group may be
 * shorter); group g of sequence b owns row (b, g) of `cand`:
 *   cand     [B, ceil(T/group_size), n_cand] int32 (required): token ids; of each row the first
 *            cand_cnt[b, g] entries are read (all n_cand when cand_cnt is NULL; counts are
 *            clamped into [0, n_cand]);
 *   cand_cnt [B, ceil(T/group_size)] int32 (optional).
 * A row's candidate set is the set of the values read that are tokens of the sequence's cache,
 * [0, k_len[b]): -1 padding and other values are dropped, repeated values count once. Every member then scores the
 * candidates inside its own prefix with its own query and weights and keeps its top k (ties
 * keep the lowest tokens), exactly as the refine step of idx_group_proxy_refine.
 *   out_idx [B, T, k] int32 (required), out_score [B, T, k] fp32 (optional).
 * group_size = 1 gives each query its own set; a set holding the whole prefix gives
 * idx_score_topk's result. Requires N <= 1048576 (IDX_ERR_UNSUPPORTED otherwise). */
int idx_refine_given(const idx_problem* p, int32_t k, int32_t group_size, const int32_t* cand,
                     const int32_t* cand_cnt, int32_t n_cand, int32_t* out_idx, float* out_score,
                     void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes needed by one call. op = IDX_OP_*; p1, p2 = (group_size, n_cand) for
 * IDX_OP_GROUP and IDX_OP_REFINE, (block_size, n_blocks_keep) for IDX_OP_BLOCK (also enough for
 * idx_block_coarse_refine_pooled), (group_size,
 * ignored) for IDX_OP_REUSE, ignored for IDX_OP_SCORE_TOPK.
 * Only the shape fields of *p are read (pointers may be NULL). Returns 0 for invalid arguments. */
size_t idx_workspace_bytes(int op, const idx_problem* p, int32_t k, int32_t p1, int32_t p2);

/* Static, human-readable text for a status code. */
const char* idx_strerror(int status);

/* Kernel timing (host-side switch, for benchmarking). While enabled, every library call
 * records a HIP event pair around each kernel launch on the call's stream. idx_timer_read
 * waits for the recorded events and returns the summed milliseconds and the launch count of
 * the kernels whose name contains `kernel_substr` (all kernels if NULL or ""); kernel names are
 * "score", "topk", "sort", "proxy", "pool", "block_refine", "reuse", "decode_scan" and
 * "decode_select".
 * idx_timer_enable(on) clears the record and switches recording on or off; switching it on
 * creates a pool of 8192 HIP events once (IDX_ERR_HIP if that fails), so library calls never
 * create events. At most 4096 launches are recorded per enable; idx_timer_read returns
 * IDX_ERR_INTERNAL (with the recorded totals) when launches went unrecorded. Not thread safe. */
int idx_timer_enable(int on);
int idx_timer_read(const char* kernel_substr, double* total_ms, int32_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* IDX_H_ */
