// Internal kernel argument blocks and launchers (host side of the library only; not part of
// the public C ABI in include/idx.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idx {

// Score a tile of queries against a key set and write one fp32 score per (query, slot).
//   RANGE mode: slot j is key j of the sequence's key array, visible to query t iff
//               j * pos_stride <= q_pos[t] and j < ceil(k_len / count_div). Used by the dense
//               indexer (pos_stride = count_div = 1) and by the pooled-block coarse scan
//               (pos_stride = count_div = block size; key j = pooled block j).
//   LIST  mode: slot j is key list[g][j] for the query's group g = t / group_size; a slot whose
//               key is beyond q_pos[t] gets -inf. Used by the group refine.
enum { MODE_RANGE = 0, MODE_LIST = 1 };

struct ScoreArgs {
  const void* q; int q_dtype;      // [B, T, H, D]
  const float* q_scale;            // [B, T, H] (FP8 queries) or null
  const float* w;                  // [B, T, H]
  const int32_t* q_pos;            // [B, T]
  const void* keys; int k_dtype;   // [B, key_cap, D]
  const float* k_scale;            // [B, key_cap] (fp8 keys) or null
  const int32_t* k_len;            // [B] tokens in the cache, or null (= tok_cap)
  int B, T, H, D;
  int key_cap;                     // key rows per sequence in `keys`
  int tok_cap;                     // token capacity per sequence (N), for a null k_len
  int mode, pos_stride, count_div;
  const int32_t* list; const int32_t* list_len; int list_stride; int group_size; int n_groups;
  int c0, c1;                      // RANGE: query range [c0,c1); LIST: group range [c0,c1)
  float* scores; int64_t score_stride;
  int32_t* row_len;                // slots per row, written by split 0
  int32_t* row_meta;               // optional [rows][4] selection summary (needs one key split)
  int topk_k;                      // selection size the summary is computed for
  int digit_bits;                  // width of the summary's radix digit (11, or 12 for rows < 65536)
  int rows_per_seq;                // score rows per sequence in this chunk
  int tiles_per_seq;
  int split_keys;                  // keys per grid.y split (multiple of the key tile)
  // optional selection by the score kernel itself (key range, bf16, one key split, 12-bit
  // summary): the top topk_k slots of row (b, t) go to sel_idx/sel_score [B, sel_T, topk_k].
  // Rows then have room for 16-bit slots from float offset slot_off (score_stride >= slot_off *
  // 3 / 2, slot_off >= rows' slots + 64, a multiple of 64); with sel_list the row holds a
  // candidate list (scores from the row start, their slots there) instead of every slot
  int32_t* sel_idx; float* sel_score; int sel_T;
  int slot_off, sel_list;
  int32_t* sel_cnt;                // optional [B, sel_T]: selections per row (min(topk_k, finite))
};

// Pick rows from per-row score arrays: the top-k slots of each row (a set; with a row summary
// from the score kernel the order within the row is unspecified, otherwise ascending).
enum { MAP_IDENT = 0, MAP_LIST = 1, MAP_BLOCKS = 2 };

// Row selection summary written by a score kernel next to each score row (first radix digit, 11
// or 12 bits, of the order-preserving key image): {finite slots, bin of the k-th largest key or -1 when every
// finite slot is selected, slots in higher bins, slots in that bin}.
enum { META_NVALID = 0, META_BIN = 1, META_ABOVE = 2, META_INBIN = 3 };

struct TopkArgs {
  const float* scores; int64_t score_stride;
  const int32_t* row_len;
  const int32_t* row_meta;         // optional: summaries from the score kernel
  int digit_bits;                  // their radix digit width
  int n_rows, k;
  int rows_per_seq, T_out, t_off;  // output row = (r / rows_per_seq) * T_out + t_off + r % rows_per_seq
  int32_t* out_idx; float* out_score; int out_stride;
  int32_t* out_count;              // optional: selections per output row
  int map_mode;
  const int32_t* list; int list_stride; int group_size; int n_groups;
  const int32_t* blocks; int blocks_stride; int block_size;
};

struct ProxyArgs {
  const void* q; int q_dtype; const float* w; const int32_t* q_pos;
  int B, T, H, D, G, n_groups;
  void* pq; float* pw; int32_t* ppos;   // [B, NG, H, D], [B, NG, H], [B, NG]
};

struct ReuseArgs {
  const int32_t* gidx; const float* gsc; const int32_t* gcnt;   // [B, NG, k], [B, NG, k], [B, NG]
  const int32_t* q_pos; const int32_t* k_len;
  int B, T, N, G, NG, k;
  int32_t* out_idx; float* out_score;                           // [B, T, k]
};

struct PoolArgs {
  const void* keys; int k_dtype; const int32_t* k_len;
  const float* k_scale;                  // [B, N] for FP8 keys
  int B, N, D, block_size, n_blocks;    // n_blocks = ceil(N / block_size) (row capacity)
  void* pooled;                          // [B, n_blocks, D]: fp32 for fp32 keys, else bf16
};

struct BlockRefineArgs {
  const void* q; int q_dtype; const float* w; const int32_t* q_pos;
  const void* keys; int k_dtype; const int32_t* k_len;
  int B, T, H, D, N;
  const int32_t* blocks; const int32_t* n_kept; int keep_stride; int block_size;
  int t0, t1;                            // query range of this chunk
  float* scores; int64_t score_stride;   // slot = kept position * block_size + offset
  int32_t* row_len; int rows_per_seq; int tiles_per_seq;
  int32_t* row_meta; int topk_k;
};

// Decode scan + selection (few queries per sequence, long cache): see decode.hip.
constexpr int DECODE_BINS = 4096;  // first-digit histogram bins per row
constexpr int DECODE_SUB = 16384;  // keys per scan sub-chunk (scores held in LDS)
struct DecodeArgs {
  const void* q; const float* w; const int32_t* q_pos;      // bf16 [B, T, H, D], [B, T, H], [B, T]
  const void* keys; int k_dtype; const float* k_scale;      // [B, N, D] FP8 or bf16, [B, N]
  const int32_t* k_len;
  int B, T, H, D, N;
  int nchunk, chunk, sub;          // key chunks per sequence (scan work-groups), keys per chunk,
                                   // keys per sub-chunk (multiple of 64, at most DECODE_SUB,
                                   // dividing chunk)
  uint32_t* ccount;                // [B*T][nsegs] candidates per sub-chunk (written by the scan)
  uint32_t* shist;                 // [B*T][nsegs][DECODE_BINS / 2] each sub-chunk's first-digit
                                   // histogram: bins w and w + 2048 in the low and high 16-bit
                                   // halves of word w (written by the scan)
  int nsegs;                       // sub-chunks per row: ceil(N / sub)
  uint32_t* cand_key; uint32_t* cand_idx;                    // [B*T][cand_cap] scan candidates
  uint32_t* cand2_key; uint32_t* cand2_idx;                  // [B*T][cand_cap] bin-b1 candidates
  int cand_cap;                    // >= N, multiple of 64
  int k;                           // selection size
  int32_t* out_idx; float* out_score;                        // [B, T, k]
  int32_t* out_cnt;                // optional [B*T]: selections per row (the select writes it)
  int pair;                        // queries per scan work-group: 2, or 1 where a pair would span
                                   // two kept-block lists
  int vn;                          // slots per row: N, or keep_stride << blk_shift with blocks
  // kept-block mode (blocks != NULL): the slots of row b*T+t are the tokens of the kept blocks of
  // list row b*n_groups + t/group_size, ascending: slot j is token
  // (blocks[row][j >> blk_shift] << blk_shift) + (j & (2^blk_shift - 1)); n_kept[row] blocks
  const int32_t* blocks; const int32_t* n_kept;
  int keep_stride, blk_shift, group_size, n_groups;
};
constexpr int DECODE_KEEP_MAX = 2048;  // kept blocks per list in the kept-block scan (LDS table)

hipError_t launch_score(const ScoreArgs& a, int n_splits, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, int max_row_len, hipStream_t s);
hipError_t launch_proxy(const ProxyArgs& a, hipStream_t s);
hipError_t launch_pool(const PoolArgs& a, hipStream_t s);
hipError_t launch_reuse_rows(const ReuseArgs& a, hipStream_t s);
// kept blocks (ascending) -> ascending token lists inside the cache, keep * block_size per row
hipError_t launch_expand_blocks(const int32_t* blocks, const int32_t* n_kept, int keep, int block_size,
                                int N, const int32_t* k_len, int n_groups, int32_t* list, int32_t* cnt,
                                int n_rows, hipStream_t s);
// caller-supplied candidate lists -> ascending sets of ids in [0, k_len[b]) (rows of C entries)
hipError_t launch_given_lists(const int32_t* src, const int32_t* cnt, int C, int N, const int32_t* k_len,
                              int n_groups, int32_t* dst, int32_t* dst_cnt, int n_rows, hipStream_t s);
hipError_t launch_block_refine(const BlockRefineArgs& a, hipStream_t s);
// Sorts rows of distinct values in [0, max_value) ascending (count[r] values in row r).
hipError_t launch_sort_rows(int32_t* rows, int stride, const int32_t* count, int n_rows, int max_count,
                            int max_value, hipStream_t s);
bool score_supported(int q_dtype, int k_dtype, int H, int D);
bool decode_supported(int q_dtype, int k_dtype, int H, int D, int T, int N);
// the kept-block scan: 2^blk_shift-token blocks with blk_shift >= 4, at most DECODE_KEEP_MAX kept
bool decode_blocks_supported(int q_dtype, int k_dtype, int H, int D, int T, int N, int block_size, int keep);
hipError_t launch_decode_scan(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_select(const DecodeArgs& a, hipStream_t s);
// absorbed queries: out[m, j] = bf16(sum_d q[m, d] * wk[j, d]) for m < M (bf16 [M, D], [Dc, D], [M, Dc])
hipError_t launch_absorb(const void* q, const void* wk, void* out, int64_t M, int D, int Dc, hipStream_t s);

constexpr int KEY_TILE = 64;       // keys per LDS tile of the score kernels
constexpr int Q_TILE = 8;          // queries per work-group tile (one per wave)

}  // namespace idx
