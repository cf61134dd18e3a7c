// C ABI of the indexer library: argument validation, workspace planning and carving, and the
// kernel sequence of each entry point (all enqueued on the caller's stream, no allocation, no
// synchronisation). See include/idx.h for the contract.
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/idx.h"
#include "kernels.h"

namespace idx {

int score_queries_per_tile(int H);

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kScoreBudget = size_t(1) << 30;     // score rows held per chunk (bytes)
constexpr int kTargetGroups = 1024;                  // work-groups wanted per score launch

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
// score-row stride (floats): rows start 256-byte aligned so that the selector can use 16-byte loads
int64_t rstride(int64_t n) { return (n + 63) / 64 * 64; }

// ---------------------------------------------------------------------------------------------
// kernel timing (idx_timer_enable / idx_timer_read)

struct TimerRec {
  const char* name;
  hipEvent_t a, b;
};
bool g_timer_on = false;
std::vector<TimerRec> g_recs;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& f) {
  if (!g_timer_on) return f();
  hipEvent_t a = pool_event(), b = pool_event();
  if (a) hipEventRecord(a, s);
  hipError_t e = f();
  if (b) hipEventRecord(b, s);
  if (a && b) g_recs.push_back({name, a, b});
  return e;
}

// ---------------------------------------------------------------------------------------------
// validation

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int validate(const idx_problem* p, int32_t k, const int32_t* out_idx, const float* out_score) {
  if (!p) return IDX_ERR_INVALID_ARG;
  if (p->B <= 0 || p->T <= 0 || p->H <= 0 || p->D <= 0 || p->N <= 0 || k <= 0)
    return IDX_ERR_INVALID_ARG;
  if (!p->q || !p->k || !p->w || !p->q_pos || !out_idx) return IDX_ERR_INVALID_ARG;
  if (p->q_dtype != IDX_F32 && p->q_dtype != IDX_BF16) return IDX_ERR_UNSUPPORTED;
  if (p->k_dtype != IDX_F32 && p->k_dtype != IDX_BF16 && p->k_dtype != IDX_FP8_E4M3)
    return IDX_ERR_UNSUPPORTED;
  if (p->k_dtype == IDX_FP8_E4M3 && !p->k_scale) return IDX_ERR_INVALID_ARG;
  if (!score_supported(p->q_dtype, p->k_dtype, p->H, p->D)) return IDX_ERR_UNSUPPORTED;
  if ((int64_t)p->B * p->T > (int64_t)INT32_MAX / 4 || (int64_t)p->B * p->N > (int64_t)INT32_MAX)
    return IDX_ERR_UNSUPPORTED;
  if (!aligned(p->q, 16) || !aligned(p->k, 16) || !aligned(p->w, 4) || !aligned(p->q_pos, 4) ||
      (p->k_len && !aligned(p->k_len, 4)) || (p->k_scale && !aligned(p->k_scale, 4)) ||
      !aligned(out_idx, 4) || (out_score && !aligned(out_score, 4)))
    return IDX_ERR_ALIGN;
  return IDX_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? IDX_OK : IDX_ERR_HIP; }

// ---------------------------------------------------------------------------------------------
// workspace plans

struct Carver {
  uint8_t* base;
  size_t off = 0;
  explicit Carver(void* p) : base(static_cast<uint8_t*>(p)) {}
  template <class T>
  T* take(size_t n) {
    T* r = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(n * sizeof(T));
    return r;
  }
};

int chunk_rows(int B, int64_t row_bytes, int rows) {
  int64_t c = (int64_t)kScoreBudget / std::max<int64_t>(1, (int64_t)B * row_bytes);
  c = std::max<int64_t>(1, std::min<int64_t>(c, rows));
  return (int)c;
}

// split of the key range so that a launch has about kTargetGroups work-groups
int key_split(int n_groups, int n_keys, int* split_keys) {
  int splits = 1;
  if (n_groups < kTargetGroups) splits = (kTargetGroups + n_groups - 1) / n_groups;
  int sk = (n_keys + splits - 1) / splits;
  sk = std::max(KEY_TILE * 4, (sk + KEY_TILE - 1) / KEY_TILE * KEY_TILE);
  *split_keys = sk;
  return (n_keys + sk - 1) / sk;
}

struct DensePlan {
  int chunkT;
  float* scores;
  int32_t* row_len;
  int32_t* meta;
  size_t bytes;
};

DensePlan plan_dense(const idx_problem* p, void* ws) {
  DensePlan d;
  Carver c(ws);
  d.chunkT = chunk_rows(p->B, rstride(p->N) * 4, p->T);
  d.scores = c.take<float>((size_t)p->B * d.chunkT * rstride(p->N));
  d.row_len = c.take<int32_t>((size_t)p->B * d.chunkT);
  d.meta = c.take<int32_t>((size_t)p->B * d.chunkT * 4);
  d.bytes = c.off + kAlign;
  return d;
}

struct ReusePlan {
  int NG, chunkP;
  void* pq;
  float* pw;
  int32_t* ppos;
  float* pscores;
  int32_t* gidx;
  float* gsc;
  int32_t* gcnt;
  int32_t* row_len;
  int32_t* meta;
  size_t bytes;
};

struct GroupBlockPlan {
  int NG, NB, chunkP, chunkG;
  void* pq;
  float* pw;
  int32_t* ppos;
  void* pooled;
  float* cscores;
  int32_t* blocks;
  int32_t* n_kept;
  int32_t* list;
  int32_t* cnt;
  float* mscores;
  int32_t* row_len;
  int32_t* meta;
  size_t bytes;
};

struct RefinePlan {
  int NG, chunkG;
  int32_t* list;
  int32_t* cnt;
  float* mscores;
  int32_t* row_len;
  int32_t* meta;
  size_t bytes;
};

struct GroupPlan {
  int NG, chunkP, chunkG;
  void* pq;
  float* pw;
  int32_t* ppos;
  float* pscores;
  int32_t* cand;
  int32_t* cand_cnt;
  float* mscores;
  int32_t* row_len;
  int32_t* meta;
  size_t bytes;
};

GroupPlan plan_group(const idx_problem* p, int G, int C, void* ws, int32_t* out_cand) {
  GroupPlan g;
  Carver c(ws);
  g.NG = (p->T + G - 1) / G;
  const size_t qeb = p->q_dtype == IDX_BF16 ? 2 : 4;
  g.pq = c.take<uint8_t>((size_t)p->B * g.NG * p->H * p->D * qeb);
  g.pw = c.take<float>((size_t)p->B * g.NG * p->H);
  g.ppos = c.take<int32_t>((size_t)p->B * g.NG);
  g.chunkP = chunk_rows(p->B, rstride(p->N) * 4, g.NG);
  g.pscores = c.take<float>((size_t)p->B * g.chunkP * rstride(p->N));
  g.cand = out_cand ? out_cand : c.take<int32_t>((size_t)p->B * g.NG * C);
  g.cand_cnt = c.take<int32_t>((size_t)p->B * g.NG);
  g.chunkG = chunk_rows(p->B, (int64_t)G * rstride(C) * 4, g.NG);
  g.mscores = c.take<float>((size_t)p->B * std::min(p->T, g.chunkG * G) * rstride(C));
  g.row_len = c.take<int32_t>((size_t)p->B * std::max(std::min(p->T, g.chunkG * G), g.chunkP));
  g.meta = c.take<int32_t>((size_t)p->B * std::max(std::min(p->T, g.chunkG * G), g.chunkP) * 4);
  g.bytes = c.off + kAlign;
  return g;
}

struct BlockPlan {
  int NB, chunkT1, chunkT2;
  void* pooled;
  float* cscores;
  int32_t* blocks;
  int32_t* n_kept;
  float* rscores;
  int32_t* row_len;
  int32_t* meta;
  size_t bytes;
};

BlockPlan plan_block(const idx_problem* p, int Bs, int keep, void* ws, int32_t* out_blocks) {
  BlockPlan b;
  Carver c(ws);
  b.NB = (p->N + Bs - 1) / Bs;
  const size_t keb = p->k_dtype == IDX_BF16 ? 2 : 4;
  b.pooled = c.take<uint8_t>((size_t)p->B * b.NB * p->D * keb);
  b.chunkT1 = chunk_rows(p->B, rstride(b.NB) * 4, p->T);
  b.cscores = c.take<float>((size_t)p->B * b.chunkT1 * rstride(b.NB));
  b.blocks = out_blocks ? out_blocks : c.take<int32_t>((size_t)p->B * p->T * keep);
  b.n_kept = c.take<int32_t>((size_t)p->B * p->T);
  b.chunkT2 = chunk_rows(p->B, rstride((int64_t)keep * Bs) * 4, p->T);
  b.rscores = c.take<float>((size_t)p->B * b.chunkT2 * rstride((int64_t)keep * Bs));
  b.row_len = c.take<int32_t>((size_t)p->B * std::max(b.chunkT1, b.chunkT2));
  b.meta = c.take<int32_t>((size_t)p->B * std::max(b.chunkT1, b.chunkT2) * 4);
  b.bytes = c.off + kAlign;
  return b;
}

// Decode-shaped problems (few queries per sequence over a long cache) take the streaming path.
bool use_decode(const idx_problem* p) {
  return decode_supported(p->q_dtype, p->k_dtype, p->H, p->D, p->T, p->N);
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

struct DecodePlan {
  int nchunk, chunk, sub, nsegs, cand_cap;
  uint32_t* ccount;
  uint32_t* shist;
  uint32_t* cand_key;
  uint32_t* cand_idx;
  uint32_t* cand2_key;
  uint32_t* cand2_idx;
  size_t bytes;
};

DecodePlan plan_decode(const idx_problem* p, void* ws) {
  DecodePlan d;
  Carver c(ws);
  const int64_t rows = (int64_t)p->B * p->T;
  const int pairs = (p->T + 1) / 2;
  // about one scan work-group per compute unit (each holds a whole unit's LDS), chunks of at
  // least 1024 keys
  int nchunk = std::max(1, (cu_count() + p->B * pairs - 1) / (p->B * pairs));
  int chunk = (int)std::max<int64_t>(1024, ((int64_t)p->N + nchunk - 1) / nchunk);
  chunk = (chunk + 63) / 64 * 64;
  if (chunk > DECODE_SUB) chunk = (chunk + DECODE_SUB - 1) / DECODE_SUB * DECODE_SUB;
  d.chunk = chunk;
  d.nchunk = (p->N + chunk - 1) / chunk;
  d.sub = std::min(chunk, DECODE_SUB);
  d.nsegs = (p->N + d.sub - 1) / d.sub;
  d.cand_cap = (int)rstride(p->N);
  d.ccount = c.take<uint32_t>((size_t)rows * d.nsegs);
  d.shist = c.take<uint32_t>((size_t)rows * d.nsegs * (DECODE_BINS / 2));
  d.cand_key = c.take<uint32_t>((size_t)rows * d.cand_cap);
  d.cand_idx = c.take<uint32_t>((size_t)rows * d.cand_cap);
  d.cand2_key = c.take<uint32_t>((size_t)rows * d.cand_cap);
  d.cand2_idx = c.take<uint32_t>((size_t)rows * d.cand_cap);
  d.bytes = c.off + kAlign;
  return d;
}

void* align_ws(void* ws) {
  uintptr_t u = reinterpret_cast<uintptr_t>(ws);
  return reinterpret_cast<void*>((u + kAlign - 1) / kAlign * kAlign);
}

// ---------------------------------------------------------------------------------------------
// shared launch helpers

ScoreArgs base_score_args(const idx_problem* p) {
  ScoreArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = p->q; a.q_dtype = p->q_dtype; a.w = p->w; a.q_pos = p->q_pos;
  a.keys = p->k; a.k_dtype = p->k_dtype; a.k_scale = p->k_scale; a.k_len = p->k_len;
  a.B = p->B; a.T = p->T; a.H = p->H; a.D = p->D;
  a.key_cap = p->N; a.tok_cap = p->N;
  a.mode = MODE_RANGE; a.pos_stride = 1; a.count_div = 1;
  return a;
}

// Launches the score kernel; when the key range is not split, the kernel also writes each row's
// selection summary into `meta` for the selector, and *fused is set.
hipError_t run_score(ScoreArgs& a, int n_keys_max, int topk_k, int32_t* meta, bool* fused,
                     hipStream_t s) {
  const int qt = score_queries_per_tile(a.H);
  if (a.mode == MODE_RANGE) {
    a.tiles_per_seq = (a.c1 - a.c0 + qt - 1) / qt;
  } else {
    a.tiles_per_seq = (a.c1 - a.c0) * ((a.group_size + qt - 1) / qt);
  }
  const int nsplit = key_split(a.B * a.tiles_per_seq, n_keys_max, &a.split_keys);
  *fused = nsplit == 1 && meta != nullptr;
  a.row_meta = *fused ? meta : nullptr;
  a.topk_k = topk_k;
  a.digit_bits = n_keys_max < 65536 ? 12 : 11;
  return timed("score", s, [&] { return launch_score(a, nsplit, s); });
}

hipError_t run_topk(TopkArgs& t, int max_row_len, hipStream_t s) {
  return timed("topk", s, [&] { return launch_topk(t, max_row_len, s); });
}

TopkArgs topk_args(const float* scores, int64_t stride, const int32_t* row_len, int n_rows, int k,
                   int rows_per_seq, int T_out, int t_off, int32_t* out_idx, float* out_score,
                   int out_stride) {
  TopkArgs t;
  std::memset(&t, 0, sizeof(t));
  t.scores = scores; t.score_stride = stride; t.row_len = row_len; t.n_rows = n_rows; t.k = k;
  t.rows_per_seq = rows_per_seq; t.T_out = T_out; t.t_off = t_off;
  t.out_idx = out_idx; t.out_score = out_score; t.out_stride = out_stride;
  t.map_mode = MAP_IDENT;
  return t;
}

// ---------------------------------------------------------------------------------------------
// entry points

int decode_impl(const idx_problem* p, int32_t k, int32_t* out_idx, float* out_score, void* ws,
                size_t ws_bytes, hipStream_t s) {
  DecodePlan pl = plan_decode(p, nullptr);
  if (!ws || ws_bytes < pl.bytes) return IDX_ERR_WORKSPACE;
  pl = plan_decode(p, align_ws(ws));
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = p->q; a.w = p->w; a.q_pos = p->q_pos;
  a.keys = p->k; a.k_dtype = p->k_dtype; a.k_scale = p->k_scale; a.k_len = p->k_len;
  a.B = p->B; a.T = p->T; a.H = p->H; a.D = p->D; a.N = p->N;
  a.nchunk = pl.nchunk; a.chunk = pl.chunk; a.sub = pl.sub;
  a.ccount = pl.ccount; a.nsegs = pl.nsegs; a.shist = pl.shist;
  a.cand_key = pl.cand_key; a.cand_idx = pl.cand_idx;
  a.cand2_key = pl.cand2_key; a.cand2_idx = pl.cand2_idx; a.cand_cap = pl.cand_cap;
  a.k = k;
  a.out_idx = out_idx; a.out_score = out_score;
  int st;
  if ((st = from_hip(timed("decode_scan", s, [&] { return launch_decode_scan(a, s); })))) return st;
  return from_hip(timed("decode_select", s, [&] { return launch_decode_select(a, s); }));
}

int score_topk_impl(const idx_problem* p, int32_t k, int32_t* out_idx, float* out_score,
                    void* ws, size_t ws_bytes, hipStream_t s) {
  int st = validate(p, k, out_idx, out_score);
  if (st) return st;
  if (use_decode(p)) return decode_impl(p, k, out_idx, out_score, ws, ws_bytes, s);
  DensePlan pl = plan_dense(p, nullptr);
  if (!ws || ws_bytes < pl.bytes) return IDX_ERR_WORKSPACE;
  pl = plan_dense(p, align_ws(ws));
  for (int c0 = 0; c0 < p->T; c0 += pl.chunkT) {
    const int c1 = std::min(p->T, c0 + pl.chunkT);
    ScoreArgs a = base_score_args(p);
    a.c0 = c0; a.c1 = c1;
    a.scores = pl.scores; a.score_stride = rstride(p->N); a.row_len = pl.row_len;
    a.rows_per_seq = c1 - c0;
    // bf16 rows shorter than 64K slots: each score-kernel wave selects its own row
    const bool self_select = p->q_dtype == IDX_BF16 && p->k_dtype == IDX_BF16 && p->N < 65536;
    if (self_select) {
      a.sel_idx = out_idx; a.sel_score = out_score; a.sel_T = p->T;
    }
    bool fused;
    if ((st = from_hip(run_score(a, p->N, k, pl.meta, &fused, s)))) return st;
    if (fused && self_select) continue;
    TopkArgs t = topk_args(pl.scores, rstride(p->N), pl.row_len, p->B * (c1 - c0), k, c1 - c0, p->T, c0,
                           out_idx, out_score, k);
    t.row_meta = fused ? pl.meta : nullptr;
    t.digit_bits = a.digit_bits;
    if ((st = from_hip(run_topk(t, p->N, s)))) return st;
  }
  return IDX_OK;
}

// Per-query refine over per-group candidate lists (rows of C token ids in ascending order, the
// first cnt[b * NG + g] used): members t of group g score the list's tokens inside their own
// prefix (LIST mode of the score kernel) and keep their top k, mapped back to tokens.
int refine_lists(const idx_problem* p, int32_t k, int G, int C, int NG, int chunkG, const int32_t* list,
                 const int32_t* cnt, float* mscores, int32_t* row_len, int32_t* meta, int32_t* out_idx,
                 float* out_score, hipStream_t s) {
  int st;
  for (int g0 = 0; g0 < NG; g0 += chunkG) {
    const int g1 = std::min(NG, g0 + chunkG);
    const int rows = std::min(p->T, g1 * G) - g0 * G;
    ScoreArgs a = base_score_args(p);
    a.mode = MODE_LIST;
    a.list = list; a.list_len = cnt; a.list_stride = C; a.group_size = G;
    a.n_groups = NG;
    a.c0 = g0; a.c1 = g1;
    a.scores = mscores; a.score_stride = rstride(C); a.row_len = row_len;
    a.rows_per_seq = rows;
    bool fused;
    if ((st = from_hip(run_score(a, C, k, meta, &fused, s)))) return st;
    TopkArgs t = topk_args(mscores, rstride(C), row_len, p->B * rows, k, rows, p->T, g0 * G, out_idx,
                           out_score, k);
    t.row_meta = fused ? meta : nullptr;
    t.digit_bits = a.digit_bits;
    t.map_mode = MAP_LIST;
    t.list = list; t.list_stride = C; t.group_size = G; t.n_groups = NG;
    if ((st = from_hip(run_topk(t, C, s)))) return st;
  }
  return IDX_OK;
}

int group_impl(const idx_problem* p, int32_t k, int32_t G, int32_t C, int32_t* out_idx,
               float* out_score, int32_t* out_cand, void* ws, size_t ws_bytes, hipStream_t s) {
  int st = validate(p, k, out_idx, out_score);
  if (st) return st;
  if (G < 1 || C < 1 || C > p->N) return IDX_ERR_INVALID_ARG;
  if (out_cand && !aligned(out_cand, 4)) return IDX_ERR_ALIGN;
  GroupPlan pl = plan_group(p, G, C, nullptr, out_cand);
  if (!ws || ws_bytes < pl.bytes) return IDX_ERR_WORKSPACE;
  pl = plan_group(p, G, C, align_ws(ws), out_cand);

  ProxyArgs pa;
  pa.q = p->q; pa.q_dtype = p->q_dtype; pa.w = p->w; pa.q_pos = p->q_pos;
  pa.B = p->B; pa.T = p->T; pa.H = p->H; pa.D = p->D; pa.G = G; pa.n_groups = pl.NG;
  pa.pq = pl.pq; pa.pw = pl.pw; pa.ppos = pl.ppos;
  if ((st = from_hip(timed("proxy", s, [&] { return launch_proxy(pa, s); })))) return st;

  // proxy scans and candidate sets
  for (int c0 = 0; c0 < pl.NG; c0 += pl.chunkP) {
    const int c1 = std::min(pl.NG, c0 + pl.chunkP);
    ScoreArgs a = base_score_args(p);
    a.q = pl.pq; a.w = pl.pw; a.q_pos = pl.ppos; a.T = pl.NG;
    a.c0 = c0; a.c1 = c1;
    a.scores = pl.pscores; a.score_stride = rstride(p->N); a.row_len = pl.row_len;
    a.rows_per_seq = c1 - c0;
    bool fused;
    if ((st = from_hip(run_score(a, p->N, C, pl.meta, &fused, s)))) return st;
    TopkArgs t = topk_args(pl.pscores, rstride(p->N), pl.row_len, p->B * (c1 - c0), C, c1 - c0, pl.NG, c0,
                           pl.cand, nullptr, C);
    t.out_count = pl.cand_cnt;
    t.row_meta = fused ? pl.meta : nullptr;
    t.digit_bits = a.digit_bits;
    if ((st = from_hip(run_topk(t, p->N, s)))) return st;
  }
  // candidate lists in ascending token order (the refine indexes them by slot)
  if ((st = from_hip(timed("sort", s, [&] {
         return launch_sort_rows(pl.cand, C, pl.cand_cnt, p->B * pl.NG, C, p->N, s);
       }))))
    return st;
  return refine_lists(p, k, G, C, pl.NG, pl.chunkG, pl.cand, pl.cand_cnt, pl.mscores, pl.row_len,
                      pl.meta, out_idx, out_score, s);
}

ReusePlan plan_reuse(const idx_problem* p, int G, int k, void* ws) {
  ReusePlan g;
  Carver c(ws);
  g.NG = (p->T + G - 1) / G;
  const size_t qeb = p->q_dtype == IDX_BF16 ? 2 : 4;
  g.pq = c.take<uint8_t>((size_t)p->B * g.NG * p->H * p->D * qeb);
  g.pw = c.take<float>((size_t)p->B * g.NG * p->H);
  g.ppos = c.take<int32_t>((size_t)p->B * g.NG);
  g.chunkP = chunk_rows(p->B, rstride(p->N) * 4, g.NG);
  g.pscores = c.take<float>((size_t)p->B * g.chunkP * rstride(p->N));
  g.gidx = c.take<int32_t>((size_t)p->B * g.NG * k);
  g.gsc = c.take<float>((size_t)p->B * g.NG * k);
  g.gcnt = c.take<int32_t>((size_t)p->B * g.NG);
  g.row_len = c.take<int32_t>((size_t)p->B * g.chunkP);
  g.meta = c.take<int32_t>((size_t)p->B * g.chunkP * 4);
  g.bytes = c.off + kAlign;
  return g;
}

// PIVOT-Reuse: the proxies' prefix scans keep each group's top k (tokens and proxy scores), and
// every member takes the part of it inside its own prefix.
int reuse_impl(const idx_problem* p, int32_t k, int32_t G, int32_t* out_idx, float* out_score,
               void* ws, size_t ws_bytes, hipStream_t s) {
  int st = validate(p, k, out_idx, out_score);
  if (st) return st;
  if (G < 1) return IDX_ERR_INVALID_ARG;
  ReusePlan pl = plan_reuse(p, G, k, nullptr);
  if (!ws || ws_bytes < pl.bytes) return IDX_ERR_WORKSPACE;
  pl = plan_reuse(p, G, k, align_ws(ws));

  ProxyArgs pa;
  pa.q = p->q; pa.q_dtype = p->q_dtype; pa.w = p->w; pa.q_pos = p->q_pos;
  pa.B = p->B; pa.T = p->T; pa.H = p->H; pa.D = p->D; pa.G = G; pa.n_groups = pl.NG;
  pa.pq = pl.pq; pa.pw = pl.pw; pa.ppos = pl.ppos;
  if ((st = from_hip(timed("proxy", s, [&] { return launch_proxy(pa, s); })))) return st;
  for (int c0 = 0; c0 < pl.NG; c0 += pl.chunkP) {
    const int c1 = std::min(pl.NG, c0 + pl.chunkP);
    ScoreArgs a = base_score_args(p);
    a.q = pl.pq; a.w = pl.pw; a.q_pos = pl.ppos; a.T = pl.NG;
    a.c0 = c0; a.c1 = c1;
    a.scores = pl.pscores; a.score_stride = rstride(p->N); a.row_len = pl.row_len;
    a.rows_per_seq = c1 - c0;
    bool fused;
    if ((st = from_hip(run_score(a, p->N, k, pl.meta, &fused, s)))) return st;
    TopkArgs t = topk_args(pl.pscores, rstride(p->N), pl.row_len, p->B * (c1 - c0), k, c1 - c0, pl.NG, c0,
                           pl.gidx, pl.gsc, k);
    t.out_count = pl.gcnt;
    t.row_meta = fused ? pl.meta : nullptr;
    t.digit_bits = a.digit_bits;
    if ((st = from_hip(run_topk(t, p->N, s)))) return st;
  }
  ReuseArgs r;
  r.gidx = pl.gidx; r.gsc = pl.gsc; r.gcnt = pl.gcnt;
  r.q_pos = p->q_pos; r.k_len = p->k_len;
  r.B = p->B; r.T = p->T; r.N = p->N; r.G = G; r.NG = pl.NG; r.k = k;
  r.out_idx = out_idx; r.out_score = out_score;
  return from_hip(timed("reuse", s, [&] { return launch_reuse_rows(r, s); }));
}

GroupBlockPlan plan_group_block(const idx_problem* p, int G, int Bs, int keep, void* ws,
                                int32_t* out_blocks) {
  GroupBlockPlan g;
  Carver c(ws);
  g.NG = (p->T + G - 1) / G;
  g.NB = (p->N + Bs - 1) / Bs;
  const int C = keep * Bs;
  const size_t qeb = p->q_dtype == IDX_BF16 ? 2 : 4;
  const size_t keb = p->k_dtype == IDX_BF16 ? 2 : 4;
  g.pq = c.take<uint8_t>((size_t)p->B * g.NG * p->H * p->D * qeb);
  g.pw = c.take<float>((size_t)p->B * g.NG * p->H);
  g.ppos = c.take<int32_t>((size_t)p->B * g.NG);
  g.pooled = c.take<uint8_t>((size_t)p->B * g.NB * p->D * keb);
  g.chunkP = chunk_rows(p->B, rstride(g.NB) * 4, g.NG);
  g.cscores = c.take<float>((size_t)p->B * g.chunkP * rstride(g.NB));
  g.blocks = out_blocks ? out_blocks : c.take<int32_t>((size_t)p->B * g.NG * keep);
  g.n_kept = c.take<int32_t>((size_t)p->B * g.NG);
  g.list = c.take<int32_t>((size_t)p->B * g.NG * C);
  g.cnt = c.take<int32_t>((size_t)p->B * g.NG);
  g.chunkG = chunk_rows(p->B, (int64_t)G * rstride(C) * 4, g.NG);
  const int rows = std::max(std::min(p->T, g.chunkG * G), g.chunkP);
  g.mscores = c.take<float>((size_t)p->B * std::min(p->T, g.chunkG * G) * rstride(C));
  g.row_len = c.take<int32_t>((size_t)p->B * rows);
  g.meta = c.take<int32_t>((size_t)p->B * rows * 4);
  g.bytes = c.off + kAlign;
  return g;
}

// Block-filtered group proxy: each group's proxy scores the pooled blocks of its prefix and
// keeps `keep` of them; every member refines the tokens of the kept blocks.
int group_block_impl(const idx_problem* p, int32_t k, int32_t G, int32_t Bs, int32_t keep,
                     int32_t* out_idx, float* out_score, int32_t* out_blocks, void* ws, size_t ws_bytes,
                     hipStream_t s) {
  int st = validate(p, k, out_idx, out_score);
  if (st) return st;
  if (G < 1 || Bs < 1 || keep < 1) return IDX_ERR_INVALID_ARG;
  if (p->k_dtype == IDX_FP8_E4M3) return IDX_ERR_UNSUPPORTED;
  if ((p->N + (int64_t)Bs - 1) / Bs > 65536 || keep > 32767) return IDX_ERR_UNSUPPORTED;
  if ((int64_t)keep * Bs > (int64_t)INT32_MAX / 4) return IDX_ERR_UNSUPPORTED;
  if (out_blocks && !aligned(out_blocks, 4)) return IDX_ERR_ALIGN;
  GroupBlockPlan pl = plan_group_block(p, G, Bs, keep, nullptr, out_blocks);
  if (!ws || ws_bytes < pl.bytes) return IDX_ERR_WORKSPACE;
  pl = plan_group_block(p, G, Bs, keep, align_ws(ws), out_blocks);

  ProxyArgs pa;
  pa.q = p->q; pa.q_dtype = p->q_dtype; pa.w = p->w; pa.q_pos = p->q_pos;
  pa.B = p->B; pa.T = p->T; pa.H = p->H; pa.D = p->D; pa.G = G; pa.n_groups = pl.NG;
  pa.pq = pl.pq; pa.pw = pl.pw; pa.ppos = pl.ppos;
  if ((st = from_hip(timed("proxy", s, [&] { return launch_proxy(pa, s); })))) return st;
  PoolArgs po;
  po.keys = p->k; po.k_dtype = p->k_dtype; po.k_len = p->k_len;
  po.B = p->B; po.N = p->N; po.D = p->D; po.block_size = Bs; po.n_blocks = pl.NB;
  po.pooled = pl.pooled;
  if ((st = from_hip(timed("pool", s, [&] { return launch_pool(po, s); })))) return st;
  // coarse: the proxies against the pooled blocks, block j sits at position j * Bs
  for (int c0 = 0; c0 < pl.NG; c0 += pl.chunkP) {
    const int c1 = std::min(pl.NG, c0 + pl.chunkP);
    ScoreArgs a = base_score_args(p);
    a.q = pl.pq; a.w = pl.pw; a.q_pos = pl.ppos; a.T = pl.NG;
    a.keys = pl.pooled; a.k_scale = nullptr; a.key_cap = pl.NB;
    a.pos_stride = Bs; a.count_div = Bs;
    a.c0 = c0; a.c1 = c1;
    a.scores = pl.cscores; a.score_stride = rstride(pl.NB); a.row_len = pl.row_len;
    a.rows_per_seq = c1 - c0;
    bool fused;
    if ((st = from_hip(run_score(a, pl.NB, keep, pl.meta, &fused, s)))) return st;
    TopkArgs t = topk_args(pl.cscores, rstride(pl.NB), pl.row_len, p->B * (c1 - c0), keep, c1 - c0, pl.NG,
                           c0, pl.blocks, nullptr, keep);
    t.out_count = pl.n_kept;
    t.row_meta = fused ? pl.meta : nullptr;
    t.digit_bits = a.digit_bits;
    if ((st = from_hip(run_topk(t, pl.NB, s)))) return st;
  }
  if ((st = from_hip(timed("sort", s, [&] {
         return launch_sort_rows(pl.blocks, keep, pl.n_kept, p->B * pl.NG, keep, pl.NB, s);
       }))))
    return st;
  const int C = keep * Bs;
  if ((st = from_hip(timed("sort", s, [&] {
         return launch_expand_blocks(pl.blocks, pl.n_kept, keep, Bs, p->N, p->k_len, pl.NG, pl.list, pl.cnt,
                                     p->B * pl.NG, s);
       }))))
    return st;
  return refine_lists(p, k, G, C, pl.NG, pl.chunkG, pl.list, pl.cnt, pl.mscores, pl.row_len, pl.meta,
                      out_idx, out_score, s);
}

RefinePlan plan_refine(const idx_problem* p, int G, int C, void* ws) {
  RefinePlan g;
  Carver c(ws);
  g.NG = (p->T + G - 1) / G;
  g.list = c.take<int32_t>((size_t)p->B * g.NG * C);
  g.cnt = c.take<int32_t>((size_t)p->B * g.NG);
  g.chunkG = chunk_rows(p->B, (int64_t)G * rstride(C) * 4, g.NG);
  const int rows = std::min(p->T, g.chunkG * G);
  g.mscores = c.take<float>((size_t)p->B * rows * rstride(C));
  g.row_len = c.take<int32_t>((size_t)p->B * rows);
  g.meta = c.take<int32_t>((size_t)p->B * rows * 4);
  g.bytes = c.off + kAlign;
  return g;
}

int refine_impl(const idx_problem* p, int32_t k, int32_t G, int32_t C, const int32_t* cand,
                const int32_t* cand_cnt, int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                hipStream_t s) {
  int st = validate(p, k, out_idx, out_score);
  if (st) return st;
  if (G < 1 || C < 1 || !cand) return IDX_ERR_INVALID_ARG;
  if (!aligned(cand, 4) || (cand_cnt && !aligned(cand_cnt, 4))) return IDX_ERR_ALIGN;
  if (p->N > 32768 * 32) return IDX_ERR_UNSUPPORTED;  // the set is built in an LDS bitmap of N bits
  RefinePlan pl = plan_refine(p, G, C, nullptr);
  if (!ws || ws_bytes < pl.bytes) return IDX_ERR_WORKSPACE;
  pl = plan_refine(p, G, C, align_ws(ws));
  // the caller's lists as ascending sets of token ids (the refine indexes them by slot)
  if ((st = from_hip(timed("sort", s, [&] {
         return launch_given_lists(cand, cand_cnt, C, p->N, p->k_len, pl.NG, pl.list, pl.cnt, p->B * pl.NG, s);
       }))))
    return st;
  return refine_lists(p, k, G, C, pl.NG, pl.chunkG, pl.list, pl.cnt, pl.mscores, pl.row_len, pl.meta,
                      out_idx, out_score, s);
}

int block_impl(const idx_problem* p, int32_t k, int32_t Bs, int32_t keep, int32_t* out_idx,
               float* out_score, int32_t* out_blocks, void* ws, size_t ws_bytes, hipStream_t s) {
  int st = validate(p, k, out_idx, out_score);
  if (st) return st;
  if (Bs < 1 || keep < 1) return IDX_ERR_INVALID_ARG;
  if (p->k_dtype == IDX_FP8_E4M3) return IDX_ERR_UNSUPPORTED;
  if ((p->N + (int64_t)Bs - 1) / Bs > 65536 || keep > 32767) return IDX_ERR_UNSUPPORTED;
  if ((int64_t)keep * Bs > (int64_t)INT32_MAX / 4) return IDX_ERR_UNSUPPORTED;
  if (out_blocks && !aligned(out_blocks, 4)) return IDX_ERR_ALIGN;
  BlockPlan pl = plan_block(p, Bs, keep, nullptr, out_blocks);
  if (!ws || ws_bytes < pl.bytes) return IDX_ERR_WORKSPACE;
  pl = plan_block(p, Bs, keep, align_ws(ws), out_blocks);

  PoolArgs po;
  po.keys = p->k; po.k_dtype = p->k_dtype; po.k_len = p->k_len;
  po.B = p->B; po.N = p->N; po.D = p->D; po.block_size = Bs; po.n_blocks = pl.NB;
  po.pooled = pl.pooled;
  if ((st = from_hip(timed("pool", s, [&] { return launch_pool(po, s); })))) return st;

  // coarse: pooled blocks, block j sits at position j * Bs
  for (int c0 = 0; c0 < p->T; c0 += pl.chunkT1) {
    const int c1 = std::min(p->T, c0 + pl.chunkT1);
    ScoreArgs a = base_score_args(p);
    a.keys = pl.pooled; a.k_scale = nullptr; a.key_cap = pl.NB;
    a.pos_stride = Bs; a.count_div = Bs;
    a.c0 = c0; a.c1 = c1;
    a.scores = pl.cscores; a.score_stride = rstride(pl.NB); a.row_len = pl.row_len;
    a.rows_per_seq = c1 - c0;
    bool fused;
    if ((st = from_hip(run_score(a, pl.NB, keep, pl.meta, &fused, s)))) return st;
    TopkArgs t = topk_args(pl.cscores, rstride(pl.NB), pl.row_len, p->B * (c1 - c0), keep, c1 - c0, p->T,
                           c0, pl.blocks, nullptr, keep);
    t.out_count = pl.n_kept;
    t.row_meta = fused ? pl.meta : nullptr;
    t.digit_bits = a.digit_bits;
    if ((st = from_hip(run_topk(t, pl.NB, s)))) return st;
  }
  if ((st = from_hip(timed("sort", s, [&] {
         return launch_sort_rows(pl.blocks, keep, pl.n_kept, p->B * p->T, keep, pl.NB, s);
       }))))
    return st;
  // token refine inside the kept blocks
  const int qt = score_queries_per_tile(p->H);
  for (int c0 = 0; c0 < p->T; c0 += pl.chunkT2) {
    const int c1 = std::min(p->T, c0 + pl.chunkT2);
    BlockRefineArgs r;
    r.q = p->q; r.q_dtype = p->q_dtype; r.w = p->w; r.q_pos = p->q_pos;
    r.keys = p->k; r.k_dtype = p->k_dtype; r.k_len = p->k_len;
    r.B = p->B; r.T = p->T; r.H = p->H; r.D = p->D; r.N = p->N;
    r.blocks = pl.blocks; r.n_kept = pl.n_kept; r.keep_stride = keep; r.block_size = Bs;
    r.t0 = c0; r.t1 = c1;
    r.scores = pl.rscores; r.score_stride = rstride((int64_t)keep * Bs);
    r.row_len = pl.row_len; r.rows_per_seq = c1 - c0;
    r.row_meta = nullptr; r.topk_k = k;
    r.tiles_per_seq = (c1 - c0 + qt - 1) / qt;
    if ((st = from_hip(timed("block_refine", s, [&] { return launch_block_refine(r, s); }))))
      return st;
    TopkArgs t = topk_args(pl.rscores, rstride((int64_t)keep * Bs), pl.row_len, p->B * (c1 - c0), k,
                           c1 - c0, p->T, c0, out_idx, out_score, k);
    t.map_mode = MAP_BLOCKS;
    t.blocks = pl.blocks; t.blocks_stride = keep; t.block_size = Bs;
    if ((st = from_hip(run_topk(t, keep * Bs, s)))) return st;
  }
  return IDX_OK;
}

}  // namespace
}  // namespace idx

using namespace idx;

extern "C" {

int idx_score_topk(const idx_problem* p, int32_t k, int32_t* out_idx, float* out_score, void* ws,
                   size_t ws_bytes, void* stream) {
  try {
    return score_topk_impl(p, k, out_idx, out_score, ws, ws_bytes,
                           static_cast<hipStream_t>(stream));
  } catch (...) {
    return IDX_ERR_INTERNAL;
  }
}

int idx_group_proxy_refine(const idx_problem* p, int32_t k, int32_t group_size, int32_t n_cand,
                           int32_t* out_idx, float* out_score, int32_t* out_cand, void* ws,
                           size_t ws_bytes, void* stream) {
  try {
    return group_impl(p, k, group_size, n_cand, out_idx, out_score, out_cand, ws, ws_bytes,
                      static_cast<hipStream_t>(stream));
  } catch (...) {
    return IDX_ERR_INTERNAL;
  }
}

int idx_block_coarse_refine(const idx_problem* p, int32_t k, int32_t block_size,
                            int32_t n_blocks_keep, int32_t* out_idx, float* out_score,
                            int32_t* out_blocks, void* ws, size_t ws_bytes, void* stream) {
  try {
    return block_impl(p, k, block_size, n_blocks_keep, out_idx, out_score, out_blocks, ws,
                      ws_bytes, static_cast<hipStream_t>(stream));
  } catch (...) {
    return IDX_ERR_INTERNAL;
  }
}

int idx_group_proxy_reuse(const idx_problem* p, int32_t k, int32_t group_size, int32_t* out_idx,
                          float* out_score, void* ws, size_t ws_bytes, void* stream) {
  try {
    return reuse_impl(p, k, group_size, out_idx, out_score, ws, ws_bytes,
                      static_cast<hipStream_t>(stream));
  } catch (...) {
    return IDX_ERR_INTERNAL;
  }
}

int idx_group_block_refine(const idx_problem* p, int32_t k, int32_t group_size, int32_t block_size,
                           int32_t n_blocks_keep, int32_t* out_idx, float* out_score,
                           int32_t* out_blocks, void* ws, size_t ws_bytes, void* stream) {
  try {
    return group_block_impl(p, k, group_size, block_size, n_blocks_keep, out_idx, out_score, out_blocks, ws,
                            ws_bytes, static_cast<hipStream_t>(stream));
  } catch (...) {
    return IDX_ERR_INTERNAL;
  }
}

size_t idx_group_block_workspace_bytes(const idx_problem* p, int32_t k, int32_t group_size,
                                       int32_t block_size, int32_t n_blocks_keep) {
  try {
    if (!p || p->B <= 0 || p->T <= 0 || p->H <= 0 || p->D <= 0 || p->N <= 0 || k <= 0) return 0;
    if (group_size < 1 || block_size < 1 || n_blocks_keep < 1) return 0;
    if ((int64_t)n_blocks_keep * block_size > (int64_t)INT32_MAX / 4) return 0;
    return plan_group_block(p, group_size, block_size, n_blocks_keep, nullptr, nullptr).bytes;
  } catch (...) {
  }
  return 0;
}

int idx_refine_given(const idx_problem* p, int32_t k, int32_t group_size, const int32_t* cand,
                     const int32_t* cand_cnt, int32_t n_cand, int32_t* out_idx, float* out_score,
                     void* ws, size_t ws_bytes, void* stream) {
  try {
    return refine_impl(p, k, group_size, n_cand, cand, cand_cnt, out_idx, out_score, ws, ws_bytes,
                       static_cast<hipStream_t>(stream));
  } catch (...) {
    return IDX_ERR_INTERNAL;
  }
}

size_t idx_workspace_bytes(int op, const idx_problem* p, int32_t k, int32_t p1, int32_t p2) {
  try {
    if (!p || p->B <= 0 || p->T <= 0 || p->H <= 0 || p->D <= 0 || p->N <= 0 || k <= 0) return 0;
    if (op == IDX_OP_SCORE_TOPK)
      return use_decode(p) ? plan_decode(p, nullptr).bytes : plan_dense(p, nullptr).bytes;
    if (op == IDX_OP_GROUP) {
      if (p1 < 1 || p2 < 1) return 0;
      return plan_group(p, p1, p2, nullptr, nullptr).bytes;
    }
    if (op == IDX_OP_BLOCK) {
      if (p1 < 1 || p2 < 1) return 0;
      return plan_block(p, p1, p2, nullptr, nullptr).bytes;
    }
    if (op == IDX_OP_REUSE) {
      if (p1 < 1) return 0;
      return plan_reuse(p, p1, k, nullptr).bytes;
    }
    if (op == IDX_OP_REFINE) {
      if (p1 < 1 || p2 < 1) return 0;
      return plan_refine(p, p1, p2, nullptr).bytes;
    }
  } catch (...) {
  }
  return 0;
}

const char* idx_strerror(int status) {
  switch (status) {
    case IDX_OK: return "ok";
    case IDX_ERR_INVALID_ARG: return "invalid argument";
    case IDX_ERR_UNSUPPORTED: return "unsupported dtype/shape combination";
    case IDX_ERR_ALIGN: return "misaligned pointer";
    case IDX_ERR_WORKSPACE: return "workspace missing or too small";
    case IDX_ERR_HIP: return "HIP launch error";
    case IDX_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

int idx_timer_enable(int on) {
  try {
    for (auto& r : g_recs) {
      g_event_pool.push_back(r.a);
      g_event_pool.push_back(r.b);
    }
    g_recs.clear();
    g_timer_on = on != 0;
    return IDX_OK;
  } catch (...) {
    return IDX_ERR_INTERNAL;
  }
}

int idx_timer_read(const char* kernel_substr, double* total_ms, int32_t* launches) {
  try {
    double tot = 0.0;
    int32_t n = 0;
    int st = IDX_OK;
    for (auto& r : g_recs) {
      if (kernel_substr && kernel_substr[0] && !std::strstr(r.name, kernel_substr)) continue;
      if (hipEventSynchronize(r.b) != hipSuccess) { st = IDX_ERR_HIP; continue; }
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) { st = IDX_ERR_HIP; continue; }
      tot += ms;
      ++n;
    }
    if (total_ms) *total_ms = tot;
    if (launches) *launches = n;
    return st;
  } catch (...) {
    return IDX_ERR_INTERNAL;
  }
}

}  // extern "C"
