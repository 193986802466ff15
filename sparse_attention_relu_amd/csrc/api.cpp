// C-ABI entry points of libdsa.so: host-side validation, workspace carving
// and kernel launches. Every argument is checked before anything is
// launched; on an error nothing is written and dsa_last_error() says why.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/dsa.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return DSA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxCap = 1 << 24;  // positions per sequence (MP * PS)

long scores_ld(int MP, int PS) { return (((long)MP * PS) + 63) / 64 * 64; }

long pages_ld(int MP) { return ((long)MP + 63) / 64 * 64; }

int check_ragged(int T, int S, int PS, int MP, int num_pages) {
  if (T < 0) return fail(DSA_ERR_INVALID_ARG, "T=%d must be >= 0", T);
  if (S < 0) return fail(DSA_ERR_INVALID_ARG, "S=%d must be >= 0", S);
  if (PS < 1 || PS > 4096) return fail(DSA_ERR_INVALID_ARG, "PS=%d out of [1, 4096]", PS);
  if (MP < 1) return fail(DSA_ERR_INVALID_ARG, "MP=%d must be >= 1", MP);
  if ((long)MP * PS > kMaxCap)
    return fail(DSA_ERR_UNSUPPORTED, "MP*PS=%ld exceeds %d positions", (long)MP * PS, kMaxCap);
  if (num_pages < 1) return fail(DSA_ERR_INVALID_ARG, "num_pages=%d must be >= 1", num_pages);
  return DSA_OK;
}

// The fused indexer path (scores never stored) replaces the score matrix
// when it would exceed this many bytes for a batch of query chunks.
constexpr size_t kMaterializeMax = size_t(256) << 20;

size_t fused_ws(int T, int MP, int PS, int k) {
  int G = 1, L = 0, C = 0;
  dsa::fused_plan(T, MP * PS, k, &G, &L, &C);
  return align256((size_t)T * G * C * 8) + align256((size_t)T * G * 4);
}

bool use_fused(int T, int MP, int PS, int max_q_len) {
  return max_q_len > 1 && (size_t)T * scores_ld(MP, PS) * 4 > kMaterializeMax;
}

size_t decode_ws(int T, int H, int k) {
  const int ch = dsa::mla_decode_chunk(T, k);
  const size_t nch = (size_t)((k + ch - 1) / ch);
  if (nch == 1) return 0;  // one chunk per row: the kernel writes the output itself
  return align256((size_t)T * nch * H * 512 * 2) + align256((size_t)T * nch * H * 2 * 4);
}

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_err; }

int dsa_abi_version(void) { return 2; }

// ---------------------------------------------------------------------------
size_t dsa_indexer_topk_workspace(int T, int S, int H, int D, int PS, int MP, int k,
                                  int max_q_len) {
  (void)S; (void)H; (void)D;
  if (T <= 0 || PS <= 0 || MP <= 0 || k <= 0) return 0;
  if (use_fused(T, MP, PS, max_q_len)) return fused_ws(T, MP, PS, k);
  return align256((size_t)T * scores_ld(MP, PS) * 4) +
         align256((size_t)T * dsa::score_ext_ld(max_q_len, MP * PS) * 8);
}

size_t dsa_indexer_topk_fused_workspace(int T, int S, int H, int D, int PS, int MP, int k) {
  (void)S; (void)H; (void)D;
  if (T <= 0 || PS <= 0 || MP <= 0 || k <= 0) return 0;
  return fused_ws(T, MP, PS, k);
}

namespace {
int indexer_topk_impl(const void* q_idx, const float* w, const void* idx_cache, int num_pages,
                      const int32_t* page_table, const int32_t* seq_lens,
                      const int32_t* cu_q_lens, int T, int S, int H, int D, int PS, int MP, int k,
                      int max_q_len, bool fused, int order, int32_t* topk, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_ragged(T, S, PS, MP, num_pages);
  if (st) return st;
  if (order != DSA_ORDER_SCORE && order != DSA_ORDER_POSITION)
    return fail(DSA_ERR_INVALID_ARG, "order=%d is neither DSA_ORDER_SCORE nor DSA_ORDER_POSITION",
                order);
  if (H < 1 || H > 64) return fail(DSA_ERR_UNSUPPORTED, "indexer H=%d not in [1, 64]", H);
  if (D != 32 && D != 64 && D != 128)
    return fail(DSA_ERR_UNSUPPORTED, "indexer D=%d not in {32, 64, 128}", D);
  if (k < 1 || k > 4096) return fail(DSA_ERR_UNSUPPORTED, "k=%d not in [1, 4096]", k);
  // one direct load stages up to 16 consecutive key rows of one page
  if (PS % 16 != 0) return fail(DSA_ERR_UNSUPPORTED, "indexer PS=%d is not a multiple of 16", PS);
  if (T == 0) return ok();
  if (!q_idx || !w || !idx_cache || !page_table || !seq_lens || !cu_q_lens || !topk)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q_idx) || !aligned16(idx_cache))
    return fail(DSA_ERR_INVALID_ARG, "q_idx and idx_cache must be 16-byte aligned");
  const size_t need = fused ? fused_ws(T, MP, PS, k)
                            : dsa_indexer_topk_workspace(T, S, H, D, PS, MP, k, max_q_len);
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "indexer workspace %zu < %zu bytes", workspace_bytes, need);
  dsa::IndexerArgs a;
  a.q = static_cast<const uint16_t*>(q_idx);
  a.w = w;
  a.cache = static_cast<const uint16_t*>(idx_cache);
  a.num_pages = num_pages;
  a.pt = page_table;
  a.seq_lens = seq_lens;
  a.cu = cu_q_lens;
  a.T = T; a.S = S; a.H = H; a.D = D; a.PS = PS; a.MP = MP; a.k = k;
  a.max_q_len = max_q_len;
  a.topk = topk;
  a.by_pos = order == DSA_ORDER_POSITION;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fused) {
    int G = 1, L = 0, C = 0;
    dsa::fused_plan(T, MP * PS, k, &G, &L, &C);
    a.cand = static_cast<uint2*>(workspace);
    a.cand_cnt = reinterpret_cast<int*>(static_cast<char*>(workspace) +
                                        align256((size_t)T * G * C * 8));
    return hip_status(dsa::indexer_fused_topk(a, s), "fused indexer launch");
  }
  a.scores = static_cast<float*>(workspace);
  a.ld = scores_ld(MP, PS);
  a.ext_ld = dsa::score_ext_ld(max_q_len, MP * PS);
  if (a.ext_ld > 0)
    a.ext = reinterpret_cast<uint2*>(static_cast<char*>(workspace) +
                                     align256((size_t)T * a.ld * 4));
  hipError_t e = dsa::indexer_score(a, s);
  if (e != hipSuccess) return hip_status(e, "indexer score launch");
  e = dsa::indexer_select(a, s);
  if (e != hipSuccess || !a.by_pos) return hip_status(e, "indexer top-k launch");
  return hip_status(dsa::topk_rows_distinct_order(topk, T, k, MP * PS, s), "top-k order launch");
}
}  // namespace

int dsa_indexer_topk(const void* q_idx, const float* w, const void* idx_cache, int num_pages,
                     const int32_t* page_table, const int32_t* seq_lens,
                     const int32_t* cu_q_lens, int T, int S, int H, int D, int PS, int MP, int k,
                     int max_q_len, int32_t* topk, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return indexer_topk_impl(q_idx, w, idx_cache, num_pages, page_table, seq_lens, cu_q_lens, T,
                           S, H, D, PS, MP, k, max_q_len, use_fused(T, MP, PS, max_q_len),
                           DSA_ORDER_SCORE, topk, workspace, workspace_bytes, stream);
}

int dsa_indexer_topk_ordered(const void* q_idx, const float* w, const void* idx_cache,
                             int num_pages, const int32_t* page_table, const int32_t* seq_lens,
                             const int32_t* cu_q_lens, int T, int S, int H, int D, int PS, int MP,
                             int k, int max_q_len, int order, int32_t* topk, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return indexer_topk_impl(q_idx, w, idx_cache, num_pages, page_table, seq_lens, cu_q_lens, T,
                           S, H, D, PS, MP, k, max_q_len, use_fused(T, MP, PS, max_q_len), order,
                           topk, workspace, workspace_bytes, stream);
}

int dsa_indexer_topk_fused(const void* q_idx, const float* w, const void* idx_cache,
                           int num_pages, const int32_t* page_table, const int32_t* seq_lens,
                           const int32_t* cu_q_lens, int T, int S, int H, int D, int PS, int MP,
                           int k, int order, int32_t* topk, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return indexer_topk_impl(q_idx, w, idx_cache, num_pages, page_table, seq_lens, cu_q_lens, T,
                           S, H, D, PS, MP, k, 2, true, order, topk, workspace, workspace_bytes,
                           stream);
}

int dsa_topk_position_order(const int32_t* topk, int32_t* out, int T, int k, void* stream) {
  if (T < 0) return fail(DSA_ERR_INVALID_ARG, "T=%d must be >= 0", T);
  if (k < 1 || k > 4096) return fail(DSA_ERR_UNSUPPORTED, "k=%d not in [1, 4096]", k);
  if (T == 0) return ok();
  if (!topk || !out) return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  return hip_status(dsa::topk_position_order(topk, out, T, k, static_cast<hipStream_t>(stream)),
                    "top-k order launch");
}

// ---------------------------------------------------------------------------
size_t dsa_indexer_page_topk_workspace(int T, int S, int H, int D, int PS, int MP, int k_pages,
                                       int max_q_len) {
  (void)S; (void)H; (void)D; (void)k_pages; (void)max_q_len;
  if (T <= 0 || PS <= 0 || MP <= 0) return 0;
  return align256((size_t)T * scores_ld(MP, PS) * 4) + align256((size_t)T * pages_ld(MP) * 4);
}

int dsa_indexer_page_topk(const void* q_idx, const float* w, const void* idx_cache,
                          int num_pages, const int32_t* page_table, const int32_t* seq_lens,
                          const int32_t* cu_q_lens, int T, int S, int H, int D, int PS, int MP,
                          int k_pages, int max_q_len, int32_t* pages, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_ragged(T, S, PS, MP, num_pages);
  if (st) return st;
  if (H < 1 || H > 64) return fail(DSA_ERR_UNSUPPORTED, "indexer H=%d not in [1, 64]", H);
  if (D != 32 && D != 64 && D != 128)
    return fail(DSA_ERR_UNSUPPORTED, "indexer D=%d not in {32, 64, 128}", D);
  if (k_pages < 1 || k_pages > 4096)
    return fail(DSA_ERR_UNSUPPORTED, "k_pages=%d not in [1, 4096]", k_pages);
  if (PS % 16 != 0 || PS > 64)
    return fail(DSA_ERR_UNSUPPORTED, "page top-k PS=%d is not a multiple of 16 up to 64", PS);
  if (T == 0) return ok();
  if (!q_idx || !w || !idx_cache || !page_table || !seq_lens || !cu_q_lens || !pages)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q_idx) || !aligned16(idx_cache))
    return fail(DSA_ERR_INVALID_ARG, "q_idx and idx_cache must be 16-byte aligned");
  const size_t need = dsa_indexer_page_topk_workspace(T, S, H, D, PS, MP, k_pages, max_q_len);
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "page top-k workspace %zu < %zu bytes", workspace_bytes,
                need);
  dsa::IndexerArgs a;
  a.q = static_cast<const uint16_t*>(q_idx);
  a.w = w;
  a.cache = static_cast<const uint16_t*>(idx_cache);
  a.num_pages = num_pages;
  a.pt = page_table;
  a.seq_lens = seq_lens;
  a.cu = cu_q_lens;
  a.T = T; a.S = S; a.H = H; a.D = D; a.PS = PS; a.MP = MP; a.k = k_pages;
  a.max_q_len = max_q_len;
  a.scores = static_cast<float*>(workspace);
  a.ld = scores_ld(MP, PS);
  a.page_scores = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           align256((size_t)T * a.ld * 4));
  a.ldp = pages_ld(MP);
  a.topk = pages;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dsa::indexer_score(a, s);
  if (e != hipSuccess) return hip_status(e, "indexer score launch");
  e = dsa::indexer_page_pool(a, s);
  if (e != hipSuccess) return hip_status(e, "page pool launch");
  return hip_status(dsa::indexer_page_select(a, s), "page top-k launch");
}

int dsa_page_tokens(const int32_t* pages, int T, int k_pages, int PS, int32_t* tokens,
                    void* stream) {
  if (T < 0 || k_pages < 1 || PS < 1 || (long)k_pages * PS > 65536)
    return fail(DSA_ERR_INVALID_ARG, "page tokens: T=%d, k_pages=%d, PS=%d (need T >= 0 and "
                "1 <= k_pages * PS <= 65536)", T, k_pages, PS);
  if (T == 0) return ok();
  if (!pages || !tokens) return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  return hip_status(dsa::page_tokens(pages, T, k_pages, PS, tokens,
                                     static_cast<hipStream_t>(stream)),
                    "page tokens launch");
}

int dsa_paged_write(const void* src, int src_stride, int cols, int col0, void* cache,
                    int row_stride, int num_pages, const int32_t* page_table,
                    const int32_t* seq_lens, const int32_t* cu_q_lens, int T, int S, int PS,
                    int MP, void* stream) {
  int st = check_ragged(T, S, PS, MP, num_pages);
  if (st) return st;
  if (cols < 8 || cols % 8 || col0 < 0 || col0 % 8 || row_stride % 8 ||
      (long)col0 + cols > row_stride || src_stride < cols || src_stride % 8)
    return fail(DSA_ERR_INVALID_ARG,
                "paged write: cols=%d, col0=%d, row_stride=%d, src_stride=%d (need multiples "
                "of 8 with col0 + cols <= row_stride and cols <= src_stride)",
                cols, col0, row_stride, src_stride);
  if (T == 0) return ok();
  if (!src || !cache || !page_table || !seq_lens || !cu_q_lens)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(src) || !aligned16(cache))
    return fail(DSA_ERR_INVALID_ARG, "src and cache must be 16-byte aligned");
  dsa::CacheWriteArgs a = {};
  a.job[0].src = static_cast<const uint16_t*>(src);
  a.job[0].src_stride = src_stride;
  a.job[0].cols = cols;
  a.job[0].col0 = col0;
  a.job[0].cache = static_cast<uint16_t*>(cache);
  a.job[0].row_stride = row_stride;
  a.job[0].num_pages = num_pages;
  a.njobs = 1;
  a.pt = page_table;
  a.seq_lens = seq_lens;
  a.cu = cu_q_lens;
  a.T = T; a.S = S; a.PS = PS; a.MP = MP;
  return hip_status(dsa::paged_write(a, static_cast<hipStream_t>(stream)), "paged write launch");
}

int dsa_paged_write_layer(const void* idx_src, int D, void* idx_cache, const void* kv_src,
                          int kv_cols, void* kv_cache, int row_stride, int num_pages,
                          const int32_t* page_table, const int32_t* seq_lens,
                          const int32_t* cu_q_lens, int T, int S, int PS, int MP, void* stream) {
  int st = check_ragged(T, S, PS, MP, num_pages);
  if (st) return st;
  if (!idx_src && !kv_src)
    return fail(DSA_ERR_INVALID_ARG, "layer write: neither indexer keys nor latent rows given");
  if (idx_src && (D < 8 || D % 8 || !idx_cache))
    return fail(DSA_ERR_INVALID_ARG, "layer write: D=%d must be a positive multiple of 8 with "
                "an indexer cache", D);
  if (kv_src && (kv_cols < 8 || kv_cols % 8 || row_stride % 8 || kv_cols > row_stride ||
                 !kv_cache))
    return fail(DSA_ERR_INVALID_ARG, "layer write: kv_cols=%d, row_stride=%d (need multiples "
                "of 8 with kv_cols <= row_stride) and a latent cache", kv_cols, row_stride);
  if (T == 0) return ok();
  if (!page_table || !seq_lens || !cu_q_lens)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if ((idx_src && (!aligned16(idx_src) || !aligned16(idx_cache))) ||
      (kv_src && (!aligned16(kv_src) || !aligned16(kv_cache))))
    return fail(DSA_ERR_INVALID_ARG, "sources and caches must be 16-byte aligned");
  dsa::CacheWriteArgs a = {};
  if (idx_src) {
    dsa::CacheWriteJob& j = a.job[a.njobs++];
    j.src = static_cast<const uint16_t*>(idx_src);
    j.src_stride = D;
    j.cols = D;
    j.col0 = 0;
    j.cache = static_cast<uint16_t*>(idx_cache);
    j.row_stride = D;
    j.num_pages = num_pages;
  }
  if (kv_src) {
    dsa::CacheWriteJob& j = a.job[a.njobs++];
    j.src = static_cast<const uint16_t*>(kv_src);
    j.src_stride = kv_cols;
    j.cols = kv_cols;
    j.col0 = 0;
    j.cache = static_cast<uint16_t*>(kv_cache);
    j.row_stride = row_stride;
    j.num_pages = num_pages;
  }
  a.pt = page_table;
  a.seq_lens = seq_lens;
  a.cu = cu_q_lens;
  a.T = T; a.S = S; a.PS = PS; a.MP = MP;
  return hip_status(dsa::paged_write(a, static_cast<hipStream_t>(stream)), "layer write launch");
}

// ---------------------------------------------------------------------------
size_t dsa_block_union_workspace(int T, int S, int MP, int QB, int u_max) {
  (void)u_max;
  if (T <= 0 || QB <= 0 || S <= 0 || MP <= 0) return 0;
  const size_t nqb = (size_t)((T + QB - 1) / QB);
  const size_t nw = (size_t)dsa::union_words(S, MP);
  return align256(nqb * nw * 8) + align256(nqb * nw * 4);
}

int dsa_block_union(const int32_t* topk, const int32_t* seq_lens, const int32_t* cu_q_lens,
                    int T, int S, int k, int PS, int MP, int QB, int u_max, int32_t* blk_units,
                    int32_t* blk_counts, uint64_t* blk_member, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_ragged(T, S, PS, MP, 1);
  if (st) return st;
  if (S < 1) return fail(DSA_ERR_INVALID_ARG, "S=%d must be >= 1", S);
  if (PS > 64) return fail(DSA_ERR_UNSUPPORTED, "union PS=%d > 64 (one 64-bit word per page)", PS);
  if (k < 1) return fail(DSA_ERR_INVALID_ARG, "k=%d must be >= 1", k);
  if (QB < 1 || QB > 1024) return fail(DSA_ERR_UNSUPPORTED, "QB=%d not in [1, 1024]", QB);
  if (u_max < 1 || (size_t)u_max * 8 > dsa::kUnionTileBytes)
    return fail(DSA_ERR_UNSUPPORTED, "u_max=%d not in [1, %zu]", u_max, dsa::kUnionTileBytes / 8);
  if ((long)S * MP > (1L << 18))
    return fail(DSA_ERR_UNSUPPORTED, "S*MP=%ld page keys exceed 2^18", (long)S * MP);
  if (T == 0) return ok();
  if (!topk || !seq_lens || !cu_q_lens || !blk_units || !blk_counts)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  const size_t need = dsa_block_union_workspace(T, S, MP, QB, u_max);
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "union workspace %zu < %zu bytes", workspace_bytes, need);
  const size_t nqb = (size_t)((T + QB - 1) / QB);
  const size_t nw = (size_t)dsa::union_words(S, MP);
  dsa::UnionArgs a;
  a.topk = topk;
  a.seq_lens = seq_lens;
  a.cu = cu_q_lens;
  a.T = T; a.S = S; a.k = k; a.PS = PS; a.MP = MP; a.QB = QB; a.u_max = u_max;
  a.units = blk_units;
  a.counts = blk_counts;
  a.member = blk_member;  // NULL: units and counts only
  a.bits = static_cast<uint64_t*>(workspace);
  a.prefix = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align256(nqb * nw * 8));
  return hip_status(dsa::block_union(a, static_cast<hipStream_t>(stream)), "union launch");
}

// ---------------------------------------------------------------------------
static int check_mla_common(const void* q, const void* kv, int row_stride, int H, int PS,
                            void* out) {
  if (H < 1 || H > 64) return fail(DSA_ERR_UNSUPPORTED, "MLA H=%d not in [1, 64]", H);
  if (row_stride < 576 || row_stride % 8 != 0)
    return fail(DSA_ERR_INVALID_ARG, "row_stride=%d must be >= 576 and a multiple of 8",
                row_stride);
  if (!q || !kv || !out) return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned16(q) || !aligned16(kv))
    return fail(DSA_ERR_INVALID_ARG, "q and kv_cache must be 16-byte aligned");
  (void)PS;
  return DSA_OK;
}

size_t dsa_sparse_mla_decode_workspace(int T, int H, int k) {
  if (T <= 0 || H <= 0 || k <= 0) return 0;
  return decode_ws(T, H, k);
}

int dsa_sparse_mla_decode(const void* q, const void* kv_cache, int row_stride, int num_pages,
                          const int32_t* page_table, const int32_t* seq_lens,
                          const int32_t* cu_q_lens, const int32_t* topk, int T, int S, int H,
                          int k, int PS, int MP, float sm_scale, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int st = check_ragged(T, S, PS, MP, num_pages);
  if (st) return st;
  if (k < 1 || k > 65536) return fail(DSA_ERR_UNSUPPORTED, "k=%d not in [1, 65536]", k);
  if (T == 0) return ok();
  st = check_mla_common(q, kv_cache, row_stride, H, PS, out);
  if (st) return st;
  if (!page_table || !seq_lens || !cu_q_lens || !topk)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  const size_t need = dsa_sparse_mla_decode_workspace(T, H, k);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "decode workspace %zu < %zu bytes", workspace_bytes, need);
  const int ch = dsa::mla_decode_chunk(T, k);
  const size_t nch = (size_t)((k + ch - 1) / ch);
  dsa::MlaArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv_cache);
  a.row_stride = row_stride;
  a.num_pages = num_pages;
  a.pt = page_table;
  a.seq_lens = seq_lens;
  a.cu = cu_q_lens;
  a.topk = topk;
  a.T = T; a.S = S; a.H = H; a.k = k; a.PS = PS; a.MP = MP;
  a.sm_scale = sm_scale;
  a.out = static_cast<uint16_t*>(out);
  if (need > 0) {  // split rows: partials in the workspace
    a.part_o = static_cast<uint16_t*>(workspace);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         align256((size_t)T * nch * H * 512 * 2));
  }
  return hip_status(dsa::mla_decode(a, static_cast<hipStream_t>(stream)), "decode launch");
}

int dsa_sparse_mla_decode_static(const void* q, const void* kv_cache, int row_stride,
                                 int num_pages, const int32_t* page_table,
                                 const int32_t* seq_lens, const int32_t* cu_q_lens,
                                 const int32_t* topk, int T, int S, int H, int k, int PS, int MP,
                                 float sm_scale, void* out, void* stream) {
  int st = check_ragged(T, S, PS, MP, num_pages);
  if (st) return st;
  if (k < 1 || k > 65536) return fail(DSA_ERR_UNSUPPORTED, "k=%d not in [1, 65536]", k);
  if (T == 0) return ok();
  st = check_mla_common(q, kv_cache, row_stride, H, PS, out);
  if (st) return st;
  if (!page_table || !seq_lens || !cu_q_lens || !topk)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  const size_t need = decode_ws(T, H, k);
  if (need > dsa::kStaticScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED,
                "static decode: T=%d, H=%d, k=%d needs %zu bytes of scratch, the static "
                "scratch holds %zu (use dsa_sparse_mla_decode with a workspace)",
                T, H, k, need, dsa::kStaticScratchBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (s != nullptr) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    if ((int)sdev != dev)
      return fail(DSA_ERR_INVALID_ARG, "static decode: the stream belongs to device %d, the "
                  "current device is %d", (int)sdev, dev);
  }
  void* ws = nullptr;
  e = dsa::static_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "static scratch address");
  const int ch = dsa::mla_decode_chunk(T, k);
  const size_t nch = (size_t)((k + ch - 1) / ch);
  dsa::MlaArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv_cache);
  a.row_stride = row_stride;
  a.num_pages = num_pages;
  a.pt = page_table;
  a.seq_lens = seq_lens;
  a.cu = cu_q_lens;
  a.topk = topk;
  a.T = T; a.S = S; a.H = H; a.k = k; a.PS = PS; a.MP = MP;
  a.sm_scale = sm_scale;
  a.out = static_cast<uint16_t*>(out);
  a.part_o = static_cast<uint16_t*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                       align256((size_t)T * nch * H * 512 * 2));
  return hip_status(dsa::mla_decode(a, s), "static decode launch");
}

int dsa_sparse_mla_decode_pages(const void* q, const void* kv_cache, int row_stride,
                                int num_pages, const int32_t* page_table,
                                const int32_t* seq_lens, const int32_t* cu_q_lens,
                                const int32_t* pages, int T, int S, int H, int k_pages, int PS,
                                int MP, float sm_scale, void* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  int st = check_ragged(T, S, PS, MP, num_pages);
  if (st) return st;
  if (k_pages < 1 || (long)k_pages * PS > 65536)
    return fail(DSA_ERR_UNSUPPORTED, "k_pages=%d with PS=%d: need 1 <= k_pages * PS <= 65536",
                k_pages, PS);
  if (T == 0) return ok();
  st = check_mla_common(q, kv_cache, row_stride, H, PS, out);
  if (st) return st;
  if (!page_table || !seq_lens || !cu_q_lens || !pages)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  const int k = k_pages * PS;
  const size_t need = dsa_sparse_mla_decode_workspace(T, H, k);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "decode workspace %zu < %zu bytes", workspace_bytes, need);
  const int ch = dsa::mla_decode_chunk(T, k);
  const size_t nch = (size_t)((k + ch - 1) / ch);
  dsa::MlaArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv_cache);
  a.row_stride = row_stride;
  a.num_pages = num_pages;
  a.pt = page_table;
  a.seq_lens = seq_lens;
  a.cu = cu_q_lens;
  a.topk = pages;
  a.sel_pages = true;
  a.T = T; a.S = S; a.H = H; a.k = k; a.PS = PS; a.MP = MP;
  a.sm_scale = sm_scale;
  a.out = static_cast<uint16_t*>(out);
  if (need > 0) {  // split rows: partials in the workspace
    a.part_o = static_cast<uint16_t*>(workspace);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         align256((size_t)T * nch * H * 512 * 2));
  }
  return hip_status(dsa::mla_decode(a, static_cast<hipStream_t>(stream)), "decode launch");
}

int dsa_index_share_map(const int32_t* layer_full, int num_layers, int32_t* full_slot,
                        int32_t* src_slot) {
  if (!layer_full || !full_slot || !src_slot || num_layers < 0)
    return -fail(DSA_ERR_INVALID_ARG, "index share map: null array or negative layer count");
  int last = -1, nfull = 0;
  for (int i = 0; i < num_layers; ++i) {
    if (layer_full[i] != 0 && layer_full[i] != 1)
      return -fail(DSA_ERR_INVALID_ARG, "index share map: layer %d kind %d is neither 0 nor 1",
                   i, layer_full[i]);
    if (layer_full[i] == 1) {
      last = nfull++;
      full_slot[i] = last;
    } else {
      if (last < 0)
        return -fail(DSA_ERR_INVALID_ARG, "index share map: layer %d is shared but no full "
                     "layer precedes it", i);
      full_slot[i] = -1;
    }
    src_slot[i] = last;
  }
  ok();
  return nfull;
}

namespace {
// measured on MI355X, end to end per layer: executed MFMA rate of the
// query-block kernel, and the byte rate of the per-query path (partial
// kernel plus combine)
constexpr double kQblockFlops = 1.0e15, kGatherBytes = 5.7e12;

double qblock_seconds(const int32_t* counts, int nQB, int QB, int H, int PS, int u_max) {
  double pages = 0.0;
  for (int b = 0; b < nQB; ++b) {
    const int c = counts[b];
    pages += c < 0 ? 0.0 : (c < u_max ? c : u_max);
  }
  return pages * QB * H * PS * (576.0 + 512.0) * 2.0 / kQblockFlops;
}

double per_query_seconds(int T, int H, int k) {
  const int CH = dsa::mla_decode_chunk(T, k);
  const double nch = (double)((k + CH - 1) / CH);
  const double bytes = (double)T * k * (1152.0 + 4.0) + (double)T * H * 1152.0 +
                       (double)T * nch * H * (512.0 * 2.0 + 2.0 * 4.0) * 2.0;
  return bytes / kGatherBytes;
}
}  // namespace

int dsa_extend_attend_path(const int32_t* blk_counts_host, int nQB, int T, int H, int k, int PS,
                           int QB, int u_max) {
  if (!blk_counts_host || T <= 0 || H <= 0 || k <= 0 || PS <= 0 || QB <= 0 || u_max <= 0)
    return -fail(DSA_ERR_INVALID_ARG, "extend path: null counts or a non-positive size");
  if ((long)nQB != ((long)T + QB - 1) / QB)
    return -fail(DSA_ERR_INVALID_ARG, "extend path: nQB=%d does not match T=%d, QB=%d", nQB, T,
                 QB);
  const double t_qblock = qblock_seconds(blk_counts_host, nQB, QB, H, PS, u_max);
  const double t_query = per_query_seconds(T, H, k);
  ok();
  return t_query < t_qblock ? 1 : 0;
}

int dsa_extend_attend_plan(int n_qb, const int32_t* qb_host, const int32_t* const* counts_host,
                           int T, int H, int k, int PS, int u_max) {
  if (n_qb < 0 || (n_qb > 0 && (!qb_host || !counts_host)) || T <= 0 || H <= 0 || k <= 0 ||
      PS <= 0 || u_max <= 0)
    return -fail(DSA_ERR_INVALID_ARG, "extend plan: null candidate arrays or a non-positive size");
  double best = per_query_seconds(T, H, k);
  int choice = 0;
  for (int i = 0; i < n_qb; ++i) {
    const int QB = qb_host[i];
    if (QB <= 0 || !counts_host[i])
      return -fail(DSA_ERR_INVALID_ARG, "extend plan: candidate %d has QB=%d or no counts", i,
                   QB);
    const double t = qblock_seconds(counts_host[i], (int)(((long)T + QB - 1) / QB), QB, H, PS,
                                    u_max);
    if (t < best) {
      best = t;
      choice = QB;
    }
  }
  ok();
  return choice;
}

size_t dsa_sparse_mla_extend_workspace(int T, int H, int QB, int u_max) {
  (void)T; (void)H; (void)QB; (void)u_max;
  return 0;
}

int dsa_sparse_mla_extend(const void* q, const void* kv_cache, int row_stride, int num_pages,
                          const int32_t* page_table, const int32_t* seq_lens,
                          const int32_t* cu_q_lens, const int32_t* blk_units,
                          const int32_t* blk_counts, const uint64_t* blk_member, int T, int S,
                          int H, int PS, int MP, int QB, int u_max, float sm_scale, void* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace; (void)workspace_bytes;
  int st = check_ragged(T, S, PS, MP, num_pages);
  if (st) return st;
  if (S < 1) return fail(DSA_ERR_INVALID_ARG, "S=%d must be >= 1", S);
  if (PS > 64) return fail(DSA_ERR_UNSUPPORTED, "extend PS=%d > 64", PS);
  if (QB < 1 || QB > 1024) return fail(DSA_ERR_UNSUPPORTED, "QB=%d not in [1, 1024]", QB);
  if (u_max < 1) return fail(DSA_ERR_INVALID_ARG, "u_max=%d must be >= 1", u_max);
  if ((long)S * MP > (1L << 24)) return fail(DSA_ERR_UNSUPPORTED, "S*MP too large");
  if (T == 0) return ok();
  st = check_mla_common(q, kv_cache, row_stride, H, PS, out);
  if (st) return st;
  if (!page_table || !seq_lens || !cu_q_lens || !blk_units || !blk_counts || !blk_member)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  dsa::MlaArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv_cache);
  a.row_stride = row_stride;
  a.num_pages = num_pages;
  a.pt = page_table;
  a.seq_lens = seq_lens;
  a.cu = cu_q_lens;
  a.units = blk_units;
  a.counts = blk_counts;
  a.member = blk_member;
  a.T = T; a.S = S; a.H = H; a.PS = PS; a.MP = MP; a.QB = QB; a.u_max = u_max;
  a.sm_scale = sm_scale;
  a.out = static_cast<uint16_t*>(out);
  return hip_status(dsa::mla_extend(a, static_cast<hipStream_t>(stream)), "extend launch");
}

}  // extern "C"
