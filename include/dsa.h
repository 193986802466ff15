/*
 * dsa.h — C ABI of libdsa.so, the MI355X (gfx950) DeepSeek-Sparse-Attention
 * hot path: lightning-indexer exact top-k, query-block union tables, and
 * sparse absorbed-MLA attention for decode and chunked-prefill extend.
 *
 * Sources: the sglang-jax DSA pages — "ref.py" (streamindex_topk_ref,
 * sparse_mla_ref), "sparse_mla_prefill_qblock.py" (build_block_unit_tables,
 * _qblock_kernel, sparse_mla_attention_qblock) and "dsa_sparse_backend.py"
 * (DSASparseAttentionBackend: _fixed_stride_pages, _scatter_paged, the
 * default sm_scale).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller. The library
 *   allocates nothing, keeps no pointer after a call returns, and never
 *   synchronises: work is enqueued on `stream` (a hipStream_t; NULL = the
 *   default stream) and results are visible after the caller's sync.
 * - State kept by the library: the thread-local text of dsa_last_error();
 *   the event records of the profiling hook (idle unless enabled); and, per
 *   GPU, the static scratch of dsa_sparse_mla_decode_static (part of the
 *   loaded code object) with its device address. Every other entry point is
 *   reentrant; overlapping calls of the static decode on one GPU race.
 * - bf16 tensors are raw IEEE bfloat16 (uint16 bit patterns); all layouts
 *   are dense row-major with the shapes given.
 * - Ragged batches (packed along the token axis T):
 *     seq_lens [S]     int32, kv length of sequence s INCLUDING its current
 *                      query chunk ("dsa_sparse_backend.py", _scatter_paged);
 *     cu_q_lens [S+1]  int32, row range [cu_q_lens[s], cu_q_lens[s+1]) of s;
 *     page_table [S,MP] int32, physical page of seq-local page p of s
 *                      (fixed stride MP, as built by _fixed_stride_pages).
 *   Row t of sequence s sits at absolute position
 *     abs_q(t) = seq_lens[s] - q_len(s) + (t - cu_q_lens[s])
 *   ("ref.py", streamindex_topk_ref). Rows t >= cu_q_lens[S] belong to no
 *   sequence. Positions are seq-local token indices: position j of s lives in
 *   page page_table[s, j / PS] at offset j % PS.
 * - Caller preconditions, not checked on the host (checking would need a
 *   device sync): cu_q_lens non-decreasing with cu_q_lens[0] = 0 and
 *   cu_q_lens[S] <= T; q_len(s) <= seq_lens[s] <= MP * PS; every page id
 *   reachable below seq_lens[s] lies in [0, num_pages). Kernels clamp what
 *   they read so that a violation yields unspecified values, not a fault.
 * - Host validation happens before any launch. On an error nothing is
 *   launched and nothing is written; dsa_last_error() describes the cause.
 *   DSA_ERR_HIP reports a launch failure (hipGetLastError); asynchronous
 *   faults surface at the caller's next synchronisation.
 * - Each entry point that needs scratch takes a caller-provided device
 *   workspace of at least the size its *_workspace() query returns (any
 *   alignment >= 256 B); the query takes the shape arguments that size it.
 *   dsa_sparse_mla_decode_static uses the library's static scratch instead.
 * - Status codes are returned as int (the enum values below); the host-logic
 *   functions return a non-negative result or a negated status.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* a size or pointer argument is out of range */
  DSA_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement */
  DSA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required */
  DSA_ERR_HIP = 4          /* a HIP launch or runtime call failed */
};

/* Order of the positions in a row of a top-k table. */
enum {
  DSA_ORDER_SCORE = 0,   /* by score descending, equal scores by position ascending */
  DSA_ORDER_POSITION = 1 /* the same positions in ascending position order */
};

/* Static text for a status code. */
const char* dsa_status_string(int status);
/* Detail of the most recent failure in this thread ("" if none). */
const char* dsa_last_error(void);
/* ABI revision; bumps on any signature or semantic change. */
int dsa_abi_version(void);

/*
 * dsa_indexer_topk — lightning-indexer exact top-k.
 * "ref.py", streamindex_topk_ref (decode is the q_len = 1 case).
 *
 * For each row t of sequence s with a = abs_q(t) and every position j with
 * j < seq_lens[s] and j <= a:
 *     score[t, j] = sum_h w[t, h] * relu( sum_d q_idx[t, h, d] * K[j, d] )
 * with K[j] = idx_cache[page_table[s, j / PS], j % PS, :], computed with
 * bf16 products and fp32 accumulation. topk[t, :] receives the first
 * min(k, n_valid) positions ordered by score descending, equal scores by
 * position ascending (-0.0 equals +0.0), then -1 up to k. Rows outside every
 * sequence are all -1. topk is fully written for rows 0..T-1.
 *
 *   q_idx      bf16 [T, H, D]
 *   w          fp32 [T, H]
 *   idx_cache  bf16 [num_pages, PS, D]  one key per token, shared by heads
 *   topk       int32 [T, k]             output
 *   max_q_len  host upper bound on q_len(s) over the batch (a hint that picks
 *              the streaming per-row kernel when <= 1 and the MFMA tile
 *              kernel otherwise; any value gives the same result)
 *   workspace  device scratch of at least dsa_indexer_topk_workspace(...)
 *              bytes for the same arguments. For query chunks (max_q_len > 1)
 *              whose score matrix T x ceil64(MP * PS) fp32 would exceed
 *              256 MiB, the call takes the fused path of
 *              dsa_indexer_topk_fused (workspace O(T * k)); otherwise it holds
 *              the fp32 score rows and, for the tile kernel, each row's
 *              extreme scores per 2048 positions. Both paths give the same
 *              result.
 * Supported: 1 <= H <= 64, D in {32, 64, 128}, PS a multiple of 16,
 * MP * PS <= 2^24, 1 <= k <= 4096; otherwise DSA_ERR_UNSUPPORTED.
 */
size_t dsa_indexer_topk_workspace(int T, int S, int H, int D, int PS, int MP, int k,
                                  int max_q_len);
int dsa_indexer_topk(const void* q_idx, const float* w, const void* idx_cache, int num_pages,
                     const int32_t* page_table, const int32_t* seq_lens,
                     const int32_t* cu_q_lens, int T, int S, int H, int D, int PS, int MP,
                     int k, int max_q_len, int32_t* topk, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * dsa_indexer_topk_ordered — dsa_indexer_topk with a choice of the order in
 * which each row's selected positions are written: DSA_ORDER_SCORE (the
 * order above, which is that of dsa_indexer_topk) or DSA_ORDER_POSITION (the
 * same set of positions in ascending position order, then -1 up to k).
 *
 * Position order is for consumers whose result does not depend on the order:
 * the sparse attention is a sum over the selection ("ref.py", sparse_mla_ref)
 * and the block union is a set (sparse_mla_prefill_qblock.py,
 * build_block_unit_tables). Fed in position order, the rows that neighbouring
 * queries share are gathered at about the same time, and the per-query
 * attention of a long-context extend runs about 30% faster than on the same
 * selection in score order. On the fused path it costs nothing (the
 * candidate lists are kept in position order); with a score matrix it adds
 * one sort of each row (dsa_topk_position_order).
 *
 *   arguments as in dsa_indexer_topk; order DSA_ORDER_SCORE or
 *   DSA_ORDER_POSITION, anything else DSA_ERR_INVALID_ARG
 */
int dsa_indexer_topk_ordered(const void* q_idx, const float* w, const void* idx_cache,
                             int num_pages, const int32_t* page_table, const int32_t* seq_lens,
                             const int32_t* cu_q_lens, int T, int S, int H, int D, int PS, int MP,
                             int k, int max_q_len, int order, int32_t* topk, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * dsa_topk_position_order — each row of a top-k table in ascending position
 * order: out[t, :] holds the non-negative entries of topk[t, :] ascending
 * (duplicates kept), then the -1 entries (any negative entry counts as -1
 * and is written as -1). out may be topk (in place).
 *
 *   topk  int32 [T, k]  input
 *   out   int32 [T, k]  output
 * Supported: 1 <= k <= 4096 (DSA_ERR_UNSUPPORTED otherwise); T >= 0.
 */
int dsa_topk_position_order(const int32_t* topk, int32_t* out, int T, int k, void* stream);

/*
 * dsa_indexer_topk_fused — dsa_indexer_topk without the score matrix: the
 * scores are ranked as they are computed ("dsa_sparse_backend.py", the
 * prefill indexer kernel note: the [T, max_kv] token scores are the dominant
 * temporary at long context). Same result, bit for bit, as
 * dsa_indexer_topk for the same arguments.
 *
 * Each row's positions are split into G segments (G <= 8, G * k <= 8192);
 * one workgroup scores 8 consecutive rows over one segment in ascending
 * position order and keeps, per row, a candidate list of C = k + max(k, 512)
 * (rounded up to 64) entries: when it fills, the list is cut to its exact k
 * best (ties by lower position) and only keys above the k-th are taken
 * afterwards. A second kernel merges each row's lists into the canonical
 * order. The workspace holds the lists: T * G * C * 8 + T * G * 4 bytes
 * (about 268 MB for 8192 rows at k = 2048, against 4.3 GB of scores at a
 * 131072-position context).
 *
 *   arguments as in dsa_indexer_topk, without max_q_len (any ragged layout
 *   is accepted); order as in dsa_indexer_topk_ordered (with
 *   DSA_ORDER_POSITION the merge writes the lists' order, no score sort);
 *   workspace of dsa_indexer_topk_fused_workspace(...) bytes
 * Supported: as dsa_indexer_topk.
 */
size_t dsa_indexer_topk_fused_workspace(int T, int S, int H, int D, int PS, int MP, int k);
int dsa_indexer_topk_fused(const void* q_idx, const float* w, const void* idx_cache,
                           int num_pages, const int32_t* page_table, const int32_t* seq_lens,
                           const int32_t* cu_q_lens, int T, int S, int H, int D, int PS, int MP,
                           int k, int order, int32_t* topk, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * dsa_indexer_page_topk — lightning-indexer exact top-k over pages.
 * "ref.py", streamindex_page_topk_ref.
 *
 * The scores of dsa_indexer_topk, with every position that is not valid for
 * the row (j >= seq_lens[s] or j > abs_q) at -inf, max-pooled over the PS
 * positions of each seq-local page p (positions p*PS .. p*PS + PS - 1). The
 * pages that hold a valid position are the first ceil(n_valid / PS) of the
 * row; pages[t, :] receives the first min(k_pages, that many) of them by
 * page score descending, equal scores by page id ascending, then -1 up to
 * k_pages. Rows outside every sequence are all -1; pages is fully written.
 *
 *   q_idx, w, idx_cache, page_table, seq_lens, cu_q_lens, max_q_len
 *              as in dsa_indexer_topk
 *   pages      int32 [T, k_pages]  output, seq-local page ids
 * Supported: as dsa_indexer_topk, with PS a multiple of 16 up to 64 and
 * 1 <= k_pages <= 4096; otherwise DSA_ERR_UNSUPPORTED.
 */
size_t dsa_indexer_page_topk_workspace(int T, int S, int H, int D, int PS, int MP, int k_pages,
                                       int max_q_len);
int dsa_indexer_page_topk(const void* q_idx, const float* w, const void* idx_cache,
                          int num_pages, const int32_t* page_table, const int32_t* seq_lens,
                          const int32_t* cu_q_lens, int T, int S, int H, int D, int PS, int MP,
                          int k_pages, int max_q_len, int32_t* pages, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * dsa_page_tokens — the positions of selected pages, for the token-exact
 * attention entry points: tokens[t, i] = pages[t, i / PS] * PS + i % PS, or
 * -1 where pages[t, i / PS] is -1. Attending these with
 * dsa_sparse_mla_decode (or through dsa_block_union and
 * dsa_sparse_mla_extend) attends every valid position of the selected pages
 * (the attention masks j >= seq_lens and j > abs_q itself): the page-budget
 * decode of "dsa_sparse_backend.py" (the page-scoring indexer path).
 *
 *   pages   int32 [T, k_pages]
 *   tokens  int32 [T, k_pages * PS]  output
 * Returns DSA_ERR_INVALID_ARG for T < 0, k_pages < 1, PS < 1 or
 * k_pages * PS > 65536.
 */
int dsa_page_tokens(const int32_t* pages, int T, int k_pages, int PS, int32_t* tokens,
                    void* stream);

/*
 * dsa_paged_write — the paged cache self-write of the new tokens, ahead of
 * the indexer and the attention: "dsa_sparse_backend.py", _scatter_paged
 * (indexer keys) and "sparse_mla_prefill_qblock.py", paged_write_back
 * (latent rows [c_kv | k_rope]).
 *
 * Packed row t of sequence s (q_start <= t < q_end) lands at its seq-local
 * position a = seq_lens[s] - (q_end - q_start) + (t - q_start):
 *     cache[page_table[s, a / PS], a % PS, col0 + c] = src[t, c],  c < cols.
 * Rows outside every sequence, positions outside
 * 0 <= a < min(seq_lens[s], MP * PS), and positions whose page-table entry is
 * not in [0, num_pages) (e.g. -1 for an unassigned page) are dropped. Other
 * columns and slots are left untouched, so a latent row can be written whole
 * (cols = 576) or by parts (c_kv at col0 = 0 with cols = 512, k_rope at
 * col0 = 512 with cols = 64), the indexer key by one call (cols = D). Rows of
 * one call must name distinct slots.
 *
 *   src    bf16 [T, src_stride], the first cols columns are written
 *   cache  bf16 [num_pages, PS, row_stride], written in place
 * Returns DSA_ERR_INVALID_ARG unless cols, col0, row_stride and src_stride
 * are multiples of 8 with col0 + cols <= row_stride and cols <= src_stride,
 * and src and cache are 16-byte aligned.
 */
int dsa_paged_write(const void* src, int src_stride, int cols, int col0, void* cache,
                    int row_stride, int num_pages, const int32_t* page_table,
                    const int32_t* seq_lens, const int32_t* cu_q_lens, int T, int S, int PS,
                    int MP, void* stream);

/*
 * dsa_paged_write_layer — one launch that writes a layer's new tokens into
 * both of its caches ahead of its indexer and attention: the indexer keys
 * ("dsa_sparse_backend.py", _scatter_paged) and the latent rows
 * ("sparse_mla_prefill_qblock.py", paged_write_back, the self-write of
 * prefill_write_and_attend_ragged_qblock). Each written row follows the
 * dsa_paged_write rule (same slots, same dropped rows), with
 *   idx_cache[page, a % PS, 0:D]      = idx_src[t, 0:D]
 *   kv_cache[page, a % PS, 0:kv_cols] = kv_src[t, 0:kv_cols]
 * Either source may be NULL to skip that cache (a layer that shares another
 * layer's indexer has no keys of its own to write).
 *
 *   idx_src    bf16 [T, D] dense,       idx_cache bf16 [num_pages, PS, D]
 *   kv_src     bf16 [T, kv_cols] dense, kv_cache  bf16 [num_pages, PS, row_stride]
 *              (kv_cols = 576 writes the whole [c_kv | k_rope] row)
 * Returns DSA_ERR_INVALID_ARG when both sources are NULL, when D, kv_cols or
 * row_stride is not a positive multiple of 8 or kv_cols > row_stride, when a
 * given source has no cache, or when a pointer is not 16-byte aligned.
 */
int dsa_paged_write_layer(const void* idx_src, int D, void* idx_cache, const void* kv_src,
                          int kv_cols, void* kv_cache, int row_stride, int num_pages,
                          const int32_t* page_table, const int32_t* seq_lens,
                          const int32_t* cu_q_lens, int T, int S, int PS, int MP, void* stream);

/*
 * dsa_block_union — per query-block union of selected pages and per-token
 * membership. "sparse_mla_prefill_qblock.py", build_block_unit_tables, with
 * the ragged lifting of sparse_mla_attention_qblock.
 *
 * Rows are grouped into nQB = ceil(T / QB) blocks of QB consecutive packed
 * rows (blocks may straddle sequences; the last block is padded with empty
 * rows). A selected position j >= 0 of row t in sequence s names the page
 * key s * MP + j / PS; entries j < 0 or j >= MP * PS and rows outside every
 * sequence are ignored. Per block b:
 *   blk_counts[b]        number of distinct keys (TRUE size, not capped);
 *   blk_units[b, i]      the i-th smallest key for i < min(count, u_max),
 *                        -1 after;
 *   blk_member[b, i, q]  bit r set iff row b*QB+q selected position
 *                        (key % MP) * PS + r of that page; 0 for padding
 *                        rows and for slots i >= min(count, u_max).
 * A count above u_max is data, not an error: the tables then hold only the
 * smallest u_max keys (lossy). min(QB * k, S * MP) slots are always enough.
 *
 *   topk        int32 [T, k]
 *   blk_units   int32 [nQB, u_max]       output
 *   blk_counts  int32 [nQB]              output
 *   blk_member  uint64 [nQB, u_max, QB]  output, or NULL: then only
 *               blk_units and blk_counts are written and the membership
 *               pass is not launched (the sizes a plan reads cost about
 *               half of the full call).
 * Supported: PS <= 64 (one 64-bit membership word per page), S * MP <= 2^18,
 * 1 <= u_max <= 8192, 1 <= QB <= 1024; otherwise DSA_ERR_UNSUPPORTED.
 */
size_t dsa_block_union_workspace(int T, int S, int MP, int QB, int u_max);
int dsa_block_union(const int32_t* topk, const int32_t* seq_lens, const int32_t* cu_q_lens,
                    int T, int S, int k, int PS, int MP, int QB, int u_max,
                    int32_t* blk_units, int32_t* blk_counts, uint64_t* blk_member,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_mla_decode — sparse absorbed-MLA attention, one query row per
 * selection list. "ref.py", sparse_mla_ref.
 *
 * For each row t of sequence s (a = abs_q(t)) and head h, over
 * V = { j in topk[t, :] : 0 <= j < seq_lens[s], j <= a }:
 *     l_j = sm_scale * sum_{d < 576} q[t, h, d] * R_j[d]
 *     out[t, h, :] = sum_j softmax(l)_j * R_j[0:512]
 * with R_j = kv_cache[page_table[s, j / PS], j % PS, 0:576] (the packed
 * [c_kv 512 | k_rope 64] latent row). Logits and softmax in fp32, bf16
 * products, fp32 accumulation, bf16 output. Empty V or a row outside every
 * sequence gives zeros. Selections must be duplicate-free (a duplicate would
 * be counted twice). Any ragged layout is accepted; "decode" names the
 * per-row execution: each row's selection list is split into chunks of up
 * to 2048 entries, sized so that about 512 workgroups exist, and a combine
 * merges the chunks' partials; when every list is one chunk (large
 * batches) the attention writes the output itself and
 * dsa_sparse_mla_decode_workspace returns 0 (workspace may then be NULL).
 *
 *   q          bf16 [T, H, 576]  = [q_nope absorbed (512) | q_rope (64)]
 *   kv_cache   bf16 [num_pages, PS, row_stride], row_stride >= 576
 *   topk       int32 [T, k]
 *   out        bf16 [T, H, 512]  output
 * Supported: 1 <= H <= 64, MP * PS <= 2^24, 1 <= k <= 65536; otherwise
 * DSA_ERR_UNSUPPORTED.
 */
size_t dsa_sparse_mla_decode_workspace(int T, int H, int k);
int dsa_sparse_mla_decode(const void* q, const void* kv_cache, int row_stride, int num_pages,
                          const int32_t* page_table, const int32_t* seq_lens,
                          const int32_t* cu_q_lens, const int32_t* topk, int T, int S, int H,
                          int k, int PS, int MP, float sm_scale, void* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_mla_decode_static — dsa_sparse_mla_decode without a workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). The
 * result is the dsa_sparse_mla_decode result for the same arguments (the
 * same kernels and the same split of each selection list).
 *
 * The split-list partials live in a static device array of the library,
 * 32 MiB per GPU (zero-filled at load, held until the process ends); the
 * call allocates nothing and frees nothing. Its address on a GPU is taken
 * once, on the first call with that GPU current. Calls that need more than
 * dsa_sparse_mla_decode_workspace(T, H, k) > 32 MiB return
 * DSA_ERR_UNSUPPORTED (the workspace entry point has no such limit).
 * Every call on one GPU shares that GPU's array and leaves its partials
 * there: calls that overlap on one GPU (concurrent streams, or threads)
 * race and must be serialised by the caller. `stream` must belong to the
 * current device (DSA_ERR_INVALID_ARG otherwise); GPUs beyond the 64th are
 * not supported (DSA_ERR_HIP).
 *
 *   arguments as in dsa_sparse_mla_decode, without workspace and its size
 */
int dsa_sparse_mla_decode_static(const void* q, const void* kv_cache, int row_stride,
                                 int num_pages, const int32_t* page_table,
                                 const int32_t* seq_lens, const int32_t* cu_q_lens,
                                 const int32_t* topk, int T, int S, int H, int k, int PS, int MP,
                                 float sm_scale, void* out, void* stream);

/*
 * dsa_sparse_mla_decode_pages — sparse absorbed-MLA attention over every
 * valid position of each row's selected pages: the page-budget decode of
 * "dsa_sparse_backend.py" (the page-scoring indexer path, whose pages come
 * from dsa_indexer_page_topk). The result equals dsa_sparse_mla_decode on
 * the positions dsa_page_tokens would list for the same pages (the masks
 * j < seq_lens and j <= abs_q drop the positions past the sequence end),
 * without materialising them.
 *
 *   pages   int32 [T, k_pages] seq-local page ids, -1 for none; duplicates
 *           count twice, as repeated positions do in dsa_sparse_mla_decode
 *   other arguments as in dsa_sparse_mla_decode; the workspace is
 *   dsa_sparse_mla_decode_workspace(T, H, k_pages * PS)
 * Supported: as dsa_sparse_mla_decode, with 1 <= k_pages * PS <= 65536.
 */
int dsa_sparse_mla_decode_pages(const void* q, const void* kv_cache, int row_stride,
                                int num_pages, const int32_t* page_table,
                                const int32_t* seq_lens, const int32_t* cu_q_lens,
                                const int32_t* pages, int T, int S, int H, int k_pages, int PS,
                                int MP, float sm_scale, void* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * dsa_sparse_mla_extend — query-block sparse absorbed-MLA attention.
 * "sparse_mla_prefill_qblock.py", _qblock_kernel / sparse_mla_attention_qblock.
 *
 * Block b walks its union slots i < min(blk_counts[b], u_max) in ascending
 * key order, fetching each page once for all its QB * H rows. A key r of
 * that page (position j = (key % MP) * PS + r of sequence key / MP) counts
 * for row (q, h) iff bit r of blk_member[b, i, q] is set, j <= abs_q and
 * j < seq_lens. The masked online softmax then gives, per query, exactly the
 * dsa_sparse_mla_decode result for the selection the tables were built
 * from (up to fp32 summation order), when no block overflowed u_max.
 *
 *   q, kv_cache, out   as in dsa_sparse_mla_decode
 *   blk_*              as produced by dsa_block_union with the same
 *                      (T, QB, u_max, PS, MP)
 * Supported: 1 <= H <= 64, PS <= 64, 1 <= QB <= 1024, S * MP <= 2^24;
 * otherwise DSA_ERR_UNSUPPORTED.
 */
size_t dsa_sparse_mla_extend_workspace(int T, int H, int QB, int u_max);
int dsa_sparse_mla_extend(const void* q, const void* kv_cache, int row_stride, int num_pages,
                          const int32_t* page_table, const int32_t* seq_lens,
                          const int32_t* cu_q_lens, const int32_t* blk_units,
                          const int32_t* blk_counts, const uint64_t* blk_member, int T, int S,
                          int H, int PS, int MP, int QB, int u_max, float sm_scale, void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsa_index_share_map — the static IndexShare layer mapping ("ref.py",
 * build_index_share_map; "dsa_sparse_backend.py", module docstring: shared
 * layers reuse the top-k of the last full layer). Host logic only.
 *
 *   layer_full  HOST int32 [num_layers]: 1 = full layer (runs the indexer,
 *               owns an indexer-key cache and a top-k slot), 0 = shared
 *   full_slot   HOST int32 [num_layers] output: the slot a full layer owns,
 *               slots numbered 0, 1, ... in layer order; -1 for shared layers
 *   src_slot    HOST int32 [num_layers] output: the slot whose top-k the
 *               layer attends with (its own if full, else the nearest
 *               preceding full layer's)
 * Returns the number of full layers (of slots), or DSA_ERR_INVALID_ARG as a
 * negative number when a shared layer has no full layer before it, a kind
 * is neither 0 nor 1, or an array is null.
 */
int dsa_index_share_map(const int32_t* layer_full, int num_layers, int32_t* full_slot,
                        int32_t* src_slot);

/*
 * dsa_extend_attend_path — which of the two token-exact extend attention
 * paths to run for a packed batch whose block unions are built: the query
 * block (dsa_sparse_mla_extend, one page fetch per block, MFMA work growing
 * with the union sizes) or per query (dsa_sparse_mla_decode on the packed
 * batch: every row gathers its own selected rows, HBM work growing with
 * T * k). Both give the same result per query; the choice only decides the
 * time. The query-block kernel page ("sparse_mla_prefill_qblock.py", module
 * docstring) sets the two designs against each other: one re-fetches every
 * page per query, the other walks each block's page union once.
 *
 * The estimate is each path's work at the rate this library measures on
 * MI355X: executed query-block flops sum_b min(blk_counts[b], u_max) *
 * QB * H * PS * (576 + 512) * 2 at 1.0e15 flop/s, against the per-query
 * bytes (selected latent rows of 1152 bytes, selection entries, queries and
 * the per-chunk partial results, written and read back) at 5.7e12 B/s.
 *
 *   blk_counts_host  HOST int32 [nQB], the blk_counts of dsa_block_union
 *                    copied to the host; read only, not kept
 *   nQB = ceil(T / QB); T, H, k, PS, QB, u_max as in the other calls
 * Returns 0 (query block), 1 (per query), or DSA_ERR_INVALID_ARG (as a
 * negative number) for a null pointer, a non-positive size or nQB that does
 * not match T and QB. Touches no GPU state.
 */
int dsa_extend_attend_path(const int32_t* blk_counts_host, int nQB, int T, int H, int k, int PS,
                           int QB, int u_max);

/*
 * dsa_extend_attend_plan — the extend attention to run for a packed batch,
 * chosen among the per-query path and query blocks of several sizes QB
 * (the QB sweep of "dsa_sparse_backend.py", DSA_PREFILL_QBLOCK_QB), from
 * each candidate's union sizes. The cost of each is the estimate of
 * dsa_extend_attend_path; ties keep the per-query path, then the earlier
 * candidate. Host logic only.
 *
 *   n_qb         number of query-block candidates (0: per query)
 *   qb_host      HOST int32 [n_qb], the candidates' QB
 *   counts_host  HOST [n_qb] pointers: candidate i's blk_counts from
 *                dsa_block_union at QB = qb_host[i] (ceil(T / QB) entries)
 *   T, H, k, PS, u_max  as in the other calls (u_max: the union tables' slots)
 * Returns the chosen QB, 0 for the per-query path, or DSA_ERR_INVALID_ARG
 * (as a negative number) for a null array, a non-positive QB or size.
 */
int dsa_extend_attend_plan(int n_qb, const int32_t* qb_host, const int32_t* const* counts_host,
                           int T, int H, int k, int PS, int u_max);

/*
 * Kernel timing (diagnostics). dsa_profile_enable(1) clears earlier records
 * and makes every subsequent kernel launch of the entry points above record
 * a pair of HIP events on its own stream; dsa_profile_enable(0) stops it.
 * dsa_profile_read() waits for the recorded events, reduces them per kernel
 * name in first-launch order and fills up to max_kernels entries:
 * names (max_kernels * name_len bytes, NUL-terminated, truncated to
 * name_len - 1), launches[i], total_ms[i]; *n_kernels gets the count. The
 * records are consumed. Not meant for use under graph capture.
 * Returns DSA_ERR_INVALID_ARG for bad sizes, DSA_ERR_HIP if an event failed.
 */
int dsa_profile_enable(int on);
int dsa_profile_read(int max_kernels, char* names, int name_len, int* launches,
                     double* total_ms, int* n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
