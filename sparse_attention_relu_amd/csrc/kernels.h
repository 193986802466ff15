// Internal launch interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

constexpr size_t kUnionTileBytes = 64 * 1024;   // LDS membership tile per workgroup

struct IndexerArgs {
  const uint16_t* q;
  const float* w;
  const uint16_t* cache;
  int num_pages;
  const int32_t* pt;
  const int32_t* seq_lens;
  const int32_t* cu;
  int T, S, H, D, PS, MP, k, max_q_len;
  float* scores;  // workspace [T, ld]
  long ld;
  int32_t* topk;
  // page-level selection: page scores [T, ldp] (max over each page's valid
  // positions); the select then ranks pages, ceil(n_valid / PS) per row
  float* page_scores;
  long ldp;
  // tile scorer only: per (row, 2048-position tile) minimum and maximum order
  // key of the stored scores [T, ext_ld] (nullptr: not produced)
  uint2* ext = nullptr;
  int ext_ld = 0;
  // fused scoring and top-k: per (row, segment) candidate lists [T, G, C] of
  // (order key, position) and their lengths [T, G]
  uint2* cand = nullptr;
  int* cand_cnt = nullptr;
  // 1: each row's top-k in ascending position order (-1 last) instead of
  // the canonical score order
  int by_pos = 0;
};

// Segments G of L positions and list capacity C of the fused path.
void fused_plan(int T, int cap, int k, int* G, int* L, int* C);
hipError_t indexer_fused_topk(const IndexerArgs& a, hipStream_t st);
// out[t] = in[t] in ascending position order, -1 entries last (in == out allowed)
hipError_t topk_position_order(const int32_t* in, int32_t* out, int T, int k, hipStream_t st);
// The same in place for rows of distinct positions below cap (a bitmap per
// row up to kRowsBitmapMaxCap positions, the general sort above that).
constexpr int kRowsBitmapMaxCap = 1 << 17;  // 32 KB of LDS
hipError_t topk_rows_distinct_order(int32_t* topk, int T, int k, int cap, hipStream_t st);

// Tiles per row of the per-tile extreme keys the scorer writes for rows of
// at most `cap` positions (0 when the chosen scorer writes none).
int score_ext_ld(int max_q_len, int cap);
hipError_t indexer_score(const IndexerArgs& a, hipStream_t st);
hipError_t indexer_select(const IndexerArgs& a, hipStream_t st);
hipError_t indexer_page_pool(const IndexerArgs& a, hipStream_t st);
hipError_t indexer_page_select(const IndexerArgs& a, hipStream_t st);
hipError_t page_tokens(const int32_t* pages, int T, int k_pages, int PS, int32_t* tokens,
                       hipStream_t st);
size_t topk_select_lds_bytes(int k);

struct UnionArgs {
  const int32_t* topk;
  const int32_t* seq_lens;
  const int32_t* cu;
  int T, S, k, PS, MP, QB, u_max;
  int32_t* units;
  int32_t* counts;
  uint64_t* member;
  uint64_t* bits;    // workspace [nQB, NW]
  int32_t* prefix;   // workspace [nQB, NW]
};

int union_words(int S, int MP);
int union_member_qpw(int QB, int u_max);
hipError_t block_union(const UnionArgs& a, hipStream_t st);

struct MlaArgs {
  const uint16_t* q;
  const uint16_t* kv;
  int row_stride, num_pages;
  const int32_t* pt;
  const int32_t* seq_lens;
  const int32_t* cu;
  const int32_t* topk;  // decode: positions [T, k], or pages [T, k / PS]
  bool sel_pages;       // decode: topk holds pages (k = k_pages * PS)
  const int32_t* units;  // extend
  const int32_t* counts;
  const uint64_t* member;
  int T, S, H, k, PS, MP, QB, u_max;
  float sm_scale;
  uint16_t* out;
  uint16_t* part_o;  // decode workspace: unnormalised partial O, bf16
  float* part_ml;
};

// One cache of a paged write: src bf16 [T, src_stride] (first cols columns)
// into cache bf16 [num_pages, PS, row_stride] at columns col0 ...
struct CacheWriteJob {
  const uint16_t* src;
  int src_stride, cols, col0;
  uint16_t* cache;
  int row_stride, num_pages;
};

struct CacheWriteArgs {
  CacheWriteJob job[2];  // the caches written by one launch
  int njobs;             // 1 or 2
  const int32_t* pt;
  const int32_t* seq_lens;
  const int32_t* cu;
  int T, S, PS, MP;
};

hipError_t paged_write(const CacheWriteArgs& a, hipStream_t st);

int mla_decode_chunk(int T, int k);
// Size of the per-GPU static scratch of the allocation-free decode entry point,
// and its device address on the current device (taken once per device).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t static_scratch(void** ptr);
hipError_t mla_decode(const MlaArgs& a, hipStream_t st);
hipError_t mla_extend(const MlaArgs& a, hipStream_t st);

}  // namespace dsa
