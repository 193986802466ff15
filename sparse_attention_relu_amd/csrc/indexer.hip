// Lightning-indexer scoring and exact top-k for gfx950.
//
// score[t, j] = sum_h w[t, h] * relu(q[t, h, :] . K[j, :])   (sglang-jax
// "ref.py", streamindex_topk_ref). The head contraction runs on MFMA
// v_mfma_f32_32x32x16_bf16 with heads as the M dimension and keys as N, so a
// lane ends up holding 16 heads of one key and the ReLU-weighted head sum is
// a per-lane reduction plus one cross-half add. Scores land in a caller
// workspace [T, MP * PS] (fp32); the select kernel then picks the exact
// top-k per row with a 64-bit radix select over (score, position) keys.
#include <atomic>

#include <rocprim/block/block_radix_sort.hpp>

#include "common.h"
#include "kernels.h"
#include "profile.h"

namespace dsa {

// ---------------------------------------------------------------------------
// Operand loads. The contraction over D is split between the two lane halves
// (hf = lane / 32): half hf covers d in [hf * D/2, (hf + 1) * D/2) and k-step
// i of the MFMA reads its 8 consecutive values d = hf * D/2 + 8 i .. + 8.
// A and B use the same split, so the sum over all steps is the full dot.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void load_q_frag(const uint16_t* __restrict__ qrow, bool ok,
                                            bf16x8 (&a)[D / 16]) {
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    uint4 v = ok ? *reinterpret_cast<const uint4*>(qrow + 8 * i) : zero_u4();
    a[i] = as_bf16x8(v);
  }
}

// Per-lane head weights for the 16 accumulator rows of a 32x32 MFMA block:
// accumulator r of lane l is row 8 (r / 4) + 4 (l / 32) + (r % 4).
__device__ __forceinline__ void load_head_weights(const float* __restrict__ wrow, int H, int hb,
                                                  int hf, float (&wv)[16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int head = 32 * hb + 8 * (r >> 2) + 4 * hf + (r & 3);
    wv[r] = head < H ? wrow[head] : 0.0f;
  }
}

// relu(x) as one integer max on the bit pattern: every negative float
// (-0.0 included) is a negative integer, so max(bits, 0) gives +0.0 for
// them and leaves non-negative values unchanged (fmaxf would first quiet a
// possible signalling NaN, a second instruction per element).
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// The scores of a 64-key block from the per-half head sums of its two
// 32-key sub-blocks: lane (m, hf) holds p0, the sum over its half's heads
// for key m, and p1, the same for key 32 + m. One v_permlane32_swap moves p0
// of the upper half to the lower half and p1 of the lower half to the upper
// half, so lane l ends up with the score of key l (half 0 + half 1).
__device__ __forceinline__ float block_scores(float p0, float p1) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float relu_weighted_sum(const f32x16& acc, const float (&wv)[16]) {
  float part = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) part = fmaf(wv[r], relu_bits(acc[r]), part);
  return part;
}

// ---------------------------------------------------------------------------
// Streaming scorer (decode and any ragged layout with short query runs). A
// workgroup scores NSTG consecutive stages of 128 positions of one row: the
// keys of stages s + 1 .. s + 3 stream into a four-stage LDS ring by direct
// global->LDS loads while stage s is multiplied, and each consumed stage is
// refilled at once, so the loads in flight never drain. A load fills 1024 LDS bytes with 1024 / (2 D) consecutive
// positions of one page (one page-table entry per load); the 16-byte chunk c
// of key row r sits at slot c ^ (r % (D / 8)), so the 32 rows that a lane
// group reads at one chunk hit distinct banks. Wave w multiplies positions
// 32 w .. 32 w + 31 of each stage: A = query fragments (heads as M, resident),
// B = keys from LDS (N = 32 positions). Positions past the row's valid range
// load the sequence's first key and are never stored.
// grid = (ceil(cap / (128 NSTG)), T), block = 256, static LDS 4 x 128 x 2D.
// ---------------------------------------------------------------------------
constexpr int kStreamKeys = 128;  // positions per stage
constexpr int kStreamRing = 4;    // LDS stages: three in flight while one is used

__device__ __forceinline__ void gll16_idx(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// This wave's direct loads of one stage: load I (= NL wave + n) covers stage
// rows I * RPI + l / CPR; lane l fetches the chunk that belongs at its slot
// l % CPR, i.e. chunk (l % CPR) ^ (row % CPR). Since I * RPI is a multiple of
// RPI and l / CPR < RPI, row % CPR = (I * RPI) % CPR ^ (l / CPR) % CPR.
// Physical cache rows of one wave's NL loads of a stage (RPI rows each):
// load n starts at position j = j_stage + RPI (NL wave + n). The wave's
// positions span NL * RPI = 32 consecutive positions from a multiple of 32,
// and PS is a multiple of 16, so they touch at most two pages: two
// divisions and three page-table reads (wave-uniform, scalar) instead of a
// division and a read per load. A load past the row's valid positions reads
// position 0 (any valid row; its scores are never stored).
template <int NL, int RPI>
__device__ __forceinline__ void wave_stage_rows(const int32_t* __restrict__ ptrow, int num_pages,
                                                int PS, int j_stage, int n_valid, int wave,
                                                long (&row)[NL]) {
  static_assert(NL * RPI == 32, "a wave's loads of a stage cover 32 positions");
  const int jb = j_stage + NL * RPI * wave;
  const int p_lo = jb / PS;
  const int p_hi = (jb + NL * RPI - 1) / PS;  // p_lo or p_lo + 1
  const int q_lo = jb < n_valid ? p_lo : 0;
  const int q_hi = p_hi * PS < n_valid ? p_hi : q_lo;
  const long pg_lo = (long)clamp_page(ptrow[q_lo], num_pages) * PS;
  const long pg_hi = (long)clamp_page(ptrow[q_hi], num_pages) * PS;
  const long pg_0 = (long)clamp_page(ptrow[0], num_pages) * PS;
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int j = jb + RPI * n;
    row[n] = j >= n_valid ? pg_0 : (j < p_hi * PS ? pg_lo + (j - p_lo * PS) : pg_hi + (j - p_hi * PS));
  }
}

template <int D>
__device__ __forceinline__ void stream_stage(uint32_t buf, const uint16_t* __restrict__ cache,
                                             const int32_t* __restrict__ ptrow, int num_pages,
                                             int PS, int j_stage, int n_valid, int wave, int l) {
  constexpr int RB = 2 * D;                  // bytes per key row
  constexpr int RPI = 1024 / RB;             // rows per load
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NL = kStreamKeys / RPI / 4;  // loads per wave per stage
  const int lr = l / CPR, lc = l % CPR;
  const uint32_t voff = (uint32_t)(lr * RB + 16 * (lc ^ (lr % CPR)));
  long row[NL];
  wave_stage_rows<NL, RPI>(ptrow, num_pages, PS, j_stage, n_valid, wave, row);
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int I = NL * wave + n;
    gll16_idx(voff ^ (uint32_t)(16 * ((I * RPI) % CPR)), cache + (size_t)row[n] * D,
              buf + I * 1024);
  }
}

template <int D, int HB>
__global__ __launch_bounds__(256, 1) void idx_score_stream(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint16_t* __restrict__ cache, int num_pages, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu, int T, int S, int H,
    int PS, int MP, int NSTG, float* __restrict__ scores, long ld) {
  constexpr int KS = D / 16;
  constexpr int HALF = D / 2;
  constexpr int RB = 2 * D;
  constexpr int CPR = D / 8;
  constexpr int STAGE = kStreamKeys * RB;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStreamRing][STAGE];
  const int t = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = lane_id();
  const int m = l & 31, hf = l >> 5;
  const RowInfo ri = row_info_wave(cu, seq_lens, S, t, MP * PS);
  const int n = ri.n_valid;
  const int j_begin = blockIdx.x * NSTG * kStreamKeys;
  if (ri.seq < 0 || j_begin >= n) return;
  const int nst = min(NSTG, (n - j_begin + kStreamKeys - 1) / kStreamKeys);
  const int32_t* ptrow = pt + (size_t)ri.seq * MP;
  const uint32_t lds_ring =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring[0];
  constexpr int NL = kStreamKeys / (1024 / RB) / 4;  // loads per wave per stage

#pragma unroll
  for (int q2 = 0; q2 < kStreamRing - 1; ++q2)
    if (q2 < nst)
      stream_stage<D>(lds_ring + q2 * STAGE, cache, ptrow, num_pages, PS,
                      j_begin + q2 * kStreamKeys, n, wave, l);
  bf16x8 a[HB][KS];
  float wv[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 32 * hb + m;
    load_q_frag<D>(q + ((size_t)t * H + (head < H ? head : 0)) * D + hf * HALF, head < H, a[hb]);
    load_head_weights(w + (size_t)t * H, H, hb, hf, wv[hb]);
  }
  // complete these loads here, not at their first use inside the stage loop
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int i = 0; i < KS; ++i) asm volatile("" : : "v"(a[hb][i]));
#pragma unroll
    for (int r = 0; r < 16; ++r) asm volatile("" : : "v"(wv[hb][r]));
  }
  float* srow = scores + (size_t)t * ld;
  for (int s2 = 0; s2 < nst; ++s2) {
    const int j_stage = j_begin + s2 * kStreamKeys;
    // stages s2 + 1 .. s2 + kStreamRing - 2 were issued after this one
    const int later = min(kStreamRing - 2, nst - 1 - s2);
    if (later >= 2) wait_vm<2 * NL>();
    else if (later == 1) wait_vm<NL>();
    else wait_vm<0>();
    lds_sync();  // stage s2 has landed for every wave; stage s2 - 1 is consumed
    if (s2 + kStreamRing - 1 < nst)
      stream_stage<D>(lds_ring + ((s2 + kStreamRing - 1) % kStreamRing) * STAGE, cache, ptrow,
                      num_pages, PS, j_stage + (kStreamRing - 1) * kStreamKeys, n, wave, l);
    const unsigned char* buf = ring[s2 % kStreamRing];
#pragma unroll
    for (int blk = 0; blk < 1; ++blk) {
      const int kr = 32 * wave + m;  // key row within the stage
      const int j = j_stage + kr;
      bf16x8 b[KS];
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const int chunk = hf * HALF / 8 + i;  // dims hf * D / 2 + 8 i ..
        b[i] = as_bf16x8(*reinterpret_cast<const uint4*>(buf + kr * RB +
                                                          16 * (chunk ^ (kr % CPR))));
      }
      float part = 0.0f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        f32x16 acc = {};
#pragma unroll
        for (int i = 0; i < KS; ++i)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[hb][i], b[i], acc, 0, 0, 0);
        part += relu_weighted_sum(acc, wv[hb]);
      }
      part += shfl_xor_f(part, 32);
      if (hf == 0 && j < n) srow[j] = part;
    }
  }
}

// ---------------------------------------------------------------------------
// Balanced streaming scorer for ragged batches of more sequences than the
// register scorer below stages in LDS. The batch's work is the flat list of
// (row, 128-position stage) pairs in row order; each of G persistent
// workgroups (one per compute unit) takes an equal contiguous share of it, so
// rows of any length mix without a tail of part-filled workgroups, and the
// four-stage ring keeps streaming across row boundaries (one ring fill per
// workgroup instead of one per row piece).
//
// Every workgroup first computes each row's valid length and the prefix of
// stage counts (cu_q_lens and seq_lens staged in LDS, one binary search per
// row). The query rows of 32 heads and their weights travel with the first
// stage of each row through the same direct loads, into one of two LDS
// slots (alternating by row); the issue cursor never runs more than one row
// ahead of the compute cursor, so a slot is rewritten only after its row is
// done. Stage waits count only key loads, so a query load or a score store
// issued later can only make a wait longer, never too short.
// grid = (number of compute units), block = 256.
// ---------------------------------------------------------------------------
constexpr int kFlatMaxT = 1024;

template <int D>
struct FlatShape {
  static constexpr int RB = 2 * D;                   // bytes per key (and query) row
  static constexpr int STAGE = kStreamKeys * RB;
  static constexpr int QBYTES = 32 * RB;             // 32 head rows
  static constexpr int QSLOT = QBYTES + 256;         // + 64 fp32 weights
  // cu_q_lens and seq_lens are staged in the ring before it is used
  static constexpr int MAX_S = (kStreamRing * STAGE / 4 - 1) / 2;
};

__device__ __forceinline__ void gll16_ptr(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_addr)
               : "memory", "m0");
}

__device__ __forceinline__ void gll4_ptr(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(lds_addr)
               : "memory", "m0");
}

// Query rows of row t (heads >= H repeat head H - 1; they get weight 0) in
// the key layout, then the weights.
template <int D>
__device__ __forceinline__ void flat_issue_query(uint32_t slot, const uint16_t* __restrict__ q,
                                                 const float* __restrict__ w, int t, int H,
                                                 int wave, int l) {
  constexpr int RB = 2 * D, CPR = D / 8, RPI = 1024 / RB, NQ = 32 / RPI;
#pragma unroll
  for (int I = wave; I < NQ; I += 4) {
    const int h = I * RPI + l / CPR;
    const int hs = h < H ? h : H - 1;
    const int c = (l % CPR) ^ (h % CPR);
    gll16_ptr(q + ((size_t)t * H + hs) * D + 8 * c,
              __builtin_amdgcn_readfirstlane(slot + I * 1024));
  }
  if (wave == 3) gll4_ptr(w + (size_t)t * H + (l < H ? l : H - 1), slot + 32 * RB);
}

// Keys of one stage, the page-table entries of all of this wave's loads
// fetched before the first load is issued.
template <int D>
__device__ __forceinline__ void flat_issue_keys(uint32_t buf, const uint16_t* __restrict__ cache,
                                                const int32_t* __restrict__ ptrow, int num_pages,
                                                int PS, int j_stage, int n_valid, int wave,
                                                int l) {
  constexpr int RB = 2 * D, RPI = 1024 / RB, CPR = D / 8, NL = kStreamKeys / RPI / 4;
  const int lr = l / CPR, lc = l % CPR;
  const uint32_t voff = (uint32_t)(lr * RB + 16 * (lc ^ (lr % CPR)));
  long row[NL];
  wave_stage_rows<NL, RPI>(ptrow, num_pages, PS, j_stage, n_valid, wave, row);
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int I = NL * wave + n;
    const uint64_t src = (uint64_t)(uintptr_t)(cache + (size_t)row[n] * D);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)src);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(src >> 32));
    gll16_idx(voff ^ (uint32_t)(16 * ((I * RPI) % CPR)),
              (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo),
              __builtin_amdgcn_readfirstlane(buf + I * 1024));
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void idx_score_flat(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint16_t* __restrict__ cache, int num_pages, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu, int T, int S, int H,
    int PS, int MP, float* __restrict__ scores, long ld) {
  using F = FlatShape<D>;
  constexpr int KS = D / 16, HALF = D / 2, RB = F::RB, CPR = D / 8;
  constexpr int NL = kStreamKeys / (1024 / RB) / 4;  // key loads per wave per stage
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kStreamRing][F::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char qbuf[2][F::QSLOT];
  __shared__ int s_pre[kFlatMaxT + 1];
  __shared__ int s_n[kFlatMaxT];
  __shared__ int s_seq[kFlatMaxT];
  __shared__ int s_scan[4];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = lane_id();
  const int m = l & 31, hf = l >> 5;
  const int cap = MP * PS;

  // ---- valid length of every row and the prefix of its stage counts
  int* s_cu = reinterpret_cast<int*>(ring[0]);
  int* s_sl = s_cu + (S + 1);
  for (int i = tid; i <= S; i += 256) s_cu[i] = cu[i];
  for (int i = tid; i < S; i += 256) s_sl[i] = seq_lens[i];
  __syncthreads();
  const int R = (T + 255) / 256;  // rows per thread, consecutive
  int cnt = 0;
  for (int i = 0; i < R; ++i) {
    const int t = R * tid + i;
    if (t >= T) break;
    int seq = -1, n = 0;
    if (S > 0 && t >= s_cu[0] && t < s_cu[S]) {
      int lo = 0, hi = S;  // first s with cu[s + 1] > t
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_cu[mid + 1] > t) hi = mid; else lo = mid + 1;
      }
      if (lo < S) {
        const int q0 = s_cu[lo], q1 = s_cu[lo + 1];
        const int kv = s_sl[lo];
        const int abs_q = kv - (q1 - q0) + (t - q0);
        const int kc = kv < 0 ? 0 : (kv > cap ? cap : kv);
        n = abs_q + 1 < kc ? abs_q + 1 : kc;
        n = n < 0 ? 0 : n;
        seq = lo;
      }
    }
    s_n[t] = n;
    s_seq[t] = seq;
    cnt += (n + kStreamKeys - 1) / kStreamKeys;
  }
  int total;
  int run = block_inclusive_scan<256>(cnt, s_scan, &total) - cnt;
  for (int i = 0; i < R; ++i) {
    const int t = R * tid + i;
    if (t >= T) break;
    s_pre[t] = run;
    run += (s_n[t] + kStreamKeys - 1) / kStreamKeys;
  }
  if (tid == 0) s_pre[T] = total;
  __syncthreads();  // also: the staging area is free for the ring

  // ---- this workgroup's share [f_begin, f_end) of the flat stage list
  const int G = gridDim.x;
  total = __builtin_amdgcn_readfirstlane(total);
  const int f_begin = (int)((long)blockIdx.x * total / G);
  const int f_end = (int)((long)(blockIdx.x + 1) * total / G);
  if (f_begin >= f_end) return;
  int r0 = 0;
  {
    int lo = 0, hi = T - 1;  // last row with s_pre[row] <= f_begin (it has stages)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= f_begin) lo = mid; else hi = mid - 1;
    }
    r0 = __builtin_amdgcn_readfirstlane(lo);
  }
  const uint32_t lds_ring = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring[0];
  const uint32_t lds_q = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)qbuf[0];
  auto pre = [&](int r) { return __builtin_amdgcn_readfirstlane(s_pre[r]); };

  // issue cursor: next stage fi, its row ri and the row's ordinal ki
  int fi = f_begin, ri = r0, ki = 0;
  // compute cursor: row rc and ordinal kc of the stage being computed
  int rc = r0, kc = 0;
  auto issue = [&]() {
    fi = __builtin_amdgcn_readfirstlane(fi);
    ri = __builtin_amdgcn_readfirstlane(ri);
    ki = __builtin_amdgcn_readfirstlane(ki);
    const int base = pre(ri);
    if (fi == f_begin || fi == base)
      flat_issue_query<D>(lds_q + (ki & 1) * F::QSLOT, q, w, ri, H, wave, l);
    const int seq = __builtin_amdgcn_readfirstlane(s_seq[ri]);
    const int n = __builtin_amdgcn_readfirstlane(s_n[ri]);
    flat_issue_keys<D>(lds_ring + (fi % kStreamRing) * F::STAGE, cache, pt + (size_t)seq * MP,
                       num_pages, PS, (fi - base) * kStreamKeys, n, wave, l);
    ++fi;
    if (fi < f_end && fi >= pre(ri + 1)) {
      do { ++ri; } while (pre(ri + 1) <= fi);
      ++ki;
    }
  };
  while (fi < f_end && fi < f_begin + kStreamRing - 1 && ki <= 1) issue();

  bf16x8 a[KS];
  float wv[16];
  int n_c = 0, base_c = 0;
  float* srow = scores;
  for (int fc = f_begin; fc < f_end; ++fc) {
    const int later = fi - fc - 1;  // stages issued after this one (0 .. 2)
    if (later >= 2) wait_vm<2 * NL>();
    else if (later == 1) wait_vm<NL>();
    else wait_vm<0>();
    lds_sync();  // stage fc (and its row's query) landed; stage fc - 1 is consumed
    bool fresh = fc == f_begin;
    if (fc >= pre(rc + 1)) {
      do { ++rc; } while (pre(rc + 1) <= fc);
      ++kc;
      fresh = true;
    }
    while (fi < f_end && fi <= fc + kStreamRing - 1 && ki <= kc + 1) issue();
    if (fresh) {
      const unsigned char* qs = qbuf[kc & 1];
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        const int chunk = hf * HALF / 8 + i;
        const uint4 v = *reinterpret_cast<const uint4*>(qs + m * RB + 16 * (chunk ^ (m % CPR)));
        a[i] = as_bf16x8(m < H ? v : zero_u4());
      }
      const float* wl = reinterpret_cast<const float*>(qs + F::QBYTES);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int head = 8 * (r >> 2) + 4 * hf + (r & 3);
        wv[r] = head < H ? wl[head] : 0.0f;
      }
      n_c = __builtin_amdgcn_readfirstlane(s_n[rc]);
      base_c = pre(rc);
      srow = scores + (size_t)rc * ld;
    }
    const unsigned char* buf = ring[fc % kStreamRing];
    const int kr = 32 * wave + m;  // key row within the stage
    const int j = (fc - base_c) * kStreamKeys + kr;
    bf16x8 b[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int chunk = hf * HALF / 8 + i;
      b[i] = as_bf16x8(*reinterpret_cast<const uint4*>(buf + kr * RB + 16 * (chunk ^ (kr % CPR))));
    }
    f32x16 acc = {};
#pragma unroll
    for (int i = 0; i < KS; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], acc, 0, 0, 0);
    float part = relu_weighted_sum(acc, wv);
    part += shfl_xor_f(part, 32);
    if (hf == 0 && j < n_c) srow[j] = part;
  }
}

// ---------------------------------------------------------------------------
// Register-streaming scorer for ragged batches. The work items are the
// 32-position blocks of every row, in row order, and each wave of the grid
// takes an equal contiguous share of them. A lane loads the half of its key
// that its MFMA operand needs (D / 2 values, D / 16 loads of 16 bytes)
// straight into registers: no LDS staging, and no barrier or wait that
// another wave shares stands between a block's loads and its products. While
// a block is multiplied, the keys of the next block and the page-table
// entries of the two after it are in flight. A position past the row's valid
// range loads a key of the row's last valid page (the last valid key when PS
// is not a multiple of 32) and is never stored. Each workgroup
// first finds every row's valid length and the prefix of its block counts
// (cu_q_lens and seq_lens staged in LDS, one binary search per row).
// Scores go to a per-wave LDS buffer and are stored 32 blocks at a time
// (1 KB per store instruction): the ragged decode's writes, spread one
// 128-byte line per block between its key reads, cost about 8 us of 68;
// grouped they cost about 4.
// grid = (several workgroups per compute unit), block = 256.
// ---------------------------------------------------------------------------
constexpr int kRegKeys = 32;        // positions per work item
constexpr int kRegMaxS = 1024;      // sequences the staging area holds
constexpr int kRegWavesPerSimd = 3;
constexpr int kRegBatch = 32;  // blocks whose scores a wave stores at once

template <int D, bool P32>
__global__ __launch_bounds__(256, kRegWavesPerSimd) void idx_score_regs(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint16_t* __restrict__ cache, int num_pages, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu, int T, int S, int H,
    int PS, int MP, float* __restrict__ scores, long ld) {
  constexpr int KS = D / 16;
  __shared__ int s_pre[kFlatMaxT + 1];
  __shared__ int s_n[kFlatMaxT];
  __shared__ int s_seq[kFlatMaxT];
  __shared__ int s_cu[kRegMaxS + 1];
  __shared__ int s_sl[kRegMaxS];
  __shared__ int s_scan[4];
  // per wave: the scores of up to kRegBatch blocks, stored in one pass
  __shared__ __attribute__((aligned(16))) float s_out[4][kRegBatch * kRegKeys];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = lane_id();
  const int m = l & 31, hf = l >> 5;
  const int cap = MP * PS;

  // ---- valid length of every row and the prefix of its block counts
  for (int i = tid; i <= S; i += 256) s_cu[i] = cu[i];
  for (int i = tid; i < S; i += 256) s_sl[i] = seq_lens[i];
  __syncthreads();
  const int R = (T + 255) / 256;  // rows per thread, consecutive
  int cnt = 0;
  for (int i = 0; i < R; ++i) {
    const int t = R * tid + i;
    if (t >= T) break;
    int seq = -1, n = 0;
    if (S > 0 && t >= s_cu[0] && t < s_cu[S]) {
      int lo = 0, hi = S;  // first s with cu[s + 1] > t
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_cu[mid + 1] > t) hi = mid; else lo = mid + 1;
      }
      if (lo < S) {
        const int q0 = s_cu[lo], q1 = s_cu[lo + 1];
        const int kv = s_sl[lo];
        const int abs_q = kv - (q1 - q0) + (t - q0);
        const int kc = kv < 0 ? 0 : (kv > cap ? cap : kv);
        n = abs_q + 1 < kc ? abs_q + 1 : kc;
        n = n < 0 ? 0 : n;
        seq = lo;
      }
    }
    s_n[t] = n;
    s_seq[t] = seq;
    cnt += (n + kRegKeys - 1) / kRegKeys;
  }
  int total;
  int run = block_inclusive_scan<256>(cnt, s_scan, &total) - cnt;
  for (int i = 0; i < R; ++i) {
    const int t = R * tid + i;
    if (t >= T) break;
    s_pre[t] = run;
    run += (s_n[t] + kRegKeys - 1) / kRegKeys;
  }
  if (tid == 0) s_pre[T] = total;
  __syncthreads();

  // ---- this wave's share [i_begin, i_end) of the block list
  const int G = gridDim.x * 4;
  const int gw = blockIdx.x * 4 + wave;
  total = __builtin_amdgcn_readfirstlane(total);
  const int i_begin = (int)((long)gw * total / G);
  const int i_end = (int)((long)(gw + 1) * total / G);
  if (i_begin >= i_end) return;  // no barrier follows
  auto pre = [&](int r) { return __builtin_amdgcn_readfirstlane(s_pre[r]); };
  int r = 0;
  {
    int lo = 0, hi = T - 1;  // last row with s_pre[row] <= i_begin (it has blocks)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= i_begin) lo = mid; else hi = mid - 1;
    }
    r = __builtin_amdgcn_readfirstlane(lo);
  }
  // The share is walked one row segment at a time (most waves have one).
  // Lane (m, hf) holds, for k-step x, the 8 values 16 x + 8 hf .. of its
  // query head m (operand A) and of its key m (operand B): the two lanes of
  // a key read 32 consecutive bytes per load.
  for (int i = i_begin; i < i_end;) {
    const int base = pre(r);
    const int seg_end = min(i_end, pre(r + 1));
    const int nrow = __builtin_amdgcn_readfirstlane(s_n[r]);
    const int seq = __builtin_amdgcn_readfirstlane(s_seq[r]);
    const int32_t* ptrow = pt + (size_t)seq * MP;
    bf16x8 a[KS];
    float wv[16];
    {
      const bool okq = m < H;
      const uint16_t* qrow = q + ((size_t)r * H + (okq ? m : 0)) * D + 8 * hf;
#pragma unroll
      for (int x = 0; x < KS; ++x)
        a[x] = as_bf16x8(okq ? *reinterpret_cast<const uint4*>(qrow + 16 * x) : zero_u4());
      load_head_weights(w + (size_t)r * H, H, 0, hf, wv);
    }
    const int b0 = i - base, bend = seg_end - base;
    // block bb of the row, clamped to the segment's last block (loads past
    // the segment repeat that block and are never multiplied)
    auto key_j = [&](int bb) {
      const int j = min(bb, bend - 1) * kRegKeys + m;
      return j < nrow ? j : nrow - 1;
    };
    // P32 (PS a multiple of 32): a block's 32 positions share one page, whose
    // entry is read once for the wave; positions past the row's end then
    // stay inside that page and are never stored
    auto entry = [&](int bb) {
      if constexpr (P32)
        return ptrow[__builtin_amdgcn_readfirstlane(min(bb, bend - 1) * kRegKeys) / PS];
      else
        return ptrow[key_j(bb) / PS];
    };
    const uint16_t* lane_base = cache + (size_t)m * D + 8 * hf;
    auto load = [&](int bb, int pe, bf16x8 (&kk)[KS]) __attribute__((always_inline)) {
      const uint16_t* src;
      if constexpr (P32) {
        const int j0 = __builtin_amdgcn_readfirstlane(min(bb, bend - 1) * kRegKeys);
        const int pg = clamp_page(__builtin_amdgcn_readfirstlane(pe), num_pages);
        src = lane_base + ((size_t)pg * PS + (size_t)(j0 % PS)) * D;
      } else {
        const int j = key_j(bb);
        src = cache + ((size_t)clamp_page(pe, num_pages) * PS + (size_t)(j % PS)) * D + 8 * hf;
      }
#pragma unroll
      for (int x = 0; x < KS; ++x)
        kk[x] = as_bf16x8(*reinterpret_cast<const uint4*>(src + 16 * x));
    };
    float* srow = scores + (size_t)r * ld;
    float* sbuf = s_out[wave];
    // scores of blocks fb .. fb + nb - 1 from the wave's buffer to the row:
    // lane l writes positions 4 l .. 4 l + 3 of the batch
    auto flush = [&](int fb, int nb) __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      const int lim = min(nb * kRegKeys, nrow - fb * kRegKeys);  // valid positions of the batch
#pragma unroll
      for (int u = 0; u < kRegBatch / 8; ++u) {
        const int o = 256 * u + 4 * l;           // this lane's positions in the batch
        const int p = fb * kRegKeys + o;
        const float4 v = *reinterpret_cast<const float4*>(sbuf + o);
        if (o + 3 < lim) {
          *reinterpret_cast<float4*>(srow + p) = v;
        } else if (o < lim) {
          srow[p] = v.x;
          if (o + 1 < lim) srow[p + 1] = v.y;
          if (o + 2 < lim) srow[p + 2] = v.z;
        }
      }
      asm volatile("" ::: "memory");
    };
    auto product = [&](int bb, const bf16x8 (&kk)[KS]) __attribute__((always_inline)) {
      f32x16 acc = {};
#pragma unroll
      for (int x = 0; x < KS; ++x)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[x], kk[x], acc, 0, 0, 0);
      float part = relu_weighted_sum(acc, wv);
      part += shfl_xor_f(part, 32);
      const int slot = (bb - b0) % kRegBatch;
      if (hf == 0) sbuf[slot * kRegKeys + m] = part;
      if (slot == kRegBatch - 1) flush(bb - slot, kRegBatch);
    };
    // keys one block ahead of the products, page entries three
    bf16x8 k0[KS], k1[KS];
    int b = b0;
    load(b, entry(b), k0);
    int pe_b = entry(b + 1), pe_c = entry(b + 2);
    for (; b < bend; b += 2) {
      load(b + 1, pe_b, k1);
      const int pe_d = entry(b + 3);
      // keep the loads ahead of the products (the scheduler would sink them)
      __builtin_amdgcn_sched_barrier(0);
      product(b, k0);
      if (b + 1 >= bend) break;
      load(b + 2, pe_c, k0);
      const int pe_e = entry(b + 4);
      __builtin_amdgcn_sched_barrier(0);
      product(b + 1, k1);
      pe_b = pe_d;
      pe_c = pe_e;
    }
    if ((bend - b0) % kRegBatch != 0) {  // the segment's last, partial batch
      const int nb = (bend - b0) % kRegBatch;
      flush(bend - nb, nb);
    }
    i = seg_end;
    ++r;
    while (r < T - 1 && pre(r + 1) <= i) ++r;  // skip rows without blocks
  }
}

// ---------------------------------------------------------------------------
// Tiled MFMA scorer for query chunks (extend). A workgroup of 8 waves owns 8
// consecutive packed rows (wave w: row t0 + w, its query fragments and head
// weights in registers) and a range of up to kTileMaxRK key positions. The
// keys stream through a four-stage LDS ring of 64-key blocks by direct
// global->LDS loads (three blocks in flight while one is multiplied), in the
// row-group layout of TileLayout, and every staged block serves all 8 rows.
// A wave stores its row's 64 scores of a block with one instruction
// (lane l: key l), so the waits on the ring count every outstanding memory
// operation exactly: the key loads of later blocks plus the stores of the
// last three blocks. Rows of a tile may belong to several sequences: the
// tile is walked one sequence segment at a time. With EXT each active wave
// also writes its row's smallest and largest order key over the tile to
// ext[t, tile] (the full key range when a score is NaN); the top-k of rows
// longer than one select chunk takes its bucket range from these instead of
// reading the scores an extra time.
// grid = (ceil(cap / kTileMaxRK), ceil(T / 8)), block = 512.
// ---------------------------------------------------------------------------
constexpr int kTileMaxRK = 2048;  // key range of one tile workgroup
// Rows per workgroup, one per wave. The score-matrix scorer takes 8 (two
// workgroups per compute unit). The fused scorer takes 16 with one head
// block, so that every staged block serves 16 rows and each wave issues one
// direct load per block, and 8 with two (their query fragments need twice
// the registers).
constexpr int kTileRows = 8;
template <int HB>
constexpr int fused_rows() { return HB == 1 ? 16 : 8; }
constexpr int kTileKB = 64;       // keys per staged block

// Staged block layout of the tile scorers. One direct load fills 1024 LDS
// bytes with RPI = 1024 / (2 D) consecutive key rows, a row group: slot s of
// the group holds 16-byte chunk s / RPI of row s % RPI (chunk-major), and
// consecutive groups start GS = 1024 + 16 RPI bytes apart. The fragment a
// lane reads for k-step i is then its own base address plus 16 RPI i, an
// immediate offset of the LDS read, so the reads of a block need no address
// arithmetic. A read phase (8 or 16 consecutive lanes: rows m .. m + 15 at
// one chunk) hits distinct banks: the rows of a group are contiguous, and
// each further group is shifted by 16 RPI bytes modulo 256.
// Page-table entries of a key range kept in registers: entry pg0 + 64 c + i
// of the range in lane i of pgv[c]. A direct load's source page is read back
// with v_readlane at a wave-uniform index, so staging a block needs no LDS
// round trip (an LDS read there queued behind the key fragment reads of all
// the other waves).
constexpr int kTilePgRegs = (kTileMaxRK / 16 + 1 + 63) / 64;

__device__ __forceinline__ void load_page_regs(const int32_t* __restrict__ ptrow, int n, int l,
                                               int (&pgv)[kTilePgRegs]) {
#pragma unroll
  for (int c = 0; c < kTilePgRegs; ++c) {
    const int i = 64 * c + l;
    pgv[c] = i < n ? ptrow[i] : 0;
  }
}

// entry p (wave-uniform, p < 64 kTilePgRegs)
__device__ __forceinline__ int page_reg(const int (&pgv)[kTilePgRegs], int p) {
  int v = __builtin_amdgcn_readlane(pgv[0], p & 63);
#pragma unroll
  for (int c = 1; c < kTilePgRegs; ++c)
    if (p >= 64 * c) v = __builtin_amdgcn_readlane(pgv[c], p & 63);
  return v;
}

template <int D>
struct TileLayout {
  static constexpr int RB = 2 * D;                  // bytes per key row
  static constexpr int RPI = 1024 / RB;             // rows per group (per load)
  static constexpr int GS = 1024 + 16 * RPI;        // group stride
  static constexpr int NLB = kTileKB * RB / 1024;   // groups (loads) per block
  static constexpr int BLK = NLB * GS;              // bytes per staged block
  static constexpr int SUB = (32 / RPI) * GS;       // bytes per 32 rows
  // lane l of a load fetches chunk l / RPI of group row l % RPI
  static __device__ __forceinline__ uint32_t load_off(int l) {
    return (uint32_t)((l % RPI) * RB + 16 * (l / RPI));
  }
  // base of lane (m, hf)'s fragments: row m of a 32-row sub-block, the
  // chunks of contraction half hf
  static __device__ __forceinline__ int read_base(int m, int hf) {
    return (m / RPI) * GS + 16 * (m % RPI) + 16 * RPI * (hf * (D / 16));
  }
};
constexpr int kTileRing = 4;

// s_waitcnt vmcnt(n) for a wave-uniform n in 0 .. 15
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;
    case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break;
    case 11: wait_vm<11>(); break;
    case 12: wait_vm<12>(); break;
    case 13: wait_vm<13>(); break;
    case 14: wait_vm<14>(); break;
    default: wait_vm<15>(); break;
  }
}

template <int D, int HB, bool EXT>
__global__ __launch_bounds__(64 * kTileRows, 2) void idx_score_tiles(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint16_t* __restrict__ cache, int num_pages, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu, int T, int S, int H,
    int PS, int MP, float* __restrict__ scores, long ld, uint2* __restrict__ ext, int ext_ld) {
  using TL = TileLayout<D>;
  constexpr int KS = D / 16, HALF = D / 2, RPI = TL::RPI;
  constexpr int BLK = TL::BLK;           // bytes per staged block
  constexpr int NLB = TL::NLB;           // direct loads per block (D / 8)
  constexpr int R = kTileRows;
  constexpr int NLW = (NLB + R - 1) / R;  // at most this many per wave
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kTileRing][BLK];
  __shared__ int s_seq[R], s_nv[R];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = lane_id();
  const int m = l & 31, hf = l >> 5;
  const int t0 = blockIdx.y * R;
  const int cap = MP * PS;
  if (tid < R) {
    const int t = t0 + tid;
    RowInfo ri;
    ri.seq = -1;
    ri.n_valid = 0;
    if (t < T) ri = row_info(cu, seq_lens, S, t, cap);
    s_seq[tid] = ri.seq;
    s_nv[tid] = ri.n_valid;
  }
  __syncthreads();
  const int k0 = blockIdx.x * kTileMaxRK;
  const uint32_t lds_ring = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring[0];
  const uint32_t voff = TL::load_off(l);
  const int rbase = TL::read_base(m, hf);

  int seg = 0;
  while (seg < R) {
    const int s = __builtin_amdgcn_readfirstlane(s_seq[seg]);
    int seg_end = seg + 1;
    while (seg_end < R && s_seq[seg_end] == s) ++seg_end;
    seg_end = __builtin_amdgcn_readfirstlane(seg_end);
    const int n_hi = s >= 0 ? __builtin_amdgcn_readfirstlane(s_nv[seg_end - 1]) : 0;
    const int k1 = min(k0 + kTileMaxRK, n_hi);
    if (s >= 0 && k0 < k1) {
      const int pg0 = k0 / PS;
      int pgv[kTilePgRegs];
      load_page_regs(pt + (size_t)s * MP + pg0, (k1 - 1) / PS - pg0 + 1, l, pgv);
      // this wave's row, if it belongs to the segment
      const int r = wave;
      const int nv = s_nv[r];
      const bool act = r >= seg && r < seg_end && nv > k0;
      const int t = t0 + r;
      bf16x8 a[HB][KS];
      float wv[HB][16];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const int head = 32 * hb + m;
        const bool okq = act && head < H;
        load_q_frag<D>(q + ((size_t)(okq ? t : 0) * H + (head < H ? head : 0)) * D + hf * HALF,
                       okq, a[hb]);
        load_head_weights(w + (size_t)(act ? t : 0) * H, H, hb, hf, wv[hb]);
      }
      // complete these loads before the ring loads are issued
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int i = 0; i < KS; ++i) asm volatile("" : : "v"(a[hb][i]));
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("" : : "v"(wv[hb][i]));
      }
#pragma unroll
      for (int c = 0; c < kTilePgRegs; ++c) asm volatile("" : : "v"(pgv[c]));

      const int nb = (k1 - k0 + kTileKB - 1) / kTileKB;
      const int nlw = wave < NLB % R || NLB % R == 0 ? NLW : NLW - 1;  // this wave's loads per block
      // direct loads of block b: load I = wave + R n covers rows I * RPI .. of the block
      auto stage = [&](int b) {
        const uint32_t buf = lds_ring + (b % kTileRing) * BLK;
#pragma unroll
        for (int n = 0; n < NLW; ++n) {
          const int I = wave + R * n;
          if (I < NLB) {
            int j0 = k0 + b * kTileKB + I * RPI;
            if (j0 >= k1) j0 = k0;  // past the range: any staged row, never stored
            const int page = clamp_page(page_reg(pgv, j0 / PS - pg0), num_pages);
            const uint64_t src =
                (uint64_t)(uintptr_t)(cache + ((size_t)page * PS + (j0 % PS)) * D);
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)src);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(src >> 32));
            gll16_idx(voff, (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo),
                      __builtin_amdgcn_readfirstlane(buf + I * TL::GS));
          }
        }
      };
#pragma unroll
      for (int b = 0; b < kTileRing - 1; ++b)
        if (b < nb) stage(b);
      float* srow = scores + (size_t)(act ? t : 0) * ld;
      int hist = 0;  // bit i: this wave stored a block i + 1 iterations ago
      // extremes of this lane's stored scores (a NaN widens the range to all keys)
      float fmn = __builtin_inff(), fmx = -__builtin_inff();
      int nan = 0;
      for (int b = 0; b < nb; ++b) {
        // outstanding after block b's loads: the loads of the blocks issued
        // after it and the stores of the last three iterations
        const int later = min(kTileRing - 2, nb - 1 - b);
        wait_vm_dyn(later * nlw + __popc(hist & 7));
        lds_sync();  // block b has landed for every wave; block b - 1 is consumed
        if (b + kTileRing - 1 < nb) stage(b + kTileRing - 1);
        hist <<= 1;
        if (!act || k0 + b * kTileKB >= nv) continue;  // wave-uniform
        const unsigned char* buf = ring[b % kTileRing];
        float sc[kTileKB / 32];
#pragma unroll
        for (int sb = 0; sb < kTileKB / 32; ++sb) {
          bf16x8 bk[KS];
#pragma unroll
          for (int i = 0; i < KS; ++i)
            bk[i] = as_bf16x8(*reinterpret_cast<const uint4*>(buf + rbase + sb * TL::SUB +
                                                             16 * RPI * i));
          float part = 0.0f;
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            f32x16 acc = {};
#pragma unroll
            for (int i = 0; i < KS; ++i)
              acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[hb][i], bk[i], acc, 0, 0, 0);
            part += relu_weighted_sum(acc, wv[hb]);
          }
          sc[sb] = part + shfl_xor_f(part, 32);  // both lane halves hold key sb * 32 + m
        }
        // lane l stores key l of the block (j < nv holds for lane 0 here)
        const int j = k0 + b * kTileKB + l;
        if (j < nv) {
          const float v = hf ? sc[1] : sc[0];
          srow[j] = v;
          if (EXT) {
            fmn = fminf(fmn, v);
            fmx = fmaxf(fmx, v);
            nan |= v != v;
          }
        }
        hist |= 1;
      }
      // the row's extreme order keys over this tile (at least position k0 is
      // valid when the wave is active), for the select's bucket range; the
      // order key is monotone in the score, so it is taken of the extremes
      if (EXT && act) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          fmn = fminf(fmn, __shfl_xor(fmn, o, DSA_WAVE));
          fmx = fmaxf(fmx, __shfl_xor(fmx, o, DSA_WAVE));
          nan |= __shfl_xor(nan, o, DSA_WAVE);
        }
        if (l == 0)
          ext[(size_t)t * ext_ld + blockIdx.x] =
              nan ? make_uint2(0u, ~0u) : make_uint2(score_order_bits(fmn), score_order_bits(fmx));
      }
      __syncthreads();  // the ring is free for the next segment
    }
    seg = seg_end;
  }
}

// ---------------------------------------------------------------------------
// Exact top-k per row.
//
// Every score maps to a 32-bit order key (larger key = larger score, -0.0
// folded onto +0.0). Radix select narrows down the boundary: 12-bit digits
// from the top, each a histogram pass over the row, until the keys above the
// boundary bin plus the bin itself fit the list capacity (or all 32 bits are
// fixed). A collect pass then compacts those keys, in POSITION order, into
// one list; when the bin is a single exact key, only its first ties (lowest
// positions) are taken. The answer is the list ordered by key descending,
// list index ascending (for equal keys that is position ascending), cut at k:
// entries are bucketed by key (at most 4096 buckets over the listed keys'
// span) and each one's place is its bucket's start plus the number of bucket
// members ahead of it. Should a bucket hold more than kRankBucketMax entries,
// a stable block radix sort over the bits in which the keys differ orders the
// list instead.
//
// Each thread owns M consecutive positions of a chunk (M = 8 when a score
// row holds at most 8192 positions, else 16); the first chunk (the whole row
// when it has at most kSelNT * M positions), and the second as well when a
// row holds at most two, is read once, before the row's bounds are known,
// and kept in registers for every pass.
// grid = T, block = 1024, dynamic LDS = select_lds_bytes(k).
// ---------------------------------------------------------------------------
constexpr int kSelNT = 1024;

// Bin d of an nb-bin histogram holding the need-th largest key (counting
// from the top bin down); writes (d, count above d) to out[0..1].
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nb, int need, int* s_scan,
                                           int* out) {
  constexpr int BPT = 4096 / kSelNT;
  const int tid = threadIdx.x;
  int local = 0;
#pragma unroll
  for (int c = 0; c < BPT; ++c) {
    const int b = nb - 1 - tid * BPT - c;
    if (b >= 0) local += (int)hist[b];
  }
  int total;
  const int incl = block_inclusive_scan<kSelNT>(local, s_scan, &total);
  const int excl = incl - local;
  if (excl < need && need <= incl) {
    int run = excl;
#pragma unroll
    for (int c = 0; c < BPT; ++c) {
      const int b = nb - 1 - tid * BPT - c;
      if (b < 0) break;
      const int h = (int)hist[b];
      if (run + h >= need) {
        out[0] = b;
        out[1] = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
}

// Keys of positions c0 + M * tid + e (e < M); positions >= n get 0.
template <int M>
__device__ __forceinline__ void load_keys(const float* row, int n, int c0, uint32_t (&keys)[M]) {
  const int j0 = c0 + threadIdx.x * M;
  if (j0 + M <= n) {
#pragma unroll
    for (int e = 0; e < M; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + j0 + e);
      keys[e] = score_order_bits(v.x);
      keys[e + 1] = score_order_bits(v.y);
      keys[e + 2] = score_order_bits(v.z);
      keys[e + 3] = score_order_bits(v.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) keys[e] = (j0 + e < n) ? score_order_bits(row[j0 + e]) : 0u;
  }
}

// Keys of the first chunk, read before the row's length is known: every
// position below `lim` (the workspace row length capped at the chunk, a
// multiple of M) is loaded. Keys at positions >= n hold whatever the
// workspace holds there; every later use of them is guarded by j < n.
template <int M>
__device__ __forceinline__ void load_keys_ahead(const float* row, int lim, uint32_t (&keys)[M]) {
  const int j0 = threadIdx.x * M;
  if (j0 < lim) {
#pragma unroll
    for (int e = 0; e < M; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(row + j0 + e);
      keys[e] = score_order_bits(v.x);
      keys[e + 1] = score_order_bits(v.y);
      keys[e + 2] = score_order_bits(v.z);
      keys[e + 3] = score_order_bits(v.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) keys[e] = 0u;
  }
}

template <int IPT>
struct SelectCfg {
  static constexpr int CAP = kSelNT * IPT;  // list capacity
  static_assert(CAP <= kSelNT * 8, "the short-row path keeps the row in one chunk");
  using Sorter = rocprim::block_radix_sort<uint32_t, kSelNT, IPT, int>;
  // LDS: list key/pos [CAP] | hist/cursor [4096] | bucket start [4096 + 64]
  //      | bucket-ordered key [CAP] | bucket-ordered list index (u16) [CAP]
  static constexpr size_t LIST_BYTES = (size_t)CAP * 8;
  static constexpr size_t HIST_OFF = LIST_BYTES;
  static constexpr size_t START_OFF = HIST_OFF + 4096 * 4;
  static constexpr size_t SKEY_OFF = START_OFF + (4096 + 64) * 4;
  static constexpr size_t SIDX_OFF = SKEY_OFF + (size_t)CAP * 4;
  static constexpr size_t RANK_BYTES = SIDX_OFF + (size_t)CAP * 2;
  static constexpr size_t SEL_BYTES = RANK_BYTES > sizeof(typename Sorter::storage_type)
                                          ? RANK_BYTES
                                          : sizeof(typename Sorter::storage_type);
  // direct rank of a short row (the same LDS, used before the select path):
  // cursor [4096] | bucket start [4096 + 64] | (key, position) composite
  // [CAP + 64] for the positions whose bucket starts below k (k <= CAP / 2)
  static constexpr size_t D_CUR_OFF = 0;
  static constexpr size_t D_START_OFF = 4096 * 4;
  static constexpr size_t D_KEY_OFF = D_START_OFF + (4096 + 64) * 4;
  // | speculative candidates of a row of several chunks (composites) [SPEC]
  static constexpr int SPEC = IPT == 8 ? 6144 : CAP;
  static constexpr size_t D_SPEC_OFF = D_KEY_OFF + ((size_t)CAP + 64) * 8;
  static constexpr size_t DIRECT_BYTES = D_SPEC_OFF + (size_t)SPEC * 8;
  static constexpr size_t BYTES = SEL_BYTES > DIRECT_BYTES ? SEL_BYTES : DIRECT_BYTES;
};

// Largest bucket the rank phase handles; beyond it the list is sorted.
constexpr int kRankBucketMax = 256;
// Largest bucket of the direct rank of a short row; beyond it the row takes
// the radix-select path.
constexpr int kDirectBucketMax = 64;

__device__ __forceinline__ float order_key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Direct rank of a row of n <= kDirectMaxN positions. Thread tid owns
// positions c0 + M * tid + e of every chunk c0; the first chunk's keys are in
// registers, later chunks are read again from the row. Scores are bucketed
// by value, b = (vmax - v) * 4095.5 / (vmax - vmin) (monotone, so equal
// scores share a bucket and a larger score never lands in a later bucket).
// Only positions whose bucket starts below k can be in the answer; each
// one's place is its bucket's start plus the number of bucket members ahead
// of it (larger key, or equal key and smaller position: one comparison of
// the composite key << 32 | ~position). Returns false, having written
// nothing, when the spread is degenerate or a candidate bucket holds more
// than kDirectBucketMax positions. Five block barriers. When the row fits one
// chunk, the histogram's atomic returns each key's offset inside its bucket,
// so the candidates are placed without a second round of atomics. A row of
// two chunks held in registers counts both and takes its candidates from the
// registers in a second pass. A longer row counts its first chunk alone
// (three more barriers), takes from that count a bucket beyond which the
// candidates most likely do not reach, and lists every key up to it during
// the histogram pass; when the row's last candidate bucket is within that
// bound and the list did not overflow, the candidates come from the list,
// else from a second pass.
constexpr int kDirectMaxN = 1 << 17;

struct DirectShared {
  uint32_t red[2][kSelNT / 64];  // per-wave key minimum / maximum
  int wsum[kSelNT / 64];         // per-wave bucket-count sums
  int wbig[kSelNT / 64];         // per-wave "oversized candidate bucket" flags
  int lim;                       // end of the bucket holding place k - 1
  int blast;                     // that bucket (candidates are the buckets up to it)
  int spec_n;                    // speculative candidates listed (may exceed the list)
  int spec_b;                    // their last bucket
};

template <int NT, int M, int R>
__device__ __forceinline__ bool topk_direct(const uint32_t (&k0)[M], const uint32_t (&k1)[M],
                                            const float* row, int n,
                                            int k, uint32_t* lds, size_t cur_off,
                                            size_t start_off, size_t key_off, size_t spec_off,
                                            int spec_cap, DirectShared& sh,
                                            const uint2* __restrict__ ext_row,
                                            int32_t* __restrict__ orow) {
  constexpr int C = NT * M;
  constexpr int BPT = 4096 / NT;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
  uint32_t* cursor = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(lds) + cur_off);
  int* bstart = reinterpret_cast<int*>(reinterpret_cast<char*>(lds) + start_off);
  uint64_t* scomp = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(lds) + key_off);
  uint64_t* spec = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(lds) + spec_off);
  // keys of chunk c0 (the first R chunks from registers)
  auto chunk_keys = [&](int c0, uint32_t (&keys)[M]) {
    if (c0 == 0) {
#pragma unroll
      for (int e = 0; e < M; ++e) keys[e] = k0[e];
    } else if (R == 2 && c0 == C) {
#pragma unroll
      for (int e = 0; e < M; ++e) keys[e] = k1[e];
    } else {
      load_keys<M>(row, n, c0, keys);
    }
  };
  // ---- phase 1: clear the bucket counters; key minimum and maximum
#pragma unroll
  for (int u = 0; u < BPT; ++u) cursor[tid * BPT + u] = 0u;
  if (tid == 0) {
    sh.spec_n = 0;
    sh.spec_b = -1;
  }
  uint32_t kmin = ~0u, kmax = 0u;
  if (ext_row != nullptr && n > C) {
    // a row of several chunks: the scorer's per-tile extremes instead of a
    // pass over the later chunks
    for (int i = tid; i < (n + kTileMaxRK - 1) / kTileMaxRK; i += NT) {
      const uint2 e = ext_row[i];
      kmin = min(kmin, e.x);
      kmax = max(kmax, e.y);
    }
  } else {
    for (int c0 = 0; c0 < n; c0 += C) {
      uint32_t keys[M];
      chunk_keys(c0, keys);
      const int j0 = c0 + tid * M;
#pragma unroll
      for (int e = 0; e < M; ++e)
        if (j0 + e < n) {
          kmin = min(kmin, keys[e]);
          kmax = max(kmax, keys[e]);
        }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, DSA_WAVE));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, DSA_WAVE));
  }
  if (lane == 0) {
    sh.red[0][wv] = kmin;
    sh.red[1][wv] = kmax;
  }
  __syncthreads();
  // ---- phase 2: bucket histogram
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    kmin = min(kmin, sh.red[0][i]);
    kmax = max(kmax, sh.red[1][i]);
  }
  const float vmax = order_key_value(kmax), vmin = order_key_value(kmin);
  const float scale = 4095.5f / (vmax - vmin);
  if (kmin == kmax || !(scale > 0.f) || !(scale < 3.0e38f)) return false;
  auto bucket = [&](uint32_t key) {
    const float b = (vmax - order_key_value(key)) * scale;
    return min(4095, (int)b);
  };
  // a row of one chunk keeps each key's bucket and its arrival rank inside
  // the bucket (the counter's old value, its offset in the bucket-grouped
  // list) as bucket << 16 | rank; invalid positions get bucket 4096. (With 16
  // positions per thread the extra registers would spill: atomics instead.)
  const bool one_chunk = M <= 8 && n <= C;
  uint32_t rk0[M];
  if (one_chunk) {
    const int j0 = tid * M;
#pragma unroll
    for (int e = 0; e < M; ++e) {
      const uint32_t b = j0 + e < n ? (uint32_t)bucket(k0[e]) : 4096u;
      rk0[e] = b < 4096u ? (b << 16) | atomicAdd(&cursor[b], 1u) : (4096u << 16);
    }
  } else if (n <= C) {
    const int j0 = tid * M;
#pragma unroll
    for (int e = 0; e < M; ++e)
      if (j0 + e < n) atomicAdd(&cursor[bucket(k0[e])], 1u);
  } else if (R == 2 && n <= 2 * C) {
    // both chunks are in registers: count them here and take the candidates
    // from the registers in phase 5 (no speculative list)
#pragma unroll
    for (int e = 0; e < M; ++e) atomicAdd(&cursor[bucket(k0[e])], 1u);
    const int j1 = C + tid * M;
#pragma unroll
    for (int e = 0; e < M; ++e)
      if (j1 + e < n) atomicAdd(&cursor[bucket(k1[e])], 1u);
  } else {
    // A row of several chunks. The first chunk (all valid) is counted alone;
    // the bucket at which its count reaches 1.3 k C / n + 16 estimates where
    // the row's candidates end. Every key up to that bucket is listed as
    // counted, so that the candidates are taken from the list instead of a
    // second pass over the row whenever the estimate covers them and the
    // list did not overflow (checked once the row's counts are known).
#pragma unroll
    for (int e = 0; e < M; ++e) atomicAdd(&cursor[bucket(k0[e])], 1u);
    __syncthreads();
    {
      int c[BPT], local = 0;
#pragma unroll
      for (int u = 0; u < BPT; ++u) {
        c[u] = (int)cursor[tid * BPT + u];
        local += c[u];
      }
      int incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, DSA_WAVE);
        if (lane >= off) incl += v;
      }
      if (lane == 63) sh.wsum[wv] = incl;
      __syncthreads();
      int run = incl - local;
#pragma unroll
      for (int i = 0; i < NT / 64; ++i) run += i < wv ? sh.wsum[i] : 0;
      const int target = (int)(1.3f * (float)k * (float)C / (float)n) + 16;  // < C
#pragma unroll
      for (int u = 0; u < BPT; ++u) {
        if (run < target && run + c[u] >= target) sh.spec_b = tid * BPT + u;
        run += c[u];
      }
    }
    __syncthreads();
    const int gb = sh.spec_b;
    // list the keys of buckets up to gb (bit e of `take`: key e of the
    // thread's M), one LDS atomic per wave and chunk
    auto spec_list = [&](const uint32_t (&keys)[M], uint32_t take, int j0) {
      const int cnt = __popc(take);
      int incl = cnt;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, DSA_WAVE);
        if (lane >= off) incl += v;
      }
      int base = 0;
      if (lane == 63) base = atomicAdd(&sh.spec_n, incl);
      int slot = __shfl(base, 63, DSA_WAVE) + incl - cnt;
#pragma unroll
      for (int e = 0; e < M; ++e)
        if ((take >> e) & 1u) {
          if (slot < spec_cap) spec[slot] = ((uint64_t)keys[e] << 32) | (uint64_t)(~(uint32_t)(j0 + e));
          ++slot;
        }
    };
    {
      uint32_t take = 0;
#pragma unroll
      for (int e = 0; e < M; ++e) take |= (uint32_t)(bucket(k0[e]) <= gb) << e;
      spec_list(k0, take, tid * M);
    }
    for (int c0 = C; c0 < n; c0 += C) {
      uint32_t keys[M];
      chunk_keys(c0, keys);
      const int j0 = c0 + tid * M;
      uint32_t take = 0;
#pragma unroll
      for (int e = 0; e < M; ++e)
        if (j0 + e < n) {
          const int b = bucket(keys[e]);
          atomicAdd(&cursor[b], 1u);
          take |= (uint32_t)(b <= gb) << e;
        }
      spec_list(keys, take, j0);
    }
  }
  __syncthreads();
  // ---- phase 3: exclusive prefix of the counts (wave scan, then wave sums)
  int c[BPT], local = 0;
#pragma unroll
  for (int u = 0; u < BPT; ++u) {
    c[u] = (int)cursor[tid * BPT + u];
    local += c[u];
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, DSA_WAVE);
    if (lane >= off) incl += v;
  }
  if (lane == 63) sh.wsum[wv] = incl;
  __syncthreads();
  // ---- phase 4: bucket starts and cursors; the bucket holding place k - 1
  // (exactly one when n > k) records where the candidate range ends
  {
    int run = incl - local, total = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      const int x = sh.wsum[i];
      run += i < wv ? x : 0;
      total += x;
    }
    int big = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      bstart[tid * BPT + u] = run;
      if (!one_chunk) cursor[tid * BPT + u] = (uint32_t)run;
      if (run < k) big = max(big, c[u]);
      if (run < k && run + c[u] >= k) {
        sh.lim = run + c[u];
        sh.blast = tid * BPT + u;
      }
      run += c[u];
    }
    if (tid == NT - 1) bstart[4096] = total;
    const bool wbig = __ballot(big > kDirectBucketMax) != 0;
    if (lane == 0) sh.wbig[wv] = wbig ? 1 : 0;
  }
  __syncthreads();
  {
    int anybig = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) anybig |= sh.wbig[i];
    if (anybig) return false;
  }
  // bucket starts grow with the bucket, so "start below k" is "bucket <= blast"
  const int lim = n <= k ? n : sh.lim;
  const int blast = n <= k ? 4095 : sh.blast;
  // ---- phase 5: scatter the candidates (bucket start below k) by bucket
  if (one_chunk) {
    const int j0 = tid * M;
    int bs[M];
#pragma unroll
    for (int e = 0; e < M; ++e) bs[e] = (int)(rk0[e] >> 16) <= blast ? bstart[rk0[e] >> 16] : 0;
#pragma unroll
    for (int e = 0; e < M; ++e)
      if ((int)(rk0[e] >> 16) <= blast)
        scomp[bs[e] + (int)(rk0[e] & 0xffffu)] =
            ((uint64_t)k0[e] << 32) | (uint64_t)(~(uint32_t)(j0 + e));
  } else if (n > C && blast <= sh.spec_b && sh.spec_n <= spec_cap) {
    // the listed keys hold every candidate
    const int ns = sh.spec_n;
    for (int i = tid; i < ns; i += NT) {
      const uint64_t cm = spec[i];
      const int b = bucket((uint32_t)(cm >> 32));
      if (b <= blast) scomp[atomicAdd(&cursor[b], 1u)] = cm;
    }
  } else {
    for (int c0 = 0; c0 < n; c0 += C) {
      uint32_t keys[M];
      chunk_keys(c0, keys);
      const int j0 = c0 + tid * M;
#pragma unroll
      for (int e = 0; e < M; ++e)
        if (j0 + e < n) {
          const int b = bucket(keys[e]);
          if (b <= blast) {
            const uint32_t slot = atomicAdd(&cursor[b], 1u);
            scomp[slot] = ((uint64_t)keys[e] << 32) | (uint64_t)(~(uint32_t)(j0 + e));
          }
        }
    }
  }
  __syncthreads();
  // ---- phase 6: place of every candidate; a thread's (up to) four entries
  // have their reads issued together
  for (int s0 = tid; s0 < lim; s0 += 4 * NT) {
    uint64_t cm[4];
    int b0[4], b1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) cm[r] = s0 + r * NT < lim ? scomp[s0 + r * NT] : 0ull;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int b = s0 + r * NT < lim ? bucket((uint32_t)(cm[r] >> 32)) : 0;
      b0[r] = s0 + r * NT < lim ? bstart[b] : 0;
      b1[r] = s0 + r * NT < lim ? bstart[b + 1] : 0;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int rk = 0, u = b0[r];
      for (; u + 4 <= b1[r]; u += 4) {  // four independent reads in flight
        const uint64_t x0 = scomp[u], x1 = scomp[u + 1], x2 = scomp[u + 2], x3 = scomp[u + 3];
        rk += (int)(x0 > cm[r]) + (int)(x1 > cm[r]) + (int)(x2 > cm[r]) + (int)(x3 > cm[r]);
      }
      for (; u < b1[r]; ++u) rk += scomp[u] > cm[r];
      if (b0[r] < b1[r] && b0[r] + rk < k) orow[b0[r] + rk] = (int)(~(uint32_t)cm[r]);
    }
  }
  for (int i = n + tid; i < k; i += NT) orow[i] = -1;
  return true;
}

template <int IPT, int M, int R>
__global__ __launch_bounds__(kSelNT) void topk_select(const float* __restrict__ scores, long ld,
                                                      const int32_t* __restrict__ cu,
                                                      const int32_t* __restrict__ seq_lens,
                                                      int S, int cap, int unit, int k,
                                                      const uint2* __restrict__ ext, int ext_ld,
                                                      int32_t* __restrict__ topk) {
  constexpr int NT = kSelNT;
  constexpr int CHUNK = NT * M;
  using Cfg = SelectCfg<IPT>;
  constexpr int CAP = Cfg::CAP;
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t* list_key = lds;                // CAP
  uint32_t* list_pos = list_key + CAP;     // CAP
  uint32_t* hist = list_pos + CAP;         // 4096
  // the sort's scratch reuses the whole region once the list is in registers
  auto& sort_storage = *reinterpret_cast<typename Cfg::Sorter::storage_type*>(lds);
  __shared__ int s_scan[NT / 64];
  __shared__ int s_dig[2];
  __shared__ uint32_t s_bits[4][NT / 64];
  __shared__ DirectShared s_direct;

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const float* row = scores + (size_t)t * ld;
  // chunk 0 (and with R = 2 chunk 1), resident for all passes; the loads
  // overlap the row lookup
  uint32_t k0[M], k1[M];
  load_keys_ahead<M>(row, ld < (long)CHUNK ? (int)ld : CHUNK, k0);
  if (R == 2) load_keys_ahead<M>(row + CHUNK, (int)(ld < 2l * CHUNK ? ld : 2l * CHUNK) - CHUNK, k1);
  const RowInfo ri = row_info_wave(cu, seq_lens, S, t, cap);
  // positions of the row: its valid tokens, or (unit = PS) the pages that
  // hold one
  const int n = (ri.n_valid + unit - 1) / unit;
  int32_t* orow = topk + (size_t)t * k;
  if (n == 0) {
    for (int i = tid; i < k; i += NT) orow[i] = -1;
    return;
  }
  if (n <= kDirectMaxN &&
      topk_direct<NT, M, R>(k0, k1, row, n, k, lds, Cfg::D_CUR_OFF, Cfg::D_START_OFF, Cfg::D_KEY_OFF,
                         Cfg::D_SPEC_OFF, Cfg::SPEC, s_direct,
                         ext != nullptr ? ext + (size_t)t * ext_ld : nullptr, orow))
    return;
  __syncthreads();  // the select path reuses the LDS
  // OR / AND / min / max of the keys this thread lists
  uint32_t bor = 0u, band = ~0u, kmin = ~0u, kmax = 0u;

  int count;
  if (n <= CAP) {  // everything fits the sort: no selection needed
    const int j0 = tid * M;
#pragma unroll
    for (int e = 0; e < M; ++e) {
      const int j = j0 + e;
      if (j < n) {
        list_key[j] = k0[e];
        list_pos[j] = (uint32_t)j;
        bor |= k0[e];
        band &= k0[e];
        kmin = min(kmin, k0[e]);
        kmax = max(kmax, k0[e]);
      }
    }
    count = n;
  } else {
    // ---- global digits until (above + boundary bin) fits, or the key is exact
    uint32_t prefix = 0;
    int pbits = 0;
    int need = k;
    int nbin = n;
    while (pbits == 0 || ((k - need) + nbin > CAP && pbits < 32)) {
      const int w = min(12, 32 - pbits);
      const int nb = 1 << w;
      for (int i = tid; i < nb; i += NT) hist[i] = 0;
      __syncthreads();
      const int shift = 32 - pbits - w;
      for (int c0 = 0; c0 < n; c0 += CHUNK) {
        uint32_t keys[M];
        if (c0 == 0) {
#pragma unroll
          for (int e = 0; e < M; ++e) keys[e] = k0[e];
        } else if (R == 2 && c0 == CHUNK) {
#pragma unroll
          for (int e = 0; e < M; ++e) keys[e] = k1[e];
        } else {
          load_keys<M>(row, n, c0, keys);
        }
        const int j0 = c0 + tid * M;
#pragma unroll
        for (int e = 0; e < M; ++e) {
          const uint32_t key = keys[e];
          if (j0 + e < n && (pbits == 0 || (key >> (32 - pbits)) == prefix))
            atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1u);
        }
      }
      __syncthreads();
      find_digit(hist, nb, need, s_scan, s_dig);
      const int d = s_dig[0];
      need -= s_dig[1];
      prefix = (pbits == 0 ? 0u : (prefix << w)) | (uint32_t)d;
      pbits += w;
      nbin = (int)hist[d];
      __syncthreads();
    }
    const bool exact = pbits >= 32;  // the bin is one key: take its first `need` ties
    const int above = k - need;
    // ---- collect in position order: above -> [0, above), bin -> [above, ...)
    int nabove = 0, nbnd = 0;
    for (int c0 = 0; c0 < n; c0 += CHUNK) {
      uint32_t keys[M];
      if (c0 == 0) {
#pragma unroll
        for (int e = 0; e < M; ++e) keys[e] = k0[e];
      } else if (R == 2 && c0 == CHUNK) {
#pragma unroll
        for (int e = 0; e < M; ++e) keys[e] = k1[e];
      } else {
        load_keys<M>(row, n, c0, keys);
      }
      const int j0 = c0 + tid * M;
      int fa = 0, fb = 0;
#pragma unroll
      for (int e = 0; e < M; ++e) {
        const uint32_t v = exact ? keys[e] : (keys[e] >> (32 - pbits));
        const bool ok = j0 + e < n;
        fa += ok && v > prefix;
        fb += ok && v == prefix;
      }
      int total;
      const int packed = fa | (fb << 16);
      const int excl = block_inclusive_scan<NT>(packed, s_scan, &total) - packed;
      int ia = nabove + (excl & 0xffff);
      int ib = nbnd + (excl >> 16);
#pragma unroll
      for (int e = 0; e < M; ++e) {
        const int j = j0 + e;
        const uint32_t v = exact ? keys[e] : (keys[e] >> (32 - pbits));
        if (j < n && v > prefix) {
          if (ia < CAP) {
            list_key[ia] = keys[e];
            list_pos[ia] = (uint32_t)j;
            bor |= keys[e];
            band &= keys[e];
            kmin = min(kmin, keys[e]);
            kmax = max(kmax, keys[e]);
          }
          ++ia;
        } else if (j < n && v == prefix) {
          const int dst = above + ib;
          if ((!exact || ib < need) && dst < CAP) {
            list_key[dst] = keys[e];
            list_pos[dst] = (uint32_t)j;
            bor |= keys[e];
            band &= keys[e];
            kmin = min(kmin, keys[e]);
            kmax = max(kmax, keys[e]);
          }
          ++ib;
        }
      }
      nabove += total & 0xffff;
      nbnd += total >> 16;
    }
    count = exact ? k : min(above + nbnd, CAP);
  }
  // ---- reduce OR / AND / min / max of the listed keys
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    bor |= (uint32_t)__shfl_xor((int)bor, o, DSA_WAVE);
    band &= (uint32_t)__shfl_xor((int)band, o, DSA_WAVE);
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, DSA_WAVE));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, DSA_WAVE));
  }
  if (lane_id() == 0) {
    s_bits[0][tid >> 6] = bor;
    s_bits[1][tid >> 6] = band;
    s_bits[2][tid >> 6] = kmin;
    s_bits[3][tid >> 6] = kmax;
  }
  __syncthreads();
  {
    uint32_t o = 0u, an = ~0u, mn = ~0u, mx = 0u;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
      o |= s_bits[0][i];
      an &= s_bits[1][i];
      mn = min(mn, s_bits[2][i]);
      mx = max(mx, s_bits[3][i]);
    }
    bor = o;
    band = an;
    kmin = mn;
    kmax = mx;
  }
  const uint32_t diff = bor ^ band;  // bits in which the listed keys differ
  const int nout = min(count, k);
  for (int i = nout + tid; i < k; i += NT) orow[i] = -1;
  if (diff == 0u) {  // one key: the list (position order) is the order
    for (int i = tid; i < nout; i += NT) orow[i] = (int)list_pos[i];
    return;
  }
  // ---- rank: bucket b = (kmax - key) >> sh (ascending b = descending key,
  // at most 4096 buckets; one key per bucket whenever the keys' span allows).
  // An entry's place is its bucket's start plus the number of bucket members
  // that precede it (larger key, or equal key and smaller list index, which
  // for equal keys is the smaller position).
  const int lo = __builtin_ctz(diff);
  const uint32_t span = (kmax - kmin) >> lo;
  const int nbits = 32 - __builtin_clz(span);
  const int sh = lo + (nbits > 12 ? nbits - 12 : 0);
  uint32_t* cursor = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(lds) + Cfg::HIST_OFF);
  int* bstart = reinterpret_cast<int*>(reinterpret_cast<char*>(lds) + Cfg::START_OFF);
  uint32_t* skey = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(lds) + Cfg::SKEY_OFF);
  uint16_t* sidx = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(lds) + Cfg::SIDX_OFF);
  for (int b = tid; b < 4096; b += NT) cursor[b] = 0u;
  __syncthreads();
  for (int i = tid; i < count; i += NT) atomicAdd(&cursor[(kmax - list_key[i]) >> sh], 1u);
  __syncthreads();
  {
    constexpr int BPT = 4096 / NT;
    int c[BPT], local = 0, big = 0;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      c[u] = (int)cursor[tid * BPT + u];
      local += c[u];
      big = max(big, c[u]);
    }
    int total;
    int run = block_inclusive_scan<NT>(local, s_scan, &total) - local;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      bstart[tid * BPT + u] = run;
      cursor[tid * BPT + u] = (uint32_t)run;
      run += c[u];
    }
    if (tid == 0) {
      bstart[4096] = total;
      s_dig[0] = 0;
    }
    __syncthreads();
    if (__ballot(big > kRankBucketMax) != 0 && lane_id() == 0) s_dig[0] = 1;
    __syncthreads();
  }
  if (s_dig[0] == 0) {  // no bucket above kRankBucketMax
    for (int i = tid; i < count; i += NT) {
      const uint32_t key = list_key[i];
      const uint32_t slot = atomicAdd(&cursor[(kmax - key) >> sh], 1u);
      skey[slot] = key;
      sidx[slot] = (uint16_t)i;
    }
    __syncthreads();
    for (int sl = tid; sl < count; sl += NT) {
      const uint32_t key = skey[sl];
      const int idx = sidx[sl];
      const int b = (int)((kmax - key) >> sh);
      const int b0 = bstart[b], b1 = bstart[b + 1];
      int r = 0;
      for (int u = b0; u < b1; ++u) {
        const uint32_t ku = skey[u];
        r += (ku > key) | ((ku == key) & ((int)sidx[u] < idx));
      }
      if (b0 + r < k) orow[b0 + r] = (int)list_pos[idx];
    }
    return;
  }
  // ---- a crowded bucket: stable descending radix sort of the list over the
  // bits in which its keys differ (entries past `count` carry key 0 and stay
  // last: they sort below or, on ties, after every listed key)
  uint32_t keys[IPT];
  int vals[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int idx = tid * IPT + i;
    keys[i] = idx < count ? list_key[idx] : 0u;
    vals[i] = idx < count ? (int)list_pos[idx] : -1;
  }
  __syncthreads();
  typename Cfg::Sorter().sort_desc(keys, vals, sort_storage, (unsigned)lo,
                                   32u - (unsigned)__builtin_clz(diff));
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int idx = tid * IPT + i;
    if (idx < nout) orow[idx] = vals[i];
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
// Stages per workgroup, from the batch's upper bound of T * cap positions:
// a small batch gets one round of workgroups (one per compute unit, the ring
// fills the LDS), a large one about four per unit; 1 .. 32 stages each.
static int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

template <int D, int HB>
static hipError_t launch_rows(const IndexerArgs& a, hipStream_t st) {
  const long cap = (long)a.MP * a.PS;
  const long total = (long)a.T * ((cap + kStreamKeys - 1) / kStreamKeys);
  if (HB == 1 && total > 2048 && total < (1L << 30) && a.T <= kFlatMaxT && a.S <= kRegMaxS) {
    ProfScope prof("idx_score_regs", st);
    if (a.PS % kRegKeys == 0)
      hipLaunchKernelGGL((idx_score_regs<D, true>), dim3(compute_units() * kRegWavesPerSimd),
                         dim3(256), 0, st, a.q, a.w, a.cache, a.num_pages, a.pt, a.seq_lens, a.cu,
                         a.T, a.S, a.H, a.PS, a.MP, a.scores, a.ld);
    else
      hipLaunchKernelGGL((idx_score_regs<D, false>), dim3(compute_units() * kRegWavesPerSimd),
                         dim3(256), 0, st, a.q, a.w, a.cache, a.num_pages, a.pt, a.seq_lens, a.cu,
                         a.T, a.S, a.H, a.PS, a.MP, a.scores, a.ld);
    return hipGetLastError();
  }
  if (HB == 1 && total > 2048 && total < (1L << 30) && a.T <= kFlatMaxT &&
      a.S <= FlatShape<D>::MAX_S) {
    ProfScope prof("idx_score_flat", st);
    hipLaunchKernelGGL((idx_score_flat<D>), dim3(compute_units()), dim3(256), 0, st, a.q, a.w,
                       a.cache, a.num_pages, a.pt, a.seq_lens, a.cu, a.T, a.S, a.H, a.PS, a.MP,
                       a.scores, a.ld);
    return hipGetLastError();
  }
  const long target = total <= 2048 ? 256 : 1024;
  long nstg = (total + target - 1) / target;
  if (nstg < 1) nstg = 1;
  if (nstg > 32) nstg = 32;
  const long per = nstg * kStreamKeys;
  dim3 grid((unsigned)((cap + per - 1) / per), a.T);
  ProfScope prof("idx_score_stream", st);
  hipLaunchKernelGGL((idx_score_stream<D, HB>), grid, dim3(256), 0, st, a.q, a.w, a.cache,
                     a.num_pages, a.pt, a.seq_lens, a.cu, a.T, a.S, a.H, a.PS, a.MP, (int)nstg,
                     a.scores, a.ld);
  return hipGetLastError();
}

template <int D, int HB>
static hipError_t launch_tiles(const IndexerArgs& a, hipStream_t st) {
  const int cap = a.MP * a.PS;
  constexpr int R = kTileRows;
  dim3 grid((cap + kTileMaxRK - 1) / kTileMaxRK, (a.T + R - 1) / R);
  ProfScope prof("idx_score_tiles", st);
  if (a.ext != nullptr)
    hipLaunchKernelGGL((idx_score_tiles<D, HB, true>), grid, dim3(64 * R), 0, st, a.q, a.w,
                       a.cache, a.num_pages, a.pt, a.seq_lens, a.cu, a.T, a.S, a.H, a.PS, a.MP,
                       a.scores, a.ld, a.ext, a.ext_ld);
  else
    hipLaunchKernelGGL((idx_score_tiles<D, HB, false>), grid, dim3(64 * R), 0, st, a.q, a.w,
                       a.cache, a.num_pages, a.pt, a.seq_lens, a.cu, a.T, a.S, a.H, a.PS, a.MP,
                       a.scores, a.ld, nullptr, 0);
  return hipGetLastError();
}

template <int D, int HB>
static hipError_t launch_score(const IndexerArgs& a, hipStream_t st) {
  return a.max_q_len <= 1 ? launch_rows<D, HB>(a, st) : launch_tiles<D, HB>(a, st);
}

// only rows longer than one select chunk (kSelNT x 16 positions) use them
int score_ext_ld(int max_q_len, int cap) {
  return max_q_len <= 1 || cap <= kSelNT * 16 ? 0 : (cap + kTileMaxRK - 1) / kTileMaxRK;
}

hipError_t indexer_score(const IndexerArgs& a, hipStream_t st) {
  const int HB = (a.H + 31) / 32;
  switch (a.D) {
    case 32: return HB == 1 ? launch_score<32, 1>(a, st) : launch_score<32, 2>(a, st);
    case 64: return HB == 1 ? launch_score<64, 1>(a, st) : launch_score<64, 2>(a, st);
    case 128: return HB == 1 ? launch_score<128, 1>(a, st) : launch_score<128, 2>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// sort capacity 2k (at least 2048): room for the keys above the boundary bin
// plus the bin itself in the common case
static int select_ipt(int k) { return k <= 1024 ? 2 : (k <= 2048 ? 4 : 8); }

size_t topk_select_lds_bytes(int k) {
  switch (select_ipt(k)) {
    case 2: return SelectCfg<2>::BYTES;
    case 4: return SelectCfg<4>::BYTES;
    default: return SelectCfg<8>::BYTES;
  }
}

// One select launch: rows of `ld` scores, n = ceil(n_valid / unit) of them
// valid, k kept.
struct SelectJob {
  const float* scores;
  long ld;
  int unit, k;
  int32_t* out;
  const uint2* ext;  // per-tile extreme keys of the rows, or nullptr
  int ext_ld;
};

template <int IPT, int M, int R>
static hipError_t launch_select(const IndexerArgs& a, const SelectJob& j, hipStream_t st) {
  const size_t lds = SelectCfg<IPT>::BYTES;
  // raise the dynamic-LDS limit once per device
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load() & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_select<IPT, M, R>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit);
  }
  ProfScope prof("topk_select", st);
  hipLaunchKernelGGL((topk_select<IPT, M, R>), dim3(a.T), dim3(kSelNT), lds, st, j.scores, j.ld,
                     a.cu, a.seq_lens, a.S, a.MP * a.PS, j.unit, j.k, j.ext, j.ext_ld, j.out);
  return hipGetLastError();
}

// positions per thread: 8 when a whole score row fits one chunk of 8192,
// else 16; rows of two chunks (up to 32768 scores) keep both in registers
template <int IPT>
static hipError_t launch_select_m(const IndexerArgs& a, const SelectJob& j, hipStream_t st) {
  if (j.ld <= (long)kSelNT * 8) return launch_select<IPT, 8, 1>(a, j, st);
  if (j.ld <= (long)kSelNT * 16 || j.ld > (long)kSelNT * 32)
    return launch_select<IPT, 16, 1>(a, j, st);
  return launch_select<IPT, 16, 2>(a, j, st);
}

static hipError_t select_job(const IndexerArgs& a, const SelectJob& j, hipStream_t st) {
  switch (select_ipt(j.k)) {
    case 2: return launch_select_m<2>(a, j, st);
    case 4: return launch_select_m<4>(a, j, st);
    default: return launch_select_m<8>(a, j, st);
  }
}

hipError_t indexer_select(const IndexerArgs& a, hipStream_t st) {
  return select_job(a, SelectJob{a.scores, a.ld, 1, a.k, a.topk, a.ext, a.ext_ld}, st);
}

hipError_t indexer_page_select(const IndexerArgs& a, hipStream_t st) {
  return select_job(a, SelectJob{a.page_scores, a.ldp, a.PS, a.k, a.topk, nullptr, 0}, st);
}

// ---------------------------------------------------------------------------
// Page scores ("ref.py", streamindex_page_topk_ref: masked positions at
// -inf, then the maximum over each page). grid = (T, ceil(MP / 64)), block =
// 256: workgroup (t, c) pools pages 64 c .. 64 c + 63 of row t. A 16-lane
// group covers one page (PS <= 64: four scores per lane); wave w takes pages
// 64 c + 16 w + 4 it + group (it < 4) with all its loads issued before any
// reduction. Pages at or past ceil(n_valid / PS) are not written: the select
// never reads them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void page_pool(const float* __restrict__ scores, long ld,
                                                 const int32_t* __restrict__ cu,
                                                 const int32_t* __restrict__ seq_lens, int S,
                                                 int cap, int PS, float* __restrict__ pscores,
                                                 long ldp) {
  const int t = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const RowInfo ri = row_info_wave(cu, seq_lens, S, t, cap);
  const int n = ri.n_valid;
  const int npg = (n + PS - 1) / PS;
  const int p_base = 64 * (int)blockIdx.y + 16 * wave;
  if (p_base >= npg) return;  // wave-uniform; no block barrier follows
  const int l = lane_id(), grp = l >> 4, i = l & 15;
  const float* row = scores + (size_t)t * ld;
  float m[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int p = p_base + 4 * it + grp;
    m[it] = -INFINITY;
    if (p < npg && 4 * i < PS) {
      const int j = p * PS + 4 * i;
      if (j + 4 <= n) {
        const float4 v = *reinterpret_cast<const float4*>(row + j);
        m[it] = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
      } else {
        for (int e = 0; e < 4; ++e)
          if (j + e < n) m[it] = fmaxf(m[it], row[j + e]);
      }
    }
  }
  float* prow = pscores + (size_t)t * ldp;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    float v = m[it];
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, shfl_xor_f(v, o));
    const int p = p_base + 4 * it + grp;
    if (p < npg && i == 0) prow[p] = v;
  }
}

hipError_t indexer_page_pool(const IndexerArgs& a, hipStream_t st) {
  ProfScope prof("page_pool", st);
  hipLaunchKernelGGL(page_pool, dim3(a.T, (a.MP + 63) / 64), dim3(256), 0, st, a.scores, a.ld,
                     a.cu, a.seq_lens, a.S, a.MP * a.PS, a.PS, a.page_scores, a.ldp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Positions of selected pages: tokens[t, i] = pages[t, i / PS] * PS + i % PS,
// or -1 for a -1 page slot. grid = (T, ceil(k_pages * PS / 256)).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void page_token_list(const int32_t* __restrict__ pages,
                                                       int k_pages, int PS,
                                                       int32_t* __restrict__ tokens) {
  const int t = blockIdx.x;
  const int n = k_pages * PS;
  const int i = blockIdx.y * 256 + threadIdx.x;
  if (i >= n) return;
  const int p = pages[(size_t)t * k_pages + i / PS];
  tokens[(size_t)t * n + i] = p >= 0 ? p * PS + i % PS : -1;
}

hipError_t page_tokens(const int32_t* pages, int T, int k_pages, int PS, int32_t* tokens,
                       hipStream_t st) {
  const int n = k_pages * PS;
  ProfScope prof("page_token_list", st);
  hipLaunchKernelGGL(page_token_list, dim3(T, (n + 255) / 256), dim3(256), 0, st, pages,
                     k_pages, PS, tokens);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused prefill scoring and exact top-k: the [T, cap] score matrix of a long
// extend batch is never stored ("dsa_sparse_backend.py", the prefill indexer
// kernel note: token scores of that size are the dominant temporary at long
// context).
//
// idx_score_topk: a workgroup of R waves (fused_rows: 16 with one head
// block) owns R consecutive packed rows (one per wave, query fragments and
// head weights resident, as idx_score_tiles) and one segment of the key
// positions, which it walks in ascending order: ranges of kTileMaxRK
// positions, each streamed through a ring of 64-key blocks in the row-group
// layout and shared by the rows of one sequence. With 16 rows a workgroup
// scores two blocks between barriers (a ring of five: three blocks in flight
// beyond the two being scored), and computes both blocks' scores before it
// takes their keys, so that head sums and products of neighbouring
// sub-blocks overlap. Every wave
// keeps its row's candidates of the segment in a global list of C entries
// (order key, position), appending each scored key above the row's bar.
// When the next block might not fit, the wave compacts the list to exactly k
// entries — every key above the k-th largest key kappa, then the first keys
// equal to kappa in list order — and the bar becomes kappa.
//
// Exactness. The list is in ascending position order (keys are appended in
// position order, a compaction keeps the order), so the kept entries beat,
// in the canonical order (key descending, position ascending), every dropped
// entry and every later key that is not above kappa: each of those is below
// kappa, or equal to it at a larger position than all k kept entries. So the
// row's top k always lie in the list plus the later keys above the bar. The
// bar starts unset (every key is taken).
//
// The compaction is a radix select of the k-th key over the list, one 8-bit
// digit per pass with a 256-bin LDS histogram per wave, then an
// order-keeping pass; list reads bypass the vector L1 (agent-scope loads),
// so they see the wave's own earlier list stores.
// grid = (G segments of L positions, ceil(T / R)), block = 64 R.
//
// topk_merge: one workgroup per row sorts the G lists of the row (at most
// G * k <= kMergeMax entries) by composite key (order key << 32 | ~position)
// with a bitonic sort in LDS and writes the first min(k, total) positions,
// then -1. Composite keys are distinct, so the order is the canonical one.
// ---------------------------------------------------------------------------
constexpr int kMergeMax = 8192;
constexpr int kCutSoon = 192;  // a list this close to full asks the workgroup for a cut

__device__ __forceinline__ uint32_t list_load_key(const uint2* p) {
  return __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint2 list_load(const uint2* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}

// Compact list[0 .. cnt), cnt > k, to exactly k entries in list order (see
// above); returns kappa. Wave-level: hist is this wave's 256 LDS words. Every
// key lies in [lo, hi], so the bits above the highest bit in which lo and hi
// differ are common to all keys and the digit passes start below them (one
// pass per 8 bits left; none when every key is equal). Each lane has eight
// list loads in flight at a time.
constexpr int kListBatch = 8;

// The bin d of a wave's 256-bin histogram at which the count from the top
// bin down reaches need (1 <= need <= total), and the count above it.
__device__ __forceinline__ void hist_find(const uint32_t* hist, int need, int* d_out,
                                          int* above_out) {
  const int l = lane_id();
  // lane l holds bins 255 - 4 l - c (c < 4), descending
  uint32_t c4[4];
  int lane_sum = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    c4[c] = hist[255 - 4 * l - c];
    lane_sum += (int)c4[c];
  }
  int incl = lane_sum;
#pragma unroll
  for (int off = 1; off < DSA_WAVE; off <<= 1) {
    const int u = __shfl_up(incl, off, DSA_WAVE);
    if (l >= off) incl += u;
  }
  const int excl = incl - lane_sum;
  const uint64_t hit = __ballot(excl < need && incl >= need);
  const int src = (int)__builtin_ctzll(hit);
  int d = 0, above = 0;
  if (l == src) {
    int run = excl;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (run + (int)c4[c] >= need) {
        d = 255 - 4 * l - c;
        above = run;
        break;
      }
      run += (int)c4[c];
    }
  }
  *d_out = __shfl(d, src, DSA_WAVE);
  *above_out = __shfl(above, src, DSA_WAVE);
}

__device__ uint32_t list_compact(uint2* list, int cnt, int k, uint32_t* hist, uint32_t lo,
                                 uint32_t hi) {
  const int l = lane_id();
  uint32_t prefix = lo;
  int need = k;  // kappa is the need-th largest key among those matching prefix
  const uint32_t diff = lo ^ hi;
  if (diff != 0u) {
    const int top = 31 - __builtin_clz(diff);
    const int start = top & ~7;
    prefix = lo & ~((2u << top) - 1u);  // the common high bits (none when top = 31)
    if (top == 31) prefix = 0u;
    for (int shift = start; shift >= 0; shift -= 8) {
      for (int i = l; i < 256; i += DSA_WAVE) hist[i] = 0u;
      const uint32_t hmask = shift + 8 >= 32 ? 0u : ~((1u << (shift + 8)) - 1u);
      for (int base = 0; base < cnt; base += DSA_WAVE * kListBatch) {
        uint32_t key[kListBatch];
#pragma unroll
        for (int u = 0; u < kListBatch; ++u) {
          const int i = base + u * DSA_WAVE + l;
          key[u] = list_load_key(list + min(i, cnt - 1));  // clamped: never a branch
        }
#pragma unroll
        for (int u = 0; u < kListBatch; ++u) {
          const int i = base + u * DSA_WAVE + l;
          if (i < cnt && (key[u] & hmask) == (prefix & hmask))
            atomicAdd(&hist[(key[u] >> shift) & 255u], 1u);
        }
      }
      int d, above;
      hist_find(hist, need, &d, &above);
      prefix = (prefix & hmask) | ((uint32_t)d << shift);
      need -= above;
    }
  }
  const uint32_t kappa = prefix;
  // keep: keys above kappa, and the first `need` keys equal to kappa
  int kept = 0, ties = 0;
  for (int base = 0; base < cnt; base += DSA_WAVE * kListBatch) {
    uint2 e[kListBatch];
#pragma unroll
    for (int u = 0; u < kListBatch; ++u) {
      const int i = base + u * DSA_WAVE + l;
      e[u] = list_load(list + min(i, cnt - 1));  // clamped: never a branch
    }
#pragma unroll
    for (int u = 0; u < kListBatch; ++u) {
      const int i = base + u * DSA_WAVE + l;
      const bool gt = i < cnt && e[u].x > kappa;
      const bool eq = i < cnt && e[u].x == kappa;
      const uint64_t beq = __ballot(eq);
      const bool keep = gt || (eq && ties + ballot_rank(beq) < need);
      const uint64_t bk = __ballot(keep);
      if (keep) list[kept + ballot_rank(bk)] = e[u];  // never past index i
      kept += __popcll(bk);
      ties += __popcll(beq);
    }
  }
  wait_vm<0>();
  return kappa;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, DSA_WAVE));
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, DSA_WAVE));
  return v;
}

// The histogram window of a list: 256 bins of 2^shift keys from base, the
// last bin also holding every larger key.
__device__ __forceinline__ int window_shift(uint32_t base, uint32_t hi) {
  const uint32_t span = hi > base ? hi - base : 0u;
  const int bits = span ? 32 - __builtin_clz(span) : 0;
  return bits > 8 ? bits - 8 : 0;
}

__device__ __forceinline__ uint32_t window_bin(uint32_t key, uint32_t base, int shift) {
  const uint32_t b = (key - base) >> shift;
  return b < 255u ? b : 255u;
}

// Count the keys of list[0 .. cnt) (all >= base) into hist under the window
// (base, shift).
__device__ void list_hist(const uint2* list, int cnt, uint32_t base, int shift, uint32_t* hist) {
  const int l = lane_id();
  for (int i = l; i < 256; i += DSA_WAVE) hist[i] = 0u;
  for (int b0 = 0; b0 < cnt; b0 += DSA_WAVE * kListBatch) {
    uint32_t key[kListBatch];
#pragma unroll
    for (int u = 0; u < kListBatch; ++u) {
      const int i = b0 + u * DSA_WAVE + l;
      key[u] = list_load_key(list + min(i, cnt - 1));  // clamped: never a branch
    }
#pragma unroll
    for (int u = 0; u < kListBatch; ++u)
      if (b0 + u * DSA_WAVE + l < cnt) atomicAdd(&hist[window_bin(key[u], base, shift)], 1u);
  }
}

// Keep the entries of list[0 .. cnt) with key >= theta, in list order, and
// bin them into hist under the window (theta, shift). Returns the count kept.
__device__ int list_cut_rebin(uint2* list, int cnt, uint32_t theta, int shift, uint32_t* hist) {
  const int l = lane_id();
  for (int i = l; i < 256; i += DSA_WAVE) hist[i] = 0u;
  int kept = 0;
  for (int base = 0; base < cnt; base += DSA_WAVE * kListBatch) {
    uint2 e[kListBatch];
#pragma unroll
    for (int u = 0; u < kListBatch; ++u) {
      const int i = base + u * DSA_WAVE + l;
      e[u] = list_load(list + min(i, cnt - 1));  // clamped: never a branch
    }
#pragma unroll
    for (int u = 0; u < kListBatch; ++u) {
      const int i = base + u * DSA_WAVE + l;
      const bool keep = i < cnt && e[u].x >= theta;
      const uint64_t bk = __ballot(keep);
      if (keep) {
        list[kept + ballot_rank(bk)] = e[u];  // never past index i
        atomicAdd(&hist[window_bin(e[u].x, theta, shift)], 1u);
      }
      kept += __popcll(bk);
    }
  }
  wait_vm<0>();
  return kept;
}

template <int D, int HB>
__global__ __launch_bounds__(64 * fused_rows<HB>(), HB == 1 ? 4 : 2) void idx_score_topk(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint16_t* __restrict__ cache, int num_pages, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu, int T, int S, int H,
    int PS, int MP, int k, int G, int L, int C, uint2* __restrict__ cand,
    int* __restrict__ cand_cnt) {
  using TL = TileLayout<D>;
  constexpr int KS = D / 16, HALF = D / 2, RPI = TL::RPI;
  constexpr int BLK = TL::BLK;           // bytes per staged block
  constexpr int NLB = TL::NLB;           // direct loads per block (D / 8)
  constexpr int R = fused_rows<HB>();
  constexpr int NLW = (NLB + R - 1) / R;  // at most this many per wave
  // blocks scored between two barriers, and the ring: three blocks in flight
  // beyond the ones being scored
  constexpr int BPI = R == 16 ? 2 : 1;
  constexpr int RING = 3 + BPI;
  // iterations whose list stores were issued after the last load of the
  // blocks an iteration waits for
  constexpr int SI = BPI == 1 ? 3 : 1;
  constexpr int kCutSoonB = kCutSoon + 64 * (BPI - 1);
  __shared__ __attribute__((aligned(1024))) unsigned char ring[RING][BLK];
  __shared__ int s_seq[R], s_nv[R];
  __shared__ uint32_t s_hist[R][256];
  __shared__ int s_cutreq[2];  // by block parity: the block in which waves are to cut

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = lane_id();
  const int m = l & 31, hf = l >> 5;
  const int t0 = blockIdx.y * R;
  const int cap = MP * PS;
  if (tid < R) {
    const int t = t0 + tid;
    RowInfo ri;
    ri.seq = -1;
    ri.n_valid = 0;
    if (t < T) ri = row_info(cu, seq_lens, S, t, cap);
    s_seq[tid] = ri.seq;
    s_nv[tid] = ri.n_valid;
  }
  if (tid < 2) s_cutreq[tid] = -1;
  __syncthreads();
  const int seg0 = blockIdx.x * L;
  const int seg1 = min(seg0 + L, cap);
  const int t = t0 + wave;
  const int my_nv = __builtin_amdgcn_readfirstlane(s_nv[wave]);
  const bool has = t < T && s_seq[wave] >= 0 && my_nv > seg0;
  uint2* list = cand + ((size_t)(t < T ? t : 0) * G + blockIdx.x) * C;
  int cnt = 0;            // entries in the list (wave-uniform)
  bool barred = false;    // a bar exists: only keys above it are taken
  uint32_t bar = 0u;
  // bounds of the keys this lane appended (the list's keys lie between the
  // wave's minimum, or the bar once there is one, and the wave's maximum)
  uint32_t key_lo = 0xffffffffu, key_hi = 0u;
  // once barred: s_hist[wave] counts the list's keys in 256 bins of
  // 2^win_shift keys from win_base (= the bar), the last bin open above
  uint32_t win_base = 0u;
  int win_shift = 0;
  int gblk = 0;  // iterations walked so far (the same in every wave)
  // Cut the list: at the lower edge of the window bin that holds the k-th key
  // when that keeps at most k + (C - k) / 2 entries, else exactly to k. Every
  // list key is >= win_base (the bar, or the minimum before the first cut).
  auto cut_list = [&]() __attribute__((always_inline)) {
    const uint32_t hi = wave_max_u32(key_hi);
    if (!barred) {  // the first cut: a window over the keys seen so far
      win_base = wave_min_u32(key_lo);
      win_shift = window_shift(win_base, hi);
      list_hist(list, cnt, win_base, win_shift, s_hist[wave]);
    }
    int d = 0, above = 0;
    hist_find(s_hist[wave], k, &d, &above);
    const int keep_n = above + (int)s_hist[wave][d];
    if (keep_n <= k + (C - k) / 2) {
      bar = win_base + ((uint32_t)d << win_shift);
      win_shift = window_shift(bar, hi);
      cnt = list_cut_rebin(list, cnt, bar, win_shift, s_hist[wave]);
    } else {  // a crowded bin: exact cut to k entries
      bar = list_compact(list, cnt, k, s_hist[wave], win_base, hi);
      win_shift = window_shift(bar, hi);
      cnt = list_cut_rebin(list, k, bar, win_shift, s_hist[wave]);
    }
    win_base = bar;
    barred = true;
  };

  // this wave's query fragments and head weights, once for the segment
  bf16x8 a[HB][KS];
  float wv[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 32 * hb + m;
    const bool okq = has && head < H;
    load_q_frag<D>(q + ((size_t)(okq ? t : 0) * H + (head < H ? head : 0)) * D + hf * HALF, okq,
                   a[hb]);
    load_head_weights(w + (size_t)(has ? t : 0) * H, H, hb, hf, wv[hb]);
  }
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int i = 0; i < KS; ++i) asm volatile("" : : "v"(a[hb][i]));
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : : "v"(wv[hb][i]));
  }
  const uint32_t lds_ring = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ring[0];
  const uint32_t voff = TL::load_off(l);
  const int rbase = TL::read_base(m, hf);

  for (int k0 = seg0; k0 < seg1; k0 += kTileMaxRK) {
    int seg = 0;
    while (seg < R) {
      const int s = __builtin_amdgcn_readfirstlane(s_seq[seg]);
      int seg_end = seg + 1;
      while (seg_end < R && s_seq[seg_end] == s) ++seg_end;
      seg_end = __builtin_amdgcn_readfirstlane(seg_end);
      const int n_hi = s >= 0 ? __builtin_amdgcn_readfirstlane(s_nv[seg_end - 1]) : 0;
      const int k1 = min(min(k0 + kTileMaxRK, n_hi), seg1);
      if (s >= 0 && k0 < k1) {
        const int pg0 = k0 / PS;
        int pgv[kTilePgRegs];
        load_page_regs(pt + (size_t)s * MP + pg0, (k1 - 1) / PS - pg0 + 1, l, pgv);
#pragma unroll
        for (int c = 0; c < kTilePgRegs; ++c) asm volatile("" : : "v"(pgv[c]));
        const bool act = has && wave >= seg && wave < seg_end && my_nv > k0;
        const int nv = min(my_nv, seg1);

        const int nb = (k1 - k0 + kTileKB - 1) / kTileKB;
        const int nlw = wave < NLB % R || NLB % R == 0 ? NLW : NLW - 1;
        auto stage = [&](int b) {
          const uint32_t buf = lds_ring + (b % RING) * BLK;
#pragma unroll
          for (int n = 0; n < NLW; ++n) {
            const int I = wave + R * n;
            if (I < NLB) {
              int j0 = k0 + b * kTileKB + I * RPI;
              if (j0 >= k1) j0 = k0;  // past the range: any staged row, never used
              const int page = clamp_page(page_reg(pgv, j0 / PS - pg0), num_pages);
              const uint64_t src =
                  (uint64_t)(uintptr_t)(cache + ((size_t)page * PS + (j0 % PS)) * D);
              const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)src);
              const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(src >> 32));
              gll16_idx(voff, (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo),
                        __builtin_amdgcn_readfirstlane(buf + I * TL::GS));
            }
          }
        };
        // list stores per iteration, four bits each, the last iteration lowest
        int sh = 0;
        // scores of block b: lane l gets key l
        auto score_block = [&](int b) __attribute__((always_inline)) -> float {
          const unsigned char* buf = ring[b % RING];
          float p[2];
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            bf16x8 bk[KS];
#pragma unroll
            for (int i = 0; i < KS; ++i)
              bk[i] = as_bf16x8(
                  *reinterpret_cast<const uint4*>(buf + rbase + sb * TL::SUB + 16 * RPI * i));
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
              f32x16 acc = {};
#pragma unroll
              for (int i = 0; i < KS; ++i)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[hb][i], bk[i], acc, 0, 0, 0);
              const float r = relu_weighted_sum(acc, wv[hb]);
              p[sb] = hb == 0 ? r : p[sb] + r;
            }
          }
          return block_scores(p[0], p[1]);
        };
        // take block b's keys (lane l: score v of key l) into the list;
        // returns the list stores issued (0 or 1)
        auto take_block = [&](int b, float v) __attribute__((always_inline)) -> int {
          const int j = k0 + b * kTileKB + l;
          const uint32_t key = score_order_bits(v);
          bool take = j < nv && (!barred || key > bar);
          uint64_t bal = __ballot(take);
          if (bal == 0ull) return 0;
          if (cnt + __popcll(bal) > C) {  // no room (cnt > C - 64 > k): cut the list
            cut_list();
            sh = 0;  // the cut waited for every outstanding operation
            take = take && key > bar;
            bal = __ballot(take);
            if (bal == 0ull) return 0;
          }
          if (take) {
            list[cnt + ballot_rank(bal)] = make_uint2(key, (uint32_t)j);
            key_lo = min(key_lo, key);
            key_hi = max(key_hi, key);
            if (barred) atomicAdd(&s_hist[wave][window_bin(key, win_base, win_shift)], 1u);
          }
          cnt += __popcll(bal);
          if (cnt > C - kCutSoonB) s_cutreq[gblk & 1] = gblk;  // ask for a cut next iteration
          return 1;
        };
#pragma unroll
        for (int b = 0; b < 3; ++b)
          if (b < nb) stage(b);
        for (int b = 0; b < nb; b += BPI) {
          // outstanding after the last load of blocks b .. b + BPI - 1: the
          // loads of the blocks staged after it and the list stores of the
          // last SI iterations
          const int later = min(RING - 2 * BPI, max(nb - b - BPI, 0));
          int pend = 0;
#pragma unroll
          for (int i = 0; i < SI; ++i) pend += (sh >> (4 * i)) & 15;
          wait_vm_dyn(later * nlw + pend);
          lds_sync();  // blocks b .. b + BPI - 1 have landed; the previous ones are consumed
#pragma unroll
          for (int i = 0; i < BPI; ++i)
            if (b + 3 + i < nb) stage(b + 3 + i);
          sh <<= 4;
          // a cut asked for during the previous iteration: every wave whose
          // list is a quarter full above k cuts now, so that the waves of the
          // workgroup wait at the barrier for one cut rather than one each
          const bool cut_asked = s_cutreq[gblk & 1] == gblk;
          ++gblk;
          if (!act || k0 + b * kTileKB >= nv) continue;  // wave-uniform
          if (cut_asked && cnt > k + (C - k) / 4) {
            cut_list();
            sh = 0;
          }
          // the scores of the iteration's blocks first (straight-line code,
          // so that the head sums of one sub-block overlap the products of
          // the next), then their keys in position order
          const int nbk =
              min(min(BPI, nb - b), (nv - k0 - b * kTileKB + kTileKB - 1) / kTileKB);  // >= 1
          // (a block past the row's range scores whatever its ring slot
          // holds, never taken: no branch between the products)
          float v[BPI];
          // the products of this wave go first when waves compete for issue
          // (the other waves' head sums and list work fill the gaps)
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int i = 0; i < BPI; ++i) v[i] = score_block(b + i);
          __builtin_amdgcn_s_setprio(0);
          int ns = 0;
#pragma unroll
          for (int i = 0; i < BPI; ++i)
            if (i < nbk) ns += take_block(b + i, v[i]);
          sh |= ns;
        }
        __syncthreads();  // the ring is free for the next pass
      }
      seg = seg_end;
    }
  }
  if (cnt > k) {
    const uint32_t lo = barred ? bar : wave_min_u32(key_lo);
    list_compact(list, cnt, k, s_hist[wave], lo, wave_max_u32(key_hi));
    cnt = k;
  }
  if (t < T && l == 0) cand_cnt[(size_t)t * G + blockIdx.x] = cnt;
}

constexpr int kMergeNT = 256;

__global__ __launch_bounds__(kMergeNT) void topk_merge(const uint2* __restrict__ cand,
                                                       const int* __restrict__ cand_cnt, int G,
                                                       int C, int k, int by_pos,
                                                       int32_t* __restrict__ topk) {
  extern __shared__ uint64_t s_key[];  // merge_width(G, k) entries
  __shared__ int s_off[9];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) {
    int run = 0;
    for (int g = 0; g < G; ++g) {
      s_off[g] = run;
      run += cand_cnt[(size_t)t * G + g];
    }
    s_off[G] = run;
  }
  __syncthreads();
  const int total = min(s_off[G], kMergeMax);
  int nb = 64;
  while (nb < total) nb <<= 1;
  for (int i = tid; i < nb; i += kMergeNT) {
    uint64_t v = 0ull;
    if (i < total) {
      int g = 0;
      while (g + 1 < G && s_off[g + 1] <= i) ++g;
      const uint2 e = cand[((size_t)t * G + g) * C + (i - s_off[g])];
      v = ((uint64_t)e.x << 32) | (uint64_t)(0xffffffffu - e.y);
    }
    s_key[i] = v;
  }
  __syncthreads();
  for (int size = 2; size <= nb; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (nb >> 1); i += kMergeNT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t x = s_key[lo], y = s_key[hi];
        if ((x < y) == up) {
          s_key[lo] = y;
          s_key[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  const int n_out = min(k, total);
  int32_t* out = topk + (size_t)t * k;
  if (by_pos) {  // the same entries in ascending position order: a second sort
    int nb2 = 64;
    while (nb2 < n_out) nb2 <<= 1;
    for (int i = tid; i < nb2; i += kMergeNT)
      s_key[i] = i < n_out ? (uint64_t)(uint32_t)topk_key_pos(s_key[i]) : ~0ull;
    __syncthreads();
    for (int size = 2; size <= nb2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < (nb2 >> 1); i += kMergeNT) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint64_t x = s_key[lo], y = s_key[hi];
          if ((x > y) == up) {
            s_key[lo] = y;
            s_key[hi] = x;
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < k; i += kMergeNT) out[i] = i < n_out ? (int)(uint32_t)s_key[i] : -1;
    return;
  }
  for (int i = tid; i < k; i += kMergeNT) out[i] = i < n_out ? topk_key_pos(s_key[i]) : -1;
}

// One list per row (G = 1): the list holds the row's top min(k, n_valid)
// entries in ascending position order, so a stable sort by key descending
// (rocPRIM's block radix sort, over the bits in which the keys differ) gives
// the canonical order. grid = T, block = kMergeNT.
template <int IPT>
__global__ __launch_bounds__(kMergeNT) void topk_order(const uint2* __restrict__ cand,
                                                       const int* __restrict__ cand_cnt, int C,
                                                       int k, int by_pos,
                                                       int32_t* __restrict__ topk) {
  using Sorter = rocprim::block_radix_sort<uint32_t, kMergeNT, IPT, int>;
  __shared__ typename Sorter::storage_type storage;
  __shared__ uint32_t s_red[2][kMergeNT / DSA_WAVE];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int cnt = min(cand_cnt[t], k);
  const uint2* list = cand + (size_t)t * C;
  if (by_pos) {  // the list is in ascending position order already
    int32_t* out = topk + (size_t)t * k;
    for (int i = tid; i < k; i += kMergeNT) out[i] = i < cnt ? (int)list[i].y : -1;
    return;
  }
  uint32_t keys[IPT];
  int vals[IPT];
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int idx = tid * IPT + i;
    const uint2 e = idx < cnt ? list[idx] : make_uint2(0u, 0xffffffffu);
    keys[i] = e.x;
    vals[i] = (int)e.y;
    if (idx < cnt) {
      mn = min(mn, e.x);
      mx = max(mx, e.x);
    }
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane_id() == 0) {
    s_red[0][tid >> 6] = mn;
    s_red[1][tid >> 6] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kMergeNT / DSA_WAVE; ++w) {
    mn = min(mn, s_red[0][w]);
    mx = max(mx, s_red[1][w]);
  }
  const uint32_t diff = cnt > 0 ? mn ^ mx : 0u;
  if (diff != 0u)  // block-uniform; entries past cnt carry key 0 and stay last
    Sorter().sort_desc(keys, vals, storage, 0u, 32u - (unsigned)__builtin_clz(diff));
  int32_t* out = topk + (size_t)t * k;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int idx = tid * IPT + i;
    if (idx < k) out[idx] = idx < cnt ? vals[i] : -1;
  }
}

void fused_plan(int T, int cap, int k, int* G, int* L, int* C) {
  const int nrt = (T + 15) / 16;  // row tiles of 16 (of 8 with two head blocks: twice as many)
  const int gmax_k = kMergeMax / k < 8 ? kMergeMax / k : 8;
  const int gmax_cap = (cap + kTileMaxRK - 1) / kTileMaxRK;
  // about one workgroup per compute unit (a 16-row workgroup fills one);
  // more segments cost a merge of their lists per row
  int g = (256 + nrt - 1) / nrt;
  if (g > gmax_k) g = gmax_k;
  if (g > gmax_cap) g = gmax_cap;
  if (g < 1) g = 1;
  int len = (cap + g - 1) / g;
  len = (len + kTileMaxRK - 1) / kTileMaxRK * kTileMaxRK;
  *L = len;
  *G = (cap + len - 1) / len;
  // room above k: a cut keeps k to 1.5 k entries, so about k / 2 or more
  // keys are taken between cuts
  const int c = k + (k > 512 ? k : 512);
  *C = (c + 63) / 64 * 64;
}

template <int D, int HB>
static hipError_t launch_fused(const IndexerArgs& a, hipStream_t st) {
  int G = 1, L = 0, C = 0;
  fused_plan(a.T, a.MP * a.PS, a.k, &G, &L, &C);
  {
    ProfScope prof("idx_score_topk", st);
    constexpr int R = fused_rows<HB>();
    hipLaunchKernelGGL((idx_score_topk<D, HB>), dim3(G, (a.T + R - 1) / R), dim3(64 * R), 0, st,
                       a.q, a.w, a.cache, a.num_pages, a.pt, a.seq_lens, a.cu, a.T, a.S, a.H, a.PS,
                       a.MP, a.k, G, L, C, a.cand, a.cand_cnt);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (G == 1) {
    ProfScope prof("topk_order", st);
    if (a.k <= kMergeNT * 8)
      hipLaunchKernelGGL((topk_order<8>), dim3(a.T), dim3(kMergeNT), 0, st, a.cand, a.cand_cnt,
                         C, a.k, a.by_pos, a.topk);
    else
      hipLaunchKernelGGL((topk_order<16>), dim3(a.T), dim3(kMergeNT), 0, st, a.cand,
                         a.cand_cnt, C, a.k, a.by_pos, a.topk);
    return hipGetLastError();
  }
  // the LDS sort holds the row's lists, at most G * k entries, padded to a
  // power of two
  int nbmax = 64;
  while (nbmax < G * a.k) nbmax <<= 1;
  const size_t lds = (size_t)nbmax * 8;
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load() & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_merge),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kMergeMax * 8);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit);
  }
  ProfScope prof("topk_merge", st);
  hipLaunchKernelGGL(topk_merge, dim3(a.T), dim3(kMergeNT), lds, st, a.cand, a.cand_cnt, G, C,
                     a.k, a.by_pos, a.topk);
  return hipGetLastError();
}

// Each row of a top-k table in ascending position order, -1 entries last
// (as unsigned keys they are the largest): rocPRIM's block radix sort over
// the bits below the row's largest valid position + 1, so that -1 sorts as
// the all-ones key of that width, above every valid one. In place is fine: a
// row is read whole before the sort and written after it.
// grid = T, block = kMergeNT.
template <int IPT>
__global__ __launch_bounds__(kMergeNT) void topk_rows_ascending(const int32_t* __restrict__ in,
                                                                int k, int32_t* __restrict__ out) {
  using Sorter = rocprim::block_radix_sort<uint32_t, kMergeNT, IPT>;
  __shared__ typename Sorter::storage_type storage;
  __shared__ uint32_t s_red[kMergeNT / DSA_WAVE];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* row = in + (size_t)t * k;
  uint32_t keys[IPT];
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int idx = tid * IPT + i;
    const int v = idx < k ? row[idx] : -1;
    keys[i] = (uint32_t)v;
    if (v >= 0) mx = max(mx, (uint32_t)v);
  }
  mx = wave_max_u32(mx);
  if (lane_id() == 0) s_red[tid >> 6] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kMergeNT / DSA_WAVE; ++w) mx = max(mx, s_red[w]);
  const unsigned bits = 32u - (unsigned)__builtin_clz(mx + 1u);  // mx + 1 < 2^31
  Sorter().sort(keys, storage, 0u, bits);
  int32_t* orow = out + (size_t)t * k;
  const uint32_t all = bits >= 32u ? 0xffffffffu : (1u << bits) - 1u;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int idx = tid * IPT + i;
    if (idx < k) orow[idx] = (keys[i] & all) == all ? -1 : (int)keys[i];
  }
}

// The same for a top-k table whose rows hold distinct positions below cap
// (an indexer's): each row's positions become bits of an LDS bitmap of cap
// bits, whose prefix popcounts give every position its place. In place.
// grid = T, block = 256, dynamic LDS: 2 * ceil(cap / 32) words.
constexpr int kRowsMaxIPT = 16;  // k <= 4096 entries per row over 256 threads
__global__ __launch_bounds__(256) void topk_rows_bitmap(int32_t* __restrict__ topk, int k,
                                                        int cap) {
  extern __shared__ uint32_t s_bits[];  // nw bitmap words, then nw prefix counts
  __shared__ int s_scan[4];
  const int nw = (cap + 31) / 32;
  uint32_t* s_pre = s_bits + nw;
  const int tid = threadIdx.x;
  int32_t* row = topk + (size_t)blockIdx.x * k;
  for (int i = tid; i < nw; i += 256) s_bits[i] = 0u;
  __syncthreads();
  int v[kRowsMaxIPT];
#pragma unroll
  for (int e = 0; e < kRowsMaxIPT; ++e) {
    const int i = tid + 256 * e;
    v[e] = i < k ? row[i] : -1;
    if (v[e] >= cap) v[e] = -1;
    if (v[e] >= 0) atomicOr(&s_bits[v[e] >> 5], 1u << (v[e] & 31));
  }
  __syncthreads();
  // exclusive prefix of the words' popcounts: each thread a contiguous range
  const int wpt = (nw + 255) / 256, w0 = min(tid * wpt, nw), w1 = min(w0 + wpt, nw);
  int local = 0;
  for (int i = w0; i < w1; ++i) local += __popc(s_bits[i]);
  int total;
  int run = block_inclusive_scan<256>(local, s_scan, &total) - local;
  for (int i = w0; i < w1; ++i) {
    s_pre[i] = (uint32_t)run;
    run += __popc(s_bits[i]);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kRowsMaxIPT; ++e)
    if (v[e] >= 0) {
      const int wd = v[e] >> 5;
      row[s_pre[wd] + __popc(s_bits[wd] & ((1u << (v[e] & 31)) - 1u))] = v[e];
    }
  for (int i = total + tid; i < k; i += 256) row[i] = -1;
}

hipError_t topk_rows_distinct_order(int32_t* topk, int T, int k, int cap, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const size_t lds = (size_t)2 * ((cap + 31) / 32) * 4;
  if (cap > kRowsBitmapMaxCap) return topk_position_order(topk, topk, T, k, st);
  ProfScope prof("topk_rows_bitmap", st);
  hipLaunchKernelGGL(topk_rows_bitmap, dim3(T), dim3(256), lds, st, topk, k, cap);
  return hipGetLastError();
}

hipError_t topk_position_order(const int32_t* in, int32_t* out, int T, int k, hipStream_t st) {
  if (T == 0) return hipSuccess;
  ProfScope prof("topk_rows_ascending", st);
  if (k <= kMergeNT * 4)
    hipLaunchKernelGGL((topk_rows_ascending<4>), dim3(T), dim3(kMergeNT), 0, st, in, k, out);
  else if (k <= kMergeNT * 8)
    hipLaunchKernelGGL((topk_rows_ascending<8>), dim3(T), dim3(kMergeNT), 0, st, in, k, out);
  else
    hipLaunchKernelGGL((topk_rows_ascending<16>), dim3(T), dim3(kMergeNT), 0, st, in, k, out);
  return hipGetLastError();
}

hipError_t indexer_fused_topk(const IndexerArgs& a, hipStream_t st) {
  const int HB = (a.H + 31) / 32;
  switch (a.D) {
    case 32: return HB == 1 ? launch_fused<32, 1>(a, st) : launch_fused<32, 2>(a, st);
    case 64: return HB == 1 ? launch_fused<64, 1>(a, st) : launch_fused<64, 2>(a, st);
    case 128: return HB == 1 ? launch_fused<128, 1>(a, st) : launch_fused<128, 2>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dsa
