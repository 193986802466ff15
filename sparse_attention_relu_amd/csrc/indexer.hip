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

#include "common.h"
#include "kernels.h"

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

__device__ __forceinline__ float relu_weighted_sum(const f32x16& acc, const float (&wv)[16]) {
  float part = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) part += wv[r] * fmaxf(acc[r], 0.0f);
  return part;
}

// ---------------------------------------------------------------------------
// Streaming per-row scorer (decode and any ragged layout). One wave scores
// KPW consecutive positions of one row; keys go straight from HBM to the
// MFMA B operand, the query fragment stays in registers.
// grid = (ceil(cap / (4 * KPW)), T), block = 256.
// ---------------------------------------------------------------------------
template <int D, int HB, int KPW>
__global__ __launch_bounds__(256) void idx_score_rows(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint16_t* __restrict__ cache, int num_pages, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu, int T, int S, int H,
    int PS, int MP, float* __restrict__ scores, long ld) {
  constexpr int KS = D / 16;
  constexpr int HALF = D / 2;
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int m = l & 31, hf = l >> 5;
  const RowInfo ri = row_info(cu, seq_lens, S, t, MP * PS);
  const int j_begin = (blockIdx.x * 4 + wave) * KPW;
  if (ri.seq < 0 || j_begin >= ri.n_valid) return;
  const int j_end = min(j_begin + KPW, ri.n_valid);

  bf16x8 a[HB][KS];
  float wv[HB][16];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 32 * hb + m;
    load_q_frag<D>(q + ((size_t)t * H + (head < H ? head : 0)) * D + hf * HALF, head < H, a[hb]);
    load_head_weights(w + (size_t)t * H, H, hb, hf, wv[hb]);
  }
  const int32_t* ptrow = pt + (size_t)ri.seq * MP;
  float* srow = scores + (size_t)t * ld;

  for (int jb = j_begin; jb < j_end; jb += 32) {
    const int j = jb + m;
    const bool ok = j < j_end;
    const uint16_t* kp = cache;
    if (ok) {
      const int page = clamp_page(ptrow[j / PS], num_pages);
      kp = cache + ((size_t)page * PS + (j % PS)) * D + hf * HALF;
    }
    bf16x8 b[KS];
#pragma unroll
    for (int i = 0; i < KS; ++i)
      b[i] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(kp + 8 * i) : zero_u4());
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
    if (hf == 0 && ok) srow[j] = part;
  }
}

// ---------------------------------------------------------------------------
// Tiled MFMA scorer for query chunks (extend). A workgroup owns TR = NW * QPW
// consecutive packed rows and a range of RK key positions; every wave keeps
// QPW query fragments in registers, and 64-key blocks of the owning
// sequence's keys are staged once per workgroup through a double-buffered
// LDS ring and reused by all its rows. Rows of a tile may belong to several
// sequences: the tile is walked one sequence segment at a time.
// grid = (ceil(cap / RK), ceil(T / TR)), block = NW * 64.
// ---------------------------------------------------------------------------
template <int D, int HB, int QPW, int NW>
__global__ __launch_bounds__(NW * 64) void idx_score_tiles(
    const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint16_t* __restrict__ cache, int num_pages, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu, int T, int S, int H,
    int PS, int MP, int RK, float* __restrict__ scores, long ld) {
  constexpr int KS = D / 16;
  constexpr int HALF = D / 2;
  constexpr int TR = NW * QPW;
  constexpr int KB = 64;             // keys per LDS block
  constexpr int RS = D + 8;          // LDS row stride in bf16 (16 B pad)
  constexpr int CPR = D / 8;         // 16-byte chunks per key row
  constexpr int LOADS = (KB * CPR + NW * 64 - 1) / (NW * 64);
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[2][KB * RS];
  __shared__ __attribute__((aligned(16))) float s_w[TR][HB * 32];
  __shared__ int s_seq[TR], s_nv[TR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = lane_id();
  const int m = l & 31, hf = l >> 5;
  const int t0 = blockIdx.y * TR;
  const int cap = MP * PS;
  if (tid < TR) {
    const int t = t0 + tid;
    RowInfo ri;
    ri.seq = -1;
    ri.n_valid = 0;
    if (t < T) ri = row_info(cu, seq_lens, S, t, cap);
    s_seq[tid] = ri.seq;
    s_nv[tid] = ri.n_valid;
  }
  // head weights of the tile's rows (0 for padding heads and rows)
  for (int i = tid; i < TR * HB * 32; i += NW * 64) {
    const int r = i / (HB * 32), h = i % (HB * 32);
    const int t = t0 + r;
    s_w[r][h] = (t < T && h < H) ? w[(size_t)t * H + h] : 0.0f;
  }
  __syncthreads();
  const int r_lo = blockIdx.x * RK;

  int seg = 0;
  while (seg < TR) {
    const int s = s_seq[seg];
    int seg_end = seg + 1;
    while (seg_end < TR && s_seq[seg_end] == s) ++seg_end;
    const int n_hi = s >= 0 ? s_nv[seg_end - 1] : 0;
    const int k0 = r_lo, k1 = min(r_lo + RK, n_hi);
    if (s >= 0 && k0 < k1) {
      // this wave's query rows inside the segment
      bf16x8 a[QPW][HB][KS];
      bool act[QPW];
      int nv[QPW];
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        const int r = wave * QPW + qi;
        nv[qi] = s_nv[r];
        act[qi] = (r >= seg) && (r < seg_end) && (nv[qi] > k0);
        const int t = t0 + r;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const int head = 32 * hb + m;
          const bool okq = act[qi] && head < H;
          load_q_frag<D>(q + ((size_t)(okq ? t : 0) * H + (head < H ? head : 0)) * D + hf * HALF,
                         okq, a[qi][hb]);
        }
      }
      const int32_t* ptrow = pt + (size_t)s * MP;

      // staged loads of one 64-key block into registers, then LDS
      uint4 stage[LOADS];
      auto fetch = [&](int kb) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int idx = tid + i * NW * 64;
          const int row = idx / CPR, c = idx % CPR;
          const int j = kb + row;
          uint4 v = zero_u4();
          if (idx < KB * CPR && j < k1) {
            const int page = clamp_page(ptrow[j / PS], num_pages);
            v = *reinterpret_cast<const uint4*>(cache + ((size_t)page * PS + (j % PS)) * D + 8 * c);
          }
          stage[i] = v;
        }
      };
      auto commit = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int idx = tid + i * NW * 64;
          if (idx < KB * CPR) {
            const int row = idx / CPR, c = idx % CPR;
            *reinterpret_cast<uint4*>(&kbuf[buf][row * RS + 8 * c]) = stage[i];
          }
        }
      };

      fetch(k0);
      commit(0);
      __syncthreads();
      int buf = 0;
      for (int kb = k0; kb < k1; kb += KB) {
        const bool more = kb + KB < k1;
        if (more) fetch(kb + KB);
#pragma unroll 1
        for (int sb = 0; sb < KB / 32; ++sb) {
          const int jrow = sb * 32 + m;
          bf16x8 b[KS];
#pragma unroll
          for (int i = 0; i < KS; ++i)
            b[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&kbuf[buf][jrow * RS + hf * HALF + 8 * i]));
          const int j = kb + jrow;
#pragma unroll
          for (int qi = 0; qi < QPW; ++qi) {
            if (!act[qi]) continue;
            float part = 0.0f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
              f32x16 acc = {};
#pragma unroll
              for (int i = 0; i < KS; ++i)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[qi][hb][i], b[i], acc, 0, 0, 0);
              // weights of accumulator rows 8 c + 4 hf + (0..3), c = 0..3
              const float* wr = &s_w[wave * QPW + qi][32 * hb + 4 * hf];
              float wv[16];
#pragma unroll
              for (int c4 = 0; c4 < 4; ++c4) {
                const float4 v = *reinterpret_cast<const float4*>(wr + 8 * c4);
                wv[4 * c4 + 0] = v.x;
                wv[4 * c4 + 1] = v.y;
                wv[4 * c4 + 2] = v.z;
                wv[4 * c4 + 3] = v.w;
              }
              part += relu_weighted_sum(acc, wv);
            }
            part += shfl_xor_f(part, 32);
            if (hf == 0 && j < nv[qi])
              scores[(size_t)(t0 + wave * QPW + qi) * ld + j] = part;
          }
        }
        if (more) commit(buf ^ 1);
        __syncthreads();
        buf ^= 1;
      }
    }
    seg = seg_end;
  }
}

// ---------------------------------------------------------------------------
// Exact top-k per row: radix select over 64-bit keys
//   key(j) = order_bits(score[j]) << 32 | (2^32 - 1 - j)
// (distinct per position; larger key = earlier in the canonical order).
// 12-bit digits from the top narrow the search until the boundary bin fits
// the candidate buffer; a collect pass then moves every key above the
// boundary bin into the output list and the boundary bin's keys into the
// candidate list, which is sorted to take the missing ones. The k winners
// are finally sorted in LDS (bitonic, descending key) and written as
// positions, -1 padded.
// grid = T, block = NT, dynamic LDS = (kp2 + cand_cap) * 8 + 4096 * 4.
// ---------------------------------------------------------------------------
template <int NT>
__device__ void bitonic_sort_desc(uint64_t* a, int n) {
  for (int k2 = 2; k2 <= n; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += NT) {
        const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int hi = lo + j;
        const uint64_t x = a[lo], y = a[hi];
        const bool desc = (lo & k2) == 0;
        if (desc ? (x < y) : (x > y)) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// wave-aggregated append to an LDS counter; returns this lane's slot
__device__ __forceinline__ int wave_append(bool pred, int* counter) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return -1;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  int base = 0;
  if (lane_id() == leader) base = atomicAdd(counter, __popcll(mask));
  base = __shfl(base, leader, DSA_WAVE);
  return pred ? base + ballot_rank(mask) : -1;
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_select(const float* __restrict__ scores, long ld,
                                                  const int32_t* __restrict__ cu,
                                                  const int32_t* __restrict__ seq_lens, int S,
                                                  int cap, int k, int kp2, int cand_cap,
                                                  int32_t* __restrict__ topk) {
  extern __shared__ uint64_t smem64[];
  uint64_t* outk = smem64;
  uint64_t* cand = outk + kp2;
  uint32_t* hist = reinterpret_cast<uint32_t*>(cand + cand_cap);
  __shared__ int s_cnt[4];
  __shared__ int s_scan[NT / 64];

  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const RowInfo ri = row_info(cu, seq_lens, S, t, cap);
  const int n = ri.n_valid;
  const float* row = scores + (size_t)t * ld;
  int32_t* orow = topk + (size_t)t * k;
  if (n == 0) {
    for (int i = tid; i < k; i += NT) orow[i] = -1;
    return;
  }
  if (tid == 0) {
    s_cnt[0] = 0;
    s_cnt[1] = 0;
    s_cnt[2] = 0;
    s_cnt[3] = 0;
  }
  __syncthreads();

  int count;
  if (n <= k) {
    for (int j = tid; j < n; j += NT) outk[j] = topk_key(row[j], j);
    count = n;
  } else {
    uint64_t prefix = 0;
    int pbits = 0;
    int need = k;
    while (true) {
      const int width = min(12, 64 - pbits);
      const int shift = 64 - pbits - width;
      const int nb = 1 << width;
      for (int i = tid; i < 4096; i += NT) hist[i] = 0;
      __syncthreads();
      for (int j = tid; j < n; j += NT) {
        const uint64_t key = topk_key(row[j], j);
        if (pbits == 0 || (key >> (64 - pbits)) == prefix)
          atomicAdd(&hist[(key >> shift) & (uint64_t)(nb - 1)], 1u);
      }
      __syncthreads();
      // suffix counts from the highest bin down: thread tid owns the
      // 4096 / NT bins nb-1-tid*BPT .. nb-BPT-tid*BPT
      constexpr int BPT = 4096 / NT;
      int local = 0;
#pragma unroll
      for (int c = 0; c < BPT; ++c) {
        const int b = nb - 1 - tid * BPT - c;
        if (b >= 0) local += (int)hist[b];
      }
      int total;
      const int incl = block_inclusive_scan<NT>(local, s_scan, &total);
      const int excl = incl - local;
      if (excl < need && need <= incl) {
        int run = excl;
#pragma unroll
        for (int c = 0; c < BPT; ++c) {
          const int b = nb - 1 - tid * BPT - c;
          if (b < 0) break;
          const int h = (int)hist[b];
          if (run + h >= need) {
            s_cnt[2] = b;
            s_cnt[3] = run;
            break;
          }
          run += h;
        }
      }
      __syncthreads();
      const int dstar = s_cnt[2];
      const int above = s_cnt[3];
      need -= above;
      prefix = (pbits == 0 ? 0ull : (prefix << width)) | (uint64_t)dstar;
      pbits += width;
      const int bin = (int)hist[dstar];
      __syncthreads();
      if (bin <= cand_cap || pbits >= 64) break;
    }
    // collect
    for (int j0 = 0; j0 < n; j0 += NT) {
      const int j = j0 + tid;
      uint64_t key = 0;
      uint64_t v = 0;
      const bool in = j < n;
      if (in) {
        key = topk_key(row[j], j);
        v = pbits >= 64 ? key : (key >> (64 - pbits));
      }
      const int io = wave_append(in && v > prefix, &s_cnt[0]);
      if (io >= 0 && io < kp2) outk[io] = key;
      const int ic = wave_append(in && v == prefix, &s_cnt[1]);
      if (ic >= 0 && ic < cand_cap) cand[ic] = key;
    }
    __syncthreads();
    const int nc = min(s_cnt[1], cand_cap);
    const int base = min(s_cnt[0], k);
    need = min(need, min(nc, k - base));
    const int cp2 = next_pow2(nc);
    for (int i = nc + tid; i < cp2; i += NT) cand[i] = 0;
    __syncthreads();
    bitonic_sort_desc<NT>(cand, cp2);
    for (int i = tid; i < need; i += NT) outk[base + i] = cand[i];
    count = base + need;
  }
  __syncthreads();
  const int op2 = next_pow2(count);
  for (int i = count + tid; i < op2; i += NT) outk[i] = 0;
  __syncthreads();
  bitonic_sort_desc<NT>(outk, op2);
  for (int i = tid; i < k; i += NT) orow[i] = i < count ? topk_key_pos(outk[i]) : -1;
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------
template <int D, int HB>
static hipError_t launch_rows(const IndexerArgs& a, hipStream_t st) {
  constexpr int KPW = 64;
  const int cap = a.MP * a.PS;
  dim3 grid((cap + 4 * KPW - 1) / (4 * KPW), a.T);
  hipLaunchKernelGGL((idx_score_rows<D, HB, KPW>), grid, dim3(256), 0, st, a.q, a.w, a.cache,
                     a.num_pages, a.pt, a.seq_lens, a.cu, a.T, a.S, a.H, a.PS, a.MP, a.scores,
                     a.ld);
  return hipGetLastError();
}

template <int D, int HB>
static hipError_t launch_tiles(const IndexerArgs& a, hipStream_t st) {
  constexpr int QPW = 4 / HB, NW = 8, TR = QPW * NW;
  const int cap = a.MP * a.PS;
  const int RK = 2048;
  dim3 grid((cap + RK - 1) / RK, (a.T + TR - 1) / TR);
  hipLaunchKernelGGL((idx_score_tiles<D, HB, QPW, NW>), grid, dim3(NW * 64), 0, st, a.q, a.w,
                     a.cache, a.num_pages, a.pt, a.seq_lens, a.cu, a.T, a.S, a.H, a.PS, a.MP, RK,
                     a.scores, a.ld);
  return hipGetLastError();
}

template <int D, int HB>
static hipError_t launch_score(const IndexerArgs& a, hipStream_t st) {
  return a.max_q_len <= 1 ? launch_rows<D, HB>(a, st) : launch_tiles<D, HB>(a, st);
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

size_t topk_select_lds_bytes(int k) {
  int kp2 = 1;
  while (kp2 < k) kp2 <<= 1;
  return (size_t)(kp2 + kTopkCandCap) * 8 + 4096 * 4;
}

hipError_t indexer_select(const IndexerArgs& a, hipStream_t st) {
  constexpr int NT = 1024;
  int kp2 = 1;
  while (kp2 < a.k) kp2 <<= 1;
  const size_t lds = topk_select_lds_bytes(a.k);
  // raise the dynamic-LDS limit of the select kernel once per device
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load() & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_select<NT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit);
  }
  hipLaunchKernelGGL((topk_select<NT>), dim3(a.T), dim3(NT), lds, st, a.scores, a.ld, a.cu,
                     a.seq_lens, a.S, a.MP * a.PS, a.k, kp2, kTopkCandCap, a.topk);
  return hipGetLastError();
}

}  // namespace dsa
