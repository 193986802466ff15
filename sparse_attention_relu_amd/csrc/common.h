// Device helpers shared by the libdsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define DSA_WAVE 64

// ---------------------------------------------------------------------------
// Ragged row bookkeeping: which sequence owns packed row t, and its absolute
// position abs_q = seq_len - q_len + (t - q_start) (sglang-jax "ref.py",
// streamindex_topk_ref). Binary search over cu_q_lens; rows at or beyond
// cu_q_lens[S] (or before cu_q_lens[0]) own no sequence (seq = -1).
// ---------------------------------------------------------------------------
struct RowInfo {
  int seq;      // owning sequence or -1
  int abs_q;    // absolute position of the row's query
  int kv;       // seq_len clamped to [0, cap]
  int n_valid;  // number of positions j with j < kv and j <= abs_q, in [0, cap]
};

__device__ __forceinline__ RowInfo row_info(const int32_t* __restrict__ cu,
                                            const int32_t* __restrict__ seq_lens, int S, int t,
                                            int cap) {
  RowInfo r;
  r.seq = -1;
  r.abs_q = -1;
  r.kv = 0;
  r.n_valid = 0;
  if (S <= 0 || t < cu[0] || t >= cu[S]) return r;
  int lo = 0, hi = S;  // first s with cu[s + 1] > t
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (cu[mid + 1] > t) hi = mid; else lo = mid + 1;
  }
  if (lo >= S) return r;
  const int s = lo;
  const int q0 = cu[s], q1 = cu[s + 1];
  int kv = seq_lens[s];
  r.seq = s;
  r.abs_q = kv - (q1 - q0) + (t - q0);
  kv = kv < 0 ? 0 : (kv > cap ? cap : kv);
  r.kv = kv;
  int n = r.abs_q + 1;
  n = n < kv ? n : kv;
  r.n_valid = n < 0 ? 0 : n;
  return r;
}

// Same result as row_info for a row index t that is uniform across the wave,
// called with every lane active: each lane loads one sequence's bounds and
// length, so the owner is found with one round of loads (per 64 sequences)
// and a ballot instead of a chain of dependent loads.
__device__ __forceinline__ RowInfo row_info_wave(const int32_t* __restrict__ cu,
                                                 const int32_t* __restrict__ seq_lens, int S,
                                                 int t, int cap) {
  RowInfo r;
  r.seq = -1;
  r.abs_q = -1;
  r.kv = 0;
  r.n_valid = 0;
  const int l = threadIdx.x & (DSA_WAVE - 1);
  for (int base = 0; base < S; base += DSA_WAVE) {
    const int i = base + l;
    const bool in = i < S;
    const int q0 = in ? cu[i] : 0;
    const int q1 = in ? cu[i + 1] : 0;
    const int kv = in ? seq_lens[i] : 0;
    // sequences of this group that end at or before t (cu is non-decreasing)
    const uint64_t done = __ballot(in && q1 <= t);
    const int c = __popcll(done);
    const int last = (S - base < DSA_WAVE ? S - base : DSA_WAVE);
    if (c < last) {
      // the same value in every lane; readfirstlane tells the compiler so
      const int s0 = __builtin_amdgcn_readfirstlane(__shfl(q0, c, DSA_WAVE));
      const int s1 = __builtin_amdgcn_readfirstlane(__shfl(q1, c, DSA_WAVE));
      const int sk = __builtin_amdgcn_readfirstlane(__shfl(kv, c, DSA_WAVE));
      if (t < s0) return r;  // before the owner's first row: no sequence
      r.seq = base + c;
      r.abs_q = sk - (s1 - s0) + (t - s0);
      const int kc = sk < 0 ? 0 : (sk > cap ? cap : sk);
      r.kv = kc;
      int n = r.abs_q + 1;
      n = n < kc ? n : kc;
      r.n_valid = n < 0 ? 0 : n;
      return r;
    }
  }
  return r;
}

__device__ __forceinline__ int clamp_page(int p, int num_pages) {
  return p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
}

// ---------------------------------------------------------------------------
// Lane helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & (DSA_WAVE - 1); }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, DSA_WAVE); }

// Number of set bits of a wave ballot below this lane.
__device__ __forceinline__ int ballot_rank(uint64_t mask) {
  const int l = lane_id();
  return __popcll(mask & ((l == 0) ? 0ull : (~0ull >> (64 - l))));
}

// ---------------------------------------------------------------------------
// Block-wide inclusive prefix sum of one int per thread (NT threads, NT a
// multiple of 64). `scratch` holds NT / 64 ints. Returns the inclusive sum;
// *total receives the block total. Contains two __syncthreads().
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* scratch, int* total) {
  const int l = lane_id();
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int u = __shfl_up(v, off, DSA_WAVE);
    if (l >= off) v += u;
  }
  if (l == 63) scratch[w] = v;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    int x = scratch[i];
    if (i < w) base += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return v + base;
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (round to nearest even; NaN stays NaN)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// Pack two floats into one dword of two bf16 (low = a), round to nearest
// even (one v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// Radix keys for exact top-k: larger key = earlier in the canonical order
// (score descending, then position ascending). -0.0 is folded onto +0.0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_order_bits(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t topk_key(float s, int pos) {
  return ((uint64_t)score_order_bits(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)pos);
}

__device__ __forceinline__ int topk_key_pos(uint64_t key) {
  return (int)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
}
