// Sparse absorbed-MLA attention for gfx950: decode (per-row selection lists)
// and query-block extend (shared page union + per-token membership).
//
// Semantics: sglang-jax "ref.py", sparse_mla_ref — logits over the packed
// 576-wide latent row [c_kv 512 | k_rope 64] times sm_scale, softmax over the
// valid selected positions, value = the row's first 512 columns. The extend
// kernel follows "sparse_mla_prefill_qblock.py", _qblock_kernel: one fetch per
// union page for all QB * H rows of a block, per-row validity = membership
// bit AND causal AND kv_len, flash-style online softmax.
//
// MFMA v_mfma_f32_16x16x32_bf16 is used for both products. Operand layout
// (per lane l, group g = l / 16, column c = l % 16):
//   A: row c, k-values 8 g .. 8 g + 7 of the step;  B: column c, same k;
//   C: rows 4 g + r (r < 4), column c.
#include <atomic>

#include "common.h"
#include "kernels.h"
#include "profile.h"

namespace dsa {

constexpr int DK = 576;
constexpr int DV = 512;
constexpr int NR = 32;        // latent rows staged per step
constexpr int KRS = DK + 8;   // LDS row stride in bf16 (1168 B) -> conflict-free b128 reads
constexpr int PRS = NR + 8;   // P row stride in bf16

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// B operand of P.V: 8 consecutive staged rows (keys) of one value column.
__device__ __forceinline__ bf16x8 load_v_col(const uint16_t* kvs, int key0, int col) {
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = kvs[(key0 + e) * KRS + col];
  bf16x8 r;
  __builtin_memcpy(&r, v, 16);
  return r;
}

// Stage NR latent rows into LDS; rows with pos < 0 are zero-filled (never read
// from HBM, so poisoned or unmapped slots cannot leak in).
__device__ __forceinline__ void stage_rows(uint16_t* kvs, const uint16_t* __restrict__ kv,
                                           int row_stride, const int* s_src, int nthreads) {
  constexpr int CPR = DK / 8;  // 72 chunks of 16 B per row
  for (int idx = threadIdx.x; idx < NR * CPR; idx += nthreads) {
    const int row = idx / CPR, c = idx % CPR;
    const int src = s_src[row];
    uint4 v = zero_u4();
    if (src >= 0) v = *reinterpret_cast<const uint4*>(kv + (size_t)src * row_stride + 8 * c);
    *reinterpret_cast<uint4*>(&kvs[row * KRS + 8 * c]) = v;
  }
}

// ---------------------------------------------------------------------------
// Decode: grid = (nch, T), block = 256. Workgroup (c, t) attends row t over
// selections [c * CH, (c + 1) * CH) in stages of NR rows, and leaves its
// partial (row max m, sum l, unnormalised O) per head for the combine
// kernel. The source slot of every selection is resolved first; each stage's
// rows are then staged through registers one stage ahead, so the next
// stage's HBM reads are in flight while the current one is computed.
// ---------------------------------------------------------------------------
constexpr int kDecMaxCH = 256;
constexpr int kStageLoads = NR * (DK / 8) / 256;  // 16-byte loads per thread per stage

__device__ __forceinline__ void fetch_stage(uint4 (&r)[kStageLoads], const uint16_t* __restrict__ kv,
                                            int row_stride, const int* s_src) {
  constexpr int CPR = DK / 8;
#pragma unroll
  for (int i = 0; i < kStageLoads; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int row = idx / CPR, c = idx % CPR;
    const int src = s_src[row];
    r[i] = src >= 0 ? *reinterpret_cast<const uint4*>(kv + (size_t)src * row_stride + 8 * c)
                    : zero_u4();
  }
}

__device__ __forceinline__ void commit_stage(const uint4 (&r)[kStageLoads], uint16_t* kvs) {
  constexpr int CPR = DK / 8;
#pragma unroll
  for (int i = 0; i < kStageLoads; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int row = idx / CPR, c = idx % CPR;
    *reinterpret_cast<uint4*>(&kvs[row * KRS + 8 * c]) = r[i];
  }
}

template <int HB>
__global__ __launch_bounds__(256) void mla_decode_partial(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int row_stride,
    int num_pages, const int32_t* __restrict__ pt, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ topk, int T, int S, int H, int k,
    int PS, int MP, float sm_scale, int CH, int nch, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int NH = HB * 16;
  __shared__ __attribute__((aligned(16))) uint16_t kvs[NR * KRS];
  __shared__ __attribute__((aligned(16))) uint16_t ps[NH * PRS];
  __shared__ float s_logit[NH][NR + 1];
  __shared__ float s_m[NH], s_l[NH], s_alpha[NH];
  __shared__ int s_src[kDecMaxCH];
  __shared__ int s_any[kDecMaxCH / NR];

  const int c = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, l = lane_id();
  const int g = l >> 4, col = l & 15;
  const RowInfo ri = row_info_wave(cu, seq_lens, S, t, MP * PS);
  const int i_begin = c * CH, i_end = min(i_begin + CH, k);
  const int nst = ri.seq >= 0 ? (i_end - i_begin + NR - 1) / NR : 0;
  if (tid < NH) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.0f;
  }
  if (tid < kDecMaxCH / NR) s_any[tid] = 0;
  __syncthreads();
  if (ri.seq >= 0) {
    const int32_t* sel = topk + (size_t)t * k;
    const int32_t* ptrow = pt + (size_t)ri.seq * MP;
    for (int i = tid; i < nst * NR; i += 256) {
      const int ii = i_begin + i;
      int src = -1;
      if (ii < i_end) {
        const int j = sel[ii];
        if (j >= 0 && j < ri.kv && j <= ri.abs_q)
          src = clamp_page(ptrow[j / PS], num_pages) * PS + (j % PS);
      }
      s_src[i] = src;
      if (src >= 0) s_any[i / NR] = 1;
    }
  }
  __syncthreads();
  f32x4 acc[HB][8];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 stage[kStageLoads];
  if (nst > 0) fetch_stage(stage, kv, row_stride, s_src);
  for (int st = 0; st < nst; ++st) {
    const int* src_st = s_src + st * NR;
    if (!s_any[st]) {  // nothing valid here; keep the pipeline moving
      if (st + 1 < nst) fetch_stage(stage, kv, row_stride, src_st + NR);
      continue;
    }
    __syncthreads();  // previous stage's readers of kvs / ps are done
    commit_stage(stage, kvs);
    if (st + 1 < nst) fetch_stage(stage, kv, row_stride, src_st + NR);
    __syncthreads();
    // logits: tiles (hb, nb) of 16 heads x 16 keys, spread over the waves
    for (int tile = wave; tile < HB * 2; tile += 4) {
      const int hb = tile >> 1, nb = tile & 1;
      const int head = hb * 16 + col;
      const uint16_t* qrow = q + ((size_t)t * H + (head < H ? head : 0)) * DK + 8 * g;
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 6
      for (int i = 0; i < DK / 32; ++i) {
        const bf16x8 a = as_bf16x8(head < H ? *reinterpret_cast<const uint4*>(qrow + 32 * i) : zero_u4());
        const bf16x8 b = as_bf16x8(*reinterpret_cast<const uint4*>(&kvs[(16 * nb + col) * KRS + 32 * i + 8 * g]));
        sacc = mfma16(a, b, sacc);
      }
      const bool kvalid = src_st[16 * nb + col] >= 0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s_logit[hb * 16 + 4 * g + r][16 * nb + col] = kvalid ? sacc[r] * sm_scale : -INFINITY;
    }
    __syncthreads();
    // online softmax: 16 threads per head, 2 keys each
    for (int hh = tid >> 4; hh < NH; hh += 16) {
      const int kk = (tid & 15) * 2;
      const float x0 = s_logit[hh][kk], x1 = s_logit[hh][kk + 1];
      float mx = fmaxf(x0, x1);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
      const float m_old = s_m[hh];
      const float m_new = fmaxf(m_old, mx);
      float p0 = 0.f, p1 = 0.f, alpha = 1.f;
      if (m_new != -INFINITY) {
        p0 = __expf(x0 - m_new);
        p1 = __expf(x1 - m_new);
        alpha = __expf(m_old - m_new);
      }
      float sum = p0 + p1;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) sum += shfl_xor_f(sum, o);
      *reinterpret_cast<uint32_t*>(&ps[hh * PRS + kk]) = pack_bf16x2(p0, p1);
      if ((tid & 15) == 0) {
        s_alpha[hh] = alpha;
        s_m[hh] = m_new;
        s_l[hh] = s_l[hh] * alpha + sum;
      }
    }
    __syncthreads();
    // P.V for this wave's 128 value columns
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&ps[(hb * 16 + col) * PRS + 8 * g]));
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = s_alpha[hb * 16 + 4 * g + r];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[hb][nb][r] *= al[r];
        const bf16x8 b = load_v_col(kvs, 8 * g, 128 * wave + 16 * nb + col);
        acc[hb][nb] = mfma16(a, b, acc[hb][nb]);
      }
    }
  }
  __syncthreads();
  const size_t base = ((size_t)t * nch + c) * H;
  if (tid < H) {
    part_ml[(base + tid) * 2 + 0] = s_m[tid];
    part_ml[(base + tid) * 2 + 1] = s_l[tid];
  }
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int head = hb * 16 + 4 * g + r;
      if (head >= H) continue;
      float* orow = part_o + (base + head) * DV + 128 * wave + col;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) orow[16 * nb] = acc[hb][nb][r];
    }
}

// grid = (T, H), block = 128 (4 value columns per thread): merge the nch
// partials of (t, h): out = sum_c e^(m_c - M) O_c / sum_c e^(m_c - M) l_c.
__global__ __launch_bounds__(128) void mla_decode_combine(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int H, int nch,
                                                          uint16_t* __restrict__ out) {
  extern __shared__ float s_w[];  // nch weights
  __shared__ float s_red[2];
  const int t = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const size_t base = (size_t)t * nch * H;
  // row maximum over chunks with mass
  float mx = -INFINITY;
  for (int c = tid; c < nch; c += 128) {
    const float m = part_ml[(base + (size_t)c * H + h) * 2];
    const float l = part_ml[(base + (size_t)c * H + h) * 2 + 1];
    if (l > 0.f) mx = fmaxf(mx, m);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
  if (lane_id() == 0) s_red[threadIdx.x >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(s_red[0], s_red[1]);
  __syncthreads();
  float L = 0.f;
  for (int c = tid; c < nch; c += 128) {
    const float m = part_ml[(base + (size_t)c * H + h) * 2];
    const float l = part_ml[(base + (size_t)c * H + h) * 2 + 1];
    const float wgt = l > 0.f ? __expf(m - M) : 0.f;
    s_w[c] = wgt;
    L += wgt * l;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += shfl_xor_f(L, o);
  if (lane_id() == 0) s_red[threadIdx.x >> 6] = L;
  __syncthreads();
  const float Lt = s_red[0] + s_red[1];
  const float inv = Lt > 0.f ? 1.0f / Lt : 0.f;
  const int d = 4 * tid;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  // batches of independent loads so the partials stream instead of one
  // dependent round trip per chunk
  constexpr int U = 8;
  for (int c0 = 0; c0 < nch; c0 += U) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u;
      v[u] = (c < nch && s_w[c] != 0.f)
                 ? *reinterpret_cast<const float4*>(part_o + (base + (size_t)c * H + h) * DV + d)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wgt = c0 + u < nch ? s_w[c0 + u] : 0.f;
      o.x += wgt * v[u].x;
      o.y += wgt * v[u].y;
      o.z += wgt * v[u].z;
      o.w += wgt * v[u].w;
    }
  }
  uint2 packed;
  packed.x = pack_bf16x2(o.x * inv, o.y * inv);
  packed.y = pack_bf16x2(o.z * inv, o.w * inv);
  *reinterpret_cast<uint2*>(out + ((size_t)t * H + h) * DV + d) = packed;
}

int mla_decode_chunk(int T, int k) {
  // aim at about one workgroup per compute unit, 32 .. kDecMaxCH selections each
  const int nsub = (k + NR - 1) / NR;
  long per = ((long)T * nsub) / 256;
  if (per < 1) per = 1;
  if (per > kDecMaxCH / NR) per = kDecMaxCH / NR;
  return (int)per * NR;
}

hipError_t mla_decode(const MlaArgs& a, hipStream_t st) {
  const int CH = mla_decode_chunk(a.T, a.k);
  const int nch = (a.k + CH - 1) / CH;
  if (a.T == 0) return hipSuccess;
  dim3 grid(nch, a.T);
  const int HB = (a.H + 15) / 16;
#define DSA_DEC(hb)                                                                           \
  hipLaunchKernelGGL((mla_decode_partial<hb>), grid, dim3(256), 0, st, a.q, a.kv, a.row_stride, \
                     a.num_pages, a.pt, a.seq_lens, a.cu, a.topk, a.T, a.S, a.H, a.k, a.PS,    \
                     a.MP, a.sm_scale, CH, nch, a.part_o, a.part_ml)
  {
    ProfScope prof("mla_decode_partial", st);
    switch (HB) {
      case 1: DSA_DEC(1); break;
      case 2: DSA_DEC(2); break;
      case 3: DSA_DEC(3); break;
      case 4: DSA_DEC(4); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef DSA_DEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ProfScope prof("mla_decode_combine", st);
  hipLaunchKernelGGL(mla_decode_combine, dim3(a.T, a.H), dim3(128), (size_t)nch * sizeof(float),
                     st, a.part_o, a.part_ml, a.H, nch, a.out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Extend (query block): one fetch of each union page for all QB * H rows of
// a block ("sparse_mla_prefill_qblock.py", _qblock_kernel).
//
// Workgroup = 2 wave pairs x 32 rows (row = q * H + h of the block). Both
// waves of a pair keep the same 32 rows' query fragments in registers; per
// page, wave `role` of the pair computes
//   S^T = K . Q^T for keys 32 role .. 32 role + 31 of the page
//     (v_mfma_f32_32x32x16_bf16: M = keys, N = rows, K = 576), and
//   O^T += V^T . P^T for value columns 256 role .. 256 role + 255 over all
//     64 keys (M = value columns, N = rows, K = keys).
// The two halves meet through LDS twice per page: the row maxima (for the
// shared online-softmax offset) and the bf16 P^T fragments. A lane's S^T
// accumulator holds 16 keys of ONE row, which is exactly the layout of the
// P^T operand, so P is packed in place. V^T fragments come from the
// row-major page through transposed 16-bit LDS reads (ds_read_b64_tr_b16:
// inside each 16-lane group, lanes 4k..4k+3 supply 16 consecutive values of
// row k and lane j receives column j of the 4 rows), so one row-major copy
// of the page serves both products.
//
// Pages are staged with direct global->LDS 16-byte loads into two 72 KB
// buffers (double buffering: page s+1 is in flight while page s is used).
// Within a 1152-byte row, 16-byte chunk c < 64 is stored at c ^ (row & 15)
// so that the rows read by a lane group hit distinct banks. Rows beyond the
// page or at positions >= kv_len are filled from the page's row 0 (a valid
// row whenever the page has any); their keys are masked, so they only ever
// meet probability 0 on finite data.
//
// The softmax offset is updated lazily: the accumulator is rescaled only
// when a row's maximum grows by more than kLazyMax (probabilities stay below
// e^8 before normalisation), which leaves the normalised result unchanged.
// ---------------------------------------------------------------------------
constexpr int XW = 4;                          // waves per workgroup (2 pairs)
constexpr int XROWS = 64;                      // rows per workgroup
constexpr int PROWS = 64;                      // rows per staged page (PS <= 64)
constexpr int NOPE_B = 1024;                   // staged bytes per row, columns 0..511
constexpr int ROPE_B = 128;                    // staged bytes per row, columns 512..575
constexpr int ROPE_OFF = PROWS * NOPE_B;       // rope region after the 64 nope rows
constexpr int PAGE_BYTES = PROWS * (NOPE_B + ROPE_B);  // 73728
constexpr int GLL_N = PAGE_BYTES / 1024 / XW;  // direct loads per wave per page (18)
constexpr float kLazyMax = 8.0f;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

// Swizzles of 16-byte chunks. Nope row r keeps chunk c (0..63) at slot
// c ^ nope_x(r), nope_x(r) = 2 (r & 7) + ((r >> 3) & 1): any 16 consecutive
// rows read at one chunk hit 16 distinct bank groups (S^T reads), and the 4
// consecutive rows x 2 adjacent chunks of one transposed read hit 8 (V^T
// reads). Rope row r keeps chunk c (0..7) at c ^ ((r >> 1) & 7).
__device__ __forceinline__ int nope_x(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int rope_x(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// [15:14], expcnt[6:4] and lgkmcnt[11:8] left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

struct PageMeta {
  int page, lp, sp, kvp;
};

__device__ __forceinline__ PageMeta page_meta(const int32_t* __restrict__ units,
                                              const int32_t* __restrict__ pt,
                                              const int32_t* __restrict__ seq_lens, int b,
                                              int u_max, int slot, int S, int MP, int cap,
                                              int num_pages) {
  PageMeta pm;
  int key = units[(size_t)b * u_max + slot];
  key = key < 0 ? 0 : (key >= S * MP ? S * MP - 1 : key);
  pm.sp = key / MP;
  pm.lp = key % MP;
  int kvp = seq_lens[pm.sp];
  pm.kvp = kvp < 0 ? 0 : (kvp > cap ? cap : kvp);
  pm.page = clamp_page(pt[key], num_pages);
  return pm;
}

// Issue this wave's GLL_N direct loads of one page into an LDS buffer. Load
// I of the page (I = GLL_N * wave + n) fills LDS bytes [1024 I, 1024 I + 1024),
// 16 bytes per lane: loads 0..63 are the nope rows (one row each), loads
// 64..71 the rope rows (8 rows each). Rows beyond the page or at positions
// >= kv_len read the page's row 0 instead.
__device__ __forceinline__ void stage_page(unsigned char* buf, const uint16_t* __restrict__ kv,
                                           int row_stride, const PageMeta& pm, int PS,
                                           int wave, int) {
  // lane id from a volatile instruction keeps this cheap arithmetic at its use
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  const uint16_t* pg = kv + (size_t)pm.page * PS * row_stride;
  const int valid_rows = min(PS, pm.kvp - pm.lp * PS);  // rows [0, valid_rows) are live
#pragma unroll
  for (int n = 0; n < GLL_N; ++n) {
    const int I = GLL_N * wave + n;  // wave-uniform
    int r, c;
    if (I < PROWS) {
      r = I;
      c = l ^ nope_x(r);
    } else {
      r = ((I - PROWS) << 3) + (l >> 3);
      c = 64 + ((l & 7) ^ rope_x(r));
    }
    const int use = r < valid_rows ? r : 0;
    const uint16_t* src = pg + (size_t)use * row_stride + 8 * c;
    // issued as inline assembly so that the compiler does not make every
    // later LDS read wait for these loads; completion is awaited explicitly
    const uint32_t dst =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)(buf + I * 1024));
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(dst)
                 : "memory", "m0");
  }
}

// Workgroup barrier that publishes this wave's LDS writes but, unlike
// __syncthreads(), does not wait for outstanding global->LDS loads (their
// completion is awaited explicitly with wait_vmcnt where it matters).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

struct ExtArgs {
  const uint16_t* __restrict__ kv;
  const int32_t* __restrict__ pt;
  const int32_t* __restrict__ seq_lens;
  const int32_t* __restrict__ units;
  const uint64_t* __restrict__ member;
  int row_stride, num_pages, S, PS, MP, QB, u_max, cap, b, u_lim;
  float sm_scale;
};

struct ExtLane {
  int wave, l, pr, role, g, m, qloc;
  int soff[12];    // S^T reads: byte offsets of this lane's 36 chunks (see ext_offsets)
  int toff[2][4];  // V^T transposed reads: per-lane parts of the byte offsets
  RowInfo ri;
  bf16x8 qb[DK / 16];
  f32x16 o[8];
  float m_used, l_part;
};

// One union page: `cur` holds it, `nxt` receives the next one meanwhile.
// The __restrict__ LDS pointers let the compiler see that reads of `cur`
// and of the exchange buffers never alias the loads in flight into `nxt`.
__device__ __forceinline__ void ext_step(const ExtArgs& A, ExtLane& X, int slot,
                                         unsigned char* __restrict__ cur,
                                         unsigned char* __restrict__ nxt,
                                         bf16x8* __restrict__ pf, float* __restrict__ smax) {
  const int l = X.l, g = X.g, m = X.m, pr = X.pr, role = X.role;
  const PageMeta pm = page_meta(A.units, A.pt, A.seq_lens, A.b, A.u_max, slot, A.S, A.MP, A.cap,
                                A.num_pages);
  // membership word of this lane's query (loaded unconditionally so that the
  // wait below provably covers it)
  const uint64_t mem = A.member[((size_t)A.b * A.u_max + slot) * A.QB + X.qloc];
  const int lim = min(X.ri.abs_q + 1, pm.kvp) - pm.lp * A.PS;
  uint64_t mk = 0;
  if (X.ri.seq == pm.sp && lim > 0) mk = lim >= 64 ? mem : (mem & ((1ull << lim) - 1));
  if (A.PS < 64) mk &= (1ull << A.PS) - 1;
  // this wave's loads of page `slot` (issued one step earlier) and the
  // metadata above have landed; after the barrier every wave's have, and
  // nobody reads `nxt` (the previous page) any more
  wait_vmcnt<0>();
  lds_barrier();
  if (slot + 1 < A.u_lim) {
    const PageMeta pn = page_meta(A.units, A.pt, A.seq_lens, A.b, A.u_max, slot + 1, A.S, A.MP,
                                  A.cap, A.num_pages);
    stage_page(nxt, A.kv, A.row_stride, pn, A.PS, X.wave, X.l);  // overlaps this page's math
  }
  // both waves of a pair hold the same rows, hence the same masks
  const bool pair_any = __ballot(mk != 0ull) != 0;
  const uint32_t hm = (uint32_t)(mk >> (32 * role));
  f32x16 sacc = {};
  float mx = -INFINITY;
  if (pair_any) {
    // ---- S^T tile: keys 32 role + m (A from LDS), rows m (B = resident q);
    // step i reads chunk 2 i + g of key row 32 role + m
    auto s_off = [&](int i) { return i < 32 ? X.soff[i & 7] + 256 * (i >> 3) : X.soff[8 + (i - 32)]; };
    // operands are read two steps ahead of the MFMA that consumes them
    bf16x8 a0 = as_bf16x8(*reinterpret_cast<const uint4*>(cur + s_off(0)));
    bf16x8 a1 = as_bf16x8(*reinterpret_cast<const uint4*>(cur + s_off(1)));
#pragma unroll
    for (int i = 0; i < DK / 16; ++i) {
      bf16x8 a2 = a1;
      if (i + 2 < DK / 16) a2 = as_bf16x8(*reinterpret_cast<const uint4*>(cur + s_off(i + 2)));
      sacc = mfma32(a0, X.qb[i], sacc);
      a0 = a1;
      a1 = a2;
    }
    // accumulator r of this lane holds key 8 (r / 4) + 4 g + (r % 4) of the half
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * g + (r & 3);
      sacc[r] = ((hm >> key) & 1u) ? sacc[r] * A.sm_scale : -INFINITY;
      mx = fmaxf(mx, sacc[r]);
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    if (g == 0) smax[(pr * 2 + role) * 32 + m] = mx;
  }
  lds_barrier();
  bf16x8 pb[2];
  float alpha = 1.f;
  if (pair_any) {
    mx = fmaxf(mx, smax[(pr * 2 + (role ^ 1)) * 32 + m]);
    if (mx > X.m_used + kLazyMax) {
      alpha = __expf(X.m_used - mx);  // 0 while nothing was accumulated
      X.m_used = mx;
      X.l_part *= alpha;
    }
    uint32_t w[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = sacc[r] != -INFINITY ? __expf(sacc[r] - X.m_used) : 0.f;
      const float p1 = sacc[r + 1] != -INFINITY ? __expf(sacc[r + 1] - X.m_used) : 0.f;
      X.l_part += p0 + p1;
      w[r >> 1] = pack_bf16x2(p0, p1);
    }
    __builtin_memcpy(&pb[0], w, 16);
    __builtin_memcpy(&pb[1], w + 4, 16);
    pf[((pr * 2 + role) * 2 + 0) * 64 + l] = pb[0];
    pf[((pr * 2 + role) * 2 + 1) * 64 + l] = pb[1];
  }
  lds_barrier();
  if (pair_any) {
    if (__ballot(alpha != 1.f && alpha != 0.f) != 0) {
#pragma unroll
      for (int d = 0; d < 8; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) X.o[d][r] *= alpha;
    }
    // ---- O^T += V^T P^T: four 16-key steps (own key half first, its P^T
    // fragments are in registers), value columns 256 role + 32 d + ...
    auto vfrag = [&](int kh, int st, int d) {
      const int dc = (32 * kh + 16 * st) * NOPE_B + 512 * role + 256 * (d >> 2);
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(cur + dc + X.toff[0][d & 3]));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(cur + dc + X.toff[1][d & 3]));
      bf16x8 a;
      __builtin_memcpy(&a, &lo, 8);
      __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
      return a;
    };
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kh = kk ? (role ^ 1) : role;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 pbk = kk ? pf[((pr * 2 + kh) * 2 + st) * 64 + l] : pb[st];
        bf16x8 v0 = vfrag(kh, st, 0);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          bf16x8 v1 = v0;
          if (d + 1 < 8) v1 = vfrag(kh, st, d + 1);
          X.o[d] = mfma32(v0, pbk, X.o[d]);
          v0 = v1;
        }
      }
    }
  }
}

// Per-lane LDS byte offsets, fixed for the whole kernel.
// S^T reads: lane (m, g) of wave `role` reads key row kr = 32 role + m,
// chunk 2 i + g. For i < 32 the slot is (2 i + g) ^ nope_x(kr) = 16 (i >> 3)
// + ((2 (i & 7)) ^ y), y = g ^ nope_x(kr), so 8 per-lane values plus a
// constant; for i >= 32 the rope chunk 2 (i - 32) + g of row kr.
// V^T reads: the lane supplies row key0 = 32 kh + 16 st + 4 g + kq (read 0)
// or key0 + 8 (read 1), 16-byte chunk 32 role + 4 d + c0 and byte boff, with
// kq = (l & 15) >> 2, c0 = 2 ((l >> 4) & 1) + ((l & 3) >> 1), boff =
// 8 (l & 1). Its slot is 32 role + 4 (d ^ z) + (c0 ^ w_e) with z = 2 g +
// (kq >> 1), w_e = 2 (kq & 1) + e, so 4 per-lane values per read plus the
// constants 1024 (32 kh + 16 st), 512 role and 256 (d >> 2).
__device__ __forceinline__ void ext_offsets(ExtLane& X) {
  const int kr = 32 * X.role + X.m;
  const int y = X.g ^ nope_x(kr);
#pragma unroll
  for (int j = 0; j < 8; ++j) X.soff[j] = kr * NOPE_B + 16 * ((2 * j) ^ y);
#pragma unroll
  for (int j = 0; j < 4; ++j) X.soff[8 + j] = ROPE_OFF + kr * ROPE_B + 16 * ((2 * j + X.g) ^ rope_x(kr));
  const int l = X.l;
  const int kq = (l & 15) >> 2, qq = l & 3;
  const int c0 = 2 * ((l >> 4) & 1) + (qq >> 1);
  const int boff = 8 * (qq & 1);
  const int z = 2 * X.g + (kq >> 1);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int key = 4 * X.g + kq + 8 * e;
    const int w = c0 ^ (2 * (kq & 1) + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) X.toff[e][j] = key * NOPE_B + 64 * (j ^ z) + 16 * w + boff;
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_extend_qblock(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int row_stride,
    int num_pages, const int32_t* __restrict__ pt, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ units,
    const int32_t* __restrict__ counts, const uint64_t* __restrict__ member, int T, int S, int H,
    int PS, int MP, int QB, int u_max, float sm_scale, uint16_t* __restrict__ out) {
  // two distinct page buffers, so reads of one provably never alias the
  // loads in flight into the other
  __shared__ __attribute__((aligned(1024))) unsigned char page0[PAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char page1[PAGE_BYTES];
  __shared__ bf16x8 pfrag[2 * 2 * 2 * 64];  // P^T fragments [pair][role][step][lane]
  __shared__ float s_max[2 * 2 * 32];        // row maxima [pair][role][row]
  const int TPB = (QB * H + XROWS - 1) / XROWS;
  const int nqb = (T + QB - 1) / QB;
  // the TPB workgroups of a block get ids of one residue mod 8, i.e. one XCD
  const int L = blockIdx.x;
  const int jj = L >> 3;
  const int b = (jj / TPB) * 8 + (L & 7);
  const int tile = jj % TPB;
  if (b >= nqb) return;

  ExtLane X;
  X.wave = threadIdx.x >> 6;
  X.l = lane_id();
  X.pr = X.wave >> 1;
  X.role = X.wave & 1;
  X.g = X.l >> 5;
  X.m = X.l & 31;
  const int cap = MP * PS;
  const int row = tile * XROWS + X.pr * 32 + X.m;
  const bool row_live = row < QB * H;
  X.qloc = row_live ? row / H : 0;
  ext_offsets(X);
  const int h = row_live ? row % H : 0;
  const int t = b * QB + X.qloc;
  X.ri.seq = -1;
  X.ri.abs_q = -1;
  const bool out_live = row_live && t < T;
  if (out_live) X.ri = row_info(cu, seq_lens, S, t, cap);
  {
    const bool okq = X.ri.seq >= 0;
    const uint16_t* qrow = q + ((size_t)(okq ? t : 0) * H + h) * DK + 8 * X.g;
#pragma unroll
    for (int i = 0; i < DK / 16; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 16 * i);
      X.qb[i] = as_bf16x8(okq ? v : zero_u4());
    }
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) X.o[d] = f32x16{};
  X.m_used = -INFINITY;
  X.l_part = 0.f;

  ExtArgs A;
  A.kv = kv;
  A.pt = pt;
  A.seq_lens = seq_lens;
  A.units = units;
  A.member = member;
  A.row_stride = row_stride;
  A.num_pages = num_pages;
  A.S = S;
  A.PS = PS;
  A.MP = MP;
  A.QB = QB;
  A.u_max = u_max;
  A.cap = cap;
  A.b = b;
  A.u_lim = min(counts[b], u_max);
  A.sm_scale = sm_scale;

  if (A.u_lim > 0) {
    const PageMeta pm0 = page_meta(units, pt, seq_lens, b, u_max, 0, S, MP, cap, num_pages);
    stage_page(page0, kv, row_stride, pm0, PS, X.wave, X.l);
  }
  for (int slot = 0; slot < A.u_lim; ++slot) {
    unsigned char* cur = (slot & 1) ? page1 : page0;
    unsigned char* nxt = (slot & 1) ? page0 : page1;
    ext_step(A, X, slot, cur, nxt, pfrag, s_max);
  }
  // ---- row sums over both key halves, then normalise and store this
  // wave's value columns 256 role + 32 d + 8 (r / 4) + 4 g + (r % 4)
  const float lw = X.l_part + shfl_xor_f(X.l_part, 32);
  __syncthreads();
  if (X.g == 0) s_max[(X.pr * 2 + X.role) * 32 + X.m] = lw;
  __syncthreads();
  const float lt = s_max[(X.pr * 2 + 0) * 32 + X.m] + s_max[(X.pr * 2 + 1) * 32 + X.m];
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (out_live) {
    uint16_t* orow = out + ((size_t)t * H + h) * DV + 256 * X.role;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint2 v;
        v.x = pack_bf16x2(X.o[d][4 * r4] * inv, X.o[d][4 * r4 + 1] * inv);
        v.y = pack_bf16x2(X.o[d][4 * r4 + 2] * inv, X.o[d][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * d + 8 * r4 + 4 * X.g) = v;
      }
  }
}

hipError_t mla_extend(const MlaArgs& a, hipStream_t st) {
  const int nqb = (a.T + a.QB - 1) / a.QB;
  if (nqb == 0) return hipSuccess;
  const int TPB = (a.QB * a.H + XROWS - 1) / XROWS;
  const int nwg = ((nqb + 7) / 8) * 8 * TPB;
  ProfScope prof("mla_extend_qblock", st);
  hipLaunchKernelGGL(mla_extend_qblock, dim3(nwg), dim3(256), 0, st, a.q, a.kv, a.row_stride,
                     a.num_pages, a.pt, a.seq_lens, a.cu, a.units, a.counts, a.member, a.T, a.S,
                     a.H, a.PS, a.MP, a.QB, a.u_max, a.sm_scale, a.out);
  return hipGetLastError();
}

}  // namespace dsa
