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
#include "common.h"
#include "kernels.h"

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
// selections [c * CH, (c + 1) * CH) in steps of NR, and leaves its partial
// (row max m, sum l, unnormalised O) per head for the combine kernel.
// ---------------------------------------------------------------------------
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
  __shared__ int s_src[NR];
  __shared__ int s_any;

  const int c = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, l = lane_id();
  const int g = l >> 4, col = l & 15;
  const RowInfo ri = row_info(cu, seq_lens, S, t, MP * PS);
  const int i_begin = c * CH, i_end = min(i_begin + CH, k);
  if (tid < NH) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.0f;
  }
  f32x4 acc[HB][8];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[hb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (ri.seq >= 0) {
    const int32_t* sel = topk + (size_t)t * k;
    const int32_t* ptrow = pt + (size_t)ri.seq * MP;
    for (int i0 = i_begin; i0 < i_end; i0 += NR) {
      __syncthreads();
      if (tid == 0) s_any = 0;
      __syncthreads();
      if (tid < NR) {
        const int i = i0 + tid;
        int src = -1;
        if (i < i_end) {
          const int j = sel[i];
          if (j >= 0 && j < ri.kv && j <= ri.abs_q)
            src = clamp_page(ptrow[j / PS], num_pages) * PS + (j % PS);
        }
        s_src[tid] = src;
        if (src >= 0) s_any = 1;
      }
      __syncthreads();
      if (!s_any) continue;
      stage_rows(kvs, kv, row_stride, s_src, 256);
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
        const bool kvalid = s_src[16 * nb + col] >= 0;
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

// grid = (T, H), block = 256: merge the nch partials of (t, h) into bf16.
__global__ __launch_bounds__(256) void mla_decode_combine(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int H, int nch,
                                                          uint16_t* __restrict__ out) {
  extern __shared__ float s_w[];  // nch weights
  __shared__ float s_inv;
  const int t = blockIdx.x, h = blockIdx.y;
  const size_t base = (size_t)t * nch * H;
  if (threadIdx.x == 0) {
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) {
      const float l = part_ml[((base + (size_t)c * H + h) * 2) + 1];
      if (l > 0.f) M = fmaxf(M, part_ml[(base + (size_t)c * H + h) * 2]);
    }
    float L = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float m = part_ml[(base + (size_t)c * H + h) * 2];
      const float l = part_ml[(base + (size_t)c * H + h) * 2 + 1];
      const float wgt = l > 0.f ? __expf(m - M) : 0.f;
      s_w[c] = wgt;
      L += wgt * l;
    }
    s_inv = L > 0.f ? 1.0f / L : 0.f;
  }
  __syncthreads();
  const float inv = s_inv;
  for (int d = threadIdx.x; d < DV; d += 256) {
    float o = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float wgt = s_w[c];
      if (wgt != 0.f) o += wgt * part_o[(base + (size_t)c * H + h) * DV + d];
    }
    out[((size_t)t * H + h) * DV + d] = f32_to_bf16_bits(o * inv);
  }
}

int mla_decode_chunk(int T, int k) {
  const int nsub = (k + NR - 1) / NR;
  long per = ((long)T * nsub) / 1024;
  if (per < 1) per = 1;
  if (per > 8) per = 8;
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
  switch (HB) {
    case 1: DSA_DEC(1); break;
    case 2: DSA_DEC(2); break;
    case 3: DSA_DEC(3); break;
    case 4: DSA_DEC(4); break;
    default: return hipErrorInvalidValue;
  }
#undef DSA_DEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_decode_combine, dim3(a.T, a.H), dim3(256), (size_t)nch * sizeof(float),
                     st, a.part_o, a.part_ml, a.H, nch, a.out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Extend (query block): grid = (nQB, ceil(QB * H / 64)), block = 256.
// A workgroup owns 64 consecutive rows (row = q * H + h) of block b; rows of
// several queries may share a wave when H < 16. Wave w computes logits and
// the online softmax for rows 16 w .. 16 w + 15 (query fragments resident in
// registers), and P.V for value columns 128 w .. 128 w + 127 of all 64 rows.
// Union pages are walked in ascending key order, 32 positions at a time;
// each row carries its own 64-bit validity mask per page (membership AND
// causal AND kv_len), and a step no row of the workgroup selected is skipped
// without fetching.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_extend_qblock(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int row_stride,
    int num_pages, const int32_t* __restrict__ pt, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ units,
    const int32_t* __restrict__ counts, const uint64_t* __restrict__ member, int T, int S, int H,
    int PS, int MP, int QB, int u_max, float sm_scale, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t kvs[NR * KRS];
  __shared__ __attribute__((aligned(16))) uint16_t ps[64 * PRS];
  __shared__ float s_alpha[64], s_l[64];
  __shared__ uint64_t s_mask[64];
  __shared__ int s_rt[64], s_rseq[64], s_rabs[64], s_rq[64];
  __shared__ uint32_t s_any[2], s_mbany[4];
  __shared__ int s_src[NR];

  const int b = blockIdx.x;
  const int r0 = blockIdx.y * 64;
  const int tid = threadIdx.x, wave = tid >> 6, l = lane_id();
  const int g = l >> 4, col = l & 15;
  const int cap = MP * PS;
  const int rows_total = QB * H;

  if (tid < 64) {  // per-row bookkeeping
    const int r = r0 + tid;
    const int qloc = r / H;
    const int t = b * QB + qloc;
    RowInfo ri;
    ri.seq = -1;
    ri.abs_q = -1;
    const bool live = r < rows_total && t < T;
    if (live) ri = row_info(cu, seq_lens, S, t, cap);
    s_rt[tid] = live ? t : -1;
    s_rseq[tid] = ri.seq;
    s_rabs[tid] = ri.abs_q;
    s_rq[tid] = qloc < QB ? qloc : 0;
  }
  __syncthreads();

  bf16x8 qa[DK / 32];
  {
    const int row = 16 * wave + col;
    const int tq = s_rseq[row] >= 0 ? s_rt[row] : -1;
    const int h = (r0 + row) % H;
    const uint16_t* qrow = q + ((size_t)(tq >= 0 ? tq : 0) * H + h) * DK + 8 * g;
#pragma unroll
    for (int i = 0; i < DK / 32; ++i)
      qa[i] = as_bf16x8(tq >= 0 ? *reinterpret_cast<const uint4*>(qrow + 32 * i) : zero_u4());
  }
  float m_run[4], l_run[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
  f32x4 acc[4][8];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int u_lim = min(counts[b], u_max);
  const int halves = (PS + NR - 1) / NR;
  for (int slot = 0; slot < u_lim; ++slot) {
    int key = units[(size_t)b * u_max + slot];
    key = key < 0 ? 0 : (key >= S * MP ? S * MP - 1 : key);
    const int sp = key / MP, lp = key % MP;
    int kvp = seq_lens[sp];
    kvp = kvp < 0 ? 0 : (kvp > cap ? cap : kvp);
    const int page = clamp_page(pt[key], num_pages);
    __syncthreads();  // every reader of the previous slot's LDS state is done
    if (tid < 64) {
      uint64_t mk = 0;
      if (s_rseq[tid] == sp) {
        const uint64_t mem = member[((size_t)b * u_max + slot) * QB + s_rq[tid]];
        const int lim = min(s_rabs[tid] + 1, kvp) - lp * PS;  // valid offsets [0, lim)
        if (lim > 0) mk = lim >= 64 ? mem : (mem & ((1ull << lim) - 1));
        if (PS < 64) mk &= (1ull << PS) - 1;
      }
      s_mask[tid] = mk;
      const uint64_t any0 = __ballot((uint32_t)mk != 0u);
      const uint64_t any1 = __ballot((uint32_t)(mk >> 32) != 0u);
      if (tid == 0) {
        s_any[0] = any0 != 0;
        s_any[1] = any1 != 0;
      }
    }
    __syncthreads();
    for (int hv = 0; hv < halves; ++hv) {
      if (!s_any[hv]) continue;
      if (tid < NR) {
        const int off = NR * hv + tid;
        const int pos = lp * PS + off;
        s_src[tid] = (off < PS && pos < kvp) ? page * PS + off : -1;
      }
      __syncthreads();  // also: the previous half's P.V readers are done
      stage_rows(kvs, kv, row_stride, s_src, 256);
      uint32_t hm[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) hm[r] = (uint32_t)(s_mask[16 * wave + 4 * g + r] >> (NR * hv));
      const bool wave_any = __ballot((hm[0] | hm[1] | hm[2] | hm[3]) != 0u) != 0;
      if (l == 0) s_mbany[wave] = wave_any;
      __syncthreads();
      if (wave_any) {
        f32x4 sacc[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          sacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < DK / 32; ++i) {
            const bf16x8 bk = as_bf16x8(*reinterpret_cast<const uint4*>(&kvs[(16 * nb + col) * KRS + 32 * i + 8 * g]));
            sacc[nb] = mfma16(qa[i], bk, sacc[nb]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x0 = ((hm[r] >> col) & 1u) ? sacc[0][r] * sm_scale : -INFINITY;
          const float x1 = ((hm[r] >> (16 + col)) & 1u) ? sacc[1][r] * sm_scale : -INFINITY;
          float mx = fmaxf(x0, x1);
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
          const float m_new = fmaxf(m_run[r], mx);
          float p0 = 0.f, p1 = 0.f, alpha = 1.f;
          if (m_new != -INFINITY) {
            p0 = __expf(x0 - m_new);
            p1 = __expf(x1 - m_new);
            alpha = __expf(m_run[r] - m_new);
          }
          float sum = p0 + p1;
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) sum += shfl_xor_f(sum, o);
          m_run[r] = m_new;
          l_run[r] = l_run[r] * alpha + sum;
          const int prow = 16 * wave + 4 * g + r;
          ps[prow * PRS + col] = f32_to_bf16_bits(p0);
          ps[prow * PRS + 16 + col] = f32_to_bf16_bits(p1);
          if (col == 0) s_alpha[prow] = alpha;
        }
      }
      __syncthreads();
      // P.V: value columns 128 * wave .. + 127, all row blocks with work
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const bf16x8 bv = load_v_col(kvs, 8 * g, 128 * wave + 16 * nb + col);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if (!s_mbany[mb]) continue;
          const bf16x8 ap = as_bf16x8(*reinterpret_cast<const uint4*>(&ps[(16 * mb + col) * PRS + 8 * g]));
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mb][nb][r] *= s_alpha[16 * mb + 4 * g + r];
          acc[mb][nb] = mfma16(ap, bv, acc[mb][nb]);
        }
      }
    }
  }
  __syncthreads();
  if (col == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s_l[16 * wave + 4 * g + r] = l_run[r];
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * mb + 4 * g + r;
      const int tq = s_rt[row];
      if (tq < 0) continue;
      const int h = (r0 + row) % H;
      const float lsum = s_l[row];
      const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
      uint16_t* orow = out + ((size_t)tq * H + h) * DV + 128 * wave + col;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) orow[16 * nb] = f32_to_bf16_bits(acc[mb][nb][r] * inv);
    }
  }
}

hipError_t mla_extend(const MlaArgs& a, hipStream_t st) {
  const int nqb = (a.T + a.QB - 1) / a.QB;
  if (nqb == 0) return hipSuccess;
  dim3 grid(nqb, (a.QB * a.H + 63) / 64);
  hipLaunchKernelGGL(mla_extend_qblock, grid, dim3(256), 0, st, a.q, a.kv, a.row_stride,
                     a.num_pages, a.pt, a.seq_lens, a.cu, a.units, a.counts, a.member, a.T, a.S,
                     a.H, a.PS, a.MP, a.QB, a.u_max, a.sm_scale, a.out);
  return hipGetLastError();
}

}  // namespace dsa
