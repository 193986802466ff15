// Query-block union of selected pages and per-token membership (gfx950).
//
// sglang-jax "sparse_mla_prefill_qblock.py", build_block_unit_tables: per
// block of QB packed rows, the ascending list of distinct page keys
// (s * MP + j / PS), its true size, and per (slot, query) membership. The
// page's TPU version sorts the flattened selections and compacts by rank;
// here the key space of one block is small (S * MP), so the union is a
// presence bitmap: mark bits (LDS, then OR into a per-block global bitmap),
// compact by a popcount prefix over the bitmap words, and look a key's slot
// up as prefix[word] + popcount(word & below(bit)). Membership words are
// built in LDS per group of queries and written slot-major.
#include "common.h"
#include "kernels.h"
#include "profile.h"

namespace dsa {

__global__ void union_clear(uint64_t* __restrict__ bits, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    bits[i] = 0ull;
}

// grid = (nQB, ceil(QB / RPW)), block = 256; LDS bitmap of NW words. The
// sequences of the workgroup's rows are looked up in parallel first; then
// one flat loop over (row, selection) pairs keeps many loads in flight.
constexpr int kUnionRowsMax = 1024;  // rows of one workgroup (QB <= 1024)
constexpr int kUnionWordsLds = 512;  // bitmap words staged in LDS by union_member

__global__ __launch_bounds__(256) void union_mark(const int32_t* __restrict__ topk,
                                                  const int32_t* __restrict__ seq_lens,
                                                  const int32_t* __restrict__ cu, int T, int S,
                                                  int k, int PS, int MP, int QB, int RPW, int NW,
                                                  uint64_t* __restrict__ bits) {
  extern __shared__ uint64_t lbits[];
  __shared__ int s_seq[kUnionRowsMax];
  const int b = blockIdx.x;
  const int r0 = blockIdx.y * RPW;
  const int nr = max(0, min(min(r0 + RPW, QB), T - b * QB) - r0);  // live rows
  const int cap = MP * PS;
  for (int i = threadIdx.x; i < NW; i += 256) lbits[i] = 0ull;
  for (int r = threadIdx.x; r < nr; r += 256)
    s_seq[r] = row_info(cu, seq_lens, S, b * QB + r0 + r, cap).seq;
  __syncthreads();
  const int32_t* sel = topk + ((size_t)b * QB + r0) * k;
  auto mark = [&](int idx, int j) {
    const int seq = s_seq[idx / k];
    if (seq < 0 || j < 0 || j >= cap) return;
    const int key = seq * MP + j / PS;
    atomicOr(reinterpret_cast<unsigned long long*>(&lbits[key >> 6]), 1ull << (key & 63));
  };
  const int n = nr * k;
  if ((k & 3) == 0 && ((uintptr_t)topk & 15) == 0) {  // 16-byte loads, issued first
    constexpr int U = 4;
    for (int i0 = 4 * threadIdx.x; i0 < n; i0 += 4 * 256 * U) {
      int4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + 4 * 256 * u;
        v[u] = i < n ? *reinterpret_cast<const int4*>(sel + i) : make_int4(-1, -1, -1, -1);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + 4 * 256 * u;
        mark(i, v[u].x);
        mark(i + 1, v[u].y);
        mark(i + 2, v[u].z);
        mark(i + 3, v[u].w);
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < n; idx += 256) mark(idx, sel[idx]);
  }
  __syncthreads();
  uint64_t* gb = bits + (size_t)b * NW;
  for (int i = threadIdx.x; i < NW; i += 256) {
    const uint64_t v = lbits[i];
    if (v) atomicOr(reinterpret_cast<unsigned long long*>(&gb[i]), (unsigned long long)v);
  }
}

// grid = nQB, block = 256. Each thread owns a contiguous run of words.
__global__ __launch_bounds__(256) void union_compact(const uint64_t* __restrict__ bits, int NW,
                                                     int u_max, int32_t* __restrict__ prefix,
                                                     int32_t* __restrict__ units,
                                                     int32_t* __restrict__ counts) {
  __shared__ int s_scan[4];
  const int b = blockIdx.x;
  const uint64_t* gb = bits + (size_t)b * NW;
  const int per = (NW + 255) / 256;
  const int w0 = threadIdx.x * per;
  const int w1 = min(w0 + per, NW);
  int local = 0;
  for (int i = w0; i < w1; ++i) local += __popcll(gb[i]);
  int total;
  const int incl = block_inclusive_scan<256>(local, s_scan, &total);
  int rank = incl - local;
  int32_t* ub = units + (size_t)b * u_max;
  for (int i = w0; i < w1; ++i) {
    uint64_t v = gb[i];
    prefix[(size_t)b * NW + i] = rank;
    while (v) {
      const int bit = __ffsll((unsigned long long)v) - 1;
      v &= v - 1;
      if (rank < u_max) ub[rank] = i * 64 + bit;
      ++rank;
    }
  }
  for (int i = total + threadIdx.x; i < u_max; i += 256) ub[i] = -1;
  if (threadIdx.x == 0) counts[b] = total;
}

// grid = (nQB, ceil(QB / QPW)), block = 256; LDS tile [u_max][QPW] uint64.
// As in union_mark, the rows' sequences are looked up in parallel and one
// flat loop covers every (query, selection) pair.
__global__ __launch_bounds__(256) void union_member(
    const int32_t* __restrict__ topk, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu, int T, int S, int k, int PS, int MP, int QB, int u_max,
    int QPW, int NW, const uint64_t* __restrict__ bits, const int32_t* __restrict__ prefix,
    const int32_t* __restrict__ counts, uint64_t* __restrict__ member) {
  extern __shared__ uint64_t tile[];
  __shared__ int s_seq[kUnionRowsMax];
  __shared__ uint64_t s_bits[kUnionWordsLds];
  __shared__ int32_t s_pre[kUnionWordsLds];
  const int b = blockIdx.x;
  const int q0 = blockIdx.y * QPW;
  const int nq = min(QPW, QB - q0);
  const int nlive = max(0, min(nq, T - b * QB - q0));  // queries that are rows of the batch
  const int u_lim = min(counts[b], u_max);
  const int cap = MP * PS;
  for (int i = threadIdx.x; i < u_lim * QPW; i += 256) tile[i] = 0ull;
  for (int qi = threadIdx.x; qi < nlive; qi += 256)
    s_seq[qi] = row_info(cu, seq_lens, S, b * QB + q0 + qi, cap).seq;
  __syncthreads();
  // the block's bitmap words and their rank prefixes, from LDS when they fit
  const bool in_lds = NW <= kUnionWordsLds;
  if (in_lds)
    for (int i = threadIdx.x; i < NW; i += 256) {
      s_bits[i] = bits[(size_t)b * NW + i];
      s_pre[i] = prefix[(size_t)b * NW + i];
    }
  __syncthreads();
  const uint64_t* gb = in_lds ? s_bits : bits + (size_t)b * NW;
  const int32_t* gp = in_lds ? s_pre : prefix + (size_t)b * NW;
  const int32_t* sel = topk + ((size_t)b * QB + q0) * k;
  auto add = [&](int idx, int j) {
    const int qi = idx / k;
    const int seq = s_seq[qi];
    if (seq < 0 || j < 0 || j >= cap) return;
    const int key = seq * MP + j / PS;
    const int wd = key >> 6, bit = key & 63;
    const uint64_t below = bit ? (gb[wd] & (~0ull >> (64 - bit))) : 0ull;
    const int slot = gp[wd] + __popcll(below);
    if (slot < u_lim)
      atomicOr(reinterpret_cast<unsigned long long*>(&tile[slot * QPW + qi]), 1ull << (j % PS));
  };
  const int n = nlive * k;
  if ((k & 3) == 0 && ((uintptr_t)topk & 15) == 0) {  // 16-byte loads, issued first
    constexpr int U = 4;
    for (int i0 = 4 * threadIdx.x; i0 < n; i0 += 4 * 256 * U) {
      int4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + 4 * 256 * u;
        v[u] = i < n ? *reinterpret_cast<const int4*>(sel + i) : make_int4(-1, -1, -1, -1);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + 4 * 256 * u;
        add(i, v[u].x);
        add(i + 1, v[u].y);
        add(i + 2, v[u].z);
        add(i + 3, v[u].w);
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < n; idx += 256) add(idx, sel[idx]);
  }
  __syncthreads();
  uint64_t* mb = member + (size_t)b * u_max * QB;
  for (int i = threadIdx.x; i < u_max * QPW; i += 256) {
    const int slot = i / QPW, qi = i % QPW;
    if (qi >= nq) continue;
    mb[(size_t)slot * QB + q0 + qi] = slot < u_lim ? tile[i] : 0ull;
  }
}

int union_words(int S, int MP) { return (S * MP + 63) / 64; }

int union_member_qpw(int QB, int u_max) {
  int qpw = 1;
  while (qpw * 2 <= QB && (size_t)u_max * qpw * 2 * 8 <= kUnionTileBytes) qpw *= 2;
  return qpw;
}

hipError_t block_union(const UnionArgs& a, hipStream_t st) {
  const int NW = union_words(a.S, a.MP);
  const int nqb = (a.T + a.QB - 1) / a.QB;
  if (nqb == 0) return hipSuccess;
  const long nbits = (long)nqb * NW;
  long nblk = (nbits + 255) / 256;
  if (nblk > 4096) nblk = 4096;
  {
    ProfScope prof("union_clear", st);
    hipLaunchKernelGGL(union_clear, dim3((unsigned)nblk), dim3(256), 0, st, a.bits, nbits);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int RPW = 4;
  {
    ProfScope prof("union_mark", st);
    hipLaunchKernelGGL(union_mark, dim3(nqb, (a.QB + RPW - 1) / RPW), dim3(256),
                       (size_t)NW * 8, st, a.topk, a.seq_lens, a.cu, a.T, a.S, a.k, a.PS, a.MP,
                       a.QB, RPW, NW, a.bits);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    ProfScope prof("union_compact", st);
    hipLaunchKernelGGL(union_compact, dim3(nqb), dim3(256), 0, st, a.bits, NW, a.u_max, a.prefix,
                       a.units, a.counts);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!a.member) return hipSuccess;  // sizes only, for planning
  const int qpw = union_member_qpw(a.QB, a.u_max);
  ProfScope prof("union_member", st);
  hipLaunchKernelGGL(union_member, dim3(nqb, (a.QB + qpw - 1) / qpw), dim3(256),
                     (size_t)a.u_max * qpw * 8, st, a.topk, a.seq_lens, a.cu, a.T, a.S, a.k,
                     a.PS, a.MP, a.QB, a.u_max, qpw, NW, a.bits, a.prefix, a.counts, a.member);
  return hipGetLastError();
}

}  // namespace dsa
