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

// grid = (nQB, ceil(QB / RPW)), block = 256; LDS bitmap of NW words.
__global__ __launch_bounds__(256) void union_mark(const int32_t* __restrict__ topk,
                                                  const int32_t* __restrict__ seq_lens,
                                                  const int32_t* __restrict__ cu, int T, int S,
                                                  int k, int PS, int MP, int QB, int RPW, int NW,
                                                  uint64_t* __restrict__ bits) {
  extern __shared__ uint64_t lbits[];
  const int b = blockIdx.x;
  const int r0 = blockIdx.y * RPW;
  const int r1 = min(r0 + RPW, QB);
  for (int i = threadIdx.x; i < NW; i += 256) lbits[i] = 0ull;
  __syncthreads();
  const int cap = MP * PS;
  for (int r = r0; r < r1; ++r) {
    const int t = b * QB + r;
    if (t >= T) break;
    const RowInfo ri = row_info(cu, seq_lens, S, t, cap);
    if (ri.seq < 0) continue;
    const int32_t* sel = topk + (size_t)t * k;
    for (int i = threadIdx.x; i < k; i += 256) {
      const int j = sel[i];
      if (j < 0 || j >= cap) continue;
      const int key = ri.seq * MP + j / PS;
      atomicOr(reinterpret_cast<unsigned long long*>(&lbits[key >> 6]), 1ull << (key & 63));
    }
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
__global__ __launch_bounds__(256) void union_member(
    const int32_t* __restrict__ topk, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu, int T, int S, int k, int PS, int MP, int QB, int u_max,
    int QPW, int NW, const uint64_t* __restrict__ bits, const int32_t* __restrict__ prefix,
    const int32_t* __restrict__ counts, uint64_t* __restrict__ member) {
  extern __shared__ uint64_t tile[];
  const int b = blockIdx.x;
  const int q0 = blockIdx.y * QPW;
  const int nq = min(QPW, QB - q0);
  const int u_lim = min(counts[b], u_max);
  for (int i = threadIdx.x; i < u_lim * QPW; i += 256) tile[i] = 0ull;
  __syncthreads();
  const int cap = MP * PS;
  const uint64_t* gb = bits + (size_t)b * NW;
  const int32_t* gp = prefix + (size_t)b * NW;
  for (int qi = 0; qi < nq; ++qi) {
    const int t = b * QB + q0 + qi;
    if (t >= T) break;
    const RowInfo ri = row_info(cu, seq_lens, S, t, cap);
    if (ri.seq < 0) continue;
    const int32_t* sel = topk + (size_t)t * k;
    for (int i = threadIdx.x; i < k; i += 256) {
      const int j = sel[i];
      if (j < 0 || j >= cap) continue;
      const int key = ri.seq * MP + j / PS;
      const int wd = key >> 6, bit = key & 63;
      const uint64_t below = bit ? (gb[wd] & (~0ull >> (64 - bit))) : 0ull;
      const int slot = gp[wd] + __popcll(below);
      if (slot < u_lim)
        atomicOr(reinterpret_cast<unsigned long long*>(&tile[slot * QPW + qi]),
                 1ull << (j % PS));
    }
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
  const int RPW = 16;
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
  const int qpw = union_member_qpw(a.QB, a.u_max);
  ProfScope prof("union_member", st);
  hipLaunchKernelGGL(union_member, dim3(nqb, (a.QB + qpw - 1) / qpw), dim3(256),
                     (size_t)a.u_max * qpw * 8, st, a.topk, a.seq_lens, a.cu, a.T, a.S, a.k,
                     a.PS, a.MP, a.QB, a.u_max, qpw, NW, a.bits, a.prefix, a.counts, a.member);
  return hipGetLastError();
}

}  // namespace dsa
