// Paged cache self-write of the new tokens, ahead of the attention:
// "dsa_sparse_backend.py", _scatter_paged (indexer keys) and
// "sparse_mla_prefill_qblock.py", paged_write_back (latent rows
// [c_kv | k_rope]). Packed row t of sequence s lands at seq-local position
// a = seq_lens[s] - q_len(s) + (t - q_start): physical page
// page_table[s, a / PS], offset a % PS, columns col0 .. col0 + cols - 1.
// Rows outside every sequence, with a outside [0, min(seq_len, MP * PS)), or
// whose page-table entry is not a page of the cache, are dropped. One launch
// serves up to two caches (the indexer keys and the latent rows of a layer).
#include "common.h"
#include "kernels.h"
#include "profile.h"

namespace dsa {

constexpr int kWriteRowsPerWave = 4;

// One cache written by a launch: row t of src (cols columns) goes to columns
// col0 .. col0 + cols - 1 of its slot.
struct WriteJob {
  const uint16_t* src;
  long src_stride;
  int cols, col0;
  uint16_t* cache;
  long row_stride;
  int num_pages;
};

// grid = (ceil(T / (4 * kWriteRowsPerWave)), number of jobs), block = 256:
// blockIdx.y picks the cache; wave w of block b writes rows
// (4 b + w) * kWriteRowsPerWave + r, lane l copying 16-byte chunks l, l + 64,
// ... (8 bf16 values each) of a row. The owner of each row is found from one
// pass over the sequence bounds per wave. Rows up to 512 columns (one chunk
// per lane) load all of the wave's rows before the first store, from in-bounds
// addresses, so that no load waits for another.
__global__ __launch_bounds__(256) void paged_write_rows(
    WriteJob j0, WriteJob j1, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu, int T, int S, int PS,
    int MP) {
  const WriteJob& j = blockIdx.y == 0 ? j0 : j1;
  const int l = lane_id();
  const int wave = threadIdx.x >> 6;
  const int t0 = (4 * (int)blockIdx.x + wave) * kWriteRowsPerWave;
  if (t0 >= T) return;
  const int cap = MP * PS;
  const int cols = j.cols;
  long slot[kWriteRowsPerWave];
#pragma unroll
  for (int r = 0; r < kWriteRowsPerWave; ++r) slot[r] = -1;
  // owners: sequences in groups of 64 lanes (one load round for S <= 64)
  for (int base = 0; base < S; base += DSA_WAVE) {
    const int i = base + l;
    const bool in = i < S;
    const int q0 = in ? cu[i] : 0, q1 = in ? cu[i + 1] : 0, kv = in ? seq_lens[i] : 0;
#pragma unroll
    for (int r = 0; r < kWriteRowsPerWave; ++r) {
      const int t = t0 + r;
      const uint64_t own = __ballot(in && q0 <= t && t < q1);
      if (own != 0ull) {  // at most one sequence owns a row (cu is non-decreasing)
        const int src_l = (int)__builtin_ctzll(own);
        const int s = base + src_l;
        const int a0 = __shfl(q0, src_l, DSA_WAVE), a1 = __shfl(q1, src_l, DSA_WAVE);
        const int sk = __shfl(kv, src_l, DSA_WAVE);
        const int a = sk - (a1 - a0) + (t - a0);
        const int lim = sk < cap ? sk : cap;
        if (t < T && a >= 0 && a < lim) {
          // an entry that names no page of this cache gives the row no slot
          const int page = pt[(size_t)s * MP + a / PS];
          if (page >= 0 && page < j.num_pages) slot[r] = (long)page * PS + a % PS;
        }
      }
    }
  }
  if (cols <= 8 * DSA_WAVE) {
    const int c = 8 * l < cols ? 8 * l : 0;
    uint4 v[kWriteRowsPerWave];
#pragma unroll
    for (int r = 0; r < kWriteRowsPerWave; ++r) {
      const int t = slot[r] >= 0 ? t0 + r : t0;  // t0 < T is a valid row
      v[r] = *reinterpret_cast<const uint4*>(j.src + (size_t)t * j.src_stride + c);
    }
#pragma unroll
    for (int r = 0; r < kWriteRowsPerWave; ++r)
      if (slot[r] >= 0 && 8 * l < cols)
        *reinterpret_cast<uint4*>(j.cache + (size_t)slot[r] * j.row_stride + j.col0 + c) = v[r];
    return;
  }
#pragma unroll
  for (int r = 0; r < kWriteRowsPerWave; ++r) {
    if (slot[r] < 0) continue;  // wave-uniform
    const uint16_t* srow = j.src + (size_t)(t0 + r) * j.src_stride;
    uint16_t* drow = j.cache + (size_t)slot[r] * j.row_stride + j.col0;
    for (int c = 8 * l; c < cols; c += 8 * DSA_WAVE)
      *reinterpret_cast<uint4*>(drow + c) = *reinterpret_cast<const uint4*>(srow + c);
  }
}

static WriteJob job_of(const CacheWriteJob& c) {
  WriteJob j;
  j.src = c.src;
  j.src_stride = c.src_stride;
  j.cols = c.cols;
  j.col0 = c.col0;
  j.cache = c.cache;
  j.row_stride = c.row_stride;
  j.num_pages = c.num_pages;
  return j;
}

hipError_t paged_write(const CacheWriteArgs& a, hipStream_t st) {
  const int rows_per_block = 4 * kWriteRowsPerWave;
  const int njobs = a.njobs;
  if (a.T == 0 || njobs == 0) return hipSuccess;
  const WriteJob j0 = job_of(a.job[0]);
  const WriteJob j1 = njobs > 1 ? job_of(a.job[1]) : j0;
  ProfScope prof("paged_write_rows", st);
  hipLaunchKernelGGL(paged_write_rows, dim3((a.T + rows_per_block - 1) / rows_per_block, njobs),
                     dim3(256), 0, st, j0, j1, a.pt, a.seq_lens, a.cu, a.T, a.S, a.PS, a.MP);
  return hipGetLastError();
}

}  // namespace dsa
