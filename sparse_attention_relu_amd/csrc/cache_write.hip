// Paged cache self-write of the new tokens, ahead of the attention:
// "dsa_sparse_backend.py", _scatter_paged (indexer keys) and
// "sparse_mla_prefill_qblock.py", paged_write_back (latent rows
// [c_kv | k_rope]). Packed row t of sequence s lands at seq-local position
// a = seq_lens[s] - q_len(s) + (t - q_start): physical page
// page_table[s, a / PS], offset a % PS, columns col0 .. col0 + cols - 1.
// Rows outside every sequence, or with a outside [0, min(seq_len, MP * PS)),
// are dropped.
#include "common.h"
#include "kernels.h"
#include "profile.h"

namespace dsa {

// grid = (T, ceil(cols / 8 / 256)), block = 256: thread i copies the 16-byte
// chunk i (8 bf16 values) of its row.
__global__ __launch_bounds__(256) void paged_write_rows(
    const uint16_t* __restrict__ src, long src_stride, int cols, int col0,
    uint16_t* __restrict__ cache, long row_stride, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu, int S, int PS, int MP,
    int num_pages) {
  const int t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  const int cap = MP * PS;
  const RowInfo ri = row_info_wave(cu, seq_lens, S, t, cap);
  // ri.kv is seq_len clamped to [0, MP * PS]
  if (ri.seq < 0 || ri.abs_q < 0 || ri.abs_q >= ri.kv || c >= cols) return;
  const int a = ri.abs_q;
  const long slot = (long)clamp_page(pt[(size_t)ri.seq * MP + a / PS], num_pages) * PS + a % PS;
  const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)t * src_stride + c);
  *reinterpret_cast<uint4*>(cache + slot * row_stride + col0 + c) = v;
}

hipError_t paged_write(const CacheWriteArgs& a, hipStream_t st) {
  const int chunks = (a.cols / 8 + 255) / 256;
  ProfScope prof("paged_write_rows", st);
  hipLaunchKernelGGL(paged_write_rows, dim3(a.T, chunks), dim3(256), 0, st, a.src,
                     (long)a.src_stride, a.cols, a.col0, a.cache, (long)a.row_stride, a.pt,
                     a.seq_lens, a.cu, a.S, a.PS, a.MP, a.num_pages);
  return hipGetLastError();
}

}  // namespace dsa
