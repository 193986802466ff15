// Sparse absorbed-MLA attention for gfx950: decode (per-row selection lists)
// and query-block extend (shared page union + per-token membership).
//
// Semantics: sglang-jax "ref.py", sparse_mla_ref — logits over the packed
// 576-wide latent row [c_kv 512 | k_rope 64] times sm_scale, softmax over the
// valid selected positions, value = the row's first 512 columns. The extend
// kernel follows "sparse_mla_prefill_qblock.py", _qblock_kernel: one fetch per
// union page for all QB * H rows of a block, per-row validity = membership
// bit AND causal AND kv_len, flash-style online softmax.
#include <atomic>
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "profile.h"

namespace dsa {

// ---------------------------------------------------------------------------
// Staged latent rows. A staged row keeps its 512 "nope" columns (1024 bytes)
// and its 64 rope columns (128 bytes) in two separate regions, so that 16-byte
// chunk c of a row sits at a power-of-two stride and can be XOR-swizzled:
// nope row r keeps chunk c (0..63) at slot c ^ nope_x(r), with
// nope_x(r) = 4 (r & 3) + 2 ((r >> 2) & 1) + ((r >> 3) & 1). Slot s of any row
// lies in bank group s mod 16 (16 groups of four 4-byte banks), so:
//   - 16 consecutive rows (from a multiple of 16) read at one chunk hit all
//     16 groups (nope_x is a bijection there);
//   - 4 consecutive rows (from a multiple of 4) x 4 aligned chunks, the half
//     wave of an extend transposed read, hit all 16 (bits 2..3 of nope_x
//     differ between the 4 rows, and the chunks fill bits 0..1);
//   - 8 consecutive rows (from a multiple of 8) x 2 aligned chunks, the half
//     wave of a decode transposed read, hit all 16 (nope_x >> 1 differs).
// Rope row r keeps chunk c (0..7) at c ^ ((r >> 1) & 7). Rows are filled by direct global->LDS 16-byte
// loads (global_load_lds_dwordx4): one wave instruction writes 1024
// consecutive LDS bytes, 16 per lane, so a lane simply fetches the chunk that
// belongs at its slot.
// ---------------------------------------------------------------------------
constexpr int DK = 576;
constexpr int DV = 512;
constexpr int NOPE_B = 1024;  // staged bytes per row, columns 0..511
constexpr int ROPE_B = 128;   // staged bytes per row, columns 512..575

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int nope_x(int r) {
  return ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
}
__device__ __forceinline__ int rope_x(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] and
// [15:14], expcnt[6:4] and lgkmcnt[11:8] left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that publishes this wave's LDS writes but, unlike
// __syncthreads(), does not wait for outstanding global->LDS loads (their
// completion is awaited explicitly with wait_vmcnt where it matters).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// Lane id from a volatile instruction, which keeps cheap address arithmetic
// next to its use instead of live across a loop.
__device__ __forceinline__ int lane_id_volatile() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// One direct 16-byte global->LDS load per lane (global_load_lds_dwordx4):
// lane l writes LDS bytes lds_addr + 16 l .. + 15 (lds_addr wave-uniform).
// Issued as inline assembly so that the compiler does not make later LDS
// reads wait for it; completion is awaited explicitly. This form takes a
// wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset (the
// "saddr" form), so a lane's address costs one 32-bit VALU operation.
__device__ __forceinline__ void gll16_s(uint32_t voff, const void* sbase, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}

// The same load with a full 64-bit per-lane source address and a
// wave-uniform LDS byte address.
__device__ __forceinline__ void gll16_a(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_addr)
               : "memory", "m0");
}

// max of two floats as one v_max_f32 (the operands are results of
// arithmetic or of lane permutations of such results, so no quieting of
// signalling NaNs is needed before the compare)
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// ---------------------------------------------------------------------------
// Decode: grid = (nch * HB, T), block = 256, two workgroups per compute unit.
// Workgroup (c, hb, t) attends row t over selections [c * CH, (c + 1) * CH)
// for heads 16 hb .. 16 hb + 15. With several chunks per row it leaves its
// partial (max m, sum l, unnormalised O) per head for the combine kernel;
// with one (CH = k, large batches) it writes the normalised output itself
// and no combine runs. The source slot of every selection is resolved first;
// stages of 32 selected rows then stream through a two-stage LDS ring (the
// next stage in flight while one is used): the 512 nope columns of a row by
// direct loads, staged like an extend page, and the 64 rope columns into the
// registers of the odd waves, whose half of the contraction ends with the
// two rope steps (so the ring holds only nope columns and the source table
// fits 2048 entries). Two resident workgroups per compute unit keep two
// stages in flight per compute unit and overlap one workgroup's arithmetic
// and barriers with the other's loads (one workgroup with a four-stage ring
// ran the long-context per-query attend at 3.0 ms, two with two stages at
// 2.0 ms: rows that neighbouring queries share then come from L2).
// S^T = K . Q^T of a stage is two 16-key tiles for the 16 heads
// (v_mfma_f32_16x16x32_bf16: M = keys, N = heads); waves 2 i and 2 i + 1
// compute tile i over one half each of the contraction over the 576 latent
// columns (k steps 0..8 and 9..17 of 32 columns), so each staged key is read
// from LDS once, and the four half tiles meet through LDS, summed in the same
// order by every wave. A lane then holds keys 4 g .. 4 g + 3 of both tiles for
// head `col`, which is exactly its P^T operand for one 32-key step, and its
// O^T accumulators belong to the same head, so every wave runs the same
// online softmax on its own: wave w computes O^T += V^T . P^T for value
// columns 128 w .. 128 w + 127, reading V^T with transposed LDS reads in the
// same key order. Logits are kept in log2 units. Invalid selections load a
// valid row of the same stage and are masked to probability 0; stages without
// any valid selection load cache row 0 and skip the arithmetic.
// ---------------------------------------------------------------------------
constexpr int kDecWPC = 2;                                    // workgroups per compute unit
constexpr int kDecRows = 32;                                  // selections per stage
constexpr int kDecRing = 2;                                   // LDS stages
constexpr int kDecStage = kDecRows * NOPE_B;                  // 32768 bytes (nope columns)
constexpr int kDecMaxCH = 2048;
constexpr float kDecLazy = 8.0f;  // headroom of the running maximum (log2 units)
// s_src entries: the cache slot a selection loads; an invalid selection
// carries this bit over the slot of a valid row of its stage (or slot 0)
constexpr int kDecInvalid = (int)0x80000000;

// This wave's direct loads of one stage: nope rows r = 4 n + wave (n < 8) at
// LDS bytes [1024 r, 1024 r + 1024). `ent` holds in lane n the stage's
// source entry of row 4 n + wave (read from the source table beforehand, so
// that the eight rows cost one LDS round trip, not eight). (The rope columns
// of a stage go to the registers of the waves whose part of the contraction
// holds them.)
// roff[n] is the lane's swizzled byte offset within row 4 n + wave.
__device__ __forceinline__ void stage_rows(uint32_t buf, const uint16_t* __restrict__ kv,
                                           int row_stride, int ent, int wave,
                                           const uint32_t (&roff)[kDecRows / 4]) {
#pragma unroll
  for (int n = 0; n < kDecRows / 4; ++n) {
    const int r = 4 * n + wave;
    const int src = __builtin_amdgcn_readlane(ent, n) & ~kDecInvalid;
    gll16_s(roff[n], kv + (size_t)src * row_stride, buf + r * NOPE_B);
  }
}

// PAGED = 1: the selection of a row is a list of sel_ld seq-local pages, and
// entry i of the row (k = sel_ld * PS entries) is position
// page[i / PS] * PS + i % PS, or none for a -1 page.
template <int PAGED>
__global__ __launch_bounds__(256, kDecWPC) void mla_decode_partial(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int row_stride,
    int num_pages, const int32_t* __restrict__ pt, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ topk, int sel_ld, int T, int S,
    int H, int k, int PS, int MP, float sm_scale, int CH, int nch, int HB,
    uint16_t* __restrict__ part_o, float* __restrict__ part_ml, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kDecRing][kDecStage];
  __shared__ int s_src[kDecMaxCH];
  __shared__ f32x4 s_part[4][64];  // per wave: its half of one S^T tile

  const int c = blockIdx.x / HB, hb = blockIdx.x - c * HB, t = blockIdx.y;
  const int tid = threadIdx.x, l = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = l >> 4, col = l & 15;
  const int i_begin = c * CH, i_end = min(i_begin + CH, k);
  const float scale2 = sm_scale * 1.44269504088896341f;

  // ---- this wave's S^T tile (keys 16 tile .. 16 tile + 15 of a stage) and
  // its half of the 18 k steps of 32 latent columns; the odd waves' half
  // ends with the two rope steps, whose key fragments they load to registers
  const int tile = wave >> 1;
  const int kb = 9 * (wave & 1);
  const bool rope_wave = (wave & 1) != 0;
  // ---- the selection entries of this chunk (entry i = 64 (4 p + wave) + l
  // of pass p, two stages per wave and pass) and this lane's query fragments
  // (head 16 hb + col, k values 32 (kb + u) + 8 g ..) depend only on the row
  // index, so they are loaded together with the row's sequence bounds
  constexpr int NP = kDecMaxCH / 256;
  int j[NP];
  {
    const int32_t* sel = topk + (size_t)t * sel_ld;
#pragma unroll
    for (int p2 = 0; p2 < NP; ++p2) {
      const int ii = i_begin + 256 * p2 + 64 * wave + l;
      if (PAGED) {
        const int pi = ii / PS;
        const int pg = ii < i_end ? sel[pi] : -1;
        j[p2] = pg >= 0 ? pg * PS + (ii - pi * PS) : -1;
      } else {
        j[p2] = ii < i_end ? sel[ii] : -1;
      }
    }
  }
  const int head = 16 * hb + col;
  bf16x8 qf[9];
  {
    const uint16_t* qrow = q + ((size_t)t * H + (head < H ? head : 0)) * DK + 8 * g;
#pragma unroll
    for (int u = 0; u < 9; ++u)
      qf[u] = as_bf16x8(head < H ? *reinterpret_cast<const uint4*>(qrow + 32 * (kb + u))
                                 : zero_u4());
  }
  const RowInfo ri = row_info_wave(cu, seq_lens, S, t, MP * PS);
  const int nst = ri.seq >= 0 ? (i_end - i_begin + kDecRows - 1) / kDecRows : 0;
  // ---- resolve sources and per-stage validity masks
  if (nst > 0) {
    const int32_t* ptrow = pt + (size_t)ri.seq * MP;
    int src[NP];
#pragma unroll
    for (int p2 = 0; p2 < NP; ++p2) {
      const int jj = j[p2];
      const bool ok = jj >= 0 && jj < ri.kv && jj <= ri.abs_q;
      src[p2] = ok ? clamp_page(ptrow[jj / PS], num_pages) * PS + (jj % PS) : -1;
    }
#pragma unroll
    for (int p2 = 0; p2 < NP; ++p2) {
      const int i = 256 * p2 + 64 * wave + l;
      if (i - l >= nst * kDecRows) break;  // wave-uniform
      const uint64_t m = __ballot(src[p2] >= 0);
      const uint32_t mh = (uint32_t)(l < 32 ? m : m >> 32);  // this lane's stage
      const int first = mh ? (int)__builtin_ctz(mh) + (l & 32) : l;
      const int fsrc = __shfl(src[p2], first, DSA_WAVE);
      // a stage without any valid selection still stages cache row 0 (read,
      // never used), so that every stage issues the same loads
      s_src[i] = src[p2] >= 0 ? src[p2] : ((mh ? fsrc : 0) | kDecInvalid);
    }
  }
  // complete the query loads here: a first use inside the stage loop would
  // make the compiler wait for every outstanding load there, ring loads included
#pragma unroll
  for (int u = 0; u < 9; ++u) asm volatile("" : : "v"(qf[u]));
  __syncthreads();

  // per-lane LDS offsets. S^T reads: key row 16 tile + col, chunk 4 i + g of
  // k step i (nope_x of row 16 + col equals that of col), for the nope steps
  // i < 16; the rope steps 16 and 17 read rope chunks g and 4 + g of the row
  // from registers.
  const int nx = nope_x(col);
  const int kr = 16 * tile + col;
  int koff[7];
#pragma unroll
  for (int u = 0; u < 7; ++u) koff[u] = kr * NOPE_B + 16 * ((4 * (kb + u) + g) ^ nx);
  // rope fragments of stage st (kernel-visible loads, waited for with the
  // ring): this lane's two 16-byte chunks of key row kr
  auto rope_load = [&](int ent, bf16x8 (&rp)[2]) __attribute__((always_inline)) {
    const uint16_t* r = kv + (size_t)(ent & ~kDecInvalid) * row_stride + DV + 8 * g;
    rp[0] = as_bf16x8(*reinterpret_cast<const uint4*>(r));
    rp[1] = as_bf16x8(*reinterpret_cast<const uint4*>(r + 32));
  };
  // source entries of stage st: lane n < 8 of stage_rows' operand holds row
  // 4 n + wave, the rope operand row kr, the mask operand row l % 32
  auto ent_rows = [&](int st) { return s_src[st * kDecRows + 4 * (l & 7) + wave]; };
  auto ent_rope = [&](int st) { return s_src[st * kDecRows + kr]; };
  auto ent_mask = [&](int st) { return s_src[st * kDecRows + (l & 31)]; };
  // V^T reads: key row 4 g + col / 4 (+16), columns 128 wave + 16 ct + 4 (col & 3),
  // i.e. 16-byte chunk 16 wave + 2 ct + (col & 3) / 2, byte 8 (col & 1)
  const int vr = 4 * g + (col >> 2), vq = col & 3;
  const int vx = nope_x(vr);
  int voff[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
    voff[ct] = vr * NOPE_B + 256 * wave + 16 * ((2 * ct + (vq >> 1)) ^ vx) + 8 * (vq & 1);

  f32x4 o[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const uint32_t lds_ring = lds_addr_of(ring[0]);

  // rope fragments: two register sets, used alternately by even and odd
  // stages (the loop body is instantiated once per ring slot, so that slot
  // offsets fold into the LDS instructions and no register copies are made)
  bf16x8 rope_a[2], rope_b[2];
  rope_a[0] = rope_a[1] = rope_b[0] = rope_b[1] = as_bf16x8(zero_u4());
  static_assert(kDecRing == 2, "the stage loop issues one stage ahead");
  uint32_t roff[kDecRows / 4];
#pragma unroll
  for (int n = 0; n < kDecRows / 4; ++n) roff[n] = 16u * (uint32_t)(l ^ nope_x(4 * n + wave));
  auto run_stage = [&](const int st, const int slot, bf16x8 (&rope_cur)[2],
                       bf16x8 (&rope_next)[2]) __attribute__((always_inline)) {
    // the entries of the stage issued below and this stage's mask, read
    // before the barrier, whose LDS wait covers them
    const bool ahead = st + 1 < nst;
    const int e_rows = ahead ? ent_rows(st + 1) : 0;
    const int e_rope = ahead ? ent_rope(st + 1) : 0;
    const int e_mask = ent_mask(st);
    wait_vmcnt<0>();
    lds_barrier();  // stage st has landed for every wave; stage st - 1 is consumed
    if (ahead) {
      stage_rows(lds_ring + (1 - slot) * kDecStage, kv, row_stride, e_rows, wave, roff);
      if (rope_wave) rope_load(e_rope, rope_next);
    }
    // the stage's validity mask: bit r for selection r of the stage
    const uint32_t mask = (uint32_t)__ballot(e_mask >= 0);
    if (mask == 0) return;
    const unsigned char* buf = ring[slot];
    // ---- this wave's half of its S^T tile (16 keys), then both tiles summed
    // in the same order by every wave
    f32x4 sp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 7; ++u)
      sp = mfma16(as_bf16x8(*reinterpret_cast<const uint4*>(buf + koff[u])), qf[u], sp);
    if (rope_wave) {
      sp = mfma16(rope_cur[0], qf[7], sp);
      sp = mfma16(rope_cur[1], qf[8], sp);
    } else {
#pragma unroll
      for (int u = 7; u < 9; ++u)
        sp = mfma16(as_bf16x8(*reinterpret_cast<const uint4*>(buf + kr * NOPE_B +
                                                              16 * ((4 * (kb + u) + g) ^ nx))),
                    qf[u], sp);
    }
    s_part[wave][l] = sp;
    lds_barrier();
    f32x4 s0 = s_part[0][l] + s_part[1][l];
    f32x4 s1 = s_part[2][l] + s_part[3][l];
    // ---- masked online softmax over the stage's 32 keys (log2 units)
    if (mask != 0xffffffffu) {  // wave-uniform: only stages with invalid entries
      const uint32_t m0 = mask >> (4 * g), m1 = mask >> (16 + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!((m0 >> r) & 1u)) s0[r] = -INFINITY;
        if (!((m1 >> r) & 1u)) s1[r] = -INFINITY;
      }
    }
    float x0[4], x1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x0[r] = s0[r] * scale2;
      x1[r] = s1[r] * scale2;
    }
    // the head's maximum over the four lane groups: rows of 16 lanes swapped
    // in pairs, then halves
    float mx = fmaxf(fmaxf(fmaxf(x0[0], x1[0]), fmaxf(x0[1], x1[1])),
                     fmaxf(fmaxf(x0[2], x1[2]), fmaxf(x0[3], x1[3])));
    {
      const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
      mx = max_raw(__uint_as_float(a[0]), __uint_as_float(a[1]));
      const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                      false, false);
      mx = max_raw(__uint_as_float(b[0]), __uint_as_float(b[1]));
    }
    // The subtracted maximum moves only when the stage's maximum exceeds it
    // by more than kDecLazy (log2 units): softmax does not depend on the
    // constant subtracted, so the accumulators are rescaled rarely, and the
    // exponentials stay below 2^kDecLazy.
    const bool grow = mx > m_run + kDecLazy;  // always at the first stage (m_run = -inf)
    const float m_use = grow ? mx : m_run;
    float p0[4], p1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p0[r] = __builtin_amdgcn_exp2f(x0[r] - m_use);
      p1[r] = __builtin_amdgcn_exp2f(x1[r] - m_use);
    }
    const float psum = ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3]));
    if (__ballot(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;  // 0 at first
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[ct][r] *= alpha;
      l_run *= alpha;
      m_run = m_use;
    }
    l_run += psum;
    uint4 pb4;
    pb4.x = pack_bf16x2(p0[0], p0[1]);
    pb4.y = pack_bf16x2(p0[2], p0[3]);
    pb4.z = pack_bf16x2(p1[0], p1[1]);
    pb4.w = pack_bf16x2(p1[2], p1[3]);
    const bf16x8 pb = as_bf16x8(pb4);
    // ---- O^T (value columns 128 wave + 16 ct + 4 g + r, head col) += V^T P^T
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int off = voff[ct];
      const v4s vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(buf + off));
      const v4s vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(buf + off + 16 * NOPE_B));
      bf16x8 va;
      __builtin_memcpy(&va, &vlo, 8);
      __builtin_memcpy(reinterpret_cast<char*>(&va) + 8, &vhi, 8);
      o[ct] = mfma16(va, pb, o[ct]);
    }
  };
  if (nst > 0) {
    stage_rows(lds_ring, kv, row_stride, ent_rows(0), wave, roff);
    if (rope_wave) rope_load(ent_rope(0), rope_a);
  }
  for (int st = 0; st < nst; st += 2) {
    run_stage(st, 0, rope_a, rope_b);
    if (st + 1 < nst) run_stage(st + 1, 1, rope_b, rope_a);
  }
  // ---- partials: m (natural-log units), l summed over the lane groups, O
  l_run += shfl_xor_f(l_run, 16);
  l_run += shfl_xor_f(l_run, 32);
  if (nch == 1) {  // the row's whole selection: the normalised output itself
    if (head < H) {
      const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
      uint16_t* orow = out + ((size_t)t * H + head) * DV + 128 * wave + 4 * g;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        uint2 v;
        v.x = pack_bf16x2(o[ct][0] * inv, o[ct][1] * inv);
        v.y = pack_bf16x2(o[ct][2] * inv, o[ct][3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * ct) = v;
      }
    }
    return;
  }
  const size_t base = ((size_t)t * nch + c) * H;
  if (head < H) {
    if (wave == 0 && g == 0) {
      part_ml[(base + head) * 2 + 0] = m_run * 0.693147180559945309f;
      part_ml[(base + head) * 2 + 1] = l_run;
    }
  }
  // the unnormalised O goes out in bf16: the combine forms a convex
  // combination of the chunks, so each value's rounding (2^-9 relative)
  // stays that small in the result, and the partial traffic halves. It goes
  // through the ring slot that the last stage did not use (every wave had
  // consumed that slot's stage before the last stage's barrier, and no load
  // targets it any more): written there in the accumulator layout and read
  // back so that each store is 16 bytes per lane over whole 256-byte head
  // segments (rows padded to 136 values against bank conflicts).
  {
    constexpr int TS = 136;
    uint16_t* tb = reinterpret_cast<uint16_t*>(ring[nst & 1]) + wave * 16 * TS;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      uint2 v;
      v.x = pack_bf16x2(o[ct][0], o[ct][1]);
      v.y = pack_bf16x2(o[ct][2], o[ct][3]);
      *reinterpret_cast<uint2*>(tb + col * TS + 16 * ct + 4 * g) = v;
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * i + (l >> 4);  // head of the block
      const uint4 v = *reinterpret_cast<const uint4*>(tb + hh * TS + 8 * (l & 15));
      if (16 * hb + hh < H)
        *reinterpret_cast<uint4*>(part_o + (base + 16 * hb + hh) * DV + 128 * wave +
                                  8 * (l & 15)) = v;
    }
  }
}

// grid = (T, ceil(H / 4)), block = 256: wave w merges the nch partials of
// (t, h = 4 blockIdx.y + w),
//   out = sum_c e^(m_c - M) O_c / sum_c e^(m_c - M) l_c  over chunks with l_c > 0,
// M = max m_c. Lane c holds chunk c's (m, l) (chunks in groups of 64); the
// maximum and the normaliser are wave reductions, and chunk c's weight
// reaches the other lanes by a shuffle. Lane l sums value columns
// 8 l .. 8 l + 7 (one 16-byte bf16 load per chunk), the first kCombAhead
// chunks' loads issued unconditionally before the (m, l) loads (a chunk past
// nch reads the last one and gets weight 0). No block barrier.
constexpr int kCombAhead = 16;  // O partials per lane loaded with the (m, l) pairs

// acc[0..7] += w * (eight bf16 values packed in v)
__device__ __forceinline__ void fma_bf16x8(float (&acc)[8], float w, uint4 v) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(w, __uint_as_float(u[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = fmaf(w, __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
  }
}

__global__ __launch_bounds__(256) void mla_decode_combine(const uint16_t* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int H, int nch,
                                                          uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
  if (h >= H) return;  // wave-uniform
  const int l = lane_id();
  const size_t base = (size_t)t * nch * H;
  auto orow = [&](int c) { return part_o + (base + (size_t)c * H + h) * DV + 8 * l; };
  uint4 va[kCombAhead];
#pragma unroll
  for (int u = 0; u < kCombAhead; ++u)
    va[u] = *reinterpret_cast<const uint4*>(orow(min(u, nch - 1)));
  // ---- M and L over the live chunks (l_c > 0), 64 chunks per pass
  float M = -INFINITY;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + l;
    const size_t r = base + (size_t)min(c, nch - 1) * H + h;
    const float m = part_ml[r * 2], lc = part_ml[r * 2 + 1];
    M = fmaxf(M, c < nch && lc > 0.f ? m : -INFINITY);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + l;
    const size_t r = base + (size_t)min(c, nch - 1) * H + h;
    const float m = part_ml[r * 2], lc = part_ml[r * 2 + 1];
    const float wl = c < nch && lc > 0.f ? __expf(m - M) : 0.f;  // this lane's chunk weight
    L += wl * (c < nch ? lc : 0.f);
    const int n = min(64, nch - c0);
    int u0 = 0;
    if (c0 == 0) {
#pragma unroll
      for (int u = 0; u < kCombAhead; ++u)
        fma_bf16x8(acc, u < n ? __shfl(wl, u, DSA_WAVE) : 0.f, va[u]);
      u0 = kCombAhead;
    }
    // the rest in batches of eight loads issued together (clamped, weight 0
    // past the last chunk)
    for (; u0 < n; u0 += 8) {
      uint4 vb[8];
#pragma unroll
      for (int v = 0; v < 8; ++v)
        vb[v] = *reinterpret_cast<const uint4*>(orow(c0 + min(u0 + v, n - 1)));
#pragma unroll
      for (int v = 0; v < 8; ++v)
        fma_bf16x8(acc, u0 + v < n ? __shfl(wl, (u0 + v) & 63, DSA_WAVE) : 0.f, vb[v]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) L += shfl_xor_f(L, o);
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  uint4 packed;
  packed.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  packed.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  packed.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  packed.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(out + ((size_t)t * H + h) * DV + 8 * l) = packed;
}

// Many chunks (nch > kCombAhead). grid = (T, H), block = 256: merge the nch
// partials of (t, h),
//   out = sum_c e^(m_c - M) O_c / sum_c e^(m_c - M) l_c  over chunks with l_c > 0,
// M = max m_c. Thread (g, d4) = (tid / 128, tid % 128) sums chunks g, g + 2,
// ... for value columns 4 d4 .. 4 d4 + 3. The first kWideAhead of this
// thread's O partials (bf16) and the (m, l) pairs are all loaded at once; the
// chunk weights e^(m_c - M) are then computed once, in LDS, and the two
// halves of the sum meet through LDS.
constexpr int kCombMaxCH = 1024;  // partials per (row, head) the wide combine handles
constexpr int kWideAhead = 16;    // O partials per thread loaded with the (m, l) pairs

// acc += w * (four bf16 partial values packed in v)
__device__ __forceinline__ void fma_bf16x4(float4& acc, float w, uint2 v) {
  acc.x = fmaf(w, __uint_as_float(v.x << 16), acc.x);
  acc.y = fmaf(w, __uint_as_float(v.x & 0xffff0000u), acc.y);
  acc.z = fmaf(w, __uint_as_float(v.y << 16), acc.z);
  acc.w = fmaf(w, __uint_as_float(v.y & 0xffff0000u), acc.w);
}

__global__ __launch_bounds__(256) void mla_decode_combine_wide(const uint16_t* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          int H, int nch,
                                                          uint16_t* __restrict__ out) {
  __shared__ float s_w[kCombMaxCH];
  __shared__ float4 s_o[128];
  __shared__ float s_red[8];
  const int t = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, l = lane_id(), wave = tid >> 6;
  const int g = tid >> 7, d4 = tid & 127;
  const size_t base = (size_t)t * nch * H;
  // ---- this thread's first O partials, then the (m, l) pairs: all in
  // flight together. The O loads are unconditional (a chunk past nch reads
  // the last chunk and gets weight 0), so that none of them waits for another
  uint2 va[kWideAhead];
#pragma unroll
  for (int u = 0; u < kWideAhead; ++u) {
    const int c = min(g + 2 * u, nch - 1);
    va[u] = *reinterpret_cast<const uint2*>(part_o + (base + (size_t)c * H + h) * DV + 4 * d4);
  }
  float mloc = -INFINITY;
  for (int c = tid; c < nch; c += 256) {
    const size_t r = base + (size_t)c * H + h;
    const float m = part_ml[r * 2], lc = part_ml[r * 2 + 1];
    const float mm = lc > 0.f ? m : -INFINITY;
    s_w[c] = mm;
    mloc = fmaxf(mloc, mm);
  }
  // ---- M = max over live chunks (l_c > 0)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, shfl_xor_f(mloc, o));
  if (l == 0) s_red[wave] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  // ---- weights and L = sum_c w_c l_c
  float lloc = 0.f;
  for (int c = tid; c < nch; c += 256) {
    const size_t r = base + (size_t)c * H + h;
    const float w = s_w[c] == -INFINITY ? 0.f : __expf(s_w[c] - M);
    s_w[c] = w;
    lloc += w * part_ml[r * 2 + 1];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lloc += shfl_xor_f(lloc, o);
  __syncthreads();  // every M is read and every weight written; s_red is free
  if (l == 0) s_red[4 + wave] = lloc;
  // ---- O: this thread's half of the chunks
  // (a chunk without live selections has w = 0 and a zero partial O)
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kWideAhead; ++u) {
    const int c = g + 2 * u;
    fma_bf16x4(acc, c < nch ? s_w[c] : 0.f, va[u]);
  }
  for (int c0 = g + 2 * kWideAhead; c0 < nch; c0 += 8) {
    uint2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = min(c0 + 2 * u, nch - 1);
      v[u] = *reinterpret_cast<const uint2*>(part_o + (base + (size_t)c * H + h) * DV + 4 * d4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + 2 * u;
      fma_bf16x4(acc, c < nch ? s_w[c] : 0.f, v[u]);
    }
  }
  if (g == 1) s_o[d4] = acc;
  __syncthreads();
  if (g == 0) {
    const float4 b = s_o[d4];
    const float L = (s_red[4] + s_red[5]) + (s_red[6] + s_red[7]);
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    uint2 packed;
    packed.x = pack_bf16x2((acc.x + b.x) * inv, (acc.y + b.y) * inv);
    packed.y = pack_bf16x2((acc.z + b.z) * inv, (acc.w + b.w) * inv);
    *reinterpret_cast<uint2*>(out + ((size_t)t * H + h) * DV + 4 * d4) = packed;
  }
}

// Few chunks (nch <= kCombFew), many rows. grid = (ceil(T / kCombRows), ceil(H / 4)),
// block = 256: wave w merges the partials of head h = 4 blockIdx.y + w for
// kCombRows consecutive rows, with every load of those rows (each row's nch
// (m, l) pairs and O chunks) issued before the first reduction; lane l sums
// value columns 8 l .. 8 l + 7. The merge is that of mla_decode_combine.
constexpr int kCombFew = 4;
constexpr int kCombRows = 4;

__global__ __launch_bounds__(256) void mla_decode_combine_rows(const uint16_t* __restrict__ part_o,
                                                               const float* __restrict__ part_ml,
                                                               int T, int H, int nch,
                                                               uint16_t* __restrict__ out) {
  const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
  if (h >= H) return;  // wave-uniform
  const int l = lane_id();
  const int t0 = kCombRows * blockIdx.x;
  uint4 va[kCombRows][kCombFew];
  float2 ml[kCombRows][kCombFew];
#pragma unroll
  for (int r = 0; r < kCombRows; ++r) {
    const int t = min(t0 + r, T - 1);  // a row past T reloads the last row, never stored
#pragma unroll
    for (int c = 0; c < kCombFew; ++c) {
      const size_t idx = ((size_t)t * nch + min(c, nch - 1)) * H + h;
      va[r][c] = *reinterpret_cast<const uint4*>(part_o + idx * DV + 8 * l);
      ml[r][c] = *reinterpret_cast<const float2*>(part_ml + idx * 2);
    }
  }
#pragma unroll
  for (int r = 0; r < kCombRows; ++r) {
    const int t = t0 + r;
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kCombFew; ++c)
      if (c < nch && ml[r][c].y > 0.f) M = fmaxf(M, ml[r][c].x);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
#pragma unroll
    for (int c = 0; c < kCombFew; ++c) {
      const float wc = c < nch && ml[r][c].y > 0.f ? __expf(ml[r][c].x - M) : 0.f;
      L += wc * (c < nch ? ml[r][c].y : 0.f);
      fma_bf16x8(acc, wc, va[r][c]);
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    uint4 packed;
    packed.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    packed.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    packed.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
    packed.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
    if (t < T) *reinterpret_cast<uint4*>(out + ((size_t)t * H + h) * DV + 8 * l) = packed;
  }
}

int mla_decode_chunk(int T, int k) {
  // about kDecWPC workgroups per compute unit, 1 .. kDecMaxCH / 64 blocks of
  // 64 selections each: a large batch gets long chunks, which cuts both the
  // one-time prologues and the partials the combine reads
  const long nsub = (k + 63) / 64;
  const long slots = 256L * kDecWPC;
  long per = ((long)T * nsub + slots - 1) / slots;
  if (per < 1) per = 1;
  if (per > kDecMaxCH / 64) per = kDecMaxCH / 64;
  return (int)per * 64;
}

hipError_t mla_decode(const MlaArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int CH = mla_decode_chunk(a.T, a.k);
  const int nch = (a.k + CH - 1) / CH;
  const int HB = (a.H + 15) / 16;
  {
    ProfScope prof("mla_decode_partial", st);
    if (a.sel_pages)
      hipLaunchKernelGGL((mla_decode_partial<1>), dim3(nch * HB, a.T), dim3(256), 0, st, a.q,
                         a.kv, a.row_stride, a.num_pages, a.pt, a.seq_lens, a.cu, a.topk,
                         a.k / a.PS, a.T, a.S, a.H, a.k, a.PS, a.MP, a.sm_scale, CH, nch, HB,
                         a.part_o, a.part_ml, a.out);
    else
      hipLaunchKernelGGL((mla_decode_partial<0>), dim3(nch * HB, a.T), dim3(256), 0, st, a.q,
                         a.kv, a.row_stride, a.num_pages, a.pt, a.seq_lens, a.cu, a.topk, a.k,
                         a.T, a.S, a.H, a.k, a.PS, a.MP, a.sm_scale, CH, nch, HB, a.part_o,
                         a.part_ml, a.out);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nch == 1) return hipSuccess;  // the partial wrote the output
  ProfScope prof("mla_decode_combine", st);
  if (nch <= kCombFew && a.T >= 1024)  // many rows of few chunks: several rows per wave
    hipLaunchKernelGGL(mla_decode_combine_rows, dim3((a.T + kCombRows - 1) / kCombRows,
                                                     (a.H + 3) / 4),
                       dim3(256), 0, st, a.part_o, a.part_ml, a.T, a.H, nch, a.out);
  else if (nch > kCombAhead)  // many chunks: two thread groups per (row, head) share them
    hipLaunchKernelGGL(mla_decode_combine_wide, dim3(a.T, a.H), dim3(256), 0, st, a.part_o,
                       a.part_ml, a.H, nch, a.out);
  else
    hipLaunchKernelGGL(mla_decode_combine, dim3(a.T, (a.H + 3) / 4), dim3(256), 0, st, a.part_o,
                       a.part_ml, a.H, nch, a.out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Extend (query block): one fetch of each union page for all QB * H rows of
// a block ("sparse_mla_prefill_qblock.py", _qblock_kernel).
//
// Workgroup = 2 wave pairs x 32 rows (row = q * H + h of the block). Both
// waves of a pair keep the same 32 rows' query fragments in registers; per
// page, wave `role` of pair `pr` computes
//   S^T = K . Q^T for keys 32 role .. 32 role + 31 of the page and the rows
//     of its pair (v_mfma_f32_32x32x16_bf16: M = keys, N = rows, K = 576);
// the pair meets through LDS for the row maxima (the shared online-softmax
// offset). A lane's S^T accumulator holds 16 keys of ONE row, which is
// exactly the layout of a P^T operand, so P is packed in place and published
// in LDS. Then wave w computes
//   O^T += V^T . P^T for value columns 128 w .. 128 w + 127 and all 64 rows
//     (M = value columns, N = rows of one pair, K = keys),
// so each V^T fragment serves the MFMAs of both pairs. V^T fragments come
// from the row-major page through transposed 16-bit LDS reads
// (ds_read_b64_tr_b16: inside each 16-lane group, lanes 4k..4k+3 supply 16
// consecutive values of row k and lane j receives column j of the 4 rows),
// so one row-major copy of the page serves both products; transposed reads
// move about half the bytes per clock of 16-byte reads, which is why each
// one is used twice.
//
// Pages are staged with direct global->LDS 16-byte loads into two 72 KB
// buffers (double buffering: page s+1 is in flight while page s is used),
// in the swizzled nope/rope layout described at the top of this file. Rows
// beyond the page or at positions >= kv_len are filled from the page's row 0
// (a valid row whenever the page has any); their keys are masked, so they
// only ever meet probability 0 on finite data. The metadata of a union slot
// (page, sequence, length, membership word) is loaded a step or two before
// its page is used.
//
// Logits are kept in log2 units (sm_scale * log2 e folded in, exp2 on the
// hardware). The softmax offset is updated lazily: the accumulator is
// rescaled only when a row's maximum grows by more than e^8 (probabilities
// stay below e^8 before normalisation), which leaves the normalised result
// unchanged.
// ---------------------------------------------------------------------------
constexpr int XW = 4;                          // waves per workgroup (2 pairs)
constexpr int XROWS = 64;                      // rows per workgroup
constexpr int PROWS = 64;                      // rows per staged page (PS <= 64)
constexpr int ROPE_OFF = PROWS * NOPE_B;       // rope region after the 64 nope rows
constexpr int PAGE_BYTES = PROWS * (NOPE_B + ROPE_B);  // 73728
constexpr float kLazyMax2 = 11.5415603f;  // 8 nats in log2 units: rescale when the
                                          // offset would grow by more than e^8

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

// Metadata of a union slot as loaded (clamped key, its page-table entry and
// its sequence length), fetched a step ahead of its use.
struct SlotRaw {
  int key, sp, lp, ptv, slv;  // key = sp * MP + lp
};

__device__ __forceinline__ int clamp_key(int key, int S, int MP) {
  return key < 0 ? 0 : (key >= S * MP ? S * MP - 1 : key);
}

__device__ __forceinline__ SlotRaw slot_raw(const int32_t* __restrict__ pt,
                                            const int32_t* __restrict__ seq_lens, int key,
                                            int MP) {
  SlotRaw r;
  r.key = key;
  r.sp = key / MP;
  r.lp = key - r.sp * MP;
  r.ptv = pt[key];
  r.slv = seq_lens[r.sp];
  return r;
}

__device__ __forceinline__ PageMeta meta_from_raw(const SlotRaw& r, int MP, int cap,
                                                  int num_pages) {
  PageMeta pm;
  pm.sp = r.sp;
  pm.lp = r.lp;
  pm.kvp = r.slv < 0 ? 0 : (r.slv > cap ? cap : r.slv);
  pm.page = clamp_page(r.ptv, num_pages);
  return pm;
}

// Issue this wave's direct loads of one page into the LDS buffer at byte
// address `buf`: wave w fills nope rows r = 4 n + w (n < 16, LDS bytes
// [1024 r, 1024 r + 1024)) and the rope parts of rows 8 G .. 8 G + 7 for
// G = w and w + 4 (bytes ROPE_OFF + 1024 G ..). Rows beyond the page or at
// positions >= kv_len read the page's row 0 instead. `wave` must be
// wave-uniform to the compiler (readfirstlane), so that the row choices and
// the row base addresses are scalar.
__device__ __forceinline__ void stage_page(uint32_t buf, const uint16_t* __restrict__ kv,
                                           int row_stride, const PageMeta& pm, int PS,
                                           int wave) {
  const int l = lane_id_volatile();
  const unsigned char* pg =
      reinterpret_cast<const unsigned char*>(kv + (size_t)pm.page * PS * row_stride);
  const int valid_rows = min(PS, pm.kvp - pm.lp * PS);  // rows [0, valid_rows) are live
  const size_t rs = (size_t)row_stride * 2;
  const uint32_t l16 = 16u * (uint32_t)l;
#pragma unroll
  for (int n = 0; n < PROWS / XW; ++n) {
    const int r = XW * n + wave;
    const int use = r < valid_rows ? r : 0;
    gll16_s(l16 ^ (16u * (uint32_t)nope_x(r)), pg + use * rs, buf + r * NOPE_B);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int G = wave + XW * j;
    const int r = 8 * G + (l >> 3);
    const int use = r < valid_rows ? r : 0;
    gll16_s((uint32_t)(use * (int)rs) + 2 * DV + 16u * (uint32_t)((l & 7) ^ rope_x(r)), pg,
            buf + ROPE_OFF + G * 1024);
  }
}

// The same page staging split into its 18 loads (n < 16: nope row 4 n + wave;
// n = 16, 17: rope groups wave, wave + 4), so that they can be spread over
// the matrix work of a step instead of stalling the wave in one burst.
struct StageCtx {
  const unsigned char* pg;
  uint32_t rs;  // bytes per cache row; a page (PS <= 64 rows) spans far less than 4 GiB
  uint32_t buf;
  int valid_rows, wave;
};

__device__ __forceinline__ StageCtx stage_ctx(uint32_t buf, const uint16_t* __restrict__ kv,
                                              int row_stride, const PageMeta& pm, int PS,
                                              int wave) {
  StageCtx c;
  c.pg = reinterpret_cast<const unsigned char*>(kv + (size_t)pm.page * PS * row_stride);
  c.rs = (uint32_t)row_stride * 2u;
  c.buf = buf;
  c.valid_rows = min(PS, pm.kvp - pm.lp * PS);
  c.wave = wave;
  return c;
}

__device__ __forceinline__ void stage_one(const StageCtx& c, int n, int l) {
  if (n < PROWS / XW) {
    const int r = XW * n + c.wave;
    const uint32_t use = r < c.valid_rows ? (uint32_t)r : 0u;
    gll16_s((16u * (uint32_t)l) ^ (16u * (uint32_t)nope_x(r)), c.pg + use * c.rs,
            c.buf + r * NOPE_B);
  } else {
    const int G = c.wave + XW * (n - PROWS / XW);
    const int r = 8 * G + (l >> 3);
    const int use = r < c.valid_rows ? r : 0;
    gll16_s((uint32_t)use * c.rs + 2 * DV + 16u * (uint32_t)((l & 7) ^ rope_x(r)), c.pg,
            c.buf + ROPE_OFF + G * 1024);
  }
}

constexpr int kStageLoads = PROWS / XW + 2;  // 18 direct loads per wave per page
constexpr int kSAhead = 6;  // S^T operand reads in flight per wave

struct ExtArgs {
  const uint16_t* __restrict__ kv;
  const int32_t* __restrict__ pt;
  const int32_t* __restrict__ seq_lens;
  const int32_t* __restrict__ units;
  const uint64_t* __restrict__ member;
  int row_stride, num_pages, S, PS, MP, QB, u_max, cap, b, u_lim;
  float scale2;  // sm_scale * log2(e)
};

struct ExtLane {
  int wave, l, pr, role, g, m, qloc;
  int soff[12];    // S^T reads: byte offsets of this lane's 36 chunks (see ext_offsets)
  int toff[2][4];  // V^T transposed reads: per-lane parts of the byte offsets
  RowInfo ri;
  bf16x8 qb[DK / 16];
  f32x16 o[2][4];  // O^T tiles: [pair of the rows][32-column block of this wave]
  float m_used[2];  // softmax offsets of rows m of pair 0 and pair 1 (log2 units)
  float l_part;
};

// Metadata carried from step to step: slot s's page (complete), slot s + 1's
// raw entries, slot s + 2's key, and this lane's membership word of slot s.
struct ExtPipe {
  PageMeta cur;
  SlotRaw next;
  int key2;
  uint64_t mem;
};

// One union page: `cur` holds it, `nxt` receives the next one meanwhile.
// The __restrict__ LDS pointers let the compiler see that reads of `cur`
// and of the exchange buffers never alias the loads in flight into `nxt`.
// Every global load issued here is consumed one step later, after that
// step's wait, so no load latency is exposed inside a step.
__device__ __forceinline__ void ext_step(const ExtArgs& A, ExtLane& X, ExtPipe& P, int slot,
                                         const unsigned char* __restrict__ cur, uint32_t nxt,
                                         bf16x8* __restrict__ pf, float* __restrict__ smax) {
  const int l = X.l, g = X.g, m = X.m, pr = X.pr, role = X.role;
  // this wave's loads of page `slot` (issued one step earlier) and the
  // metadata loads of the previous step have landed; after the barrier
  // every wave's have, and nobody reads `nxt` (the previous page) any more
  wait_vmcnt<0>();
  lds_barrier();
  const PageMeta pm = P.cur;
  const PageMeta pn = meta_from_raw(P.next, A.MP, A.cap, A.num_pages);
  // the next page's loads are issued during this page's S^T products. The
  // last step stages the slot it already holds in P.next (a clamped, valid
  // key) into the buffer nobody reads again: unconditional loads keep the
  // matrix loop free of branches.
  const bool do_stage = true;
  const StageCtx sc = stage_ctx(nxt, A.kv, A.row_stride, pn, A.PS, X.wave);
  // metadata for the coming steps
  uint64_t mem_n = 0;
  if (slot + 1 < A.u_lim) mem_n = A.member[((size_t)A.b * A.u_max + slot + 1) * A.QB + X.qloc];
  SlotRaw raw2 = P.next;
  if (slot + 2 < A.u_lim) raw2 = slot_raw(A.pt, A.seq_lens, clamp_key(P.key2, A.S, A.MP), A.MP);
  int key3 = 0;
  if (slot + 3 < A.u_lim) key3 = A.units[(size_t)A.b * A.u_max + slot + 3];

  const int lim = min(X.ri.abs_q + 1, pm.kvp) - pm.lp * A.PS;
  uint64_t mk = 0;
  if (X.ri.seq == pm.sp && lim > 0) mk = lim >= 64 ? P.mem : (P.mem & ((1ull << lim) - 1));
  if (A.PS < 64) mk &= (1ull << A.PS) - 1;
  P.cur = pn;
  P.next = raw2;
  P.key2 = key3;
  P.mem = mem_n;
  // both waves of a pair hold the same rows, hence the same masks
  const bool pair_any = __ballot(mk != 0ull) != 0;
  if (!pair_any && do_stage) {
#pragma unroll
    for (int n = 0; n < kStageLoads; ++n) stage_one(sc, n, l);
  }
  const uint32_t hm = (uint32_t)(mk >> (32 * role));
  f32x16 sacc = {};
  float mx = -INFINITY;
  if (pair_any) {
    // ---- S^T tile: keys 32 role + m (A from LDS), rows m (B = resident q);
    // step i reads chunk 2 i + g of key row 32 role + m
    auto s_off = [&](int i) { return i < 32 ? X.soff[i & 7] + 256 * (i >> 3) : X.soff[8 + (i - 32)]; };
    // operands are read kSAhead steps ahead of the MFMA that consumes them,
    // so that several LDS reads per wave are in flight
    bf16x8 aq[kSAhead];
#pragma unroll
    for (int i = 0; i < kSAhead; ++i)
      aq[i] = as_bf16x8(*reinterpret_cast<const uint4*>(cur + s_off(i)));
#pragma unroll
    for (int i = 0; i < DK / 16; ++i) {
      const bf16x8 a = aq[i % kSAhead];
      if (i + kSAhead < DK / 16)
        aq[i % kSAhead] = as_bf16x8(*reinterpret_cast<const uint4*>(cur + s_off(i + kSAhead)));
      sacc = mfma32(a, X.qb[i], sacc);
      if (do_stage && (i & 1) == 0 && (i >> 1) < kStageLoads) stage_one(sc, i >> 1, l);
    }
    // accumulator r of this lane holds key 8 (r / 4) + 4 g + (r % 4) of the
    // half; logits are kept in log2 units (sm_scale * log2 e folded in). A
    // masked key becomes -inf by a bit select on the sign-extended mask bit.
    const uint32_t hg = hm >> (4 * g);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + (r & 3);
      const uint32_t sel = (uint32_t)((int)(hg << (31 - key)) >> 31);
      const uint32_t v = __float_as_uint(sacc[r] * A.scale2);
      sacc[r] = __uint_as_float((v & sel) | (0xff800000u & ~sel));
      mx = fmaxf(mx, sacc[r]);
    }
  }
  // every half-wave publishes its own maximum (-inf without selections); the
  // four partial maxima of a row (two halves, two roles) meet after the
  // barrier, and every wave combines them for the rows of BOTH pairs: the
  // lazy offset update is deterministic, so each wave tracks the offsets of
  // both pairs' rows itself and rescales its accumulators without a second
  // exchange
  smax[((pr * 2 + role) * 2 + g) * 32 + m] = mx;
  lds_barrier();
  float al[2];
#pragma unroll
  for (int p2 = 0; p2 < 2; ++p2) {
    const float* sm = smax + p2 * 4 * 32 + m;
    const float rm = fmaxf(fmaxf(sm[0], sm[32]), fmaxf(sm[64], sm[96]));
    al[p2] = 1.f;
    if (rm > X.m_used[p2] + kLazyMax2) {
      al[p2] = __builtin_amdgcn_exp2f(X.m_used[p2] - rm);  // 0 while nothing was accumulated
      X.m_used[p2] = rm;
    }
  }
  const float alpha = pr ? al[1] : al[0];
  const float m_own = pr ? X.m_used[1] : X.m_used[0];
  X.l_part *= alpha;
  bf16x8 pb[2];
  if (pair_any) {
    // exp2(-inf) is 0, so masked keys need no test; a row with no offset
    // yet has only masked keys and subtracts 0 instead of -inf
    const float off = m_own == -INFINITY ? 0.f : m_own;
    uint32_t w[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sacc[r] - off);
      const float p1 = __builtin_amdgcn_exp2f(sacc[r + 1] - off);
      X.l_part += p0 + p1;
      w[r >> 1] = pack_bf16x2(p0, p1);
    }
    __builtin_memcpy(&pb[0], w, 16);
    __builtin_memcpy(&pb[1], w + 4, 16);
  } else {
    pb[0] = as_bf16x8(zero_u4());
    pb[1] = pb[0];
  }
  pf[((pr * 2 + role) * 2 + 0) * 64 + l] = pb[0];
  pf[((pr * 2 + role) * 2 + 1) * 64 + l] = pb[1];
  // ---- rescale the O rows whose softmax offset moved (rows m of both pairs)
  if (__ballot(al[0] != 1.f || al[1] != 1.f) != 0) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        X.o[0][ct][r] *= al[0];
        X.o[1][ct][r] *= al[1];
      }
  }
  lds_barrier();
  // ---- O^T += V^T P^T for value columns 128 wave + 32 ct + ..., all 64 rows:
  // four 16-key steps; each V^T fragment feeds the MFMAs of both pairs
  auto vfrag = [&](int j) {  // j = (kh * 2 + st) * 4 + ct
    const int kh = j >> 3, st = (j >> 2) & 1, ct = j & 3;
    const int dc = (32 * kh + 16 * st) * NOPE_B + 256 * X.wave;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(cur + dc + X.toff[0][ct]));
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(cur + dc + X.toff[1][ct]));
    bf16x8 a;
    __builtin_memcpy(&a, &lo, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
    return a;
  };
  bf16x8 v0 = vfrag(0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int kh = ks >> 1, st = ks & 1;
    const bf16x8 b0 = pf[((0 * 2 + kh) * 2 + st) * 64 + l];
    const bf16x8 b1 = pf[((1 * 2 + kh) * 2 + st) * 64 + l];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int j = ks * 4 + ct;
      bf16x8 v1 = v0;
      if (j + 1 < 16) v1 = vfrag(j + 1);
      X.o[0][ct] = mfma32(v0, b0, X.o[0][ct]);
      X.o[1][ct] = mfma32(v0, b1, X.o[1][ct]);
      v0 = v1;
    }
  }
}

// Per-lane LDS byte offsets, fixed for the whole kernel.
// S^T reads: lane (m, g) of wave `role` reads key row kr = 32 role + m,
// chunk 2 i + g. For i < 32 the slot is (2 i + g) ^ nope_x(kr) = 16 (i >> 3)
// + ((2 (i & 7)) ^ y), y = g ^ nope_x(kr), so 8 per-lane values plus a
// constant; for i >= 32 the rope chunk 2 (i - 32) + g of row kr.
// V^T reads: the lane supplies row key0 = 32 kh + 16 st + 4 g + kq (read 0)
// or key0 + 8 (read 1), 16-byte chunk 16 wave + 4 ct + c0 and byte boff,
// with kq = (l & 15) >> 2, c0 = 2 ((l >> 4) & 1) + ((l & 3) >> 1), boff =
// 8 (l & 1). nope_x depends on the row modulo 16 only, so the slot is
// 16 wave + ((4 ct + c0) ^ nope_x(4 g + kq + 8 e)): 4 per-lane values per
// read plus the constants 1024 (32 kh + 16 st) and 256 wave.
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
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int key = 4 * X.g + kq + 8 * e;
    const int x = nope_x(key);
#pragma unroll
    for (int j = 0; j < 4; ++j) X.toff[e][j] = key * NOPE_B + 16 * ((4 * j + c0) ^ x) + boff;
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
  __shared__ float s_max[2 * 2 * 2 * 32];    // row maxima [pair][role][half][row]
  const int TPB = (QB * H + XROWS - 1) / XROWS;
  const int nqb = (T + QB - 1) / QB;
  // the TPB workgroups of a block get ids of one residue mod 8, i.e. one XCD
  const int L = blockIdx.x;
  const int jj = L >> 3;
  const int b = (jj / TPB) * 8 + (L & 7);
  const int tile = jj % TPB;
  if (b >= nqb) return;

  ExtLane X;
  X.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  for (int p2 = 0; p2 < 2; ++p2)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) X.o[p2][ct] = f32x16{};
  X.m_used[0] = -INFINITY;
  X.m_used[1] = -INFINITY;
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
  A.scale2 = sm_scale * 1.44269504088896341f;

  ExtPipe P;
  P.mem = 0;
  P.key2 = 0;
  if (A.u_lim > 0) {
    P.cur = page_meta(units, pt, seq_lens, b, u_max, 0, S, MP, cap, num_pages);
    stage_page(lds_addr_of(page0), kv, row_stride, P.cur, PS, X.wave);
    P.mem = member[(size_t)b * u_max * QB + X.qloc];
    const int k1 = A.u_lim > 1 ? clamp_key(units[(size_t)b * u_max + 1], S, MP) : 0;
    P.next = slot_raw(pt, seq_lens, k1, MP);
    if (A.u_lim > 2) P.key2 = units[(size_t)b * u_max + 2];
  }
  const uint32_t lds0 = lds_addr_of(page0), lds1 = lds_addr_of(page1);
  for (int slot = 0; slot < A.u_lim; ++slot) {
    const unsigned char* cur = (slot & 1) ? page1 : page0;
    ext_step(A, X, P, slot, cur, (slot & 1) ? lds0 : lds1, pfrag, s_max);
  }
  wait_vmcnt<0>();  // the last step's staging loads land before the workgroup ends
  // ---- row sums over both key halves, then normalise and store this
  // wave's value columns 128 wave + 32 ct + 8 (r / 4) + 4 g + (r % 4) of the
  // rows m of both pairs
  const float lw = X.l_part + shfl_xor_f(X.l_part, 32);
  __syncthreads();
  if (X.g == 0) s_max[(X.pr * 2 + X.role) * 32 + X.m] = lw;
  __syncthreads();
#pragma unroll
  for (int p2 = 0; p2 < 2; ++p2) {
    const float lt = s_max[(p2 * 2 + 0) * 32 + X.m] + s_max[(p2 * 2 + 1) * 32 + X.m];
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int row2 = tile * XROWS + p2 * 32 + X.m;
    if (row2 >= QB * H) continue;
    const int t2 = b * QB + row2 / H, h2 = row2 % H;
    if (t2 >= T) continue;
    uint16_t* orow = out + ((size_t)t2 * H + h2) * DV + 128 * X.wave;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint2 v;
        v.x = pack_bf16x2(X.o[p2][ct][4 * r4] * inv, X.o[p2][ct][4 * r4 + 1] * inv);
        v.y = pack_bf16x2(X.o[p2][ct][4 * r4 + 2] * inv, X.o[p2][ct][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * ct + 8 * r4 + 4 * X.g) = v;
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

// ---------------------------------------------------------------------------
// Device-resident scratch of the allocation-free decode entry point: the
// split-list partials (unnormalised O and (m, l)) live in this array instead
// of a caller workspace. Each GPU the library runs on holds its own copy,
// zero-filled when the code object loads and kept until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): the per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_dev[kMaxScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    per_dev[dev] = p;
  }
  *ptr = per_dev[dev];
  return hipSuccess;
}

}  // namespace dsa
