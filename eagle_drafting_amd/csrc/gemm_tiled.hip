// Projections for larger draft batches (M = B*K rows > 32): LDS-tiled bf16 MFMA GEMM with the same fused
// epilogues as the small-batch kernel.
//
// Workgroup tile 128 rows x 128 columns, 4 waves in a 2 x 2 arrangement (each wave 64 x 64: 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16, the bf16 MFMA with the highest sustained rate on gfx950). Each stage covers 64
// of the reduction dimension. Activations are staged through two LDS buffers as 16 x 32 fragments (the
// layout of the packed weights); weights go from the packed fragments straight into registers (each
// fragment is used by the two waves of a column half). Activation loads run two stages ahead, weight
// loads one; the stage loop is branch-free (even stage count, zero activations past the end), so the
// compiler's wait counts stay exact. The 12 global loads of a stage are issued three at a time between
// the four MFMA groups (the per-CU vector-memory path takes ~16 cycles per 1 KiB wave load, so issuing
// them back to back stalls the wave for most of a stage), and the next fragment pair is read from LDS
// while the current products run.
//
// Epilogue: the 128 x 128 fp32 product tile is written into the same 64 KiB of LDS (column XOR-swizzle so
// the two lane halves of the accumulator layout hit distinct banks), then read back as 16-byte row chunks:
// half a wave covers one 128-column row, so global reads and writes of the residual stream, the caches and
// the logits are coalesced, and per-row reductions (sums of squares, argmax) are 32-lane shuffles. Gate/up
// and RoPE pairs, which the weight repack put 8 columns apart, are read as two chunks of the same row.
#include "common.h"
#include <type_traits>
#include "kernels.h"

namespace pe {

// cache policy of the K-split partial stores: device scope (sc1), so that they are written through to
// the memory side during the product rather than left dirty in the L2 for the end-of-kernel write-back
// before the reduce kernel (measured: Qwen B 8 K 11 581 -> 571 us per draft step, B 128 K 7 2087 ->
// 2072 us, GPT-OSS B 64 K 10 2653 -> 2642 us; non-temporal stores were no faster than plain ones)
// cache policy of the weight loads of the kernels that read every weight byte once per launch (the
// weight-stream and burst kernels): non-temporal (measured on a streaming read of this part: 7.0 TB/s
// against 6.3 TB/s with plain loads)
#ifndef PE_WNT
#define PE_WNT 2
#endif
#ifndef PE_PART_AUX
#define PE_PART_AUX 16
#endif

// Product tile epilogue (defined below): Cs holds the 128 x 128 fp32 tile, column-swizzled; with SCALE,
// s_inv[r] is row r's 1/RMS.
template <int EP, bool SCALE>
__device__ void tile_epilogue(const GemmArgs& g, const float* Cs, const float* s_inv, int m0, int nt0, int ng,
                              int rbeg = 0, int rend = 128, int etid = -1);

// 1 / RMS of the 128 rows of a tile from the producer's partial sums of squares, TPR threads per row (TPR =
// threads / 128): start() issues the loads of up to eight partials per thread before the product loop, so
// that their latency overlaps it, and finish() adds them (in a fixed order, then across the row's threads)
// after it; partials beyond TPR * 8 are loaded there (none for the producers of these tiles' operands).
template <int NTH>
struct RowScale {
  static constexpr int TPR = NTH / 128, PRE = 8;
  float v[PRE];
  const float* src = nullptr;
  __device__ __forceinline__ void start(const GemmArgs& g, int m0, int tid) {
    const int r = tid / TPR, h = tid % TPR;
    if (m0 + r < g.M) src = g.ssq_in + (size_t)gemm_a_row(g, m0 + r) * g.nssq;
#pragma unroll
    for (int u = 0; u < PRE; ++u) v[u] = src && h + TPR * u < g.nssq ? src[h + TPR * u] : 0.f;
  }
  __device__ __forceinline__ void finish(const GemmArgs& g, float* s_inv, int tid) {
    const int r = tid / TPR, h = tid % TPR;
    float t = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    for (int i = h + TPR * PRE; src && i < g.nssq; i += TPR) t += src[i];
    t = group_sum<TPR>(t);
    if (h == 0) s_inv[r] = rsqrtf(t / (float)g.Kd + g.eps);
  }
};

// SPLIT: the workgroup covers k-steps [blockIdx.y * g.kper, + g.kper) and writes its fp32 partial tile
// (row-scaled for a normalised operand) to g.part[blockIdx.y]; gemm_split_reduce_kernel adds the partials
// in a fixed order and runs the epilogue.
// F8: E4M3 weight fragment pairs (one 16-byte lane load holds the stage's two k-steps), converted to the
// bf16 operand in registers; product columns scaled as the tile goes to LDS.
template <int AM, int EP, bool SPLIT, int F8 = 0>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmArgs g) {
  constexpr int BM = 128, BN = 128;
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * 2 * 8 * 64 * 16];  // 64 KiB: product tile; A buffers in the first half
  __shared__ float s_inv[BM];
  bf16x8_t(*As)[2][8][64] = (bf16x8_t(*)[2][8][64])smem;                      // [buffer][k-step][m-tile][lane]
  float* Cs = (float*)smem;                                                  // [BM][BN], after the main loop

  const int M = g.M, Ks = g.Ks, Nt = g.Nt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  // Workgroup w runs on XCD w % 8 (round-robin dispatch). Each XCD takes every 8th column group and runs
  // all row blocks of one column group back to back, so a weight tile is fetched from HBM once and its
  // other row blocks hit that XCD's L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int ng = (slot / g.mblocks) * 8 + xcd;
  if (ng >= g.ngroups) return;
  const int m0 = (slot % g.mblocks) * BM;
  const int nt0 = ng * 8;
  // stages of 64 reduction columns, rounded up to an even count; activation loads past the last k-step
  // return zeros (out-of-range buffer offset), so padded stages add nothing and the loop has no branches
  const int kb = SPLIT ? blockIdx.y * g.kper : 0;                // first k-step of this workgroup
  const int ke = SPLIT ? min(Ks, kb + g.kper) : Ks;               // end of its k-steps
  const int nstage = SPLIT ? g.kper / 2 : ((Ks + 1) / 2 + 1) & ~1;  // even (kper is a multiple of 4)

  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, gemm_a_rows(g) * g.lda * 2, 0x00020000);
  const uint4* W8 = (const uint4*)g.Wp_raw;  // F8: fragment pairs, (Ks + 1) / 2 per tile
  const int Ks2 = (Ks + 1) / 2;

  // Activations go through LDS (shared by the two waves of a row half); weights go straight from the
  // packed fragments into the registers of the waves that use them (each fragment is needed by the two
  // waves of a column half). Activations: piece p = tid + 256 q covers row p / 8 and 16-byte segment p % 8
  // of the stage's 64 columns (8 lanes read one 128-byte row segment); their LDS slot is fragment lane
  // (row % 16) + 16 (segment % 4) of k-step segment / 4, XOR-swizzled by 4 (segment % 4).
  auto asw = [](int lp) { return lp ^ ((lp >> 4) << 2); };
  typedef bf16x8_t RegA[4];
  typedef bf16x8_t RegB16[8];  // [(ks * 2 + u) * 2 + j]
  typedef uint4 RegB8[4];      // F8: [u * 2 + j], both k-steps of the stage
  using RegB = std::conditional_t<(F8 != 0), RegB8, RegB16>;
  RegA ra0, ra1;
  RegB rb0, rb1;
  // 32 x 32 x 16 products out of the 16 x 32 fragments: lane l of the operand of rows (or columns)
  // 32 b .. 32 b + 31 and k-half u takes fragment 2 b + (l % 32) / 16, fragment lane l % 16 + 16 (2 u + l / 32)
  const int fr_t = (lane & 31) >> 4, fr_l = (lane & 15) + 16 * (lane >> 5);
  // operand row start (elements) of each of this thread's four load pieces, or -1 past the last row;
  // resolved once, before the loop
  int a_row0[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = m0 + ((tid + 256 * q) >> 3);
    a_row0[q] = row < M ? gemm_a_row(g, row) * g.lda : -1;
  }
  // Load offsets are fixed per lane for the whole loop and a stage adds a wave-uniform amount (fewer
  // address instructions per load). Activations: the byte offset of the piece at the first stage, and the
  // number of k-steps its row still has from there (beyond them, and for rows past M, the load takes an
  // out-of-range offset and returns zeros). Weights (bf16): the fragment's offset inside the column
  // group's eight tiles, from a descriptor based at the group's first tile (so 32-bit offsets suffice for
  // any weight size), plus the k-step (1 KiB) as the scalar offset.
  uint32_t a_off[4];
  int a_lim[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int seg = (tid + 256 * q) & 7;
    a_off[q] = a_row0[q] >= 0 ? (uint32_t)((a_row0[q] + (kb + (seg >> 2)) * 32 + 8 * (seg & 3)) * 2) : 0u;
    a_lim[q] = a_row0[q] >= 0 ? ke - kb - (seg >> 2) : -1;
  }
  uint32_t b_off[4];  // [u * 2 + j]
#pragma unroll
  for (int uj = 0; uj < 4; ++uj) {
    const int ntile = min(nt0 + wn * 4 + 2 * (uj & 1) + fr_t, Nt - 1);
    b_off[uj] = (uint32_t)(((ntile - nt0) * Ks * 64 + fr_l + 32 * (uj >> 1)) * 16);
  }
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)g.Wp_raw + (size_t)nt0 * Ks * 1024), (short)0, 0x7ffffff0, 0x00020000);
  auto gload_a1 = [&](RegA& r, int st, int q) {
    const uint32_t off = 2 * st < a_lim[q] ? a_off[q] + 128u * st : 0x7ffffff0u;
    r[q] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, off, 0, 0));
  };
  auto gload_b1 = [&](RegB& r, int st, int idx) {  // idx = (ks * 2 + u) * 2 + j
    const int ks = idx >> 2, u = (idx >> 1) & 1, j = idx & 1;
    const int ntile = min(nt0 + wn * 4 + 2 * j + fr_t, Nt - 1);
    if constexpr (F8 != 0) {
      if (ks == 0) {  // one load brings both k-steps of the stage (kb and 2 st are even)
        const int pr = min(kb + 2 * st, Ks - 1) >> 1;
        r[u * 2 + j] = W8[((size_t)ntile * Ks2 + pr) * 64 + fr_l + 32 * u];
      }
    } else {
      const int kstep = min(kb + 2 * st + ks, Ks - 1);
      r[idx] = __builtin_bit_cast(bf16x8_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, b_off[u * 2 + j], kstep * 1024, 0));
    }
  };
  auto gload_a = [&](RegA& r, int st) {
#pragma unroll
    for (int q = 0; q < 4; ++q) gload_a1(r, st, q);
  };
  auto gload_b = [&](RegB& r, int st) {
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) gload_b1(r, st, idx);
  };
  auto sstore = [&](const RegA& r, int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int p = tid + 256 * q;
      const int arow = p >> 3, seg = p & 7;
      As[buf][seg >> 2][arow >> 4][asw((arow & 15) + 16 * (seg & 3))] = r[q];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // four groups (k-step, k-half) of four products; each group first reads the next group's A fragments
  // from LDS and issues three of the 12 global loads of a later stage (one activation piece, two weight
  // fragments), so the vector-memory path works while the products run instead of before them
  auto compute_load = [&](int buf, const RegB& rb, RegA& ra_next, int st_a, RegB& rb_next, int st_b) {
    bf16x8_t af[2], an[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) af[i] = As[buf][0][wm * 4 + 2 * i + fr_t][asw(fr_l)];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int ks = gi >> 1, u = gi & 1;
      if (gi < 3) {
        const int ks1 = (gi + 1) >> 1, u1 = (gi + 1) & 1;
#pragma unroll
        for (int i = 0; i < 2; ++i) an[i] = As[buf][ks1][wm * 4 + 2 * i + fr_t][asw(fr_l + 32 * u1)];
      }
      gload_a1(ra_next, st_a, gi);
      gload_b1(rb_next, st_b, 2 * gi);
      gload_b1(rb_next, st_b, 2 * gi + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8_t bw;
        if constexpr (F8 != 0) {
          const uint4 q = rb[u * 2 + j];
          bw = fp8x8_to_bf16x8(ks ? make_uint2(q.z, q.w) : make_uint2(q.x, q.y));
        } else {
          bw = rb[(ks * 2 + u) * 2 + j];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bw, acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (gi < 3) {
        af[0] = an[0];
        af[1] = an[1];
      }
    }
  };

  RowScale<256> rs;
  if (AM == A_NORM && !SPLIT) rs.start(g, m0, tid);
  // activations run two stages ahead (register set, then LDS buffer), weights one stage ahead
  gload_a(ra0, 0);
  gload_b(rb0, 0);
  gload_a(ra1, 1);
  sstore(ra0, 0);
  __syncthreads();
  for (int st = 0; st < nstage; st += 2) {
    // loads past the end (stages nstage, nstage + 1) read zeros / valid clamped weights and are unused
    compute_load(0, rb0, ra0, st + 2, rb1, st + 1);
    sstore(ra1, 1);
    __syncthreads();
    compute_load(1, rb1, ra1, st + 3, rb0, st + 2);
    sstore(ra0, 0);
    __syncthreads();
  }

  // product tile -> LDS. Lane l holds, for e = 0..15, row 8 (e / 4) + 4 (l / 32) + e % 4 of column l % 32 of
  // each 32 x 32 block; the column of local row R is stored at col ^ swz(R), swz(R) = 32 ((R >> 2) & 1), so
  // the two lane halves (rows 4 apart) write different banks.
  {
    const int c = lane & 31, hq = lane >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = 64 * wm + 32 * i + 8 * (e >> 2) + 4 * hq + (e & 3);
          const int col = (64 * wn + 32 * j + c) ^ (hq << 5);
          Cs[row * BN + col] =
              F8 ? acc[i][j][e] * g.wscale[min(nt0 * 16 + 64 * wn + 32 * j + c, Nt * 16 - 1)] : acc[i][j][e];
        }
  }
  // 1 / RMS per row (a K-split product leaves the row scale to the reduce kernel)
  if (AM == A_NORM && !SPLIT) rs.finish(g, s_inv, tid);
  __syncthreads();

  if (SPLIT) tile_epilogue<EPI_PARTIAL, false>(g, Cs, s_inv, m0, nt0, ng);
  else tile_epilogue<EP, AM == A_NORM>(g, Cs, s_inv, m0, nt0, ng);
}

// Vocabulary projection above 128 rows (bound by the bf16 MFMA rate), and gate/up where it pays: 128 x 64 NWV
// workgroup tiles (NWV 8: 128 x 512, one workgroup per compute unit; NWV 4: 128 x 256, two), NWV waves side
// by side, each 128 rows x 64 columns (4 x 2 blocks of v_mfma_f32_32x32x16_bf16). Each weight fragment is
// used by exactly one wave, so weights go from the packed fragments straight into that wave's registers
// (16-byte lane loads in operand order), two k-steps ahead; the activations, used by every wave, go from
// memory straight into LDS with buffer loads that write LDS (one 1 KiB wave load per 16 x 32 fragment, in the
// order the operand reads use, so the reads are lane-linear 16-byte chunks; zeros past the last row) through
// three k-step buffers. Per 32-deep k-step a compute unit then moves 40 (NWV 8) or 48 KiB (NWV 4) through its
// vector-memory path and 72 or 80 KiB through LDS for 128 products per SIMD. Workgroups are ordered XCD-aware
// as in the 128 x 128 kernel (a weight column group leaves HBM once; its other row blocks hit the XCD's L2).
// The product goes through LDS as 128 x 128 quarters, QP at a time, into the shared epilogue (each quarter's
// run by four waves).
template <int AM, int EP, int NWV, int NS>
__global__ __launch_bounds__(NWV * 64) void gemm_wide_kernel(GemmArgs g) {
  constexpr int BM = 128;
  constexpr int TW = 4 * NWV;               // 16-column tiles per workgroup (64 columns per wave)
  constexpr int QP = NWV / 4;               // 128 x 128 quarters per epilogue pass
  constexpr int AD = 8 / NWV;               // activation fragments each wave moves per k-step
  constexpr int SB = 8 * 1024;              // bytes per k-step activation buffer (8 fragments)
  constexpr int SMEM = QP * 128 * 128 * 4;  // the epilogue's 128 x 128 fp32 quarters
  // NS k-step buffers and weight register sets: loads run NS - 1 k-steps ahead
  static_assert(NS * SB <= SMEM, "k-step buffers exceed the epilogue area");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  __shared__ float s_inv[BM];

  const int M = g.M, Ks = g.Ks, Nt = g.Nt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // columns 64 wave .. + 63 of the tile
  const int nwide = (Nt + TW - 1) / TW;     // column groups of TW tiles
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int gw = (slot / g.mblocks) * 8 + xcd;
  if (gw >= nwide) return;
  const int m0 = (slot % g.mblocks) * BM;
  const int nt0 = gw * TW;                  // first 16-column tile

  // operand lane l of 32 rows (or columns) 32 b .. + 31, k-half u: fragment 2 b + (l % 32) / 16, fragment
  // lane l % 16 + 16 (2 u + l / 32)
  const int fr_t = (lane & 31) >> 4, fr_l = (lane & 15) + 16 * (lane >> 5);
  // weights: load (j, u) of a k-step brings column block j, k-half u of this wave's 64 columns (fragment
  // tile nt0 + 4 wave + 2 j + fr_t); tiles past the last one read zeros (descriptor bound)
  const int ntw = min(TW, Nt - nt0);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)g.Wp_raw + (size_t)nt0 * Ks * 1024), (short)0, ntw * Ks * 1024, 0x00020000);
  uint32_t w_off[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int u = 0; u < 2; ++u) w_off[j][u] = (uint32_t)(((4 * wave + 2 * j + fr_t) * Ks * 64 + fr_l + 32 * u) * 16);
  typedef bf16x8_t RegW[4];  // [2 j + u]
  auto wload = [&](RegW& r, int ks) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        r[2 * j + u] =
            __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_off[j][u], ks * 1024, 0));
  };
  // activations: wave w moves fragment w (rows m0 + 16 w .. + 15; fragment lane l holds row l % 16, k
  // elements 8 (l / 16) .. + 7). The load is inline assembly so that the compiler, which does not see it
  // write LDS, does not wait for it before every fragment read; the explicit waits below order it.
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  i32x4_t a_rsrc;
  {
    const uint64_t a = (uint64_t)(uintptr_t)g.A;
    a_rsrc.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    a_rsrc.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    a_rsrc.z = __builtin_amdgcn_readfirstlane(gemm_a_rows(g) * g.lda * 2);
    a_rsrc.w = __builtin_amdgcn_readfirstlane(0x00020000);
  }
  // wave w moves activation fragments w + NWV q (q < AD)
  bool a_ok[AD];
  uint32_t a_off[AD];
#pragma unroll
  for (int q = 0; q < AD; ++q) {
    const int arow = m0 + 16 * (wave + NWV * q) + (lane & 15);
    a_ok[q] = arow < M;
    a_off[q] = a_ok[q] ? (uint32_t)((gemm_a_row(g, arow) * g.lda + 8 * (lane >> 4)) * 2) : 0x7ffffff0u;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  auto adma = [&](int ks, int buf) {  // k-steps past the last one read zeros
#pragma unroll
    for (int q = 0; q < AD; ++q) {
      const uint32_t aoff = a_ok[q] && ks < Ks ? a_off[q] + 64u * ks : 0x7ffffff0u;
      const uint32_t m0a = lds_base + (uint32_t)(buf * SB + (wave + NWV * q) * 1024);
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(aoff), "s"(a_rsrc), "{m0}"(m0a) : "memory");
    }
  };
  const int a_lane = (fr_t * 64 + fr_l) * 16;  // row block i: + 2048 i; k-half 1: + 512

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // k-step ks (its weights in wr, its activations in buffer ks % NS): this wave's loads of ks are done once
  // only those of the next NS - 2 k-steps (four weight loads, then AD activation loads, each) may remain,
  // and the barrier then covers every wave's activation load of ks and every wave's reads of ks - 1, whose
  // buffer takes the activations of ks + NS - 1. The loop runs a multiple of NS k-steps with every load
  // unconditional, so the compiler's own wait counts for the weight registers stay exact; k-steps past the
  // last one multiply zero activations (their weight loads repeat the last k-step)
  auto step = [&](int ks, const RegW& wr, RegW& wnext) {
    __builtin_amdgcn_s_waitcnt(0x0070 | ((NS - 2) * (4 + AD)));  // vmcnt((NS - 2)(4 + AD)) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    wload(wnext, min(ks + NS - 1, Ks - 1));
    adma(ks + NS - 1, (ks + NS - 1) % NS);
    const char* b = smem + (ks % NS) * SB + a_lane;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8_t af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8_t*)(b + i * 2048 + u * 512);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], wr[2 * j + u], acc[i][j], 0, 0, 0);
    }
  };

  RowScale<NWV * 64> rs;
  if (AM == A_NORM) rs.start(g, m0, tid);
  RegW w[NS];
#pragma unroll
  for (int q = 0; q < NS - 1; ++q) {
    wload(w[q], min(q, Ks - 1));
    adma(q, q);
  }
  const int nsteps = (Ks + NS - 1) / NS * NS;
  for (int ks = 0; ks < nsteps; ks += NS) {
#pragma unroll
    for (int q = 0; q < NS; ++q) step(ks + q, w[q], w[(q + NS - 1) % NS]);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // the loads of the k-steps past the loop have landed

  if (AM == A_NORM) rs.finish(g, s_inv, tid);  // 1 / RMS per row
  // two passes of QP 128 x 128 quarters: quarter QP p + s (columns 128 (QP p + s) ..) is held by waves
  // 2 (QP p + s) and 2 (QP p + s) + 1 and goes to LDS quarter s (column XOR-swizzle as in the 128 x 128
  // kernel), then waves 4 s .. 4 s + 3 run its epilogue
  const int c = lane & 31, hq = lane >> 5;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    __syncthreads();  // the k-step buffers (or the previous pass's quarters) are no longer read
    if ((wave >> 1) / QP == p) {
      float* C = (float*)smem + ((wave >> 1) % QP) * 128 * 128;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = 32 * i + 8 * (e >> 2) + 4 * hq + (e & 3);
            const int col = (64 * (wave & 1) + 32 * j + c) ^ (hq << 5);
            C[row * 128 + col] = acc[i][j][e];
          }
    }
    __syncthreads();
    const int s = wave >> 2;
    const int ng = nt0 / 8 + QP * p + s;
    if (ng < g.ngroups)
      tile_epilogue<EP, AM == A_NORM>(g, (const float*)smem + s * 128 * 128, s_inv, m0, ng * 8, ng, 0, 128, tid & 255);
  }
}

// the fixed-order sum of the K-split partials of rows [RS y, RS y + RS) of one 128 x 128 tile
// (y = blockIdx.y), then the epilogue of those rows. SCALE: the operand was normalised and the partials
// are unscaled; each row's 1/RMS comes from the producer's partial sums of squares, whose loads are
// issued before the partials' so that both wait on memory once (256 / RS threads per row). RS = 4 for the
// products of at most 128 rows and for the row build (whose epilogue writes every request's placeholder
// rows too): four times the workgroups for the same rows.
template <int EP, bool SCALE, int RS = 16>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(GemmArgs g) {
  constexpr int BN = 128;
  constexpr int TPR = 256 / RS;  // threads per row of the row scale
  __shared__ __attribute__((aligned(16))) float Cl[RS * BN];
  __shared__ float s_il[RS];
  const int M = g.M, N = g.N;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int ng = (slot / g.mblocks) * 8 + xcd;
  if (ng >= g.ngroups) return;
  const int m0 = (slot % g.mblocks) * 128;
  const int rbeg = RS * blockIdx.y;
  if (m0 + rbeg >= M) return;
  float* Cs = Cl - rbeg * BN;  // tile-row indexing: rows rbeg .. rbeg + RS - 1 live in Cl
  // SCALE: TPR threads per row, partials h, h + TPR, ... (eight per thread per pass)
  const int sr = threadIdx.x / TPR, sh = threadIdx.x % TPR;
  float sv[8];
  const float* ssrc = nullptr;
  if (SCALE) {
    const int m = m0 + rbeg + sr;
    if (m < M) ssrc = g.ssq_in + (size_t)gemm_a_row(g, m) * g.nssq;
#pragma unroll
    for (int u = 0; u < 8; ++u) sv[u] = ssrc && sh + TPR * u < g.nssq ? ssrc[sh + TPR * u] : 0.f;
  }
  const int nt0 = ng * 8;
  const int n0 = nt0 * 16;
  const bool vec = (N & 3) == 0;
  for (int q = threadIdx.x; q < RS * BN / 4; q += 256) {
    const int rl = rbeg + (q >> 5), c0 = 4 * (q & 31);
    const int m = m0 + rl, n = n0 + c0;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m < M && vec && n + 3 < N) {
      // four partials' loads in flight at a time; added in split order
      const float* src = g.part + (size_t)m * N + n;
      const size_t stride = (size_t)M * N;
      int k = 0;
      for (; k + 4 <= g.ksplit; k += 4) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const float4*)(src + (k + u) * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
        }
      }
      for (; k < g.ksplit; ++k) {
        const float4 v = *(const float4*)(src + k * stride);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
      }
    } else if (m < M) {
      for (int k = 0; k < g.ksplit; ++k) {
        const float* src = g.part + ((size_t)k * M + m) * N + n;
        {
          if (n < N) acc.x += src[0];
          if (n + 1 < N) acc.y += src[1];
          if (n + 2 < N) acc.z += src[2];
          if (n + 3 < N) acc.w += src[3];
        }
      }
    }
    *(float4*)&Cs[rl * BN + (c0 ^ (((rl >> 2) & 1) << 5))] = acc;
  }
  if (SCALE) {
    float st = ((sv[0] + sv[1]) + (sv[2] + sv[3])) + ((sv[4] + sv[5]) + (sv[6] + sv[7]));
    for (int i0 = sh + 8 * TPR; ssrc && i0 < g.nssq; i0 += TPR) st += ssrc[i0];  // more than 8 TPR partials
    st = group_sum<TPR>(st);
    if (sh == 0) s_il[sr] = rsqrtf(st / (float)g.Kd + g.eps);
  }
  __syncthreads();
  tile_epilogue<EP, SCALE>(g, Cs, s_il - rbeg, m0, nt0, ng, rbeg, rbeg + RS);
}

template <int EP, bool SCALE>
__device__ void tile_epilogue(const GemmArgs& g, const float* Cs, const float* s_inv, int m0, int nt0, int ng,
                              int rbeg, int rend, int etid) {
  constexpr int BN = 128;
  const int M = g.M, N = g.N, Nt = g.Nt;
  // 256 threads run the epilogue (etid: the caller's thread index among them; default threadIdx.x)
  const int tid = etid >= 0 ? etid : (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // 4 consecutive columns [c0, c0 + 4) of local row rl, scaled by 1/RMS for a normalised operand
  auto cload = [&](int rl, int c0) {
    float4 v = *(const float4*)&Cs[rl * BN + (c0 ^ (((rl >> 2) & 1) << 5))];
    if (SCALE) {
      const float s = s_inv[rl];
      v.x *= s; v.y *= s; v.z *= s; v.w *= s;
    }
    return v;
  };
  const int n0 = nt0 * 16;

  if (EP == EPI_PARTIAL) {
    // raw partial tile of K-split blockIdx.y
    const int h = lane & 31;
    const int c0 = 4 * h, n = n0 + c0;
    const size_t pbytes = (size_t)g.ksplit * M * N * 4;
    const __amdgpu_buffer_rsrc_t p_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.part, (short)0, (int)(pbytes < 0x7fffffffu ? pbytes : 0x7fffffffu), 0x00020000);
    for (int rl = rbeg + 2 * wave + (lane >> 5); rl < rend; rl += 8) {
      const int m = m0 + rl;
      if (m >= M) continue;
      const float4 v = cload(rl, c0);
      const size_t idx = ((size_t)blockIdx.y * M + m) * N + n;
      float* dst = g.part + idx;
      if (n + 3 < N && (N & 3) == 0 && pbytes < 0x7fffffffu) {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), p_rsrc, (int)(idx * 4), 0, PE_PART_AUX);
      } else if (n + 3 < N && (N & 3) == 0) {
        *(float4*)dst = v;
      } else {
        if (n < N) dst[0] = v.x;
        if (n + 1 < N) dst[1] = v.y;
        if (n + 2 < N) dst[2] = v.z;
        if (n + 3 < N) dst[3] = v.w;
      }
    }
    return;
  }

  if (EP == EPI_ARGMAX || EP == EPI_RESID || EP == EPI_ROWS) {
    // half a wave per row: lane h (0..31) holds columns 4h..4h+3; 8 rows per pass
    const int h = lane & 31;
    const int c0 = 4 * h, n = n0 + c0;
    for (int rl = rbeg + 2 * wave + (lane >> 5); rl < rend; rl += 8) {
      const int m = m0 + rl;
      const float4 v = cload(rl, c0);
      const float vv[4] = {v.x, v.y, v.z, v.w};
      if (EP == EPI_ARGMAX) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N && am_better(vv[e], n + e, bv, bi)) { bv = vv[e]; bi = n + e; }
        if (g.logits && m < M) {
          float* z = g.logits + (size_t)m * g.ldz;
          if (n + 3 < N && (N & 3) == 0 && (g.ldz & 3) == 0) *(float4*)(z + n) = v;
          else
            for (int e = 0; e < 4; ++e)
              if (n + e < N) z[n + e] = vv[e];
        }
        am_group_reduce<32>(bv, bi);
        if (h == 0 && m < M) {
          g.am_val[(size_t)m * g.ngroups + ng] = bv;
          g.am_idx[(size_t)m * g.ngroups + ng] = bi;
        }
      } else {
        float sq0 = 0.f, sq1 = 0.f;
        if (m < M) {
          float x[4], x1[4];
          float gn[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) gn[e] = n + e < N ? bf16_to_f32(g.gain_next[n + e]) : 0.f;
          if (EP == EPI_RESID) {
            // X += y; XG = bf16(X * gain_next)
            float* xr = g.Xout + (size_t)m * N;
            const bool full = n + 3 < N && (N & 3) == 0;
            if (full) {
              const float4 o = *(const float4*)(xr + n);
              x[0] = o.x + vv[0]; x[1] = o.y + vv[1]; x[2] = o.z + vv[2]; x[3] = o.w + vv[3];
              *(float4*)(xr + n) = make_float4(x[0], x[1], x[2], x[3]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                x[e] = n + e < N ? xr[n + e] + vv[e] : 0.f;
                if (n + e < N) xr[n + e] = x[e];
              }
            }
            bf16_t* xg = g.XGout + (size_t)m * N;
            if (full) {
              uint2 w;
              w.x = (uint32_t)f32_to_bf16(x[0] * gn[0]) | ((uint32_t)f32_to_bf16(x[1] * gn[1]) << 16);
              w.y = (uint32_t)f32_to_bf16(x[2] * gn[2]) | ((uint32_t)f32_to_bf16(x[3] * gn[3]) << 16);
              *(uint2*)(xg + n) = w;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (!full && n + e < N) xg[n + e] = f32_to_bf16(x[e] * gn[e]);
              sq0 += x[e] * x[e];
            }
          } else {
            // m is real row i = m % R of request b = m / R (R = 1 for a plain step): layer row b Kr + i =
            // fc . concat(h) + embed[token] when i < n_real[b], else h_shared + emb_mask; real row 0 also
            // writes the placeholder rows R .. Kr - 1
            const int Kr = g.Kdraft, R = max(g.rows_real, 1);
            const int b = m / R, i = m % R;
            const bool real = i < gemm_n_real(g, b);
            const int tok = g.last_token[m];
            const bool tok_ok = tok >= 0 && tok < g.V;
            if (real && !tok_ok && h == 0 && ng == 0) raise_flag(g.flags, PE_FLAG_TOKEN);
            // concatenated rows keep the embedding half apart (Xe); summed rows add it to the hidden half
            float xe[4], xe1[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool ok = n + e < N;
              xe1[e] = ok ? bf16_to_f32(g.emb_mask[n + e]) : 0.f;
              xe[e] = ok && real && tok_ok ? bf16_to_f32(g.embed[(size_t)tok * N + n + e]) : real ? 0.f : xe1[e];
              x1[e] = ok ? bf16_to_f32(g.h_shared[n + e]) + (g.Xe ? 0.f : xe1[e]) : 0.f;
              x[e] = !ok ? 0.f : real ? vv[e] + (g.Xe ? 0.f : xe[e]) : x1[e];
              sq0 += x[e] * x[e];
              sq1 += x1[e] * x1[e];
            }
            auto put = [&](int lr, const float* src, const float* srce) {  // layer row b Kr + lr
              float* xr = g.Xout + (size_t)(b * Kr + lr) * N;
              bf16_t* xg = g.XGout + (size_t)(b * Kr + lr) * N;
              if (n + 3 < N && (N & 3) == 0) {  // whole 4-column pieces: 16- and 8-byte stores
                *(float4*)(xr + n) = make_float4(src[0], src[1], src[2], src[3]);
                uint2 w;
                w.x = (uint32_t)f32_to_bf16(src[0] * gn[0]) | ((uint32_t)f32_to_bf16(src[1] * gn[1]) << 16);
                w.y = (uint32_t)f32_to_bf16(src[2] * gn[2]) | ((uint32_t)f32_to_bf16(src[3] * gn[3]) << 16);
                *(uint2*)(xg + n) = w;
                if (g.Xe) *(float4*)(g.Xe + (size_t)(b * Kr + lr) * N + n) = make_float4(srce[0], srce[1], srce[2], srce[3]);
                return;
              }
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) {
                  xr[n + e] = src[e];
                  xg[n + e] = f32_to_bf16(src[e] * gn[e]);
                  if (g.Xe) g.Xe[(size_t)(b * Kr + lr) * N + n + e] = srce[e];
                }
            };
            put(i, x, xe);
            if (i == 0)
              for (int j = R; j < Kr; ++j) put(j, x1, xe1);
          }
        }
        // one partial sum of squares per row and 128-column workgroup tile
        sq0 = group_sum<32>(sq0);
        if (EP == EPI_ROWS) sq1 = group_sum<32>(sq1);
        if (h == 0 && m < M) {
          if (EP == EPI_RESID) {
            g.ssq_out[(size_t)m * g.nssq_out + ng] = sq0;
          } else {
            const int Kr = g.Kdraft, R = max(g.rows_real, 1);
            const int b = m / R, i = m % R;
            g.ssq_out[(size_t)(b * Kr + i) * g.nssq_out + ng] = sq0;
            if (i == 0)
              for (int j = R; j < Kr; ++j) g.ssq_out[(size_t)(b * Kr + j) * g.nssq_out + ng] = sq1;
          }
        }
      }
    }
    return;
  }

  // paired epilogues: within 16-column tile t, columns e and 8 + e (e < 8) form pair 8 (nt0 + t) + e.
  // Sixteen threads per row, each taking 4 consecutive pairs (chunk ch: tile ch / 2, e0 = 4 (ch % 2)).
  const int ch = tid & 15;
  const int t = ch >> 1, e0 = 4 * (ch & 1);
  const int nt = nt0 + t;
  for (int rl = rbeg + (tid >> 4); rl < rend; rl += 16) {
    const int m = m0 + rl;
    if (m >= M || nt >= Nt) continue;
    const float4 a4 = cload(rl, 16 * t + e0), b4 = cload(rl, 16 * t + 8 + e0);
    const float x1[4] = {a4.x, a4.y, a4.z, a4.w}, x2[4] = {b4.x, b4.y, b4.z, b4.w};
    if (EP == EPI_SWIGLU) {
      // gate of f = 8 nt + e, up of the same f
      const int f0 = 8 * nt + e0;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (f0 + e < g.F) g.Aout[(size_t)m * g.F + f0 + e] = f32_to_bf16(x1[e] / (1.f + __expf(-x1[e])) * x2[e]);
    } else if (EP == EPI_QKV) {
      // the two halves of RoPE pair ip = 8 tt + e of head u
      const int hd = g.hd, half = hd / 2, tph = hd / 16;
      const int u = nt / tph, tt = nt % tph, ip0 = 8 * tt + e0;
      const int b = m / g.Kdraft, jr = m % g.Kdraft;
      const int pos = g.seq_len[b] + jr;
      const int slot = g.req_slot[b];
      const bool pos_ok = pos >= 0 && pos < g.max_ctx;
      const bool slot_ok = slot >= 0 && slot < g.n_slots;
      if (ch == 0 && ng == 0) {
        if (!pos_ok) raise_flag(g.flags, PE_FLAG_POS);
        if (!slot_ok) raise_flag(g.flags, PE_FLAG_SLOT);
      }
      bf16_t* dst;
      bool rot = true;
      if (u < g.Hq) {
        dst = g.Q + ((size_t)m * g.Hq + u) * hd;
      } else {
        if (!(pos_ok && slot_ok)) continue;
        const bool isv = u >= g.Hq + g.Hkv;
        bf16_t* cache = isv ? g.Vc : g.Kc;
        dst = cache + (((size_t)slot * g.Hkv + (u - g.Hq - (isv ? g.Hkv : 0))) * g.max_ctx + pos) * hd;
        rot = !isv;
      }
      float y1[4], y2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (rot) {
          const float2 cs = g.rope[(size_t)(pos_ok ? pos : 0) * half + ip0 + e];
          y1[e] = x1[e] * cs.x - x2[e] * cs.y;
          y2[e] = x2[e] * cs.x + x1[e] * cs.y;
        } else {
          y1[e] = x1[e];
          y2[e] = x2[e];
        }
      }
      // 4 consecutive bf16 of each half (8-byte stores)
      uint2 w1, w2;
      w1.x = (uint32_t)f32_to_bf16(y1[0]) | ((uint32_t)f32_to_bf16(y1[1]) << 16);
      w1.y = (uint32_t)f32_to_bf16(y1[2]) | ((uint32_t)f32_to_bf16(y1[3]) << 16);
      w2.x = (uint32_t)f32_to_bf16(y2[0]) | ((uint32_t)f32_to_bf16(y2[1]) << 16);
      w2.y = (uint32_t)f32_to_bf16(y2[2]) | ((uint32_t)f32_to_bf16(y2[3]) << 16);
      *(uint2*)(dst + ip0) = w1;
      *(uint2*)(dst + ip0 + half) = w2;
    }
  }
}

// Projections for 9..128 rows: a weight stream with the activations staged once per reduction chunk.
//
// At these row counts every weight byte is used by at most 128 rows, so the product is bound by the weight
// stream. A workgroup covers all rows (RB blocks of 32) and 128 columns; wave w owns columns 32 w ..
// 32 w + 31 and every row, so each weight fragment is loaded by exactly one wave, straight into
// registers, whole chunks (CH k-steps of 32) ahead of its use. The activations of a chunk (32 RB rows x
// 32 CH columns) are loaded once per workgroup with row-contiguous 16-byte reads and stored into one of
// two LDS buffers in fragment order, so a chunk costs a single barrier and no wave waits for another's
// weights. v_mfma_f32_32x32x16_bf16 throughout (lane layout as in the 128 x 128 kernel above).
// The product tile then goes through LDS (same swizzled layout as above) into the shared epilogues; with
// SPLIT the workgroup covers k-steps [blockIdx.y * kper, + kper) and writes an fp32 partial tile that
// gemm_split_reduce_kernel sums in a fixed order.
// F8: E4M3 weight fragment pairs (16 bytes per lane hold two k-steps' codes), converted to the bf16 operand
// in registers; each product column is multiplied by its scale as the tile goes to LDS (so K-split partials
// are already scaled).
template <int AM, int EP, bool SPLIT, int RB, int CH, int NWB, int F8 = 0>
// (three 96-row workgroups fit a compute unit when the compiler keeps to 168 registers: at B 8 K 11 the
// 88-row vocabulary projection 136 -> 131 us; the other row counts were no faster with the hint)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(RB == 3 ? 3 : 1))) void gemm_stream_kernel(
    GemmArgs g) {
  static_assert(!F8 || CH % 2 == 0, "FP8 loads bring k-steps in pairs");
  constexpr int BN = 128;
  constexpr int MTL = 2 * RB;                       // 16-row fragments per chunk k-step
  constexpr int ABUF = CH * MTL * 64;               // bf16x8 slots per LDS buffer
  constexpr int NPIECE = (32 * RB * 4 * CH) / 256;  // 16-byte activation pieces per thread
  static_assert(2 * ABUF * 16 >= 32 * RB * BN * 4, "product tile must fit in the two activation buffers");
  __shared__ __attribute__((aligned(16))) bf16x8_t smem[2 * ABUF];
  __shared__ float s_inv[BN];
  float* Cs = (float*)smem;  // [32 RB][BN] product tile, after the main loop

  const int M = g.M, Ks = g.Ks, Nt = g.Nt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ng = blockIdx.x;
  const int nt0 = ng * 8;
  const int kb = SPLIT ? blockIdx.y * g.kper : 0;
  const int ke = SPLIT ? min(Ks, kb + g.kper) : Ks;
  const int nchunk = (ke - kb + CH - 1) / CH;  // chunks holding this workgroup's k-steps

  // Both operands through raw buffer descriptors: the per-lane part of every offset is fixed for the whole
  // kernel (one register per activation piece, one for the weights) and the chunk / k-step part is
  // wave-uniform (a scalar offset). Out-of-range offsets read zeros without a memory request: activation
  // rows >= M, weight tiles past the last one, and weight k-steps past this workgroup's range (a scalar
  // offset beyond the buffer), so padded k-steps contribute exact zeros.
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, gemm_a_rows(g) * g.lda * 2, 0x00020000);
  const int Kw = F8 ? (Ks + 1) / 2 : Ks;  // 1 KiB weight fragments (FP8: fragment pairs) per tile
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.Wp_raw, (short)0, (int)((uint32_t)Nt * (uint32_t)Kw * 1024u), 0x00020000);
  auto asw = [](int lp) { return lp ^ ((lp >> 4) << 2); };
  const int fr_t = (lane & 31) >> 4, fr_l = (lane & 15) + 16 * (lane >> 5);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int w_lane = fr_t * Kw * 1024 + fr_l * 16;
  const int w_tile = (nt0 + 2 * wv) * Kw * 1024;

  typedef bf16x8_t RegW16[CH][2];
  typedef uint4 RegW8[CH / 2 > 0 ? CH / 2 : 1][2];
  using RegW = std::conditional_t<(F8 != 0), RegW8, RegW16>;
  typedef bf16x8_t RegA[NPIECE];
  // piece p = tid + 256 q: row p / (4 CH), 16-byte segment p % (4 CH) of the chunk's 32 CH columns
  int a_off[NPIECE];
#pragma unroll
  for (int q = 0; q < NPIECE; ++q) {
    const int p = tid + 256 * q;
    const int row = p / (4 * CH), seg = p % (4 * CH);
    a_off[q] = row < M ? (gemm_a_row(g, row) * g.lda + kb * 32 + (seg >> 2) * 32 + 8 * (seg & 3)) * 2 : 0x7ffffff0;
  }
  // activation k-steps past the workgroup's range meet zero weights, so they need no mask
  auto gload_a = [&](RegA& r, int c) {
    const int so = CH * c * 64;
#pragma unroll
    for (int q = 0; q < NPIECE; ++q)
      r[q] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_off[q], so, 0));
  };
  auto sstore = [&](const RegA& r, int buf) {
#pragma unroll
    for (int q = 0; q < NPIECE; ++q) {
      const int p = tid + 256 * q;
      const int row = p / (4 * CH), seg = p % (4 * CH);
      smem[buf * ABUF + ((seg >> 2) * MTL + (row >> 4)) * 64 + asw((row & 15) + 16 * (seg & 3))] = r[q];
    }
  };
  auto gload_w = [&](RegW& r, int c) {
    if constexpr (F8 != 0) {
      // k-steps in pairs (kb, kper and CH are even): pair p holds k-steps 2p and 2p + 1
#pragma unroll
      for (int kp = 0; kp < CH / 2; ++kp) {
        const int kstep = kb + CH * c + 2 * kp;
        const int so = kstep < ke ? w_tile + (kstep >> 1) * 1024 : 0x7ffffff0;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          r[kp][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_lane + 512 * u, so, PE_WNT));
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < CH; ++ks) {
        const int kstep = kb + CH * c + ks;
        const int so = kstep < ke ? w_tile + kstep * 1024 : 0x7ffffff0;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          r[ks][u] =
              __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_lane + 512 * u, so, PE_WNT));
      }
    }
  };

  f32x16_t acc[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  auto compute = [&](int buf, const RegW& r) {
#pragma unroll
    for (int ks = 0; ks < CH; ++ks)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t af[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) af[i] = smem[buf * ABUF + (ks * MTL + 2 * i + fr_t) * 64 + asw(fr_l + 32 * u)];
        bf16x8_t wk;
        if constexpr (F8 != 0) {
          const uint4 q = r[ks / 2][u];
          wk = fp8x8_to_bf16x8(ks & 1 ? make_uint2(q.z, q.w) : make_uint2(q.x, q.y));
        } else {
          wk = r[ks][u];
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], wk, acc[i], 0, 0, 0);
      }
  };

  // Vector-memory loads complete in issue order as far as the wait counter is concerned, so waiting for
  // an activation chunk also waits for every weight load issued before it. Each step therefore stores
  // the activations of the next chunk (loaded earlier) and issues the activation loads for a later chunk
  // BEFORE its weight loads, so the weight loads of the chunks after the current one stay in flight
  // through that wait. Chunk j uses LDS buffer j % 2. Steps past the workgroup's last chunk still issue
  // their (zero) loads and barriers, so that every wait count is static, but skip the products.
  if constexpr (NWB == 3) {
    // weights two chunks ahead (three register sets), activations two chunks ahead (two register sets);
    // at step j: ra[(j + 1) % 2] holds chunk j + 1, ra[j % 2] chunk j + 2, w[j % 3] chunk j
    RegW w0, w1, w2;
    RegA ra0, ra1;
    gload_a(ra0, 0);
    gload_a(ra1, 1);
    gload_w(w0, 0);
    gload_w(w1, 1);
    gload_w(w2, 2);
    sstore(ra0, 0);
    gload_a(ra0, 2);
    __syncthreads();
    auto step = [&](RegA& ra, int sbuf, RegW& w, int j) {
      sstore(ra, sbuf);
      gload_a(ra, j + 3);
      if (j < nchunk) compute(sbuf ^ 1, w);
      gload_w(w, j + 3);
      __syncthreads();
    };
    for (int c = 0; c < nchunk; c += 6) {
      step(ra1, 1, w0, c);
      step(ra0, 0, w1, c + 1);
      step(ra1, 1, w2, c + 2);
      step(ra0, 0, w0, c + 3);
      step(ra1, 1, w1, c + 4);
      step(ra0, 0, w2, c + 5);
    }
  } else {
    // weights one chunk ahead (two register sets), activations one chunk ahead
    RegW w0, w1;
    RegA ra;
    gload_a(ra, 0);
    gload_w(w0, 0);
    sstore(ra, 0);
    gload_a(ra, 1);
    gload_w(w1, 1);
    __syncthreads();
    auto step = [&](int sbuf, RegW& w, int j) {
      sstore(ra, sbuf);
      gload_a(ra, j + 2);
      if (j < nchunk) compute(sbuf ^ 1, w);
      gload_w(w, j + 2);
      __syncthreads();
    };
    for (int c = 0; c < nchunk; c += 2) {
      step(1, w0, c);
      step(0, w1, c + 1);
    }
  }

  // product tile -> LDS (row R's columns XOR-swizzled by 32 ((R >> 2) & 1), as the epilogue reads them)
  {
    const int c = lane & 31, hq = lane >> 5;
    const float wsc = F8 ? g.wscale[min(nt0 * 16 + 32 * wave + c, Nt * 16 - 1)] : 1.f;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 32 * i + 8 * (e >> 2) + 4 * hq + (e & 3);
        Cs[row * BN + ((32 * wave + c) ^ (hq << 5))] = F8 ? acc[i][e] * wsc : acc[i][e];
      }
  }
  if (AM == A_NORM && !SPLIT) {
    // 1 / RMS of each row from the producer's partial sums of squares (up to 512 per row): TPR threads per
    // row, eight loads in flight per thread, partials combined in a fixed order (a K-split product leaves
    // the row scale to the reduce kernel)
    constexpr int TPR = RB == 1 ? 8 : RB == 2 ? 4 : 2;
    const int r = tid / TPR, h = tid % TPR;
    float t = 0.f;
    if (r < M) {
      const float* src = g.ssq_in + (size_t)gemm_a_row(g, r) * g.nssq;
      for (int i0 = h; i0 < g.nssq; i0 += 8 * TPR) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = i0 + u * TPR < g.nssq ? src[i0 + u * TPR] : 0.f;
        t += ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
      }
    }
    t = group_sum<TPR>(t);
    if (h == 0 && r < 32 * RB) s_inv[r] = rsqrtf(t / (float)g.Kd + g.eps);
  }
  __syncthreads();
  if (SPLIT) tile_epilogue<EPI_PARTIAL, false>(g, Cs, s_inv, 0, nt0, ng, 0, 32 * RB);
  else tile_epilogue<EP, AM == A_NORM>(g, Cs, s_inv, 0, nt0, ng, 0, 32 * RB);
}

// Short K-split products of 17..32 rows: every load of the workgroup in flight at once.
//
// A workgroup covers all rows (RB blocks of 32), 32 NWV columns (wave w: columns 32 w .. 32 w + 31) and at
// most GEMM_BURST_KS k-steps (K-split blockIdx.y). With so few k-steps per workgroup, the chunk pipeline of
// the weight-stream kernel waits about one memory latency per chunk; here each wave first moves its share
// of the activations of all k-steps straight into LDS (buffer loads that write LDS, one 1 KiB wave load per
// 16 x 32 fragment, in the order the operand reads use; rows >= M and k-steps past the split read zeros),
// then issues every weight fragment of its columns into registers (two 16-byte lane loads per k-step), and
// only then waits: once for the activations (and a barrier), then per k-step for that k-step's weights,
// which arrive in issue order while the earlier products run. Workgroups take their k-steps in rotated
// orders, so that concurrent ones start at different offsets of the weight tiles. The fp32 product goes
// through LDS (the layout of the 128 x 128 kernel, one 128-column quarter per four waves) into the partial
// epilogue, and gemm_split_reduce_kernel adds the splits in a fixed order and applies a normalised operand's
// row scale. (With 64 or 96 rows the products
// that follow the loads take as long as the loads, and the weight-stream kernel, which overlaps them, is as
// fast or faster; measured.)
template <int AM, int RB, int NWV>
__global__ __launch_bounds__(NWV * 64) void gemm_burst_kernel(GemmArgs g) {
  constexpr int KS = GEMM_BURST_KS;            // k-steps per workgroup (at most)
  constexpr int FR = 2 * RB;                   // 16-row activation fragments per k-step
  constexpr int KW = KS / NWV;                 // k-steps whose activations each wave moves
  constexpr int SMEM = KS * FR * 1024;         // activations of every k-step; later the product quarters
  static_assert(KS % NWV == 0, "every wave moves the activations of the same number of k-steps");
  static_assert(SMEM >= (NWV / 4) * 32 * RB * 128 * 4, "product quarters must fit in the activation area");
  static_assert(2 * KS <= 63 - 0, "weight loads outstanding must fit the vector-memory counter");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int M = g.M, Ks = g.Ks, Nt = g.Nt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt0 = blockIdx.x * 2 * NWV;  // first 16-column tile
  const int kb = blockIdx.y * g.kper;
  const int ke = min(Ks, kb + g.kper);

  // activations: wave w moves every fragment (rows 16 r .. + 15, r < FR) of k-steps w + NWV j (j < KW);
  // fragment lane l holds row l % 16, k elements 8 (l / 16) .. + 7. The per-lane row offsets are resolved
  // before the first load, so that no wait on them separates the loads.
  uint32_t a_off[FR];
#pragma unroll
  for (int r = 0; r < FR; ++r) {
    const int row = 16 * r + (lane & 15);
    a_off[r] = row < M ? (uint32_t)((gemm_a_row(g, row) * g.lda + 8 * (lane >> 4)) * 2) : 0x7ffffff0u;
  }
  typedef int i32x4_t __attribute__((ext_vector_type(4)));
  i32x4_t a_rsrc;
  {
    const uint64_t a = (uint64_t)(uintptr_t)g.A;
    a_rsrc.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    a_rsrc.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    a_rsrc.z = __builtin_amdgcn_readfirstlane(gemm_a_rows(g) * g.lda * 2);
    a_rsrc.w = __builtin_amdgcn_readfirstlane(0x00020000);
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
#pragma unroll
  for (int j = 0; j < KW; ++j) {
    const int s = wave + NWV * j, ks = kb + s;
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      const uint32_t aoff = ks < ke && a_off[r] != 0x7ffffff0u ? a_off[r] + 64u * ks : 0x7ffffff0u;
      const uint32_t m0a = lds_base + (uint32_t)((s * FR + r) * 1024);
      asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(aoff), "s"(a_rsrc), "{m0}"(m0a) : "memory");
    }
  }

  // weights: k-step s, k-half u of this wave's 32 columns (tiles nt0 + 2 w + fr_t); tiles past the last one
  // and k-steps past the split read zeros
  const int fr_t = (lane & 31) >> 4, fr_l = (lane & 15) + 16 * (lane >> 5);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g.Wp_raw, (short)0, (int)((uint32_t)Nt * (uint32_t)Ks * 1024u), 0x00020000);
  const int w_lane = fr_t * Ks * 1024 + fr_l * 16;
  const int w_tile = (nt0 + 2 * wave) * Ks * 1024;
  bf16x8_t wr[KS][2];
  const int rot = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * 5 + blockIdx.y * 3) % KS));  // first k-step
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const int s = (j + rot) % KS;
    const int so = kb + s < ke && nt0 + 2 * wave < Nt ? w_tile + (kb + s) * 1024 : 0x7ffffff0;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      wr[j][u] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_lane + 512 * u, so, PE_WNT));
  }

  f32x16_t acc[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  // this wave's activation loads (issued before its weight loads) and the first k-step's weights have
  // landed once at most the other 2 (KS - 1) weight loads are outstanding; the barrier then covers every
  // wave's activation loads. Later k-steps wait (compiler-counted) for their own weights only.
  constexpr int VM = 2 * (KS - 1);
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0070);  // vmcnt(VM) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  const int a_lane = (fr_t * 64 + fr_l) * 16;  // row block i: + 2048 i; k-half 1: + 512
  const int nk = ke - kb;
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const int s = (j + rot) % KS;
    if (s < nk) {
      const char* b = smem + s * FR * 1024 + a_lane;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t af[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) af[i] = *(const bf16x8_t*)(b + i * 2048 + u * 512);
#pragma unroll
        for (int i = 0; i < RB; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], wr[j][u], acc[i], 0, 0, 0);
      }
    }
  }

  __syncthreads();  // every wave is done reading the activations
  {
    // quarter wave / 4 (columns 128 (wave / 4) ..), row R's columns XOR-swizzled by 32 ((R >> 2) & 1)
    float* Cs = (float*)smem + (wave >> 2) * 32 * RB * 128;
    const int c = lane & 31, hq = lane >> 5;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 32 * i + 8 * (e >> 2) + 4 * hq + (e & 3);
        Cs[row * 128 + ((32 * (wave & 3) + c) ^ (hq << 5))] = acc[i][e];
      }
  }
  __syncthreads();
  const int q = tid >> 8;
  if (nt0 + 8 * q < Nt)
    tile_epilogue<EPI_PARTIAL, false>(g, (const float*)smem + q * 32 * RB * 128, nullptr, 0, nt0 + 8 * q,
                                      nt0 / 8 + q, 0, 32 * RB, tid & 255);
}

template <int RB, int CH, int NWB, int F8 = 0>
static hipError_t launch_stream_rb(const GemmPlan& p, const GemmArgs& a, int a_mode, int epi, hipStream_t st) {
  const dim3 block(256);
  if (p.ksplit > 1) {
    if (!a.part || epi == EPI_ARGMAX) return hipErrorInvalidValue;
    const dim3 grid(p.ngroups, p.ksplit);
    if (a_mode == A_BF16) hipLaunchKernelGGL((gemm_stream_kernel<A_BF16, EPI_PARTIAL, true, RB, CH, NWB, F8>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((gemm_stream_kernel<A_NORM, EPI_PARTIAL, true, RB, CH, NWB, F8>), grid, block, 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid(p.ngroups);
  if (a_mode == A_BF16 && epi == EPI_RESID) hipLaunchKernelGGL((gemm_stream_kernel<A_BF16, EPI_RESID, false, RB, CH, NWB, F8>), grid, block, 0, st, a);
  else if (a_mode == A_BF16 && epi == EPI_ROWS) hipLaunchKernelGGL((gemm_stream_kernel<A_BF16, EPI_ROWS, false, RB, CH, NWB, F8>), grid, block, 0, st, a);
  else if (a_mode == A_NORM && epi == EPI_QKV) hipLaunchKernelGGL((gemm_stream_kernel<A_NORM, EPI_QKV, false, RB, CH, NWB, F8>), grid, block, 0, st, a);
  else if (!F8 && a_mode == A_BF16 && epi == EPI_QKV) hipLaunchKernelGGL((gemm_stream_kernel<A_BF16, EPI_QKV, false, RB, CH, NWB>), grid, block, 0, st, a);
  else if (a_mode == A_NORM && epi == EPI_SWIGLU) hipLaunchKernelGGL((gemm_stream_kernel<A_NORM, EPI_SWIGLU, false, RB, CH, NWB, F8>), grid, block, 0, st, a);
  else if (a_mode == A_NORM && epi == EPI_ARGMAX) hipLaunchKernelGGL((gemm_stream_kernel<A_NORM, EPI_ARGMAX, false, RB, CH, NWB, F8>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// the K-split partials of a weight-stream product: sum and epilogue
// (one 128-row block of at most 128 rows: 4-row slices, four times the workgroups of 16-row ones; measured:
// Qwen B8 K11 552 -> 536 us per draft step, B8 K3 421 -> 401 us, B4 K11 490 -> 463 us; on the 128 x 128
// kernel's products, with several row blocks, 4-row slices changed nothing)
static hipError_t launch_split_reduce(const GemmPlan& p, const GemmArgs& a, int a_mode, int epi, hipStream_t st) {
  const dim3 rgrid(8 * ((p.ngroups + 7) / 8), 32);  // 4-row slices of each 128-column tile
  const dim3 block(256);
  if (epi == EPI_RESID && a_mode == A_BF16) hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_RESID, false, 4>), rgrid, block, 0, st, a);
  else if (epi == EPI_ROWS && a_mode == A_BF16) hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_ROWS, false, 4>), rgrid, block, 0, st, a);
  else if (epi == EPI_QKV && a_mode == A_NORM) hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_QKV, true, 4>), rgrid, block, 0, st, a);
  else if (epi == EPI_QKV && a_mode == A_BF16) hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_QKV, false, 4>), rgrid, block, 0, st, a);
  else if (epi == EPI_SWIGLU && a_mode == A_NORM) hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_SWIGLU, true, 4>), rgrid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int RB>
static hipError_t launch_burst_rb(const GemmPlan& p, const GemmArgs& a, int a_mode, hipStream_t st) {
  const int nb = (p.Nt + 2 * p.burst - 1) / (2 * p.burst);
  const dim3 grid(nb, p.ksplit);
  if (p.burst == 8) {
    if (a_mode == A_BF16) hipLaunchKernelGGL((gemm_burst_kernel<A_BF16, RB, 8>), grid, dim3(512), 0, st, a);
    else hipLaunchKernelGGL((gemm_burst_kernel<A_NORM, RB, 8>), grid, dim3(512), 0, st, a);
  } else {
    if (a_mode == A_BF16) hipLaunchKernelGGL((gemm_burst_kernel<A_BF16, RB, 4>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((gemm_burst_kernel<A_NORM, RB, 4>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

static hipError_t launch_gemm_stream(const GemmPlan& p, const GemmArgs& a, int a_mode, int epi, hipStream_t st) {
  if (a.M < 1 || a.M > 128) return hipErrorInvalidValue;
  if (p.burst && !a.wscale) {
    if (p.ksplit <= 1 || p.kper > GEMM_BURST_KS || !a.part || epi == EPI_ARGMAX) return hipErrorInvalidValue;
    if (a.M > 32) return hipErrorInvalidValue;
    const hipError_t e = launch_burst_rb<1>(p, a, a_mode, st);
    if (e != hipSuccess) return e;
    return launch_split_reduce(p, a, a_mode, epi, st);
  }
  if (a.wscale) {  // FP8 weights
    hipError_t e;
    if (a.M <= 32) e = launch_stream_rb<1, GEMM_STREAM_CH, 2, 1>(p, a, a_mode, epi, st);
    else if (a.M <= 64) e = launch_stream_rb<2, GEMM_STREAM_CH, 2, 1>(p, a, a_mode, epi, st);
    else if (a.M <= 96) e = launch_stream_rb<3, GEMM_STREAM_CH, 2, 1>(p, a, a_mode, epi, st);
    else e = launch_stream_rb<4, GEMM_STREAM_CH, 2, 1>(p, a, a_mode, epi, st);
    if (e != hipSuccess || p.ksplit <= 1) return e;
    return launch_split_reduce(p, a, a_mode, epi, st);
  }
  // weights one chunk ahead (measured: two chunks ahead, with a six-step unroll, was no faster for the
  // 88-row vocabulary projection and slower for the four-chunk K-split products)
  hipError_t e;
  if (a.M <= 32) e = launch_stream_rb<1, GEMM_STREAM_CH, 2>(p, a, a_mode, epi, st);
  else if (a.M <= 64) e = launch_stream_rb<2, GEMM_STREAM_CH, 2>(p, a, a_mode, epi, st);
  else if (a.M <= 96) e = launch_stream_rb<3, GEMM_STREAM_CH, 2>(p, a, a_mode, epi, st);
  else e = launch_stream_rb<4, GEMM_STREAM_CH, 2>(p, a, a_mode, epi, st);
  if (e != hipSuccess || p.ksplit <= 1) return e;
  return launch_split_reduce(p, a, a_mode, epi, st);
}

template <int F8>
static hipError_t launch_tiled(const GemmPlan& p, const GemmArgs& a, int a_mode, int epi, hipStream_t st) {
  const int tiles = 8 * ((p.ngroups + 7) / 8) * p.mblocks;
  const dim3 block(256);
  if (p.ksplit > 1) {
    if (!a.part || epi == EPI_ARGMAX) return hipErrorInvalidValue;
    const dim3 grid(tiles, p.ksplit);
    if (a_mode == A_BF16) hipLaunchKernelGGL((gemm_tiled_kernel<A_BF16, EPI_PARTIAL, true, F8>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((gemm_tiled_kernel<A_NORM, EPI_PARTIAL, true, F8>), grid, block, 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 rgrid(tiles, 8);  // 16-row slices of each tile
    if (epi == EPI_RESID && a_mode == A_BF16) hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_RESID, false>), rgrid, block, 0, st, a);
    else if (epi == EPI_ROWS && a_mode == A_BF16)  // 4-row slices
      hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_ROWS, false, 4>), dim3(tiles, 32), block, 0, st, a);
    else if (epi == EPI_QKV && a_mode == A_NORM) hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_QKV, true>), rgrid, block, 0, st, a);
    else if (epi == EPI_QKV && a_mode == A_BF16) hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_QKV, false>), rgrid, block, 0, st, a);
    else if (epi == EPI_SWIGLU && a_mode == A_NORM) hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI_SWIGLU, true>), rgrid, block, 0, st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const dim3 grid(tiles);
  if (a_mode == A_BF16 && epi == EPI_RESID) hipLaunchKernelGGL((gemm_tiled_kernel<A_BF16, EPI_RESID, false, F8>), grid, block, 0, st, a);
  else if (a_mode == A_BF16 && epi == EPI_ROWS) hipLaunchKernelGGL((gemm_tiled_kernel<A_BF16, EPI_ROWS, false, F8>), grid, block, 0, st, a);
  else if (a_mode == A_NORM && epi == EPI_QKV) hipLaunchKernelGGL((gemm_tiled_kernel<A_NORM, EPI_QKV, false, F8>), grid, block, 0, st, a);
  else if (!F8 && a_mode == A_BF16 && epi == EPI_QKV) hipLaunchKernelGGL((gemm_tiled_kernel<A_BF16, EPI_QKV, false>), grid, block, 0, st, a);
  else if (a_mode == A_NORM && epi == EPI_SWIGLU) hipLaunchKernelGGL((gemm_tiled_kernel<A_NORM, EPI_SWIGLU, false, F8>), grid, block, 0, st, a);
  else if (a_mode == A_NORM && epi == EPI_ARGMAX) hipLaunchKernelGGL((gemm_tiled_kernel<A_NORM, EPI_ARGMAX, false, F8>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(const GemmPlan& p, const GemmArgs& a, int a_mode, int epi, hipStream_t st) {
  if (p.tiled == 2) return launch_gemm_stream(p, a, a_mode, epi, st);
  if (p.tiled == 1 && !a.wscale && p.ksplit == 1 && a_mode == A_NORM && epi == EPI_SWIGLU && a.Ks > 64 &&
      (p.Nt + 15) / 16 * p.mblocks >= 256) {
    // gate/up with a long reduction and at least one 128 x 256 tile per compute unit (measured: GPT-OSS
    // B 64 K 10 (90 k-steps, 408 tiles) 123 -> 105 us; Qwen B 128 K 7 (64 k-steps, 384 tiles) 76 -> 79 us,
    // so it stays on the 128 x 128 kernel)
    const int nwide = (p.Nt + 15) / 16;
    if (a.Ks % 3 != 0 && a.Ks % 4 == 0)
      hipLaunchKernelGGL((gemm_wide_kernel<A_NORM, EPI_SWIGLU, 4, 4>), dim3(8 * ((nwide + 7) / 8) * p.mblocks), dim3(256),
                         0, st, a);
    else
      hipLaunchKernelGGL((gemm_wide_kernel<A_NORM, EPI_SWIGLU, 4, 3>), dim3(8 * ((nwide + 7) / 8) * p.mblocks), dim3(256),
                         0, st, a);
    return hipGetLastError();
  }
  if (p.tiled == 3 && !a.wscale && p.ksplit == 1 && a_mode == A_NORM && epi == EPI_ARGMAX) {
    // 8 waves (128 x 512, one workgroup per compute unit) or 4 waves (128 x 256, two per compute unit).
    // Measured LM heads: Qwen (d 2048) B 128 K 7 668 -> 624 us and B 32 K 7 246 -> 222 us with 4 waves,
    // GPT-OSS (d 2880) B 64 K 10 800 -> 811-829 us, so the longer reduction keeps 8
    if (a.Ks <= 64) {
      const int nwide = (p.Nt + 15) / 16;
      if (a.Ks % 3 != 0 && a.Ks % 4 == 0)
        hipLaunchKernelGGL((gemm_wide_kernel<A_NORM, EPI_ARGMAX, 4, 4>), dim3(8 * ((nwide + 7) / 8) * p.mblocks),
                           dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((gemm_wide_kernel<A_NORM, EPI_ARGMAX, 4, 3>), dim3(8 * ((nwide + 7) / 8) * p.mblocks),
                           dim3(256), 0, st, a);
    } else {
      const int nwide = (p.Nt + 31) / 32;
      hipLaunchKernelGGL((gemm_wide_kernel<A_NORM, EPI_ARGMAX, 8, 3>), dim3(8 * ((nwide + 7) / 8) * p.mblocks),
                         dim3(512), 0, st, a);
    }
    return hipGetLastError();
  }
  return a.wscale ? launch_tiled<1>(p, a, a_mode, epi, st) : launch_tiled<0>(p, a, a_mode, epi, st);
}

}  // namespace pe
