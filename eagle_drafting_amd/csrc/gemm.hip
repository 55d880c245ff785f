// Projections of the drafter (fc, QKV, O, gate/up, down, LM head): y = A . W^T, with the neighbouring
// row-wise steps fused into the projection so that a draft step is a short chain of kernels.
//
// Weights are repacked once (pe_init) into 1 KiB MFMA fragments: a wave's B-operand load for one
// 16-column x 32-k tile is one contiguous 1 KiB read (64 lanes x 16 B). The repack may also permute the
// output columns inside a 16-column tile so that values one epilogue combines sit in the same tile:
// the two halves of every RoPE pair (QKV) and each gate/up pair (SwiGLU).
//
// A workgroup owns NT 16-column tiles and one block of MT*16 rows over the WHOLE reduction dimension;
// its NW waves split the k range (NW/NT parts), each accumulating MT 16x16 fp32 tiles with
// v_mfma_f32_16x16x32_bf16, and the parts are summed through LDS in a fixed order. No workgroup depends
// on another, so results are deterministic and no device-wide synchronisation is needed.
// The A operand is a bf16 matrix that every wave reads straight from global memory into MFMA fragments
// (it is tiny: M = B*K rows, and stays in cache). A normalised operand is bf16(x * g), written by the kernel that last
// updated the residual stream x together with per-16-column sums of squares; RMSNorm is a per-row scale,
// so the epilogue multiplies each product row by 1/RMS(x): y = (x * g / rms) . W^T = ((x * g) . W^T) / rms.
//
// MFMA lane layout (16x16x32, wave64): A lane l holds A[l%16][k-group l/16] (8 values), B lane l holds
// B[k-group l/16][l%16], D lane l holds D[4(l/16)+r][l%16], r = 0..3. A and B use the same k grouping,
// so any consistent assignment of the 32 k values to (group, element) gives the same sum.
#include "common.h"
#include "kernels.h"

namespace pe {

// Source row of packed row r (0..15) of tile t.
__device__ __forceinline__ int pack_src_row(int mode, int t, int r, int hd, int* which) {
  *which = 0;
  if (mode == PACK_PAIRS) {  // tile holds 8 RoPE pairs of one head: first halves, then second halves
    const int tph = hd / 16, h = t / tph, tt = t % tph;
    return h * hd + (r < 8 ? 8 * tt + r : hd / 2 + 8 * tt + (r - 8));
  }
  if (mode == PACK_GATEUP) {  // tile holds gate rows 8t..8t+7, then up rows 8t..8t+7
    *which = r < 8 ? 0 : 1;
    return 8 * t + (r & 7);
  }
  return 16 * t + r;
}

__global__ __launch_bounds__(256) void pack_bf16_kernel(const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
                                                        int N, int Kd, bf16x8_t* __restrict__ dst, int Nt, int Ks,
                                                        int mode, int hd) {
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)Nt * Ks * 64;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const size_t frag = gid >> 6;
  const int s = (int)(frag % Ks);
  const int t = (int)(frag / Ks);
  int which = 0, row, col;
  if (mode == PACK_KI4) {
    row = 4 * t + (lane & 3);
    col = 128 * s + 8 * (4 * (lane >> 4) + ((lane >> 2) & 3));
  } else {
    row = pack_src_row(mode, t, lane & 15, hd, &which);
    col = 32 * s + 8 * (lane >> 4);
  }
  const bf16_t* W = which ? W1 : W0;
  bf16x8_t v;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    short x = 0;
    if (row < N && col + e < Kd) x = (short)W[(size_t)row * Kd + col + e];
    v[e] = x;
  }
  dst[frag * 64 + lane] = v;
}

// one wave per packed output column: the largest magnitude of its source row, scale = that / 448
__global__ __launch_bounds__(256) void fp8_scale_kernel(const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
                                                        int N, int Kd, int Nt, int mode, int hd,
                                                        float* __restrict__ scales) {
  const int col = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (col >= Nt * 16) return;
  int which = 0;
  const int row = pack_src_row(mode, col / 16, col % 16, hd, &which);
  const bf16_t* W = which ? W1 : W0;
  float m = 0.f;
  if (row < N)
    for (int k = lane; k < Kd; k += 64) m = fmaxf(m, fabsf(bf16_to_f32(W[(size_t)row * Kd + k])));
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, PE_WAVE));
  if (lane == 0) scales[col] = m > 0.f ? m / 448.f : 1.f;
}

// fragment pair (t, p), lane l: 16 bytes, the 8 codes of k-step 2p then the 8 of k-step 2p + 1, each of
// source row src(t, l % 16), columns 32 s + 8 (l / 16) .. + 7 (zero past Kd): one 16-byte load per lane
// brings two k-steps
__global__ __launch_bounds__(256) void pack_fp8_kernel(const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
                                                       int N, int Kd, uint4* __restrict__ dst, int Nt, int Ks2,
                                                       int mode, int hd, const float* __restrict__ scales) {
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)Nt * Ks2 * 64;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const size_t frag = gid >> 6;
  const int pr = (int)(frag % Ks2);
  const int t = (int)(frag / Ks2);
  int which = 0;
  const int row = pack_src_row(mode, t, lane & 15, hd, &which);
  const bf16_t* W = which ? W1 : W0;
  const float sc = scales[t * 16 + (lane & 15)];
  uint32_t w4[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = 32 * (2 * pr + h) + 8 * (lane >> 4);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = 0.f;
      if (row < N && col + e < Kd) v = bf16_to_f32(W[(size_t)row * Kd + col + e]) / sc;
      x[e] = fminf(fmaxf(v, -448.f), 448.f);  // |w| / s <= 448 already; the clamp only guards rounding
    }
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0u, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], lo, true);
    uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0u, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], hi, true);
    w4[2 * h] = lo;
    w4[2 * h + 1] = hi;
  }
  dst[frag * 64 + lane] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
}

hipError_t launch_pack_fp8(const void* W0, const void* W1, int N, int Kd, int mode, int hd, void* dst, float* scales,
                           hipStream_t st) {
  if (mode == PACK_KI4) return hipErrorInvalidValue;
  const int Nt = mode == PACK_GATEUP ? (2 * N + 15) / 16 : n_tiles(N);
  const int Ks2 = (k_steps(Kd) + 1) / 2;
  hipLaunchKernelGGL(fp8_scale_kernel, dim3((unsigned)((Nt * 16 + 3) / 4)), dim3(256), 0, st, (const bf16_t*)W0,
                     (const bf16_t*)W1, N, Kd, Nt, mode, hd, scales);
  const size_t total = (size_t)Nt * Ks2 * 64;
  hipLaunchKernelGGL(pack_fp8_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, (const bf16_t*)W0,
                     (const bf16_t*)W1, N, Kd, (uint4*)dst, Nt, Ks2, mode, hd, (const float*)scales);
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const void* W0, const void* W1, int N, int Kd, int mode, int hd, void* dst,
                            hipStream_t st) {
  const int Nt = mode == PACK_GATEUP ? (2 * N + 15) / 16 : mode == PACK_KI4 ? n_tiles_ki4(N) : n_tiles(N);
  const int Ks = mode == PACK_KI4 ? k_steps_ki4(Kd) : k_steps(Kd);
  const size_t total = (size_t)Nt * Ks * 64;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, (const bf16_t*)W0,
                     (const bf16_t*)W1, N, Kd, (bf16x8_t*)dst, Nt, Ks, mode, hd);
  return hipGetLastError();
}

GemmPlan plan_gemm(int M, int N, int Kd, bool argmax, bool ki4_ok, bool skinny_only, bool fp8) {
  GemmPlan p;
  const int Ks = k_steps(Kd);
  p.Nt = n_tiles(N);
  p.tiled = 0;
  p.ksplit = 1;
  p.kper = Ks;
  p.ki4 = 0;
  p.burst = 0;
  if (ki4_ok && !argmax && M <= 4 && p.Nt < 256) {
    // up to 4 rows and a narrow output: 4-column tiles (4x the workgroups of 16-column ones, so every
    // compute unit streams weights); 4 or 8 waves split the 128-wide k-steps so that each loads its share
    // in one round of at most 8 (measured: O 4 waves x 8 k-steps 5.9 us, down 8 x 6 8.2 us, 4 x 12 8.8 us)
    p.ki4 = 1;
    p.Nt = n_tiles_ki4(N);
    p.kper = k_steps_ki4(Kd);
    p.MT = 1;
    p.mblocks = 1;
    p.NT = 1;
    p.NW = p.kper > 32 ? 8 : 4;
    p.ngroups = p.Nt;
    return p;
  }
  // (measured: the vocabulary projection is faster in the stream kernel from 9 rows, the layer projections
  // from 17; the stream kernel addresses the packed weights with 32-bit buffer offsets)
  if (!skinny_only && M > (argmax ? 8 : 16) && M <= 128 && (long long)p.Nt * Ks * 1024 < 0x7ff00000LL) {
    // up to 128 rows: the weight-stream kernel (all rows and 128 columns per workgroup, activations staged
    // once per chunk). Narrow or short products split the reduction into whole 16-k-step (four-chunk)
    // pieces, as many as give about 192 workgroups; the split reduce kernel then runs the epilogue.
    // (Measured at 96 rows: two-chunk pieces for 256-384 workgroups were 2-3 % slower per step; taking the
    // split count directly instead of doubling it while the fp32 partials stayed within the weight bytes
    // runs down in 12 pieces instead of 6: Qwen B8 K11 540 -> 531 us, B8 K7 490 -> 481 us per draft step.)
    const int tg = (p.Nt + 7) / 8;
    constexpr int step = 4 * GEMM_STREAM_CH;
    p.tiled = 2;
    p.MT = 8;
    p.NT = 8;
    p.NW = 4;
    p.mblocks = 1;
    p.ngroups = tg;
    if (!argmax && !fp8 && M <= 32 && Ks > GEMM_BURST_KS) {
      // up to 32 rows: K-split on the burst kernel, GEMM_BURST_KS k-steps per workgroup with every load
      // issued at once; 256-column workgroups when 128-column ones would exceed one per compute unit
      // (measured: B 8 K 3 474 -> 454 us and B 4 K 7 467 -> 452 us per draft step; with 64 or 96 rows the
      // weight-stream kernel stays as fast or faster)
      p.ksplit = (Ks + GEMM_BURST_KS - 1) / GEMM_BURST_KS;
      p.kper = GEMM_BURST_KS;
      p.burst = tg * p.ksplit > 256 ? 8 : 4;
      return p;
    }
    if (!argmax) {
      const int want = (192 + tg - 1) / tg;  // splits for about 192 workgroups
      if (want > 1 && Ks >= 2 * step) {
        p.kper = (((Ks + want - 1) / want) + step - 1) / step * step;  // whole 16-k-step pieces
        p.ksplit = (Ks + p.kper - 1) / p.kper;
        if (p.ksplit <= 1) p.kper = Ks;
      }
    }
    return p;
  }
  if (!skinny_only && M > 32) {
    // 128 x 128 tiles read each weight once per 128 rows and each activation once per 128 columns (the
    // skinny kernel re-reads the activations once per 16 columns). Narrow or short products get too few
    // tiles to keep the weight stream going; they split the reduction over workgroups (about 512 in all,
    // at least 8 k-steps each) as long as the fp32 partials stay within the weight bytes
    // (2 ksplit M N 4 <= N Kd 2), and beyond that while the grid does not yet cover the 256 compute units
    // once (many rows, narrow output: the product is bound by the idle units, not by bytes); a second
    // kernel adds the partials and runs the epilogue.
    const int tg = (p.Nt + 7) / 8, tm = (M + 127) / 128;
    p.tiled = 1;
    p.MT = 8;
    p.NT = 8;
    p.NW = 4;
    p.mblocks = tm;
    p.ngroups = tg;
    // the vocabulary projection runs on 128 x 512 tiles when that still gives at least two workgroups per
    // compute unit; FP8 weights keep the 128 x 128 kernel
    if (argmax && (long long)((tg + 3) / 4) * tm >= 512) p.tiled = 3;
    if (!argmax) {
      int ks = 1;
      while (tg * tm * ks < 512 && Ks >= 16 * ks && (8LL * ks * M <= Kd || tg * tm * ks < 256)) ks *= 2;
      // a two-way split that leaves room for exactly one more split in the first residency round takes
      // it (measured: GPT-OSS B 64 K 10, 138 tiles: O 54 -> 50 us, down 86 -> 76 us with three splits;
      // filling the round further lost 2-16 % at B 128 and B 32)
      if (ks == 2 && tg * tm * 3 <= 512 && tg * tm * 4 > 512 && Ks >= 48) ks = 3;
      if (ks > 1) {
        p.kper = (((Ks + ks - 1) / ks) + 3) & ~3;
        p.ksplit = (Ks + p.kper - 1) / p.kper;
      }
    }
    return p;
  }
  p.MT = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
  p.mblocks = (M + 16 * p.MT - 1) / (16 * p.MT);
  if (argmax) {
    // vocabulary projection: up to 16 rows, one 16-column tile per workgroup with 8 waves splitting k
    // (about 9.5 k short workgroups balance across the compute units better than fewer long ones);
    // more rows keep four tiles per workgroup, one wave each
    p.NT = p.MT == 1 ? 1 : 4;
    p.NW = p.MT == 1 ? 8 : 4;
  } else {
    p.NT = 1;
    // about one residency round of waves in total (~4096), each wave streaming at least 8 k-steps and
    // not a partial second round of 8 (measured: 24 k-steps per wave beat 12, 8 beat 16);
    // the register budget caps NW by MT (LDS for the cross-wave sum is NW * MT KiB)
    const int cap = p.MT == 1 ? 16 : p.MT == 2 ? 8 : 4;
    const int groups = p.Nt * p.mblocks;
    int nw = 4;
    auto per_wave = [&](int w) { return Ks / w; };
    while (nw < cap && groups * nw * 2 <= 4096 && per_wave(2 * nw) >= 8 &&
           !(per_wave(2 * nw) > 8 && per_wave(2 * nw) < 16))
      nw *= 2;
    if (p.MT == 1) {
      // one 16-row block: the most waves whose k share is whole 8-step load rounds (measured at 4 rows:
      // QKV and gate/up 8 waves x 8 k-steps beat 4 x 16 and 16 x 4; down 8 x 24 beat 16 x 12)
      for (int w = cap; w >= 4; w /= 2)
        if (((Ks + w - 1) / w) % 8 == 0) {
          nw = w;
          break;
        }
    }
    p.NW = nw;
  }
  p.ngroups = (p.Nt + p.NT - 1) / p.NT;
  return p;
}

template <int MT>
struct KChunk {
  static constexpr int value = MT <= 2 ? 8 : (MT == 4 ? 4 : 2);
};

// KI: PACK_KI4 weights (MT == 1, NT == 1, M <= 4): 4-column tiles, activation row m at MFMA rows m + 4h
// F8: E4M3 weight fragments (8 bytes per lane) with per-column scales applied in the epilogue
template <int MT, int NW, int NT, int AM, int EP, int KI, int F8 = 0>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(GemmArgs g) {
  static_assert(!KI || (MT == 1 && NT == 1 && (EP == EPI_RESID || EP == EPI_ROWS)), "KI4 layout: residual producers");
  static_assert(!(KI && F8), "FP8 weights use the 16-column layout");
  constexpr int CW = KI ? 4 : 16;  // output columns per tile
  constexpr int KP = NW / NT;            // k parts
  constexpr int KC = KChunk<MT>::value;  // k-steps loaded per round
  constexpr int NTH = NW * 64;
  __shared__ float s_red[NW * MT * 256];
  __shared__ float s_inv[MT * 16];

  const int M = g.M, N = g.N, Ks = g.Ks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tl = wave % NT, kp = wave / NT;
  const int nt = blockIdx.x * NT + tl;
  const int ntc = min(nt, g.Nt - 1);  // clamped tile: a wave past the last tile streams a valid one, unused
  const int m0 = blockIdx.y * MT * 16;
  // (FP8: k parts start on even k-steps, since one 16-byte load brings a pair of k-steps)
  const int kps = F8 ? (((Ks + KP - 1) / KP + 1) & ~1) : (Ks + KP - 1) / KP;
  const int s_begin = kp * kps;
  const int s_end = min(Ks, s_begin + kps);
  const int nrows = min(MT * 16, M - m0);

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bf16x8_t* wsrc = (const bf16x8_t*)g.Wp_raw + (size_t)ntc * Ks * 64 + lane;
  const int Ks2 = (Ks + 1) / 2;
  const uint4* wsrc8 = (const uint4*)g.Wp_raw + (size_t)ntc * Ks2 * 64 + lane;

  // Main loop, KC k-steps per round. Every load is unconditional (addresses clamped into range; rows >= M
  // and k-steps past the split are computed but never used), so the weight loads of a round are all in
  // flight before the first MFMA waits. The first round is peeled so that its loads are issued before
  // anything else in the kernel.
  // A through a raw buffer descriptor: lanes of padding rows (row >= M) use an out-of-range offset, which
  // returns zeros without any memory request, so only real rows cost bandwidth.
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.A, (short)0, gemm_a_rows(g) * g.lda * 2, 0x00020000);
  bf16x8_t a[KC][MT], b[KC];
  static_assert(KC % 2 == 0, "FP8 loads bring k-steps in pairs");
  uint4 b8[KC / 2];  // FP8: raw codes of two k-steps, converted just before their products (loads stay in flight)
  // each lane's operand row start (elements), or -1 for a padding row; resolved once, before the loop
  int a_row0[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = KI ? lane & 3 : m0 + mt * 16 + (lane & 15);
    a_row0[mt] = row < M ? gemm_a_row(g, row) * g.lda : -1;
  }
  auto load_round = [&](int c0) {
    const int nk = max(1, min(KC, s_end - c0));
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const int ks = min(c0 + min(kk, nk - 1), Ks - 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        int off;
        if (KI) {  // MFMA row m + 4h: activation row m, k chunk 4(lane >> 4) + h of the 128-wide step
          const int h = (lane >> 2) & 3;
          off = a_row0[mt] >= 0 ? (a_row0[mt] + ks * 128 + 8 * (4 * (lane >> 4) + h)) * 2 : 0x7ffffff0;
        } else {
          off = a_row0[mt] >= 0 ? (a_row0[mt] + ks * 32 + 8 * (lane >> 4)) * 2 : 0x7ffffff0;
        }
        a[kk][mt] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, off, 0, 0));
      }
    }
    // weights are read once per launch: non-temporal loads (measured on a streaming read: 7.0 TB/s against
    // 6.3 TB/s with plain loads)
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    if (F8) {
#pragma unroll
      for (int kk = 0; kk < KC; kk += 2)
        b8[kk / 2] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
            (const u32x4_t*)(wsrc8 + (size_t)(min(c0 + min(kk, nk - 1), Ks - 1) >> 1) * 64)));
    } else {
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) b[kk] = __builtin_nontemporal_load(wsrc + (size_t)min(c0 + min(kk, nk - 1), Ks - 1) * 64);
    }
  };
  auto mma_round = [&](int c0) {
    const int nk = min(KC, s_end - c0);
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      if (kk < nk) {
        const bf16x8_t bk = F8 ? fp8x8_to_bf16x8(kk & 1 ? make_uint2(b8[kk / 2].z, b8[kk / 2].w)
                                                       : make_uint2(b8[kk / 2].x, b8[kk / 2].y))
                               : b[kk];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk][mt], bk, acc[mt], 0, 0, 0);
      }
    }
  };
  load_round(s_begin);

  // Side inputs of the epilogue, issued right after the first weight round so that their latency overlaps it.
  // Loads are unconditional, with indices clamped into range (values that are not needed are ignored),
  // so that no branch forces the weight loads to wait for them.
  // (up to 512 partials: a producer on 4-column tiles writes d / 4 of them)
  float pre_ssq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (AM == A_NORM) {
    const float* src = g.ssq_in + (size_t)gemm_a_row(g, m0 + min(wave, nrows - 1)) * g.nssq;
#pragma unroll
    for (int i = 0; i < 8; ++i) pre_ssq[i] = src[min(lane + 64 * i, g.nssq - 1)];  // masked when used
  }
  const int pr16 = min((int)threadIdx.x / CW, nrows - 1);  // first epilogue row of a CW-wide epilogue
  const int pr8 = min((int)threadIdx.x >> 3, nrows - 1);   // ... of an 8-wide epilogue
  float pre_x = 0.f;
  if (EP == EPI_RESID) pre_x = g.Xout[(size_t)(m0 + pr16) * N + min(ntc * CW + (int)(threadIdx.x % CW), N - 1)];
  int pre_seq = 0, pre_slot = 0;  // raw values; arithmetic on them waits until the epilogue
  if (EP == EPI_QKV) {
    pre_seq = g.seq_len[(m0 + pr8) / g.Kdraft];
    pre_slot = g.req_slot[(m0 + pr8) / g.Kdraft];
  }
  int pre_tok = 0;
  if (EP == EPI_ROWS) pre_tok = g.last_token[m0 + pr16];

  mma_round(s_begin);
  for (int c0 = s_begin + KC; c0 < s_end; c0 += KC) {
    load_round(c0);
    mma_round(c0);
  }

  if (AM == A_NORM) {
    // 1 / RMS of each row of x from the per-16-column partial sums of squares: one wave per row, all
    // partials loaded at once (the first row's were prefetched), fixed reduction order
    for (int r = wave; r < nrows; r += NW) {
      const float* src = g.ssq_in + (size_t)gemm_a_row(g, m0 + r) * g.nssq;
      float t = 0.f;
      if (r == wave) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = lane + 64 * i < g.nssq ? pre_ssq[i] : 0.f;
        t = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
        for (int i = lane + 512; i < g.nssq; i += 64) t += src[i];
      } else {
        for (int i = lane; i < g.nssq; i += 64) t += src[i];
      }
      t = wave_sum(t);
      if (lane == 0) s_inv[r] = rsqrtf(t / (float)g.Kd + g.eps);
    }
  }

  // cross-wave sum of the k parts (fixed order): s_red[((kp * NT + tl) * MT + mt) * 256 + row16 * 16 + col]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      s_red[((kp * NT + tl) * MT + mt) * 256 + (4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[mt][r];
  __syncthreads();
  if (KP > 1) {
    for (int idx = threadIdx.x; idx < NT * MT * 256; idx += NTH) {
      float v = s_red[idx];
#pragma unroll
      for (int q = 1; q < KP; ++q) v += s_red[q * NT * MT * 256 + idx];
      s_red[idx] = v;
    }
    __syncthreads();
  }
  // reduced tile: y(tile t, local row r, column c), scaled by the row's 1/RMS for a normalised operand
  auto Y = [&](int t, int r, int c) {
    float v;
    if (KI)  // diagonal blocks: row r with chunk h sits at MFMA row r + 4h, column c with chunk h at c + 4h
      v = ((s_red[r * 16 + c] + s_red[(r + 4) * 16 + c + 4]) + s_red[(r + 8) * 16 + c + 8]) +
          s_red[(r + 12) * 16 + c + 12];
    else
      v = s_red[(t * MT + (r >> 4)) * 256 + (r & 15) * 16 + c];
    if (F8) v *= g.wscale[min((int)blockIdx.x * NT + t, g.Nt - 1) * 16 + c];
    return AM == A_NORM ? v * s_inv[r] : v;
  };
  const int rows = nrows;

  if (EP == EPI_ARGMAX) {
    // best (value, index) of each row over the workgroup's NT*16 columns; optional logits
    for (int r = wave; r < rows; r += NW) {
      const int m = m0 + r;
      const int t = lane >> 4, c = lane & 15;
      const int n = (blockIdx.x * NT + t) * 16 + c;
      const bool ok = t < NT && n < N;
      float v = ok ? Y(t, r, c) : -INFINITY;
      int idx = ok ? n : 0x7fffffff;
      if (g.logits && ok) g.logits[(size_t)m * g.ldz + n] = v;
      am_group_reduce<64>(v, idx);
      if (lane == 0) {
        g.am_val[(size_t)m * g.ngroups + blockIdx.x] = v;
        g.am_idx[(size_t)m * g.ngroups + blockIdx.x] = idx;
      }
    }
  } else if (EP == EPI_RESID) {
    // X[m][n] += y; XG = bf16(X * gain_next); per-row sum of squares of the new X over this tile
    for (int idx = threadIdx.x; idx < rows * CW; idx += NTH) {
      const int r = idx / CW, c = idx % CW;
      const int m = m0 + r, n = nt * CW + c;
      float v = 0.f;
      if (n < N) {
        v = (idx == (int)threadIdx.x ? pre_x : g.Xout[(size_t)m * N + n]) + Y(0, r, c);
        g.Xout[(size_t)m * N + n] = v;
        g.XGout[(size_t)m * N + n] = f32_to_bf16(v * bf16_to_f32(g.gain_next[n]));
      }
      float sq = v * v;
      sq = group_sum<CW>(sq);
      if (c == 0) g.ssq_out[(size_t)m * g.nssq_out + nt] = sq;
    }
  } else if (EP == EPI_ROWS) {
    // parallel-draft input rows. Product row m is real row i = m % R of request b = m / R (R = 1 for a
    // plain step): layer row b Kr + i = fc . concat(h) + embed[token] when i < n_real[b], else the
    // placeholder h_shared + emb_mask; real row 0 also writes the placeholder rows R .. Kr - 1.
    const int Kr = g.Kdraft, R = max(g.rows_real, 1);
    for (int idx = threadIdx.x; idx < rows * CW; idx += NTH) {
      const int r = idx / CW, c = idx % CW;
      const int m = m0 + r, n = nt * CW + c;
      const int b = m / R, i = m % R;
      const bool real = i < gemm_n_real(g, b);
      const bool first = idx == (int)threadIdx.x;
      const int tok = first ? pre_tok : g.last_token[m];
      const bool tok_ok = tok >= 0 && tok < g.V;
      if (real && !tok_ok && c == 0) raise_flag(g.flags, PE_FLAG_TOKEN);
      float x0 = 0.f, ph = 0.f;
      if (n < N) {
        const float e = tok_ok ? bf16_to_f32(g.embed[(size_t)tok * N + n]) : 0.f;
        const float em = bf16_to_f32(g.emb_mask[n]);
        // concatenated rows keep the embedding half apart (Xe); summed rows add it to the hidden half
        ph = bf16_to_f32(g.h_shared[n]) + (g.Xe ? 0.f : em);
        x0 = real ? Y(0, r, c) + (g.Xe ? 0.f : e) : ph;
        const float gn = bf16_to_f32(g.gain_next[n]);
        g.Xout[(size_t)(b * Kr + i) * N + n] = x0;
        g.XGout[(size_t)(b * Kr + i) * N + n] = f32_to_bf16(x0 * gn);
        if (g.Xe) g.Xe[(size_t)(b * Kr + i) * N + n] = real ? e : em;
        const bf16_t phg = f32_to_bf16(ph * gn);
        if (i == 0)
          for (int j = R; j < Kr; ++j) {
            g.Xout[(size_t)(b * Kr + j) * N + n] = ph;
            g.XGout[(size_t)(b * Kr + j) * N + n] = phg;
            if (g.Xe) g.Xe[(size_t)(b * Kr + j) * N + n] = em;
          }
      }
      float s0 = x0 * x0, s1 = ph * ph;
      s0 = group_sum<CW>(s0);
      s1 = group_sum<CW>(s1);
      if (c == 0) {
        g.ssq_out[(size_t)(b * Kr + i) * g.nssq_out + nt] = s0;
        if (i == 0)
          for (int j = R; j < Kr; ++j) g.ssq_out[(size_t)(b * Kr + j) * g.nssq_out + nt] = s1;
      }
    }
  } else if (EP == EPI_SWIGLU) {
    // tile nt: columns 0..7 = gate of f = 8 nt + e, columns 8..15 = up of the same f
    const int F = g.F;
    for (int idx = threadIdx.x; idx < rows * 8; idx += NTH) {
      const int r = idx >> 3, e = idx & 7;
      const int m = m0 + r, f = 8 * nt + e;
      if (f >= F) continue;
      const float gs = Y(0, r, e), us = Y(0, r, 8 + e);
      const float silu = gs / (1.f + __expf(-gs));
      g.Aout[(size_t)m * F + f] = f32_to_bf16(silu * us);
    }
  } else if (EP == EPI_QKV) {
    // tile nt of head u holds pairs i = 8 tt + e: columns e (first half) and 8 + e (second half).
    // q, k: rotate-half RoPE at position seq_len[b] + j; k and v are appended to the cache.
    const int hd = g.hd, half = hd / 2, Hq = g.Hq, Hkv = g.Hkv;
    const int tph = hd / 16, u = nt / tph, tt = nt % tph;
    for (int idx = threadIdx.x; idx < rows * 8; idx += NTH) {
      const int r = idx >> 3, e = idx & 7;
      const int m = m0 + r, i = 8 * tt + e;
      const int b = m / g.Kdraft, j = m % g.Kdraft;
      const bool first = idx == (int)threadIdx.x;
      const int pos = (first ? pre_seq : g.seq_len[b]) + j;
      const int slot = first ? pre_slot : g.req_slot[b];
      const bool pos_ok = pos >= 0 && pos < g.max_ctx;
      const bool slot_ok = slot >= 0 && slot < g.n_slots;
      if (e == 0 && tt == 0) {
        if (!pos_ok) raise_flag(g.flags, PE_FLAG_POS);
        if (!slot_ok) raise_flag(g.flags, PE_FLAG_SLOT);
      }
      const float x1 = Y(0, r, e), x2 = Y(0, r, 8 + e);
      if (u >= Hq + Hkv) {
        if (pos_ok && slot_ok) {
          bf16_t* v = g.Vc + (((size_t)slot * Hkv + (u - Hq - Hkv)) * g.max_ctx + pos) * hd;
          v[i] = f32_to_bf16(x1);
          v[i + half] = f32_to_bf16(x2);
        }
        continue;
      }
      const float2 t = g.rope[(size_t)(pos_ok ? pos : 0) * half + i];
      const float y1 = x1 * t.x - x2 * t.y;
      const float y2 = x2 * t.x + x1 * t.y;
      if (u < Hq) {
        bf16_t* q = g.Q + ((size_t)m * Hq + u) * hd;
        q[i] = f32_to_bf16(y1);
        q[i + half] = f32_to_bf16(y2);
      } else if (pos_ok && slot_ok) {
        bf16_t* k = g.Kc + (((size_t)slot * Hkv + (u - Hq)) * g.max_ctx + pos) * hd;
        k[i] = f32_to_bf16(y1);
        k[i + half] = f32_to_bf16(y2);
      }
    }
  }
}

template <int MT, int NW, int NT, int AM, int EP, int KI = 0, int F8 = 0>
static void launch_one(const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((gemm_kernel<MT, NW, NT, AM, EP, KI, F8>), dim3(p.ngroups, p.mblocks), dim3(NW * 64), 0, st, a);
}

template <int AM, int EP, int F8 = 0>
static hipError_t launch_split_nw(const GemmPlan& p, const GemmArgs& a, hipStream_t st) {
#define PE_NW_CASES(MT_)                                            \
  if (p.MT == MT_) {                                                \
    if (p.NW == 16) launch_one<MT_, (MT_ == 1 ? 16 : 4), 1, AM, EP, 0, F8>(p, a, st); \
    else if (p.NW == 8) launch_one<MT_, (MT_ <= 2 ? 8 : 4), 1, AM, EP, 0, F8>(p, a, st); \
    else launch_one<MT_, 4, 1, AM, EP, 0, F8>(p, a, st);            \
    return hipGetLastError();                                       \
  }
  PE_NW_CASES(1)
  if (F8) return hipErrorInvalidValue;  // FP8 weights: products of up to 16 rows
  PE_NW_CASES(2)
  PE_NW_CASES(4)
  PE_NW_CASES(8)
#undef PE_NW_CASES
  return hipErrorInvalidValue;
}

// FP8 weights: the small-batch kernel (up to 16 rows, 16-column tiles), or the weight-stream and tiled kernels
static hipError_t launch_gemm_fp8(const GemmPlan& p, const GemmArgs& a, int a_mode, int epi, hipStream_t st) {
  if (p.tiled) return launch_gemm_tiled(p, a, a_mode, epi, st);  // weight-stream (17-128 rows) or 128 x 128 tiles
  if (p.ki4 || p.MT != 1) return hipErrorInvalidValue;
  if (epi == EPI_ARGMAX) {
    if (a_mode != A_NORM || p.NW != 8) return hipErrorInvalidValue;
    if (p.NT == 4) launch_one<1, 8, 4, A_NORM, EPI_ARGMAX, 0, 1>(p, a, st);
    else if (p.NT == 2) launch_one<1, 8, 2, A_NORM, EPI_ARGMAX, 0, 1>(p, a, st);
    else if (p.NT == 1) launch_one<1, 8, 1, A_NORM, EPI_ARGMAX, 0, 1>(p, a, st);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (p.NT != 1) return hipErrorInvalidValue;
  if (a_mode == A_BF16 && epi == EPI_RESID) return launch_split_nw<A_BF16, EPI_RESID, 1>(p, a, st);
  if (a_mode == A_BF16 && epi == EPI_ROWS) return launch_split_nw<A_BF16, EPI_ROWS, 1>(p, a, st);
  if (a_mode == A_NORM && epi == EPI_QKV) return launch_split_nw<A_NORM, EPI_QKV, 1>(p, a, st);
  if (a_mode == A_NORM && epi == EPI_SWIGLU) return launch_split_nw<A_NORM, EPI_SWIGLU, 1>(p, a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmPlan& p, GemmArgs a, int a_mode, int epi, hipStream_t st) {
  a.Nt = p.Nt;
  a.Ks = p.ki4 ? k_steps_ki4(a.Kd) : k_steps(a.Kd);
  a.ngroups = p.ngroups;
  a.mblocks = p.mblocks;
  if (a.ldz == 0) a.ldz = a.N;
  a.ksplit = p.ksplit;
  a.kper = p.kper;
  if (a.wscale) return launch_gemm_fp8(p, a, a_mode, epi, st);
  if (p.tiled) return launch_gemm_tiled(p, a, a_mode, epi, st);
  if (p.ki4) {
    if (a_mode != A_BF16 || (p.NW != 4 && p.NW != 8) || a.M > 4) return hipErrorInvalidValue;
    if (epi == EPI_RESID && p.NW == 4) launch_one<1, 4, 1, A_BF16, EPI_RESID, 1>(p, a, st);
    else if (epi == EPI_RESID) launch_one<1, 8, 1, A_BF16, EPI_RESID, 1>(p, a, st);
    else if (epi == EPI_ROWS && p.NW == 4) launch_one<1, 4, 1, A_BF16, EPI_ROWS, 1>(p, a, st);
    else if (epi == EPI_ROWS) launch_one<1, 8, 1, A_BF16, EPI_ROWS, 1>(p, a, st);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (epi == EPI_ARGMAX) {
    if (a_mode != A_NORM) return hipErrorInvalidValue;
    if (p.MT == 1 && p.NT == 1 && p.NW == 8) {
      launch_one<1, 8, 1, A_NORM, EPI_ARGMAX>(p, a, st);
      return hipGetLastError();
    }
    if (p.NT != 4 || p.NW != 4) return hipErrorInvalidValue;
    switch (p.MT) {
      case 1: launch_one<1, 4, 4, A_NORM, EPI_ARGMAX>(p, a, st); break;
      case 2: launch_one<2, 4, 4, A_NORM, EPI_ARGMAX>(p, a, st); break;
      case 4: launch_one<4, 4, 4, A_NORM, EPI_ARGMAX>(p, a, st); break;
      default: launch_one<8, 4, 4, A_NORM, EPI_ARGMAX>(p, a, st); break;
    }
    return hipGetLastError();
  }
  if (p.NT != 1) return hipErrorInvalidValue;
  if (a_mode == A_BF16 && epi == EPI_RESID) return launch_split_nw<A_BF16, EPI_RESID>(p, a, st);
  if (a_mode == A_BF16 && epi == EPI_ROWS) return launch_split_nw<A_BF16, EPI_ROWS>(p, a, st);
  if (a_mode == A_NORM && epi == EPI_QKV) return launch_split_nw<A_NORM, EPI_QKV>(p, a, st);
  if (a_mode == A_BF16 && epi == EPI_QKV) return launch_split_nw<A_BF16, EPI_QKV>(p, a, st);
  if (a_mode == A_NORM && epi == EPI_SWIGLU) return launch_split_nw<A_NORM, EPI_SWIGLU>(p, a, st);
  return hipErrorInvalidValue;
}

// X = caller rows; per-16-column sums of squares and XG = bf16(x * gain) (the operand of the first
// normalised projection)
__global__ __launch_bounds__(256) void rows_ssq_kernel(const float* __restrict__ rows, float* __restrict__ X,
                                                       float* __restrict__ ssq, bf16_t* __restrict__ XG,
                                                       const bf16_t* __restrict__ gain, int d, int nssq) {
  const int m = blockIdx.x;
  for (int c0 = 0; c0 < nssq * 16; c0 += 256) {
    const int c = c0 + threadIdx.x;
    float v = 0.f;
    if (c < d) {
      v = rows[(size_t)m * d + c];
      X[(size_t)m * d + c] = v;
      XG[(size_t)m * d + c] = f32_to_bf16(v * bf16_to_f32(gain[c]));
    }
    float sq = v * v;
    sq = group_sum<16>(sq);
    if ((c & 15) == 0 && c / 16 < nssq) ssq[(size_t)m * nssq + c / 16] = sq;
  }
}

hipError_t launch_rows_ssq(const float* rows, float* X, float* ssq, uint16_t* XG, const uint16_t* gain, int M, int d,
                           hipStream_t st) {
  hipLaunchKernelGGL(rows_ssq_kernel, dim3(M), dim3(256), 0, st, rows, X, ssq, (bf16_t*)XG, (const bf16_t*)gain, d,
                     (d + 15) / 16);
  return hipGetLastError();
}

// autoregressive pass >= 1: the previous pass's residual stream plus the embedding of the token it drafted
__global__ __launch_bounds__(256) void ar_rows_kernel(float* __restrict__ X, bf16_t* __restrict__ XG,
                                                      float* __restrict__ ssq, const bf16_t* __restrict__ embed,
                                                      const bf16_t* __restrict__ gain, const int* __restrict__ prev_tok,
                                                      int* __restrict__ draft_tokens, int K, int pass,
                                                      const int* __restrict__ seq_len, int* __restrict__ seq_cur,
                                                      int d, int V, int* flags) {
  const int b = blockIdx.x;
  const int tok = prev_tok[b];
  const bool ok = tok >= 0 && tok < V;
  if (threadIdx.x == 0) {
    draft_tokens[(size_t)b * K + pass - 1] = tok;
    seq_cur[b] = seq_len[b] + pass;
    if (!ok) raise_flag(flags, PE_FLAG_TOKEN);
  }
  const int nssq = (d + 15) / 16;
  for (int c0 = 0; c0 < nssq * 16; c0 += 256) {
    const int c = c0 + threadIdx.x;
    float v = 0.f;
    if (c < d) {
      v = X[(size_t)b * d + c] + (ok ? bf16_to_f32(embed[(size_t)tok * d + c]) : 0.f);
      X[(size_t)b * d + c] = v;
      XG[(size_t)b * d + c] = f32_to_bf16(v * bf16_to_f32(gain[c]));
    }
    float sq = v * v;
    sq = group_sum<16>(sq);
    if ((c & 15) == 0 && c / 16 < nssq) ssq[(size_t)b * nssq + c / 16] = sq;
  }
}

hipError_t launch_ar_rows(float* X, uint16_t* XG, float* ssq, const uint16_t* embed, const uint16_t* gain,
                          const int* prev_tok, int* draft_tokens, int K, int pass, const int* seq_len, int* seq_cur,
                          int B, int d, int V, int* flags, hipStream_t st) {
  if (pass < 1 || pass > K) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ar_rows_kernel, dim3(B), dim3(256), 0, st, X, (bf16_t*)XG, ssq, (const bf16_t*)embed,
                     (const bf16_t*)gain, prev_tok, draft_tokens, K, pass, seq_len, seq_cur, d, V, flags);
  return hipGetLastError();
}

// fp32 weights (the small fp32 drafter): one wave per output column, lanes stride over k.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda, int M, int Kd,
                                                       const float* __restrict__ W, int N, float* __restrict__ out,
                                                       int ldo, int rows_in, int rows_out) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  const float* w = W + (size_t)n * Kd;
  for (int m = 0; m < M; ++m) {
    const int ar = rows_out > 0 ? (m / rows_out) * rows_in + m % rows_out : m;
    const float* a = A + (size_t)ar * lda;
    float s = 0.f;
    for (int k = lane; k < Kd; k += 64) s = fmaf(a[k], w[k], s);
    s = wave_sum(s);
    if (lane == 0) out[(size_t)m * ldo + n] = s;
  }
}

hipError_t launch_gemm_f32(const float* A, int lda, int M, int Kd, const float* W, int N, float* out, int ldo,
                           hipStream_t st, int rows_in, int rows_out) {
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((N + 3) / 4), dim3(256), 0, st, A, lda, M, Kd, W, N, out, ldo, rows_in,
                     rows_out);
  return hipGetLastError();
}

}  // namespace pe
