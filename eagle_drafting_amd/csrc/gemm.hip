// Projections of the drafter (fc, QKV, O, gate/up, down, LM head): y = A . W^T.
//
// bf16 path: the weight matrix is repacked once (pe_init) into 1 KiB MFMA fragments, so a wave's
// B-operand load for one 16 x 32 tile is a single contiguous 1 KiB read (64 lanes x 16 B). The
// activations (M = B*K rows, small) are staged through LDS in A-fragment order and shared by the four
// waves of a workgroup; each wave owns one 16-column tile and accumulates MT 16x16 fp32 tiles with
// v_mfma_f32_16x16x32_bf16. Split-K partials are written in fp32 and summed, in a fixed order, by the
// consumer kernel, so results do not depend on scheduling.
//
// MFMA lane layout (16x16x32, wave64): A lane l holds A[l%16][k-group l/16] (8 values), B lane l holds
// B[k-group l/16][l%16], D lane l holds D[4(l/16)+r][l%16], r = 0..3. A and B use the same k grouping,
// so any consistent assignment of the 32 k values to (group, element) gives the same sum.
#include "common.h"
#include "kernels.h"

namespace pe {

__global__ __launch_bounds__(256) void pack_bf16_kernel(const bf16_t* __restrict__ W, int N, int Kd,
                                                        bf16x8_t* __restrict__ dst, int Nt, int Ks, int mul,
                                                        int add) {
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)Nt * Ks * 64;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const size_t frag = gid >> 6;
  const int s = (int)(frag % Ks);
  const int t = (int)(frag / Ks);
  const int row = 16 * t + (lane & 15);
  const int col = 32 * s + 8 * (lane >> 4);
  bf16x8_t v;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    short x = 0;
    if (row < N && col + e < Kd) x = (short)W[(size_t)row * Kd + col + e];
    v[e] = x;
  }
  dst[((size_t)(t * mul + add) * Ks + s) * 64 + lane] = v;
}

hipError_t launch_pack_bf16(const void* W, int N, int Kd, void* dst, int tile_mul, int tile_add, hipStream_t st) {
  const int Nt = n_tiles(N), Ks = k_steps(Kd);
  const size_t total = (size_t)Nt * Ks * 64;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(grid), dim3(256), 0, st, (const bf16_t*)W, N, Kd, (bf16x8_t*)dst, Nt,
                     Ks, tile_mul, tile_add);
  return hipGetLastError();
}

GemmPlan plan_gemm(int M, int N, int Kd, bool argmax_epilogue) {
  GemmPlan p;
  const int Nt = n_tiles(N), Ks = k_steps(Kd);
  p.MT = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
  p.mblocks = (M + 16 * p.MT - 1) / (16 * p.MT);
  p.ngroups = (Nt + 3) / 4;
  int S = 1;
  if (!argmax_epilogue) {
    const int base = p.ngroups * p.mblocks;
    S = (1024 + base - 1) / base;
    const int smax = Ks / 4 > 1 ? Ks / 4 : 1;  // at least 4 k-steps (128 k) per split
    if (S > smax) S = smax;
    if (S < 1) S = 1;
  }
  p.kps = (Ks + S - 1) / S;
  p.S = (Ks + p.kps - 1) / p.kps;
  return p;
}

constexpr int GEMM_KC = 8;  // k-steps staged per chunk

template <int MT, bool ARGMAX>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const bf16_t* __restrict__ A, int lda, int M, int Kd,
                                                        const bf16x8_t* __restrict__ Wp, int Nt, int Ks, int N,
                                                        int kps, float* __restrict__ P,
                                                        float* __restrict__ am_val, int* __restrict__ am_idx,
                                                        int ngroups, float* __restrict__ logits) {
  __shared__ bf16x8_t sA[MT * GEMM_KC * 64];
  __shared__ float s_rv[ARGMAX ? 4 * MT * 16 : 1];
  __shared__ int s_ri[ARGMAX ? 4 * MT * 16 : 1];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nt = blockIdx.x * 4 + wave;
  const bool active = nt < Nt;
  const int m0 = blockIdx.y * MT * 16;
  const int split = blockIdx.z;
  const int s_begin = split * kps;
  const int s_end = min(Ks, s_begin + kps);

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const bf16x8_t* wsrc = Wp + (size_t)(active ? nt : 0) * Ks * 64 + lane;
  const bf16x8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  for (int c0 = s_begin; c0 < s_end; c0 += GEMM_KC) {
    const int nk = min(GEMM_KC, s_end - c0);
    bf16x8_t b[GEMM_KC];
#pragma unroll
    for (int kk = 0; kk < GEMM_KC; ++kk) b[kk] = (active && kk < nk) ? wsrc[(size_t)(c0 + kk) * 64] : zero8;
    for (int p = threadIdx.x; p < MT * GEMM_KC * 64; p += 256) {
      const int ln = p & 63, kk = (p >> 6) % GEMM_KC, mt = (p >> 6) / GEMM_KC;
      const int row = m0 + mt * 16 + (ln & 15);
      const int col = (c0 + kk) * 32 + 8 * (ln >> 4);
      bf16x8_t v = zero8;
      if (kk < nk && row < M && col < Kd) v = *(const bf16x8_t*)(A + (size_t)row * lda + col);
      sA[p] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GEMM_KC; ++kk) {
      if (kk < nk) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sA[(mt * GEMM_KC + kk) * 64 + lane], b[kk], acc[mt], 0,
                                                            0, 0);
      }
    }
    __syncthreads();
  }

  const int n = nt * 16 + (lane & 15);
  if (!ARGMAX) {
    if (active && n < N) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + mt * 16 + 4 * (lane >> 4) + r;
          if (m < M) P[((size_t)split * M + m) * N + n] = acc[mt][r];
        }
    }
  } else {
    const bool ok = active && n < N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = mt * 16 + 4 * (lane >> 4) + r;
        const int m = m0 + rl;
        float v = ok ? acc[mt][r] : -INFINITY;
        int idx = ok ? n : 0x7fffffff;
        if (logits && ok && m < M) logits[(size_t)m * N + n] = acc[mt][r];
        am_wave_reduce(v, idx, 16);
        if ((lane & 15) == 0) {
          s_rv[wave * MT * 16 + rl] = v;
          s_ri[wave * MT * 16 + rl] = idx;
        }
      }
    __syncthreads();
    for (int rl = threadIdx.x; rl < MT * 16; rl += 256) {
      float bv = s_rv[rl];
      int bi = s_ri[rl];
      for (int w = 1; w < 4; ++w) {
        const float v = s_rv[w * MT * 16 + rl];
        const int i = s_ri[w * MT * 16 + rl];
        if (am_better(v, i, bv, bi)) { bv = v; bi = i; }
      }
      const int m = m0 + rl;
      if (m < M) {
        am_val[(size_t)m * ngroups + blockIdx.x] = bv;
        am_idx[(size_t)m * ngroups + blockIdx.x] = bi;
      }
    }
  }
}

template <bool ARGMAX>
static hipError_t launch_gemm_bf16(const GemmPlan& p, const void* A, int lda, int M, int Kd, const void* Wp, int N,
                                   float* P, float* am_val, int* am_idx, float* logits, hipStream_t st) {
  const int Nt = n_tiles(N), Ks = k_steps(Kd);
  dim3 grid(p.ngroups, p.mblocks, p.S), block(256);
  const bf16_t* a = (const bf16_t*)A;
  const bf16x8_t* w = (const bf16x8_t*)Wp;
  switch (p.MT) {
    case 1: hipLaunchKernelGGL((gemm_bf16_kernel<1, ARGMAX>), grid, block, 0, st, a, lda, M, Kd, w, Nt, Ks, N, p.kps, P, am_val, am_idx, p.ngroups, logits); break;
    case 2: hipLaunchKernelGGL((gemm_bf16_kernel<2, ARGMAX>), grid, block, 0, st, a, lda, M, Kd, w, Nt, Ks, N, p.kps, P, am_val, am_idx, p.ngroups, logits); break;
    case 4: hipLaunchKernelGGL((gemm_bf16_kernel<4, ARGMAX>), grid, block, 0, st, a, lda, M, Kd, w, Nt, Ks, N, p.kps, P, am_val, am_idx, p.ngroups, logits); break;
    default: hipLaunchKernelGGL((gemm_bf16_kernel<8, ARGMAX>), grid, block, 0, st, a, lda, M, Kd, w, Nt, Ks, N, p.kps, P, am_val, am_idx, p.ngroups, logits); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_partial(const GemmPlan& p, const void* A, int lda, int M, int Kd, const void* Wp, int N,
                                    float* P, hipStream_t st) {
  return launch_gemm_bf16<false>(p, A, lda, M, Kd, Wp, N, P, nullptr, nullptr, nullptr, st);
}

hipError_t launch_gemm_bf16_argmax(const GemmPlan& p, const void* A, int lda, int M, int Kd, const void* Wp, int N,
                                   float* am_val, int* am_idx, float* logits, hipStream_t st) {
  return launch_gemm_bf16<true>(p, A, lda, M, Kd, Wp, N, nullptr, am_val, am_idx, logits, st);
}

// fp32 weights (the small fp32 drafter): one wave per output column, lanes stride over k.
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda, int M, int Kd,
                                                       const float* __restrict__ W, int N, float* __restrict__ out,
                                                       int ldo) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  const float* w = W + (size_t)n * Kd;
  for (int m = 0; m < M; ++m) {
    const float* a = A + (size_t)m * lda;
    float s = 0.f;
    for (int k = lane; k < Kd; k += 64) s = fmaf(a[k], w[k], s);
    s = wave_sum(s);
    if (lane == 0) out[(size_t)m * ldo + n] = s;
  }
}

hipError_t launch_gemm_f32(const float* A, int lda, int M, int Kd, const float* W, int N, float* out, int ldo,
                           hipStream_t st) {
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((N + 3) / 4), dim3(256), 0, st, A, lda, M, Kd, W, N, out, ldo);
  return hipGetLastError();
}

}  // namespace pe
