// Row-wise kernels of the draft step: input-row builder (+ first RMSNorm), residual add + RMSNorm,
// SwiGLU, RoPE + KV append, and the RoPE table.
//
// Row m of the drafter batch is request b = m / K, draft position j = m % K, at sequence position
// seq_len[b] + j. The residual stream X is fp32; normalised activations U are stored in the weight
// dtype for the next projection. Split-K partials P[s][m][n] are summed in increasing s.
#include "common.h"
#include "kernels.h"

namespace pe {

// RMSNorm of one row held in X (already written by this thread for its own columns):
// U[c] = X[c] * (mean(X^2) + eps)^-1/2 * g[c]
template <typename T>
__device__ __forceinline__ void norm_row(const float* __restrict__ x, T* __restrict__ u, const T* __restrict__ g,
                                         int d, float eps, float sumsq, float* red) {
  const float tot = block_sum<256>(sumsq, red);
  const float inv = rsqrtf(tot / (float)d + eps);
  for (int c = threadIdx.x; c < d; c += 256) u[c] = from_f32<T>(x[c] * inv * to_f32<T>(g[c]));
}

// Input rows of the parallel draft (solution overview, step 2):
//   row 0:      fc . concat(h_low, h_mid, h_high) + embed[last_token]   (fc output = sum of split partials)
//   rows 1..K-1: h_shared + emb_mask
// or, when rows_in is given, the caller's rows. Then U = RMSNorm(X, gain).
template <typename T>
__global__ __launch_bounds__(256) void rowbuild_norm_kernel(float* __restrict__ X, T* __restrict__ U,
                                                            const float* __restrict__ P, int S,
                                                            const float* __restrict__ rows_in, int B, int K, int d,
                                                            const int* __restrict__ last_token,
                                                            const T* __restrict__ embed,
                                                            const T* __restrict__ emb_mask,
                                                            const T* __restrict__ h_shared, const T* __restrict__ g,
                                                            float eps, int V, int* flags) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int b = m / K, j = m % K;
  float* x = X + (size_t)m * d;
  float sumsq = 0.f;
  if (rows_in) {
    const float* r = rows_in + (size_t)m * d;
    for (int c = threadIdx.x; c < d; c += 256) {
      const float v = r[c];
      x[c] = v;
      sumsq += v * v;
    }
  } else if (j == 0) {
    int tok = last_token[b];
    const bool ok = tok >= 0 && tok < V;
    if (!ok && threadIdx.x == 0) raise_flag(flags, PE_FLAG_TOKEN);
    const T* e = embed + (size_t)(ok ? tok : 0) * d;
    for (int c = threadIdx.x; c < d; c += 256) {
      float v = 0.f;
      for (int s = 0; s < S; ++s) v += P[((size_t)s * B + b) * d + c];
      v += ok ? to_f32<T>(e[c]) : 0.f;
      x[c] = v;
      sumsq += v * v;
    }
  } else {
    for (int c = threadIdx.x; c < d; c += 256) {
      const float v = to_f32<T>(h_shared[c]) + to_f32<T>(emb_mask[c]);
      x[c] = v;
      sumsq += v * v;
    }
  }
  norm_row<T>(x, U + (size_t)m * d, g, d, eps, sumsq, red);
}

hipError_t launch_rowbuild_norm(int dtype, float* X, void* U, const float* P, int S, const float* rows_in, int B,
                                int K, int d, const int* last_token, const void* embed, const void* emb_mask,
                                const void* h_shared, const void* gain, float eps, int V, int* flags,
                                hipStream_t st) {
  dim3 grid(B * K), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(rowbuild_norm_kernel<float>, grid, block, 0, st, X, (float*)U, P, S, rows_in, B, K, d,
                       last_token, (const float*)embed, (const float*)emb_mask, (const float*)h_shared,
                       (const float*)gain, eps, V, flags);
  else
    hipLaunchKernelGGL(rowbuild_norm_kernel<bf16_t>, grid, block, 0, st, X, (bf16_t*)U, P, S, rows_in, B, K, d,
                       last_token, (const bf16_t*)embed, (const bf16_t*)emb_mask, (const bf16_t*)h_shared,
                       (const bf16_t*)gain, eps, V, flags);
  return hipGetLastError();
}

// X += sum_s P[s]; U = RMSNorm(X, gain)
template <typename T>
__global__ __launch_bounds__(256) void residual_norm_kernel(float* __restrict__ X, T* __restrict__ U,
                                                            const float* __restrict__ P, int S, int M, int d,
                                                            const T* __restrict__ g, float eps) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  float* x = X + (size_t)m * d;
  float sumsq = 0.f;
  for (int c = threadIdx.x; c < d; c += 256) {
    float v = x[c];
    for (int s = 0; s < S; ++s) v += P[((size_t)s * M + m) * d + c];
    x[c] = v;
    sumsq += v * v;
  }
  norm_row<T>(x, U + (size_t)m * d, g, d, eps, sumsq, red);
}

hipError_t launch_residual_norm(int dtype, float* X, void* U, const float* P, int S, int M, int d,
                                const void* gain, float eps, hipStream_t st) {
  if (dtype == 0)
    hipLaunchKernelGGL(residual_norm_kernel<float>, dim3(M), dim3(256), 0, st, X, (float*)U, P, S, M, d,
                       (const float*)gain, eps);
  else
    hipLaunchKernelGGL(residual_norm_kernel<bf16_t>, dim3(M), dim3(256), 0, st, X, (bf16_t*)U, P, S, M, d,
                       (const bf16_t*)gain, eps);
  return hipGetLastError();
}

// a[m][f] = silu(gate) * up, gate/up = sums of split partials. With interleaved = true the projection
// output columns alternate 16-wide gate and up tiles (gate f at 32(f/16) + f%16, up 16 columns later);
// otherwise gate occupies columns [0, F) and up [F, 2F).
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(T* __restrict__ Aout, const float* __restrict__ P, int S, int M,
                                                     int F, int interleaved) {
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (size_t)M * F) return;
  const int m = (int)(gid / F), f = (int)(gid % F);
  const int N = 2 * F;
  const int cg = interleaved ? 32 * (f >> 4) + (f & 15) : f;
  const int cu = interleaved ? cg + 16 : f + F;
  float gs = 0.f, us = 0.f;
  for (int s = 0; s < S; ++s) {
    const float* row = P + ((size_t)s * M + m) * N;
    gs += row[cg];
    us += row[cu];
  }
  const float silu = gs / (1.f + __expf(-gs));
  Aout[gid] = from_f32<T>(silu * us);
}

hipError_t launch_swiglu(int dtype, void* Aout, const float* P, int S, int M, int F, bool interleaved,
                         hipStream_t st) {
  const size_t total = (size_t)M * F;
  dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == 0)
    hipLaunchKernelGGL(swiglu_kernel<float>, grid, dim3(256), 0, st, (float*)Aout, P, S, M, F, interleaved ? 1 : 0);
  else
    hipLaunchKernelGGL(swiglu_kernel<bf16_t>, grid, dim3(256), 0, st, (bf16_t*)Aout, P, S, M, F, interleaved ? 1 : 0);
  return hipGetLastError();
}

// q, k, v from the QKV projection of row m; rotate-half RoPE of q and k at position seq_len[b] + j;
// q -> Q[m], k and v -> cache slot req_slot[b], that position. cs[pos][i] = (cos, sin) of
// pos * base^(-2i/hd).
template <typename T>
__global__ __launch_bounds__(256) void rope_kv_kernel(T* __restrict__ Q, T* __restrict__ Kc, T* __restrict__ Vc,
                                                      const float* __restrict__ P, int S, int B, int K, int Hq,
                                                      int Hkv, int hd, const int* __restrict__ seq_len,
                                                      const int* __restrict__ req_slot, int max_ctx, int n_slots,
                                                      const float2* __restrict__ cs, int* flags) {
  const int m = blockIdx.x;
  const int b = m / K, j = m % K;
  const int N = (Hq + 2 * Hkv) * hd;
  const int half = hd / 2;
  const int pos = seq_len[b] + j;
  const int slot = req_slot[b];
  const bool pos_ok = pos >= 0 && pos < max_ctx;
  const bool slot_ok = slot >= 0 && slot < n_slots;
  if (threadIdx.x == 0) {
    if (!pos_ok) raise_flag(flags, PE_FLAG_POS);
    if (!slot_ok) raise_flag(flags, PE_FLAG_SLOT);
  }
  const float2* csr = cs + (size_t)(pos_ok ? pos : 0) * half;
  auto col = [&](int n) {
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += P[((size_t)s * B * K + m) * N + n];
    return v;
  };
  // rotary pairs of q heads and k heads
  const int npairs = (Hq + Hkv) * half;
  for (int p = threadIdx.x; p < npairs; p += 256) {
    const int head = p / half, i = p % half;
    const int base = head * hd;  // q heads first, then k heads: same column offsets in the projection
    const float x1 = col(base + i), x2 = col(base + i + half);
    const float2 t = csr[i];
    const float y1 = x1 * t.x - x2 * t.y;
    const float y2 = x2 * t.x + x1 * t.y;
    if (head < Hq) {
      T* q = Q + (size_t)m * Hq * hd + base;
      q[i] = from_f32<T>(y1);
      q[i + half] = from_f32<T>(y2);
    } else if (pos_ok && slot_ok) {
      const int g = head - Hq;
      T* k = Kc + (((size_t)slot * Hkv + g) * max_ctx + pos) * hd;
      k[i] = from_f32<T>(y1);
      k[i + half] = from_f32<T>(y2);
    }
  }
  if (pos_ok && slot_ok) {
    for (int e = threadIdx.x; e < Hkv * hd; e += 256) {
      const int g = e / hd, c = e % hd;
      Vc[(((size_t)slot * Hkv + g) * max_ctx + pos) * hd + c] = from_f32<T>(col((Hq + Hkv) * hd + e));
    }
  }
}

hipError_t launch_rope_kv(int dtype, void* Q, void* Kc, void* Vc, const float* P, int S, int B, int K, int Hq,
                          int Hkv, int hd, const int* seq_len, const int* req_slot, int max_ctx, int n_slots,
                          const float2* cs, int* flags, hipStream_t st) {
  dim3 grid(B * K), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(rope_kv_kernel<float>, grid, block, 0, st, (float*)Q, (float*)Kc, (float*)Vc, P, S, B, K, Hq,
                       Hkv, hd, seq_len, req_slot, max_ctx, n_slots, cs, flags);
  else
    hipLaunchKernelGGL(rope_kv_kernel<bf16_t>, grid, block, 0, st, (bf16_t*)Q, (bf16_t*)Kc, (bf16_t*)Vc, P, S, B,
                       K, Hq, Hkv, hd, seq_len, req_slot, max_ctx, n_slots, cs, flags);
  return hipGetLastError();
}

// cs[pos][i] = (cos, sin)(pos * base^(-2i/hd)), angles and trig in fp64, stored fp32
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ cs, int max_ctx, int hd, double base) {
  const int half = hd / 2;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (size_t)max_ctx * half) return;
  const int pos = (int)(gid / half), i = (int)(gid % half);
  const double inv_freq = pow(base, -2.0 * (double)i / (double)hd);
  const double a = (double)pos * inv_freq;
  cs[gid] = make_float2((float)cos(a), (float)sin(a));
}

hipError_t launch_rope_table(float2* cs, int max_ctx, int hd, double base, hipStream_t st) {
  const size_t total = (size_t)max_ctx * (hd / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, cs, max_ctx, hd,
                     base);
  return hipGetLastError();
}

// Concatenated input rows: U[m] = [bf16(xe * g_e / rms(xe)) || bf16(x * g_h / rms(x))], rms(v) =
// sqrt(mean(v^2) + eps) over each d-wide half (the embedding half first). One workgroup per row; the two
// sums of squares are reduced in a fixed order (per thread, then per wave by xor-shuffles, then the four
// waves in order), so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void concat_norm_kernel(const float* __restrict__ X, const float* __restrict__ Xe,
                                                          const bf16_t* __restrict__ g_h,
                                                          const bf16_t* __restrict__ g_e, bf16_t* __restrict__ U,
                                                          int d, float eps) {
  __shared__ float red[2][4];
  const int m = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* x = X + (size_t)m * d;
  const float* xe = Xe + (size_t)m * d;
  float sh = 0.f, se = 0.f;
  for (int c = tid; c < d; c += 256) {
    sh += x[c] * x[c];
    se += xe[c] * xe[c];
  }
  sh = group_sum<64>(sh);
  se = group_sum<64>(se);
  if (lane == 0) {
    red[0][wave] = sh;
    red[1][wave] = se;
  }
  __syncthreads();
  const float th = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
  const float te = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  const float ih = rsqrtf(th / (float)d + eps), ie = rsqrtf(te / (float)d + eps);
  bf16_t* u = U + (size_t)m * 2 * d;
  for (int c = tid; c < d; c += 256) {
    u[c] = f32_to_bf16(xe[c] * ie * bf16_to_f32(g_e[c]));
    u[d + c] = f32_to_bf16(x[c] * ih * bf16_to_f32(g_h[c]));
  }
}

hipError_t launch_concat_norm(const float* X, const float* Xe, const uint16_t* g_h, const uint16_t* g_e, uint16_t* U,
                              int M, int d, float eps, hipStream_t st) {
  hipLaunchKernelGGL(concat_norm_kernel, dim3(M), dim3(256), 0, st, X, Xe, (const bf16_t*)g_h, (const bf16_t*)g_e,
                     (bf16_t*)U, d, eps);
  return hipGetLastError();
}

}  // namespace pe
