// Vocabulary argmax (draft tokens on the fp32 path, target tokens in verify) and the greedy
// accept / batch-metadata rebuild.
//
// Argmax convention everywhere: the largest value wins; among equal values the lowest index.
#include "common.h"
#include "kernels.h"

namespace pe {

int plan_argmax_chunks(int rows, int V) {
  // ~1024 workgroups, each scanning at least 2048 entries of its row
  int c = (1024 + rows - 1) / rows;
  const int cmax = (V + 2047) / 2048;
  if (c > cmax) c = cmax;
  if (c < 1) c = 1;
  return c;
}

// One workgroup per (row, chunk); 16-byte loads; partial (value, index) per (row, chunk).
template <typename T>
__global__ __launch_bounds__(256) void argmax_rows_kernel(const T* __restrict__ X, int V, int chunk, int nchunks,
                                                          float* __restrict__ pv, int* __restrict__ pi) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ float sv[4];
  __shared__ int si[4];
  const int row = blockIdx.x, c = blockIdx.y;
  const int begin = c * chunk;
  const int end = min(V, begin + chunk);
  const T* x = X + (size_t)row * V;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = begin + threadIdx.x * VEC; i < end; i += 256 * VEC) {
    if (i + VEC <= end) {
      union { uint4 u; T e[VEC]; } ld;
      ld.u = *(const uint4*)(x + i);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float v = to_f32<T>(ld.e[e]);
        if (v > best) { best = v; bi = i + e; }
      }
    } else {
      for (int e = i; e < end; ++e) {
        const float v = to_f32<T>(x[e]);
        if (v > best) { best = v; bi = e; }
      }
    }
  }
  am_wave_reduce(best, bi, 64);
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = sv[0];
    int i = si[0];
    for (int w = 1; w < 4; ++w)
      if (am_better(sv[w], si[w], b, i)) { b = sv[w]; i = si[w]; }
    pv[(size_t)row * nchunks + c] = b;
    pi[(size_t)row * nchunks + c] = i;
  }
}

hipError_t launch_argmax_rows(int dtype, const void* X, int rows, int V, int nchunks, float* pv, int* pi,
                              hipStream_t st) {
  int chunk = (V + nchunks - 1) / nchunks;
  chunk = (chunk + 7) / 8 * 8;  // keeps every chunk start 16-byte aligned (V % 8 == 0)
  dim3 grid(rows, nchunks), block(256);
  if (dtype == 0)
    hipLaunchKernelGGL(argmax_rows_kernel<float>, grid, block, 0, st, (const float*)X, V, chunk, nchunks, pv, pi);
  else
    hipLaunchKernelGGL(argmax_rows_kernel<bf16_t>, grid, block, 0, st, (const bf16_t*)X, V, chunk, nchunks, pv, pi);
  return hipGetLastError();
}

// best (value, index) over the nchunks partials of one row, by the calling wave (all lanes get it)
__device__ __forceinline__ int am_row_reduce(const float* __restrict__ pv, const int* __restrict__ pi, int nchunks,
                                             int lane) {
  float b = -INFINITY;
  int i = 0x7fffffff;
  // the first 256 partials are loaded before any is compared (one memory round trip for up to 256)
  float v4[4];
  int k4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = lane + 64 * u;
    v4[u] = c < nchunks ? pv[c] : -INFINITY;
    k4[u] = c < nchunks ? pi[c] : 0x7fffffff;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (am_better(v4[u], k4[u], b, i)) { b = v4[u]; i = k4[u]; }
  for (int c = lane + 256; c < nchunks; c += 64) {
    const float v = pv[c];
    const int k = pi[c];
    if (am_better(v, k, b, i)) { b = v; i = k; }
  }
  am_wave_reduce(b, i, 64);
  return i;
}

// one workgroup of 16 waves per row: every thread reduces a strided share of the partials, then the waves
// are combined in a fixed order
__global__ __launch_bounds__(1024) void argmax_final_kernel(const float* __restrict__ pv, const int* __restrict__ pi,
                                                            int rows, int nchunks, int* __restrict__ out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int row = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* v = pv + (size_t)row * nchunks;
  const int* ix = pi + (size_t)row * nchunks;
  float b = -INFINITY;
  int i = 0x7fffffff;
  // the first 12 chunks of every thread (12288 partials: the whole row of a 16-column-tile LM head at
  // V < 196608) are loaded before any is compared; the winner does not depend on the visiting order
  // (ties go to the smaller index)
  constexpr int U = 12;
  float x[U];
  int k[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = threadIdx.x + u * 1024;
    x[u] = c < nchunks ? v[c] : -INFINITY;
    k[u] = c < nchunks ? ix[c] : 0x7fffffff;
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (am_better(x[u], k[u], b, i)) { b = x[u]; i = k[u]; }
  for (int c = threadIdx.x + U * 1024; c < nchunks; c += 1024)
    if (am_better(v[c], ix[c], b, i)) { b = v[c]; i = ix[c]; }
  am_wave_reduce(b, i, 64);
  if (lane == 0) { sv[wave] = b; si[wave] = i; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 16; ++w)
      if (am_better(sv[w], si[w], b, i)) { b = sv[w]; i = si[w]; }
    out[row] = i;
  }
}

hipError_t launch_argmax_final(const float* pv, const int* pi, int rows, int nchunks, int* out, hipStream_t st) {
  hipLaunchKernelGGL(argmax_final_kernel, dim3(rows), dim3(1024), 0, st, pv, pi, rows, nchunks, out);
  return hipGetLastError();
}

// inclusive scan over the 1024 threads of the block: a shuffle scan inside each wave, then each wave adds
// the totals of the waves before it (two barriers; buf holds the 16 wave totals)
__device__ __forceinline__ int block_scan_incl(int v, int* buf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, PE_WAVE);
    if (lane >= off) v += t;
  }
  if (lane == 63) buf[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += buf[w];
  __syncthreads();  // buf is reused by the next scan
  return v + add;
}

// Greedy acceptance (the target verifies the K drafts in one pass; standard rule, greedy form) and the
// batch-metadata rebuild. One workgroup of 1024 threads; thread b handles request b (B <= 1024).
__global__ __launch_bounds__(1024) void accept_compact_kernel(
    const float* __restrict__ pv, const int* __restrict__ pi, int nchunks, int B, int K,
    const int* __restrict__ draft, const uint8_t* __restrict__ finished, const int* __restrict__ req_slot,
    const int* __restrict__ seq_len, int* __restrict__ t_ws, int* __restrict__ accept_len,
    int* __restrict__ cu_accept, int* __restrict__ out_tokens, int* __restrict__ keep_index,
    int* __restrict__ n_keep, int* __restrict__ slot_next, int* __restrict__ seq_next, int* __restrict__ last_next) {
  __shared__ int buf[16];  // per-wave totals of the block scans
  const int tid = threadIdx.x;
  const int rows = B * (K + 1);
  // this request's draft tokens, loaded before anything waits (K <= max_k <= PE_MAX_K = 16)
  constexpr int KMAX = 16;
  int dk[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) dk[i] = (tid < B && i < K) ? draft[(size_t)tid * K + i] : -1;
  // target argmax t[b][i] from the scan partials: one wave per row
  {
    const int wave = tid >> 6, lane = tid & 63;
    for (int r = wave; r < rows; r += 16) {
      const int i = am_row_reduce(pv + (size_t)r * nchunks, pi + (size_t)r * nchunks, nchunks, lane);
      if (lane == 0) t_ws[r] = i;
    }
  }
  __syncthreads();
  int n = 0, al = 0, bonus = 0, keep = 0;
  if (tid < B) {
    const int* t = t_ws + (size_t)tid * (K + 1);
    int tk[KMAX + 1];
#pragma unroll
    for (int i = 0; i <= KMAX; ++i) tk[i] = i <= K ? t[i] : 0;  // all loads in flight together
    // accepted prefix: the first position whose draft differs from the target argmax
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (n == i && i < K && dk[i] == tk[i]) n = i + 1;
    al = n + 1;
#pragma unroll
    for (int i = 0; i <= KMAX; ++i)
      if (i == n) bonus = tk[i];
    accept_len[tid] = al;
    keep = finished ? (finished[tid] == 0 ? 1 : 0) : 1;
  }
  const int incl = block_scan_incl(al, buf);
  const int excl = incl - al;
  if (tid < B) {
    cu_accept[tid] = excl;
    if (tid == B - 1) cu_accept[B] = incl;
    const int* t = t_ws + (size_t)tid * (K + 1);
    for (int i = 0; i < al; ++i) out_tokens[excl + i] = t[i];
  }
  const int kincl = block_scan_incl(keep, buf);
  if (tid < B && keep) {
    const int pos = kincl - 1;
    keep_index[pos] = tid;
    slot_next[pos] = req_slot[tid];
    seq_next[pos] = seq_len[tid] + al;
    last_next[pos] = bonus;
  }
  if (tid == B - 1) n_keep[0] = kincl;
}

hipError_t launch_accept_compact(const float* pv, const int* pi, int nchunks, int B, int K, const int* draft,
                                 const uint8_t* finished, const int* req_slot, const int* seq_len, int* t_ws,
                                 int* accept_len, int* cu_accept, int* out_tokens, int* keep_index, int* n_keep,
                                 int* slot_next, int* seq_next, int* last_next, hipStream_t st) {
  hipLaunchKernelGGL(accept_compact_kernel, dim3(1), dim3(1024), 0, st, pv, pi, nchunks, B, K, draft, finished,
                     req_slot, seq_len, t_ws, accept_len, cu_accept, out_tokens, keep_index, n_keep, slot_next,
                     seq_next, last_next);
  return hipGetLastError();
}

}  // namespace pe
