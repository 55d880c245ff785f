// Vocabulary argmax (draft tokens on the fp32 path, target tokens in verify) and the greedy
// accept / batch-metadata rebuild.
//
// Argmax convention everywhere: the largest value wins; among equal values the lowest index.
#include "common.h"
#include "kernels.h"

namespace pe {

// 16 bytes of a row that is read once (target or draft logits): non-temporal load
template <typename T>
__device__ __forceinline__ uint4 nt_load16(const T* p) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_t*)p));
}

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
  int i = begin + threadIdx.x * VEC;
  // four 16-byte loads in flight per thread, then their elements in order
  for (; i + 3 * 256 * VEC + VEC <= end; i += 4 * 256 * VEC) {
    union { uint4 u; T e[VEC]; } ld[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ld[q].u = nt_load16(x + i + q * 256 * VEC);
#pragma unroll
    for (int q = 0; q < 4; ++q)  // increasing index order, so a strict > keeps the first maximum
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float v = to_f32<T>(ld[q].e[e]);
        if (v > best) { best = v; bi = i + q * 256 * VEC + e; }
      }
  }
  for (; i < end; i += 256 * VEC) {
    if (i + VEC <= end) {
      union { uint4 u; T e[VEC]; } ld;
      ld.u = nt_load16(x + i);
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
  am_group_reduce<64>(best, bi);
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
  am_group_reduce<64>(b, i);
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
  am_group_reduce<64>(b, i);
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

// Batch-metadata rebuild after the acceptance decision (thread b < B holds request b's accept_len al, the
// emitted token after its accepted drafts, and keep = not finished): cu_accept = exclusive scan of al,
// out_tokens[cu_accept[b] + i] = t[b][i] for i < al, stable compaction of the surviving requests.
__device__ __forceinline__ void compact_tail(int al, int bonus, int keep, int* buf, int B, int K,
                                             const int* __restrict__ t_ws, const int* __restrict__ req_slot,
                                             const int* __restrict__ seq_len, int* __restrict__ cu_accept,
                                             int* __restrict__ out_tokens, int* __restrict__ keep_index,
                                             int* __restrict__ n_keep, int* __restrict__ slot_next,
                                             int* __restrict__ seq_next, int* __restrict__ last_next) {
  const int tid = threadIdx.x;
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
  // target argmax t[b][i] from the scan partials: one thread per row when rows have few partials (large
  // batches: many rows, few chunks each), else one wave per row
  if (nchunks <= 32) {
    for (int r = tid; r < rows; r += 1024) {
      const float* v = pv + (size_t)r * nchunks;
      const int* ix = pi + (size_t)r * nchunks;
      float b = -INFINITY;
      int i = 0x7fffffff;
      for (int c = 0; c < nchunks; ++c)
        if (am_better(v[c], ix[c], b, i)) { b = v[c]; i = ix[c]; }
      t_ws[r] = i;
    }
  } else {
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
  compact_tail(al, bonus, keep, buf, B, K, t_ws, req_slot, seq_len, cu_accept, out_tokens, keep_index, n_keep,
               slot_next, seq_next, last_next);
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

// ---- sampled verification (temperature > 0): standard speculative sampling with a greedy drafter ------
// p_i = softmax(T[b][i] / temperature). Draft x_i is accepted iff u[b][i] < p_i(x_i); at the first rejection
// n the emitted token is drawn with v[b][n] from p_n without x_n (inverse CDF over the vocabulary); after K
// acceptances the bonus token is drawn with v[b][K] from p_K.

__device__ __forceinline__ void sm_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

// (max, sum of exp(x - max)) of x = logit / temperature over one chunk of one row. WPC waves per chunk: 1 (four
// chunks per workgroup, no block barrier; many rows) or 4 (one chunk per workgroup; few rows, so more waves
// share the scan). Each lane keeps its running pair over its elements in order (32 at a time: the batch
// maximum, one rescale, then the batch's exponentials); lanes merge by xor-shuffles
// in a fixed pattern, then (WPC = 4) the four waves in order.
template <typename T, int WPC>
__global__ __launch_bounds__(256) void softmax_stats_kernel(const T* __restrict__ X, int V, int chunk, int nchunks,
                                                            float inv_temp, float* __restrict__ pm,
                                                            float* __restrict__ ps) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int STEP = 64 * WPC * VEC;  // elements one pass of the chunk's waves covers
  __shared__ float sm[4], ss[4];
  const int row = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.y * (4 / WPC) + wave / WPC;
  if (WPC == 1 && c >= nchunks) return;  // (WPC = 4: the grid holds exactly nchunks workgroups)
  const int begin = c * chunk;
  const int end = min(V, begin + chunk);
  const T* x = X + (size_t)row * V;
  float m = -INFINITY, s = 0.f;
  auto add = [&](float v) {
    v *= inv_temp;
    if (v > m) {
      s = s * __expf(m - v) + 1.f;
      m = v;
    } else {
      s += __expf(v - m);
    }
  };
  int i = begin + ((wave % WPC) * 64 + lane) * VEC;
  // four 16-byte loads in flight per lane, then their elements in order
  for (; i + 3 * STEP + VEC <= end; i += 4 * STEP) {
    union { uint4 u; T e[VEC]; } ld[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ld[q].u = nt_load16(x + i + q * STEP);
    // the batch's maximum first: one rescale per batch, then a plain sum of exponentials (measured: sampled
    // verify at GPT-OSS B 64 K 10 108 -> 92 us, Qwen B 128 K 7 112 -> 94 us, against a running
    // maximum per element with its branch)
    float v[4 * VEC], bm = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        v[q * VEC + e] = to_f32<T>(ld[q].e[e]) * inv_temp;
        bm = fmaxf(bm, v[q * VEC + e]);
      }
    if (bm > m) {
      s *= __expf(m - bm);
      m = bm;
    }
#pragma unroll
    for (int k = 0; k < 4 * VEC; ++k) s += __expf(v[k] - m);
  }
  for (; i < end; i += STEP) {
    if (i + VEC <= end) {
      union { uint4 u; T e[VEC]; } ld;
      ld.u = nt_load16(x + i);
#pragma unroll
      for (int e = 0; e < VEC; ++e) add(to_f32<T>(ld.e[e]));
    } else {
      for (int e = i; e < end; ++e) add(to_f32<T>(x[e]));
    }
  }
  for (int off = 1; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off, PE_WAVE), s2 = __shfl_xor(s, off, PE_WAVE);
    sm_merge(m, s, m2, s2);
  }
  if (WPC == 4) {
    if (lane == 0) { sm[wave] = m; ss[wave] = s; }
    __syncthreads();
    if (threadIdx.x != 0) return;
    m = sm[0];
    s = ss[0];
    for (int w = 1; w < 4; ++w) sm_merge(m, s, sm[w], ss[w]);
  } else if (lane != 0) {
    return;
  }
  pm[(size_t)row * nchunks + c] = m;
  ps[(size_t)row * nchunks + c] = s;
}

// One workgroup per request. Every position's row maximum and total (its chunk statistics merged by one
// wave in a fixed order), draft weight and acceptance test are computed up front, one wave per position;
// one thread then takes the first rejection n. The draw at n finds its chunk by a prefix over the chunk
// totals and its token by a block scan inside the chunk.
template <typename T>
__global__ __launch_bounds__(256) void sample_decide_kernel(const T* __restrict__ X, int V, int chunk, int nchunks,
                                                            float inv_temp, const float* __restrict__ pm,
                                                            const float* __restrict__ ps, int K,
                                                            const int* __restrict__ draft, const float* __restrict__ u,
                                                            const float* __restrict__ v, int* __restrict__ t_ws,
                                                            int* __restrict__ accept_len) {
  constexpr int PMAX = 17;  // positions per request (K <= 16)
  __shared__ float cm[PE_SAMPLE_MAX_CHUNKS], cs[PE_SAMPLE_MAX_CHUNKS];
  __shared__ float red[256];
  __shared__ float sM[PMAX], sS[PMAX], sEd[PMAX];
  __shared__ int sAcc[PMAX];
  __shared__ float sh_base;
  __shared__ int sh_k, sh_x, sh_n;
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // per position: (max, total) of the row, the draft's weight and the acceptance test
  for (int i = wave; i <= K; i += 4) {
    const int r = b * (K + 1) + i;
    float m = -INFINITY, sum = 0.f;
    for (int c = lane; c < nchunks; c += 64) sm_merge(m, sum, pm[(size_t)r * nchunks + c], ps[(size_t)r * nchunks + c]);
    for (int off = 1; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m, off, PE_WAVE), s2 = __shfl_xor(sum, off, PE_WAVE);
      sm_merge(m, sum, m2, s2);
    }
    if (lane == 0) {
      sM[i] = m;
      sS[i] = sum;
      float ed = 0.f;
      int acc = 0;
      if (i < K) {
        const int d = draft[(size_t)b * K + i];
        if (d >= 0 && d < V) {
          ed = __expf(to_f32<T>(X[(size_t)r * V + d]) * inv_temp - m);
          acc = u[(size_t)b * K + i] < ed / sum ? 1 : 0;
        }
      }
      sEd[i] = ed;
      sAcc[i] = acc;
    }
  }
  __syncthreads();
  if (tid == 0) {
    int n = K;
    for (int i = 0; i < K; ++i)
      if (!sAcc[i]) { n = i; break; }
    sh_n = n;
  }
  __syncthreads();
  const int n = sh_n;
  if (tid < n) t_ws[(size_t)b * (K + 1) + tid] = draft[(size_t)b * K + tid];  // the accepted drafts
  const int r = b * (K + 1) + n;
  for (int c = tid; c < nchunks; c += 256) {
    cm[c] = pm[(size_t)r * nchunks + c];
    cs[c] = ps[(size_t)r * nchunks + c];
  }
  const float M = sM[n], S = sS[n];
  const T* x = X + (size_t)r * V;
  int excl = -1;
  float ed = 0.f, theta;
  if (n < K) {  // rejection: draw from p_n without the draft
    const int d = draft[(size_t)b * K + n];
    excl = d >= 0 && d < V ? d : -1;
    ed = sEd[n];
    theta = v[(size_t)b * (K + 1) + n] * (S - ed);
  } else {  // every draft accepted: the bonus draw from p_K
    theta = v[(size_t)b * (K + 1) + K] * S;
  }
  __syncthreads();
  // the chunk holding the draw: first chunk whose running total (without the excluded token) passes theta
  if (tid == 0) {
    float acc = 0.f;
    int k = -1, last = 0;
    for (int c = 0; c < nchunks; ++c) {
      float w = cs[c] * __expf(cm[c] - M);
      if (excl >= c * chunk && excl < (c + 1) * chunk) w = fmaxf(w - ed, 0.f);
      if (w > 0.f) last = c;
      if (k < 0 && acc + w > theta) { k = c; sh_base = acc; }
      acc += w;
    }
    if (k < 0) {  // rounding left theta at or past the total: the last chunk with weight
      k = last;
      float a2 = 0.f;
      for (int c = 0; c < last; ++c) {
        float w = cs[c] * __expf(cm[c] - M);
        if (excl >= c * chunk && excl < (c + 1) * chunk) w = fmaxf(w - ed, 0.f);
        a2 += w;
      }
      sh_base = a2;
    }
    sh_k = k;
    sh_x = -1;
  }
  __syncthreads();
  const int k = sh_k;
  const int cb = k * chunk, ce = min(V, cb + chunk);
  const int per = (ce - cb + 255) / 256;
  const int lb = cb + tid * per, le = min(ce, lb + per);
  auto wt = [&](int e) { return e == excl ? 0.f : __expf(to_f32<T>(x[e]) * inv_temp - M); };
  float local = 0.f;
  for (int e = lb; e < le; ++e) local += wt(e);
  // inclusive block scan of the per-thread totals (thread order); thread j owns [lo_j, hi_j) with
  // lo_j = base + scan[j - 1] and hi_j = base + scan[j] = lo_{j+1}, the last thread also everything past
  // the chunk's total, so exactly one thread owns theta (theta >= base)
  red[tid] = local;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const float add = tid >= off ? red[tid - off] : 0.f;
    __syncthreads();
    red[tid] += add;
    __syncthreads();
  }
  const float base = sh_base;
  const float lo = base + (tid == 0 ? 0.f : red[tid - 1]);
  const float hi = tid == 255 ? INFINITY : base + red[tid];
  if (lo <= theta && theta < hi) {
    float a = lo;
    int pick = -1;
    for (int e = lb; e < le; ++e) {
      const float w = wt(e);
      if (w > 0.f) {
        pick = e;
        a += w;
        if (a > theta) break;
      }
    }
    sh_x = pick;  // rounding may end the range before theta: then its last token with weight
  }
  __syncthreads();
  if (tid == 0) {
    int xs = sh_x;
    if (xs < 0) {  // the owner holds no weight: the last token of the chunk with weight
      xs = cb;
      for (int e = ce - 1; e >= cb; --e)
        if (wt(e) > 0.f) { xs = e; break; }
    }
    t_ws[r] = xs;
  }
  if (tid == 0) accept_len[b] = n + 1;
}

// metadata rebuild for the sampled path: one workgroup of 1024 threads, thread b < B handles request b
__global__ __launch_bounds__(1024) void sampled_compact_kernel(int B, int K, const int* __restrict__ t_ws,
                                                               const int* __restrict__ accept_len_in,
                                                               const uint8_t* __restrict__ finished,
                                                               const int* __restrict__ req_slot,
                                                               const int* __restrict__ seq_len,
                                                               int* __restrict__ cu_accept, int* __restrict__ out_tokens,
                                                               int* __restrict__ keep_index, int* __restrict__ n_keep,
                                                               int* __restrict__ slot_next, int* __restrict__ seq_next,
                                                               int* __restrict__ last_next) {
  __shared__ int buf[16];
  const int tid = threadIdx.x;
  int al = 0, bonus = 0, keep = 0;
  if (tid < B) {
    al = accept_len_in[tid];
    bonus = t_ws[(size_t)tid * (K + 1) + al - 1];
    keep = finished ? (finished[tid] == 0 ? 1 : 0) : 1;
  }
  compact_tail(al, bonus, keep, buf, B, K, t_ws, req_slot, seq_len, cu_accept, out_tokens, keep_index, n_keep,
               slot_next, seq_next, last_next);
}

hipError_t launch_sampled_verify(int dtype, const void* X, int B, int K, int V, int nchunks, float temperature,
                                 const int* draft, const float* u, const float* v, const uint8_t* finished,
                                 const int* req_slot, const int* seq_len, float* pm, float* ps, int* t_ws,
                                 int* accept_len, int* cu_accept, int* out_tokens, int* keep_index, int* n_keep,
                                 int* slot_next, int* seq_next, int* last_next, hipStream_t st) {
  if (nchunks < 1 || nchunks > PE_SAMPLE_MAX_CHUNKS || B < 1 || B > 1024 || K < 1 || K > 16)
    return hipErrorInvalidValue;
  int chunk = (V + nchunks - 1) / nchunks;
  chunk = (chunk + 7) / 8 * 8;  // every chunk start 16-byte aligned (V % 8 == 0)
  const int rows = B * (K + 1);
  const float inv_temp = 1.f / temperature;
  // one wave per chunk once there are enough chunks to fill the compute units with them (measured: B 128 K 7
  // 119 -> 112 us; four waves per chunk stay faster for a few rows, B 1 K 3 20 against 23 us)
  const bool many = (long long)rows * nchunks >= 8192;
  if (dtype == 0) {
    if (many) hipLaunchKernelGGL((softmax_stats_kernel<float, 1>), dim3(rows, (nchunks + 3) / 4), dim3(256), 0, st,
                                 (const float*)X, V, chunk, nchunks, inv_temp, pm, ps);
    else hipLaunchKernelGGL((softmax_stats_kernel<float, 4>), dim3(rows, nchunks), dim3(256), 0, st, (const float*)X, V,
                            chunk, nchunks, inv_temp, pm, ps);
    hipLaunchKernelGGL(sample_decide_kernel<float>, dim3(B), dim3(256), 0, st, (const float*)X, V, chunk, nchunks,
                       inv_temp, pm, ps, K, draft, u, v, t_ws, accept_len);
  } else {
    if (many) hipLaunchKernelGGL((softmax_stats_kernel<bf16_t, 1>), dim3(rows, (nchunks + 3) / 4), dim3(256), 0, st,
                                 (const bf16_t*)X, V, chunk, nchunks, inv_temp, pm, ps);
    else hipLaunchKernelGGL((softmax_stats_kernel<bf16_t, 4>), dim3(rows, nchunks), dim3(256), 0, st, (const bf16_t*)X,
                            V, chunk, nchunks, inv_temp, pm, ps);
    hipLaunchKernelGGL(sample_decide_kernel<bf16_t>, dim3(B), dim3(256), 0, st, (const bf16_t*)X, V, chunk, nchunks,
                       inv_temp, pm, ps, K, draft, u, v, t_ws, accept_len);
  }
  hipLaunchKernelGGL(sampled_compact_kernel, dim3(1), dim3(1024), 0, st, B, K, t_ws, accept_len, finished, req_slot,
                     seq_len, cu_accept, out_tokens, keep_index, n_keep, slot_next, seq_next, last_next);
  return hipGetLastError();
}

}  // namespace pe
