// Drafter attention: request b's K new rows against its cache slot, causal inside the K block.
//
// Row j of request b sits at position L_b + j and sees cache positions 0 .. L_b + j (the L_b context
// positions plus new rows 0..j, whose rotated keys and values were just appended). Grouped-query
// attention: q head h reads kv head h / G. Scores are scaled by 1/sqrt(hd); softmax in fp32.
//
// bf16 path (gfx950 MFMA): one workgroup per (request, kv head, key split). The G*K query rows of the
// kv head form the MFMA column operand, so every staged key/value tile is used by all of them: scores are
// computed transposed, S^T = K_tile . Q^T (keys x rows), which leaves each lane owning one query row —
// the same row ownership as O^T = V^T . P^T — so the online-softmax rescaling needs no lane exchange
// beyond two xor-shuffles for the per-row max and sum. Key/value rounds are loaded into registers one
// round ahead of the round being multiplied (coalesced 16-byte loads), then staged in LDS: keys in the
// order the score tiles use (so that each lane's eight probabilities are eight consecutive keys), values
// transposed (dimension-major), so the V^T operand is one 16-byte LDS read per lane. Each (split,
// sub-stream) writes an unnormalised partial (O, m, l); a second kernel merges them in a fixed order
// (log-sum-exp), so results are independent of scheduling.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace pe {

#define ATTN_MAX_PARTIALS 1024  // split partials per query row

static inline int attn_sub_streams(int R) {
  const int RT = (R + 15) / 16;
  return RT == 1 ? 4 : RT == 2 ? 2 : 1;
}

static inline int attn_round_keys(int hd) { return hd == 128 ? 64 : 128; }

AttnPlan plan_attention(int B, int K, int Hq, int Hkv, int hd, int max_ctx) {
  AttnPlan p;
  const int R = (Hq / Hkv) * K;
  const int KEYS = attn_round_keys(hd);
  p.sub = attn_sub_streams(R);
  // Keys per split: a power of two, at least twice the query rows of a kv head (a split's fp32 partial,
  // R x (hd + 2) floats, then stays well below the keys it summarises) and at least the share that gives
  // ~1024 workgroups at full context, at most 1024 keys (measured on the MI355X: B 1 K 3 best at 64 keys,
  // B 8 K 11 at 256, B 32 K 7 at 256-1024, B 64 K 10 at 1024; whole staging rounds in every case).
  const long long want = (long long)B * Hkv * (long long)(max_ctx + K) / 1024;
  const long long need = std::max<long long>(std::max<long long>(2LL * R, want), KEYS);
  int chunk = KEYS;
  while (chunk < need && chunk < 1024) chunk *= 2;
  if (chunk < KEYS) chunk = KEYS;
  while ((max_ctx + K + chunk - 1) / chunk > ATTN_MAX_PARTIALS) chunk *= 2;
  p.chunk = chunk;
  p.nsplit = (max_ctx + K + chunk - 1) / chunk;
  // Workgroup order: with many splits per (request, kv head), the workgroups that run together take
  // neighbouring splits of few heads rather than the same split of many heads (measured on the MI355X:
  // GPT-OSS B 64 K 10, 9 splits, 211 -> 194 us per layer; Qwen B 128 K 7, 5 splits, 171 -> 176 us, so
  // it stays head-major there; B 8 K 11, 17 splits, unchanged)
  p.split_major = p.nsplit >= 8;
  return p;
}

size_t attn_partial_floats(int M, int Hq, int hd, const AttnPlan& p) {
  return (size_t)M * Hq * p.nsplit * (hd + 2);
}

// NW: waves per workgroup, 4 or (when more than 64 query rows share a kv head) 8; each wave owns one
// 16-row tile of the kv head's query rows
template <int HD, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3))) void attn_bf16_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kc,
                                                        const bf16_t* __restrict__ Vc,
                                                        const int* __restrict__ seq_len,
                                                        const int* __restrict__ req_slot, int K, int Hq, int Hkv,
                                                        int max_ctx, int n_slots, int chunk, int nsplit, int sub, int smaj,
                                                        float* __restrict__ part, float scale) {
  constexpr int KT = 32;                      // keys per MFMA key tile
  constexpr int KEYS = HD == 128 ? 64 : 128;  // keys staged per round (16 KiB of K and of V)
  constexpr int NKT = KEYS / KT;              // key tiles per round
  constexpr int STR = HD + 8;                 // sK row stride (elements), 16 B of padding
  constexpr int VSTR = KEYS + 8;              // sVt row stride (elements)
  constexpr int HS = HD / 32;                 // k-steps of the score contraction
  constexpr int CT = HD / 16;                 // 16-column tiles of the output
  constexpr int C8 = HD / 8;                  // 16-byte pieces per key row
  constexpr int PK = KEYS * C8 / (NW * 64);   // keys staged per thread per round (4 or 2)
  constexpr int NR = 1;
  // sVt row d holds key k at column k ^ 8 vsw(d): rotating whole 8-key blocks keeps every read of 8
  // consecutive keys contiguous while the staging writes (4 or 2 keys of 8 dimensions per thread) hit
  // distinct banks
  auto vsw = [](int dim) { return HD == 128 ? (dim >> 4) & 7 : (dim >> 3) & 14; };
  // sK row of key k within a round: key 32 a' + 8 a + 4 h + r sits at row 32 a' + 16 h + 4 a + r, so score
  // tile h's MFMA row 4 a + r is key 8 a + 4 h + r
  __shared__ __attribute__((aligned(16))) char smem[(KEYS * STR + HD * VSTR) * sizeof(bf16_t)];
  bf16_t* sK = (bf16_t*)smem;                 // [key][dim]
  bf16_t* sVt = sK + KEYS * STR;              // [dim][key]

  const int bg = smaj ? blockIdx.y : blockIdx.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const int split = smaj ? blockIdx.x : blockIdx.y;
  const int G = Hq / Hkv, R = G * K, RT = (R + 15) / 16;
  const int L = seq_len[b], slot = req_slot[b];
  if (slot < 0 || slot >= n_slots || L < 0 || L + K > max_ctx) return;
  const int Lk = L + K;
  const int k_begin = split * chunk;
  if (k_begin >= Lk) return;
  const int k_end = min(Lk, k_begin + chunk);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  int rt0, nrt, ks_id;
  if (sub > 1) {  // RT * sub == NW: waves share row tiles and take alternate key tiles
    rt0 = wave % RT;
    nrt = 1;
    ks_id = wave / RT;
  } else {  // wave w owns row tile w
    rt0 = wave;
    nrt = wave < RT ? 1 : 0;
    ks_id = 0;
  }

  const size_t head_off = ((size_t)slot * Hkv + g) * max_ctx * HD;
  const bf16_t* kb = Kc + head_off;
  const bf16_t* vb = Vc + head_off;

  // staging: this thread moves keys PK kq .. PK kq + PK - 1, dimensions 8 c8 .. 8 c8 + 7 of each round.
  // Keys past k_end are clamped to the last valid key (finite values; their scores are masked out).
  const int kq = tid / C8, c8 = tid % C8;
  typedef bf16x8_t RoundRegs[PK];
  RoundRegs rkA, rvA;
  auto gload = [&](int base, RoundRegs& rk, RoundRegs& rv) {
    if (base + KEYS <= k_end) {  // the whole round is inside the split: one address, immediate offsets
      const size_t o = (size_t)(base + PK * kq) * HD + 8 * c8;
      // context keys and values are read once: non-temporal loads keep them from displacing other lines
      // (measured: Qwen B 128 K 7 172 -> 162 us per layer; GPT-OSS B 64 K 10 unchanged)
#pragma unroll
      for (int q = 0; q < PK; ++q) {
        rk[q] = __builtin_nontemporal_load((const bf16x8_t*)(kb + o + q * HD));
        rv[q] = __builtin_nontemporal_load((const bf16x8_t*)(vb + o + q * HD));
      }
    } else {
#pragma unroll
      for (int q = 0; q < PK; ++q) {
        const int kp = min(base + PK * kq + q, k_end - 1);
        rk[q] = *(const bf16x8_t*)(kb + (size_t)kp * HD + 8 * c8);
        rv[q] = *(const bf16x8_t*)(vb + (size_t)kp * HD + 8 * c8);
      }
    }
  };
  auto sstore = [&](const RoundRegs& rk, const RoundRegs& rv) {
#pragma unroll
    for (int q = 0; q < PK; ++q) {
      const int k = PK * kq + q;  // k = 32 a' + 8 a + 4 h + r  ->  row 32 a' + 16 h + 4 a + r
      const int row = (k >> 5) * 32 + ((k >> 2) & 1) * 16 + 4 * ((k >> 3) & 3) + (k & 3);
      *(bf16x8_t*)(sK + row * STR + 8 * c8) = rk[q];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16_t* dst = sVt + (8 * c8 + e) * VSTR + ((PK * kq) ^ (8 * vsw(8 * c8 + e)));
      const uint32_t w0 = (uint32_t)(uint16_t)rv[0][e] | ((uint32_t)(uint16_t)rv[1][e] << 16);
      if (PK == 4) {
        uint2 w;
        w.x = w0;
        w.y = (uint32_t)(uint16_t)rv[PK - 2][e] | ((uint32_t)(uint16_t)rv[PK - 1][e] << 16);
        *(uint2*)dst = w;
      } else {
        *(uint32_t*)dst = w0;
      }
    }
  };

  gload(k_begin, rkA, rvA);

  const bf16x8_t zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  bf16x8_t qf[NR][HS];
  f32x4_t o[NR][CT];
  float m_run[NR], l_run[NR];
#pragma unroll
  for (int t = 0; t < NR; ++t) {
    m_run[t] = -1e30f;
    l_run[t] = 0.f;
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) qf[t][hs] = zero8;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) o[t][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (t < nrt) {
      const int row = (rt0 + 4 * t) * 16 + lr;
      if (row < R) {
        const int hl = row / K, j = row % K;
        const bf16_t* q = Q + ((size_t)(b * K + j) * Hq + (g * G + hl)) * HD;
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) qf[t][hs] = *(const bf16x8_t*)(q + 32 * hs + 8 * lq);
      }
    }
  }

  // (measured: a second register set two rounds ahead made the 8-wave kernels slower, 222 -> 262 us per
  // GPT-OSS layer: its registers cost the second workgroup per compute unit)
  for (int base = k_begin; base < k_end; base += KEYS) {
    if (base != k_begin) __syncthreads();  // every wave is done with the previous round's tiles
    sstore(rkA, rvA);
    __syncthreads();
    if (base + KEYS < k_end) gload(base + KEYS, rkA, rvA);
    // a round every query row fully sees (all its keys are context keys, inside the split) on a straight
    // path: all score products, one running-max update for the round's keys, all value products (head
    // dimension 64 only: with 128 the path's registers cost the 8-wave kernel its second workgroup per
    // compute unit. Measured: GPT-OSS B 64 K 10 224 -> 210 us per layer; with 128 included, Qwen B 8 K 11 went 28 -> 31 us)
    if (HD == 64 && nrt > 0 && sub == 1 && base + KEYS <= k_end && base + KEYS <= L + 1) {
      f32x4_t sc[NKT][2];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        bf16x8_t ka[HS][2];
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) {
          ka[hs][0] = *(const bf16x8_t*)(sK + (kt * KT + lr) * STR + 32 * hs + 8 * lq);
          ka[hs][1] = *(const bf16x8_t*)(sK + (kt * KT + 16 + lr) * STR + 32 * hs + 8 * lq);
        }
        sc[kt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        sc[kt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) {
          sc[kt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[hs][0], qf[0][hs], sc[kt][0], 0, 0, 0);
          sc[kt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[hs][1], qf[0][hs], sc[kt][1], 0, 0, 0);
        }
      }
      float rmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) rmax = fmaxf(rmax, fmaxf(sc[kt][0][r], sc[kt][1][r]));
      rmax = rows_max(rmax);
      const float mnew = fmaxf(m_run[0], rmax * scale);
      float psum = 0.f;
      bf16x8_t pf[NKT];
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        float pe[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {  // element e: key base + kt KT + 8 lq + e
          pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(e < 4 ? sc[kt][0][e] : sc[kt][1][e - 4], scale, -mnew));
          psum += pe[e];
        }
        const u32x4_t pk = {f32x2_to_bf16x2(pe[0], pe[1]), f32x2_to_bf16x2(pe[2], pe[3]),
                            f32x2_to_bf16x2(pe[4], pe[5]), f32x2_to_bf16x2(pe[6], pe[7])};
        pf[kt] = __builtin_bit_cast(bf16x8_t, pk);
      }
      const float alpha = __builtin_amdgcn_exp2f(m_run[0] - mnew);
      psum = rows_sum(psum);
      l_run[0] = l_run[0] * alpha + psum;
      m_run[0] = mnew;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[0][ct][r] *= alpha;
      }
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        bf16x8_t va[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          va[ct] = *(const bf16x8_t*)(sVt + (ct * 16 + lr) * VSTR + ((kt * KT + 8 * lq) ^ (8 * vsw(ct * 16 + lr))));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o[0][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ct], pf[kt], o[0][ct], 0, 0, 0);
      }
    } else {
      if (nrt > 0) {
        for (int kt = 0; kt < NKT; ++kt) {
          const int tb = base + kt * KT;
          if (tb >= k_end) break;
          if (sub > 1 && (((tb - k_begin) / KT) % sub) != ks_id) continue;
          bf16x8_t pf[NR];
          float alpha[NR];
#pragma unroll
          for (int t = 0; t < NR; ++t) {
            pf[t] = zero8;
            alpha[t] = 1.f;
            if (t >= nrt) continue;
            f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            // every key fragment of the tile is read before the first product, so the LDS reads overlap
            // instead of each product waiting for its own
            bf16x8_t ka[HS][2];
#pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
              ka[hs][0] = *(const bf16x8_t*)(sK + (kt * KT + lr) * STR + 32 * hs + 8 * lq);
              ka[hs][1] = *(const bf16x8_t*)(sK + (kt * KT + 16 + lr) * STR + 32 * hs + 8 * lq);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
              s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[hs][0], qf[t][hs], s0, 0, 0, 0);
              s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[hs][1], qf[t][hs], s1, 0, 0, 0);
            }
            const int row = (rt0 + 4 * t) * 16 + lr;
            float psum = 0.f, pe[8], mnew;
            if (tb + KT <= L + 1 && tb + KT <= k_end) {
              // every query row sees every key of the tile (row j sees keys < L + j + 1): no mask; the
              // scale (which includes log2 e, so scores are in log2 units) is applied inside the exponent
              const float sr[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
              float rmax = fmaxf(fmaxf(fmaxf(sr[0], sr[4]), fmaxf(sr[1], sr[5])),
                                 fmaxf(fmaxf(sr[2], sr[6]), fmaxf(sr[3], sr[7])));
              rmax = rows_max(rmax);  // over the 4 lanes (l, l ^ 16, l ^ 32, l ^ 48) of query row lr
              mnew = fmaxf(m_run[t], rmax * scale);
#pragma unroll
              for (int e = 0; e < 8; ++e) {  // pf element e: key tb + 8 lq + e
                const int r = e & 3, hi = e >> 2;
                pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sr[4 * hi + r], scale, -mnew));
                psum += pe[e];
              }
            } else {
              const int lim = row < R ? min(k_end, L + (row % K) + 1) : 0;  // visible keys: < lim
              float sv[8];
              float tmax = -INFINITY;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int k0 = tb + 8 * lq + r, k1 = k0 + 4;  // keys of score rows 4 lq + r of tiles 0 and 1
                sv[r] = k0 < lim ? s0[r] * scale : -INFINITY;
                sv[4 + r] = k1 < lim ? s1[r] * scale : -INFINITY;
                tmax = fmaxf(tmax, fmaxf(sv[r], sv[4 + r]));
              }
              tmax = rows_max(tmax);
              mnew = fmaxf(m_run[t], tmax);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                pe[e] = __builtin_amdgcn_exp2f(sv[e] - mnew);
                psum += pe[e];
              }
            }
            alpha[t] = __builtin_amdgcn_exp2f(m_run[t] - mnew);
            typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
            const u32x4_t pk = {f32x2_to_bf16x2(pe[0], pe[1]), f32x2_to_bf16x2(pe[2], pe[3]),
                                f32x2_to_bf16x2(pe[4], pe[5]), f32x2_to_bf16x2(pe[6], pe[7])};
            pf[t] = __builtin_bit_cast(bf16x8_t, pk);
            psum = rows_sum(psum);
            l_run[t] = l_run[t] * alpha[t] + psum;
            m_run[t] = mnew;
          }
          // the running max rarely moves after the first tiles: rescale only when some lane's did (a
          // wave-uniform branch of its own, so the common case costs no multiplies or selects)
#pragma unroll
          for (int t = 0; t < NR; ++t) {
            if (t < nrt && __any(alpha[t] != 1.f)) {
#pragma unroll
              for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[t][ct][r] *= alpha[t];
            }
          }
          // value fragments likewise: all reads first, then the products
          bf16x8_t va[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            va[ct] = *(const bf16x8_t*)(sVt + (ct * 16 + lr) * VSTR + ((kt * KT + 8 * lq) ^ (8 * vsw(ct * 16 + lr))));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
            for (int t = 0; t < NR; ++t) {
              if (t >= nrt) continue;
              o[t][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ct], pf[t], o[t][ct], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  if (sub > 1) {
    // merge the key sub-streams of each row tile inside the workgroup (fixed order), so that a split
    // leaves one partial per row: sub-stream s > 0 parks (O, m, l) in LDS, sub-stream 0 folds them in
    static_assert((HD + 2) * 16 * 3 * sizeof(float) <= sizeof(smem), "merge scratch exceeds LDS");
    float* red = (float*)smem;
    __syncthreads();  // every wave is done with the staged tiles
    if (ks_id > 0) {
      float* slot = red + (size_t)((ks_id - 1) * RT + rt0) * 16 * (HD + 2) + lr * (HD + 2);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) slot[ct * 16 + 4 * lq + r] = o[0][ct][r];
      if (lq == 0) {
        slot[HD] = m_run[0];
        slot[HD + 1] = l_run[0];
      }
    }
    __syncthreads();
    if (ks_id > 0) return;
    for (int q = 1; q < sub; ++q) {
      const float* slot = red + (size_t)((q - 1) * RT + rt0) * 16 * (HD + 2) + lr * (HD + 2);
      const float mq = slot[HD], lqs = slot[HD + 1];
      const float mn = fmaxf(m_run[0], mq);
      const float a0 = __builtin_amdgcn_exp2f(m_run[0] - mn), aq = __builtin_amdgcn_exp2f(mq - mn);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[0][ct][r] = o[0][ct][r] * a0 + slot[ct * 16 + 4 * lq + r] * aq;
      l_run[0] = l_run[0] * a0 + lqs * aq;
      m_run[0] = mn;
    }
  }

#pragma unroll
  for (int t = 0; t < NR; ++t) {
    if (t >= nrt) continue;
    const int row = (rt0 + 4 * t) * 16 + lr;
    if (row >= R) continue;
    const int hl = row / K, j = row % K;
    const size_t rid = ((size_t)b * Hq + (g * G + hl)) * K + j;
    float* dst = part + (rid * nsplit + split) * (HD + 2);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[ct * 16 + 4 * lq + r] = o[t][ct][r];
    if (lq == 0) {
      dst[HD] = m_run[t];
      dst[HD + 1] = l_run[t];
    }
  }
}

// O[b*K + j][h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits that hold keys (m in log2
// units, as the partial kernel keeps its scores). One workgroup per query row. Every wave computes the
// max and the denominator itself (lane l takes splits l, l + 64, ...; the denominator is summed in four
// residue classes of 64-split blocks, added in a fixed order), and wave w accumulates the numerator of
// splits w, w + 4, ... (HD / 64 columns per lane); the four numerators are added in a fixed order. All
// loads of the first rounds are issued before any result is used, so the kernel waits on memory once.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part, bf16_t* __restrict__ O,
                                                           const int* __restrict__ seq_len,
                                                           const int* __restrict__ req_slot, int K, int Hq,
                                                           int max_ctx, int n_slots, int chunk, int nsplit) {
  constexpr int CPT = HD / 64;  // columns per lane
  constexpr int PF = 12;        // numerator splits per wave loaded up front
  constexpr int QB = 4;         // 64-split blocks of (m, l) loaded up front
  constexpr int RS = HD + 2;    // floats per partial
  const int rid = blockIdx.x;
  const int j = rid % K, h = (rid / K) % Hq, b = rid / (K * Hq);
  bf16_t* out = O + ((size_t)(b * K + j) * Hq + h) * HD;
  const int L = seq_len[b], slot = req_slot[b];
  if (slot < 0 || slot >= n_slots || L < 0 || L + K > max_ctx) {
    for (int c = threadIdx.x; c < HD; c += 256) out[c] = 0;
    return;
  }
  __shared__ float sred[4][HD];
  const int ns = (L + K + chunk - 1) / chunk;
  const float* src = part + (size_t)rid * nsplit * RS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  // (wave-uniform guards: a row with few splits issues only the loads it needs)
  float pm[PF], po[PF][CPT], mv[QB], lv[QB];
#pragma unroll
  for (int t = 0; t < PF; ++t) {
    pm[t] = 0.f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) po[t][e] = 0.f;
    if (wave + 4 * t < ns) {
      const int sp = wave + 4 * t;
      pm[t] = src[(size_t)sp * RS + HD];
#pragma unroll
      for (int e = 0; e < CPT; ++e) po[t][e] = src[(size_t)sp * RS + CPT * lane + e];
    }
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    mv[q] = 0.f;
    lv[q] = 0.f;
    if (64 * q < ns) {
      const int sp = min(64 * q + lane, ns - 1);  // clamped lanes are masked below
      mv[q] = src[(size_t)sp * RS + HD];
      lv[q] = src[(size_t)sp * RS + HD + 1];
    }
  }

  float M = -1e30f;
#pragma unroll
  for (int q = 0; q < QB; ++q)
    if (64 * q + lane < ns) M = fmaxf(M, mv[q]);
  for (int sp = 64 * QB + lane; sp < ns; sp += 64) M = fmaxf(M, src[(size_t)sp * RS + HD]);
  M = wave_max(M);

  float dq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < QB; ++q)
    if (64 * q + lane < ns) dq[q & 3] += __builtin_amdgcn_exp2f(mv[q] - M) * lv[q];
  for (int q = QB; 64 * q < ns; ++q) {
    const int sp = 64 * q + lane;
    if (sp < ns) dq[q & 3] += __builtin_amdgcn_exp2f(src[(size_t)sp * RS + HD] - M) * src[(size_t)sp * RS + HD + 1];
  }
  float den[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) den[c] = wave_sum(dq[c]);

  float num[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) num[e] = 0.f;
#pragma unroll
  for (int t = 0; t < PF; ++t) {
    if (wave + 4 * t < ns) {
      const float w = __builtin_amdgcn_exp2f(pm[t] - M);
#pragma unroll
      for (int e = 0; e < CPT; ++e) num[e] += w * po[t][e];
    }
  }
#pragma unroll 4
  for (int sp = wave + 4 * PF; sp < ns; sp += 4) {
    const float* ps = src + (size_t)sp * RS;
    const float w = __builtin_amdgcn_exp2f(ps[HD] - M);
#pragma unroll
    for (int e = 0; e < CPT; ++e) num[e] += w * ps[CPT * lane + e];
  }
#pragma unroll
  for (int e = 0; e < CPT; ++e) sred[wave][CPT * lane + e] = num[e];
  __syncthreads();
  const float inv = 1.f / ((den[0] + den[1]) + (den[2] + den[3]));
  for (int c = threadIdx.x; c < HD; c += 256)
    out[c] = f32_to_bf16(((sred[0][c] + sred[1][c]) + (sred[2][c] + sred[3][c])) * inv);
}

// Same merge for rows with at most 16 splits: a quarter wave (16 lanes) per (row, head) pair, four pairs per
// wave, sixteen per workgroup. Lane s of a quarter holds split s's (m, l); every lane loads HD / 16 columns
// (as 8-byte pieces: a partial row is HD + 2 floats) of every split up front; the maximum and the
// denominator are 16-lane shuffle reductions in a fixed pattern and the numerator adds the splits in order.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_quarter_kernel(const float* __restrict__ part,
                                                                   bf16_t* __restrict__ O,
                                                                   const int* __restrict__ seq_len,
                                                                   const int* __restrict__ req_slot, int K, int Hq,
                                                                   int max_ctx, int n_slots, int chunk, int nsplit,
                                                                   int npairs) {
  constexpr int CPT = HD / 16, RS = HD + 2, SMAX = 16;
  const int ql = threadIdx.x & 15;
  const int rid = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (rid >= npairs) return;  // whole quarters leave together (the shuffles stay inside a quarter)
  const int j = rid % K, h = (rid / K) % Hq, b = rid / (K * Hq);
  bf16_t* out = O + ((size_t)(b * K + j) * Hq + h) * HD + CPT * ql;
  const int L = seq_len[b], slot = req_slot[b];
  if (slot < 0 || slot >= n_slots || L < 0 || L + K > max_ctx) {
#pragma unroll
    for (int e = 0; e < CPT; ++e) out[e] = 0;
    return;
  }
  const int ns = (L + K + chunk - 1) / chunk;  // 1 .. nsplit <= SMAX
  const float* src = part + (size_t)rid * nsplit * RS;
  const int sl = min(ql, ns - 1);
  const float m_l = src[(size_t)sl * RS + HD], l_l = src[(size_t)sl * RS + HD + 1];
  float o[SMAX][CPT];
#pragma unroll
  for (int t = 0; t < SMAX; ++t) {
#pragma unroll
    for (int e = 0; e < CPT; ++e) o[t][e] = 0.f;
    if (t < ns) {
#pragma unroll
      for (int e = 0; e < CPT; e += 2) {
        const float2 v = *(const float2*)(src + (size_t)t * RS + CPT * ql + e);
        o[t][e] = v.x;
        o[t][e + 1] = v.y;
      }
    }
  }
  float M = ql < ns ? m_l : -1e30f;
  M = group_max<16>(M);
  const float w_l = ql < ns ? __builtin_amdgcn_exp2f(m_l - M) : 0.f;  // m in log2 units
  float den = w_l * l_l;
  den = group_sum<16>(den);
  float num[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) num[e] = 0.f;
  // split t's weight: lane t of the quarter (a 16-lane DPP row) broadcast to the row (row_newbcast)
  static_for<0, SMAX>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    if (t < ns) {
      const float wt = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(w_l), 0x150 + t, 0xF, 0xF, false));
#pragma unroll
      for (int e = 0; e < CPT; ++e) num[e] += wt * o[t][e];
    }
  });
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < CPT; ++e) out[e] = f32_to_bf16(num[e] * inv);
}

// Same merge for rows with at most 32 splits (larger batches: many (row, head) pairs, few splits each):
// one wave per pair, four pairs per workgroup. Lane s holds split s's (m, l); every lane loads its HD / 64
// columns of every split up front; the numerator adds the splits in order.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_wave_kernel(const float* __restrict__ part,
                                                                bf16_t* __restrict__ O,
                                                                const int* __restrict__ seq_len,
                                                                const int* __restrict__ req_slot, int K, int Hq,
                                                                int max_ctx, int n_slots, int chunk, int nsplit,
                                                                int npairs) {
  constexpr int CPT = HD / 64, RS = HD + 2, SMAX = 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rid = blockIdx.x * 4 + wave;
  if (rid >= npairs) return;
  const int j = rid % K, h = (rid / K) % Hq, b = rid / (K * Hq);
  bf16_t* out = O + ((size_t)(b * K + j) * Hq + h) * HD;
  const int L = seq_len[b], slot = req_slot[b];
  if (slot < 0 || slot >= n_slots || L < 0 || L + K > max_ctx) {
#pragma unroll
    for (int e = 0; e < CPT; ++e) out[CPT * lane + e] = 0;
    return;
  }
  const int ns = (L + K + chunk - 1) / chunk;  // 1 .. nsplit <= SMAX
  const float* src = part + (size_t)rid * nsplit * RS;
  const int sl = min(lane, ns - 1);
  const float m_l = src[(size_t)sl * RS + HD], l_l = src[(size_t)sl * RS + HD + 1];
  float o[SMAX][CPT];
#pragma unroll
  for (int t = 0; t < SMAX; ++t) {
#pragma unroll
    for (int e = 0; e < CPT; ++e) o[t][e] = 0.f;
    if (t < ns) {
#pragma unroll
      for (int e = 0; e < CPT; ++e) o[t][e] = src[(size_t)t * RS + CPT * lane + e];
    }
  }
  const float M = wave_max(lane < ns ? m_l : -1e30f);
  const float w_l = lane < ns ? __builtin_amdgcn_exp2f(m_l - M) : 0.f;  // m in log2 units
  const float den = wave_sum(w_l * l_l);
  float num[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) num[e] = 0.f;
#pragma unroll
  for (int t = 0; t < SMAX; ++t) {
    if (t < ns) {
      const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), t));  // lane t's weight
#pragma unroll
      for (int e = 0; e < CPT; ++e) num[e] += wt * o[t][e];
    }
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < CPT; ++e) out[CPT * lane + e] = f32_to_bf16(num[e] * inv);
}

hipError_t launch_attention_bf16(const AttnPlan& p, const void* Q, const void* Kc, const void* Vc,
                                 const int* seq_len, const int* req_slot, int B, int K, int Hq, int Hkv, int hd,
                                 int max_ctx, int n_slots, float* part, hipStream_t st) {
  const dim3 grid = p.split_major ? dim3(p.nsplit, B * Hkv) : dim3(B * Hkv, p.nsplit);
  // 1/sqrt(hd) and log2(e): scores, maxima and partial m are kept in log2 units (exp2 on the hardware)
  const float scale = 1.0f / sqrtf((float)hd) * 1.4426950408889634f;
  const bool eight = (Hq / Hkv) * K > 64;
#define PE_ATTN_LAUNCH(HDV, NWV)                                                                                   \
  hipLaunchKernelGGL((attn_bf16_kernel<HDV, NWV>), grid, dim3(NWV * 64), 0, st, (const bf16_t*)Q, (const bf16_t*)Kc, \
                     (const bf16_t*)Vc, seq_len, req_slot, K, Hq, Hkv, max_ctx, n_slots, p.chunk, p.nsplit, p.sub,  \
                     p.split_major, part, scale)
  if (hd == 128) {
    if (eight) PE_ATTN_LAUNCH(128, 8);
    else PE_ATTN_LAUNCH(128, 4);
  } else {
    if (eight) PE_ATTN_LAUNCH(64, 8);
    else PE_ATTN_LAUNCH(64, 4);
  }
#undef PE_ATTN_LAUNCH
  return hipGetLastError();
}

hipError_t launch_attention_combine_bf16(const AttnPlan& p, const float* part, void* O, const int* seq_len,
                                         const int* req_slot, int B, int K, int Hq, int Hkv, int hd, int max_ctx,
                                         int n_slots, hipStream_t st) {
  (void)Hkv;
  if (p.nsplit <= 16) {
    const int npairs = B * Hq * K;
    dim3 grid((npairs + 15) / 16), block(256);
    if (hd == 128)
      hipLaunchKernelGGL(attn_combine_quarter_kernel<128>, grid, block, 0, st, part, (bf16_t*)O, seq_len, req_slot, K,
                         Hq, max_ctx, n_slots, p.chunk, p.nsplit, npairs);
    else
      hipLaunchKernelGGL(attn_combine_quarter_kernel<64>, grid, block, 0, st, part, (bf16_t*)O, seq_len, req_slot, K,
                         Hq, max_ctx, n_slots, p.chunk, p.nsplit, npairs);
    return hipGetLastError();
  }
  if (p.nsplit <= 32) {
    const int npairs = B * Hq * K;
    dim3 grid((npairs + 3) / 4), block(256);
    if (hd == 128)
      hipLaunchKernelGGL(attn_combine_wave_kernel<128>, grid, block, 0, st, part, (bf16_t*)O, seq_len, req_slot, K,
                         Hq, max_ctx, n_slots, p.chunk, p.nsplit, npairs);
    else
      hipLaunchKernelGGL(attn_combine_wave_kernel<64>, grid, block, 0, st, part, (bf16_t*)O, seq_len, req_slot, K,
                         Hq, max_ctx, n_slots, p.chunk, p.nsplit, npairs);
    return hipGetLastError();
  }
  dim3 grid(B * Hq * K), block(256);
  if (hd == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, grid, block, 0, st, part, (bf16_t*)O, seq_len, req_slot, K, Hq,
                       max_ctx, n_slots, p.chunk, p.nsplit);
  else
    hipLaunchKernelGGL(attn_combine_kernel<64>, grid, block, 0, st, part, (bf16_t*)O, seq_len, req_slot, K, Hq,
                       max_ctx, n_slots, p.chunk, p.nsplit);
  return hipGetLastError();
}

// fp32 path (small fp32 drafter): one workgroup per (request, q head, row); scores of all visible keys in
// LDS, exact two-pass softmax, then the value sum.
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ Q, const float* __restrict__ Kc,
                                                       const float* __restrict__ Vc, const int* __restrict__ seq_len,
                                                       const int* __restrict__ req_slot, int K, int Hq, int Hkv,
                                                       int hd, int max_ctx, int n_slots, float* __restrict__ O,
                                                       float scale) {
  extern __shared__ float smem[];
  float* sc = smem;              // [max_ctx]
  float* sq = smem + max_ctx;    // [hd]
  float* red = sq + hd;          // [256]
  const int rid = blockIdx.x;
  const int j = rid % K, h = (rid / K) % Hq, b = rid / (K * Hq);
  const int g = h / (Hq / Hkv);
  const int m = b * K + j;
  float* out = O + ((size_t)m * Hq + h) * hd;
  const int L = seq_len[b], slot = req_slot[b];
  if (slot < 0 || slot >= n_slots || L < 0 || L + K > max_ctx) {
    for (int c = threadIdx.x; c < hd; c += 256) out[c] = 0.f;
    return;
  }
  const int n = L + j + 1;
  for (int c = threadIdx.x; c < hd; c += 256) sq[c] = Q[((size_t)m * Hq + h) * hd + c];
  __syncthreads();
  const float* kb = Kc + ((size_t)slot * Hkv + g) * max_ctx * hd;
  const float* vb = Vc + ((size_t)slot * Hkv + g) * max_ctx * hd;
  float lmax = -INFINITY;
  for (int t = threadIdx.x; t < n; t += 256) {
    float s = 0.f;
    for (int c = 0; c < hd; ++c) s = fmaf(sq[c], kb[(size_t)t * hd + c], s);
    s *= scale;
    sc[t] = s;
    lmax = fmaxf(lmax, s);
  }
  lmax = wave_max(lmax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = lmax;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float lsum = 0.f;
  for (int t = threadIdx.x; t < n; t += 256) {
    const float p = __expf(sc[t] - M);
    sc[t] = p;
    lsum += p;
  }
  const float den = block_sum<256>(lsum, red);  // also orders the score writes before the value pass
  const int groups = 256 / hd;
  const int c = threadIdx.x % hd, grp = threadIdx.x / hd;
  float acc = 0.f;
  if (grp < groups)
    for (int t = grp; t < n; t += groups) acc = fmaf(sc[t], vb[(size_t)t * hd + c], acc);
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < hd) {
    float tot = 0.f;
    for (int q = 0; q < groups; ++q) tot += red[q * hd + threadIdx.x];
    out[threadIdx.x] = tot / den;
  }
}

hipError_t launch_attention_f32(const float* Q, const float* Kc, const float* Vc, const int* seq_len,
                                const int* req_slot, int B, int K, int Hq, int Hkv, int hd, int max_ctx, int n_slots,
                                float* O, hipStream_t st) {
  const size_t shmem = (size_t)(max_ctx + hd + 256) * sizeof(float);
  hipLaunchKernelGGL(attn_f32_kernel, dim3(B * Hq * K), dim3(256), shmem, st, Q, Kc, Vc, seq_len, req_slot, K, Hq,
                     Hkv, hd, max_ctx, n_slots, O, 1.0f / sqrtf((float)hd));
  return hipGetLastError();
}

}  // namespace pe
