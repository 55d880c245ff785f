// Internal launch interface of the gfx950 kernels (host side). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pe {

// ---- weight packing: W [N, Kd] bf16 -> 1 KiB MFMA fragments ----------------------------------
// Fragment (t, s) holds 16 output rows and columns 32s..32s+31 of the reduction dimension; lane l's 16
// bytes are W[src(t, l & 15)][32s + 8(l >> 4) .. +7]. Fragments are stored tile-major: (t * Ks + s).
// PACK_PLAIN: src(t, r) = 16t + r.
// PACK_PAIRS: the 16 rows of a tile are 8 RoPE pairs of one head of width hd: rows 8tt+e and
//             hd/2 + 8tt + e of head t / (hd/16), tt = t % (hd/16) (q, k and v heads alike).
// PACK_GATEUP: rows 8t..8t+7 of W0 (gate) then rows 8t..8t+7 of W1 (up); 2N/16 tiles.
// PACK_KI4 (products of at most 4 rows): fragment (t, s) holds 4 output rows and reduction columns
// 128s..128s+127; lane l's 16 bytes are W[4t + (l & 3)][128s + 8(4(l >> 4) + ((l >> 2) & 3)) .. +7]: the
// MFMA's 16 columns are 4 output columns x 4 interleaved 8-wide k chunks. With the activation row m at
// MFMA row m + 4h reading chunk h the same way, the product of output column c is the sum over h of
// D[m + 4h][c + 4h]. ceil(N/4) tiles of ceil(Kd/128) fragments: 4x the workgroups of the plain layout.
enum { PACK_PLAIN = 0, PACK_PAIRS = 1, PACK_GATEUP = 2, PACK_KI4 = 3 };
hipError_t launch_pack_bf16(const void* W0, const void* W1, int N, int Kd, int mode, int hd, void* dst,
                            hipStream_t st);
inline int n_tiles(int N) { return (N + 15) / 16; }
inline int k_steps(int Kd) { return (Kd + 31) / 32; }
inline int n_tiles_ki4(int N) { return (N + 3) / 4; }
inline int k_steps_ki4(int Kd) { return (Kd + 127) / 128; }

// ---- GEMM y = A . W^T with fused prologue / epilogue ---------------------------------------------
// k-steps (of 32) per activation chunk of the 9..128-row weight-stream kernel; its K-split plans use
// multiples of four chunks per split
constexpr int GEMM_STREAM_CH = 4;
// k-steps per workgroup of the burst kernel (K-split weight-stream products with every load issued at once)
constexpr int GEMM_BURST_KS = 16;
struct GemmPlan {
  int Nt;       // 16-column tiles
  int MT;       // 16-row MFMA tiles per workgroup (1, 2, 4 or 8)
  int mblocks;  // workgroups along M
  int NT;       // 16-column tiles per workgroup
  int NW;       // waves per workgroup (they split the reduction dimension NW/NT ways)
  int ngroups;  // workgroups along N
  int tiled;    // 2: weight-stream kernel (9..128 rows); 1: LDS-tiled 128 x 128 kernel (larger M); 3: the vocabulary
                // projection's 128 x 512 kernel (128 x 128 with FP8 weights); 0: skinny split-K kernel
  int ksplit;   // tiled: workgroups along the reduction dimension (1 = none); > 1 adds a reduce kernel
  int kper;     // tiled: k-steps (32 columns each) per split, a multiple of 4
  int ki4;      // skinny on PACK_KI4 weights: 4-column tiles (Nt counts them), 128-wide k-steps
  int burst;    // weight-stream K-split on the burst kernel: its waves per workgroup (4 or 8), else 0
};
// ki4_ok: the weights are also packed as PACK_KI4 (the residual-stream producers: fc, O, down), which the
// plan uses for up to 4 rows when the plain layout would leave most compute units idle
// skinny_only: the small-batch kernel whatever M (FP8 weights; M <= 16)
// fp8: FP8 weights (the burst kernel has no FP8 path)
GemmPlan plan_gemm(int M, int N, int Kd, bool argmax, bool ki4_ok = false, bool skinny_only = false,
                   bool fp8 = false);
// Partial sums of squares per row that a residual-stream producer with plan p writes (one per 16 columns
// for the skinny kernel, one per 4 columns on PACK_KI4 weights, one per 128-column workgroup tile for the
// tiled one); the consumer sums exactly that many.
inline int gemm_ssq_parts(const GemmPlan& p) { return p.tiled ? p.ngroups : p.Nt; }

// A operand: always a bf16 matrix. A_NORM marks a normalised operand: A = bf16(x * g) of the residual stream
// (written by the producer of x), and the epilogue scales each product row by 1/RMS(x) from the
// producer's per-16-column sums of squares (RMSNorm is a per-row scale).
enum { A_BF16 = 0, A_NORM = 1 };
enum { EPI_RESID = 0, EPI_ROWS = 1, EPI_SWIGLU = 2, EPI_QKV = 3, EPI_ARGMAX = 4,
       EPI_PARTIAL = 5 /* tiled K-split: raw partial tile, internal */ };

struct GemmArgs {
  int M, Kd, N;
  int Nt, Ks, ngroups, mblocks;  // filled by launch_gemm from the plan (with ksplit, kper)
  // A operand
  const uint16_t* A; int lda;
  const float* ssq_in; int nssq; float eps;  // A_NORM
  const void* Wp_raw;  // packed weights
  // EPI_RESID / EPI_ROWS: residual stream (+=, or rows written), per-16-column sums of squares, and the
  // next normalised operand XG = bf16(x * gain_next)
  float* Xout; float* ssq_out; int nssq_out; uint16_t* XGout; const uint16_t* gain_next;
  // EPI_SWIGLU: A [M][F]
  uint16_t* Aout; int F;
  // EPI_QKV
  uint16_t* Q; uint16_t* Kc; uint16_t* Vc;
  const int* seq_len; const int* req_slot; const float2* rope;
  int Kdraft, Hq, Hkv, hd, max_ctx, n_slots; int* flags;
  // EPI_ROWS; with Xe (concatenated rows) the embedding half is written to Xe [rows, d] instead of being
  // added to the hidden half in Xout
  const int* last_token; const uint16_t* embed; const uint16_t* emb_mask; const uint16_t* h_shared; int V;
  float* Xe;
  // EPI_ARGMAX: per (row, workgroup) best (value, index); optional fp32 logits, row m at logits + m * ldz
  // (ldz = 0 means N)
  float* am_val; int* am_idx; float* logits; int ldz;
  // row m of the product reads operand row (m / rows_out) * rows_in + m % rows_out (and that row's sums
  // of squares): the LM head runs on rows_out of every rows_in rows per request. 0 = identity.
  int rows_in, rows_out;
  // catch-up steps: request b has n_real[b] (1 .. rows_real) real input rows; the row build reads rows_real
  // tokens / hidden triples per request, and the LM head's rows of request b start at operand row
  // n_real[b] - 1 of its block. NULL = one real row per request.
  const int* n_real; int rows_real;
  // tiled K-split: fp32 partial tiles [ksplit][M][N] (workspace) and the plan's split shape
  float* part; int ksplit, kper;
  // FP8 weights (small-batch kernel only): Wp_raw holds E4M3 fragment pairs (16 bytes per lane: two k-steps) and
  // wscale one float per packed output column (tile t, column c at 16 t + c); y = wscale * (q . x)
  const float* wscale;
};
// real input rows of request b (clamped into 1 .. rows_real, so that a bad value stays in bounds)
__device__ inline int gemm_n_real(const GemmArgs& g, int b) {
  return g.n_real ? min(max(g.n_real[b], 1), max(g.rows_real, 1)) : 1;
}
// operand row of product row m
__device__ inline int gemm_a_row(const GemmArgs& g, int m) {
  if (g.rows_out <= 0) return m;
  const int b = m / g.rows_out;
  return b * g.rows_in + m % g.rows_out + (g.n_real ? gemm_n_real(g, b) - 1 : 0);
}
// operand rows the product may read (the size of its buffer range)
__device__ inline int gemm_a_rows(const GemmArgs& g) {
  return g.rows_out > 0 ? (g.M + g.rows_out - 1) / g.rows_out * g.rows_in : g.M;
}
hipError_t launch_gemm(const GemmPlan& p, GemmArgs a, int a_mode, int epi, hipStream_t st);
// FP8 repack of one projection (PACK_PLAIN / PACK_PAIRS / PACK_GATEUP layouts): per packed output column the
// scale s = max |w| / 448 of its source row (1 for a zero row), then E4M3 codes of w / s (round to nearest
// even), two k-steps per 16-byte lane chunk; dst needs Nt ceil(Ks / 2) 1024 bytes, scales Nt 16 floats
hipError_t launch_pack_fp8(const void* W0, const void* W1, int N, int Kd, int mode, int hd, void* dst, float* scales,
                           hipStream_t st);
hipError_t launch_gemm_tiled(const GemmPlan& p, const GemmArgs& a, int a_mode, int epi, hipStream_t st);
// Autoregressive pass `pass` >= 1: row b = X[b] (the previous pass's residual stream after the last layer)
// + embed[prev_tok[b]]; records prev_tok[b] as draft pass - 1 of request b (draft_tokens [B, K]), writes the
// pass's positions seq_cur[b] = seq_len[b] + pass, XG = bf16(x * gain) and per-16-column sums of squares.
hipError_t launch_ar_rows(float* X, uint16_t* XG, float* ssq, const uint16_t* embed, const uint16_t* gain,
                          const int* prev_tok, int* draft_tokens, int K, int pass, const int* seq_len, int* seq_cur,
                          int B, int d, int V, int* flags, hipStream_t st);
// Concatenated rows: U [M, 2d] = [bf16(RMSNorm(Xe) * g_e) || bf16(RMSNorm(X) * g_h)], one row per workgroup.
hipError_t launch_concat_norm(const float* X, const float* Xe, const uint16_t* g_h, const uint16_t* g_e, uint16_t* U,
                              int M, int d, float eps, hipStream_t st);
hipError_t launch_rows_ssq(const float* rows, float* X, float* ssq, uint16_t* XG, const uint16_t* gain, int M, int d,
                           hipStream_t st);
// fp32 weights, unpacked [N, Kd]: out[m * ldo + n]
hipError_t launch_gemm_f32(const float* A, int lda, int M, int Kd, const float* W, int N, float* out, int ldo,
                           hipStream_t st, int rows_in = 0, int rows_out = 0);

// ---- row-wise kernels (dtype: 0 = f32, 1 = bf16 for activations / weights) -------------------
hipError_t launch_rowbuild_norm(int dtype, float* X, void* U, const float* P, int S, const float* rows_in, int B,
                                int K, int d, const int* last_token, const void* embed, const void* emb_mask,
                                const void* h_shared, const void* gain, float eps, int V, int* flags,
                                hipStream_t st);
hipError_t launch_residual_norm(int dtype, float* X, void* U, const float* P, int S, int M, int d,
                                const void* gain, float eps, hipStream_t st);
hipError_t launch_swiglu(int dtype, void* Aout, const float* P, int S, int M, int F, bool interleaved,
                         hipStream_t st);
hipError_t launch_rope_kv(int dtype, void* Q, void* Kc, void* Vc, const float* P, int S, int B, int K, int Hq,
                          int Hkv, int hd, const int* seq_len, const int* req_slot, int max_ctx, int n_slots,
                          const float2* cs, int* flags, hipStream_t st);
hipError_t launch_rope_table(float2* cs, int max_ctx, int hd, double base, hipStream_t st);

// ---- attention --------------------------------------------------------------------------------
struct AttnPlan {
  int chunk;   // keys per split
  int nsplit;  // splits (grid y)
  int sub;     // key sub-streams per split inside a workgroup
  int split_major;  // 1: consecutive workgroups take consecutive splits of one (request, kv head)
};
AttnPlan plan_attention(int B, int K, int Hq, int Hkv, int hd, int max_ctx);
size_t attn_partial_floats(int M, int Hq, int hd, const AttnPlan& p);
hipError_t launch_attention_bf16(const AttnPlan& p, const void* Q, const void* Kc, const void* Vc,
                                 const int* seq_len, const int* req_slot, int B, int K, int Hq, int Hkv, int hd,
                                 int max_ctx, int n_slots, float* part, hipStream_t st);
hipError_t launch_attention_combine_bf16(const AttnPlan& p, const float* part, void* O, const int* seq_len,
                                         const int* req_slot, int B, int K, int Hq, int Hkv, int hd,
                                         int max_ctx, int n_slots, hipStream_t st);
hipError_t launch_attention_f32(const float* Q, const float* Kc, const float* Vc, const int* seq_len,
                                const int* req_slot, int B, int K, int Hq, int Hkv, int hd, int max_ctx,
                                int n_slots, float* O, hipStream_t st);

// ---- argmax and verify ------------------------------------------------------------------------
int plan_argmax_chunks(int rows, int V);
hipError_t launch_argmax_rows(int dtype, const void* X, int rows, int V, int nchunks, float* pv, int* pi,
                              hipStream_t st);
hipError_t launch_argmax_final(const float* pv, const int* pi, int rows, int nchunks, int* out, hipStream_t st);
// sampled verification (temperature > 0): chunk softmax statistics, per-request decisions and draws, then the
// metadata rebuild; pm / ps hold rows x nchunks floats each (nchunks = plan_sample_chunks(V))
constexpr int PE_SAMPLE_MAX_CHUNKS = 1024;
// chunks per row of the sampled verify: about 2048 tokens each, so that a draw scans one short chunk
// (measured: 2-chunk rows at B 128 K 7 made the draws scan 76 k tokens each, 119 -> 198 us)
inline int plan_sample_chunks(int V) {
  const int c = (V + 2047) / 2048;
  return c < 1 ? 1 : (c > PE_SAMPLE_MAX_CHUNKS ? PE_SAMPLE_MAX_CHUNKS : c);
}
hipError_t launch_sampled_verify(int dtype, const void* X, int B, int K, int V, int nchunks, float temperature,
                                 const int* draft, const float* u, const float* v, const uint8_t* finished,
                                 const int* req_slot, const int* seq_len, float* pm, float* ps, int* t_ws,
                                 int* accept_len, int* cu_accept, int* out_tokens, int* keep_index, int* n_keep,
                                 int* slot_next, int* seq_next, int* last_next, hipStream_t st);
hipError_t launch_accept_compact(const float* pv, const int* pi, int nchunks, int B, int K, const int* draft,
                                 const uint8_t* finished, const int* req_slot, const int* seq_len, int* t_ws,
                                 int* accept_len, int* cu_accept, int* out_tokens, int* keep_index, int* n_keep,
                                 int* slot_next, int* seq_next, int* last_next, hipStream_t st);

}  // namespace pe
