// Internal launch interface of the gfx950 kernels (host side). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pe {

// ---- weight packing: W [N, Kd] bf16 -> 1 KiB MFMA fragments ----------------------------------
// Fragment (t, s) holds rows 16t..16t+15, columns 32s..32s+31; lane l's 16 bytes are
// W[16t + (l & 15)][32s + 8(l >> 4) .. +7]. Fragments are stored tile-major: ((t*mul+add) * Ks + s).
hipError_t launch_pack_bf16(const void* W, int N, int Kd, void* dst, int tile_mul, int tile_add, hipStream_t st);
inline int n_tiles(int N) { return (N + 15) / 16; }
inline int k_steps(int Kd) { return (Kd + 31) / 32; }

// ---- GEMM y = A . W^T -------------------------------------------------------------------------
struct GemmPlan {
  int MT;       // 16-row MFMA tiles per workgroup (1, 2, 4 or 8)
  int mblocks;  // workgroups along M
  int ngroups;  // workgroups along N (64 columns each)
  int S;        // K splits (fp32 partials [S][M][N])
  int kps;      // k-steps (of 32) per split
};
GemmPlan plan_gemm(int M, int N, int Kd, bool argmax_epilogue);

// partial mode: P[s][m][n] = sum over split s's k range
hipError_t launch_gemm_bf16_partial(const GemmPlan& p, const void* A, int lda, int M, int Kd, const void* Wp,
                                    int N, float* P, hipStream_t st);
// argmax mode (S == 1): per (row, 64-column group) best (value, index); optional fp32 logits [M][N]
hipError_t launch_gemm_bf16_argmax(const GemmPlan& p, const void* A, int lda, int M, int Kd, const void* Wp,
                                   int N, float* am_val, int* am_idx, float* logits, hipStream_t st);
// fp32 weights, unpacked [N, Kd]: out[m * ldo + n] (one split)
hipError_t launch_gemm_f32(const float* A, int lda, int M, int Kd, const float* W, int N, float* out, int ldo,
                           hipStream_t st);

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
};
AttnPlan plan_attention(int B, int K, int Hq, int Hkv, int max_ctx);
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
hipError_t launch_accept_compact(const float* pv, const int* pi, int nchunks, int B, int K, const int* draft,
                                 const uint8_t* finished, const int* req_slot, const int* seq_len, int* t_ws,
                                 int* accept_len, int* cu_accept, int* out_tokens, int* keep_index, int* n_keep,
                                 int* slot_next, int* seq_next, int* last_next, hipStream_t st);

}  // namespace pe
