// C ABI of the P-EAGLE draft / verify path (declared in include/pe.h): argument checks, workspace,
// weight repacking, and the launch sequence of one parallel draft step and one greedy verify.
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pe.h"
#include "common.h"
#include "kernels.h"

using namespace pe;

struct pe_ctx {
  pe_config cfg{};
  pe_weights w{};
  pe_kv kv{};
  hipStream_t stream = nullptr;
  int device = 0;
  bool bf16 = true;

  // bf16 path: projections repacked into MFMA fragments (library-owned)
  char* packed = nullptr;
  const void* p_fc = nullptr;
  const void* p_qkv[PE_MAX_LAYERS] = {};
  const void* p_o[PE_MAX_LAYERS] = {};
  const void* p_gu[PE_MAX_LAYERS] = {};  // gate and up, 16-column tiles interleaved
  const void* p_down[PE_MAX_LAYERS] = {};
  const void* p_lm = nullptr;
  // the residual-stream producers again in the 4-column layout (PACK_KI4) for draft steps of up to 4 rows
  const void* p_fc4 = nullptr;
  const void* p_o4[PE_MAX_LAYERS] = {};
  const void* p_down4[PE_MAX_LAYERS] = {};
  // FP8 weights (weight_fp8): E4M3 fragments and per-column scales of every projection
  bool fp8 = false;
  char* packed8 = nullptr;
  const void* q_fc = nullptr; const void* q_qkv[PE_MAX_LAYERS] = {}; const void* q_o[PE_MAX_LAYERS] = {};
  const void* q_gu[PE_MAX_LAYERS] = {}; const void* q_down[PE_MAX_LAYERS] = {}; const void* q_lm = nullptr;
  const float* s_fc = nullptr; const float* s_qkv[PE_MAX_LAYERS] = {}; const float* s_o[PE_MAX_LAYERS] = {};
  const float* s_gu[PE_MAX_LAYERS] = {}; const float* s_down[PE_MAX_LAYERS] = {}; const float* s_lm = nullptr;

  // workspace
  char* ws = nullptr;
  float* X = nullptr;      // residual stream [Mmax, d] fp32
  void* U = nullptr;       // normalised activations [Mmax, d]
  void* Qb = nullptr;      // rotated queries [Mmax, Hq hd]
  void* Ob = nullptr;      // attention output [Mmax, Hq hd]
  void* Ab = nullptr;      // SwiGLU output [Mmax, F]
  float* P = nullptr;      // fp32 path: projection outputs
  float* part = nullptr;   // tiled projections: K-split partial tiles
  float* attn = nullptr;   // attention split partials
  float* am_val = nullptr; // argmax partials
  int* am_idx = nullptr;
  int* t_ws = nullptr;     // target argmax [max_batch, max_k + 1]
  float* samp = nullptr;   // sampled verify: per-chunk softmax statistics, 2 x [max_batch (max_k + 1), chunks]
  float* logits_ws = nullptr;  // fp32 path: logits when the caller passes none
  float2* rope = nullptr;  // [max_ctx, hd/2] (cos, sin)
  float* ssq = nullptr;    // partial sums of squares of X rows [Mmax, d/4] (per 16 or per 4 columns)
  int* flags = nullptr;
  int* ar_tok = nullptr;   // autoregressive drafting: the token each request drafted in the latest pass [max_batch]
  int* ar_seq = nullptr;   // ... and the positions of the current pass [max_batch]
  float* Xe = nullptr;     // concatenated rows: embedding halves [Mmax, d] fp32
  void* Ucat = nullptr;    // concatenated rows: layer 0's normalised operand [Mmax, 2d] bf16

  std::string err;

  int prof = 0;  // bitmask of recorded kernels
  std::vector<hipEvent_t> ev_a[PE_PROF_COUNT], ev_b[PE_PROF_COUNT];
  size_t ev_used[PE_PROF_COUNT] = {};
};

static std::string g_init_err;

static pe_status fail(pe_ctx* c, pe_status s, const std::string& msg) {
  if (c) c->err = msg; else g_init_err = msg;
  return s;
}

#define HIP_TRY(ctx, call)                                                                   \
  do {                                                                                       \
    hipError_t e_ = (call);                                                                  \
    if (e_ != hipSuccess)                                                                    \
      return fail(ctx, PE_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_));       \
  } while (0)

static pe_status check_cfg(const pe_config* c, std::string& why) {
  if (!c) { why = "cfg is NULL"; return PE_ERR_INVALID; }
  if (c->n_layers < 1 || c->n_layers > PE_MAX_LAYERS) { why = "n_layers out of [1, 8]"; return PE_ERR_INVALID; }
  if (c->d_model <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->ffn_dim <= 0 ||
      c->vocab <= 0) { why = "non-positive dimension"; return PE_ERR_INVALID; }
  if (c->n_q_heads % c->n_kv_heads) { why = "n_q_heads must be a multiple of n_kv_heads"; return PE_ERR_INVALID; }
  if (c->head_dim % 2) { why = "head_dim must be even"; return PE_ERR_INVALID; }
  if (c->dtype != PE_F32 && c->dtype != PE_BF16) { why = "dtype must be PE_F32 or PE_BF16"; return PE_ERR_INVALID; }
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 1.f)) { why = "rms_eps < 0 or rope_base <= 1"; return PE_ERR_INVALID; }
  if (c->max_batch < 1 || c->max_batch > PE_MAX_BATCH) { why = "max_batch out of [1, 1024]"; return PE_ERR_INVALID; }
  if (c->max_k < 1 || c->max_k > PE_MAX_K) { why = "max_k out of [1, 16]"; return PE_ERR_INVALID; }
  if (c->max_ctx < c->max_k + 1 || c->n_slots < 1) { why = "max_ctx < max_k + 1 or n_slots < 1"; return PE_ERR_INVALID; }
  if (c->head_dim != 64 && c->head_dim != 128) { why = "head_dim must be 64 or 128"; return PE_ERR_UNSUPPORTED; }
  if (c->d_model % 32 || c->ffn_dim % 32) { why = "d_model and ffn_dim must be multiples of 32"; return PE_ERR_UNSUPPORTED; }
  if (c->vocab % 8) { why = "vocab must be a multiple of 8"; return PE_ERR_UNSUPPORTED; }
  if (c->dtype == PE_BF16 && (c->n_q_heads / c->n_kv_heads) * (c->max_k + 1) > 128) {
    why = "(n_q_heads / n_kv_heads) * (max_k + 1) must be <= 128"; return PE_ERR_UNSUPPORTED;
  }
  if (c->row_concat != 0 && c->row_concat != 1) { why = "row_concat must be 0 or 1"; return PE_ERR_INVALID; }
  if (c->row_concat && c->dtype != PE_BF16) { why = "concatenated rows need a bf16 drafter"; return PE_ERR_UNSUPPORTED; }
  if (c->weight_fp8 != 0 && c->weight_fp8 != 1) { why = "weight_fp8 must be 0 or 1"; return PE_ERR_INVALID; }
  if (c->weight_fp8 && (c->dtype != PE_BF16 || c->row_concat)) {
    why = "FP8 weights need a bf16 drafter with summed rows"; return PE_ERR_UNSUPPORTED;
  }
  if (c->dtype == PE_F32 && c->max_ctx > 12288) { why = "fp32 drafter supports max_ctx <= 12288"; return PE_ERR_UNSUPPORTED; }
  if ((long long)c->n_slots * c->n_kv_heads * c->max_ctx * c->head_dim > (1LL << 40)) {
    why = "KV cache too large"; return PE_ERR_UNSUPPORTED;
  }
  return PE_OK;
}

extern "C" pe_status pe_config_validate(const pe_config* cfg) {
  std::string why;
  pe_status s = check_cfg(cfg, why);
  if (s != PE_OK) g_init_err = why;
  return s;
}

extern "C" const char* pe_status_string(pe_status s) {
  switch (s) {
    case PE_OK: return "ok";
    case PE_ERR_INVALID: return "invalid argument";
    case PE_ERR_UNSUPPORTED: return "unsupported";
    case PE_ERR_OOM: return "out of device memory";
    case PE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" const char* pe_last_error(const pe_ctx* ctx) { return ctx ? ctx->err.c_str() : g_init_err.c_str(); }

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// projection plan; FP8 weights always run on the small-batch kernel (16-column tiles). The FP8 vocabulary
// projection takes four tiles per workgroup (8 waves: 4 tiles x 2 k parts; one tile's codes are half its
// bf16 bytes, so a workgroup of one tile was too short: measured at B 1 K 3, 84 us with one tile, 72 with
// two, 69 with four)
static GemmPlan plan_for(const pe_ctx* ctx, int M, int N, int Kd, bool argmax, bool ki4_ok = false) {
  if (!ctx->fp8) return plan_gemm(M, N, Kd, argmax, ki4_ok);
  if (M > 16) return plan_gemm(M, N, Kd, argmax, false, false, true);  // weight-stream or tiled kernel
  GemmPlan p = plan_gemm(M, N, Kd, argmax, false, true);
  if (argmax && p.MT == 1) {
    p.NT = 4;
    p.NW = 8;
    p.ngroups = (p.Nt + 3) / 4;
  }
  return p;
}


static size_t packed_bytes(int N, int Kd) { return (size_t)n_tiles(N) * k_steps(Kd) * 1024; }
static size_t packed_ki4_bytes(int N, int Kd) { return (size_t)n_tiles_ki4(N) * k_steps_ki4(Kd) * 1024; }

static void free_ctx(pe_ctx* c) {
  if (!c) return;
  for (int k = 0; k < PE_PROF_COUNT; ++k) {
    for (auto e : c->ev_a[k]) (void)hipEventDestroy(e);
    for (auto e : c->ev_b[k]) (void)hipEventDestroy(e);
  }
  if (c->packed) (void)hipFree(c->packed);
  if (c->packed8) (void)hipFree(c->packed8);
  if (c->ws) (void)hipFree(c->ws);
  delete c;
}

extern "C" pe_status pe_init(const pe_config* cfg, const pe_weights* w, const pe_kv* kv, void* stream,
                             pe_ctx** out) {
  std::string why;
  if (!out) return fail(nullptr, PE_ERR_INVALID, "out is NULL");
  *out = nullptr;
  pe_status s = check_cfg(cfg, why);
  if (s != PE_OK) return fail(nullptr, s, why);
  if (!w || !kv) return fail(nullptr, PE_ERR_INVALID, "weights or kv is NULL");
  const pe_config& c = *cfg;
  if (!w->fc || !w->embed || !w->emb_mask || !w->h_shared || !w->final_norm || !w->lm_head)
    return fail(nullptr, PE_ERR_INVALID, "a global weight pointer is NULL");
  if (c.row_concat && !w->embed_norm) return fail(nullptr, PE_ERR_INVALID, "row_concat needs embed_norm");
  for (int l = 0; l < c.n_layers; ++l)
    if (!w->attn_norm[l] || !w->wqkv[l] || !w->wo[l] || !w->mlp_norm[l] || !w->wgate[l] || !w->wup[l] ||
        !w->wdown[l] || !kv->k[l] || !kv->v[l])
      return fail(nullptr, PE_ERR_INVALID, "a per-layer weight or cache pointer is NULL");
  for (int l = 0; l < c.n_layers; ++l)
    if (((uintptr_t)kv->k[l] | (uintptr_t)kv->v[l]) & 15)
      return fail(nullptr, PE_ERR_INVALID, "KV cache pointers must be 16-byte aligned");

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(nullptr, PE_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess)
    return fail(nullptr, PE_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, PE_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", not gfx950");

  pe_ctx* ctx = new pe_ctx();
  ctx->cfg = c;
  ctx->w = *w;
  ctx->kv = *kv;
  ctx->stream = (hipStream_t)stream;
  ctx->device = dev;
  ctx->bf16 = c.dtype == PE_BF16;
  const int d = c.d_model, F = c.ffn_dim, V = c.vocab, hd = c.head_dim;
  const int qd = c.n_q_heads * hd, qkvd = (c.n_q_heads + 2 * c.n_kv_heads) * hd;
  // a draft step runs K + 1 rows per request (the K draft rows and one trailing placeholder row)
  const int Mmax = c.max_batch * (c.max_k + 1);
  const size_t es = ctx->bf16 ? 2 : 4;

  // ---- packed weights (bf16 path)
  if (ctx->bf16) {
    size_t off = 0;
    std::vector<size_t> offs;
    auto take = [&](size_t b) { size_t o = off; off = align256(off + b); return o; };
    const size_t o_fc = take(packed_bytes(d, 3 * d));
    size_t o_qkv[PE_MAX_LAYERS], o_o[PE_MAX_LAYERS], o_gu[PE_MAX_LAYERS], o_dn[PE_MAX_LAYERS];
    for (int l = 0; l < c.n_layers; ++l) {
      o_qkv[l] = take(packed_bytes(qkvd, l == 0 && c.row_concat ? 2 * d : d));
      o_o[l] = take(packed_bytes(d, qd));
      o_gu[l] = take(2 * packed_bytes(F, d));
      o_dn[l] = take(packed_bytes(d, F));
    }
    const size_t o_lm = take(packed_bytes(V, d));
    const size_t o_fc4 = take(packed_ki4_bytes(d, 3 * d));
    size_t o_o4[PE_MAX_LAYERS], o_dn4[PE_MAX_LAYERS];
    for (int l = 0; l < c.n_layers; ++l) {
      o_o4[l] = take(packed_ki4_bytes(d, qd));
      o_dn4[l] = take(packed_ki4_bytes(d, F));
    }
    if (hipMalloc((void**)&ctx->packed, off) != hipSuccess) {
      free_ctx(ctx);
      return fail(nullptr, PE_ERR_OOM, "hipMalloc of packed weights failed");
    }
    char* base = ctx->packed;
    hipStream_t st = ctx->stream;
    auto chk = [&](hipError_t r) { return r == hipSuccess; };
    bool ok = chk(launch_pack_bf16(w->fc, nullptr, d, 3 * d, PACK_PLAIN, 0, base + o_fc, st));
    ctx->p_fc = base + o_fc;
    for (int l = 0; l < c.n_layers && ok; ++l) {
      ok = ok && chk(launch_pack_bf16(w->wqkv[l], nullptr, qkvd, l == 0 && c.row_concat ? 2 * d : d, PACK_PAIRS, hd,
                                      base + o_qkv[l], st));
      ok = ok && chk(launch_pack_bf16(w->wo[l], nullptr, d, qd, PACK_PLAIN, 0, base + o_o[l], st));
      ok = ok && chk(launch_pack_bf16(w->wgate[l], w->wup[l], F, d, PACK_GATEUP, 0, base + o_gu[l], st));
      ok = ok && chk(launch_pack_bf16(w->wdown[l], nullptr, d, F, PACK_PLAIN, 0, base + o_dn[l], st));
      ctx->p_qkv[l] = base + o_qkv[l];
      ctx->p_o[l] = base + o_o[l];
      ctx->p_gu[l] = base + o_gu[l];
      ctx->p_down[l] = base + o_dn[l];
    }
    ok = ok && chk(launch_pack_bf16(w->lm_head, nullptr, V, d, PACK_PLAIN, 0, base + o_lm, st));
    ctx->p_lm = base + o_lm;
    ok = ok && chk(launch_pack_bf16(w->fc, nullptr, d, 3 * d, PACK_KI4, 0, base + o_fc4, st));
    ctx->p_fc4 = base + o_fc4;
    for (int l = 0; l < c.n_layers && ok; ++l) {
      ok = ok && chk(launch_pack_bf16(w->wo[l], nullptr, d, qd, PACK_KI4, 0, base + o_o4[l], st));
      ok = ok && chk(launch_pack_bf16(w->wdown[l], nullptr, d, F, PACK_KI4, 0, base + o_dn4[l], st));
      ctx->p_o4[l] = base + o_o4[l];
      ctx->p_down4[l] = base + o_dn4[l];
    }
    if (!ok) {
      free_ctx(ctx);
      return fail(nullptr, PE_ERR_HIP, "weight packing launch failed");
    }
  }

  // ---- FP8 copies of the projections (weight_fp8)
  if (ctx->bf16 && c.weight_fp8) {
    ctx->fp8 = true;
    size_t off = 0;
    auto take = [&](size_t b) { size_t o = off; off = align256(off + b); return o; };
    auto q_bytes = [](int Nt, int Kd) { return (size_t)Nt * ((k_steps(Kd) + 1) / 2) * 1024; };
    auto s_bytes = [](int Nt) { return (size_t)Nt * 16 * 4; };
    const size_t o_fc = take(q_bytes(n_tiles(d), 3 * d)), os_fc = take(s_bytes(n_tiles(d)));
    size_t o_q[PE_MAX_LAYERS][4], os_q[PE_MAX_LAYERS][4];
    const int nts[4] = {n_tiles(qkvd), n_tiles(d), (2 * F + 15) / 16, n_tiles(d)};
    const int kds[4] = {d, qd, d, F};
    for (int l = 0; l < c.n_layers; ++l)
      for (int j = 0; j < 4; ++j) {
        o_q[l][j] = take(q_bytes(nts[j], kds[j]));
        os_q[l][j] = take(s_bytes(nts[j]));
      }
    const size_t o_lm = take(q_bytes(n_tiles(V), d)), os_lm = take(s_bytes(n_tiles(V)));
    if (hipMalloc((void**)&ctx->packed8, off) != hipSuccess) {
      free_ctx(ctx);
      return fail(nullptr, PE_ERR_OOM, "hipMalloc of FP8 weights failed");
    }
    char* base = ctx->packed8;
    hipStream_t st = ctx->stream;
    auto chk = [&](hipError_t r) { return r == hipSuccess; };
    bool ok = chk(launch_pack_fp8(w->fc, nullptr, d, 3 * d, PACK_PLAIN, 0, base + o_fc, (float*)(base + os_fc), st));
    ctx->q_fc = base + o_fc;
    ctx->s_fc = (const float*)(base + os_fc);
    for (int l = 0; l < c.n_layers && ok; ++l) {
      ok = ok && chk(launch_pack_fp8(w->wqkv[l], nullptr, qkvd, d, PACK_PAIRS, hd, base + o_q[l][0],
                                     (float*)(base + os_q[l][0]), st));
      ok = ok && chk(launch_pack_fp8(w->wo[l], nullptr, d, qd, PACK_PLAIN, 0, base + o_q[l][1],
                                     (float*)(base + os_q[l][1]), st));
      ok = ok && chk(launch_pack_fp8(w->wgate[l], w->wup[l], F, d, PACK_GATEUP, 0, base + o_q[l][2],
                                     (float*)(base + os_q[l][2]), st));
      ok = ok && chk(launch_pack_fp8(w->wdown[l], nullptr, d, F, PACK_PLAIN, 0, base + o_q[l][3],
                                     (float*)(base + os_q[l][3]), st));
      ctx->q_qkv[l] = base + o_q[l][0]; ctx->s_qkv[l] = (const float*)(base + os_q[l][0]);
      ctx->q_o[l] = base + o_q[l][1]; ctx->s_o[l] = (const float*)(base + os_q[l][1]);
      ctx->q_gu[l] = base + o_q[l][2]; ctx->s_gu[l] = (const float*)(base + os_q[l][2]);
      ctx->q_down[l] = base + o_q[l][3]; ctx->s_down[l] = (const float*)(base + os_q[l][3]);
    }
    ok = ok && chk(launch_pack_fp8(w->lm_head, nullptr, V, d, PACK_PLAIN, 0, base + o_lm, (float*)(base + os_lm), st));
    ctx->q_lm = base + o_lm;
    ctx->s_lm = (const float*)(base + os_lm);
    if (!ok) {
      free_ctx(ctx);
      return fail(nullptr, PE_ERR_HIP, "FP8 weight packing launch failed");
    }
  }

  // ---- workspace sizes (maxima over every B <= max_batch, K <= max_k)
  size_t p_floats = 0, attn_floats = 0, am_floats = 0, part_floats = 0;
  for (int M = 1; M <= Mmax; ++M) {
    if (ctx->bf16) {
      GemmPlan pl = plan_for(ctx, M, V, d, true);
      am_floats = std::max(am_floats, (size_t)M * pl.ngroups);
      // K-split partials of the layer projections and of the row build (B rows, or B R for a catch-up step)
      // (and layer 0's QKV over concatenated rows, 2d wide)
      const int shapes[6][2] = {{qkvd, d}, {d, qd}, {2 * F, d}, {d, F}, {d, 3 * d}, {qkvd, 2 * d}};
      for (int sh = 0; sh < (c.row_concat ? 6 : 5); ++sh) {
        const GemmPlan ps = plan_for(ctx, M, shapes[sh][0], shapes[sh][1], false);
        if (ps.ksplit > 1) part_floats = std::max(part_floats, (size_t)ps.ksplit * M * shapes[sh][0]);
      }
    } else {
      p_floats = std::max(p_floats, (size_t)M * std::max(std::max(qkvd, 2 * F), d));
      am_floats = std::max(am_floats, (size_t)M * plan_argmax_chunks(M, V));
    }
  }
  for (int B = 1; B <= c.max_batch; ++B) {
    if (ctx->bf16) {
      for (int K = 1; K <= c.max_k + 1; ++K) {
        AttnPlan ap = plan_attention(B, K, c.n_q_heads, c.n_kv_heads, hd, c.max_ctx);
        attn_floats = std::max(attn_floats, attn_partial_floats(B * K, c.n_q_heads, hd, ap));
      }
    } else {
      p_floats = std::max(p_floats, (size_t)B * d);
    }
    for (int K = 1; K <= c.max_k; ++K) {
      const int rows = B * (K + 1);
      am_floats = std::max(am_floats, (size_t)rows * plan_argmax_chunks(rows, V));
    }
  }
  const int nssq = (d + 3) / 4;  // the finest producer granularity (4-column tiles)
  size_t off = 0;
  auto take = [&](size_t b) { size_t o = off; off = align256(off + b); return o; };
  const size_t oX = take((size_t)Mmax * d * 4), oU = take((size_t)Mmax * d * es), oQ = take((size_t)Mmax * qd * es),
               oO = take((size_t)Mmax * qd * es), oA = take((size_t)Mmax * F * es), oP = take(p_floats * 4),
               oAt = take(std::max(attn_floats, (size_t)1) * 4), oAv = take(am_floats * 4), oAi = take(am_floats * 4),
               oT = take((size_t)c.max_batch * (c.max_k + 1) * 4),
               oL = take(ctx->bf16 ? 0 : (size_t)Mmax * V * 4), oR = take((size_t)c.max_ctx * (hd / 2) * 8),
               oS = take((size_t)Mmax * nssq * 4), oF = take(256), oK = take(part_floats * 4),
               oArT = take((size_t)c.max_batch * 4), oArS = take((size_t)c.max_batch * 4),
               oSm = take((size_t)2 * c.max_batch * (c.max_k + 1) * plan_sample_chunks(V) * 4),
               oXe = take(c.row_concat ? (size_t)Mmax * d * 4 : 0), oUc = take(c.row_concat ? (size_t)Mmax * 2 * d * 2 : 0);
  if (hipMalloc((void**)&ctx->ws, off) != hipSuccess) {
    free_ctx(ctx);
    return fail(nullptr, PE_ERR_OOM, "hipMalloc of workspace failed");
  }
  char* b = ctx->ws;
  ctx->X = (float*)(b + oX);
  ctx->U = b + oU;
  ctx->Qb = b + oQ;
  ctx->Ob = b + oO;
  ctx->Ab = b + oA;
  ctx->P = (float*)(b + oP);
  ctx->attn = (float*)(b + oAt);
  ctx->am_val = (float*)(b + oAv);
  ctx->am_idx = (int*)(b + oAi);
  ctx->t_ws = (int*)(b + oT);
  ctx->logits_ws = ctx->bf16 ? nullptr : (float*)(b + oL);
  ctx->rope = (float2*)(b + oR);
  ctx->ssq = (float*)(b + oS);
  ctx->flags = (int*)(b + oF);
  ctx->part = part_floats ? (float*)(b + oK) : nullptr;
  ctx->ar_tok = (int*)(b + oArT);
  ctx->ar_seq = (int*)(b + oArS);
  ctx->samp = (float*)(b + oSm);
  ctx->Xe = c.row_concat ? (float*)(b + oXe) : nullptr;
  ctx->Ucat = c.row_concat ? (void*)(b + oUc) : nullptr;

  hipError_t r = launch_rope_table(ctx->rope, c.max_ctx, hd, (double)c.rope_base, ctx->stream);
  if (r == hipSuccess) r = hipMemsetAsync(ctx->flags, 0, 256, ctx->stream);
  if (r == hipSuccess) r = hipStreamSynchronize(ctx->stream);
  if (r != hipSuccess) {
    std::string msg = std::string("pe_init: ") + hipGetErrorString(r);
    free_ctx(ctx);
    return fail(nullptr, PE_ERR_HIP, msg);
  }
  *out = ctx;
  return PE_OK;
}

extern "C" pe_status pe_destroy(pe_ctx* ctx) {
  if (!ctx) return PE_OK;
  hipError_t e = hipStreamSynchronize(ctx->stream);
  free_ctx(ctx);
  if (e != hipSuccess) return fail(nullptr, PE_ERR_HIP, std::string("pe_destroy: ") + hipGetErrorString(e));
  return PE_OK;
}

// ---- per-launch event timing of selected kernels
static hipError_t prof_mark(pe_ctx* c, int which, bool begin) {
  if (!(c->prof & (1 << which))) return hipSuccess;
  auto& pool = begin ? c->ev_a[which] : c->ev_b[which];
  size_t i = c->ev_used[which];
  if (i >= 65536) return hipSuccess;  // stop recording beyond the cap
  while (pool.size() <= i) {
    hipEvent_t e;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) return r;
    pool.push_back(e);
  }
  hipError_t r = hipEventRecord(pool[i], c->stream);
  if (!begin) c->ev_used[which] = i + 1;
  return r;
}

extern "C" pe_status pe_profile_enable(pe_ctx* ctx, int32_t mask) {
  if (!ctx) return fail(nullptr, PE_ERR_INVALID, "ctx is NULL");
  HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
  ctx->prof = mask & ((1 << PE_PROF_COUNT) - 1);
  for (int k = 0; k < PE_PROF_COUNT; ++k) ctx->ev_used[k] = 0;
  return PE_OK;
}

extern "C" pe_status pe_profile_read(pe_ctx* ctx, int32_t which, double* total_ms, int64_t* launches) {
  if (!ctx || !total_ms || !launches) return fail(ctx, PE_ERR_INVALID, "NULL argument");
  if (which < 0 || which >= PE_PROF_COUNT) return fail(ctx, PE_ERR_INVALID, "unknown kernel id");
  HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
  double tot = 0.0;
  for (size_t i = 0; i < ctx->ev_used[which]; ++i) {
    float ms = 0.f;
    HIP_TRY(ctx, hipEventElapsedTime(&ms, ctx->ev_a[which][i], ctx->ev_b[which][i]));
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)ctx->ev_used[which];
  return PE_OK;
}

extern "C" pe_status pe_device_flags(pe_ctx* ctx, int32_t clear, int32_t* flags) {
  if (!ctx || !flags) return fail(ctx, PE_ERR_INVALID, "NULL argument");
  HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
  HIP_TRY(ctx, hipMemcpy(flags, ctx->flags, sizeof(int32_t), hipMemcpyDeviceToHost));
  if (clear) {
    HIP_TRY(ctx, hipMemsetAsync(ctx->flags, 0, sizeof(int32_t), ctx->stream));
    HIP_TRY(ctx, hipStreamSynchronize(ctx->stream));
  }
  return PE_OK;
}

#define LAUNCH(call) HIP_TRY(ctx, (call))

// fp32 drafter: one kernel per step of the layer (small shapes only)
static pe_status draft_f32(pe_ctx* ctx, int32_t B, int32_t K, int32_t Kout, const int32_t* req_slot,
                           const int32_t* seq_len,
                           const int32_t* last_token, const void* target_hidden, const float* rows,
                           int32_t* draft_tokens, float* logits) {
  const pe_config& c = ctx->cfg;
  hipStream_t st = ctx->stream;
  const int d = c.d_model, F = c.ffn_dim, V = c.vocab, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int qd = Hq * hd, qkvd = (Hq + 2 * Hkv) * hd;
  const int M = B * K;
  const float eps = c.rms_eps;
  const pe_weights& w = ctx->w;
  float* P = ctx->P;
  if (!rows) LAUNCH(launch_gemm_f32((const float*)target_hidden, 3 * d, B, 3 * d, (const float*)w.fc, d, P, d, st));
  LAUNCH(launch_rowbuild_norm(0, ctx->X, ctx->U, P, 1, rows, B, K, d, last_token, w.embed, w.emb_mask, w.h_shared,
                              w.attn_norm[0], eps, V, ctx->flags, st));
  for (int l = 0; l < c.n_layers; ++l) {
    LAUNCH(launch_gemm_f32((const float*)ctx->U, d, M, d, (const float*)w.wqkv[l], qkvd, P, qkvd, st));
    LAUNCH(launch_rope_kv(0, ctx->Qb, ctx->kv.k[l], ctx->kv.v[l], P, 1, B, K, Hq, Hkv, hd, seq_len, req_slot,
                          c.max_ctx, c.n_slots, ctx->rope, ctx->flags, st));
    LAUNCH(prof_mark(ctx, PE_PROF_ATTENTION, true));
    LAUNCH(launch_attention_f32((const float*)ctx->Qb, (const float*)ctx->kv.k[l], (const float*)ctx->kv.v[l], seq_len,
                                req_slot, B, K, Hq, Hkv, hd, c.max_ctx, c.n_slots, (float*)ctx->Ob, st));
    LAUNCH(prof_mark(ctx, PE_PROF_ATTENTION, false));
    LAUNCH(launch_gemm_f32((const float*)ctx->Ob, qd, M, qd, (const float*)w.wo[l], d, P, d, st));
    LAUNCH(launch_residual_norm(0, ctx->X, ctx->U, P, 1, M, d, w.mlp_norm[l], eps, st));
    LAUNCH(prof_mark(ctx, PE_PROF_GATE_UP, true));
    LAUNCH(launch_gemm_f32((const float*)ctx->U, d, M, d, (const float*)w.wgate[l], F, P, 2 * F, st));
    LAUNCH(launch_gemm_f32((const float*)ctx->U, d, M, d, (const float*)w.wup[l], F, P + F, 2 * F, st));
    LAUNCH(prof_mark(ctx, PE_PROF_GATE_UP, false));
    LAUNCH(launch_swiglu(0, ctx->Ab, P, 1, M, F, false, st));
    LAUNCH(launch_gemm_f32((const float*)ctx->Ab, F, M, F, (const float*)w.wdown[l], d, P, d, st));
    const void* g_next = l + 1 < c.n_layers ? w.attn_norm[l + 1] : w.final_norm;
    LAUNCH(launch_residual_norm(0, ctx->X, ctx->U, P, 1, M, d, g_next, eps, st));
  }
  // LM head and argmax on the Kout emitted rows of every request
  const int Mo = B * Kout;
  float* z = logits ? logits : ctx->logits_ws;
  LAUNCH(prof_mark(ctx, PE_PROF_LM_HEAD, true));
  LAUNCH(launch_gemm_f32((const float*)ctx->U, d, Mo, d, (const float*)w.lm_head, V, z, V, st, K, Kout));
  LAUNCH(prof_mark(ctx, PE_PROF_LM_HEAD, false));
  const int nch = plan_argmax_chunks(Mo, V);
  LAUNCH(launch_argmax_rows(0, z, Mo, V, nch, ctx->am_val, ctx->am_idx, st));
  LAUNCH(launch_argmax_final(ctx->am_val, ctx->am_idx, Mo, nch, draft_tokens, st));
  return PE_OK;
}

// bf16 drafter: per layer six kernels (QKV+RoPE+KV append, attention, combine, O+residual, gate/up+SwiGLU,
// down+residual); RMSNorm is applied while the next projection reads its input.
static GemmArgs gemm_base(pe_ctx* ctx) {
  GemmArgs base{};
  base.Xout = ctx->X;
  base.XGout = (uint16_t*)ctx->U;  // XG = bf16(x * g) of the next normalised projection lives in the U buffer
  base.ssq_in = ctx->ssq;
  base.ssq_out = ctx->ssq;
  base.eps = ctx->cfg.rms_eps;
  base.flags = ctx->flags;
  base.part = ctx->part;
  return base;
}

// a1 (+ the sums of squares for layer 0's RMSNorm): Kr input rows per request from the row builder. With
// n_real, request b's first n_real[b] of its R token / hidden pairs are real rows (catch-up); else R = 1.
static pe_status rows_bf16(pe_ctx* ctx, int32_t B, int32_t Kr, const int32_t* last_token, const void* target_hidden,
                           int& nssq, int32_t R = 1, const int32_t* n_real = nullptr) {
  const pe_config& c = ctx->cfg;
  const int d = c.d_model;
  GemmArgs a = gemm_base(ctx);
  a.M = B * R; a.Kd = 3 * d; a.N = d;
  a.A = (const uint16_t*)target_hidden; a.lda = 3 * d;
  a.Kdraft = Kr; a.last_token = last_token; a.V = c.vocab;
  a.rows_real = R; a.n_real = n_real;
  a.Xe = ctx->Xe;
  a.embed = (const uint16_t*)ctx->w.embed; a.emb_mask = (const uint16_t*)ctx->w.emb_mask;
  a.h_shared = (const uint16_t*)ctx->w.h_shared;
  a.gain_next = (const uint16_t*)ctx->w.attn_norm[0];
  const GemmPlan p = plan_for(ctx, B * R, d, 3 * d, false, true);
  a.Wp_raw = ctx->fp8 ? ctx->q_fc : p.ki4 ? ctx->p_fc4 : ctx->p_fc;
  a.wscale = ctx->fp8 ? ctx->s_fc : nullptr;
  a.nssq_out = nssq = gemm_ssq_parts(p);
  hipStream_t st = ctx->stream;
  LAUNCH(prof_mark(ctx, PE_PROF_ROWS, true));
  LAUNCH(launch_gemm(p, a, A_BF16, EPI_ROWS, st));
  LAUNCH(prof_mark(ctx, PE_PROF_ROWS, false));
  return PE_OK;
}

// a2-a8 for every layer over the B * K rows in X (and their normalised operand); row j of request b sits
// at position seq_len[b] + j. nssq: the partial sums of squares per row of X on entry, updated on exit.
static pe_status layers_bf16(pe_ctx* ctx, int32_t B, int32_t K, const int32_t* req_slot, const int32_t* seq_len,
                             int& nssq) {
  const pe_config& c = ctx->cfg;
  hipStream_t st = ctx->stream;
  const int d = c.d_model, F = c.ffn_dim, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int qd = Hq * hd, qkvd = (Hq + 2 * Hkv) * hd;
  const int M = B * K;
  const pe_weights& w = ctx->w;
  uint16_t* XG = (uint16_t*)ctx->U;
  const GemmArgs base = gemm_base(ctx);
  for (int l = 0; l < c.n_layers; ++l) {
    {  // a2-a4: RMSNorm, QKV, RoPE, KV append (concatenated rows: layer 0 reads the normalised 2d-wide rows)
      const bool cat = l == 0 && ctx->Ucat;
      GemmArgs a = base;
      a.M = M; a.Kd = cat ? 2 * d : d; a.N = qkvd;
      a.A = cat ? (const uint16_t*)ctx->Ucat : XG; a.lda = a.Kd;
      a.Wp_raw = ctx->fp8 ? ctx->q_qkv[l] : ctx->p_qkv[l];
      a.wscale = ctx->fp8 ? ctx->s_qkv[l] : nullptr;
      a.Q = (uint16_t*)ctx->Qb; a.Kc = (uint16_t*)ctx->kv.k[l]; a.Vc = (uint16_t*)ctx->kv.v[l];
      a.seq_len = seq_len; a.req_slot = req_slot; a.rope = ctx->rope;
      a.Kdraft = K; a.Hq = Hq; a.Hkv = Hkv; a.hd = hd; a.max_ctx = c.max_ctx; a.n_slots = c.n_slots;
      a.nssq = nssq;
      if (cat)
        LAUNCH(launch_concat_norm(ctx->X, ctx->Xe, (const uint16_t*)w.attn_norm[0], (const uint16_t*)w.embed_norm,
                                  (uint16_t*)ctx->Ucat, M, d, c.rms_eps, st));
      LAUNCH(prof_mark(ctx, PE_PROF_QKV, true));
      LAUNCH(launch_gemm(plan_for(ctx, M, qkvd, a.Kd, false), a, cat ? A_BF16 : A_NORM, EPI_QKV, st));
      LAUNCH(prof_mark(ctx, PE_PROF_QKV, false));
    }
    // a5: attention
    AttnPlan ap = plan_attention(B, K, Hq, Hkv, hd, c.max_ctx);
    LAUNCH(prof_mark(ctx, PE_PROF_ATTENTION, true));
    LAUNCH(launch_attention_bf16(ap, ctx->Qb, ctx->kv.k[l], ctx->kv.v[l], seq_len, req_slot, B, K, Hq, Hkv, hd,
                                 c.max_ctx, c.n_slots, ctx->attn, st));
    LAUNCH(launch_attention_combine_bf16(ap, ctx->attn, ctx->Ob, seq_len, req_slot, B, K, Hq, Hkv, hd, c.max_ctx,
                                         c.n_slots, st));
    LAUNCH(prof_mark(ctx, PE_PROF_ATTENTION, false));
    {  // a6: output projection + residual
      GemmArgs a = base;
      a.M = M; a.Kd = qd; a.N = d;
      a.A = (const uint16_t*)ctx->Ob; a.lda = qd;
      a.gain_next = (const uint16_t*)w.mlp_norm[l];
      const GemmPlan p = plan_for(ctx, M, d, qd, false, true);
      a.Wp_raw = ctx->fp8 ? ctx->q_o[l] : p.ki4 ? ctx->p_o4[l] : ctx->p_o[l];
      a.wscale = ctx->fp8 ? ctx->s_o[l] : nullptr;
      a.nssq_out = nssq = gemm_ssq_parts(p);
      LAUNCH(prof_mark(ctx, PE_PROF_O_PROJ, true));
      LAUNCH(launch_gemm(p, a, A_BF16, EPI_RESID, st));
      LAUNCH(prof_mark(ctx, PE_PROF_O_PROJ, false));
    }
    {  // a7: RMSNorm, gate/up, SwiGLU
      GemmArgs a = base;
      a.M = M; a.Kd = d; a.N = 2 * F;
      a.A = XG; a.lda = d;
      a.Wp_raw = ctx->fp8 ? ctx->q_gu[l] : ctx->p_gu[l];
      a.wscale = ctx->fp8 ? ctx->s_gu[l] : nullptr;
      a.Aout = (uint16_t*)ctx->Ab;
      a.F = F;
      a.nssq = nssq;
      LAUNCH(prof_mark(ctx, PE_PROF_GATE_UP, true));
      LAUNCH(launch_gemm(plan_for(ctx, M, 2 * F, d, false), a, A_NORM, EPI_SWIGLU, st));
      LAUNCH(prof_mark(ctx, PE_PROF_GATE_UP, false));
    }
    {  // a8: down projection + residual
      GemmArgs a = base;
      a.M = M; a.Kd = F; a.N = d;
      a.A = (const uint16_t*)ctx->Ab; a.lda = F;
      a.gain_next = (const uint16_t*)(l + 1 < c.n_layers ? w.attn_norm[l + 1] : w.final_norm);
      const GemmPlan p = plan_for(ctx, M, d, F, false, true);
      a.Wp_raw = ctx->fp8 ? ctx->q_down[l] : p.ki4 ? ctx->p_down4[l] : ctx->p_down[l];
      a.wscale = ctx->fp8 ? ctx->s_down[l] : nullptr;
      a.nssq_out = nssq = gemm_ssq_parts(p);
      LAUNCH(prof_mark(ctx, PE_PROF_DOWN, true));
      LAUNCH(launch_gemm(p, a, A_BF16, EPI_RESID, st));
      LAUNCH(prof_mark(ctx, PE_PROF_DOWN, false));
    }
  }
  return PE_OK;
}

// a9-a10: final RMSNorm, LM head, argmax on Kout of the K rows of every request (the first Kout, or with
// n_real those from row n_real[b] - 1 on); tokens [B * Kout]; logits row (b, j) at logits + (b * Kout + j) * ldz
static pe_status lm_head_bf16(pe_ctx* ctx, int32_t B, int32_t K, int32_t Kout, int nssq, int32_t* tokens,
                              float* logits, int ldz, int32_t R = 1, const int32_t* n_real = nullptr) {
  const pe_config& c = ctx->cfg;
  hipStream_t st = ctx->stream;
  const int Mo = B * Kout;
  GemmArgs a = gemm_base(ctx);
  a.M = Mo; a.Kd = c.d_model; a.N = c.vocab;
  a.A = (const uint16_t*)ctx->U; a.lda = c.d_model;
  a.rows_in = K; a.rows_out = Kout;
  a.rows_real = R; a.n_real = n_real;
  a.Wp_raw = ctx->fp8 ? ctx->q_lm : ctx->p_lm;
  a.wscale = ctx->fp8 ? ctx->s_lm : nullptr;
  a.am_val = ctx->am_val; a.am_idx = ctx->am_idx; a.logits = logits; a.ldz = ldz;
  a.nssq = nssq;
  GemmPlan p = plan_for(ctx, Mo, c.vocab, c.d_model, true);
  LAUNCH(prof_mark(ctx, PE_PROF_LM_HEAD, true));
  LAUNCH(launch_gemm(p, a, A_NORM, EPI_ARGMAX, st));
  LAUNCH(prof_mark(ctx, PE_PROF_LM_HEAD, false));
  LAUNCH(launch_argmax_final(ctx->am_val, ctx->am_idx, Mo, p.ngroups, tokens, st));
  return PE_OK;
}

#define PE_TRY(expr)                    \
  do {                                  \
    const pe_status s_ = (expr);        \
    if (s_ != PE_OK) return s_;         \
  } while (0)

static pe_status draft_bf16(pe_ctx* ctx, int32_t B, int32_t K, int32_t Kout, const int32_t* req_slot,
                            const int32_t* seq_len,
                            const int32_t* last_token, const void* target_hidden, const float* rows,
                            int32_t* draft_tokens, float* logits) {
  int nssq = 0;
  if (!rows) {
    PE_TRY(rows_bf16(ctx, B, K, last_token, target_hidden, nssq));
  } else {
    hipStream_t st = ctx->stream;
    const int d = ctx->cfg.d_model;
    LAUNCH(launch_rows_ssq(rows, ctx->X, ctx->ssq, (uint16_t*)ctx->U, (const uint16_t*)ctx->w.attn_norm[0], B * K, d,
                           st));
    nssq = (d + 15) / 16;
  }
  PE_TRY(layers_bf16(ctx, B, K, req_slot, seq_len, nssq));
  return lm_head_bf16(ctx, B, K, Kout, nssq, draft_tokens, logits, ctx->cfg.vocab);
}

// Autoregressive drafting on the same kernels: pass 0 runs the parallel step's row 0 at position L_b; pass
// i >= 1 runs the row (residual stream of pass i - 1) + E[token of pass i - 1] at position L_b + i; one more
// pass (layers only) at L_b + K writes the K/V an all-accepted verify keeps.
static pe_status draft_ar_bf16(pe_ctx* ctx, int32_t B, int32_t K, const int32_t* req_slot, const int32_t* seq_len,
                               const int32_t* last_token, const void* target_hidden, int32_t* draft_tokens,
                               float* logits) {
  const pe_config& c = ctx->cfg;
  hipStream_t st = ctx->stream;
  int nssq = 0;
  PE_TRY(rows_bf16(ctx, B, 1, last_token, target_hidden, nssq));
  for (int i = 0;; ++i) {
    PE_TRY(layers_bf16(ctx, B, 1, req_slot, i == 0 ? seq_len : ctx->ar_seq, nssq));
    if (i == K) break;
    PE_TRY(lm_head_bf16(ctx, B, 1, 1, nssq, ctx->ar_tok, logits ? logits + (size_t)i * c.vocab : nullptr,
                        K * c.vocab));
    LAUNCH(launch_ar_rows(ctx->X, (uint16_t*)ctx->U, ctx->ssq, (const uint16_t*)ctx->w.embed,
                          (const uint16_t*)ctx->w.attn_norm[0], ctx->ar_tok, draft_tokens, K, i + 1, seq_len,
                          ctx->ar_seq, B, c.d_model, c.vocab, ctx->flags, st));
    nssq = (c.d_model + 15) / 16;
  }
  return PE_OK;
}

// Catch-up step: request b runs its n_real[b] real rows at positions seq_len[b] .. and then placeholder
// rows, R + K rows in all; the K drafts come from rows n_real[b] - 1 .. n_real[b] + K - 2.
static pe_status draft_catchup_bf16(pe_ctx* ctx, int32_t B, int32_t K, int32_t R, const int32_t* req_slot,
                                    const int32_t* seq_len, const int32_t* n_real, const int32_t* tokens,
                                    const void* target_hidden, int32_t* draft_tokens, float* logits) {
  int nssq = 0;
  const int Kr = R + K;
  PE_TRY(rows_bf16(ctx, B, Kr, tokens, target_hidden, nssq, R, n_real));
  PE_TRY(layers_bf16(ctx, B, Kr, req_slot, seq_len, nssq));
  return lm_head_bf16(ctx, B, Kr, K, nssq, draft_tokens, logits, ctx->cfg.vocab, R, n_real);
}

static pe_status run_draft(pe_ctx* ctx, int32_t B, int32_t K, const int32_t* req_slot, const int32_t* seq_len,
                           const int32_t* last_token, const void* target_hidden, const float* rows,
                           int32_t* draft_tokens, float* logits) {
  if (!ctx) return fail(nullptr, PE_ERR_INVALID, "ctx is NULL");
  const pe_config& c = ctx->cfg;
  if (B < 1 || B > c.max_batch) return fail(ctx, PE_ERR_INVALID, "B out of [1, max_batch]");
  if (K < 1 || K > c.max_k) return fail(ctx, PE_ERR_INVALID, "K out of [1, max_k]");
  if (!req_slot || !seq_len || !draft_tokens) return fail(ctx, PE_ERR_INVALID, "NULL request array");
  if (!rows && (!last_token || !target_hidden)) return fail(ctx, PE_ERR_INVALID, "NULL last_token / target_hidden");
  if (target_hidden && ((uintptr_t)target_hidden & 15)) return fail(ctx, PE_ERR_INVALID, "target_hidden not 16-byte aligned");
  if (logits && ((uintptr_t)logits & 15)) return fail(ctx, PE_ERR_INVALID, "logits not 16-byte aligned");
  if (rows && ((uintptr_t)rows & 15)) return fail(ctx, PE_ERR_INVALID, "rows not 16-byte aligned");
  // A draft step from the row builder also runs one placeholder row after the K draft rows (position
  // L_b + K), so the cache holds K/V for every position a verify can accept (accept_len <= K + 1); its
  // outputs are not emitted. Caller-built rows are run as given.
  const int Kr = rows ? K : K + 1;
  if (ctx->bf16)
    return draft_bf16(ctx, B, Kr, K, req_slot, seq_len, last_token, target_hidden, rows, draft_tokens, logits);
  return draft_f32(ctx, B, Kr, K, req_slot, seq_len, last_token, target_hidden, rows, draft_tokens, logits);
}

extern "C" pe_status pe_draft_step(pe_ctx* ctx, int32_t B, int32_t K, const int32_t* req_slot, const int32_t* seq_len,
                                   const int32_t* last_token, const void* target_hidden, int32_t* draft_tokens,
                                   float* logits) {
  if (ctx && (!last_token || !target_hidden)) return fail(ctx, PE_ERR_INVALID, "NULL last_token / target_hidden");
  return run_draft(ctx, B, K, req_slot, seq_len, last_token, target_hidden, nullptr, draft_tokens, logits);
}

extern "C" pe_status pe_draft_ar(pe_ctx* ctx, int32_t B, int32_t K, const int32_t* req_slot, const int32_t* seq_len,
                                 const int32_t* last_token, const void* target_hidden, int32_t* draft_tokens,
                                 float* logits) {
  if (!ctx) return fail(nullptr, PE_ERR_INVALID, "ctx is NULL");
  const pe_config& c = ctx->cfg;
  if (!ctx->bf16) return fail(ctx, PE_ERR_UNSUPPORTED, "autoregressive drafting needs a bf16 drafter");
  if (c.row_concat) return fail(ctx, PE_ERR_UNSUPPORTED, "autoregressive drafting with concatenated rows");
  if (B < 1 || B > c.max_batch) return fail(ctx, PE_ERR_INVALID, "B out of [1, max_batch]");
  if (K < 1 || K > c.max_k) return fail(ctx, PE_ERR_INVALID, "K out of [1, max_k]");
  if (!req_slot || !seq_len || !draft_tokens || !last_token || !target_hidden)
    return fail(ctx, PE_ERR_INVALID, "NULL argument");
  if ((uintptr_t)target_hidden & 15) return fail(ctx, PE_ERR_INVALID, "target_hidden not 16-byte aligned");
  if (logits && ((uintptr_t)logits & 15)) return fail(ctx, PE_ERR_INVALID, "logits not 16-byte aligned");
  return draft_ar_bf16(ctx, B, K, req_slot, seq_len, last_token, target_hidden, draft_tokens, logits);
}

extern "C" pe_status pe_draft_catchup(pe_ctx* ctx, int32_t B, int32_t K, int32_t R, const int32_t* req_slot,
                                      const int32_t* seq_len, const int32_t* n_real, const int32_t* tokens,
                                      const void* target_hidden, int32_t* draft_tokens, float* logits) {
  if (!ctx) return fail(nullptr, PE_ERR_INVALID, "ctx is NULL");
  const pe_config& c = ctx->cfg;
  if (!ctx->bf16) return fail(ctx, PE_ERR_UNSUPPORTED, "catch-up steps need a bf16 drafter");
  if (c.row_concat) return fail(ctx, PE_ERR_UNSUPPORTED, "catch-up steps with concatenated rows");
  if (B < 1 || B > c.max_batch) return fail(ctx, PE_ERR_INVALID, "B out of [1, max_batch]");
  if (K < 1 || K > c.max_k) return fail(ctx, PE_ERR_INVALID, "K out of [1, max_k]");
  if (R < 1 || R + K > c.max_k + 1) return fail(ctx, PE_ERR_INVALID, "R out of [1, max_k + 1 - K]");
  if (!req_slot || !seq_len || !n_real || !tokens || !target_hidden || !draft_tokens)
    return fail(ctx, PE_ERR_INVALID, "NULL argument");
  if ((uintptr_t)target_hidden & 15) return fail(ctx, PE_ERR_INVALID, "target_hidden not 16-byte aligned");
  if (logits && ((uintptr_t)logits & 15)) return fail(ctx, PE_ERR_INVALID, "logits not 16-byte aligned");
  return draft_catchup_bf16(ctx, B, K, R, req_slot, seq_len, n_real, tokens, target_hidden, draft_tokens, logits);
}

extern "C" pe_status pe_draft_rows(pe_ctx* ctx, int32_t B, int32_t K, const int32_t* req_slot, const int32_t* seq_len,
                                   const float* rows, int32_t* draft_tokens, float* logits) {
  if (ctx && !rows) return fail(ctx, PE_ERR_INVALID, "rows is NULL");
  if (ctx && ctx->cfg.row_concat) return fail(ctx, PE_ERR_UNSUPPORTED, "caller rows with concatenated rows");
  return run_draft(ctx, B, K, req_slot, seq_len, nullptr, nullptr, rows, draft_tokens, logits);
}

extern "C" pe_status pe_verify_sampled(pe_ctx* ctx, int32_t B, int32_t K, const void* target_logits,
                                       const int32_t* draft_tokens, float temperature, const float* u,
                                       const float* v, const uint8_t* finished, const int32_t* req_slot,
                                       const int32_t* seq_len, int32_t* accept_len, int32_t* cu_accept,
                                       int32_t* out_tokens, int32_t* keep_index, int32_t* n_keep,
                                       int32_t* req_slot_next, int32_t* seq_len_next, int32_t* last_token_next) {
  if (!ctx) return fail(nullptr, PE_ERR_INVALID, "ctx is NULL");
  const pe_config& c = ctx->cfg;
  if (B < 1 || B > c.max_batch) return fail(ctx, PE_ERR_INVALID, "B out of [1, max_batch]");
  if (K < 1 || K > c.max_k) return fail(ctx, PE_ERR_INVALID, "K out of [1, max_k]");
  if (!(temperature > 0.f) || temperature > 3.0e38f) return fail(ctx, PE_ERR_INVALID, "temperature must be > 0 and finite");
  if (!target_logits || !draft_tokens || !u || !v || !req_slot || !seq_len || !accept_len || !cu_accept ||
      !out_tokens || !keep_index || !n_keep || !req_slot_next || !seq_len_next || !last_token_next)
    return fail(ctx, PE_ERR_INVALID, "NULL argument");
  if ((uintptr_t)target_logits & 15) return fail(ctx, PE_ERR_INVALID, "target_logits not 16-byte aligned");
  if (c.vocab % 8) return fail(ctx, PE_ERR_UNSUPPORTED, "sampled verify needs vocab % 8 == 0");
  hipStream_t st = ctx->stream;
  const int rows = B * (K + 1);
  const int nch = plan_sample_chunks(c.vocab);
  float* pm = ctx->samp;
  float* ps = ctx->samp + (size_t)rows * nch;
  LAUNCH(launch_sampled_verify(ctx->bf16 ? 1 : 0, target_logits, B, K, c.vocab, nch, temperature, draft_tokens, u, v,
                               finished, req_slot, seq_len, pm, ps, ctx->t_ws, accept_len,
                               cu_accept, out_tokens, keep_index, n_keep, req_slot_next, seq_len_next,
                               last_token_next, st));
  return PE_OK;
}

extern "C" pe_status pe_verify(pe_ctx* ctx, int32_t B, int32_t K, const void* target_logits,
                               const int32_t* draft_tokens, const uint8_t* finished, const int32_t* req_slot,
                               const int32_t* seq_len, int32_t* accept_len, int32_t* cu_accept, int32_t* out_tokens,
                               int32_t* keep_index, int32_t* n_keep, int32_t* req_slot_next, int32_t* seq_len_next,
                               int32_t* last_token_next) {
  if (!ctx) return fail(nullptr, PE_ERR_INVALID, "ctx is NULL");
  const pe_config& c = ctx->cfg;
  if (B < 1 || B > c.max_batch) return fail(ctx, PE_ERR_INVALID, "B out of [1, max_batch]");
  if (K < 1 || K > c.max_k) return fail(ctx, PE_ERR_INVALID, "K out of [1, max_k]");
  if (!target_logits || !draft_tokens || !req_slot || !seq_len || !accept_len || !cu_accept || !out_tokens ||
      !keep_index || !n_keep || !req_slot_next || !seq_len_next || !last_token_next)
    return fail(ctx, PE_ERR_INVALID, "NULL argument");
  if ((uintptr_t)target_logits & 15) return fail(ctx, PE_ERR_INVALID, "target_logits not 16-byte aligned");
  hipStream_t st = ctx->stream;
  const int rows = B * (K + 1);
  const int nch = plan_argmax_chunks(rows, c.vocab);
  LAUNCH(prof_mark(ctx, PE_PROF_VERIFY_SCAN, true));
  LAUNCH(launch_argmax_rows(ctx->bf16 ? 1 : 0, target_logits, rows, c.vocab, nch, ctx->am_val, ctx->am_idx, st));
  LAUNCH(prof_mark(ctx, PE_PROF_VERIFY_SCAN, false));
  LAUNCH(launch_accept_compact(ctx->am_val, ctx->am_idx, nch, B, K, draft_tokens, finished, req_slot, seq_len,
                               ctx->t_ws, accept_len, cu_accept, out_tokens, keep_index, n_keep, req_slot_next,
                               seq_len_next, last_token_next, st));
  return PE_OK;
}

// ---- greedy verify without a ctx: scratch in a static device array ----------------------------------
// The argmax partials and target tokens of pe_verify live in `scratch`, a file-scope device array of which
// every GPU holds its own copy. In host code its name is only a stand-in for the symbol, so each device's
// address is looked up once (hipGetSymbolAddress with that device current) and only that address is passed
// to the kernels.
static __device__ __align__(256) char scratch[PE_VERIFY_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices] = {};
}  // namespace

static pe_status static_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(nullptr, PE_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(nullptr, PE_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(nullptr, PE_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
      return fail(nullptr, PE_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", not gfx950");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(nullptr, PE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_dev[dev] = (char*)p;
  }
  *out = g_scratch_dev[dev];
  return PE_OK;
}

extern "C" pe_status pe_verify_static(int32_t B, int32_t K, int32_t vocab, int32_t dtype, const void* target_logits,
                                      const int32_t* draft_tokens, const uint8_t* finished, const int32_t* req_slot,
                                      const int32_t* seq_len, int32_t* accept_len, int32_t* cu_accept,
                                      int32_t* out_tokens, int32_t* keep_index, int32_t* n_keep,
                                      int32_t* req_slot_next, int32_t* seq_len_next, int32_t* last_token_next,
                                      void* stream) {
  if (B < 1 || B > PE_MAX_BATCH) return fail(nullptr, PE_ERR_INVALID, "B out of [1, 1024]");
  if (K < 1 || K > PE_MAX_K) return fail(nullptr, PE_ERR_INVALID, "K out of [1, 16]");
  if (vocab < 8 || vocab % 8) return fail(nullptr, PE_ERR_INVALID, "vocab must be a positive multiple of 8");
  if (dtype != PE_F32 && dtype != PE_BF16) return fail(nullptr, PE_ERR_INVALID, "dtype must be PE_F32 or PE_BF16");
  if (!target_logits || !draft_tokens || !req_slot || !seq_len || !accept_len || !cu_accept || !out_tokens ||
      !keep_index || !n_keep || !req_slot_next || !seq_len_next || !last_token_next)
    return fail(nullptr, PE_ERR_INVALID, "NULL argument");
  if ((uintptr_t)target_logits & 15) return fail(nullptr, PE_ERR_INVALID, "target_logits not 16-byte aligned");
  // scratch layout: argmax partial values [rows, nch], their indices [rows, nch], target tokens [B, K + 1]
  const int rows = B * (K + 1);
  const int nch = plan_argmax_chunks(rows, vocab);
  const size_t part = align256((size_t)rows * nch * sizeof(float));
  const size_t need = 2 * part + (size_t)rows * sizeof(int);
  if (need > (size_t)PE_VERIFY_STATIC_SCRATCH_BYTES)
    return fail(nullptr, PE_ERR_INVALID, "B and K need more than the static scratch holds");
  char* base = nullptr;
  PE_TRY(static_scratch(&base));
  float* pv = (float*)base;
  int* pi = (int*)(base + part);
  int* t_ws = (int*)(base + 2 * part);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_argmax_rows(dtype == PE_BF16 ? 1 : 0, target_logits, rows, vocab, nch, pv, pi, st);
  if (e == hipSuccess)
    e = launch_accept_compact(pv, pi, nch, B, K, draft_tokens, finished, req_slot, seq_len, t_ws, accept_len,
                              cu_accept, out_tokens, keep_index, n_keep, req_slot_next, seq_len_next, last_token_next,
                              st);
  if (e != hipSuccess) return fail(nullptr, PE_ERR_HIP, std::string("pe_verify_static: ") + hipGetErrorString(e));
  return PE_OK;
}
