/*
 * Oracle of the speculative-verify MoE decoder layer: TEST INFRASTRUCTURE.
 *
 * A plain, slow CPU definition of what one verify pass of one decoder layer
 * computes, used only by the tests, by the package's smoke check and by the
 * benchmark's CPU-baseline leg. It shares no code with the HIP path.
 *
 * Source: "Muse Spark Open Ultrafast: Pushing beyond 1,000 Tokens per second"
 * (LMSYS; summarised on newruntime.com "What happened", ai4snews
 * "Interpretation", orcarouter.ai sections "Dove si colloca il confine del
 * kernel" and the model paragraph that follows it). The layer: sliding-window
 * (2,048) or global attention over a bf16 KV cache, 16 verified tokens,
 * a router choosing 8 of 256 experts, a pooler that shrinks the token vector
 * before the experts, NVFP4 experts, an unpooler, and the next layer's
 * QKV projection and KV write.
 *
 * Floating point is fp64 except where the method fixes a precision:
 * stored tensors keep their formats (bf16 cache rows, NVFP4 experts), and the
 * router's top-k decision is taken on fp32 logits summed in one fixed order
 * (orc_dot_canon_f32), the same order the kernel uses.
 */
#ifndef MSK_ORACLE_H
#define MSK_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t hidden;       /* H */
  int32_t n_q_heads;    /* nq */
  int32_t n_kv_heads;   /* nkv, nq % nkv == 0 */
  int32_t head_dim;     /* d */
  int32_t n_experts;    /* E */
  int32_t top_k;        /* k */
  int32_t pool_dim;     /* P, multiple of 16 */
  int32_t expert_inter; /* I, multiple of 16 */
  int32_t window;       /* 0 = global attention */
  int32_t kv_capacity;  /* rows per (request, kv head) in the caches */
  float rms_eps;
  int32_t use_norm;     /* 1: RMSNorm before attention and before the MoE */
  int32_t act_fp4;      /* 1: SwiGLU outputs quantized to NVFP4 before the down projection */
  const uint16_t* w_qkv;      /* bf16 [nq*d + 2*nkv*d][H], rows Q | K | V */
  const uint16_t* w_o;        /* bf16 [H][nq*d] */
  const float* w_router;      /* fp32 [E][H] */
  const float* b_router;      /* fp32 [E] or NULL */
  const uint16_t* w_pool;     /* bf16 [P][H] */
  const uint16_t* w_unpool;   /* bf16 [H][P] */
  const uint16_t* g_attn;     /* bf16 [H] RMSNorm gain before attention */
  const uint16_t* g_moe;      /* bf16 [H] RMSNorm gain before the MoE */
  const uint8_t* e_gate_up;        /* [E][2I][P/2] E2M1, rows gate | up */
  const uint8_t* e_gate_up_scale;  /* [E][2I][P/16] E4M3 */
  const uint8_t* e_down;           /* [E][P][I/2] E2M1 */
  const uint8_t* e_down_scale;     /* [E][P][I/16] E4M3 */
  const float* e_tensor_scale;     /* [E][2]: gate_up, down */
} orc_layer;

/* Optional stage outputs of orc_layer_forward; every pointer may be NULL. */
typedef struct {
  double* q;       /* [NT][nq*d]   */
  double* k_new;   /* [NT][nkv*d]  before the bf16 store */
  double* v_new;   /* [NT][nkv*d]  */
  double* attn;    /* [NT][nq*d]   */
  double* h1;      /* [NT][H]      */
  float* n2_f32;   /* [NT][H]      router input */
  float* logits;   /* [NT][E]      fp32, bias included */
  int32_t* ids;    /* [NT][k]      */
  double* gates;   /* [NT][k]      */
  double* p;       /* [NT][P]      */
  double* acc;     /* [NT][P]      */
} orc_stages;

double orc_bf16_value(uint16_t b);
uint16_t orc_bf16_rne(double x);
double orc_e2m1_value(uint8_t nibble);
double orc_e4m3_value(uint8_t code);
void orc_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, double s_tensor,
                       int64_t rows, int64_t cols, double* out);
float orc_dot_canon_f32(const float* x, const float* w, int32_t n);
void orc_topk(const float* logits, int32_t n, int32_t k, int32_t* ids);
void orc_gates(const float* logits, const int32_t* ids, int32_t k, double* gates);
void orc_prefetch_list(const int32_t* ids, int32_t n_ids, int32_t n_experts, int32_t p, int32_t* list);
void orc_rmsnorm(const double* x, const uint16_t* g, int32_t n, double eps, double* y);
double orc_silu(double x);
/* Verify-token trees (orcarouter.ai, "Muse Spark Open: 1.109 token al
 * secondo ...", section "Anche il modello draft e' diventato piu' veloce":
 * the 16 verified tokens form a tree of candidates rather than a chain).
 * tree[t] is the ancestor set of token t as a bitmask over the T new tokens,
 * self included; NULL means the chain (bits 0..t). Valid masks hold bit t,
 * no bit above t, and are closed (an ancestor's ancestors are ancestors);
 * depth(t) = popcount(tree[t]) - 1 is the token's distance from the prior
 * context. Returns 1 if valid. */
int32_t orc_tree_valid(const uint16_t* tree, int32_t T);
/* NVFP4 quantization of activations (orcarouter.ai, section "Dove si colloca
 * il confine del kernel": after the first expert GEMM the activations travel
 * as fp4). One block = 16 consecutive fp32 values along the expert's
 * intermediate dim; every step below is one fp32 operation:
 *   amax = max |x_i|;  s = E4M3(fl32(amax / 6))  (round to nearest even,
 *   saturating at 448);  q_i = E2M1(fl32(x_i / s))  (nearest, ties to the
 *   even code, saturating at +-6, sign kept; 0 when s = 0);
 *   deq_i = E2M1(q_i) * s  (exact). */
uint8_t orc_e4m3_rne_sat(float x);
uint8_t orc_e2m1_rne_sat(float y);
void orc_nvfp4_quant16(const float* x, uint8_t* codes, uint8_t* scale, float* deq);
void orc_attention(const double* q, const uint16_t* k_cache, const uint16_t* v_cache,
                   int32_t nq, int32_t nkv, int32_t d, int32_t cap, int32_t T, int32_t ctx,
                   int32_t window, const uint16_t* tree, double* out);
int32_t orc_layer_forward(const orc_layer* L, int32_t R, int32_t T, const int32_t* ctx,
                          const uint16_t* tree, const double* h_in, uint16_t* k_cache,
                          uint16_t* v_cache, double* h_out, orc_stages* st);
int32_t orc_threads(void);
/* Threads of the OpenMP loops (timing only; results do not depend on it). */
void orc_set_threads(int32_t n);
void orc_dense_swiglu(const double* x, int32_t nt, const double* wgu, const double* wd,
                      int32_t P, int32_t I, double* y);

#ifdef __cplusplus
}
#endif

#endif /* MSK_ORACLE_H */
