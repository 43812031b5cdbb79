/*
 * msk — speculative-verify MoE layer kernel for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the library. The operation is the verify pass of a
 * mixture-of-experts decoder described in "Muse Spark Open Ultrafast: Pushing
 * beyond 1,000 Tokens per second" (LMSYS, Nov 2026; summaries on
 * newruntime.com, section "What happened", and orcarouter.ai, sections
 * "Dove si colloca il confine del kernel" and the model paragraph after it):
 * one resident kernel launch per layer boundary, covering one layer's
 * attention over a bf16 KV cache, the router (top-k of E experts), the pooler,
 * the NVFP4 expert SwiGLU, the unpooler, and then the next layer's QKV
 * projection and KV write.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are device pointers owned by the caller. Weights and KV
 *    caches are borrowed by msk_load_layer and must outlive the handle; IO
 *    buffers must stay valid until the enqueued work has finished.
 *  - Every device pointer must be 16-byte aligned (128-bit loads), except
 *    msk_io.ctx_len and msk_io.tree_mask (4-byte aligned).
 *  - The library allocates no device memory: its scratch space is the
 *    caller's workspace (msk_workspace_bytes). It allocates a few bytes of
 *    pinned host memory per handle for the device error word.
 *  - Calls are asynchronous on the given stream (a hipStream_t passed as
 *    void*; NULL is the default stream) and return once the work is
 *    enqueued. They enqueue no memset and no allocation, so a caller may
 *    capture them in a hipGraph. Calls on one handle are not thread-safe.
 *  - Errors are returned as msk_status; nothing throws or aborts across the
 *    ABI. msk_last_error() describes the last failure on a handle.
 *  - Argument, shape and alignment checks run on the host before any launch.
 *    What only the device can see (the device-side ctx_len and tree_mask,
 *    and a spin-wait that exceeded its budget) sets an error word in the
 *    workspace: the failed call and every later call on the handle then do
 *    nothing on the device (their outputs are invalid) until the error has
 *    been reported, by the next call that finds the failed call complete or
 *    by msk_synchronize.
 *
 * Weight layouts (row-major, [out][in], the input dim contiguous):
 *  w_qkv    bf16 [nq*d + 2*nkv*d][H], rows Q (head-major) | K | V
 *  w_o      bf16 [H][nq*d]
 *  w_router fp32 [E][H]; b_router fp32 [E] or NULL (added to the logits)
 *  w_pool   bf16 [P][H];   w_unpool bf16 [H][P]
 *  g_attn, g_moe bf16 [H]  RMSNorm gains (pre-attention, pre-MoE)
 *  e_gate_up       [E][2I][P/2]  E2M1 codes, rows gate | up; element 2j of a
 *                                row in the low nibble of byte j
 *  e_gate_up_scale [E][2I][P/16] E4M3 (OCP, bias 7) scale per 16 elements
 *  e_down          [E][P][I/2]   E2M1
 *  e_down_scale    E4M3 scale per 16 elements of e_down, tiled (written by
 *                  msk_pack_down_scale from the row-major [E][P][I/16]):
 *                  [E][P/16][S][16][8], S = ceil(I/128); byte b of row r in
 *                  slice s of tile t scales elements 16*(8s+b) .. +15 of row
 *                  16t+r; positions past I/16 hold 0
 *  e_tensor_scale  fp32 [E][2]   per-tensor scale of gate_up and of down
 *  k_cache, v_cache bf16 [max_requests][nkv][kv_capacity][d]
 * Activations: h_in / h_out fp32 [n_requests * n_tokens][H], request-major.
 */
#ifndef MSK_H
#define MSK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct msk_handle_s* msk_handle;

typedef enum {
  MSK_OK = 0,
  MSK_E_INVALID = 1,  /* NULL or out-of-range argument */
  MSK_E_SHAPE = 2,    /* shapes the kernel does not support */
  MSK_E_ALIGN = 3,    /* pointer not 16-byte aligned */
  MSK_E_STATE = 4,    /* layer not loaded, or handle in a failed state */
  MSK_E_CAPACITY = 5, /* ctx_len + n_tokens > kv_capacity (reported from the device), or workspace too small */
  MSK_E_HIP = 6,      /* a HIP runtime call failed */
  MSK_E_TIMEOUT = 7   /* a kernel wait exceeded its spin budget (reported by the next call) */
} msk_status;

/* msk_config.flags */
#define MSK_FLAG_NO_NORM 0x1u /* skip both RMSNorms (special-case tests) */
/* NVFP4 activations between the two expert GEMMs (orcarouter.ai, "Dove si
 * colloca il confine del kernel": the output of the first expert GEMM travels
 * as fp4). Each expert's SwiGLU output is quantized in blocks of 16 along the
 * intermediate dim: block scale s = E4M3(amax / 6) (OCP E4M3FN, nearest even,
 * saturating at 448), codes E2M1(x / s) (nearest even, saturating at 6, sign
 * kept; 0 when s = 0), and the down projection reads E2M1(code) * s. */
#define MSK_FLAG_ACT_FP4 0x2u
/* Tail prefetch of the next layer's KV window (orcarouter.ai, "Su cosa
 * vengono ancora spesi i 5,9 ms": old KV rows are loaded ahead while the
 * previous operations finish). During the next layer's QKV projection at the
 * end of each launch, the workgroups read one word of every 128-byte line of
 * the prior K and V rows that layer's attention will read, so that the next
 * launch finds them in the memory-side cache. No effect on results. */
#define MSK_FLAG_KV_PREFETCH 0x4u

typedef struct {
  int32_t hidden;        /* H: a power of two in 128..4096 */
  int32_t n_q_heads;     /* nq: a multiple of nkv; nq * d a multiple of 128, <= 4096 */
  int32_t n_kv_heads;    /* nkv; nq / nkv <= 8 */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t n_experts;     /* E: 1..256 */
  int32_t top_k;         /* k: 1..min(8, E) */
  int32_t pool_dim;      /* P: a multiple of 128, <= 2048 */
  int32_t expert_inter;  /* I: a multiple of 32, <= 1024 */
  int32_t n_layers;      /* layers of the step (msk_verify_step), >= 1 */
  int32_t max_tokens;    /* verify tokens per request: 1..16 */
  int32_t max_requests;  /* 1..4 */
  int32_t kv_capacity;   /* cache rows per (request, kv head), >= 1 */
  float rms_eps;         /* >= 0 */
  uint32_t flags;        /* MSK_FLAG_* bits; any other bit is rejected */
  int32_t expert_prefetch; /* 0 (off) .. min(32, n_experts): speculative expert prefetch.
                              At the start of each layer launch, the workgroups without
                              attention work rank the layer's experts by how often the
                              previous call selected them (count descending, index
                              ascending; LMSYS post, newruntime.com "What happened":
                              likely experts of the previous step are prefetched) and
                              read the first expert_prefetch of them (codes and scales)
                              so that they sit in the memory-side cache when the expert
                              phase runs. No effect on results. On MI355X at the
                              62-layer shape, 6..10 give the shortest step. */
} msk_config;

typedef struct {
  int32_t window; /* sliding window in keys (including the query's own position); 0 = global */
  const uint16_t* w_qkv;
  const uint16_t* w_o;
  const float* w_router;
  const float* b_router; /* may be NULL */
  const uint16_t* w_pool;
  const uint16_t* w_unpool;
  const uint16_t* g_attn;
  const uint16_t* g_moe;
  const uint8_t* e_gate_up;
  const uint8_t* e_gate_up_scale;
  const uint8_t* e_down;
  const uint8_t* e_down_scale;
  const float* e_tensor_scale;
  uint16_t* k_cache;
  uint16_t* v_cache;
} msk_layer_desc;

/* Optional stage dumps of msk_verify_layer (device pointers, each may be NULL;
 * NT = n_requests * n_tokens). Used to check stages one by one. */
typedef struct {
  float* q;          /* [NT][nq*d]   query rows of the layer */
  float* k_new;      /* [NT][nkv*d]  new K rows before the bf16 store */
  float* v_new;      /* [NT][nkv*d]  */
  float* attn;       /* [NT][nq*d]   attention output */
  float* h1;         /* [NT][H]      residual after the output projection */
  float* n2;         /* [NT][H]      fp32 router input */
  float* logits;     /* [NT][E]      fp32 router logits (bias included) */
  float* p;          /* [NT][P]      pooled vector */
  float* acc;        /* [NT][P]      gated expert sum, before the unpooler */
  int32_t dq_expert; /* expert whose decoded weights are dumped (if selected) */
  uint16_t* dq_gate_up; /* f16 [2I][P]: E2M1 x E4M3 (tensor scale not applied) */
  uint16_t* dq_down;    /* f16 [P][I] */
  /* With MSK_FLAG_ACT_FP4, for expert dq_expert (if selected), every token's
   * SwiGLU output before quantization (gate weight not applied) and its
   * NVFP4 encoding; tokens not routed to the expert are included. */
  float* act;           /* fp32 [NT][I] */
  uint8_t* act_codes;   /* [NT][I/2] E2M1, element 2m in the low nibble of byte m */
  uint8_t* act_scales;  /* [NT][I/16] E4M3 block scales */
  /* With MSK_FLAG_ACT_FP4, the same encoding for every selected expert, by
   * expert id (rows of experts not selected are left untouched). */
  uint8_t* act_codes_all;  /* [E][NT][I/2] */
  uint8_t* act_scales_all; /* [E][NT][I/16] */
} msk_debug;

typedef struct {
  int32_t n_requests;     /* R, 1 .. max_requests */
  int32_t n_tokens;       /* T tokens per request, 1 .. max_tokens */
  const int32_t* ctx_len; /* device [R], 4-byte aligned: prior context length; the
                             tokens' K/V are written at cache rows ctx_len[r] ..
                             ctx_len[r] + T - 1. Read by the kernels when they run
                             (a captured graph follows the values at replay time).
                             0 <= ctx_len[r] and ctx_len[r] + T <= kv_capacity, else
                             the call does nothing and reports MSK_E_INVALID /
                             MSK_E_CAPACITY later (see Conventions). */
  const float* h_in;      /* device fp32 [R*T][H] */
  float* h_out;           /* device fp32 [R*T][H] */
  int32_t* expert_ids;    /* device, may be NULL: [L][R*T][k] (verify_layer: [R*T][k]) */
  float* gates;           /* device, may be NULL: same shape as expert_ids */
  const msk_debug* debug; /* HOST struct, may be NULL; honoured by msk_verify_layer */
  int32_t* prefetch_ids;  /* device, may be NULL: [L][expert_prefetch] (verify_layer:
                             [expert_prefetch]) the prefetch list each layer used, i.e.
                             the ranking of the previous call's selections of that layer
                             (all counts zero before the first call on a handle). */
  uint64_t* trace;        /* device, may be NULL: self-timing variant of the kernel.
                             [launch][256][MSK_TRACE_SLOTS] uint64 stamps of the GPU's
                             100 MHz real-time counter, written by lane 0 of each
                             workgroup at the phase boundaries below; slots a launch
                             does not reach are left untouched. Exclusive with debug. */
  const uint16_t* tree_mask; /* device, may be NULL (= the causal chain), 4-byte
                             aligned: [R][T] ancestor bitmasks of the verify tokens. The tokens of a request
                             form a tree of candidates (orcarouter.ai, "Muse Spark
                             Open: 1.109 token al secondo ...", section "Anche il
                             modello draft e' diventato piu' veloce ..."). Bit u of
                             token t's mask = t attends to new token u. Each mask
                             must hold bit t, no bit above t, and the masks of its
                             ancestors (MSK_E_INVALID otherwise). Token t's position
                             is ctx_len + depth, depth = ancestors other than t: the
                             window covers the last `window` tokens of its own
                             sequence (prior context, then its path). K/V are still
                             written at ctx_len + t. Read by the kernels when they
                             run; an invalid mask makes the call do nothing and
                             report MSK_E_INVALID later. */
  float* layer_out;       /* device, may be NULL: [L][R*T][H] the residual leaving each
                             layer of the call (msk_verify_layer: [1][R*T][H]); the
                             last entry equals h_out. */
} msk_io;

/* Trace slots, in execution order ("_BAR" = after the grid barrier that
 * follows; "_FILL" = after the phase's activation tile is in LDS; ROUTING =
 * after top-k and the routing tables; ATTN_Q / ATTN_KV = attention's query
 * operand ready / first key-value chunk in LDS). */
enum {
  MSK_TR_START = 0, MSK_TR_QKV_OWN, MSK_TR_QKV_OWN_BAR, MSK_TR_ATTN_Q, MSK_TR_ATTN_KV, MSK_TR_ATTN,
  MSK_TR_ATTN_BAR,
  MSK_TR_MERGE, MSK_TR_MERGE_BAR, MSK_TR_OPROJ_FILL, MSK_TR_OPROJ, MSK_TR_OPROJ_BAR,
  MSK_TR_POOL_FILL, MSK_TR_ROUTER_POOL, MSK_TR_ROUTER_POOL_BAR, MSK_TR_ROUTING, MSK_TR_GEMM1,
  MSK_TR_GEMM1_BAR, MSK_TR_GEMM2, MSK_TR_GEMM2_BAR, MSK_TR_UNPOOL_FILL, MSK_TR_UNPOOL,
  MSK_TR_UNPOOL_BAR, MSK_TR_QKV_FILL, MSK_TR_QKV_NEXT, MSK_TRACE_SLOTS
};

/* Bytes of device workspace a handle needs for this configuration; 0 if the
 * configuration is invalid. */
size_t msk_workspace_bytes(const msk_config* cfg);

/* Create a handle. workspace: device memory of at least msk_workspace_bytes,
 * owned by the caller, 256-byte aligned, kept until msk_destroy. The call
 * writes the workspace's schedule tables (synchronously) and uses the current
 * HIP device. */
msk_status msk_create(const msk_config* cfg, void* workspace, size_t bytes, msk_handle* out);

/* Bytes of the library's own static workspace (one array per GPU). */
#define MSK_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)

/* Like msk_create, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the handle's workspace is a static array of
 * MSK_STATIC_WORKSPACE_BYTES that the library holds on each GPU it runs on
 * until the process ends, instead of caller memory, and no pinned host word
 * is taken. The call allocates no device or pinned memory (it uploads the
 * schedule tables and clears the array's header synchronously).
 * Returns MSK_E_CAPACITY, with a message, when msk_workspace_bytes(cfg)
 * exceeds MSK_STATIC_WORKSPACE_BYTES. Every static handle on one GPU uses
 * that GPU's single array: a second msk_create_static on the same GPU takes
 * it over (the earlier handle must not be used afterwards), and calls that
 * overlap in time on one GPU race. Device-side errors of a static handle are
 * reported by msk_synchronize only. Release with msk_destroy. */
msk_status msk_create_static(const msk_config* cfg, msk_handle* out);

/* Register layer `layer` (0 .. n_layers-1). Pointers are borrowed. */
msk_status msk_load_layer(msk_handle h, int32_t layer, const msk_layer_desc* desc);

/* One standalone layer: its own RMSNorm + QKV projection + KV write at
 * positions ctx_len[r] .., attention, output projection, router, pooler,
 * experts, unpooler. h_out = the layer's output residual. One kernel launch
 * (plus one tiny counter-reset launch). */
msk_status msk_verify_layer(msk_handle h, int32_t layer, const msk_io* io, void* stream);

/* The whole verify step over layers 0 .. n_layers-1: one resident kernel per
 * layer boundary. Launch L runs layer L's attention through its unpooler,
 * then layer L+1's RMSNorm, QKV projection and KV write; the first launch
 * also runs layer 0's QKV and KV write first. expert_ids/gates, if given,
 * receive every layer's routing. */
msk_status msk_verify_step(msk_handle h, const msk_io* io, void* stream);

/* Waits until the last call enqueued on h (outside graph capture) has
 * finished and returns the device status of the calls made so far: MSK_OK,
 * or the first error the device recorded (MSK_E_INVALID, MSK_E_CAPACITY,
 * MSK_E_TIMEOUT), which it reports once. Outputs of a call that failed on the
 * device, and of the calls after it until the report, are invalid. */
msk_status msk_synchronize(msk_handle h);

/* Release the handle (the workspace stays the caller's). */
msk_status msk_destroy(msk_handle h);

/* Bytes of a tiled e_down_scale buffer (see Weight layouts); 0 if the shape
 * is invalid (n_experts > 0, pool_dim a multiple of 16, expert_inter a
 * multiple of 32). */
size_t msk_down_scale_bytes(int32_t n_experts, int32_t pool_dim, int32_t expert_inter);

/* Reorder the down projection's block scales from row-major [E][P][I/16]
 * (src) into the tiled order msk_load_layer takes (dst, msk_down_scale_bytes
 * bytes). GEMM2 of the experts (the down projection, "NVFP4 expert SwiGLU" of
 * the pages above) reduces over I in 128-element slices per wave and 16 rows
 * of P per tile; in this order one wave's scales for one expert are one
 * 128-byte line. Both buffers are the caller's device memory, 16-byte
 * aligned, not overlapping. Asynchronous on `stream`; the values are not
 * changed. Failures are reported through msk_last_error(NULL). */
msk_status msk_pack_down_scale(const void* src, void* dst, int32_t n_experts, int32_t pool_dim,
                               int32_t expert_inter, void* stream);

/* Description of the last error on h (or, when h is NULL, of the last
 * failure of a call made without a handle: msk_create, msk_pack_down_scale).
 * Never NULL. */
const char* msk_last_error(msk_handle h);

#ifdef __cplusplus
}
#endif

#endif /* MSK_H */
