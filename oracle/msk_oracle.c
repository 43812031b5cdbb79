/*
 * Oracle of the speculative-verify MoE decoder layer: TEST INFRASTRUCTURE.
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load this library. See msk_oracle.h for the layer definition and
 * its source passages; each function below names the passage it follows.
 *
 * Parallel loops (OpenMP) only split independent outputs; every output is
 * summed sequentially in the order written, so results do not depend on the
 * thread count.
 */
#include "msk_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int32_t orc_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads((int)n);
#else
  (void)n;
#endif
}

/* bf16, the storage format of the dense (non-expert) layers and of the KV
 * cache (newruntime.com, What happened): value = the fp32 whose high half is b. */
double orc_bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Store to bf16: round the real value to nearest, ties to even (the pages do
 * not state the rounding; nearest-even is the IEEE default). */
uint16_t orc_bf16_rne(double x) {
  uint16_t sign;
  double a, f, r;
  int e, E;
  if (isnan(x)) return 0x7FC0;
  sign = signbit(x) ? 0x8000 : 0;
  a = fabs(x);
  if (a == 0.0) return sign;
  f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  E = e - 1;        /* a = (2f) * 2^E */
  if (E < -126) {   /* subnormal bf16: lattice 2^-133 */
    r = nearbyint(ldexp(a, 133));
    return (uint16_t)(sign | (uint16_t)r); /* r == 128 encodes the smallest normal */
  }
  r = nearbyint(ldexp(f, 8)); /* 8 significant bits, in [128, 256] */
  if (r == 256.0) {
    r = 128.0;
    E += 1;
  }
  if (E > 127) return (uint16_t)(sign | 0x7F80);
  return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)((int)r - 128));
}

/* E2M1 element of NVFP4, the 4-bit format of the expert weights
 * (newruntime.com, What happened; OCP MX v1.0 for the element encoding):
 * sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * e > 0: 2^(e-1) * (1 + m/2); e = 0: m/2. */
double orc_e2m1_value(uint8_t nibble) {
  int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
  double v = e ? ldexp(1.0 + m / 2.0, e - 1) : m / 2.0;
  return s ? -v : v;
}

/* E4M3 block scale of NVFP4 (OCP FN encoding, bias 7, no infinities, the
 * all-ones mantissa at the top exponent is NaN). */
double orc_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  return s ? -v : v;
}

/* NVFP4 matrix [rows][cols]: element (r, c) is the nibble c%2 (low nibble
 * first) of byte r*cols/2 + c/2, times the E4M3 scale of its 16-element block
 * along the row, times the per-tensor fp32 scale. The product of the first two
 * is exact; in fp64 so is the third. */
uint8_t orc_e4m3_rne_sat(float x) {
  double v = x, q, r;
  int e;
  if (!(v > 0.0)) return 0;          /* 0 (and the sign-less activation scales) */
  if (v >= 448.0) return 0x7E;       /* saturate: 448 = 1.75 * 2^8 */
  if (v < ldexp(1.0, -6)) {          /* subnormal steps of 2^-9 */
    r = rint(v / ldexp(1.0, -9));
    return (uint8_t)r;               /* r = 8 is the smallest normal, code 0x08 */
  }
  frexp(v, &e);                      /* v = f * 2^e, f in [0.5, 1): exponent e - 1 */
  q = v / ldexp(1.0, e - 1 - 3);     /* [8, 16) */
  r = rint(q);
  if (r == 16.0) {
    r = 8.0;
    e += 1;
  }
  {
    int code = ((e - 1 + 7) << 3) | ((int)r - 8);
    return (uint8_t)(code > 0x7E ? 0x7E : code);
  }
}

uint8_t orc_e2m1_rne_sat(float y) {
  const uint8_t s = signbit(y) ? 8 : 0;
  const double a = fabs((double)y);
  uint8_t c;
  /* representable 0, .5, 1, 1.5, 2, 3, 4, 6; a tie goes to the code whose
     mantissa bit is 0 */
  if (a <= 0.25) c = 0;
  else if (a < 0.75) c = 1;
  else if (a <= 1.25) c = 2;
  else if (a < 1.75) c = 3;
  else if (a <= 2.5) c = 4;
  else if (a < 3.5) c = 5;
  else if (a <= 5.0) c = 6;
  else c = 7;
  return (uint8_t)(s | c);
}

void orc_nvfp4_quant16(const float* x, uint8_t* codes, uint8_t* scale, float* deq) {
  float amax = 0.0f, s32, s;
  int i;
  for (i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  s32 = amax / 6.0f;
  *scale = orc_e4m3_rne_sat(s32);
  s = (float)orc_e4m3_value(*scale);
  for (i = 0; i < 16; ++i) {
    const float y = s > 0.0f ? x[i] / s : 0.0f;
    codes[i] = orc_e2m1_rne_sat(y);
    deq[i] = (float)(orc_e2m1_value(codes[i]) * (double)s);
  }
}

void orc_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, double s_tensor,
                       int64_t rows, int64_t cols, double* out) {
  int64_t r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; ++r) {
    int64_t c;
    for (c = 0; c < cols; ++c) {
      uint8_t byte = codes[r * (cols / 2) + c / 2];
      uint8_t nib = (uint8_t)((c & 1) ? (byte >> 4) : (byte & 15));
      double sb = orc_e4m3_value(scales[r * (cols / 16) + c / 16]);
      out[r * cols + c] = orc_e2m1_value(nib) * sb * s_tensor;
    }
  }
}

/* The router's fp32 dot product in one fixed order (this build's reading;
 * the pages fix none): partial j is the fma chain over the 8 elements
 * k = 8j .. 8j+7 in ascending order, starting from +0; the n/8 partials,
 * padded with +0 to a power of two, are then added pairwise, adjacent pairs
 * first (level by level). The order makes the fp32 top-k decision
 * reproducible on both sides. n must be a multiple of 8. */
float orc_dot_canon_f32(const float* x, const float* w, int32_t n) {
  int32_t np = n / 8, P = 1, j, i, len;
  float* part;
  float r;
  while (P < np) P *= 2;
  part = (float*)calloc((size_t)P, sizeof(float));
  for (j = 0; j < np; ++j) {
    float acc = 0.0f;
    for (i = 0; i < 8; ++i) acc = fmaf(x[8 * j + i], w[8 * j + i], acc);
    part[j] = acc;
  }
  for (len = P; len > 1; len /= 2)
    for (j = 0; j < len / 2; ++j) part[j] = part[2 * j] + part[2 * j + 1];
  r = part[0];
  free(part);
  return r;
}

/* Top-k of the router (8 of 256 experts per token; newruntime.com, What
 * happened): the k largest logits, by value descending, ties to the lower
 * index (the tie rule is this build's reading). */
void orc_topk(const float* logits, int32_t n, int32_t k, int32_t* ids) {
  unsigned char* taken = (unsigned char*)calloc((size_t)n, 1);
  int32_t r, e;
  for (r = 0; r < k; ++r) {
    int32_t best = -1;
    for (e = 0; e < n; ++e) {
      if (taken[e]) continue;
      if (best < 0 || logits[e] > logits[best]) best = e;
    }
    ids[r] = best;
    if (best >= 0) taken[best] = 1;
  }
  free(taken);
}

/* Speculative prefetch list of one layer (LMSYS post as summarised on
 * newruntime.com, What happened: the experts the previous step used most are
 * prefetched): count how often each expert appears in the previous step's
 * selections ids[n_ids], then take the p experts with the largest counts,
 * ties to the lower index. Experts with count 0 rank by index after the used
 * ones. The count/tie rule is this build's reading. */
void orc_prefetch_list(const int32_t* ids, int32_t n_ids, int32_t n_experts, int32_t p, int32_t* list) {
  int32_t* count = (int32_t*)calloc((size_t)n_experts, sizeof(int32_t));
  unsigned char* taken = (unsigned char*)calloc((size_t)n_experts, 1);
  int32_t i, r, e;
  for (i = 0; i < n_ids; ++i) count[ids[i]] += 1;
  for (r = 0; r < p; ++r) {
    int32_t best = -1;
    for (e = 0; e < n_experts; ++e) {
      if (taken[e]) continue;
      if (best < 0 || count[e] > count[best]) best = e;
    }
    list[r] = best;
    if (best >= 0) taken[best] = 1;
  }
  free(taken);
  free(count);
}

/* Gate weights: softmax over the selected logits only. */
void orc_gates(const float* logits, const int32_t* ids, int32_t k, double* gates) {
  double m = -INFINITY, sum = 0.0;
  int32_t j;
  for (j = 0; j < k; ++j) m = fmax(m, (double)logits[ids[j]]);
  for (j = 0; j < k; ++j) {
    gates[j] = exp((double)logits[ids[j]] - m);
    sum += gates[j];
  }
  for (j = 0; j < k; ++j) gates[j] /= sum;
}

/* RMSNorm (pre-norm decoder reading): y = x / sqrt(mean(x^2) + eps) * g. */
void orc_rmsnorm(const double* x, const uint16_t* g, int32_t n, double eps, double* y) {
  double ss = 0.0, inv;
  int32_t i;
  for (i = 0; i < n; ++i) ss += x[i] * x[i];
  inv = 1.0 / sqrt(ss / n + eps);
  for (i = 0; i < n; ++i) y[i] = x[i] * inv * orc_bf16_value(g[i]);
}

double orc_silu(double x) { return x / (1.0 + exp(-x)); }

/* y[i][r] = sum_k x[i][k] * W[r][k] for a bf16 W [rows][K]; x is [nt][K]. */
static void linear_bf16(const double* x, int32_t nt, const uint16_t* W, int32_t rows,
                        int32_t K, double* y) {
  int32_t r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; ++r) {
    double* wr = (double*)malloc(sizeof(double) * (size_t)K);
    int32_t i, k;
    for (k = 0; k < K; ++k) wr[k] = orc_bf16_value(W[(int64_t)r * K + k]);
    for (i = 0; i < nt; ++i) {
      double s = 0.0;
      const double* xi = x + (int64_t)i * K;
      for (k = 0; k < K; ++k) s += xi[k] * wr[k];
      y[(int64_t)i * rows + r] = s;
    }
    free(wr);
  }
}

/* y[i][r] = sum_k x[i][k] * W[r][k] for an fp64 W [rows][K]. */
static void linear_f64(const double* x, int32_t nt, const double* W, int32_t rows,
                       int32_t K, double* y) {
  int32_t r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; ++r) {
    int32_t i, k;
    const double* wr = W + (int64_t)r * K;
    for (i = 0; i < nt; ++i) {
      double s = 0.0;
      const double* xi = x + (int64_t)i * K;
      for (k = 0; k < K; ++k) s += xi[k] * wr[k];
      y[(int64_t)i * rows + r] = s;
    }
  }
}

/*
 * Attention of one request's T verify tokens. Of the 62 layers, 46 attend
 * over a sliding window of the 2,048 most recent tokens and 16 over the whole
 * context (newruntime.com, What happened; orcarouter.ai, model paragraph).
 * Token t sits at position ctx + t; query head h reads kv head h / (nq/nkv);
 * it sees keys j with j <= ctx + t (causal among the verify tokens) and, for a
 * window W > 0, j > ctx + t - W (W keys including itself). Scores are
 * q.k / sqrt(d); softmax; weighted sum of V rows. Caches: [nkv][cap][d] bf16.
 */
static uint32_t tree_anc(const uint16_t* tree, int32_t t) {
  return tree ? (uint32_t)tree[t] : ((2u << t) - 1u);
}

static int32_t popcount16(uint32_t v) {
  int32_t n = 0;
  for (; v; v &= v - 1u) ++n;
  return n;
}

int32_t orc_tree_valid(const uint16_t* tree, int32_t T) {
  int32_t t, u;
  if (T < 1 || T > 16) return 0;
  if (!tree) return 1;
  for (t = 0; t < T; ++t) {
    uint32_t a = tree[t];
    if (!(a >> t & 1u) || (a >> (t + 1)) != 0u) return 0;
    for (u = 0; u < t; ++u)
      if ((a >> u & 1u) && (tree[u] & ~a) != 0u) return 0;
  }
  return 1;
}

/* Attention of token t over its visible keys (orcarouter.ai, section "Dove si
 * colloca il confine del kernel": sliding-window or global attention over the
 * KV cache; the tree of verified tokens as in orc_tree_valid). Token t stands
 * at position ctx + depth(t) on its own path. Visible keys, in ascending
 * cache order: prior rows j < ctx with j > pos - window (all of them when
 * window == 0), then new token u's row ctx + u for each ancestor u whose
 * path position ctx + depth(u) is also inside the window. With no tree this
 * is the causal chain: rows max(0, ctx + t - window + 1) .. ctx + t. */
void orc_attention(const double* q, const uint16_t* k_cache, const uint16_t* v_cache,
                   int32_t nq, int32_t nkv, int32_t d, int32_t cap, int32_t T, int32_t ctx,
                   int32_t window, const uint16_t* tree, double* out) {
  int32_t group = nq / nkv;
  double scale = 1.0 / sqrt((double)d);
  int32_t th;
#pragma omp parallel for schedule(dynamic)
  for (th = 0; th < T * nq; ++th) {
    int32_t t = th / nq, h = th % nq, g = h / group;
    uint32_t anc = tree_anc(tree, t);
    int32_t pos = ctx + popcount16(anc) - 1;
    int32_t lo = window > 0 ? (pos - window + 1 > 0 ? pos - window + 1 : 0) : 0;
    int32_t n = 0, j, c, u;
    const double* qv = q + (int64_t)t * nq * d + (int64_t)h * d;
    const uint16_t* kb = k_cache + (int64_t)g * cap * d;
    const uint16_t* vb = v_cache + (int64_t)g * cap * d;
    int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(ctx + T));
    double* s;
    double m = -INFINITY, l = 0.0;
    double* o = out + (int64_t)t * nq * d + (int64_t)h * d;
    for (j = lo; j < ctx; ++j) rows[n++] = j;
    for (u = 0; u < T; ++u)
      if ((anc >> u & 1u) && ctx + popcount16(tree_anc(tree, u)) - 1 >= lo) rows[n++] = ctx + u;
    s = (double*)malloc(sizeof(double) * (size_t)n);
    for (j = 0; j < n; ++j) {
      double dot = 0.0;
      for (c = 0; c < d; ++c) dot += qv[c] * orc_bf16_value(kb[(int64_t)rows[j] * d + c]);
      s[j] = dot * scale;
      m = fmax(m, s[j]);
    }
    for (j = 0; j < n; ++j) {
      s[j] = exp(s[j] - m);
      l += s[j];
    }
    for (c = 0; c < d; ++c) {
      double acc = 0.0;
      for (j = 0; j < n; ++j) acc += s[j] * orc_bf16_value(vb[(int64_t)rows[j] * d + c]);
      o[c] = acc / l;
    }
    free(s);
    free(rows);
  }
}

/*
 * One verify pass of one decoder layer for R requests of T tokens each.
 * Steps, in order:
 *  1. n1 = RMSNorm(h) (gain g_attn); qkv = n1 Wqkv^T, rows Q | K | V.
 *  2. KV write: K and V of token t stored as bf16 at position ctx[r] + t of
 *     the request's cache (a launch ends with the next layer's QKV
 *     projection and KV write: newruntime.com, What happened); no other
 *     cache row changes.
 *  3. Attention over the cache, including the rows just written.
 *  4. h1 = h + attn Wo^T.
 *  5. n2 = RMSNorm(h1) (gain g_moe).
 *  6. Router: fp32 logits = dot_canon(fl32(n2), Wr[e]) + b[e]; top-k; gates =
 *     softmax over the selected logits.
 *  7. Pooler, which narrows the token vector ahead of the experts
 *     (orcarouter.ai, model paragraph): p = n2 Wpool^T.
 *  8. Experts, SwiGLU on NVFP4 weights: gu = Wgu_e p (rows gate | up),
 *     a = silu(gate) * up, y = Wd_e a; acc = sum over the token's selected
 *     experts, in selection order, of gate weight * y.
 *  9. Unpooler, which widens it back (same paragraph): h2 = h1 + acc Wup^T.
 * Caches are [R][nkv][cap][d] bf16. Returns 0, or -1 on bad arguments.
 */
int32_t orc_layer_forward(const orc_layer* L, int32_t R, int32_t T, const int32_t* ctx,
                          const uint16_t* tree, const double* h_in, uint16_t* k_cache,
                          uint16_t* v_cache, double* h_out, orc_stages* st) {
  const int32_t H = L->hidden, nq = L->n_q_heads, nkv = L->n_kv_heads, d = L->head_dim;
  const int32_t E = L->n_experts, K = L->top_k, P = L->pool_dim, I = L->expert_inter;
  const int32_t Dq = nq * d, Dkv = nkv * d, Nqkv = Dq + 2 * Dkv, NT = R * T;
  const int32_t cap = L->kv_capacity;
  double *n1, *qkv, *q, *attn, *h1, *n2, *p, *acc, *tmp, *yk;
  float *n2f, *logits;
  int32_t *ids, *used;
  double* gates;
  int32_t i, r, t, e, j;

  if (!L || R <= 0 || T <= 0 || nq % nkv != 0 || P % 16 != 0 || I % 16 != 0 || K > E) return -1;
  for (r = 0; r < R; ++r) {
    if (ctx[r] < 0 || ctx[r] + T > cap) return -1;
    if (!orc_tree_valid(tree ? tree + (int64_t)r * T : NULL, T)) return -1;
  }

  n1 = (double*)malloc(sizeof(double) * (size_t)NT * H);
  qkv = (double*)malloc(sizeof(double) * (size_t)NT * Nqkv);
  q = (double*)malloc(sizeof(double) * (size_t)NT * Dq);
  attn = (double*)malloc(sizeof(double) * (size_t)NT * Dq);
  h1 = (double*)malloc(sizeof(double) * (size_t)NT * H);
  n2 = (double*)malloc(sizeof(double) * (size_t)NT * H);
  n2f = (float*)malloc(sizeof(float) * (size_t)NT * H);
  logits = (float*)malloc(sizeof(float) * (size_t)NT * E);
  ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)NT * K);
  gates = (double*)malloc(sizeof(double) * (size_t)NT * K);
  p = (double*)malloc(sizeof(double) * (size_t)NT * P);
  acc = (double*)calloc((size_t)NT * P, sizeof(double));
  tmp = (double*)malloc(sizeof(double) * (size_t)NT * H);
  yk = (double*)calloc((size_t)NT * K * P, sizeof(double));
  used = (int32_t*)calloc((size_t)E, sizeof(int32_t));

  /* 1. pre-attention norm and QKV projection */
  for (i = 0; i < NT; ++i) {
    if (L->use_norm) orc_rmsnorm(h_in + (int64_t)i * H, L->g_attn, H, L->rms_eps, n1 + (int64_t)i * H);
    else memcpy(n1 + (int64_t)i * H, h_in + (int64_t)i * H, sizeof(double) * (size_t)H);
  }
  linear_bf16(n1, NT, L->w_qkv, Nqkv, H, qkv);
  for (i = 0; i < NT; ++i) {
    memcpy(q + (int64_t)i * Dq, qkv + (int64_t)i * Nqkv, sizeof(double) * (size_t)Dq);
    if (st && st->k_new) memcpy(st->k_new + (int64_t)i * Dkv, qkv + (int64_t)i * Nqkv + Dq, sizeof(double) * (size_t)Dkv);
    if (st && st->v_new) memcpy(st->v_new + (int64_t)i * Dkv, qkv + (int64_t)i * Nqkv + Dq + Dkv, sizeof(double) * (size_t)Dkv);
  }
  if (st && st->q) memcpy(st->q, q, sizeof(double) * (size_t)NT * Dq);

  /* 2. KV write at positions ctx[r] .. ctx[r] + T - 1 */
  for (r = 0; r < R; ++r) {
    for (t = 0; t < T; ++t) {
      const double* row = qkv + (int64_t)(r * T + t) * Nqkv;
      int32_t g, c;
      for (g = 0; g < nkv; ++g) {
        int64_t dst = (((int64_t)r * nkv + g) * cap + ctx[r] + t) * d;
        for (c = 0; c < d; ++c) {
          k_cache[dst + c] = orc_bf16_rne(row[Dq + g * d + c]);
          v_cache[dst + c] = orc_bf16_rne(row[Dq + Dkv + g * d + c]);
        }
      }
    }
  }

  /* 3. attention, per request */
  for (r = 0; r < R; ++r) {
    int64_t off = (int64_t)r * nkv * cap * d;
    orc_attention(q + (int64_t)r * T * Dq, k_cache + off, v_cache + off, nq, nkv, d, cap, T,
                  ctx[r], L->window, tree ? tree + (int64_t)r * T : NULL, attn + (int64_t)r * T * Dq);
  }
  if (st && st->attn) memcpy(st->attn, attn, sizeof(double) * (size_t)NT * Dq);

  /* 4. output projection and residual */
  linear_bf16(attn, NT, L->w_o, H, Dq, tmp);
  for (i = 0; i < NT * H; ++i) h1[i] = h_in[i] + tmp[i];
  if (st && st->h1) memcpy(st->h1, h1, sizeof(double) * (size_t)NT * H);

  /* 5. pre-MoE norm */
  for (i = 0; i < NT; ++i) {
    if (L->use_norm) orc_rmsnorm(h1 + (int64_t)i * H, L->g_moe, H, L->rms_eps, n2 + (int64_t)i * H);
    else memcpy(n2 + (int64_t)i * H, h1 + (int64_t)i * H, sizeof(double) * (size_t)H);
  }
  for (i = 0; i < NT * H; ++i) n2f[i] = (float)n2[i];
  if (st && st->n2_f32) memcpy(st->n2_f32, n2f, sizeof(float) * (size_t)NT * H);

  /* 6. fp32 router, top-k, gates */
#pragma omp parallel for schedule(static)
  for (i = 0; i < NT * E; ++i) {
    int32_t tok = i / E, ex = i % E;
    float dot = orc_dot_canon_f32(n2f + (int64_t)tok * H, L->w_router + (int64_t)ex * H, H);
    float b = L->b_router ? L->b_router[ex] : 0.0f;
    logits[i] = dot + b;
  }
  for (i = 0; i < NT; ++i) {
    orc_topk(logits + (int64_t)i * E, E, K, ids + (int64_t)i * K);
    orc_gates(logits + (int64_t)i * E, ids + (int64_t)i * K, K, gates + (int64_t)i * K);
    for (j = 0; j < K; ++j) used[ids[i * K + j]] = 1;
  }
  if (st && st->logits) memcpy(st->logits, logits, sizeof(float) * (size_t)NT * E);
  if (st && st->ids) memcpy(st->ids, ids, sizeof(int32_t) * (size_t)NT * K);
  if (st && st->gates) memcpy(st->gates, gates, sizeof(double) * (size_t)NT * K);

  /* 7. pooler */
  linear_bf16(n2, NT, L->w_pool, P, H, p);
  if (st && st->p) memcpy(st->p, p, sizeof(double) * (size_t)NT * P);

  /* 8. experts: one dequantized expert at a time, applied to its tokens */
  {
    double* wgu = (double*)malloc(sizeof(double) * (size_t)2 * I * P);
    double* wd = (double*)malloc(sizeof(double) * (size_t)P * I);
    const int64_t gu_bytes = (int64_t)2 * I * P / 2, gu_sc = (int64_t)2 * I * P / 16;
    const int64_t dn_bytes = (int64_t)P * I / 2, dn_sc = (int64_t)P * I / 16;
    for (e = 0; e < E; ++e) {
      int32_t sel;
      if (!used[e]) continue;
      orc_nvfp4_dequant(L->e_gate_up + e * gu_bytes, L->e_gate_up_scale + e * gu_sc,
                        (double)L->e_tensor_scale[2 * e], 2 * I, P, wgu);
      orc_nvfp4_dequant(L->e_down + e * dn_bytes, L->e_down_scale + e * dn_sc,
                        (double)L->e_tensor_scale[2 * e + 1], P, I, wd);
#pragma omp parallel for schedule(dynamic)
      for (sel = 0; sel < NT * K; ++sel) {
        int32_t tok = sel / K;
        double *gu, *a;
        int32_t n, c;
        if (ids[sel] != e) continue;
        gu = (double*)malloc(sizeof(double) * (size_t)2 * I);
        a = (double*)malloc(sizeof(double) * (size_t)I);
        for (n = 0; n < 2 * I; ++n) {
          double s = 0.0;
          for (c = 0; c < P; ++c) s += wgu[(int64_t)n * P + c] * p[(int64_t)tok * P + c];
          gu[n] = s;
        }
        for (n = 0; n < I; ++n) a[n] = orc_silu(gu[n]) * gu[I + n];
        if (L->act_fp4) {
          /* NVFP4 activations: blocks of 16 along I, each value first
             rounded to fp32 (see orc_nvfp4_quant16) */
          int32_t b0;
          for (b0 = 0; b0 < I; b0 += 16) {
            float xb[16], dq[16];
            uint8_t cq[16], sq;
            for (n = 0; n < 16; ++n) xb[n] = (float)a[b0 + n];
            orc_nvfp4_quant16(xb, cq, &sq, dq);
            for (n = 0; n < 16; ++n) a[b0 + n] = dq[n];
          }
        }
        for (n = 0; n < P; ++n) {
          double s = 0.0;
          for (c = 0; c < I; ++c) s += wd[(int64_t)n * I + c] * a[c];
          yk[(int64_t)sel * P + n] = s;
        }
        free(gu);
        free(a);
      }
    }
    free(wgu);
    free(wd);
    for (i = 0; i < NT; ++i)
      for (j = 0; j < K; ++j) {
        int32_t n;
        for (n = 0; n < P; ++n)
          acc[(int64_t)i * P + n] += gates[i * K + j] * yk[((int64_t)i * K + j) * P + n];
      }
  }
  if (st && st->acc) memcpy(st->acc, acc, sizeof(double) * (size_t)NT * P);

  /* 9. unpooler and residual */
  linear_bf16(acc, NT, L->w_unpool, H, P, tmp);
  for (i = 0; i < NT * H; ++i) h_out[i] = h1[i] + tmp[i];

  free(n1); free(qkv); free(q); free(attn); free(h1); free(n2); free(n2f); free(logits);
  free(ids); free(gates); free(p); free(acc); free(tmp); free(yk); free(used);
  return 0;
}

/* Dense SwiGLU feed-forward on fp64 weights: y = Wd (silu(Wg x) * (Wu x)),
 * with Wgu = [Wg | Wu] stacked as rows [2I][P]. A mixture whose experts are
 * all this network must reduce to it, since the gates sum to one. */
void orc_dense_swiglu(const double* x, int32_t nt, const double* wgu, const double* wd,
                      int32_t P, int32_t I, double* y) {
  double* gu = (double*)malloc(sizeof(double) * (size_t)nt * 2 * I);
  double* a = (double*)malloc(sizeof(double) * (size_t)nt * I);
  int32_t i, n;
  linear_f64(x, nt, wgu, 2 * I, P, gu);
  for (i = 0; i < nt; ++i)
    for (n = 0; n < I; ++n)
      a[(int64_t)i * I + n] = orc_silu(gu[(int64_t)i * 2 * I + n]) * gu[(int64_t)i * 2 * I + I + n];
  linear_f64(a, nt, wd, P, I, y);
  free(gu);
  free(a);
}
