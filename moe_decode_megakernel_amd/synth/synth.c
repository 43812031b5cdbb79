/*
 * Host filler for the seeded synthetic inputs (definitions in synth_core.h).
 * Every output element is a pure function of (seed, stream, index), so the
 * loops may run in any order or in parallel without changing a byte.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "synth_core.h"

/* fp32 scale constant of the Irwin-Hall draw for a given standard deviation. */
float msk_synth_normal_const(float std) {
  return (float)((double)std * sqrt(3.0) / 65536.0);
}

uint64_t msk_synth_base(uint64_t seed, uint64_t stream) {
  return msk_syn_base(seed, stream);
}

void msk_synth_fill_f32(float* out, int64_t n, uint64_t seed, uint64_t stream,
                        float std, int64_t idx0) {
  uint64_t base = msk_syn_base(seed, stream);
  float c = msk_synth_normal_const(std);
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = msk_syn_normal(base, (uint64_t)(idx0 + i), c);
}

void msk_synth_fill_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream,
                         float std, int64_t idx0) {
  uint64_t base = msk_syn_base(seed, stream);
  float c = msk_synth_normal_const(std);
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i)
    out[i] = msk_syn_bf16(msk_syn_normal(base, (uint64_t)(idx0 + i), c));
}

/*
 * NVFP4 matrix [rows][cols] (cols % 16 == 0): codes [rows][cols/2] with
 * element 2j of a row in the low nibble of byte j, scales [rows][cols/16].
 */
void msk_synth_fill_nvfp4(uint8_t* codes, uint8_t* scales, int64_t rows, int64_t cols,
                          uint64_t seed, uint64_t stream, float std, float s_tensor) {
  uint64_t base = msk_syn_base(seed, stream);
  float c = msk_synth_normal_const(std);
  int64_t nblk = rows * (cols / 16);
  int64_t b;
#pragma omp parallel for schedule(static)
  for (b = 0; b < nblk; ++b) {
    scales[b] = msk_syn_nvfp4_block(base, (uint64_t)b * 16u, c, s_tensor, codes + b * 8);
  }
}

/*
 * Additive router bias with a Zipf-shaped preference: a seeded permutation
 * assigns each expert a rank r in 1..n; bias = -s * ln(r). With router logits
 * whose spread is close to a standard Gumbel's, this makes the top choice
 * follow roughly a Zipf(s) law over the ranks.
 */
void msk_synth_zipf_bias(float* out, int32_t n, uint64_t seed, uint64_t stream, float s) {
  uint64_t base = msk_syn_base(seed, stream);
  int32_t perm[4096];
  int32_t i;
  if (n > 4096) return;
  for (i = 0; i < n; ++i) perm[i] = i;
  for (i = n - 1; i > 0; --i) { /* Fisher-Yates with counter-based draws */
    uint64_t h = msk_syn_mix(base + (uint64_t)i);
    int32_t j = (int32_t)(h % (uint64_t)(i + 1));
    int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  for (i = 0; i < n; ++i) out[perm[i]] = (float)(-(double)s * log((double)(i + 1)));
}

/* AR(1) mix used to make consecutive steps' inputs correlated: out = a*prev + b*noise. */
void msk_synth_ar1(float* out, const float* prev, int64_t n, uint64_t seed, uint64_t stream,
                   float a, float b) {
  uint64_t base = msk_syn_base(seed, stream);
  float c = msk_synth_normal_const(1.0f);
  int64_t i;
  for (i = 0; i < n; ++i) {
    float e = msk_syn_normal(base, (uint64_t)i, c);
    float x = a * prev[i];
    float y = b * e;
    out[i] = x + y;
  }
}
