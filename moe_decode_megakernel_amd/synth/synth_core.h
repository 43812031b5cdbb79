/*
 * Seeded synthetic inputs for the speculative-verify MoE layer.
 *
 * This header is the single definition of the input generator. It is
 * compiled twice: as plain C for the host filler (synth.c), and as HIP device
 * code for the device filler (synth_gpu.hip), so that both produce the same
 * bytes for the same (seed, stream, index). It holds no step of the layer's
 * arithmetic: it only defines random input bytes (weights, caches,
 * activations, router bias). The decoding of those bytes (bf16, E2M1, E4M3)
 * is implemented separately by the oracle and by the HIP path.
 *
 * Definitions:
 *  - mix(x): the SplitMix64 output function (Steele, Lea, Flood, "Fast
 *    splittable pseudorandom number generators", OOPSLA 2014): add the golden
 *    gamma 0x9E3779B97F4A7C15, then two xor-shift-multiply rounds and a final
 *    xor-shift.
 *  - stream base: mix(mix(seed) ^ stream); element i draws mix(base + i).
 *  - normal(i): Irwin-Hall sum of the four 16-bit fields of the draw,
 *    centred (sum - 131070) and scaled by one fp32 constant
 *    c = fl32(std * sqrt(3) / 65536), i.e. unit variance up to the lattice
 *    step, support bounded by +-3.46 std. One fp32 rounding, so it is
 *    reproducible on any IEEE-754 device.
 *  - bf16: round-to-nearest-even of the fp32 sample.
 *  - NVFP4 block of 16 consecutive elements of a row: amax over the block,
 *    block scale = E4M3 (OCP, bias 7) round-to-nearest-even of
 *    amax / (6 * s_tensor), then each element is E2M1 round-to-nearest-even
 *    (ties to the even code) of w / (scale * s_tensor), saturating at 6.
 */
#ifndef MSK_SYNTH_CORE_H
#define MSK_SYNTH_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define MSK_SYN_FN static inline __host__ __device__
#else
#define MSK_SYN_FN static inline
#endif

MSK_SYN_FN uint64_t msk_syn_mix(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

MSK_SYN_FN uint64_t msk_syn_base(uint64_t seed, uint64_t stream) {
  return msk_syn_mix(msk_syn_mix(seed) ^ stream);
}

/* Integer part of the Irwin-Hall draw: sum of four 16-bit fields, centred. */
MSK_SYN_FN int32_t msk_syn_ih4(uint64_t base, uint64_t idx) {
  uint64_t h = msk_syn_mix(base + idx);
  int32_t s = (int32_t)(h & 0xFFFFu) + (int32_t)((h >> 16) & 0xFFFFu) +
              (int32_t)((h >> 32) & 0xFFFFu) + (int32_t)((h >> 48) & 0xFFFFu);
  return s - 131070;
}

MSK_SYN_FN float msk_syn_normal(uint64_t base, uint64_t idx, float c) {
  return (float)msk_syn_ih4(base, idx) * c;
}

MSK_SYN_FN uint32_t msk_syn_f32_bits(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  return v.u;
}

MSK_SYN_FN float msk_syn_bits_f32(uint32_t u) {
  union { float f; uint32_t u; } v;
  v.u = u;
  return v.f;
}

/* fp32 -> bf16, round to nearest even (inputs here are finite). */
MSK_SYN_FN uint16_t msk_syn_bf16(float f) {
  uint32_t u = msk_syn_f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Exact value of an E4M3 (OCP, bias 7) code; NaN codes are never produced. */
MSK_SYN_FN float msk_syn_e4m3_value(uint8_t code) {
  int e = (code >> 3) & 0xF, m = code & 7;
  float v;
  if (e == 0) {
    v = (float)m * (1.0f / 512.0f); /* m * 2^-9 */
  } else {
    float p = 1.0f;
    int k;
    if (e >= 7) { for (k = 7; k < e; ++k) p *= 2.0f; }
    else { for (k = e; k < 7; ++k) p *= 0.5f; }
    v = (1.0f + (float)m * 0.125f) * p;
  }
  return (code & 0x80) ? -v : v;
}

/* Round to nearest integer, ties to even, for 0 <= x < 2^22. */
MSK_SYN_FN float msk_syn_rne_int(float x) {
  float r = (x + 8388608.0f) - 8388608.0f; /* 2^23 trick, exact in RNE mode */
  return r;
}

/* Positive finite t -> E4M3 code, round to nearest even, saturating at 448. */
MSK_SYN_FN uint8_t msk_syn_e4m3_encode(float t) {
  if (!(t > 0.0f)) return 0;
  if (t >= 448.0f) return 0x7E;
  if (t < 0.015625f) { /* below 2^-6: subnormal lattice m * 2^-9 */
    float m = msk_syn_rne_int(t * 512.0f);
    return (uint8_t)(int)m; /* m == 8 is the smallest normal code 0x08 */
  }
  /* find E with 2^E <= t < 2^(E+1), E in [-6, 8] */
  int E = -6;
  float p = 0.015625f;
  while (E < 8 && t >= p * 2.0f) { p *= 2.0f; ++E; }
  float mant = msk_syn_rne_int((t / p - 1.0f) * 8.0f); /* t/p exact-ish: p is 2^E */
  int m = (int)mant;
  if (m == 8) { m = 0; ++E; }
  if (E > 8 || (E == 8 && m > 6)) return 0x7E;
  return (uint8_t)(((E + 7) << 3) | m);
}

/* E2M1 round-to-nearest-even of y, saturating; sign in bit 3. */
MSK_SYN_FN uint8_t msk_syn_e2m1_encode(float y) {
  float a = y < 0.0f ? -y : y;
  uint8_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return (uint8_t)(c | (y < 0.0f ? 8u : 0u));
}

/*
 * One NVFP4 block: 16 consecutive elements of a row. Writes 8 bytes of codes
 * (element 2j in the low nibble of byte j) and returns the E4M3 scale code.
 * base/idx0 address the 16 underlying normal draws idx0 .. idx0+15.
 */
MSK_SYN_FN uint8_t msk_syn_nvfp4_block(uint64_t base, uint64_t idx0, float c,
                                       float s_tensor, uint8_t* codes8) {
  float w[16];
  float amax = 0.0f;
  int i;
  for (i = 0; i < 16; ++i) {
    w[i] = msk_syn_normal(base, idx0 + (uint64_t)i, c);
    float a = w[i] < 0.0f ? -w[i] : w[i];
    amax = a > amax ? a : amax;
  }
  float six_st = 6.0f * s_tensor;
  uint8_t sc = msk_syn_e4m3_encode(amax / six_st);
  float denom = msk_syn_e4m3_value(sc) * s_tensor;
  for (i = 0; i < 8; ++i) {
    uint8_t lo = denom > 0.0f ? msk_syn_e2m1_encode(w[2 * i] / denom) : 0;
    uint8_t hi = denom > 0.0f ? msk_syn_e2m1_encode(w[2 * i + 1] / denom) : 0;
    codes8[i] = (uint8_t)(lo | (hi << 4));
  }
  return sc;
}

/* Stream identifiers: (layer, tensor) packed so every tensor has its own stream. */
enum msk_syn_tensor {
  MSK_SYN_W_QKV = 1,
  MSK_SYN_W_O = 2,
  MSK_SYN_W_ROUTER = 3,
  MSK_SYN_W_POOL = 4,
  MSK_SYN_W_UNPOOL = 5,
  MSK_SYN_E_GATE_UP = 6,
  MSK_SYN_E_DOWN = 7,
  MSK_SYN_K_CACHE = 8,
  MSK_SYN_V_CACHE = 9,
  MSK_SYN_H_IN = 10,
  MSK_SYN_ROUTER_PERM = 11,
  MSK_SYN_H_NOISE = 12
};

MSK_SYN_FN uint64_t msk_syn_stream_id(uint64_t layer, uint64_t tensor, uint64_t sub) {
  return (layer << 40) ^ (tensor << 32) ^ sub;
}

#endif /* MSK_SYNTH_CORE_H */
