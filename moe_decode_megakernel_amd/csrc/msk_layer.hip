// Resident layer kernel of the speculative-verify MoE decoder, for gfx950.
//
// One launch covers one layer boundary (LMSYS "Muse Spark Open Ultrafast",
// newruntime.com "What happened"; orcarouter.ai "Dove si colloca il confine
// del kernel"): the layer's attention over the bf16 KV cache, the output
// projection, the fp32 router and top-k, the pooler, the NVFP4 SwiGLU experts,
// the unpooler, and then the next layer's RMSNorm, QKV projection and KV
// write. The first launch of a step (and a standalone layer) starts with the
// layer's own QKV projection and KV write.
//
// Execution model: one workgroup of 8 waves per compute unit, resident for
// the whole launch. Phases are separated by a grid barrier (one counter in
// the workspace, release/acquire at agent scope, bounded spin). Weight tiles
// of the next phase are requested before waiting on the barrier, so the
// barrier latency overlaps the first weight fetch. Every contraction runs on
// fp16 MFMA (16x16x32, fp32 accumulation) with the 16 verify tokens as one
// 16-row tile: bf16 weights and cache rows convert to fp16 exactly (in fp16's
// normal range), activations are rounded to fp16 (11-bit significand), and
// expert weights decode from E2M1 x E4M3 into exact fp16, with the fp32 tensor
// scale applied to the fp32 accumulator.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msk_internal.h"

namespace msk {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr uint64_t kSpinTicks = 200000000ull;  // 2 s of the 100 MHz real-time counter
constexpr int32_t kErrTimeout = 7;

// LDS budget (bytes), shared between phases.
constexpr int kXBytes = kMaxTok * (4096 * 2 + 16);   // activation tile [16][K<=4096] fp16 + pad
constexpr int kRedBytes = 2 * kWaves * 256 * 4;      // cross-wave partial tiles, double buffered
constexpr int kSmallBytes = 1024;

struct Smem {
  uint8_t x[kXBytes];
  float red[2][kWaves][256];
  float inv_rms[kMaxTok * kMaxReq];
  int32_t flag;
};

__device__ __forceinline__ f32x4_t mfma_f16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ float h2f(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}
// Two bf16 -> two fp16. Exact for magnitudes in fp16's normal range
// [2^-14, 65504] (bf16's 8-bit significand fits fp16's 11 bits); below it
// the value is truncated to the fp16 subnormal grid (step 2^-24).
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t x) {
  const float lo = __builtin_bit_cast(float, x << 16);
  const float hi = __builtin_bit_cast(float, x & 0xFFFF0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}
__device__ __forceinline__ uint4 bf8_to_h8(uint4 v) {
  return make_uint4(bf2_to_h2(v.x), bf2_to_h2(v.y), bf2_to_h2(v.z), bf2_to_h2(v.w));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ---------------------------------------------------------------------------
// Grid barrier: every wave publishes its stores (release fence), the
// workgroup meets, one thread adds to the counter; waiting is a bounded spin
// on the counter followed by an acquire fence in every wave.
// ---------------------------------------------------------------------------
struct Barrier {
  uint32_t* ctr;
  int32_t* err;
  uint32_t target;  // counter value that completes the next barrier
  uint32_t step;    // increment of target per barrier (= grid size)
};

__device__ void bar_arrive(Barrier& b) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(b.ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns false if the launch must stop (timeout or an error raised elsewhere).
__device__ bool bar_wait(Barrier& b, Smem& sm) {
  if (threadIdx.x == 0) {
    int32_t ok = 1;
    uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (true) {
      uint32_t v = __hip_atomic_load(b.ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v >= b.target) break;
      if (__hip_atomic_load(b.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) { ok = 0; break; }
      if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
        __hip_atomic_store(b.err, kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    sm.flag = ok;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  bool ok = sm.flag != 0;
  b.target += b.step;
  __syncthreads();
  return ok;
}

// ---------------------------------------------------------------------------
// Activation tiles in LDS: X[t][k] in fp16 for the 16 token rows (rows >= NT
// zero), row stride K*2 + 16 bytes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int x_stride(int K) { return K * 2 + 16; }

__device__ __forceinline__ uint4 lds_x_read(const Smem& sm, int K, int row, int k) {
  return *reinterpret_cast<const uint4*>(sm.x + row * x_stride(K) + k * 2);
}

// inv_rms[t] = 1/sqrt(mean(h_t^2) + eps), from per-tile partial sums (ssq
// [ntiles][NT], summed in tile order) or, when ssq is NULL, from h directly
// (lane j sums k = j mod 64 ascending, then pairwise halving).
__device__ void compute_inv_rms(const Params& p, const float* h, const float* ssq, Smem& sm) {
  const int NT = p.NT, H = p.H;
  if (!p.use_norm) {
    if (threadIdx.x < kMaxTok) sm.inv_rms[threadIdx.x] = 1.0f;
    __syncthreads();
    return;
  }
  if (ssq) {
    if (threadIdx.x < NT) {
      float s = 0.0f;
      const int nt = H / 16;
      for (int i = 0; i < nt; ++i) s += ssq[i * NT + threadIdx.x];
      sm.inv_rms[threadIdx.x] = rsqrtf(s / (float)H + p.eps);
    }
  } else {
    const int lane = lane_id();
    for (int t = wave_id(); t < NT; t += kWaves) {
      float s = 0.0f;
      for (int k = lane; k < H; k += 64) {
        float v = h[(size_t)t * H + k];
        s = fmaf(v, v, s);
      }
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0) sm.inv_rms[t] = rsqrtf(s / (float)H + p.eps);
    }
  }
  __syncthreads();
}

// X = fp16(h * inv_rms * g) (or fp16(h) without the norm), rounded to nearest even.
__device__ void fill_x_norm(const Params& p, const float* h, const uint16_t* g, Smem& sm) {
  const int K = p.H, NT = p.NT, K8 = K / 8;
  for (int i = threadIdx.x; i < kMaxTok * K8; i += kThreads) {
    int t = i / K8, k = (i % K8) * 8;
    uint4 out = make_uint4(0, 0, 0, 0);
    if (t < NT) {
      const float4* hp = reinterpret_cast<const float4*>(h + (size_t)t * K + k);
      float4 a = hp[0], b = hp[1];
      float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      float inv = sm.inv_rms[t];
      if (p.use_norm) {
        uint4 gg = *reinterpret_cast<const uint4*>(g + k);
        uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float gj = bf2f((uint16_t)(gw[j >> 1] >> ((j & 1) * 16)));
          v[j] = (v[j] * inv) * gj;
        }
      }
      out.x = pack2(f2h(v[0]), f2h(v[1]));
      out.y = pack2(f2h(v[2]), f2h(v[3]));
      out.z = pack2(f2h(v[4]), f2h(v[5]));
      out.w = pack2(f2h(v[6]), f2h(v[7]));
    }
    *reinterpret_cast<uint4*>(sm.x + t * x_stride(K) + k * 2) = out;
  }
  __syncthreads();
}

// X = copy of a 16-bit activation matrix src [NT][K] (already fp16).
__device__ void fill_x_copy(const uint16_t* src, int K, int NT, Smem& sm) {
  const int K8 = K / 8;
  for (int i = threadIdx.x; i < kMaxTok * K8; i += kThreads) {
    int t = i / K8, k = (i % K8) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < NT) v = *reinterpret_cast<const uint4*>(src + (size_t)t * K + k);
    *reinterpret_cast<uint4*>(sm.x + t * x_stride(K) + k * 2) = v;
  }
  __syncthreads();
}

// X = sum over n partial slots of fp32 [n][NT][K], rounded to fp16.
__device__ void fill_x_sum(const float* parts, int n, int K, int NT, Smem& sm) {
  const int K8 = K / 8;
  for (int i = threadIdx.x; i < kMaxTok * K8; i += kThreads) {
    int t = i / K8, k = (i % K8) * 8;
    uint4 out = make_uint4(0, 0, 0, 0);
    if (t < NT) {
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int s = 0; s < n; ++s) {
        const float4* q = reinterpret_cast<const float4*>(parts + ((size_t)s * NT + t) * K + k);
        float4 a = q[0], b = q[1];
        v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
        v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
      }
      out.x = pack2(f2h(v[0]), f2h(v[1])); out.y = pack2(f2h(v[2]), f2h(v[3]));
      out.z = pack2(f2h(v[4]), f2h(v[5])); out.w = pack2(f2h(v[6]), f2h(v[7]));
    }
    *reinterpret_cast<uint4*>(sm.x + t * x_stride(K) + k * 2) = out;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Dense projection (bf16 weights): Y[t][n] = sum_k X[t][k] W[n][k] over the units of
// this workgroup. Each unit (16 rows x klen) is split over the 8 waves in
// sub-units of 128 k (sub-unit j goes to wave j % 8); lane (r, g) loads 16 B
// of row r at k = sub*128 + s*32 + g*8 (s = 0..3), converts it to fp16 and
// feeds one MFMA per load.
// The 8 per-wave 16x16 partials are summed in LDS in wave order.
// Two units are kept in flight: the next unit's loads are issued before the
// current one is reduced.
// ---------------------------------------------------------------------------
struct DenseBuf {
  uint4 b[kMaxSubPerWave][4];
};

__device__ __forceinline__ void dense_load(const uint16_t* W, int ldw, const Unit& u, DenseBuf& buf) {
  const int lane = lane_id(), r = lane & 15, g = lane >> 4, w = wave_id();
  const int nsub = u.klen / kSubK;
  const uint16_t* row = W + (size_t)(u.tile * 16 + r) * ldw + u.k0 + g * 8;
#pragma unroll
  for (int c = 0; c < kMaxSubPerWave; ++c) {
    int j = w + c * kWaves;
    if (j < nsub) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        buf.b[c][s] = *reinterpret_cast<const uint4*>(row + j * kSubK + s * 32);
    }
  }
}

__device__ __forceinline__ f32x4_t dense_compute(const Smem& sm, int K, const Unit& u, const DenseBuf& buf) {
  const int lane = lane_id(), r = lane & 15, g = lane >> 4, w = wave_id();
  const int nsub = u.klen / kSubK;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kMaxSubPerWave; ++c) {
    int j = w + c * kWaves;
    if (j < nsub) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 a = lds_x_read(sm, K, r, u.k0 + j * kSubK + s * 32 + g * 8);
        acc = mfma_f16(a, bf8_to_h8(buf.b[c][s]), acc);
      }
    }
  }
  return acc;
}

// Writes the wave's partial tile to red[buf][wave][tok*16 + row].
__device__ __forceinline__ void red_store(Smem& sm, int rb, f32x4_t acc) {
  const int lane = lane_id(), r = lane & 15, g = lane >> 4, w = wave_id();
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.red[rb][w][(4 * g + i) * 16 + r] = acc[i];
}

__device__ __forceinline__ float red_sum(const Smem& sm, int rb, int idx) {
  float v = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) v += sm.red[rb][w][idx];
  return v;
}

// Sum of squares over the 16 rows held by 16 consecutive lanes.
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 1);
  return v;
}

enum class Epi { Qkv, OProj, Pool, Unpool };

struct EpiArgs {
  const LayerW* lw;  // layer of a QKV epilogue
  const float* res;  // residual input (OProj: h, Unpool: h1)
  float* out;        // OProj: h1, Unpool: h_out, Pool: ppart, Qkv: qpart
  float* ssq;        // partial sums of squares (OProj, Unpool)
  float* dbg_k;
  float* dbg_v;
};

template <Epi E>
__device__ __forceinline__ void dense_epilogue(const Params& p, const EpiArgs& ea, const Unit& u,
                                               const Smem& sm, int rb) {
  const int tid = threadIdx.x;
  if (tid >= 256) return;
  const int tok = tid >> 4, row = tid & 15;
  const int n = u.tile * 16 + row;
  const int NT = p.NT;
  float v = red_sum(sm, rb, tid);
  if constexpr (E == Epi::Qkv) {
    const int Dq = p.nq * p.d, Dkv = p.nkv * p.d;
    if (tok < NT) {
      if (n < Dq) {
        ea.out[((size_t)u.slot * NT + tok) * Dq + n] = v;
      } else {
        int c = n - Dq;
        bool is_v = c >= Dkv;
        if (is_v) c -= Dkv;
        int g = c / p.d, cc = c % p.d;
        int r = tok / p.T, t = tok % p.T;
        size_t dst = (((size_t)r * p.nkv + g) * p.cap + p.ctx[r] + t) * p.d + cc;
        if (is_v) {
          ea.lw->v_cache[dst] = f2bf(v);
          if (ea.dbg_v) ea.dbg_v[(size_t)tok * Dkv + c] = v;
        } else {
          ea.lw->k_cache[dst] = f2bf(v);
          if (ea.dbg_k) ea.dbg_k[(size_t)tok * Dkv + c] = v;
        }
      }
    }
  } else if constexpr (E == Epi::Pool) {
    if (tok < NT) ea.out[((size_t)u.slot * NT + tok) * p.P + n] = v;
  } else {
    // OProj / Unpool: residual add, then partial sum of squares over the tile's 16 rows.
    float h = 0.0f;
    if (tok < NT) {
      h = ea.res[(size_t)tok * p.H + n] + v;
      ea.out[(size_t)tok * p.H + n] = h;
    }
    float s = sum16(h * h);
    if (row == 0 && tok < NT) ea.ssq[u.tile * NT + tok] = s;
  }
}

// Runs this workgroup's dense units; the first unit's weights may already be
// in `first` (loaded before a barrier).
template <Epi E>
__device__ void dense_phase(const Params& p, const Sched& sc, const uint16_t* W, int ldw, int K,
                            const EpiArgs& ea, Smem& sm, DenseBuf& first, bool have_first) {
  const int b0 = sc.off[blockIdx.x], b1 = sc.off[blockIdx.x + 1];
  if (b0 >= b1) return;
  DenseBuf bufA, bufB;
  bufA = first;
  if (!have_first) dense_load(W, ldw, sc.units[b0], bufA);
  int rb = 0;
  for (int i = b0; i < b1; i += 2) {
    Unit u0 = sc.units[i];
    bool has1 = i + 1 < b1;
    Unit u1 = has1 ? sc.units[i + 1] : u0;
    if (has1) dense_load(W, ldw, u1, bufB);
    f32x4_t acc = dense_compute(sm, K, u0, bufA);
    red_store(sm, rb, acc);
    __syncthreads();
    dense_epilogue<E>(p, ea, u0, sm, rb);
    rb ^= 1;
    if (!has1) break;
    if (i + 2 < b1) dense_load(W, ldw, sc.units[i + 2], bufA);
    acc = dense_compute(sm, K, u1, bufB);
    red_store(sm, rb, acc);
    __syncthreads();
    dense_epilogue<E>(p, ea, u1, sm, rb);
    rb ^= 1;
  }
  __syncthreads();
}

__device__ __forceinline__ void dense_prefetch(const Sched& sc, const uint16_t* W, int ldw, DenseBuf& buf) {
  const int b0 = sc.off[blockIdx.x], b1 = sc.off[blockIdx.x + 1];
  if (b0 < b1) dense_load(W, ldw, sc.units[b0], buf);
}

// ---------------------------------------------------------------------------
// Attention. Work items (request r, kv head g, split s) over a contiguous key
// range; one item per workgroup. Wave w handles q head g*group + w for the T
// tokens of the request. Keys stream through LDS in chunks of 64.
// S^T = K Q^T on MFMA (rows = keys, cols = tokens), online softmax in base 2,
// O^T += V^T P^T on MFMA. Partial (m, l, o) are merged in the next phase.
// ---------------------------------------------------------------------------
struct AttnItem {
  int r, g, s, nsplit, k_begin, k_end;  // keys [k_begin, k_end)
};

__device__ __forceinline__ void attn_range(const Params& p, const LayerW& lw, int r, int& lo, int& hi) {
  const int ctx = p.ctx[r];
  lo = (lw.window > 0) ? max(0, ctx - lw.window + 1) : 0;
  hi = ctx + p.T - 1;
}

__device__ __forceinline__ int attn_splits(const Params& p, int nkeys, int grid) {
  int cap_s = grid / (p.R * p.nkv);
  if (cap_s < 1) cap_s = 1;
  int s = (nkeys + 255) / 256;
  return s < 1 ? 1 : (s > cap_s ? cap_s : s);
}

// Item of a flat index; returns false if idx is past the last item.
__device__ bool attn_item(const Params& p, const LayerW& lw, int idx, int grid, AttnItem& it) {
  for (int r = 0; r < p.R; ++r) {
    int lo, hi;
    attn_range(p, lw, r, lo, hi);
    int nk = hi - lo + 1;
    int S = attn_splits(p, nk, grid);
    int n_r = S * p.nkv;
    if (idx < n_r) {
      it.r = r;
      it.g = idx / S;
      it.s = idx % S;
      it.nsplit = S;
      int cs = (nk + S - 1) / S;
      it.k_begin = lo + it.s * cs;
      it.k_end = min(hi + 1, it.k_begin + cs);
      return true;
    }
    idx -= n_r;
  }
  return false;
}

// Index of the first item of (r, g) in the flat order.
__device__ int attn_item_base(const Params& p, const LayerW& lw, int r, int g, int grid, int& S) {
  int base = 0;
  for (int rr = 0; rr < p.R; ++rr) {
    int lo, hi;
    attn_range(p, lw, rr, lo, hi);
    int s = attn_splits(p, hi - lo + 1, grid);
    if (rr == r) {
      S = s;
      return base + g * s;
    }
    base += s * p.nkv;
  }
  S = 1;
  return base;
}

// Partial record of (item, wave, token): o[d], then m, l.
__device__ __forceinline__ float* apart_at(const Params& p, int item, int w, int t) {
  return p.apart + (((size_t)item * kWaves + w) * kMaxTok + t) * (p.d + 2);
}

template <int D>
__device__ void attention_phase(const Params& p, const LayerW& lw, Smem& sm) {
  AttnItem it;
  if (!attn_item(p, lw, blockIdx.x, gridDim.x, it)) return;
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int group = p.nq / p.nkv;
  const int Dq = p.nq * p.d;
  const bool active = w < group;
  const int h = it.g * group + w;
  const int ctx = p.ctx[it.r];
  const int window = lw.window;
  constexpr int KS = D / 32;     // MFMA steps over the head dim
  constexpr int DT = D / 16;     // d tiles of the PV product
  constexpr int RS = D + 8;      // LDS row stride (elements)
  uint16_t* Ks = reinterpret_cast<uint16_t*>(sm.x);
  uint16_t* Vs = Ks + kAttnChunk * RS;

  // Q^T operand: col = token r_, 8 consecutive dims per lane group, summed over slices.
  uint4 qb[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qb[s] = make_uint4(0, 0, 0, 0);
  if (active && r_ < p.T) {
    const int tok = it.r * p.T + r_;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int sl = 0; sl < p.q_slices; ++sl) {
        const float4* q4 = reinterpret_cast<const float4*>(
            p.qpart + ((size_t)sl * p.NT + tok) * Dq + h * D + s * 32 + g_ * 8);
        float4 a = q4[0], b = q4[1];
        v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
        v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
      }
      qb[s].x = pack2(f2h(v[0]), f2h(v[1]));
      qb[s].y = pack2(f2h(v[2]), f2h(v[3]));
      qb[s].z = pack2(f2h(v[4]), f2h(v[5]));
      qb[s].w = pack2(f2h(v[6]), f2h(v[7]));
    }
  }

  const float scale_log2 = rsqrtf((float)D) * 1.4426950408889634f;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = {0.f, 0.f, 0.f, 0.f};

  const size_t cache_off = ((size_t)it.r * p.nkv + it.g) * p.cap;
  const uint16_t* kc = lw.k_cache + cache_off * D;
  const uint16_t* vc = lw.v_cache + cache_off * D;
  constexpr int CH16 = kAttnChunk * D / 8;  // 16-byte pieces per chunk per tensor
  constexpr int PER = (CH16 + kThreads - 1) / kThreads;
  const int nchunks = (it.k_end - it.k_begin + kAttnChunk - 1) / kAttnChunk;

  uint4 kreg[PER], vreg[PER];
  auto load_chunk = [&](int c) {
    int kb = it.k_begin + c * kAttnChunk;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      int i = threadIdx.x + j * kThreads;
      kreg[j] = make_uint4(0, 0, 0, 0);
      vreg[j] = make_uint4(0, 0, 0, 0);
      if (i < CH16) {
        int key = i / (D / 8), c8 = (i % (D / 8)) * 8;
        if (kb + key < it.k_end) {
          kreg[j] = *reinterpret_cast<const uint4*>(kc + (size_t)(kb + key) * D + c8);
          vreg[j] = *reinterpret_cast<const uint4*>(vc + (size_t)(kb + key) * D + c8);
        }
      }
    }
  };
  if (nchunks > 0) load_chunk(0);
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      int i = threadIdx.x + j * kThreads;
      if (i < CH16) {
        int key = i / (D / 8), c8 = (i % (D / 8)) * 8;
        *reinterpret_cast<uint4*>(Ks + key * RS + c8) = bf8_to_h8(kreg[j]);
        *reinterpret_cast<uint4*>(Vs + key * RS + c8) = bf8_to_h8(vreg[j]);
      }
    }
    if (c + 1 < nchunks) load_chunk(c + 1);
    __syncthreads();
    if (!active) continue;
    const int kb = it.k_begin + c * kAttnChunk;
    // scores for 4 key tiles of 16
    float sc[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        uint4 a = *reinterpret_cast<const uint4*>(Ks + (kt * 16 + r_) * RS + s * 32 + g_ * 8);
        s4 = mfma_f16(a, qb[s], s4);
      }
      const int pos = ctx + r_;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int key = kb + kt * 16 + 4 * g_ + i;
        bool vis = key < it.k_end && key <= pos && (window <= 0 || key > pos - window) && r_ < p.T;
        sc[kt][i] = vis ? s4[i] * scale_log2 : -INFINITY;
      }
    }
    float cmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, sc[kt][i]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
    float psum = 0.0f;
    uint16_t pb[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pv = (sc[kt][i] == -INFINITY) ? 0.0f : exp2f(sc[kt][i] - m_new);
        psum += pv;
        pb[kt][i] = f2h(pv);
      }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] *= alpha;
    // O^T += V^T P^T over two 32-key steps
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint4 bp;
      bp.x = pack2(pb[2 * u][0], pb[2 * u][1]);
      bp.y = pack2(pb[2 * u][2], pb[2 * u][3]);
      bp.z = pack2(pb[2 * u + 1][0], pb[2 * u + 1][1]);
      bp.w = pack2(pb[2 * u + 1][2], pb[2 * u + 1][3]);
      const int k0 = u * 32 + 4 * g_;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int col = dt * 16 + r_;
        uint16_t v0 = Vs[(k0 + 0) * RS + col], v1 = Vs[(k0 + 1) * RS + col];
        uint16_t v2 = Vs[(k0 + 2) * RS + col], v3 = Vs[(k0 + 3) * RS + col];
        uint16_t v4 = Vs[(k0 + 16) * RS + col], v5 = Vs[(k0 + 17) * RS + col];
        uint16_t v6 = Vs[(k0 + 18) * RS + col], v7 = Vs[(k0 + 19) * RS + col];
        uint4 av = make_uint4(pack2(v0, v1), pack2(v2, v3), pack2(v4, v5), pack2(v6, v7));
        o[dt] = mfma_f16(av, bp, o[dt]);
      }
    }
  }
  if (active && r_ < p.T) {
    float* rec = apart_at(p, blockIdx.x, w, r_);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rec[dt * 16 + 4 * g_ + i] = o[dt][i];
    if (g_ == 0) {
      rec[D] = m_run;
      rec[D + 1] = l_run;
    }
  }
}

// Merge of the split partials: one thread per (token, q head, dim).
__device__ void merge_phase(const Params& p, const LayerW& lw, bool debug) {
  const int D = p.d, Dq = p.nq * D, group = p.nq / p.nkv;
  const int total = p.NT * p.nq * D;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads) {
    const int c = i % D, h = (i / D) % p.nq, tok = i / (D * p.nq);
    const int r = tok / p.T, t = tok % p.T;
    const int g = h / group, w = h % group;
    int S;
    const int base = attn_item_base(p, lw, r, g, gridDim.x, S);
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, apart_at(p, base + s, w, t)[D]);
    float L = 0.0f, O = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float* rec = apart_at(p, base + s, w, t);
      float m = rec[D];
      float f = (m == -INFINITY) ? 0.0f : exp2f(m - M);
      L += rec[D + 1] * f;
      O += rec[c] * f;
    }
    float out = O / L;
    p.attn[(size_t)tok * Dq + h * D + c] = f2h(out);
    if (debug && p.dbg.attn) p.dbg.attn[(size_t)tok * Dq + h * D + c] = out;
  }
}

// ---------------------------------------------------------------------------
// Router: logit(t, e) = canonical fp32 dot of n2[t] and Wr[e] (lane j: fma
// chain over k = j mod 64 ascending; then pairwise halving), plus bias.
// One expert per workgroup (strided), one token per wave (strided).
// ---------------------------------------------------------------------------
__device__ void router_phase(const Params& p, const Smem& sm, bool debug) {
  const int lane = lane_id(), w = wave_id();
  const int H = p.H;
  for (int e = blockIdx.x; e < p.E; e += gridDim.x) {
    const float* wr = p.cur.w_router + (size_t)e * H;
    const float b = p.cur.b_router ? p.cur.b_router[e] : 0.0f;
    for (int t = w; t < p.NT; t += kWaves) {
      const float inv = sm.inv_rms[t];
      const float* h = p.h1 + (size_t)t * H;
      float acc = 0.0f;
      for (int k = lane; k < H; k += 64) {
        float x = h[k];
        if (p.use_norm) x = (x * inv) * bf2f(p.cur.g_moe[k]);
        acc = fmaf(x, wr[k], acc);
      }
      for (int s = 32; s >= 1; s >>= 1) acc = acc + __shfl_xor(acc, s);
      if (lane == 0) p.logits[(size_t)t * p.E + e] = acc + b;
    }
  }
  if (debug && p.dbg.n2 && blockIdx.x == 0) {
    for (int i = threadIdx.x; i < p.NT * H; i += kThreads) {
      int t = i / H, k = i % H;
      float x = p.h1[i];
      if (p.use_norm) x = (x * sm.inv_rms[t]) * bf2f(p.cur.g_moe[k]);
      p.dbg.n2[i] = x;
    }
  }
}

// ---------------------------------------------------------------------------
// Routing tables in LDS (inside the X region, after the pooled activations):
// ids/gates per token, the selected experts in ascending order, and per
// selected expert the gate weight of every token (0 if not routed).
// ---------------------------------------------------------------------------
struct Route {
  int32_t n_sel;
  int32_t sel[kMaxE];
  int32_t ids[kMaxTok][kMaxK];
  float gates[kMaxTok][kMaxK];
  float tokgate[kMaxTok * kMaxK][kMaxTok];  // [slot][token]
  uint32_t mask[kMaxE / 32];
};

constexpr int kRouteOff = kMaxTok * (2048 * 2 + 16);  // after the pooled X (P <= 2048)
static_assert(kRouteOff + (int)sizeof(Route) <= kXBytes, "route tables must fit the X region");

__device__ __forceinline__ Route& route_of(Smem& sm) { return *reinterpret_cast<Route*>(sm.x + kRouteOff); }

// Top-k by (logit descending, index ascending); gates = softmax of the selected logits.
__device__ void routing(const Params& p, Smem& sm, bool write_out) {
  Route& rt = route_of(sm);
  const int lane = lane_id(), w = wave_id();
  const int E = p.E, K = p.topk;
  if (threadIdx.x < kMaxE / 32) rt.mask[threadIdx.x] = 0;
  __syncthreads();
  for (int t = w; t < p.NT; t += kWaves) {
    const float* lg = p.logits + (size_t)t * E;
    float v[kMaxE / 64];
    int taken = 0;
#pragma unroll
    for (int j = 0; j < kMaxE / 64; ++j) {
      int e = lane + j * 64;
      v[j] = e < E ? lg[e] : -INFINITY;
      if (e >= E) taken |= 1 << j;
    }
    float sel_v[kMaxK];
    for (int r = 0; r < K; ++r) {
      // lane best: largest value, lowest index among not taken
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kMaxE / 64; ++j) {
        int e = lane + j * 64;
        if (!(taken & (1 << j)) && (v[j] > bv || (v[j] == bv && e < bi))) { bv = v[j]; bi = e; }
      }
      for (int o = 32; o >= 1; o >>= 1) {
        float ov = __shfl_xor(bv, o);
        int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if ((bi & 63) == lane) taken |= 1 << (bi >> 6);
      sel_v[r] = bv;
      if (lane == 0) rt.ids[t][r] = bi;
    }
    if (lane == 0) {
      float m = sel_v[0];
      for (int r = 1; r < K; ++r) m = fmaxf(m, sel_v[r]);
      float ex[kMaxK], s = 0.0f;
      for (int r = 0; r < K; ++r) { ex[r] = expf(sel_v[r] - m); s += ex[r]; }
      for (int r = 0; r < K; ++r) rt.gates[t][r] = ex[r] / s;
    }
  }
  __syncthreads();
  // selected set
  if (threadIdx.x < p.NT * K) {
    int t = threadIdx.x / K, r = threadIdx.x % K;
    int e = rt.ids[t][r];
    atomicOr(&rt.mask[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    for (int q = 0; q < kMaxE / 32; ++q) {
      uint32_t m = rt.mask[q];
      while (m) {
        int b = __builtin_ctz(m);
        m &= m - 1;
        rt.sel[n++] = q * 32 + b;
      }
    }
    rt.n_sel = n;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rt.n_sel * kMaxTok; i += kThreads) {
    int j = i / kMaxTok, t = i % kMaxTok;
    float gv = 0.0f;
    if (t < p.NT)
      for (int r = 0; r < K; ++r)
        if (rt.ids[t][r] == rt.sel[j]) gv = rt.gates[t][r];
    rt.tokgate[j][t] = gv;
  }
  if (write_out && threadIdx.x < p.NT * K) {
    int t = threadIdx.x / K, r = threadIdx.x % K;
    if (p.out_ids) p.out_ids[t * K + r] = rt.ids[t][r];
    if (p.out_gates) p.out_gates[t * K + r] = rt.gates[t][r];
  }
  if (write_out && p.hist && threadIdx.x == 0) {
    for (int t = 0; t < p.NT; ++t)
      for (int r = 0; r < K; ++r) p.hist[(size_t)p.layer * E + rt.ids[t][r]] += 1;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// NVFP4 decode: 16 B of codes (32 elements, element 2j in the low nibble of
// byte j) and two E4M3 block scales -> 4 MFMA B operands of 8 fp16. The
// E2M1 x E4M3 product has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in fp16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fp4_decode(uint4 codes, uint32_t sc2, uint4 out[4]) {
  const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sc2, 0);
  const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sc2, 1);
  const f16x2_t S0 = {(_Float16)s0, (_Float16)s0};
  const f16x2_t S1 = {(_Float16)s1, (_Float16)s1};
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // dword q holds elements 8q .. 8q+7
    const f16x2_t S = q < 2 ? S0 : S1;
    f16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 0) * S;
    f16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 1) * S;
    f16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 2) * S;
    f16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw[q], 1.0f, 3) * S;
    out[q] = make_uint4(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                        __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3));
  }
}

// GEMM1: gate/up projection of the selected experts with SwiGLU.
// Unit = (selected slot j, i-tile it): rows gate[it*8 .. +8) and up[I + it*8 .. +8)
// as the 16 MFMA columns; k = P split over the waves in steps of 128
// (lane group g holds the 32 elements at step*128 + g*32).
struct G1Buf {
  uint4 c[2];
  uint32_t s[2];
};

__device__ __forceinline__ void g1_load(const Params& p, const Route& rt, int u, G1Buf& b) {
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int I = p.I, P = p.P, ntile = I / 8;
  const int j = u / ntile, it = u % ntile;
  const int e = rt.sel[j];
  const int row = r_ < 8 ? it * 8 + r_ : I + it * 8 + (r_ - 8);
  const uint8_t* codes = p.cur.e_gu + (size_t)e * (2 * I) * (P / 2) + (size_t)row * (P / 2);
  const uint8_t* scs = p.cur.e_gu_sc + (size_t)e * (2 * I) * (P / 16) + (size_t)row * (P / 16);
  const int nsteps = P / 128;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    int st = w + c * kWaves;
    if (st < nsteps) {
      int k = st * 128 + g_ * 32;
      b.c[c] = *reinterpret_cast<const uint4*>(codes + k / 2);
      b.s[c] = *reinterpret_cast<const uint16_t*>(scs + k / 16);
    }
  }
}

__device__ void gemm1_phase(const Params& p, Smem& sm, bool debug) {
  Route& rt = route_of(sm);
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int I = p.I, P = p.P, ntile = I / 8;
  const int U = rt.n_sel * ntile;
  const int u0 = (int)((long long)blockIdx.x * U / gridDim.x);
  const int u1 = (int)((long long)(blockIdx.x + 1) * U / gridDim.x);
  const int nsteps = P / 128;
  G1Buf bA, bB;
  if (u0 < u1) g1_load(p, rt, u0, bA);
  int rb = 0;
  for (int u = u0; u < u1; ++u) {
    G1Buf cur = bA;
    if (u + 1 < u1) g1_load(p, rt, u + 1, bB);
    const int j = u / ntile, it = u % ntile;
    const int e = rt.sel[j];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      int st = w + c * kWaves;
      if (st < nsteps) {
        uint4 bw[4];
        fp4_decode(cur.c[c], cur.s[c], bw);
        const int kbase = st * 128 + g_ * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint4 a = lds_x_read(sm, P, r_, kbase + q * 8);
          acc = mfma_f16(a, bw[q], acc);
        }
        if (debug && p.dbg.dq_gu && e == p.dbg.dq_expert) {
          const int row = r_ < 8 ? it * 8 + r_ : I + it * 8 + (r_ - 8);
          uint4* dst = reinterpret_cast<uint4*>(p.dbg.dq_gu + (size_t)row * P + kbase);
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = bw[q];
        }
      }
    }
    red_store(sm, rb, acc);
    __syncthreads();
    if (threadIdx.x < kMaxTok * 8) {
      const int tok = threadIdx.x >> 3, c = threadIdx.x & 7;
      if (tok < p.NT) {
        const float ts = p.cur.e_ts[2 * e];
        float gate = red_sum(sm, rb, tok * 16 + c) * ts;
        float up = red_sum(sm, rb, tok * 16 + 8 + c) * ts;
        float a = gate / (1.0f + expf(-gate)) * up;
        a *= rt.tokgate[j][tok];
        p.abuf[((size_t)j * p.NT + tok) * I + it * 8 + c] = f2h(a);
      }
    }
    rb ^= 1;
    bA = bB;
  }
  __syncthreads();
}

// GEMM2: down projection, summed over a contiguous range of selected experts.
// Workgroup = (row tile of 16 of P, expert part); k = I split over the waves
// in steps of 128; per expert the fp32 tensor scale is applied to the MFMA
// partial before it is added to the running sum.
struct G2Buf {
  uint4 c;
  uint32_t s;
  uint4 a[4];
};

__device__ __forceinline__ void g2_load(const Params& p, const Route& rt, int j, int tile, G2Buf& b) {
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int I = p.I, P = p.P;
  const int e = rt.sel[j];
  const int k = w * 128 + g_ * 32;
  const int row = tile * 16 + r_;
  b.c = make_uint4(0, 0, 0, 0);
  b.s = 0;
  if (k < I) {
    b.c = *reinterpret_cast<const uint4*>(p.cur.e_dn + (size_t)e * P * (I / 2) + (size_t)row * (I / 2) + k / 2);
    b.s = *reinterpret_cast<const uint16_t*>(p.cur.e_dn_sc + (size_t)e * P * (I / 16) + (size_t)row * (I / 16) + k / 16);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) b.a[q] = make_uint4(0, 0, 0, 0);
  if (k < I && r_ < p.NT && rt.tokgate[j][r_] != 0.0f) {
    const uint4* src = reinterpret_cast<const uint4*>(p.abuf + ((size_t)j * p.NT + r_) * I + k);
#pragma unroll
    for (int q = 0; q < 4; ++q) b.a[q] = src[q];
  }
}

__device__ void gemm2_phase(const Params& p, Smem& sm, bool debug) {
  Route& rt = route_of(sm);
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int I = p.I, P = p.P;
  const int tiles = P / 16;
  const int parts = max(1, (int)gridDim.x / tiles);
  if ((int)blockIdx.x >= tiles * parts) return;
  const int tile = blockIdx.x % tiles, part = blockIdx.x / tiles;
  const int j0 = part * rt.n_sel / parts, j1 = (part + 1) * rt.n_sel / parts;
  const bool kact = w * 128 < I;
  f32x4_t total = {0.f, 0.f, 0.f, 0.f};
  G2Buf bA, bB;
  if (j0 < j1) g2_load(p, rt, j0, tile, bA);
  for (int j = j0; j < j1; ++j) {
    G2Buf cur = bA;
    if (j + 1 < j1) g2_load(p, rt, j + 1, tile, bB);
    if (kact) {
      const int e = rt.sel[j];
      uint4 bw[4];
      fp4_decode(cur.c, cur.s, bw);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = mfma_f16(cur.a[q], bw[q], acc);
      const float ts = p.cur.e_ts[2 * e + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) total[i] = fmaf(acc[i], ts, total[i]);
      if (debug && p.dbg.dq_dn && e == p.dbg.dq_expert) {
        const int k = w * 128 + g_ * 32;
        uint4* dst = reinterpret_cast<uint4*>(p.dbg.dq_dn + (size_t)(tile * 16 + r_) * I + k);
        const int nq = min(4, (I - k) / 8);
        for (int q = 0; q < nq; ++q) dst[q] = bw[q];
      }
    }
    bA = bB;
  }
  red_store(sm, 0, total);
  __syncthreads();
  if (threadIdx.x < 256) {
    const int tok = threadIdx.x >> 4, row = threadIdx.x & 15;
    float v = red_sum(sm, 0, threadIdx.x);
    if (tok < p.NT) p.accpart[((size_t)part * p.NT + tok) * P + tile * 16 + row] = v;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <uint32_t MODE, bool DEBUG>
__global__ void __launch_bounds__(kThreads, 1) layer_kernel(const Params p) {
  __shared__ Smem sm;
  Barrier bar{p.bar, p.err, (p.bar_base + 1) * gridDim.x, gridDim.x};
  const int Dq = p.nq * p.d;
  const int Nqkv = Dq + 2 * p.nkv * p.d;
  DenseBuf pre;

  if constexpr ((MODE & kModeQkvOwn) != 0) {
    dense_prefetch(p.s_qkv_own, p.cur.w_qkv, p.H, pre);
    compute_inv_rms(p, p.h_in, nullptr, sm);
    fill_x_norm(p, p.h_in, p.cur.g_attn, sm);
    EpiArgs ea{&p.cur, nullptr, p.qpart, nullptr, DEBUG ? p.dbg.k_new : nullptr, DEBUG ? p.dbg.v_new : nullptr};
    dense_phase<Epi::Qkv>(p, p.s_qkv_own, p.cur.w_qkv, p.H, p.H, ea, sm, pre, true);
    bar_arrive(bar);
    if (!bar_wait(bar, sm)) return;
    if (DEBUG && p.dbg.q) {
      for (int i = blockIdx.x * kThreads + threadIdx.x; i < p.NT * Dq; i += gridDim.x * kThreads) {
        float v = 0.0f;
        for (int s = 0; s < p.q_slices; ++s) v += p.qpart[(size_t)s * p.NT * Dq + i];
        p.dbg.q[i] = v;
      }
    }
  }
  (void)Nqkv;

  // attention of the launch's layer
  if (p.d == 128) attention_phase<128>(p, p.cur, sm);
  else attention_phase<64>(p, p.cur, sm);
  bar_arrive(bar);
  if (!bar_wait(bar, sm)) return;

  merge_phase(p, p.cur, DEBUG);
  bar_arrive(bar);
  dense_prefetch(p.s_oproj, p.cur.w_o, Dq, pre);
  if (!bar_wait(bar, sm)) return;

  // output projection + residual
  {
    fill_x_copy(p.attn, Dq, p.NT, sm);
    EpiArgs ea{nullptr, p.h_in, p.h1, p.ssq1, nullptr, nullptr};
    dense_phase<Epi::OProj>(p, p.s_oproj, p.cur.w_o, Dq, Dq, ea, sm, pre, true);
  }
  bar_arrive(bar);
  dense_prefetch(p.s_pool, p.cur.w_pool, p.H, pre);
  if (!bar_wait(bar, sm)) return;
  if (DEBUG && p.dbg.h1) {
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < p.NT * p.H; i += gridDim.x * kThreads) p.dbg.h1[i] = p.h1[i];
  }

  // router + pooler (both read n2 = RMSNorm(h1))
  {
    compute_inv_rms(p, p.h1, p.ssq1, sm);
    fill_x_norm(p, p.h1, p.cur.g_moe, sm);
    EpiArgs ea{nullptr, nullptr, p.ppart, nullptr, nullptr, nullptr};
    dense_phase<Epi::Pool>(p, p.s_pool, p.cur.w_pool, p.H, p.H, ea, sm, pre, true);
    router_phase(p, sm, DEBUG);
  }
  bar_arrive(bar);
  if (!bar_wait(bar, sm)) return;

  // routing (every workgroup) + experts' gate/up
  fill_x_sum(p.ppart, p.p_slices, p.P, p.NT, sm);
  routing(p, sm, blockIdx.x == 0);
  if (DEBUG && blockIdx.x == 0) {
    if (p.dbg.logits)
      for (int i = threadIdx.x; i < p.NT * p.E; i += kThreads) p.dbg.logits[i] = p.logits[i];
    if (p.dbg.p)
      for (int i = threadIdx.x; i < p.NT * p.P; i += kThreads) {
        float v = 0.0f;
        for (int s = 0; s < p.p_slices; ++s) v += p.ppart[(size_t)s * p.NT * p.P + i];
        p.dbg.p[i] = v;
      }
  }
  gemm1_phase(p, sm, DEBUG);
  bar_arrive(bar);
  if (!bar_wait(bar, sm)) return;

  gemm2_phase(p, sm, DEBUG);
  bar_arrive(bar);
  dense_prefetch(p.s_unpool, p.cur.w_unpool, p.P, pre);
  if (!bar_wait(bar, sm)) return;

  // unpooler + residual
  {
    const int parts = max(1, (int)gridDim.x / (p.P / 16));
    fill_x_sum(p.accpart, parts, p.P, p.NT, sm);
    EpiArgs ea{nullptr, p.h1, p.h_out, p.ssq2, nullptr, nullptr};
    dense_phase<Epi::Unpool>(p, p.s_unpool, p.cur.w_unpool, p.P, p.P, ea, sm, pre, true);
    if (DEBUG && p.dbg.acc && blockIdx.x == 0) {
      for (int i = threadIdx.x; i < p.NT * p.P; i += kThreads) {
        float v = 0.0f;
        for (int s = 0; s < parts; ++s) v += p.accpart[(size_t)s * p.NT * p.P + i];
        p.dbg.acc[i] = v;
      }
    }
  }

  if constexpr ((MODE & kModeQkvNext) != 0) {
    bar_arrive(bar);
    dense_prefetch(p.s_qkv_next, p.nxt.w_qkv, p.H, pre);
    if (!bar_wait(bar, sm)) return;
    compute_inv_rms(p, p.h_out, p.ssq2, sm);
    fill_x_norm(p, p.h_out, p.nxt.g_attn, sm);
    EpiArgs ea{&p.nxt, nullptr, p.qpart, nullptr, nullptr, nullptr};
    dense_phase<Epi::Qkv>(p, p.s_qkv_next, p.nxt.w_qkv, p.H, p.H, ea, sm, pre, true);
  }
}

__global__ void reset_kernel(uint32_t* bar, int32_t* err) {
  if (threadIdx.x == 0) {
    *bar = 0;
    *err = 0;
  }
}

}  // namespace
}  // namespace msk

hipError_t msk_launch_layer(const msk::Params& p, int grid, bool debug, hipStream_t s) {
  using namespace msk;
  const uint32_t mode = p.mode;
  dim3 g(grid), b(kThreads);
  if (debug) {
    if (mode != kModeQkvOwn) return hipErrorInvalidValue;
    hipLaunchKernelGGL((layer_kernel<kModeQkvOwn, true>), g, b, 0, s, p);
  } else if (mode == kModeQkvOwn) {
    hipLaunchKernelGGL((layer_kernel<kModeQkvOwn, false>), g, b, 0, s, p);
  } else if (mode == (kModeQkvOwn | kModeQkvNext)) {
    hipLaunchKernelGGL((layer_kernel<kModeQkvOwn | kModeQkvNext, false>), g, b, 0, s, p);
  } else if (mode == kModeQkvNext) {
    hipLaunchKernelGGL((layer_kernel<kModeQkvNext, false>), g, b, 0, s, p);
  } else {
    hipLaunchKernelGGL((layer_kernel<0u, false>), g, b, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t msk_launch_reset(uint32_t* bar, int32_t* err, hipStream_t s) {
  hipLaunchKernelGGL(msk::reset_kernel, dim3(1), dim3(64), 0, s, bar, err);
  return hipGetLastError();
}
