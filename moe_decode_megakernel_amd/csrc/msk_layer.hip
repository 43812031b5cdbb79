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
// the whole launch. Phases are separated by a grid barrier (a sequence-number
// flag per workgroup, bounded spin; see Barrier below). Weight tiles of the
// next phase are requested before waiting on the barrier, so the barrier
// latency overlaps the first weight fetch. Every contraction runs on
// fp16 MFMA (16x16x32, fp32 accumulation) with the 16 verify tokens as one
// 16-row tile: bf16 weights and cache rows convert to fp16 exactly (in fp16's
// normal range), activations are rounded to fp16 (11-bit significand), and
// expert weights decode from E2M1 x E4M3 into exact fp16, with the fp32 tensor
// scale applied to the fp32 accumulator.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

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
  uint4 zero;  // 16 zero bytes: the A operand of lanes whose k range is out of bounds
  uint8_t x[kXBytes];
  float red[2][kWaves][256];
  float inv_rms[kMaxTok * kMaxReq];
  Unit units[kSchCount][kMaxWgUnits];  // this workgroup's dense units, per schedule
  int32_t nunits[kSchCount];
  int32_t plist[kMaxPrefetch];          // speculative expert prefetch list
  int32_t flag;
  // request metadata of the launch (read from device memory at launch start)
  int32_t ctx[kMaxReq];                 // prior context length per request of the pass
  uint32_t tanc[kMaxReq][kMaxTok];      // ancestor bitmask per verify token (self included)
  uint64_t tdepth[kMaxReq];             // 4 bits per token: its number of ancestors
  int32_t io_code;                      // 0, or the error code of invalid metadata
  int32_t err0;                         // device error word at launch start
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

// Stores of data another workgroup reads later in the same launch are
// write-through at agent scope (relaxed atomic stores, emitted with sc1), so
// no dirty copy stays in one XCD's L2 and the grid barrier needs no L2
// writeback or invalidate.
__device__ __forceinline__ void st_wt(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wt(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wt(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// 16-byte write-through store (same cache policy as the scalar st_wt above).
// The operand is taken as one whole vector: assembling it from scalar
// bit-casts of its lanes has been compiled into a splat of lane 0.
__device__ __forceinline__ void st_wt16(void* p, u32x4_t d) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(d) : "memory");
}

// Keeps the loads of consecutive ring slots in program order. Without it the
// scheduler may reorder a prologue's independent slot loads, and the wait
// counts at the loop head, which must hold for the first iteration too, then
// drain the whole ring on every iteration.
__device__ __forceinline__ void ring_fence() { __builtin_amdgcn_sched_barrier(0); }

// Waits for every outstanding vector memory operation (s_waitcnt vmcnt(0),
// other counters untouched). Placed where all loads have completed anyway
// (the end of an activation fill), it also clears the compiler's record of
// pending loads, so the wait counts of a following ring loop are computed
// from that loop alone.
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Prior context length of request r of the pass (from LDS; the caller takes
// readfirstlane where r is wave-uniform).
__device__ __forceinline__ int ctx_of(const Smem& sm, int r) { return sm.ctx[r]; }
__device__ __forceinline__ int ctx_uni(const Smem& sm, int r) { return __builtin_amdgcn_readfirstlane(sm.ctx[r]); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Verify-token tree of request r (wave-uniform) seen from token t (per lane):
// t's ancestor bitmask, and the packed depths of all the request's tokens.
__device__ __forceinline__ uint32_t tree_anc_of(const Smem& sm, int r, int t) { return sm.tanc[r][t]; }
__device__ __forceinline__ uint64_t tree_depth_of(const Smem& sm, int r) {
  const uint64_t d = sm.tdepth[r];
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(d >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)d);
}

// Phase-boundary slots of the self-timing trace (one uint64 per slot, per
// workgroup, per launch; 100 MHz real-time counter).
enum TraceSlot {
  kTrStart = 0, kTrQkvOwn, kTrQkvOwnBar, kTrAttnQ, kTrAttnKv, kTrAttn, kTrAttnBar, kTrMerge, kTrMergeBar, kTrOprojFill, kTrOproj,
  kTrOprojBar, kTrPoolFill, kTrRouterPool, kTrRouterPoolBar, kTrRouting, kTrGemm1, kTrGemm1Bar, kTrGemm2,
  kTrGemm2Bar, kTrUnpoolFill, kTrUnpool, kTrUnpoolBar, kTrQkvFill, kTrQkvNext, kTrSlots
};
static_assert(kTrSlots == kTraceSlots, "trace slot count");

// Phase-boundary stamp of the self-timing variant (row = this workgroup's
// trace row, or NULL).
__device__ __forceinline__ void trace_stamp(uint64_t* row, int slot) {
  if (row && threadIdx.x == 0) row[slot] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Pairwise tree sum over aligned groups of n lanes (n a power of two <= 64),
// adjacent pairs first: level l adds the partner block of 2^(l-1) lanes.
// After each level every lane of a block holds the same value, so any lane
// permutation that maps a block onto its partner gives the same sums (fp32
// addition is commutative): quad_perm [1,0,3,2] and [2,3,0,1], then the
// half-row and row mirrors (DPP), then read-lanes of the 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Combination with the lane 16 or 32 apart by the gfx950 lane swaps
// (v_permlane16_swap: odd 16-lane rows of the first operand with even rows of
// the second; v_permlane32_swap: upper half of the first with lower half of
// the second). Both operands are v, so in every lane the two results are v and
// its partner's v, in an order that depends on the lane: a commutative
// combination of the pair equals the combination with the partner. The two
// results are copied to named words before the bit cast: a bit cast applied
// to the builtin's second element directly compiles to its first.
template <int DIST>
__device__ __forceinline__ void lane_pair(float v, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  uint32_t r0, r1;
  if constexpr (DIST == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    static_assert(DIST == 32, "distance 16 or 32");
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
template <int DIST>
__device__ __forceinline__ float max_with_partner(float v) {
  float a, b;
  lane_pair<DIST>(v, a, b);
  return fmaxf(a, b);
}
template <int DIST>
__device__ __forceinline__ float sum_with_partner(float v) {
  float a, b;
  lane_pair<DIST>(v, a, b);
  return a + b;
}
__device__ __forceinline__ float lane_tree_sum(float acc, int n) {
  if (n >= 2) acc = acc + dpp_f32<0xB1>(acc);   // quad_perm [1,0,3,2]
  if (n >= 4) acc = acc + dpp_f32<0x4E>(acc);   // quad_perm [2,3,0,1]
  if (n >= 8) acc = acc + dpp_f32<0x141>(acc);  // row_half_mirror
  if (n >= 16) acc = acc + dpp_f32<0x140>(acc); // row_mirror
  if (n >= 32) {
    const float r0 = readlane_f32(acc, 0), r1 = readlane_f32(acc, 16);
    const float r2 = readlane_f32(acc, 32), r3 = readlane_f32(acc, 48);
    acc = (n == 32) ? (lane_id() < 32 ? r0 + r1 : r2 + r3) : (r0 + r1) + (r2 + r3);
  }
  return acc;
}


// ---------------------------------------------------------------------------
// Grid barrier. All data exchanged between workgroups inside a launch is
// written with write-through stores (st_wt) and read with ordinary loads, and
// no workgroup reads such a buffer before the phase that writes it (caches
// start clean at the launch boundary). Arriving: every wave waits for its
// stores to complete (s_waitcnt vmcnt(0)), the workgroup meets, and one
// thread publishes the barrier's sequence number in the workgroup's own flag
// word (write-through). Waiting: wave 0 polls all flags until each reaches
// the sequence number (bounded spin), then the workgroup meets again.
// Each flag has a 64-byte line of its own (kFlagStride). No atomics, no L2
// writeback or invalidate. Sequence numbers grow through a call (reset at its start).
// ---------------------------------------------------------------------------
struct Barrier {
  uint32_t* flags;  // [grid][kFlagStride] sequence numbers in word 0
  int32_t* err;
  uint32_t seq;     // sequence number of the next barrier
};

// Arrival with sequence number seq: every store of this workgroup so far is
// complete before its flag holds seq.
__device__ __forceinline__ void bar_arrive_at(const Barrier& b, uint32_t seq) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(&b.flags[blockIdx.x * kFlagStride], seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void bar_arrive(Barrier& b) { bar_arrive_at(b, b.seq); }

// Waits until every workgroup's flag holds at least seq. Returns false if the
// launch must stop (timeout or an error raised elsewhere). Wave 0 alone polls
// every workgroup's flag (4 per lane), so the other waves may have weight
// loads in flight without delaying the polls (vector-memory counts complete
// in order within a wave).
__device__ __forceinline__ bool bar_wait_at(const Barrier& b, Smem& sm, uint32_t seq) {
  if (__builtin_amdgcn_readfirstlane(wave_id()) == 0) {
    const int lane = lane_id(), G = gridDim.x;
    int ok = 1;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (uint32_t polls = 1;; ++polls) {
      // all four flag loads in flight together, combined without a
      // short-circuit (which would serialise them)
      uint32_t f[kMaxGrid / 64];
#pragma unroll
      for (int j = 0; j < kMaxGrid / 64; ++j)
        f[j] = __hip_atomic_load(&b.flags[min(lane + 64 * j, G - 1) * kFlagStride], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      int behind = 0;
#pragma unroll
      for (int j = 0; j < kMaxGrid / 64; ++j) behind += f[j] < seq ? 1 : 0;
      if (__ballot(behind != 0) == 0) break;
      if ((polls & 63u) == 0) {
        if (__hip_atomic_load(b.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) { ok = 0; break; }
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
          if (lane == 0) __hip_atomic_store(b.err, kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
      }
    }
    if (lane == 0) sm.flag = ok;
  }
  __syncthreads();
  return sm.flag != 0;
}

// The grid barrier: every workgroup has arrived with the current sequence
// number; the next barrier uses the following one.
__device__ __forceinline__ bool bar_wait(Barrier& b, Smem& sm) {
  const bool ok = bar_wait_at(b, sm, b.seq);
  b.seq += 1;
  return ok;
}

// bar_wait, with the next phase's weight prefetch issued by waves 1..7
// before the wait and by wave 0 (the poller) after it.
template <class F>
__device__ __forceinline__ bool bar_wait_prefetch(Barrier& b, Smem& sm, F&& prefetch) {
  const bool poller = __builtin_amdgcn_readfirstlane(wave_id()) == 0;
  if (!poller) prefetch();
  const bool ok = bar_wait(b, sm);
  if (poller && ok) prefetch();
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
// [ntiles][NT], summed in tile order) or, when ssq is NULL, from h directly.
// H is a power of two in 128..4096 (so H/4 is a multiple of 32).
__device__ __forceinline__ void compute_inv_rms(const Params& p, const float* h, const float* ssq, Smem& sm) {
  const int NT = p.NT, H = p.H;
  if (!p.use_norm) {
    if (threadIdx.x < kMaxTok) sm.inv_rms[threadIdx.x] = 1.0f;
    __syncthreads();
    return;
  }
  if (ssq) {
    // lane j sums tile partials j, j+64, ... in order, then pairwise halving
    const int lane = lane_id();
    const int nt = H / 16;
    for (int t = wave_id(); t < NT; t += kWaves) {
      float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = lane + q * 64;
        if (i < nt) v[q] = ssq[i * NT + t];
      }
      float s = ((v[0] + v[1]) + v[2]) + v[3];
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0) sm.inv_rms[t] = rsqrtf(s / (float)H + p.eps);
    }
  } else {
    // lane j sums elements j, j + 64, ... of the token's row in order, then
    // pairwise halving; the loads of half a row (at the largest H) are in
    // flight together
    constexpr int kE = 4096 / 64 / 2;  // elements per lane and batch at the largest H
    const int lane = lane_id();
    for (int t = wave_id(); t < NT; t += kWaves) {
      const float* hp = h + (size_t)t * H;
      float s = 0.0f;
      for (int b0 = 0; b0 < H; b0 += 64 * kE) {
        float x[kE];
#pragma unroll
        for (int i = 0; i < kE; ++i) x[i] = hp[min(b0 + lane + 64 * i, H - 1)];
#pragma unroll
        for (int i = 0; i < kE; ++i)
          if (b0 + lane + 64 * i < H) s = fmaf(x[i], x[i], s);
      }
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0) sm.inv_rms[t] = rsqrtf(s / (float)H + p.eps);
    }
  }
  __syncthreads();
}

// inv_rms from per-tile partial sums of squares in two steps, so the loads can
// be issued early: lane j of wave w holds partials j, j+64, j+128, j+192 of
// tokens w and w+8 (summed in that order, then pairwise halving over lanes).
struct SsqLoads {
  float v[kMaxTok / kWaves][4];
};
static_assert(kMaxTok / kWaves == 2, "two tokens per wave");

__device__ __forceinline__ SsqLoads ssq_issue(const Params& p, const float* ssq) {
  SsqLoads L;
  const int lane = lane_id(), w = wave_id(), NT = p.NT, nt = p.H / 16;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = min(w + r * kWaves, NT - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) L.v[r][q] = ssq[min(lane + q * 64, nt - 1) * NT + t];
  }
  return L;
}

// Writes sm.inv_rms (the caller meets on a workgroup barrier before use).
__device__ __forceinline__ void ssq_finish(const Params& p, const SsqLoads& L, Smem& sm) {
  const int lane = lane_id(), w = wave_id(), NT = p.NT, nt = p.H / 16;
  if (!p.use_norm) {
    if (threadIdx.x < kMaxTok) sm.inv_rms[threadIdx.x] = 1.0f;
    return;
  }
  // both tokens' exchange chains first (independent), then the stores
  float s[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    s[r] = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) s[r] += (lane + q * 64 < nt) ? L.v[r][q] : 0.0f;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int r = 0; r < 2; ++r) s[r] += __shfl_xor(s[r], o);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = w + r * kWaves;
    if (lane == 0 && t < NT) sm.inv_rms[t] = rsqrtf(s[r] / (float)p.H + p.eps);
  }
}

// X = fp16(h * inv_rms * g), or fp16(h) without the norm; rounded to nearest
// even. The normalised value is bounded by sqrt(H) * |g| (no element of a
// vector exceeds sqrt(n) times its RMS), so a residual of any magnitude stays
// inside fp16's range once the RMS scale is applied, and the scale is applied
// before the rounding. Item i = (token i / K8, elements 8*(i % K8)
// .. +8); a thread's items share one k range (K8 divides the workgroup
// size), and the loads of kFillBatch items are issued before any is used.
constexpr int kFillBatch = 4;

template <int B = kFillBatch>
__device__ __forceinline__ void fill_x_norm(const Params& p, const float* h, const uint16_t* g, Smem& sm) {
  const int K = p.H, NT = p.NT, K8 = K / 8;
  const int total = kMaxTok * K8;
  const int k = (threadIdx.x % K8) * 8;
  float gj[8];
  {
    const uint4 gg = *reinterpret_cast<const uint4*>(g + k);
    const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) gj[j] = p.use_norm ? bf2f((uint16_t)(gw[j >> 1] >> ((j & 1) * 16))) : 1.0f;
  }
  for (int i0 = threadIdx.x; i0 < total; i0 += B * kThreads) {
    float4 a[B], b[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int t = min((i0 + q * kThreads) / K8, NT - 1);
      const float4* hp = reinterpret_cast<const float4*>(h + (size_t)t * K + k);
      a[q] = hp[0];
      b[q] = hp[1];
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int i = i0 + q * kThreads;
      if (i >= total) break;
      const int t = i / K8;
      uint4 out = make_uint4(0, 0, 0, 0);
      if (t < NT) {
        float v[8] = {a[q].x, a[q].y, a[q].z, a[q].w, b[q].x, b[q].y, b[q].z, b[q].w};
        const float inv = sm.inv_rms[t];
        if (p.use_norm) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = (v[j] * inv) * gj[j];
        }
        out.x = pack2(f2h(v[0]), f2h(v[1]));
        out.y = pack2(f2h(v[2]), f2h(v[3]));
        out.z = pack2(f2h(v[4]), f2h(v[5]));
        out.w = pack2(f2h(v[6]), f2h(v[7]));
      }
      *reinterpret_cast<uint4*>(sm.x + t * x_stride(K) + k * 2) = out;
    }
  }
  vm_drain();
  __syncthreads();
}

// X = copy of a 16-bit activation matrix src [NT][K] (already fp16).
template <int B = 2 * kFillBatch>
__device__ __forceinline__ void fill_x_copy(const uint16_t* src, int K, int NT, Smem& sm) {
  const int K8 = K / 8, total = kMaxTok * K8;
  for (int i0 = threadIdx.x; i0 < total; i0 += B * kThreads) {
    uint4 v[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int i = i0 + q * kThreads;
      const int t = min(i / K8, NT - 1), k = (i % K8) * 8;
      v[q] = *reinterpret_cast<const uint4*>(src + (size_t)t * K + k);
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int i = i0 + q * kThreads;
      if (i >= total) break;
      const int t = i / K8, k = (i % K8) * 8;
      *reinterpret_cast<uint4*>(sm.x + t * x_stride(K) + k * 2) = t < NT ? v[q] : make_uint4(0, 0, 0, 0);
    }
  }
  vm_drain();
  __syncthreads();
}

// QKV input of the next layer: X = fp16(h * inv_rms * g) from the fp32
// residual the unpooler wrote, with inv_rms from the unpooler's per-tile
// partial sums of squares. The partial sums and the first half of the
// residual are requested together (one round trip), the second half after.
__device__ __forceinline__ void fill_x_qkv(const Params& p, const float* h, const float* ssq, const uint16_t* g,
                                           Smem& sm) {
  constexpr int B = 2 * kFillBatch;
  const int K = p.H, NT = p.NT, K8 = K / 8;
  const int total = kMaxTok * K8;
  const int k = (threadIdx.x % K8) * 8;
  const SsqLoads L = ssq_issue(p, ssq);
  float gj[8];
  {
    const uint4 gg = *reinterpret_cast<const uint4*>(g + k);
    const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) gj[j] = p.use_norm ? bf2f((uint16_t)(gw[j >> 1] >> ((j & 1) * 16))) : 1.0f;
  }
  bool first = true;
  for (int i0 = threadIdx.x; i0 < total; i0 += B * kThreads) {
    float4 a[B], b[B];
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int t = min((i0 + q * kThreads) / K8, NT - 1);
      const float4* hp = reinterpret_cast<const float4*>(h + (size_t)t * K + k);
      a[q] = hp[0];
      b[q] = hp[1];
    }
    if (first) {
      ssq_finish(p, L, sm);
      __syncthreads();
      first = false;
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int i = i0 + q * kThreads;
      if (i >= total) break;
      const int t = i / K8;
      uint4 out = make_uint4(0, 0, 0, 0);
      if (t < NT) {
        float v[8] = {a[q].x, a[q].y, a[q].z, a[q].w, b[q].x, b[q].y, b[q].z, b[q].w};
        if (p.use_norm) {
          const float inv = sm.inv_rms[t];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = (v[j] * inv) * gj[j];
        }
        out.x = pack2(f2h(v[0]), f2h(v[1]));
        out.y = pack2(f2h(v[2]), f2h(v[3]));
        out.z = pack2(f2h(v[4]), f2h(v[5]));
        out.w = pack2(f2h(v[6]), f2h(v[7]));
      }
      *reinterpret_cast<uint4*>(sm.x + t * x_stride(K) + k * 2) = out;
    }
  }
  vm_drain();
  __syncthreads();
}

// X = sum over n partial slots of fp32 [n][NT][K] (slot order), rounded to fp16.
template <int B = kFillBatch>
__device__ __forceinline__ void fill_x_sum(const float* parts, int n, int K, int NT, Smem& sm) {
  const int K8 = K / 8, total = kMaxTok * K8;
  for (int i0 = threadIdx.x; i0 < total; i0 += B * kThreads) {
    float v[B][8];
#pragma unroll
    for (int q = 0; q < B; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) v[q][j] = 0.0f;
    int s = 0;
    for (; s + 2 <= n; s += 2) {
      float4 a[2][B], b[2][B];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < B; ++q) {
          const int i = i0 + q * kThreads;
          const int t = min(i / K8, NT - 1), k = (i % K8) * 8;
          const float4* src = reinterpret_cast<const float4*>(parts + ((size_t)(s + u) * NT + t) * K + k);
          a[u][q] = src[0];
          b[u][q] = src[1];
        }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < B; ++q) {
          v[q][0] += a[u][q].x; v[q][1] += a[u][q].y; v[q][2] += a[u][q].z; v[q][3] += a[u][q].w;
          v[q][4] += b[u][q].x; v[q][5] += b[u][q].y; v[q][6] += b[u][q].z; v[q][7] += b[u][q].w;
        }
    }
    if (s < n) {
      float4 a[B], b[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int i = i0 + q * kThreads;
        const int t = min(i / K8, NT - 1), k = (i % K8) * 8;
        const float4* src = reinterpret_cast<const float4*>(parts + ((size_t)s * NT + t) * K + k);
        a[q] = src[0];
        b[q] = src[1];
      }
#pragma unroll
      for (int q = 0; q < B; ++q) {
        v[q][0] += a[q].x; v[q][1] += a[q].y; v[q][2] += a[q].z; v[q][3] += a[q].w;
        v[q][4] += b[q].x; v[q][5] += b[q].y; v[q][6] += b[q].z; v[q][7] += b[q].w;
      }
    }
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int i = i0 + q * kThreads;
      if (i >= total) break;
      const int t = i / K8, k = (i % K8) * 8;
      uint4 out = make_uint4(0, 0, 0, 0);
      if (t < NT) {
        out.x = pack2(f2h(v[q][0]), f2h(v[q][1])); out.y = pack2(f2h(v[q][2]), f2h(v[q][3]));
        out.z = pack2(f2h(v[q][4]), f2h(v[q][5])); out.w = pack2(f2h(v[q][6]), f2h(v[q][7]));
      }
      *reinterpret_cast<uint4*>(sm.x + t * x_stride(K) + k * 2) = out;
    }
  }
  vm_drain();
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Dense projection (bf16 weights): Y[t][n] = sum_k X[t][k] W[n][k] over the
// units of this workgroup. A unit is 16 weight rows x klen (<= 1024) k; wave
// w owns the 128-k sub-unit w: lane (r, g) loads 16 B of row r at
// k = k0 + w*128 + s*32 + g*8 (s = 0..3), converts it to fp16 and feeds one
// MFMA per load. The 8 per-wave 16x16 partials are summed in LDS in wave
// order. A wave whose sub-unit lies beyond klen loads a clamped in-range
// address and reads the zero A operand, so every wave issues the same loads
// for every unit: the compiler can count them, and kRing units of loads stay
// in flight across unit boundaries.
// ---------------------------------------------------------------------------
constexpr int kRing = 4;

struct DenseSlot {
  uint4 b[4];
  float res;  // residual of this thread's (token, row) output (epilogues that add one)
};

template <bool RES>
__device__ __forceinline__ void dense_issue(const Unit& u, const uint16_t* W, int ldw, const float* res, int H,
                                            int NT, DenseSlot& sl) {
  const int lane = lane_id(), r = lane & 15, g = lane >> 4, w = wave_id();
  const bool valid = w * kSubK < u.klen;
  const int k = u.k0 + (valid ? w * kSubK : 0) + g * 8;
  const uint16_t* row = W + (size_t)(u.tile * 16 + r) * ldw + k;
#pragma unroll
  for (int q = 0; q < 4; ++q) sl.b[q] = *reinterpret_cast<const uint4*>(row + q * 32);
  if constexpr (RES) {
    const int tid = threadIdx.x & 255;
    const int tok = min(tid >> 4, NT - 1);
    sl.res = res[(size_t)tok * H + u.tile * 16 + (tid & 15)];
  }
}

__device__ __forceinline__ f32x4_t dense_compute(const Smem& sm, int K, const Unit& u, const DenseSlot& sl,
                                                 f32x4_t acc) {
  const int lane = lane_id(), r = lane & 15, g = lane >> 4, w = wave_id();
  const bool valid = w * kSubK < u.klen;
  const uint8_t* abase = valid ? sm.x + r * x_stride(K) + (u.k0 + w * kSubK + g * 8) * 2
                               : reinterpret_cast<const uint8_t*>(&sm.zero);
  const int astep = valid ? 64 : 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 a = *reinterpret_cast<const uint4*>(abase + q * astep);
    acc = mfma_f16(a, bf8_to_h8(sl.b[q]), acc);
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
  uint16_t* k_cache;  // QKV epilogue: caches of the projected layer
  uint16_t* v_cache;
  const float* res;  // residual input (OProj: h, Unpool: h1)
  float* out;        // OProj: h1, Unpool: h_out, Pool: ppart, Qkv: qpart
  float* ssq;        // partial sums of squares (OProj, Unpool)
  float* dbg_k;
  float* dbg_v;
};

template <Epi E>
__device__ __forceinline__ void dense_epilogue(const Params& p, const EpiArgs& ea, const Unit& u,
                                               const Smem& sm, int rb, float res) {
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
        st_wt(&ea.out[((size_t)(u.slot & kUnitSlotMask) * NT + tok) * Dq + n], v);
      } else {
        int c = n - Dq;
        bool is_v = c >= Dkv;
        if (is_v) c -= Dkv;
        int g = c / p.d, cc = c % p.d;
        int r = tok / p.T, t = tok % p.T;
        size_t dst = (((size_t)r * p.nkv + g) * p.cap + ctx_of(sm, r) + t) * p.d + cc;
        if (is_v) {
          st_wt(&ea.v_cache[dst], f2bf(v));
          if (ea.dbg_v) ea.dbg_v[(size_t)tok * Dkv + c] = v;
        } else {
          st_wt(&ea.k_cache[dst], f2bf(v));
          if (ea.dbg_k) ea.dbg_k[(size_t)tok * Dkv + c] = v;
        }
      }
    }
  } else if constexpr (E == Epi::Pool) {
    if (tok < NT) st_wt(&ea.out[((size_t)(u.slot & kUnitSlotMask) * NT + tok) * p.P + n], v);
  } else {
    // OProj / Unpool: residual add, then partial sum of squares over the tile's 16 rows.
    float h = 0.0f;
    if (tok < NT) {
      h = res + v;
      st_wt(&ea.out[(size_t)tok * p.H + n], h);
    }
    float s = sum16(h * h);
    if (row == 0 && tok < NT) st_wt(&ea.ssq[u.tile * NT + tok], s);
  }
}

// A unit from this workgroup's LDS copy of a schedule, as wave-uniform values.
__device__ __forceinline__ Unit lds_unit(const Smem& sm, int sch, int i) {
  const Unit u = sm.units[sch][i];
  return Unit{__builtin_amdgcn_readfirstlane(u.tile), __builtin_amdgcn_readfirstlane(u.k0),
              __builtin_amdgcn_readfirstlane(u.klen), __builtin_amdgcn_readfirstlane(u.slot)};
}

// Runs this workgroup's dense units of schedule `sch`; the first kRing units'
// weights are already in flight in the ring (requested by dense_prefetch
// before the preceding barrier wait).
template <Epi E>
__device__ __forceinline__ void dense_phase(const Params& p, int sch, const uint16_t* W, int ldw, int K,
                                            const EpiArgs& ea, Smem& sm, DenseSlot (&ring)[kRing]) {
  constexpr bool RES = E == Epi::OProj || E == Epi::Unpool;
  const int n = sm.nunits[sch];
  if (n <= 0) return;
  int rb = 0;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < n; base += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int ui = base + i;
      const Unit u = lds_unit(sm, sch, min(ui, n - 1));
      if (u.slot & kUnitFirst) acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc = dense_compute(sm, K, u, ring[i], acc);
      if (ui < n && (u.slot & kUnitLast)) {
        red_store(sm, rb, acc);
        __syncthreads();
        dense_epilogue<E>(p, ea, u, sm, rb, ring[i].res);
        rb ^= 1;
      }
      dense_issue<RES>(lds_unit(sm, sch, min(ui + kRing, n - 1)), W, ldw, ea.res, p.H, p.NT, ring[i]);
      ring_fence();
    }
  }
  __syncthreads();
}

template <Epi E>
__device__ __forceinline__ void dense_prefetch(const Params& p, int sch, const uint16_t* W, int ldw,
                                               const float* res, const Smem& sm, DenseSlot (&ring)[kRing]) {
  constexpr bool RES = E == Epi::OProj || E == Epi::Unpool;
  const int n = sm.nunits[sch];
  if (n <= 0) return;
#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    dense_issue<RES>(lds_unit(sm, sch, min(i, n - 1)), W, ldw, res, p.H, p.NT, ring[i]);
    ring_fence();
  }
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

__device__ __forceinline__ void attn_range(const Params& p, const Smem& sm, const LayerW& lw, int r, int& lo,
                                           int& hi) {
  const int ctx = ctx_uni(sm, r);
  lo = (lw.window > 0) ? max(0, ctx - lw.window + 1) : 0;
  hi = ctx + p.T - 1;
}

// Keys per split: a whole number of chunks, as few as the split cap allows
// (one chunk per item where the grid has room).
__device__ __forceinline__ int attn_split_keys(const Params& p, int nkeys, int grid) {
  int cap_s = min(kMaxSplits, grid / (p.R * p.nkv));
  if (cap_s < 1) cap_s = 1;
  const int per = kAttnChunk * cap_s;
  return kAttnChunk * ((nkeys + per - 1) / per);
}
__device__ __forceinline__ int attn_splits(const Params& p, int nkeys, int grid) {
  const int cs = attn_split_keys(p, nkeys, grid);
  return (nkeys + cs - 1) / cs;
}

// Item of a flat index; returns false if idx is past the last item.
__device__ __forceinline__ bool attn_item(const Params& p, const Smem& sm, const LayerW& lw, int idx, int grid,
                                          AttnItem& it) {
  for (int r = 0; r < p.R; ++r) {
    int lo, hi;
    attn_range(p, sm, lw, r, lo, hi);
    int nk = hi - lo + 1;
    int S = attn_splits(p, nk, grid);
    int n_r = S * p.nkv;
    if (idx < n_r) {
      it.r = r;
      it.g = idx / S;
      it.s = idx % S;
      it.nsplit = S;
      const int cs = attn_split_keys(p, nk, grid);
      it.k_begin = lo + it.s * cs;
      it.k_end = min(hi + 1, it.k_begin + cs);
      return true;
    }
    idx -= n_r;
  }
  return false;
}

// Index of the first item of (r, g) in the flat order.
__device__ __forceinline__ int attn_item_base(const Params& p, const Smem& sm, const LayerW& lw, int r, int g,
                                              int grid, int& S) {
  int base = 0;
  for (int rr = 0; rr < p.R; ++rr) {
    int lo, hi;
    attn_range(p, sm, lw, rr, lo, hi);
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

// Number of attention items of the launch (workgroups at or past it are idle
// during the attention phase).
__device__ __forceinline__ int attn_item_count(const Params& p, const Smem& sm, const LayerW& lw, int grid) {
  int n = 0;
  for (int r = 0; r < p.R; ++r) {
    int lo, hi;
    attn_range(p, sm, lw, r, lo, hi);
    n += attn_splits(p, hi - lo + 1, grid) * p.nkv;
  }
  return n;
}

// Partial record of (item, wave, token): o[d], then m, l (stride d + 4 floats,
// so every record starts 16-byte aligned).
__device__ __forceinline__ float* apart_at(const Params& p, int item, int w, int t) {
  return p.apart + (((size_t)item * kWaves + w) * kMaxTok + t) * (p.d + 4);
}

template <int D>
__device__ __forceinline__ void attention_phase(const Params& p, const LayerW& lw, Smem& sm, uint64_t* trace_row) {
  AttnItem it;
  if (!attn_item(p, sm, lw, blockIdx.x, gridDim.x, it)) return;
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int group = p.nq / p.nkv;
  const int Dq = p.nq * p.d;
  const bool active = w < group;
  const int h = it.g * group + w;
  const int ctx = ctx_uni(sm, it.r);
  const int window = lw.window;
  // this lane's token: ancestor set and position ctx + depth on its own path
  const uint32_t tanc = tree_anc_of(sm, it.r, min(r_, kMaxTok - 1));
  const uint64_t tdepth = tree_depth_of(sm, it.r);
  const int tpos = ctx + (int)((tdepth >> (4 * min(r_, kMaxTok - 1))) & 15u);
  constexpr int KS = D / 32;     // MFMA steps over the head dim
  constexpr int DT = D / 16;     // d tiles of the PV product
  constexpr int RS = D + 8;               // K tile row stride (elements): Ks[key][d]
  constexpr int VS = kAttnChunk + 4;      // V^T tile row stride (elements): Vt[d][key]
  uint16_t* Ks = reinterpret_cast<uint16_t*>(sm.x);
  uint16_t* Vt = Ks + kAttnChunk * RS;
  uint16_t* Ks1 = Vt + D * VS;  // second buffer
  uint16_t* Vt1 = Ks1 + kAttnChunk * RS;
  static_assert((2 * kAttnChunk * (kMaxHeadDim + 8) + 2 * kMaxHeadDim * (kAttnChunk + 4)) * 2 <= kXBytes,
                "two K/V chunk buffers fit the X region");

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

  // K pieces: consecutive threads walk a key's dims (coalesced rows);
  // V pieces: consecutive threads walk keys at fixed dims, so the transposed
  // LDS writes of a wave land on consecutive addresses.
  // Two chunks of K/V are in flight in registers while one is computed. The
  // loads are unconditional: a chunk past the item's end re-reads its last
  // row (in bounds; masked below), so the wait counts stay static.
  uint4 kreg0[PER], vreg0[PER], kreg1[PER], vreg1[PER];
  auto load_chunk = [&](int c, uint4 (&kr)[PER], uint4 (&vr)[PER]) {
    int kb = it.k_begin + c * kAttnChunk;
    static_assert(CH16 % kThreads == 0, "a chunk is a whole number of 16-byte pieces per thread");
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      int i = threadIdx.x + j * kThreads;
      // keys past the item's end read its last row (finite values, masked later)
      const int key = i / (D / 8), c8 = (i % (D / 8)) * 8;
      kr[j] = *reinterpret_cast<const uint4*>(kc + (size_t)min(kb + key, it.k_end - 1) * D + c8);
      const int vkey = i % kAttnChunk, vc8 = (i / kAttnChunk) * 8;
      vr[j] = *reinterpret_cast<const uint4*>(vc + (size_t)min(kb + vkey, it.k_end - 1) * D + vc8);
    }
  };
  auto stage_chunk = [&](const uint4 (&kr)[PER], const uint4 (&vr)[PER], uint16_t* Ks, uint16_t* Vt) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      int i = threadIdx.x + j * kThreads;
      int key = i / (D / 8), c8 = (i % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(Ks + key * RS + c8) = bf8_to_h8(kr[j]);
      int vkey = i % kAttnChunk, vc8 = (i / kAttnChunk) * 8;
      const uint4 vh = bf8_to_h8(vr[j]);
      const uint32_t vw[4] = {vh.x, vh.y, vh.z, vh.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        Vt[(vc8 + 2 * q) * VS + vkey] = (uint16_t)(vw[q] & 0xFFFFu);
        Vt[(vc8 + 2 * q + 1) * VS + vkey] = (uint16_t)(vw[q] >> 16);
      }
    }
  };
  load_chunk(0, kreg0, vreg0);
  ring_fence();
  load_chunk(1, kreg1, vreg1);
  ring_fence();
  // Q^T operand (col = token r_, 8 consecutive dims per lane group): all
  // split-K slices of Q are requested right after the first two K/V chunks
  // (one round trip for both; lanes of inactive waves or tokens read an
  // in-range row and are zeroed), then summed in slice order.
  uint4 qb[KS];
  {
    const int tok = it.r * p.T + min(r_, p.T - 1);
    const int hq = active ? h : it.g * group;
    float4 qa[kMaxQSlices][KS], qc[kMaxQSlices][KS];
#pragma unroll
    for (int sl = 0; sl < kMaxQSlices; ++sl) {
      const int slc = min(sl, p.q_slices - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const float4* q4 = reinterpret_cast<const float4*>(
            p.qpart + ((size_t)slc * p.NT + tok) * Dq + hq * D + s * 32 + g_ * 8);
        qa[sl][s] = q4[0];
        qc[sl][s] = q4[1];
      }
    }
    const bool use = active && r_ < p.T;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int sl = 0; sl < kMaxQSlices; ++sl) {
        if (sl < p.q_slices) {
          const float4 a = qa[sl][s], b = qc[sl][s];
          v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
          v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
        }
      }
      qb[s].x = use ? pack2(f2h(v[0]), f2h(v[1])) : 0u;
      qb[s].y = use ? pack2(f2h(v[2]), f2h(v[3])) : 0u;
      qb[s].z = use ? pack2(f2h(v[4]), f2h(v[5])) : 0u;
      qb[s].w = use ? pack2(f2h(v[6]), f2h(v[7])) : 0u;
    }
  }

  trace_stamp(trace_row, kTrAttnQ);
  // One 64-key chunk: scores for 4 key tiles of 16 (the K reads and MFMAs of
  // all four tiles first, independent accumulators each summed over s in
  // order), then the mask, evaluated without short-circuit branches, the
  // online softmax in base 2, and O^T += V^T P^T over two 32-key steps.
  auto compute_chunk = [&](int c, const uint16_t* Kb, const uint16_t* Vb) {
    const int kb = it.k_begin + c * kAttnChunk;
    f32x4_t s4v[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s4v[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint4 a = *reinterpret_cast<const uint4*>(Kb + (kt * 16 + r_) * RS + s * 32 + g_ * 8);
        s4v[kt] = mfma_f16(a, qb[s], s4v[kt]);
      }
    float sc[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + kt * 16 + 4 * g_ + i;
        // prior rows by the window from the token's path position; new rows
        // of its ancestors whose path position is inside the window
        const int u = key - ctx;
        const bool prior = key < ctx;
        const int kpos = prior ? key : ctx + (int)((tdepth >> (4 * (u & 15))) & 15u);
        const bool vis = (key < it.k_end) & (r_ < p.T) & (prior | (((tanc >> (u & 15)) & 1u) != 0u)) &
                         ((window <= 0) | (kpos > tpos - window));
        sc[kt][i] = vis ? s4v[kt][i] * scale_log2 : -INFINITY;
      }
    }
    float cmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, sc[kt][i]);
    cmax = max_with_partner<16>(cmax);
    cmax = max_with_partner<32>(cmax);
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
    psum = sum_with_partner<16>(psum);
    psum = sum_with_partner<32>(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] *= alpha;
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
        const uint16_t* vrow = Vb + (dt * 16 + r_) * VS;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + k0);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + k0 + 16);
        uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[dt] = mfma_f16(av, bp, o[dt]);
      }
    }
  };
  // Two LDS buffers: chunk c+1 is staged (from registers) while chunk c is
  // computed from the other buffer, with one workgroup barrier per chunk.
  // Register sets A (even chunks) and B (odd chunks) hold the next two
  // chunks' loads; every load is issued (past the item's end it re-reads the
  // item's last row), so the wait counts stay static.
  stage_chunk(kreg0, vreg0, Ks, Vt);
  load_chunk(2, kreg0, vreg0);
  ring_fence();
  __syncthreads();
  trace_stamp(trace_row, kTrAttnKv);
  for (int c0 = 0; c0 < nchunks; c0 += 2) {
    if (c0 + 1 < nchunks) stage_chunk(kreg1, vreg1, Ks1, Vt1);
    load_chunk(c0 + 3, kreg1, vreg1);
    ring_fence();
    if (active) compute_chunk(c0, Ks, Vt);
    __syncthreads();
    if (c0 + 1 >= nchunks) break;
    if (c0 + 2 < nchunks) stage_chunk(kreg0, vreg0, Ks, Vt);
    load_chunk(c0 + 4, kreg0, vreg0);
    ring_fence();
    if (active) compute_chunk(c0 + 1, Ks1, Vt1);
    __syncthreads();
  }
  if (active && r_ < p.T) {
    float* rec = apart_at(p, blockIdx.x, w, r_);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      st_wt16(rec + dt * 16 + 4 * g_, __builtin_bit_cast(u32x4_t, o[dt]));
    if (g_ == 0) {
      const f32x4_t ml = {m_run, l_run, 0.0f, 0.0f};
      st_wt16(rec + D, __builtin_bit_cast(u32x4_t, ml));
    }
  }
}

// Merge of the split partials (log-sum-exp in base 2). One wave per
// (token, q head, 32 dims): lane l takes dim d0 + (l & 31) of the splits
// s = (l >> 5) + 2i, and lane s < S also holds split s's (m, l). The (m, l)
// words and the first kMergeChunk partials per lane are requested together;
// further splits (S > 2 * kMergeChunk) follow in a rolled loop. The split
// factors 2^(m_s - M) reach the lanes by lane exchange, and the two
// half-waves' sums meet in one exchange.
constexpr int kMergeChunk = 16;

template <bool debug>
__device__ __forceinline__ void merge_phase(const Params& p, const Smem& sm, const LayerW& lw) {
  const int D = p.d, Dq = p.nq * D, group = p.nq / p.nkv;
  const int lane = lane_id(), half = lane >> 5;
  const int qpr = D / 32;
  const int tasks = p.NT * p.nq * qpr;
  const int nw = gridDim.x * kWaves;
  for (int task = blockIdx.x * kWaves + wave_id(); task < tasks; task += nw) {
    const int row = task / qpr, dq = task - row * qpr;
    const int h = row % p.nq, tok = row / p.nq;
    const int r = tok / p.T, t = tok % p.T;
    const int g = h / group, w = h % group;
    int S;
    const int base = attn_item_base(p, sm, lw, r, g, gridDim.x, S);
    const int dim = dq * 32 + (lane & 31);
    const int nper = (S + 1) / 2;  // splits per half-wave (the odd half may have one fewer)
    float2 ml = *reinterpret_cast<const float2*>(apart_at(p, base + min(lane, S - 1), w, t) + D);
    float ov[kMergeChunk];
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) ov[i] = apart_at(p, base + min(half + 2 * i, S - 1), w, t)[dim];
    if (lane >= S) ml = make_float2(-INFINITY, 0.0f);
    float M = ml.x;
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float f = (ml.x == -INFINITY) ? 0.0f : exp2f(ml.x - M);
    float L = ml.y * f;
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    float O = 0.0f;
    for (int i0 = 0; i0 < nper; i0 += kMergeChunk) {
      if (i0 > 0) {
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) ov[i] = apart_at(p, base + min(half + 2 * (i0 + i), S - 1), w, t)[dim];
      }
#pragma unroll
      for (int i = 0; i < kMergeChunk; ++i) {
        const int sp = half + 2 * (i0 + i);
        const float fs = __shfl(f, min(sp, 63));
        O = fmaf(ov[i], sp < S ? fs : 0.0f, O);
      }
    }
    O += __shfl_xor(O, 32);
    if (half == 0) {
      const float out = O / L;
      st_wt(p.attn + (size_t)tok * Dq + h * D + dim, f2h(out));
      if (debug) if (p.dbg.attn) p.dbg.attn[(size_t)tok * Dq + h * D + dim] = out;
    }
  }
}

// ---------------------------------------------------------------------------
// Pooler input and router, from one pass over this workgroup's k-slice of h1.
// The pooler is split into S = p_slices equal k-slices and workgroup g's pool
// units all lie in slice g mod S, so its MFMA operand is needed only there.
// For every token t and k in the slice:
//   n2[k] = fl32(fl32(h1[k] * inv_rms[t]) * g[k])      (the fp32 router input)
//   X[t][k] = fp16(n2[k])                               (the pooler's MFMA operand)
// A router logit is a pairwise tree over partials j (the fma chain over
// k = 8j .. 8j+7, ascending), adjacent pairs first, plus the bias. A slice of
// H/S elements is an aligned subtree, so the router is split the same way:
// pair e*S + s is the subtree sum of expert e over slice s, workgroup g takes
// pairs g, g+G, g+2G, ... (all in its own slice, as G is a multiple of S),
// and routing adds the S subtree sums in tree order and then the bias.
// Thread (t, j) owns elements 8j .. 8j+7 of the slice: the first log2(64)
// tree levels are lane exchanges and the rest go through LDS. inv_rms comes
// from the O projection's per-tile partial sums of squares, requested
// together with the router rows and the first batch of h1.
// ---------------------------------------------------------------------------
// WIDE: the slice has at least 512 elements (K8 >= 64), so every wave holds
// 64 consecutive partials of one token per step and the token index and tree
// width are wave-uniform. RB: tokens whose router tree sums run back to back
// (the sums and their order are the same for every RB).
template <bool WIDE, int RB>
__device__ __forceinline__ void fill_x_pool_router(const Params& p, Smem& sm) {
  const int S = p.p_slices, G = gridDim.x, NT = p.NT, E = p.E;
  const int slice = (int)blockIdx.x % S;
  const int Ks = p.H / S, k0 = slice * Ks, K8 = Ks / 8;
  const int lane = lane_id();
  const int j8 = threadIdx.x % K8;
  const int tstep = kThreads / K8;
  const int nit = (kMaxTok + tstep - 1) / tstep;
  const int inwave = WIDE ? 64 : (K8 < 64 ? K8 : 64);
  const int t_base = WIDE ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / K8) : (int)threadIdx.x / K8;
  const int npairs = E * S;
  const int n_re = (int)blockIdx.x < npairs ? (npairs - 1 - (int)blockIdx.x) / G + 1 : 0;
  float* blk = &sm.red[0][0][0];  // [token][pair][64-element block] sums when K8 > 64
  const SsqLoads sq = ssq_issue(p, p.ssq1);
  float wv[kMaxRouterPerWg][8];
  int ev[kMaxRouterPerWg];
#pragma unroll
  for (int m = 0; m < kMaxRouterPerWg; ++m) {
    // rows past n_re repeat a valid row (unused), so every thread issues the
    // same loads
    ev[m] = min(((int)blockIdx.x + min(m, max(n_re - 1, 0)) * G) / S, E - 1);
    const float4* wp = reinterpret_cast<const float4*>(p.cur.w_router + (size_t)ev[m] * p.H + k0 + j8 * 8);
    const float4 a = wp[0], b = wp[1];
    wv[m][0] = a.x; wv[m][1] = a.y; wv[m][2] = a.z; wv[m][3] = a.w;
    wv[m][4] = b.x; wv[m][5] = b.y; wv[m][6] = b.z; wv[m][7] = b.w;
  }
  float gv[8];
  {
    const uint4 gg = *reinterpret_cast<const uint4*>(p.cur.g_moe + k0 + j8 * 8);
    const uint32_t gw[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) gv[j] = bf2f((uint16_t)(gw[j >> 1] >> ((j & 1) * 16)));
  }
  constexpr int B = 2 * kFillBatch;  // tokens of h1 per round trip
  float4 ha[B], hb[B];
  auto load_batch = [&](int it0) {
#pragma unroll
    for (int q = 0; q < B; ++q) {
      const int t = min(t_base + (it0 + q) * tstep, NT - 1);
      const float4* hp = reinterpret_cast<const float4*>(p.h1 + (size_t)t * p.H + k0 + j8 * 8);
      ha[q] = hp[0];
      hb[q] = hp[1];
    }
  };
  load_batch(0);
  ssq_finish(p, sq, sm);  // inv_rms of every token, from the partials requested first
  __syncthreads();
  for (int it0 = 0; it0 < nit; it0 += B) {
   if (it0 > 0) load_batch(it0);
   // Per token: normalise, write the fp16 tile, and run the router's fma
   // chains; then the lane tree sums of RB tokens back to back (independent
   // chains the scheduler can overlap, which branches between tokens would
   // prevent), and the sums are stored last. Tokens past NT are zero.
   static_assert(B % RB == 0, "token batch");
#pragma unroll
   for (int q0 = 0; q0 < B; q0 += RB) {
    float racc[RB][kMaxRouterPerWg];
#pragma unroll
    for (int qq = 0; qq < RB; ++qq) {
     const int q = q0 + qq;
     const int it = it0 + q;
     const int t = t_base + it * tstep;
     const bool live = it < nit && t < NT;
     const float4 a = ha[q], b = hb[q];
     float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
     if (p.use_norm) {
       const float inv = sm.inv_rms[min(t, kMaxTok - 1)];
#pragma unroll
       for (int j = 0; j < 8; ++j) v[j] = (v[j] * inv) * gv[j];
     }
#pragma unroll
     for (int j = 0; j < 8; ++j) v[j] = live ? v[j] : 0.0f;
     uint4 out;
     out.x = pack2(f2h(v[0]), f2h(v[1]));
     out.y = pack2(f2h(v[2]), f2h(v[3]));
     out.z = pack2(f2h(v[4]), f2h(v[5]));
     out.w = pack2(f2h(v[6]), f2h(v[7]));
     if (it < nit && t < kMaxTok) *reinterpret_cast<uint4*>(sm.x + t * x_stride(p.H) + (k0 + j8 * 8) * 2) = out;
#pragma unroll
     for (int m = 0; m < kMaxRouterPerWg; ++m) {
       float acc = 0.0f;
#pragma unroll
       for (int j = 0; j < 8; ++j) acc = fmaf(v[j], wv[m][j], acc);
       racc[qq][m] = acc;
     }
    }
#pragma unroll
    for (int qq = 0; qq < RB; ++qq)
#pragma unroll
     for (int m = 0; m < kMaxRouterPerWg; ++m)
       racc[qq][m] = WIDE ? lane_tree_sum(racc[qq][m], 64) : lane_tree_sum(racc[qq][m], inwave);
#pragma unroll
    for (int qq = 0; qq < RB; ++qq) {
     const int it = it0 + q0 + qq;
     if (it >= nit) break;
     const int t = t_base + it * tstep;
#pragma unroll
     for (int m = 0; m < kMaxRouterPerWg; ++m) {
       if (m >= n_re) break;
       if (K8 <= 64) {
         if (j8 == 0 && t < NT) st_wt(&p.logits[((size_t)slice * NT + t) * E + ev[m]], racc[qq][m]);
       } else if (lane == 0 && t < kMaxTok) {
         blk[(t * kMaxRouterPerWg + m) * 8 + j8 / 64] = racc[qq][m];
       }
     }
    }
   }
  }
  if (K8 > 64) {
    __syncthreads();
    const int nblk = K8 / 64;  // 2, 4 or 8
    for (int i = threadIdx.x; i < NT * n_re; i += kThreads) {
      const int t = i / n_re, m = i - t * n_re;
      float b[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) b[q] = q < nblk ? blk[(t * kMaxRouterPerWg + m) * 8 + q] : 0.0f;
      const float a0 = b[0] + b[1], a1 = b[2] + b[3], a2 = b[4] + b[5], a3 = b[6] + b[7];
      const float r = nblk == 2 ? a0 : (nblk == 4 ? a0 + a1 : (a0 + a1) + (a2 + a3));
      const int e = min(((int)blockIdx.x + m * G) / S, E - 1);
      st_wt(&p.logits[((size_t)slice * NT + t) * E + e], r);
    }
  }
  vm_drain();
  __syncthreads();
}

__device__ __forceinline__ void dump_n2(const Params& p, const Smem& sm) {
  for (int i = threadIdx.x; i < p.NT * p.H; i += kThreads) {
    const int t = i / p.H, k = i % p.H;
    float x = p.h1[i];
    if (p.use_norm) x = (x * sm.inv_rms[t]) * bf2f(p.cur.g_moe[k]);
    p.dbg.n2[i] = x;
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
  float ts_gu[kMaxTok * kMaxK];             // per selected slot: tensor scale of gate_up
  float ts_dn[kMaxTok * kMaxK];             // ... and of down
  int32_t count[kMaxE];                     // selections per expert (routing histogram)
  int32_t pos[kMaxE];                       // slot of a selected expert in sel, else -1
};

constexpr int kRouteOff = kMaxTok * (2048 * 2 + 16);  // after the pooled X (P <= 2048)
static_assert(kRouteOff + (int)sizeof(Route) <= kXBytes, "route tables must fit the X region");

__device__ __forceinline__ Route& route_of(Smem& sm) { return *reinterpret_cast<Route*>(sm.x + kRouteOff); }

// GEMM1's staging of SwiGLU outputs follows the route tables.
constexpr int kG1StageOff = (kRouteOff + (int)sizeof(Route) + 255) / 256 * 256;

// Order-preserving map of a finite fp32 value to uint32 (larger float =>
// larger key); key 0 is below every finite value.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v == 0.0f ? 0.0f : v);  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int popc64(uint64_t m) { return __builtin_popcountll(m); }

// Inverse of order_key on its image (-0 comes back as +0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide maximum (uniform result): DPP within 16-lane rows, then the four
// rows' maxima by read-lane.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Top-k by (logit descending, index ascending); gates = softmax of the
// selected logits. One wave per two tokens: the k entries are extracted one
// by one (wave-wide maximum of order-preserving keys, lowest index among
// equal keys), which ranks them as they come. The routing tables are then
// built without serial loops.
// The routing inputs of this thread: the logits of the wave's two tokens and
// the tensor scales of expert threadIdx.x, requested before the pooled
// activation fill so the round trips overlap.
constexpr int kTokPerWave = kMaxTok / kWaves;
constexpr int kMaxPSlices = 2;  // pooler / router k-slices

struct RouteLoads {
  float part[kTokPerWave][kMaxPSlices][kMaxE / 64];  // router subtree sums per k-slice
  float bias[kMaxE / 64];
  float ts_gu, ts_dn;
};

__device__ __forceinline__ RouteLoads routing_issue(const Params& p) {
  RouteLoads L;
  const int lane = lane_id(), w = wave_id(), E = p.E, NT = p.NT, S = p.p_slices;
#pragma unroll
  for (int tt = 0; tt < kTokPerWave; ++tt) {
    const int t = min(w + tt * kWaves, NT - 1);
#pragma unroll
    for (int s = 0; s < kMaxPSlices; ++s)
#pragma unroll
      for (int j = 0; j < kMaxE / 64; ++j)
        L.part[tt][s][j] = p.logits[((size_t)min(s, S - 1) * NT + t) * E + min(lane + j * 64, E - 1)];
  }
  const float* b = p.cur.b_router;
#pragma unroll
  for (int j = 0; j < kMaxE / 64; ++j) L.bias[j] = b ? b[min(lane + j * 64, E - 1)] : 0.0f;
  const int e = min((int)threadIdx.x, E - 1);
  L.ts_gu = p.cur.e_ts[2 * e];
  L.ts_dn = p.cur.e_ts[2 * e + 1];
  return L;
}

// Logit = the router's k-slice subtree sums combined in tree order, + bias.
__device__ __forceinline__ float route_logit(const RouteLoads& L, int S, int tt, int j) {
  const float* q = L.part[tt][0] + j;
  constexpr int J = kMaxE / 64;
  const float r = S == 1 ? q[0] : q[0] + q[J];
  return r + L.bias[j];
}

// The pooled-activation fill of the routing phase in two steps, so that its
// loads are in flight while the top-k runs: X = fp16 of the sum over the
// n <= kMaxPSlices slices of fp32 [n][NT][K], in slice order from +0 (the
// arithmetic of fill_x_sum), items as in fill_x_sum, kSumBatch items per
// thread per batch (two batches cover K <= 2048; the first is in flight during
// the top-k). Loads are unconditional
// (slice and token indices clamped in range).
constexpr int kSumBatch = 4;
static_assert(2 * kSumBatch * kThreads >= kMaxTok * 2048 / 8, "two batches cover the pooled tile");
struct SumLoads {
  float4 a[kMaxPSlices][kSumBatch], b[kMaxPSlices][kSumBatch];
};

__device__ __forceinline__ void fill_sum_issue(const float* parts, int n, int K, int NT, int i0, SumLoads& L) {
  const int K8 = K / 8;
#pragma unroll
  for (int u = 0; u < kMaxPSlices; ++u)
#pragma unroll
    for (int q = 0; q < kSumBatch; ++q) {
      const int i = i0 + q * kThreads;
      const int t = min(i / K8, NT - 1), k = (i % K8) * 8;
      const float4* src = reinterpret_cast<const float4*>(parts + ((size_t)min(u, n - 1) * NT + t) * K + k);
      L.a[u][q] = src[0];
      L.b[u][q] = src[1];
    }
}

__device__ __forceinline__ void fill_sum_finish(const SumLoads& L, int n, int K, int NT, int i0, Smem& sm) {
  const int K8 = K / 8, total = kMaxTok * K8;
#pragma unroll
  for (int q = 0; q < kSumBatch; ++q) {
    const int i = i0 + q * kThreads;
    if (i >= total) break;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kMaxPSlices; ++u) {
      if (u < n) {
        v[0] += L.a[u][q].x; v[1] += L.a[u][q].y; v[2] += L.a[u][q].z; v[3] += L.a[u][q].w;
        v[4] += L.b[u][q].x; v[5] += L.b[u][q].y; v[6] += L.b[u][q].z; v[7] += L.b[u][q].w;
      }
    }
    const int t = i / K8, k = (i % K8) * 8;
    uint4 out = make_uint4(0, 0, 0, 0);
    if (t < NT) {
      out.x = pack2(f2h(v[0]), f2h(v[1])); out.y = pack2(f2h(v[2]), f2h(v[3]));
      out.z = pack2(f2h(v[4]), f2h(v[5])); out.w = pack2(f2h(v[6]), f2h(v[7]));
    }
    *reinterpret_cast<uint4*>(sm.x + t * x_stride(K) + k * 2) = out;
  }
}

template <bool debug>
__device__ __forceinline__ void routing(const Params& p, Smem& sm, bool write_out, const RouteLoads& in) {
  Route& rt = route_of(sm);
  const int lane = lane_id(), w = __builtin_amdgcn_readfirstlane(wave_id());
  const int E = p.E, K = p.topk, NT = p.NT;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (threadIdx.x < kMaxE) {
    rt.count[threadIdx.x] = 0;
    rt.pos[threadIdx.x] = -1;
  }
  constexpr int TPW = kTokPerWave;
  float v[TPW][kMaxE / 64];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int j = 0; j < kMaxE / 64; ++j) v[tt][j] = route_logit(in, p.p_slices, tt, j);
  if (debug && p.dbg.logits && write_out) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      const int t = w + tt * kWaves;
#pragma unroll
      for (int j = 0; j < kMaxE / 64; ++j)
        if (t < NT && lane + j * 64 < E) p.dbg.logits[(size_t)t * E + lane + j * 64] = v[tt][j];
    }
  }
  __syncthreads();
  // Top-k by repeated extraction, both tokens of the wave interleaved: the
  // wave-wide largest key, and among equal keys the lowest expert index
  // (index = lane + 64 j, so the first j with a hit, then its lowest lane),
  // is taken and removed, K times. The extraction order is the ranking
  // (value descending, index ascending); rank r's expert and logit end up in
  // lane r.
  uint32_t key[TPW][kMaxE / 64];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const bool live = w + tt * kWaves < NT;
#pragma unroll
    for (int j = 0; j < kMaxE / 64; ++j) key[tt][j] = (live && lane + j * 64 < E) ? order_key(v[tt][j]) : 0u;
  }
  int rid[TPW];
  float rval[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    rid[tt] = 0;
    rval[tt] = 0.0f;
  }
#pragma unroll
  for (int r = 0; r < kMaxK; ++r) {
    if (r >= K) break;
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      uint32_t lm = key[tt][0];
#pragma unroll
      for (int j = 1; j < kMaxE / 64; ++j) lm = max(lm, key[tt][j]);
      const uint32_t m = wave_max_u32(lm);
      int jsel = kMaxE / 64, lsel = 0;
#pragma unroll
      for (int j = kMaxE / 64 - 1; j >= 0; --j) {
        const uint64_t hit = __ballot(key[tt][j] == m);
        if (hit) {
          jsel = j;
          lsel = __builtin_ctzll(hit);
        }
      }
#pragma unroll
      for (int j = 0; j < kMaxE / 64; ++j)
        if (j == jsel && lane == lsel) key[tt][j] = 0u;
      if (lane == r) {
        rid[tt] = lsel + 64 * jsel;
        rval[tt] = key_value(m);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int t = w + tt * kWaves;
    if (t >= NT) break;
    // gates: softmax of the selected logits, max-subtracted, summed in rank order
    const float mx = readlane_f32(rval[tt], 0);
    const float ev = expf(rval[tt] - mx);
    float ssum = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxK; ++q)
      if (q < K) ssum += readlane_f32(ev, q);
    if (lane < K) {
      rt.ids[t][lane] = rid[tt];
      rt.gates[t][lane] = ev / ssum;
    }
  }
  __syncthreads();
  // histogram and membership
  if (threadIdx.x < NT * K) {
    const int t = threadIdx.x / K, r = threadIdx.x % K;
    atomicAdd(&rt.count[rt.ids[t][r]], 1);
  }
  __syncthreads();
  // selected set in ascending expert order: wave 0 ranks the experts with a
  // nonzero count (lane l holds experts l, l+64, l+128, l+192)
  if (w == 0) {
    int base = 0;
#pragma unroll
    for (int j = 0; j < kMaxE / 64; ++j) {
      const int e = lane + j * 64;
      const bool used = e < E && rt.count[e] > 0;
      const uint64_t m = __ballot(used);
      if (used) {
        const int q = base + popc64(m & lt_mask);
        rt.sel[q] = e;
        rt.pos[e] = q;
      }
      base += popc64(m);
    }
    if (lane == 0) rt.n_sel = base;
  }
  __syncthreads();
  const int n_sel = rt.n_sel;
  for (int i = threadIdx.x; i < n_sel * kMaxTok; i += kThreads) (&rt.tokgate[0][0])[i] = 0.0f;
  if (threadIdx.x < E && rt.pos[threadIdx.x] >= 0) {
    rt.ts_gu[rt.pos[threadIdx.x]] = in.ts_gu;
    rt.ts_dn[rt.pos[threadIdx.x]] = in.ts_dn;
  }
  __syncthreads();
  if (threadIdx.x < NT * K) {
    const int t = threadIdx.x / K, r = threadIdx.x % K;
    rt.tokgate[rt.pos[rt.ids[t][r]]][t] = rt.gates[t][r];
    if (write_out) {
      if (p.out_ids) p.out_ids[t * K + r] = rt.ids[t][r];
      if (p.out_gates) p.out_gates[t * K + r] = rt.gates[t][r];
    }
  }
  if (write_out && p.hist_wr && threadIdx.x < E) {
    int32_t* hw = p.hist_wr + (size_t)p.layer * E + threadIdx.x;
    *hw = rt.count[threadIdx.x] + (p.hist_add ? *hw : 0);
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
// Unit = (selected slot j, i-tile it): gate rows it*8 .. +8 and up rows
// I + it*8 .. +8 as the 16 MFMA columns, contracted over the whole pooled
// dim P by one wave in P/128 steps (lane group g holds the 32 elements at
// step*128 + g*32 of its row, the A operand the same k of the 16 tokens).
// A workgroup owns a contiguous range of units and wave w takes every 8th
// unit of it, so no partial sums cross waves. Each wave's loads run
// kG1Ring steps ahead over its flat (unit, step) sequence, across unit
// boundaries; the SwiGLU outputs are staged in LDS and written out once at
// the end of the phase, so the loop issues nothing but loads and MFMA.
constexpr int kG1Ring = 8;  // steps of loads in flight per wave
static_assert(kG1StageOff + kG1StageBytes <= kXBytes, "GEMM1 staging must fit the X region");

struct G1Step {
  uint4 c;     // 32 E2M1 codes of the lane's row
  uint32_t s;  // their two E4M3 block scales (low 16 bits)
};

// Issue cursor over a wave's (unit, step) sequence, with the lane's row
// pointers of the current unit (recomputed once per unit).
struct G1Issue {
  int m, st;            // unit ordinal (wave-uniform), step in the unit
  const uint8_t* code;  // codes of the lane's row, at the lane group's 16-byte offset
  const uint8_t* scale; // scales of the lane's row, at the lane group's 2-byte offset
};

__device__ __forceinline__ void g1_point(const Params& p, const Route& rt, int u, G1Issue& is) {
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4;
  const int I = p.I, P = p.P, ntile = I / 8;
  const int j = u / ntile, it = u - j * ntile;
  const int e = __builtin_amdgcn_readfirstlane(rt.sel[j]);
  const int row = r_ < 8 ? it * 8 + r_ : I + it * 8 + (r_ - 8);
  const size_t r_all = (size_t)e * (2 * I) + row;
  is.code = p.cur.e_gu + r_all * (P / 2) + g_ * 16;
  is.scale = p.cur.e_gu_sc + r_all * (P / 16) + g_ * 2;
}

// GEMM1 with 16 steps per unit (P = 2048), the loop unrolled over one unit:
// ring slot, step, A-operand offset and epilogue position are compile-time.
// The block scales of a unit (16 rows x 128 B) are read once, with two
// 16-byte loads per lane (lane group g: bytes g*32 .. g*32+31 of its row),
// when the issue cursor enters the unit; a step takes its two bytes from
// the lane that holds them (ds_bpermute). This replaces a 2-byte scale load
// per step, which touched 16 cache lines for 8 bytes each.
constexpr int kG1UnitSteps = 16;
static_assert(kG1UnitSteps == 2 * kG1Ring, "the issue cursor enters the next unit at step 8");

__device__ __forceinline__ void g1_unit_scales(const G1Issue& is, uint4 (&sc)[2]) {
  const int g_ = lane_id() >> 4;
  // is.scale points at the lane group's 2-byte offset g*2; the row starts g*2 earlier
  const uint8_t* row = is.scale - g_ * 2;
  sc[0] = *reinterpret_cast<const uint4*>(row + g_ * 32);
  sc[1] = *reinterpret_cast<const uint4*>(row + g_ * 32 + 16);
}

template <int ST>
__device__ __forceinline__ uint32_t g1_step_scale(const uint4 (&sc)[2]) {
  // bytes ST*8 + 2g .. +1 of the lane's row: held by lane group ST/4, dword
  // (ST%4)*2 + g/2 of its 32 bytes, half g%2
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4;
  constexpr int d0 = (ST & 3) * 2;
  const uint32_t w0[8] = {sc[0].x, sc[0].y, sc[0].z, sc[0].w, sc[1].x, sc[1].y, sc[1].z, sc[1].w};
  const int src = (r_ + 16 * (ST >> 2)) * 4;
  const uint32_t x0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)w0[d0]);
  const uint32_t x1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)w0[d0 + 1]);
  const uint32_t x = (g_ >> 1) ? x1 : x0;
  return (x >> ((g_ & 1) * 16)) & 0xFFFFu;
}

// SwiGLU epilogue of one GEMM1 unit (local ordinal ul, selected slot j).
// acc[q] = D[token 4g+q][column r]: gate (r < 8) or up (r >= 8) of i-row
// it*8 + (r & 7). Without activation quantization the staged value is
// fp16(a * gate weight), 256 B per unit; with it, the fp32 SwiGLU output a
// itself, 512 B per unit, quantized block by block in the flush.
__device__ __forceinline__ void g1_epilogue(const Params& p, const Route& rt, uint8_t* stage, int ul, int j,
                                            f32x4_t acc) {
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4;
  const float ts = rt.ts_gu[j];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float up = __shfl_xor(acc[q], 8);
    const int tok = 4 * g_ + q;
    if (r_ < 8) {
      const float gate = acc[q] * ts;
      const float a = gate / (1.0f + expf(-gate)) * (up * ts);
      if (p.act_fp4) {
        reinterpret_cast<float*>(stage + (size_t)ul * 512)[tok * 8 + r_] = a;
      } else {
        reinterpret_cast<uint16_t*>(stage + (size_t)ul * 256)[tok * 8 + r_] = f2h(a * rt.tokgate[j][tok]);
      }
    }
  }
}

// NVFP4 quantization of the SwiGLU output (orcarouter.ai, "Dove si colloca il
// confine del kernel": the activations leave the first expert GEMM as fp4).
// One block = 16 consecutive fp32 values along the expert's intermediate
// dim. Block scale s = E4M3(amax / 6), nearest even, saturating at 448;
// code = E2M1(x / s), nearest even, saturating at 6, sign kept (0 when
// s = 0); value = E2M1(code) * s, exact in fp32.
//
// fp32 -> OCP E4M3FN code for x >= 0.
__device__ __forceinline__ uint32_t e4m3_code_rne_sat(float x) {
  if (!(x > 0.0f)) return 0u;
  if (x >= 448.0f) return 0x7Eu;
  if (x < 0.015625f) return (uint32_t)__builtin_rintf(x * 512.0f);  // 2^-9 grid; 8 is the smallest normal
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7FFFFu + ((u >> 20) & 1u);  // significand to 3 bits, ties to even (a carry bumps the exponent)
  return min((((u >> 23) - 120u) << 3) | ((u >> 20) & 7u), 0x7Eu);  // exponent bias 127 -> 7
}

// fp32 -> E2M1 code (bit 3 = sign). On [0,2) the grid is 0.5, on [2,4) it
// is 1, from 4 on it is 2 (only 4 and 6 exist).
__device__ __forceinline__ uint32_t e2m1_code_rne_sat(float y) {
  const uint32_t sgn = (__builtin_bit_cast(uint32_t, y) >> 28) & 8u;
  const float a = fminf(fabsf(y), 8.0f);
  uint32_t c;
  if (a < 2.0f) c = (uint32_t)__builtin_rintf(a * 2.0f);
  else if (a < 4.0f) c = 2u + (uint32_t)__builtin_rintf(a);
  else c = min(4u + (uint32_t)__builtin_rintf(a * 0.5f), 7u);
  return sgn | c;
}

// E2M1 code -> value (twice the magnitude of codes 0..7 is 0,1,2,3,4,6,8,12).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const float m = (float)((0xC8643210u >> ((c & 7u) * 4u)) & 15u) * 0.5f;
  return (c & 8u) ? -m : m;
}

template <bool debug>
__device__ __forceinline__ void gemm1_units16(const Params& p, Smem& sm, const Route& rt, int u0, int my_units,
                                              int w) {
  uint8_t* stage = sm.x + kG1StageOff;
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4;
  const int I = p.I, P = p.P, ntile = I / 8;
  uint4 ring[kG1Ring];
  G1Issue is{0, 0, nullptr, nullptr};
  g1_point(p, rt, u0 + w, is);
  uint4 scn[2], scc[2];
  g1_unit_scales(is, scn);
  ring_fence();
#pragma unroll
  for (int i = 0; i < kG1Ring; ++i) {
    ring[i] = *reinterpret_cast<const uint4*>(is.code + i * 64);
    ring_fence();
  }
  const uint8_t* abase = sm.x + r_ * x_stride(P) + g_ * 64;
  for (int m = 0; m < my_units; ++m) {
    scc[0] = scn[0];
    scc[1] = scn[1];
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int u = u0 + w + kWaves * m;
    const int j = u / ntile, it = u - j * ntile;
#define G1_STEP(ST)                                                                                   \
    {                                                                                                 \
      uint4 bw[4];                                                                                    \
      fp4_decode(ring[(ST) & (kG1Ring - 1)], g1_step_scale<(ST)>(scc), bw);                          \
      _Pragma("unroll") for (int q = 0; q < 4; ++q)                                                   \
        acc = mfma_f16(*reinterpret_cast<const uint4*>(abase + (ST) * 256 + q * 16), bw[q], acc);    \
      if constexpr (debug) {                                                                          \
        if (p.dbg.dq_gu && rt.sel[j] == p.dbg.dq_expert) {                                            \
          const int row = r_ < 8 ? it * 8 + r_ : I + it * 8 + (r_ - 8);                               \
          uint4* dst = reinterpret_cast<uint4*>(p.dbg.dq_gu + (size_t)row * P + (ST) * 128 + g_ * 32); \
          _Pragma("unroll") for (int q = 0; q < 4; ++q) dst[q] = bw[q];                               \
        }                                                                                             \
      }                                                                                               \
      if ((ST) == kG1Ring && m + 1 < my_units) g1_point(p, rt, u + kWaves, is);                       \
      if ((ST) == kG1Ring) g1_unit_scales(is, scn);                                                   \
      ring[(ST) & (kG1Ring - 1)] = *reinterpret_cast<const uint4*>(is.code + (((ST) + kG1Ring) & 15) * 64); \
      ring_fence();                                                                                   \
    }
    G1_STEP(0) G1_STEP(1) G1_STEP(2) G1_STEP(3) G1_STEP(4) G1_STEP(5) G1_STEP(6) G1_STEP(7)
    G1_STEP(8) G1_STEP(9) G1_STEP(10) G1_STEP(11) G1_STEP(12) G1_STEP(13) G1_STEP(14) G1_STEP(15)
#undef G1_STEP
    g1_epilogue(p, rt, stage, u - u0, j, acc);
  }
}

template <bool debug>
__device__ __forceinline__ void gemm1_phase(const Params& p, Smem& sm) {
  Route& rt = route_of(sm);
  uint8_t* stage = sm.x + kG1StageOff;
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  const int I = p.I, P = p.P, ntile = I / 8, nsteps = P / 128;
  const int U = rt.n_sel * ntile;
  // with activation quantization a workgroup owns whole pairs of units (one
  // 16-wide block of the intermediate dim; ntile is even, so a pair never
  // spans two experts)
  const int pu = p.act_fp4 ? 2 : 1;
  const int u0 = pu * (int)((long long)blockIdx.x * (U / pu) / gridDim.x);
  const int u1 = pu * (int)((long long)(blockIdx.x + 1) * (U / pu) / gridDim.x);
  const int my_units = (u1 - u0 - w + kWaves - 1) / kWaves;  // units u0 + w + 8*m < u1
  const int total = my_units > 0 ? my_units * nsteps : 0;
  if (total > 0 && nsteps == kG1UnitSteps) {
    gemm1_units16<debug>(p, sm, rt, u0, my_units, w);
  } else if (total > 0) {
    G1Step ring[kG1Ring];
    G1Issue is{0, 0, nullptr, nullptr};
    g1_point(p, rt, u0 + w, is);
    // loads of the step at the cursor; past the wave's last step the cursor
    // stays on that step (in-bounds reloads)
    auto issue_next = [&](G1Step& slot) {
      slot.c = *reinterpret_cast<const uint4*>(is.code + is.st * 64);
      slot.s = *reinterpret_cast<const uint16_t*>(is.scale + is.st * 8);
      if (is.st + 1 < nsteps) {
        ++is.st;
      } else if (is.m + 1 < my_units) {
        is.st = 0;
        ++is.m;
        g1_point(p, rt, u0 + w + kWaves * is.m, is);
      }
    };
#pragma unroll
    for (int i = 0; i < kG1Ring; ++i) {
      issue_next(ring[i]);
      ring_fence();
    }
    const uint8_t* abase = sm.x + r_ * x_stride(P) + g_ * 64;
    int cm = 0, cst = 0;  // compute cursor
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int base = 0; base < total; base += kG1Ring) {
#pragma unroll
      for (int i = 0; i < kG1Ring; ++i) {
        if (base + i < total) {
          uint4 bw[4];
          fp4_decode(ring[i].c, ring[i].s, bw);
          const uint8_t* ap = abase + cst * 256;
#pragma unroll
          for (int q = 0; q < 4; ++q) acc = mfma_f16(*reinterpret_cast<const uint4*>(ap + q * 16), bw[q], acc);
          if constexpr (debug) {
            const int u = u0 + w + kWaves * cm, j = u / ntile, it = u - j * ntile;
            if (p.dbg.dq_gu && rt.sel[j] == p.dbg.dq_expert) {
              const int row = r_ < 8 ? it * 8 + r_ : I + it * 8 + (r_ - 8);
              uint4* dst = reinterpret_cast<uint4*>(p.dbg.dq_gu + (size_t)row * P + cst * 128 + g_ * 32);
#pragma unroll
              for (int q = 0; q < 4; ++q) dst[q] = bw[q];
            }
          }
          if (cst == nsteps - 1) {
            const int u = u0 + w + kWaves * cm, j = u / ntile;
            g1_epilogue(p, rt, stage, u - u0, j, acc);
            acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
            cst = 0;
            ++cm;
          } else {
            ++cst;
          }
        }
        issue_next(ring[i]);
        ring_fence();
      }
    }
  }
  __syncthreads();
  const int NT = p.NT;
  if (p.act_fp4) {
    // quantize: one (unit pair, token) block of 16 per item: 8 B of E2M1
    // codes to acode[j][token][it*4 ..] and the E4M3 block scale to
    // ascale[j][token][it/2] (the gate weight is applied after the down
    // projection)
    for (int q = threadIdx.x; q < (u1 - u0) / 2 * NT; q += kThreads) {
      const int pl = q / NT, tok = q - pl * NT;
      const int u = u0 + 2 * pl, j = u / ntile, it = u - j * ntile;
      const float* s0 = reinterpret_cast<const float*>(stage + (size_t)(2 * pl) * 512) + tok * 8;
      const float* s1 = reinterpret_cast<const float*>(stage + (size_t)(2 * pl + 1) * 512) + tok * 8;
      float x[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = s0[i];
        x[8 + i] = s1[i];
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
      const uint32_t sc = e4m3_code_rne_sat(amax / 6.0f);
      const float s = __builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
      uint32_t codes[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t c = e2m1_code_rne_sat(s > 0.0f ? x[i] / s : 0.0f);
        codes[i >> 3] |= c << ((i & 7) * 4);
      }
      const size_t row = (size_t)j * NT + tok;
      __hip_atomic_store(reinterpret_cast<uint64_t*>(p.acode + row * (I / 2) + it * 4),
                         (uint64_t)codes[0] | ((uint64_t)codes[1] << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ascale + row * (I / 16) + it / 2, (uint8_t)sc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if constexpr (debug) {
        if (p.dbg.act_codes_all) {
          const size_t row = (size_t)rt.sel[j] * NT + tok;
          *reinterpret_cast<uint2*>(p.dbg.act_codes_all + row * (I / 2) + it * 4) = make_uint2(codes[0], codes[1]);
          p.dbg.act_sc_all[row * (I / 16) + it / 2] = (uint8_t)sc;
        }
        if (p.dbg.act && rt.sel[j] == p.dbg.dq_expert) {
#pragma unroll
          for (int i = 0; i < 16; ++i) p.dbg.act[(size_t)tok * I + it * 8 + i] = x[i];
          *reinterpret_cast<uint2*>(p.dbg.act_codes + (size_t)tok * (I / 2) + it * 4) = make_uint2(codes[0], codes[1]);
          p.dbg.act_sc[(size_t)tok * (I / 16) + it / 2] = (uint8_t)sc;
        }
      }
    }
  } else {
    // 16 B per (unit, token) to abuf[j][token][it*8 .. +8]
    for (int q = threadIdx.x; q < (u1 - u0) * NT; q += kThreads) {
      const int ul = q / NT, tok = q - ul * NT;
      const int u = u0 + ul, j = u / ntile, it = u - j * ntile;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + (size_t)ul * 256 + tok * 16);
      st_wt16(p.abuf + ((size_t)j * NT + tok) * I + it * 8, v);
    }
  }
  __syncthreads();
}

// GEMM2: down projection, summed over a contiguous range of selected experts.
// Workgroup = (row tile of 16 of P, expert part); wave w owns k in
// [w*128, w*128+128) of I (lane group g: 32 elements at w*128 + g*32). The A
// operand of a token not routed to the expert (or of k beyond I) is zero
// without a load; the weight loads are the same for every expert. Per
// expert the fp32 tensor scale is applied to the MFMA partial before it is
// added to the running sum.
constexpr int kG2Ring = 4;  // GEMM2 experts whose loads are in flight per wave

struct G2Slot {
  uint4 c;
  uint32_t s;
  uint4 a[4];
};

__device__ __forceinline__ void g2_issue(const Params& p, const Route& rt, int j, int tile, G2Slot& b) {
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int I = p.I, P = p.P;
  const int e = rt.sel[j];
  const int k = w * 128 + g_ * 32;
  const bool kv = k < I;
  const int kk = kv ? k : 0;
  const int row = tile * 16 + r_;
  b.c = *reinterpret_cast<const uint4*>(p.cur.e_dn + (size_t)e * P * (I / 2) + (size_t)row * (I / 2) + kk / 2);
  // tiled scales: this wave's 16 rows x 8 bytes of (e, tile) are one line
  const int nsl = dn_scale_slices(I);
  b.s = *reinterpret_cast<const uint16_t*>(p.cur.e_dn_sc + (((size_t)e * (P / 16) + tile) * nsl + min(w, nsl - 1)) * 128 +
                                           r_ * 8 + g_ * 2);
  // Only lanes of tokens routed to the expert load their A fragment; the
  // rest are zero without a memory access.
  const bool routed = kv && r_ < p.NT && rt.tokgate[j][r_] != 0.0f;
  if (routed) {
    const uint16_t* src = p.abuf + ((size_t)j * p.NT + r_) * I + k;
#pragma unroll
    for (int q = 0; q < 4; ++q) b.a[q] = *reinterpret_cast<const uint4*>(src + q * 8);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) b.a[q] = make_uint4(0, 0, 0, 0);
  }
}

// GEMM2 with NVFP4 activations: the A operand is read as E2M1 codes (16 B)
// and two E4M3 block scales per lane and expert, a quarter of the fp16
// bytes, and decoded like the weights (exact in fp16); the ring holds
// kG2Ring4 experts. The gate weight of each token multiplies the fp32 MFMA
// output together with the tensor scale. Four experts in flight ran the
// 62-layer step 0.03 ms faster than six (the deeper ring's registers cost
// more elsewhere than its extra loads in flight gain); eight spill.
constexpr int kG2Ring4 = 4;

struct G2Slot4 {
  uint4 c;
  uint32_t s;
  uint4 ac;
  uint32_t as;
};

__device__ __forceinline__ void g2_issue4(const Params& p, const Route& rt, int j, int tile, G2Slot4& b) {
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int I = p.I, P = p.P;
  const int e = rt.sel[j];
  const int k = w * 128 + g_ * 32;
  const bool kv = k < I;
  const int kk = kv ? k : 0;
  const int row = tile * 16 + r_;
  b.c = *reinterpret_cast<const uint4*>(p.cur.e_dn + (size_t)e * P * (I / 2) + (size_t)row * (I / 2) + kk / 2);
  const int nsl = dn_scale_slices(I);
  b.s = *reinterpret_cast<const uint16_t*>(p.cur.e_dn_sc + (((size_t)e * (P / 16) + tile) * nsl + min(w, nsl - 1)) * 128 +
                                           r_ * 8 + g_ * 2);
  const bool routed = kv && r_ < p.NT && rt.tokgate[j][r_] != 0.0f;
  if (routed) {
    const size_t arow = (size_t)j * p.NT + r_;
    b.ac = *reinterpret_cast<const uint4*>(p.acode + arow * (I / 2) + k / 2);
    b.as = *reinterpret_cast<const uint16_t*>(p.ascale + arow * (I / 16) + k / 16);
  } else {
    b.ac = make_uint4(0, 0, 0, 0);
    b.as = 0u;
  }
}

template <bool debug>
__device__ __forceinline__ f32x4_t gemm2_fp4_loop(const Params& p, const Route& rt, int tile, int j0, int j1) {
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int I = p.I;
  f32x4_t total = {0.f, 0.f, 0.f, 0.f};
  G2Slot4 ring[kG2Ring4];
#pragma unroll
  for (int i = 0; i < kG2Ring4; ++i) {
    g2_issue4(p, rt, min(j0 + i, j1 - 1), tile, ring[i]);
    ring_fence();
  }
  for (int base = j0; base < j1; base += kG2Ring4) {
#pragma unroll
    for (int i = 0; i < kG2Ring4; ++i) {
      const int jj = base + i;
      const int jc = min(jj, j1 - 1);
      uint4 av[4], bw[4];
      fp4_decode(ring[i].ac, ring[i].as, av);
      fp4_decode(ring[i].c, ring[i].s, bw);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = mfma_f16(av[q], bw[q], acc);
      // acc[c] is token 4g+c of row r: its gate weight times the tensor scale
      const float ts = jj < j1 ? rt.ts_dn[jc] : 0.0f;
      const float4 gt = *reinterpret_cast<const float4*>(&rt.tokgate[jc][4 * g_]);
      total[0] = fmaf(acc[0], ts * gt.x, total[0]);
      total[1] = fmaf(acc[1], ts * gt.y, total[1]);
      total[2] = fmaf(acc[2], ts * gt.z, total[2]);
      total[3] = fmaf(acc[3], ts * gt.w, total[3]);
      if constexpr (debug) {
        const int e = rt.sel[jc];
        const int k = w * 128 + g_ * 32;
        if (jj < j1 && k < I && p.dbg.dq_dn && e == p.dbg.dq_expert) {
          uint4* dst = reinterpret_cast<uint4*>(p.dbg.dq_dn + (size_t)(tile * 16 + r_) * I + k);
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[q] = bw[q];
        }
      }
      g2_issue4(p, rt, min(jj + kG2Ring4, j1 - 1), tile, ring[i]);
      ring_fence();
    }
  }
  return total;
}

template <bool debug>
__device__ __forceinline__ void gemm2_phase(const Params& p, Smem& sm) {
  Route& rt = route_of(sm);
  const int lane = lane_id(), r_ = lane & 15, g_ = lane >> 4, w = wave_id();
  const int I = p.I, P = p.P;
  const int tiles = P / 16;
  const int parts = max(1, (int)gridDim.x / tiles);
  if ((int)blockIdx.x >= tiles * parts) return;
  const int tile = blockIdx.x % tiles, part = blockIdx.x / tiles;
  const int j0 = part * rt.n_sel / parts, j1 = (part + 1) * rt.n_sel / parts;
  f32x4_t total = {0.f, 0.f, 0.f, 0.f};
  if (j0 < j1 && p.act_fp4) {
    total = gemm2_fp4_loop<debug>(p, rt, tile, j0, j1);
  } else if (j0 < j1) {
    G2Slot ring[kG2Ring];
#pragma unroll
    for (int i = 0; i < kG2Ring; ++i) {
      g2_issue(p, rt, min(j0 + i, j1 - 1), tile, ring[i]);
      ring_fence();
    }
    for (int base = j0; base < j1; base += kG2Ring) {
#pragma unroll
      for (int i = 0; i < kG2Ring; ++i) {
        const int jj = base + i;
        const int jc = min(jj, j1 - 1);
        uint4 bw[4];
        fp4_decode(ring[i].c, ring[i].s, bw);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = mfma_f16(ring[i].a[q], bw[q], acc);
        const float ts = jj < j1 ? rt.ts_dn[jc] : 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) total[c] = fmaf(acc[c], ts, total[c]);
        if constexpr (debug) {
          const int e = rt.sel[jc];
          const int k = w * 128 + g_ * 32;
          if (jj < j1 && k < I && p.dbg.dq_dn && e == p.dbg.dq_expert) {
            uint4* dst = reinterpret_cast<uint4*>(p.dbg.dq_dn + (size_t)(tile * 16 + r_) * I + k);
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = bw[q];
          }
        }
        g2_issue(p, rt, min(jj + kG2Ring, j1 - 1), tile, ring[i]);
        ring_fence();
      }
    }
  }
  red_store(sm, 0, total);
  __syncthreads();
  if (threadIdx.x < 256) {
    const int tok = threadIdx.x >> 4, row = threadIdx.x & 15;
    float v = red_sum(sm, 0, threadIdx.x);
    if (tok < p.NT) st_wt(&p.accpart[((size_t)part * p.NT + tok) * P + tile * 16 + row], v);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------

enum Variant { kPlain = 0, kDebug = 1, kTrace = 2 };

// ---------------------------------------------------------------------------
// Speculative expert prefetch. The layer's experts are ranked by how often the
// previous call selected them (the routing histogram of that call, count
// descending, index ascending) and the first n_prefetch are read once by the
// workgroups that have no attention work, so their codes and scales are in
// the memory-side cache when the expert phase of this launch reads them.
// ---------------------------------------------------------------------------
// Wave 0 writes the ranking to sm.plist (callers meet on a barrier before use).
__device__ __forceinline__ void prefetch_rank(const Params& p, Smem& sm) {
  if (wave_id() != 0) return;
  const int lane = lane_id(), E = p.E, P = p.n_prefetch;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t* cnt = p.hist_rd + (size_t)p.layer * E;
  uint32_t key[kMaxE / 64];
#pragma unroll
  for (int j = 0; j < kMaxE / 64; ++j) {
    const int e = lane + j * 64;
    // count in the high bits, 255 - e in the low byte: unique keys, larger =
    // earlier in the ranking; 0 for e >= E (below every real key)
    key[j] = e < E ? ((uint32_t)cnt[e] << 8) | (uint32_t)(255 - e) : 0u;
  }
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = T | (1u << b);
    int c = 0;
#pragma unroll
    for (int j = 0; j < kMaxE / 64; ++j) c += popc64(__ballot(key[j] >= cand));
    if (c >= P) T = cand;
  }
  // the P keys >= T, ranked by key (descending)
  int base = 0;
  uint32_t* scr = reinterpret_cast<uint32_t*>(&sm.red[1][0][0]);
#pragma unroll
  for (int j = 0; j < kMaxE / 64; ++j) {
    const bool sel = key[j] >= T && key[j] != 0u;
    const uint64_t m = __ballot(sel);
    if (sel) scr[base + popc64(m & lt_mask)] = key[j];
    base += popc64(m);
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < P) {
    const uint32_t mine = scr[lane];
    int rank = 0;
    for (int q = 0; q < P; ++q) rank += scr[q] > mine ? 1 : 0;
    sm.plist[rank] = 255 - (int)(mine & 0xFFu);
  }
}

// Reads one dword of every 128-byte line of the listed experts' gate/up and
// down codes and scales; the workgroup is number `idx` of `n` prefetchers.
__device__ __forceinline__ void prefetch_experts(const Params& p, const Smem& sm, int idx, int n) {
  const size_t I = p.I, P = p.P;
  const size_t bytes[4] = {2 * I * P / 2, 2 * I * P / 16, P * I / 2, P * (size_t)dn_scale_slices(p.I) * 8};
  const uint8_t* base[4] = {p.cur.e_gu, p.cur.e_gu_sc, p.cur.e_dn, p.cur.e_dn_sc};
  int lines[4], lpe = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    lines[r] = (int)((bytes[r] + 127) / 128);
    lpe += lines[r];
  }
  const int total = p.n_prefetch * lpe;
  uint32_t acc = 0;
  for (int l0 = idx * kThreads + threadIdx.x; l0 < total; l0 += 4 * n * kThreads) {
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int l = min(l0 + q * n * kThreads, total - 1);
      const int j = l / lpe;
      int r = l - j * lpe, reg = 0;
#pragma unroll
      for (int t = 0; t < 3; ++t)
        if (reg == t && r >= lines[t]) { r -= lines[t]; reg = t + 1; }
      const size_t off = min((size_t)r * 128, bytes[reg] - 4);
      v[q] = *reinterpret_cast<const uint32_t*>(base[reg] + (size_t)sm.plist[j] * bytes[reg] + off);
    }
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // never true (layer >= 0); keeps the loads
  if (p.layer < 0 && acc == 0x9E3779B9u) p.err[1] = (int32_t)acc;
}

// Reads one dword of every 128-byte line of the prior K and V rows that the
// next layer's attention will read (the window of every request and kv
// head; the verify tokens' own rows are being written in this phase and are
// left alone), so that the next launch finds them in the memory-side cache.
// This workgroup takes lines blockIdx.x, blockIdx.x + G, ... of the list.
__device__ __forceinline__ void prefetch_next_kv(const Params& p, const Smem& sm) {
  const LayerW& lw = p.nxt;
  const int lines_per_row = p.d * 2 / 128;  // 1 (d = 64) or 2 (d = 128)
  uint32_t acc = 0;
  int done = 0;  // lines of earlier (request, kv head) ranges
  for (int r = 0; r < p.R; ++r) {
    const int ctx = ctx_uni(sm, r);
    const int lo = lw.window > 0 ? max(0, ctx - lw.window + 1) : 0;
    const int nrows = max(0, ctx - lo);  // prior rows only
    const int nl = nrows * lines_per_row;
    for (int g = 0; g < p.nkv; ++g) {
      const size_t row0 = ((size_t)r * p.nkv + g) * p.cap + lo;
      for (int l = (int)(blockIdx.x * kThreads + threadIdx.x) - done; l < 2 * nl; l += gridDim.x * kThreads) {
        if (l < 0) continue;
        const uint16_t* base = l < nl ? lw.k_cache : lw.v_cache;
        const int ll = l < nl ? l : l - nl;
        acc ^= *reinterpret_cast<const uint32_t*>(base + (row0 + ll / lines_per_row) * p.d + (ll % lines_per_row) * 64);
      }
      done += 2 * nl;
      done %= gridDim.x * kThreads;
    }
  }
  // never true (layer >= 0); keeps the loads
  if (p.layer < 0 && acc == 0x9E3779B9u) p.err[1] = (int32_t)acc;
}

// Device error codes (the numbers of the matching msk_status values).
constexpr int32_t kErrInvalid = 1;   // a token mask breaks the tree rules, or ctx_len < 0
constexpr int32_t kErrCapacity = 5;  // ctx_len + n_tokens > kv_capacity

// Launch prologue: this workgroup's units of every dense schedule, the pass's
// context lengths and token masks, and the device error word, all read from
// device memory in one round trip (every load is unconditional with a
// clamped index, and the LDS writes follow the last load), then wave 0 checks
// the metadata and packs the token depths. Every workgroup reads the same
// words and takes the same decision, so either all of them run the launch or
// none does. Returns false when the launch must do nothing: an earlier launch
// failed (the error word is sticky until the host has read it) or the
// metadata is invalid (workgroup 0 then records the error code).
//   ctx: 0 <= ctx, ctx + T <= cap.
//   masks: bit t set, no bit above t, and each ancestor's mask contained in
//   the token's own (the tree rules of the causal verify pass).
__device__ __forceinline__ bool load_launch_words(const Params& p, Smem& sm) {
  constexpr int kN = kSchCount * kMaxWgUnits;
  static_assert(kN + kSchCount <= kThreads && kMaxReq * kMaxTok <= kThreads, "one entry per thread");
  const int tid = threadIdx.x;
  const int mr = tid / kMaxTok, mt = tid % kMaxTok;  // (request, token) of this thread's mask
  static_assert(sizeof(Unit) == sizeof(uint4), "a unit is one 16-byte load");
  const uint4 u = *reinterpret_cast<const uint4*>(p.wg_units + (size_t)blockIdx.x * kN + min(tid, kN - 1));
  const int32_t nu = p.wg_nunits[(size_t)blockIdx.x * kSchCount + min(max(tid - kN, 0), kSchCount - 1)];
  const int32_t c = p.ctx_dev[p.r0 + min(tid, p.R - 1)];
  const uint16_t* tsrc = p.tree_dev ? p.tree_dev + (size_t)(p.r0 + min(mr, p.R - 1)) * p.T + min(mt, p.T - 1) : p.zeros;
  const uint16_t tm = *tsrc;
  const int32_t e0 = __hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  ring_fence();
  if (tid < kN) reinterpret_cast<uint4*>(&sm.units[0][0])[tid] = u;
  else if (tid < kN + kSchCount) sm.nunits[tid - kN] = nu;
  if (tid < p.R) sm.ctx[tid] = c;
  if (tid < kMaxReq * kMaxTok) {
    uint32_t a = 0;
    if (mr < p.R && mt < p.T) a = p.tree_dev ? (uint32_t)tm : ((2u << mt) - 1u);
    sm.tanc[mr][mt] = a;
  }
  if (tid == 0) sm.err0 = e0;
  __syncthreads();
  if (wave_id() == 0) {
    const int lane = lane_id(), r = lane / kMaxTok, t = lane % kMaxTok;
    const bool live = r < p.R && t < p.T;
    const uint32_t a = sm.tanc[r][t];
    uint32_t anc[kMaxTok];
#pragma unroll
    for (int v = 0; v < kMaxTok; ++v) anc[v] = sm.tanc[r][v];
    // an ancestor v of t whose own mask holds a token outside t's mask
    uint32_t bad = 0;
#pragma unroll
    for (int v = 0; v < kMaxTok; ++v) bad |= (anc[v] & ~a) & (0u - ((a >> v) & 1u)) & (v < t ? ~0u : 0u);
    bool ok = !live || (((a >> t) & 1u) != 0u && (a >> (t + 1)) == 0u && bad == 0u);
    const uint64_t dep = live ? (uint64_t)(__builtin_popcount(a) - 1) << (4 * t) : 0ull;
    int code = __ballot(!ok) != 0ull ? kErrInvalid : 0;
    if (lane < p.R && sm.ctx[lane] < 0) ok = false;
    if (__ballot(!ok) != 0ull) code = kErrInvalid;
    if (code == 0) {
      const bool cap_ok = lane >= p.R || (int64_t)sm.ctx[lane] + p.T <= (int64_t)p.cap;
      if (__ballot(!cap_ok) != 0ull) code = kErrCapacity;
    }
    // depths of request r: the OR of its 16 lanes' fields (lanes 16r .. 16r+15)
    uint64_t pk = dep;
#pragma unroll
    for (int o = 1; o < kMaxTok; o <<= 1) pk |= (uint64_t)__shfl_xor((long long)pk, o);
    if (t == 0) sm.tdepth[r] = pk;
    if (lane == 0) sm.io_code = code;
  }
  __syncthreads();
  if (sm.err0 != 0) return false;
  if (sm.io_code != 0) {
    if (blockIdx.x == 0 && tid == 0) __hip_atomic_store(p.err, sm.io_code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  return true;
}

// The kernel's argument block, read through an opaque pointer to the
// kernel-argument segment. A phase that starts with its own reference loads
// the fields it uses (scalar loads that hit the scalar cache) instead of the
// compiler keeping every field loaded at launch start live in scalar
// registers through the whole launch, which spills them into vector-register
// lanes at places that shift with every change of the code.
__device__ __forceinline__ const Params& kargs() {
  const __attribute__((address_space(4))) Params* pp =
      (const __attribute__((address_space(4))) Params*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(pp));
  return *(const Params*)pp;
}

template <uint32_t MODE, int VARIANT>
__global__ void __launch_bounds__(kThreads, 1) layer_kernel(const Params p_arg) {
  (void)p_arg;  // read through kargs()
  const Params& p = kargs();
  constexpr bool DEBUG = VARIANT == kDebug;
  constexpr bool TRACE = VARIANT == kTrace;
  __shared__ Smem sm;
  Barrier bar{p.bar, p.err, p.bar_base + 1};
  uint64_t* const trace_row = TRACE ? p.trace + ((size_t)p.trace_launch * kMaxGrid + blockIdx.x) * kTraceSlots : nullptr;
  auto mark = [trace_row](int slot) {
    if constexpr (TRACE) {
      if (threadIdx.x == 0) trace_row[slot] = __builtin_amdgcn_s_memrealtime();
    }
  };
  mark(kTrStart);
  const int Dq = p.nq * p.d;
  const int Nqkv = Dq + 2 * p.nkv * p.d;
  DenseSlot ring[kRing];
  if (threadIdx.x == 0) sm.zero = make_uint4(0, 0, 0, 0);
  if (!load_launch_words(p, sm)) return;

  if constexpr ((MODE & kModeQkvOwn) != 0) {
    const Params& p = kargs();
    dense_prefetch<Epi::Qkv>(p, kSchQkv, p.cur.w_qkv, p.H, nullptr, sm, ring);
    compute_inv_rms(p, p.h_in, nullptr, sm);
    fill_x_norm(p, p.h_in, p.cur.g_attn, sm);
    EpiArgs ea{p.cur.k_cache, p.cur.v_cache, nullptr, p.qpart, nullptr, DEBUG ? p.dbg.k_new : nullptr,
               DEBUG ? p.dbg.v_new : nullptr};
    dense_phase<Epi::Qkv>(p, kSchQkv, p.cur.w_qkv, p.H, p.H, ea, sm, ring);
    mark(kTrQkvOwn);
    bar_arrive(bar);
    if (!bar_wait(bar, sm)) return;
    mark(kTrQkvOwnBar);
    if (DEBUG && p.dbg.q) {
      for (int i = blockIdx.x * kThreads + threadIdx.x; i < p.NT * Dq; i += gridDim.x * kThreads) {
        float v = 0.0f;
        for (int s = 0; s < p.q_slices; ++s) v += p.qpart[(size_t)s * p.NT * Dq + i];
        p.dbg.q[i] = v;
      }
    }
  }
  (void)Nqkv;

  {
  const Params& p = kargs();
  // attention of the launch's layer. Workgroups without an attention item
  // publish nothing in this phase: with a speculative prefetch they arrive at
  // the barrier first and read the listed experts while the others attend.
  const int n_items = p.n_prefetch > 0 ? attn_item_count(p, sm, p.cur, gridDim.x) : (int)gridDim.x;
  if ((int)blockIdx.x >= n_items) {
    bar_arrive(bar);
    prefetch_rank(p, sm);
    __syncthreads();
    prefetch_experts(p, sm, blockIdx.x - n_items, gridDim.x - n_items);
    mark(kTrAttn);
  } else {
    if (p.d == 128) attention_phase<128>(p, p.cur, sm, trace_row);
    else attention_phase<64>(p, p.cur, sm, trace_row);
    if (p.n_prefetch > 0 && blockIdx.x == 0 && p.out_prefetch) {
      prefetch_rank(p, sm);
      __syncthreads();
      if (threadIdx.x < p.n_prefetch) p.out_prefetch[threadIdx.x] = sm.plist[threadIdx.x];
    }
    mark(kTrAttn);
    bar_arrive(bar);
  }
  if (!bar_wait(bar, sm)) return;
  mark(kTrAttnBar);
  }

  {
  const Params& p = kargs();
  merge_phase<DEBUG>(p, sm, p.cur);
  mark(kTrMerge);
  bar_arrive(bar);
  if (!bar_wait_prefetch(bar, sm, [&] { dense_prefetch<Epi::OProj>(p, kSchOproj, p.cur.w_o, Dq, p.h_in, sm, ring); }))
    return;
  mark(kTrMergeBar);
  }

  // output projection + residual
  {
  const Params& p = kargs();
  {
    fill_x_copy(p.attn, Dq, p.NT, sm);
    mark(kTrOprojFill);
    EpiArgs ea{nullptr, nullptr, p.h_in, p.h1, p.ssq1, nullptr, nullptr};
    dense_phase<Epi::OProj>(p, kSchOproj, p.cur.w_o, Dq, Dq, ea, sm, ring);
  }
  mark(kTrOproj);
  bar_arrive(bar);
  if (!bar_wait_prefetch(bar, sm, [&] { dense_prefetch<Epi::Pool>(p, kSchPool, p.cur.w_pool, p.H, nullptr, sm, ring); }))
    return;
  mark(kTrOprojBar);
  if (DEBUG && p.dbg.h1) {
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < p.NT * p.H; i += gridDim.x * kThreads) p.dbg.h1[i] = p.h1[i];
  }
  }

  // router + pooler (both read n2 = RMSNorm(h1))
  {
  const Params& p = kargs();
  {
    // the stage-dump variant has no registers to spare for batched sums
    constexpr int RB = DEBUG ? 1 : 4;
    if (p.H >= 512 * p.p_slices) fill_x_pool_router<true, RB>(p, sm);
    else fill_x_pool_router<false, RB>(p, sm);
    mark(kTrPoolFill);
    if (DEBUG && p.dbg.n2 && blockIdx.x == 0) dump_n2(p, sm);
    // this workgroup's router sums are stored: announce them (sequence
    // number bar.seq) before the pooler's work, announced with bar.seq + 1
    bar_arrive_at(bar, bar.seq);
    EpiArgs ea{nullptr, nullptr, nullptr, p.ppart, nullptr, nullptr, nullptr};
    dense_phase<Epi::Pool>(p, kSchPool, p.cur.w_pool, p.H, p.H, ea, sm, ring);
  }
  mark(kTrRouterPool);
  bar_arrive_at(bar, bar.seq + 1);
  // top-k, gates and routing tables while the pooler finishes elsewhere:
  // they need every workgroup's router sums only
  if (!bar_wait_at(bar, sm, bar.seq)) return;
  routing<DEBUG>(p, sm, blockIdx.x == 0, routing_issue(p));
  if (!bar_wait_at(bar, sm, bar.seq + 1)) return;
  bar.seq += 2;
  mark(kTrRouterPoolBar);
  }

  // routing (every workgroup) + experts' gate/up
  {
  const Params& p = kargs();
  {
    // the pooled activations (the routing tables, built before the pooler's
    // barrier, lie after the pooled tile in LDS)
    SumLoads sl;
    fill_sum_issue(p.ppart, p.p_slices, p.P, p.NT, threadIdx.x, sl);
    fill_sum_finish(sl, p.p_slices, p.P, p.NT, threadIdx.x, sm);
    for (int i0 = threadIdx.x + kSumBatch * kThreads; i0 < kMaxTok * (p.P / 8); i0 += kSumBatch * kThreads) {
      fill_sum_issue(p.ppart, p.p_slices, p.P, p.NT, i0, sl);
      fill_sum_finish(sl, p.p_slices, p.P, p.NT, i0, sm);
    }
    vm_drain();
    __syncthreads();
  }
  mark(kTrRouting);
  if (DEBUG && blockIdx.x == 0) {
    if (p.dbg.p)
      for (int i = threadIdx.x; i < p.NT * p.P; i += kThreads) {
        float v = 0.0f;
        for (int s = 0; s < p.p_slices; ++s) v += p.ppart[(size_t)s * p.NT * p.P + i];
        p.dbg.p[i] = v;
      }
  }
  gemm1_phase<DEBUG>(p, sm);
  mark(kTrGemm1);
  bar_arrive(bar);
  if (!bar_wait(bar, sm)) return;
  mark(kTrGemm1Bar);
  }

  {
  const Params& p = kargs();
  gemm2_phase<DEBUG>(p, sm);
  mark(kTrGemm2);
  bar_arrive(bar);
  if (!bar_wait_prefetch(bar, sm, [&] { dense_prefetch<Epi::Unpool>(p, kSchUnpool, p.cur.w_unpool, p.P, p.h1, sm, ring); }))
    return;
  mark(kTrGemm2Bar);
  }

  // unpooler + residual
  {
  const Params& p = kargs();
    const int parts = max(1, (int)gridDim.x / (p.P / 16));
    fill_x_sum(p.accpart, parts, p.P, p.NT, sm);
    mark(kTrUnpoolFill);
    EpiArgs ea{nullptr, nullptr, p.h1, p.h_out, p.ssq2, nullptr, nullptr};
    dense_phase<Epi::Unpool>(p, kSchUnpool, p.cur.w_unpool, p.P, p.P, ea, sm, ring);
    if (DEBUG && p.dbg.acc && blockIdx.x == 0) {
      for (int i = threadIdx.x; i < p.NT * p.P; i += kThreads) {
        float v = 0.0f;
        for (int s = 0; s < parts; ++s) v += p.accpart[(size_t)s * p.NT * p.P + i];
        p.dbg.acc[i] = v;
      }
    }
  }

  mark(kTrUnpool);
  if constexpr ((MODE & kModeQkvNext) != 0) {
    const Params& p = kargs();
    bar_arrive(bar);
    if (!bar_wait_prefetch(bar, sm, [&] { dense_prefetch<Epi::Qkv>(p, kSchQkv, p.nxt.w_qkv, p.H, nullptr, sm, ring); }))
      return;
    mark(kTrUnpoolBar);
    fill_x_qkv(p, p.h_out, p.ssq2, p.nxt.g_attn, sm);
    mark(kTrQkvFill);
    if (p.kv_prefetch) prefetch_next_kv(p, sm);
    EpiArgs ea{p.nxt.k_cache, p.nxt.v_cache, nullptr, p.qpart, nullptr, nullptr, nullptr};
    dense_phase<Epi::Qkv>(p, kSchQkv, p.nxt.w_qkv, p.H, p.H, ea, sm, ring);
    mark(kTrQkvNext);
  }
}

// Start of a call: zero the barrier flags; the error word only when the
// host has read the error it holds (it stays set until then, so every later
// launch does nothing).
__global__ void reset_kernel(uint32_t* bar, int32_t* err, int32_t clear_err) {
  if (threadIdx.x < kMaxGrid) bar[threadIdx.x * kFlagStride] = 0;
  if (threadIdx.x == 0 && clear_err) *err = 0;
}

}  // namespace
}  // namespace msk

template <int V>
static hipError_t launch_mode(const msk::Params& p, dim3 g, dim3 b, hipStream_t s) {
  using namespace msk;
  switch (p.mode) {
    case kModeQkvOwn: hipLaunchKernelGGL((layer_kernel<kModeQkvOwn, V>), g, b, 0, s, p); break;
    case kModeQkvOwn | kModeQkvNext:
      hipLaunchKernelGGL((layer_kernel<kModeQkvOwn | kModeQkvNext, V>), g, b, 0, s, p); break;
    case kModeQkvNext: hipLaunchKernelGGL((layer_kernel<kModeQkvNext, V>), g, b, 0, s, p); break;
    default: hipLaunchKernelGGL((layer_kernel<0u, V>), g, b, 0, s, p); break;
  }
  return hipGetLastError();
}

hipError_t msk_launch_layer(const msk::Params& p, int grid, bool debug, hipStream_t s) {
  using namespace msk;
  dim3 g(grid), b(kThreads);
  if (debug) {
    if (p.mode != kModeQkvOwn) return hipErrorInvalidValue;
    hipLaunchKernelGGL((layer_kernel<kModeQkvOwn, kDebug>), g, b, 0, s, p);
    return hipGetLastError();
  }
  if (p.trace) return launch_mode<kTrace>(p, g, b, s);
  return launch_mode<kPlain>(p, g, b, s);
}

// Reorders the down projection's E4M3 block scales from row-major
// [E][P][I/16] to the tiled order GEMM2 reads, [E][P/16][S][16][8] with
// S = ceil(I/128): for each expert and 16-row tile, the 8 scales of k-slice s
// (128 elements) of the 16 rows are one 128-byte line. Scale positions past
// I/16 are zero. One thread per 8-byte group.
__global__ void pack_down_scale_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int E, int P, int I) {
  const int S = msk::dn_scale_slices(I), cols = I / 16;
  const size_t n = (size_t)E * (P / 16) * S * 16;
  for (size_t g = blockIdx.x * (size_t)blockDim.x + threadIdx.x; g < n; g += (size_t)gridDim.x * blockDim.x) {
    const int r = (int)(g & 15);
    const size_t ts = g >> 4;                 // (expert, tile, slice)
    const int s = (int)(ts % S);
    const size_t row = (ts / S) * 16 + r;     // expert * P + tile * 16 + r
    uint64_t v = 0;
    for (int b = 0; b < 8; ++b) {
      const int c = s * 8 + b;
      if (c < cols) v |= (uint64_t)src[row * cols + c] << (8 * b);
    }
    reinterpret_cast<uint64_t*>(dst)[g] = v;
  }
}

hipError_t msk_launch_pack_down_scale(const uint8_t* src, uint8_t* dst, int E, int P, int I, hipStream_t s) {
  const size_t n = (size_t)E * (P / 16) * msk::dn_scale_slices(I) * 16;
  const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(pack_down_scale_kernel, dim3(blocks), dim3(256), 0, s, src, dst, E, P, I);
  return hipGetLastError();
}

hipError_t msk_launch_reset(uint32_t* bar, int32_t* err, bool clear_err, hipStream_t s) {
  hipLaunchKernelGGL(msk::reset_kernel, dim3(1), dim3(msk::kMaxGrid), 0, s, bar, err, clear_err ? 1 : 0);
  return hipGetLastError();
}

template <uint32_t MODE, int V>
static int occupancy_of() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, msk::layer_kernel<MODE, V>, msk::kThreads, 0) != hipSuccess)
    return 0;
  return n;
}

int msk_layer_min_occupancy() {
  using namespace msk;
  const int v[] = {occupancy_of<kModeQkvOwn, kPlain>(), occupancy_of<kModeQkvOwn | kModeQkvNext, kPlain>(),
                   occupancy_of<kModeQkvNext, kPlain>(), occupancy_of<0u, kPlain>(),
                   occupancy_of<kModeQkvOwn, kTrace>(), occupancy_of<kModeQkvOwn | kModeQkvNext, kTrace>(),
                   occupancy_of<kModeQkvNext, kTrace>(), occupancy_of<0u, kTrace>(),
                   occupancy_of<kModeQkvOwn, kDebug>()};
  int m = v[0];
  for (int x : v) m = std::min(m, x);
  return m;
}

// Workspace of handles made by msk_create_static, for callers that cannot
// allocate device memory: one array per GPU the library runs on, held until
// the process ends. Host code never uses the array's name as an address (on
// the host it only stands for the symbol): its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// that address is what the handles, the kernels and the copies use.
static __device__ __align__(256) uint8_t scratch[msk::kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t msk_static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}
