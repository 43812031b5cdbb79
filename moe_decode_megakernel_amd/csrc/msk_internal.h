// Internal definitions shared by the host side (msk_api.cpp) and the layer
// kernel (msk_layer.hip) of libmsk. Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace msk {

constexpr int kWaves = 8;                 // waves per workgroup
constexpr int kThreads = kWaves * 64;     // threads per workgroup
constexpr int kMaxGrid = 256;             // workgroups per launch at most (one per compute unit)
// Barrier flags, one per 64-byte line: flag i at word i * kFlagStride. With
// 16 flags packed in a line a grid barrier took 2.65 us against 1.49 us on
// MI355X (256 workgroups, no other traffic): the workgroups' write-through
// stores to one line and the polls of it queue behind each other.
constexpr int kFlagStride = 16;
constexpr int kMaxReq = 4;
constexpr int kMaxTok = 16;               // tokens per launch handled as one 16-row MFMA tile
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;
constexpr int kMaxHeadDim = 128;
constexpr int kSubK = 128;                // dense k per wave sub-unit (4 MFMA steps of 32)
constexpr int kAttnChunk = 64;            // keys per attention chunk in LDS
constexpr int kTraceSlots = 25;            // phase-boundary timestamps per workgroup per launch
constexpr int kG1StageBytes = 32768;       // LDS staging of GEMM1 outputs per workgroup (256 B per unit)
constexpr int kMaxWgUnits = 32;            // dense units of one workgroup in one schedule
constexpr int kMaxQSlices = 2;             // split-K slices of the Q projection
constexpr int kMaxSplits = 64;             // attention splits per (request, kv head)
constexpr int kMaxPrefetch = 32;           // experts in a speculative prefetch list
constexpr int kMaxRouterPerWg = 2;         // router (expert, k-slice) pairs per workgroup
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;  // the library's own workspace array per device

// k-slices of 128 elements per row of the down projection: its block scales
// are stored tiled, [E][P/16][dn_scale_slices(I)][16 rows][8], so one wave's
// scales for an (expert, 16-row tile, k-slice) are one 128-byte line.
__host__ __device__ constexpr int dn_scale_slices(int I) { return (I + 127) / 128; }

// Launch modes (bit set).
enum : uint32_t {
  kModeQkvOwn = 1u,   // first phase: QKV projection + KV write of the launch's own layer
  kModeQkvNext = 2u,  // last phase: QKV projection + KV write of the next layer
};

// Phase-work unit of a dense (bf16) projection: rows [tile*16, tile*16+16),
// k in [k0, k0+klen). A tile whose k range exceeds one unit is cut into
// consecutive pieces on the same workgroup: the first piece starts the
// accumulator, the last one reduces it and runs the epilogue.
constexpr int32_t kUnitFirst = 1 << 30;
constexpr int32_t kUnitLast = 1 << 29;
constexpr int32_t kUnitSlotMask = 0xFFFF;
struct Unit {
  int32_t tile, k0, klen, slot;  // slot: partial slot | kUnitFirst | kUnitLast
};

struct LayerW {
  const uint16_t* w_qkv;
  const uint16_t* w_o;
  const float* w_router;
  const float* b_router;
  const uint16_t* w_pool;
  const uint16_t* w_unpool;
  const uint16_t* g_attn;
  const uint16_t* g_moe;
  const uint8_t* e_gu;
  const uint8_t* e_gu_sc;
  const uint8_t* e_dn;
  const uint8_t* e_dn_sc;
  const float* e_ts;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int32_t window;
};

struct Debug {
  float* q;
  float* k_new;
  float* v_new;
  float* attn;
  float* h1;
  float* n2;
  float* logits;
  float* p;
  float* acc;
  int32_t dq_expert;
  uint16_t* dq_gu;
  uint16_t* dq_dn;
  float* act;         // [NT][I] SwiGLU output of dq_expert before activation quantization
  uint8_t* act_codes; // [NT][I/2] its E2M1 codes
  uint8_t* act_sc;    // [NT][I/16] its E4M3 block scales
  uint8_t* act_codes_all; // [E][NT][I/2] E2M1 codes of every selected expert (by expert id)
  uint8_t* act_sc_all;    // [E][NT][I/16] their block scales
};

// Schedules of the dense phases, built once per handle and stored per
// workgroup: units [G][kSchCount][kMaxWgUnits] (unused entries zero) and
// counts [G][kSchCount]. A workgroup copies its own rows to LDS at launch
// start (one round trip).
enum { kSchQkv = 0, kSchOproj, kSchPool, kSchUnpool, kSchCount };

struct Params {
  // shapes
  int32_t H, nq, nkv, d, E, topk, P, I;
  int32_t R, T, NT, cap;
  int32_t use_norm;
  int32_t act_fp4;        // SwiGLU outputs quantized to NVFP4 before the down projection
  float eps;
  // Request metadata in device memory, read by every workgroup at launch
  // start: prior context lengths ctx_dev[r0 + r] and, unless tree_dev is
  // NULL (the causal chain), the ancestor bitmasks tree_dev[(r0 + r)*T + t].
  const int32_t* ctx_dev;
  const uint16_t* tree_dev;
  int32_t r0;             // first request of this launch's pass
  int32_t q_slices, p_slices;
  uint32_t mode;
  int32_t layer;          // layer whose attention .. unpooler this launch runs
  uint32_t bar_base;      // barriers completed in this call before this launch
  LayerW cur, nxt;        // nxt: layer whose QKV / KV write ends the launch
  const float* h_in;      // residual entering `layer`
  float* h_out;           // residual leaving `layer`
  // workspace
  uint32_t* bar;          // grid barrier flags [kMaxGrid][kFlagStride] (sequence numbers in word 0)
  int32_t* err;           // device error word
  float* h1;              // [NT][H]
  float* ssq1;            // [H/16][NT] partial sums of squares of h1
  float* ssq2;            // [H/16][NT] of the launch's output residual
  float* qpart;           // [q_slices][NT][Dq]
  float* apart;           // attention partials
  uint16_t* attn;         // fp16 [NT][Dq] merged attention output
  float* logits;          // [p_slices][NT][E] router subtree sums per k-slice (no bias)
  float* ppart;           // [p_slices][NT][P]
  uint16_t* abuf;         // f16 [n_sel_max][NT][I] (SwiGLU output x gate weight)
  uint8_t* acode;         // with act_fp4, in abuf's region: E2M1 codes [n_sel_max][NT][I/2]
  uint8_t* ascale;        //   and E4M3 block scales [n_sel_max][NT][I/16]
  float* accpart;         // [parts][NT][P]
  const int32_t* hist_rd; // [n_layers][E] selection counts of the previous call (prefetch ranking)
  int32_t* hist_wr;       // [n_layers][E] this call's counts
  int32_t hist_add;       // add to hist_wr (later token passes of a call) instead of overwriting
  const uint16_t* zeros;  // 256 zero bytes (A operand of masked lanes)
  const Unit* wg_units;     // QKV (own and next layer share shapes), O proj, pool, unpool
  const int32_t* wg_nunits;
  int32_t n_prefetch;     // experts to prefetch speculatively (0 = off)
  int32_t kv_prefetch;    // touch the next layer's KV window during its QKV projection
  // outputs
  int32_t* out_ids;       // [NT][k] or NULL
  float* out_gates;
  int32_t* out_prefetch;  // [n_prefetch] or NULL: this launch's prefetch list
  Debug dbg;
  uint64_t* trace;        // [launch][grid][kTraceSlots] or NULL (self-timing variant)
  int32_t trace_launch;
};

}  // namespace msk

// Launchers implemented in msk_layer.hip.
hipError_t msk_launch_layer(const msk::Params& p, int grid, bool debug, hipStream_t s);
hipError_t msk_launch_pack_down_scale(const uint8_t* src, uint8_t* dst, int E, int P, int I, hipStream_t s);
hipError_t msk_launch_reset(uint32_t* bar, int32_t* err, bool clear_err, hipStream_t s);
// Device address of the library's static workspace array on the current
// device (looked up once per device and kept).
hipError_t msk_static_scratch(void** out);
// Fewest layer-kernel workgroups of kThreads that one compute unit can hold,
// over the kernel's instantiations (the grid must be co-resident).
int msk_layer_min_occupancy();
