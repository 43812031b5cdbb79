// Host side of the msk C ABI (include/msk.h): argument validation, workspace
// carving, the static schedules of the dense projections, and the launches of
// the layer kernel (msk_layer.hip).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/msk.h"
#include "msk_internal.h"

static_assert(MSK_STATIC_WORKSPACE_BYTES == msk::kStaticScratchBytes, "static workspace size");

namespace {

using msk::kMaxGrid;

struct Layout {
  size_t bar, err, zeros, sched, h1, ssq1, ssq2, hbuf0, hbuf1, qpart, apart, attn, logits, ppart, abuf, accpart, hist;
  size_t total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct SchedHost {
  std::vector<msk::Unit> units;
  std::vector<int32_t> off;
  int64_t max_load = 0;
};

struct TileSpec {
  int tile;
  int klen;
  bool splittable;
};

constexpr int kUnitMaxK = msk::kSubK * msk::kWaves;  // one 128-k sub-unit per wave

// Longest-processing-time assignment of jobs to G workgroups. A splittable
// tile becomes `slices` jobs of equal k ranges (partial slot = slice index);
// an unsplit tile is one job. A job longer than one unit (kUnitMaxK) runs as
// consecutive pieces on one workgroup, carrying the accumulator. With
// slice_groups, a job of slice s goes only to workgroups g with g mod slices
// == s, so each workgroup's units lie in one k-slice.
SchedHost build_sched(const std::vector<TileSpec>& tiles, int slices, int G, bool slice_groups = false) {
  struct Job {
    int tile, k0, klen, slot;
  };
  std::vector<Job> jobs;
  for (const TileSpec& t : tiles) {
    if (t.splittable && slices > 1) {
      int kl = t.klen / slices;
      for (int s = 0; s < slices; ++s) jobs.push_back({t.tile, s * kl, kl, s});
    } else {
      jobs.push_back({t.tile, 0, t.klen, 0});
    }
  }
  std::stable_sort(jobs.begin(), jobs.end(), [](const Job& a, const Job& b) { return a.klen > b.klen; });
  std::vector<std::vector<msk::Unit>> per(G);
  std::vector<int64_t> load(G, 0);
  for (const Job& j : jobs) {
    const int g0 = slice_groups ? j.slot : 0, step = slice_groups ? slices : 1;
    int best = g0;
    for (int g = g0 + step; g < G; g += step)
      if (load[g] < load[best]) best = g;
    for (int k = 0; k < j.klen; k += kUnitMaxK) {
      int kl = std::min(kUnitMaxK, j.klen - k);
      int32_t slot = j.slot;
      if (k == 0) slot |= msk::kUnitFirst;
      if (k + kl == j.klen) slot |= msk::kUnitLast;
      per[best].push_back({j.tile, j.k0 + k, kl, slot});
    }
    load[best] += j.klen;
  }
  SchedHost sh;
  sh.off.push_back(0);
  for (int g = 0; g < G; ++g) {
    for (const msk::Unit& u : per[g]) sh.units.push_back(u);
    sh.off.push_back((int32_t)sh.units.size());
    sh.max_load = std::max(sh.max_load, load[g]);
  }
  return sh;
}

// Best slice count in 1 .. msk::kMaxQSlices (fewest slices among the lowest
// max load). Attention reads every slice of Q, so the bound keeps its loads
// and registers small.
SchedHost build_sched_best(const std::vector<TileSpec>& tiles, int K, int G, int* slices_out) {
  SchedHost best;
  int best_s = 1;
  for (int s = 1; s <= msk::kMaxQSlices; s *= 2) {
    if (K % (s * msk::kSubK) != 0) continue;
    SchedHost sh = build_sched(tiles, s, G);
    if (best.off.empty() || sh.max_load < best.max_load) {
      best = std::move(sh);
      best_s = s;
    }
  }
  *slices_out = best_s;
  return best;
}

// The pooler's schedule: slice count in {1, 2} (fewer slices among the
// lowest max load) with each workgroup's units in slice g mod slices, so the
// workgroup fills only that k-slice of its input. The router is split the
// same way: slice s of expert e is pair e*slices + s, and workgroup g takes
// pairs g, g+G, ...; a slice count is admitted when G is a multiple of it and
// no workgroup gets more than kMaxRouterPerWg pairs.
SchedHost build_sched_pool(const std::vector<TileSpec>& tiles, int K, int G, int E, int* slices_out) {
  SchedHost best;
  int best_s = 1;
  for (int s : {1, 2}) {
    if (K % (s * msk::kSubK) != 0 || G % s != 0) continue;
    if ((E * s + G - 1) / G > msk::kMaxRouterPerWg) continue;
    SchedHost sh = build_sched(tiles, s, G, true);
    if (best.off.empty() || sh.max_load < best.max_load) {
      best = std::move(sh);
      best_s = s;
    }
  }
  *slices_out = best_s;
  return best;
}

}  // namespace

struct msk_handle_s {
  msk_config cfg;
  int grid = 0;
  uint8_t* ws = nullptr;
  size_t ws_bytes = 0;
  Layout lay{};
  std::vector<msk_layer_desc> layers;
  std::vector<bool> loaded;
  int q_slices = 1, p_slices = 1;
  const msk::Unit* wg_units = nullptr;
  const int32_t* wg_nunits = nullptr;
  int32_t* err_host = nullptr;    // pinned copy of the device error word, written at the end of each call
  hipEvent_t done = nullptr;      // recorded after that copy (calls not under graph capture)
  bool done_pending = false;      // `done` recorded and not yet observed complete
  bool clear_err = false;         // the next call's reset zeroes the device error word
  bool is_static = false;         // workspace = the library's static array (msk_create_static)
  hipStream_t last_stream = nullptr;  // stream of the last call (static handles: msk_synchronize)
  uint64_t calls = 0;  // verify calls enqueued (selects the histogram buffers)
  std::string last_error;
};

namespace {

thread_local std::string g_create_error;

msk_status fail(msk_handle h, msk_status st, const std::string& msg) {
  if (h) h->last_error = msg;
  else g_create_error = msg;
  return st;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks; returns an empty string when the configuration is supported.
std::string check_config(const msk_config* c) {
  if (!c) return "config is NULL";
  const int Dq = c->n_q_heads * c->head_dim;
  if (c->hidden < 128 || c->hidden > 4096 || (c->hidden & (c->hidden - 1)) != 0)
    return "hidden must be a power of two in 128..4096";
  if (c->head_dim != 64 && c->head_dim != 128) return "head_dim must be 64 or 128";
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->n_q_heads % c->n_kv_heads != 0) return "n_q_heads must be a multiple of n_kv_heads";
  if (c->n_q_heads / c->n_kv_heads > msk::kWaves) return "at most 8 query heads per kv head";
  if (Dq % 128 != 0 || Dq > 4096) return "n_q_heads*head_dim must be a multiple of 128, <= 4096";
  if (c->n_experts <= 0 || c->n_experts > msk::kMaxE) return "n_experts must be in 1..256";
  if (c->top_k <= 0 || c->top_k > msk::kMaxK || c->top_k > c->n_experts) return "top_k must be in 1..min(8, n_experts)";
  if (c->pool_dim <= 0 || c->pool_dim % 128 != 0 || c->pool_dim > 2048) return "pool_dim must be a positive multiple of 128, <= 2048";
  if (c->expert_inter <= 0 || c->expert_inter % 32 != 0 || c->expert_inter > 1024) return "expert_inter must be a positive multiple of 32, <= 1024";
  if (c->n_layers <= 0) return "n_layers must be positive";
  if (c->max_tokens <= 0 || c->max_tokens > msk::kMaxTok) return "max_tokens must be in 1..16";
  if (c->max_requests <= 0 || c->max_requests > msk::kMaxReq) return "max_requests must be in 1..4";
  if (c->kv_capacity <= 0) return "kv_capacity must be positive";
  if (!(c->rms_eps >= 0.0f)) return "rms_eps must be >= 0";
  if ((c->flags & ~(MSK_FLAG_NO_NORM | MSK_FLAG_ACT_FP4 | MSK_FLAG_KV_PREFETCH)) != 0) return "unknown flag bits";
  if (c->expert_prefetch < 0 || c->expert_prefetch > msk::kMaxPrefetch || c->expert_prefetch > c->n_experts)
    return "expert_prefetch must be in 0..min(32, n_experts)";
  return std::string();
}

// A call runs its requests in passes of at most kMaxTok tokens (one 16-row
// MFMA tile): requests_per_pass whole requests each.
int requests_per_pass(int32_t tokens) { return std::max(1, msk::kMaxTok / std::max(1, tokens)); }
int pass_tokens(const msk_config* c) {
  return std::min(c->max_requests, requests_per_pass(c->max_tokens)) * c->max_tokens;
}

Layout make_layout(const msk_config* c, int G) {
  const size_t NT = (size_t)pass_tokens(c);
  const size_t H = c->hidden, Dq = (size_t)c->n_q_heads * c->head_dim, P = c->pool_dim, I = c->expert_inter;
  const size_t E = c->n_experts, K = c->top_k;
  const size_t nsel = std::min(E, NT * K);
  const size_t parts = std::max<size_t>(1, (size_t)G / (P / 16));
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  L.bar = take(msk::kMaxGrid * msk::kFlagStride * 4);
  L.err = take(256);
  L.zeros = take(256);
  // schedule tables: units of 4 schedules + offsets (generous bound)
  L.sched = take((size_t)G * msk::kSchCount * (msk::kMaxWgUnits * sizeof(msk::Unit) + sizeof(int32_t)));
  L.h1 = take(NT * H * 4);
  L.ssq1 = take((H / 16) * NT * 4);
  L.ssq2 = take((H / 16) * NT * 4);
  L.hbuf0 = take(NT * H * 4);
  L.hbuf1 = take(NT * H * 4);
  L.qpart = take(msk::kMaxQSlices * NT * Dq * 4);
  L.apart = take((size_t)G * msk::kWaves * msk::kMaxTok * (c->head_dim + 4) * 4);
  L.attn = take(NT * Dq * 2);
  L.logits = take(4 * NT * E * 4);  // router partial sums per k-slice of the pooler
  L.ppart = take(4 * NT * P * 4);
  L.abuf = take(nsel * NT * I * 2);
  L.accpart = take(parts * NT * P * 4);
  L.hist = take(2 * (size_t)c->n_layers * E * 4);  // by call parity: previous call's counts | this call's
  L.total = o;
  return L;
}

}  // namespace

extern "C" size_t msk_workspace_bytes(const msk_config* cfg) {
  if (!check_config(cfg).empty()) return 0;
  return make_layout(cfg, kMaxGrid).total;
}

namespace {

// Shared by msk_create and msk_create_static. A static handle has no pinned
// error word and no event: its device status is read by msk_synchronize.
msk_status create_impl(const msk_config* cfg, void* workspace, size_t bytes, bool is_static, msk_handle* out) {
  if (!out) return fail(nullptr, MSK_E_INVALID, "out is NULL");
  *out = nullptr;
  std::string why = check_config(cfg);
  if (!why.empty()) return fail(nullptr, MSK_E_SHAPE, why);
  if (!workspace) return fail(nullptr, MSK_E_INVALID, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(nullptr, MSK_E_ALIGN, "workspace must be 256-byte aligned");
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(nullptr, MSK_E_HIP, "no HIP device");
  const int G = std::min(prop.multiProcessorCount, kMaxGrid);
  if (cfg->n_experts > msk::kMaxRouterPerWg * G)
    return fail(nullptr, MSK_E_SHAPE, "n_experts exceeds the router rows the workgroups of one launch cover");
  // attention runs at least one work item per (request, kv head) and the
  // launch has one workgroup per compute unit
  if ((int64_t)cfg->max_requests * cfg->n_kv_heads > G)
    return fail(nullptr, MSK_E_SHAPE, "max_requests * n_kv_heads exceeds the compute units of the device");
  // the down projection gives every 16-row tile of the pooled dim a workgroup
  if (cfg->pool_dim / 16 > G)
    return fail(nullptr, MSK_E_SHAPE, "pool_dim / 16 exceeds the compute units of the device");
  // the grid barrier needs every workgroup resident at once
  if (msk_layer_min_occupancy() < 1)
    return fail(nullptr, MSK_E_SHAPE, "the layer kernel does not fit one workgroup per compute unit on this device");
  {
    // GEMM1 stages 256 B per (selected expert, 8-row i-tile) unit of a workgroup in LDS
    const int64_t nsel = std::min<int64_t>(cfg->n_experts, (int64_t)pass_tokens(cfg) * cfg->top_k);
    // (512 B per unit, in whole pairs of units, with activation quantization)
    const int64_t units = nsel * (cfg->expert_inter / 8);
    const int64_t per_wg = (cfg->flags & MSK_FLAG_ACT_FP4) ? 2 * ((units / 2 + G - 1) / G) * 512
                                                           : (units + G - 1) / G * 256;
    if (per_wg > msk::kG1StageBytes)
      return fail(nullptr, MSK_E_SHAPE, "too many expert units per workgroup for the GEMM1 staging area");
  }
  Layout lay = make_layout(cfg, kMaxGrid);
  if (bytes < lay.total) return fail(nullptr, MSK_E_CAPACITY, "workspace smaller than msk_workspace_bytes");

  msk_handle h = new (std::nothrow) msk_handle_s();
  if (!h) return fail(nullptr, MSK_E_INVALID, "out of host memory");
  h->cfg = *cfg;
  h->grid = G;
  h->is_static = is_static;
  h->ws = (uint8_t*)workspace;
  h->ws_bytes = bytes;
  h->lay = lay;
  h->layers.resize(cfg->n_layers);
  h->loaded.assign(cfg->n_layers, false);

  // dense schedules
  const int H = cfg->hidden, Dq = cfg->n_q_heads * cfg->head_dim, Dkv = cfg->n_kv_heads * cfg->head_dim;
  const int P = cfg->pool_dim;
  std::vector<TileSpec> t_qkv, t_oproj, t_pool, t_unpool;
  for (int t = 0; t < (Dq + 2 * Dkv) / 16; ++t) t_qkv.push_back({t, H, t * 16 < Dq});
  for (int t = 0; t < H / 16; ++t) t_oproj.push_back({t, Dq, false});
  for (int t = 0; t < P / 16; ++t) t_pool.push_back({t, H, true});
  for (int t = 0; t < H / 16; ++t) t_unpool.push_back({t, P, false});
  SchedHost sq = build_sched_best(t_qkv, H, G, &h->q_slices);
  SchedHost so = build_sched(t_oproj, 1, G);
  SchedHost sp = build_sched_pool(t_pool, H, G, cfg->n_experts, &h->p_slices);
  if (sp.off.empty()) {
    delete h;
    return fail(nullptr, MSK_E_SHAPE, "no pooler schedule fits this grid and expert count");
  }
  SchedHost su = build_sched(t_unpool, 1, G);

  // per-workgroup tables: units [G][kSchCount][kMaxWgUnits], counts [G][kSchCount]
  const size_t n_units = (size_t)G * msk::kSchCount * msk::kMaxWgUnits;
  std::vector<msk::Unit> tab(n_units, msk::Unit{0, 0, 0, 0});
  std::vector<int32_t> cnt((size_t)G * msk::kSchCount, 0);
  const SchedHost* all[msk::kSchCount] = {&sq, &so, &sp, &su};
  for (int i = 0; i < msk::kSchCount; ++i) {
    for (int g = 0; g < G; ++g) {
      const int n = all[i]->off[g + 1] - all[i]->off[g];
      if (n > msk::kMaxWgUnits) {
        delete h;
        return fail(nullptr, MSK_E_SHAPE, "a dense schedule gives one workgroup more units than it stages");
      }
      cnt[(size_t)g * msk::kSchCount + i] = n;
      for (int u = 0; u < n; ++u)
        tab[((size_t)g * msk::kSchCount + i) * msk::kMaxWgUnits + u] = all[i]->units[all[i]->off[g] + u];
    }
  }
  std::vector<uint8_t> blob(n_units * sizeof(msk::Unit) + cnt.size() * sizeof(int32_t));
  memcpy(blob.data(), tab.data(), n_units * sizeof(msk::Unit));
  memcpy(blob.data() + n_units * sizeof(msk::Unit), cnt.data(), cnt.size() * sizeof(int32_t));
  h->wg_units = reinterpret_cast<const msk::Unit*>(h->ws + lay.sched);
  h->wg_nunits = reinterpret_cast<const int32_t*>(h->ws + lay.sched + n_units * sizeof(msk::Unit));
  if (blob.size() > lay.h1 - lay.sched) {
    delete h;
    return fail(nullptr, MSK_E_CAPACITY, "schedule tables exceed their workspace region");
  }
  if (hipMemcpy(h->ws + lay.sched, blob.data(), blob.size(), hipMemcpyHostToDevice) != hipSuccess) {
    delete h;
    return fail(nullptr, MSK_E_HIP, "hipMemcpy of the schedule tables failed");
  }
  // zero the barrier flags, error word and routing histogram once
  const size_t bar_bytes = (size_t)kMaxGrid * msk::kFlagStride * 4;
  std::vector<uint8_t> zeros(std::max(bar_bytes, 2 * (size_t)cfg->n_layers * cfg->n_experts * 4), 0);
  if (hipMemcpy(h->ws + lay.bar, zeros.data(), bar_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(h->ws + lay.err, zeros.data(), 256, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(h->ws + lay.zeros, zeros.data(), 256, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(h->ws + lay.hist, zeros.data(), 2 * (size_t)cfg->n_layers * cfg->n_experts * 4, hipMemcpyHostToDevice) != hipSuccess) {
    delete h;
    return fail(nullptr, MSK_E_HIP, "hipMemcpy of the workspace header failed");
  }
  if (!is_static) {
    if (hipHostMalloc((void**)&h->err_host, 256, hipHostMallocDefault) != hipSuccess) {
      delete h;
      return fail(nullptr, MSK_E_HIP, "hipHostMalloc of the error word failed");
    }
    *h->err_host = 0;
    if (hipEventCreateWithFlags(&h->done, hipEventDisableTiming) != hipSuccess) {
      (void)hipHostFree(h->err_host);
      delete h;
      return fail(nullptr, MSK_E_HIP, "hipEventCreate failed");
    }
  }
  *out = h;
  return MSK_OK;
}

}  // namespace

extern "C" msk_status msk_create(const msk_config* cfg, void* workspace, size_t bytes, msk_handle* out) {
  return create_impl(cfg, workspace, bytes, false, out);
}

extern "C" msk_status msk_create_static(const msk_config* cfg, msk_handle* out) {
  if (!out) return fail(nullptr, MSK_E_INVALID, "out is NULL");
  *out = nullptr;
  const size_t need = msk_workspace_bytes(cfg);
  if (need == 0) return fail(nullptr, MSK_E_SHAPE, cfg ? check_config(cfg) : std::string("config is NULL"));
  if (need > msk::kStaticScratchBytes) {
    char buf[160];
    snprintf(buf, sizeof buf, "configuration needs %zu workspace bytes; the static workspace holds %zu", need,
             msk::kStaticScratchBytes);
    return fail(nullptr, MSK_E_CAPACITY, buf);
  }
  void* ws = nullptr;
  const hipError_t e = msk_static_scratch(&ws);
  if (e != hipSuccess)
    return fail(nullptr, MSK_E_HIP, std::string("hipGetSymbolAddress of the static workspace failed: ") + hipGetErrorString(e));
  return create_impl(cfg, ws, msk::kStaticScratchBytes, true, out);
}

extern "C" msk_status msk_load_layer(msk_handle h, int32_t layer, const msk_layer_desc* d) {
  if (!h) return fail(nullptr, MSK_E_INVALID, "handle is NULL");
  if (!d) return fail(h, MSK_E_INVALID, "desc is NULL");
  if (layer < 0 || layer >= h->cfg.n_layers) return fail(h, MSK_E_INVALID, "layer out of range");
  if (d->window < 0) return fail(h, MSK_E_INVALID, "window must be >= 0");
  const void* req[] = {d->w_qkv, d->w_o, d->w_router, d->w_pool, d->w_unpool, d->g_attn, d->g_moe,
                       d->e_gate_up, d->e_gate_up_scale, d->e_down, d->e_down_scale, d->e_tensor_scale,
                       d->k_cache, d->v_cache};
  for (const void* p : req) {
    if (!p) return fail(h, MSK_E_INVALID, "a required layer pointer is NULL");
    if (!aligned16(p)) return fail(h, MSK_E_ALIGN, "layer pointers must be 16-byte aligned");
  }
  if (d->b_router && !aligned16(d->b_router)) return fail(h, MSK_E_ALIGN, "b_router must be 16-byte aligned");
  h->layers[layer] = *d;
  h->loaded[layer] = true;
  return MSK_OK;
}

namespace {

msk::LayerW to_w(const msk_layer_desc& d) {
  msk::LayerW w;
  w.w_qkv = d.w_qkv;
  w.w_o = d.w_o;
  w.w_router = d.w_router;
  w.b_router = d.b_router;
  w.w_pool = d.w_pool;
  w.w_unpool = d.w_unpool;
  w.g_attn = d.g_attn;
  w.g_moe = d.g_moe;
  w.e_gu = d.e_gate_up;
  w.e_gu_sc = d.e_gate_up_scale;
  w.e_dn = d.e_down;
  w.e_dn_sc = d.e_down_scale;
  w.e_ts = d.e_tensor_scale;
  w.k_cache = d.k_cache;
  w.v_cache = d.v_cache;
  w.window = d.window;
  return w;
}

msk_status report_device_error(msk_handle h, int32_t e);

// Device status of completed calls: the error word a call copied back once
// its event shows the copy landed (or when no eager call is pending, a copy
// made by a graph replay). A nonzero word is reported once; the device word
// stays set (every later launch does nothing) until the next call's reset
// clears it.
msk_status poll_device_status(msk_handle h, bool wait) {
  if (h->is_static) {
    // no pinned copy: only msk_synchronize reads the word, synchronously
    if (!wait) return MSK_OK;
    if (hipStreamSynchronize(h->last_stream) != hipSuccess) return fail(h, MSK_E_HIP, "hipStreamSynchronize failed");
    int32_t word = 0;
    if (hipMemcpy(&word, h->ws + h->lay.err, sizeof word, hipMemcpyDeviceToHost) != hipSuccess)
      return fail(h, MSK_E_HIP, "reading the device error word failed");
    if (word == 0) return MSK_OK;
    h->clear_err = true;
    return report_device_error(h, word);
  }
  if (h->done_pending) {
    hipError_t q = wait ? hipEventSynchronize(h->done) : hipEventQuery(h->done);
    if (q == hipErrorNotReady) return MSK_OK;
    if (q != hipSuccess) return fail(h, MSK_E_HIP, std::string("waiting for the previous call failed: ") + hipGetErrorString(q));
    h->done_pending = false;
  }
  const int32_t e = __atomic_load_n(h->err_host, __ATOMIC_ACQUIRE);
  if (e == 0) return MSK_OK;
  __atomic_store_n(h->err_host, 0, __ATOMIC_RELEASE);
  h->clear_err = true;
  return report_device_error(h, e);
}

msk_status report_device_error(msk_handle h, int32_t e) {
  if (e == MSK_E_INVALID)
    return fail(h, MSK_E_INVALID, "a previous call was given an invalid ctx_len or tree_mask (its outputs are invalid)");
  if (e == MSK_E_CAPACITY)
    return fail(h, MSK_E_CAPACITY, "a previous call had ctx_len + n_tokens > kv_capacity (its outputs are invalid)");
  char buf[128];
  snprintf(buf, sizeof buf, "a previous call reported device error %d (spin budget exceeded; its outputs are invalid)", e);
  return fail(h, MSK_E_TIMEOUT, buf);
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

msk_status check_io(msk_handle h, const msk_io* io, hipStream_t s) {
  if (!io) return fail(h, MSK_E_INVALID, "io is NULL");
  const msk_config& c = h->cfg;
  if (io->n_requests < 1 || io->n_requests > c.max_requests) return fail(h, MSK_E_INVALID, "n_requests out of range");
  if (io->n_tokens < 1 || io->n_tokens > c.max_tokens) return fail(h, MSK_E_INVALID, "n_tokens out of range");
  if (!io->ctx_len) return fail(h, MSK_E_INVALID, "ctx_len is NULL");
  if (!aligned4(io->ctx_len)) return fail(h, MSK_E_ALIGN, "ctx_len must be 4-byte aligned");
  if (io->tree_mask && !aligned4(io->tree_mask)) return fail(h, MSK_E_ALIGN, "tree_mask must be 4-byte aligned");
  if (!io->h_in || !io->h_out) return fail(h, MSK_E_INVALID, "h_in and h_out are required");
  if (!aligned16(io->h_in) || !aligned16(io->h_out)) return fail(h, MSK_E_ALIGN, "h_in/h_out must be 16-byte aligned");
  if (io->layer_out && !aligned16(io->layer_out)) return fail(h, MSK_E_ALIGN, "layer_out must be 16-byte aligned");
  if (io->debug && io->trace) return fail(h, MSK_E_INVALID, "debug dumps and the trace are exclusive");
  if (io->trace && !aligned16(io->trace)) return fail(h, MSK_E_ALIGN, "trace must be 16-byte aligned");
  if ((io->expert_ids && !aligned16(io->expert_ids)) || (io->gates && !aligned16(io->gates)))
    return fail(h, MSK_E_ALIGN, "expert_ids/gates must be 16-byte aligned");
  if (io->prefetch_ids && !aligned16(io->prefetch_ids)) return fail(h, MSK_E_ALIGN, "prefetch_ids must be 16-byte aligned");
  // no event query while the stream is being captured (not permitted there)
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return fail(h, MSK_E_HIP, "hipStreamIsCapturing failed");
  if (cs != hipStreamCaptureStatusNone) return MSK_OK;
  return poll_device_status(h, false);
}

msk::Params base_params(msk_handle h, const msk_io* io) {
  const msk_config& c = h->cfg;
  const Layout& L = h->lay;
  msk::Params p;
  memset(&p, 0, sizeof p);
  p.H = c.hidden;
  p.nq = c.n_q_heads;
  p.nkv = c.n_kv_heads;
  p.d = c.head_dim;
  p.E = c.n_experts;
  p.topk = c.top_k;
  p.P = c.pool_dim;
  p.I = c.expert_inter;
  p.R = io->n_requests;
  p.T = io->n_tokens;
  p.NT = io->n_requests * io->n_tokens;
  p.cap = c.kv_capacity;
  p.use_norm = (c.flags & MSK_FLAG_NO_NORM) ? 0 : 1;
  p.act_fp4 = (c.flags & MSK_FLAG_ACT_FP4) ? 1 : 0;
  p.eps = c.rms_eps;
  p.ctx_dev = io->ctx_len;
  p.tree_dev = io->tree_mask;
  p.r0 = 0;
  p.q_slices = h->q_slices;
  p.p_slices = h->p_slices;
  uint8_t* ws = h->ws;
  p.bar = reinterpret_cast<uint32_t*>(ws + L.bar);
  p.err = reinterpret_cast<int32_t*>(ws + L.err);
  p.h1 = reinterpret_cast<float*>(ws + L.h1);
  p.ssq1 = reinterpret_cast<float*>(ws + L.ssq1);
  p.ssq2 = reinterpret_cast<float*>(ws + L.ssq2);
  p.qpart = reinterpret_cast<float*>(ws + L.qpart);
  p.apart = reinterpret_cast<float*>(ws + L.apart);
  p.attn = reinterpret_cast<uint16_t*>(ws + L.attn);
  p.logits = reinterpret_cast<float*>(ws + L.logits);
  p.ppart = reinterpret_cast<float*>(ws + L.ppart);
  p.abuf = reinterpret_cast<uint16_t*>(ws + L.abuf);
  {
    const size_t nsel = std::min<size_t>((size_t)c.n_experts, (size_t)pass_tokens(&c) * c.top_k);
    p.acode = ws + L.abuf;
    p.ascale = ws + L.abuf + nsel * pass_tokens(&c) * c.expert_inter / 2;
  }
  p.accpart = reinterpret_cast<float*>(ws + L.accpart);
  {
    int32_t* hist = reinterpret_cast<int32_t*>(ws + L.hist);
    const size_t n = (size_t)c.n_layers * c.n_experts;
    p.hist_wr = hist + (h->calls & 1) * n;
    p.hist_rd = hist + ((h->calls + 1) & 1) * n;
    p.hist_add = 0;
  }
  p.zeros = reinterpret_cast<const uint16_t*>(ws + L.zeros);
  p.wg_units = h->wg_units;
  p.wg_nunits = h->wg_nunits;
  p.n_prefetch = c.expert_prefetch;
  p.kv_prefetch = (c.flags & MSK_FLAG_KV_PREFETCH) ? 1 : 0;
  return p;
}

// Sequence numbers one launch uses: one per grid barrier, plus the router
// sums' own arrival before the pooler's.
int barriers_of(uint32_t mode) {
  int n = 7;
  if (mode & msk::kModeQkvOwn) n += 1;
  if (mode & msk::kModeQkvNext) n += 1;
  return n;
}

msk_status finish(msk_handle h, hipStream_t s) {
  const Layout& L = h->lay;
  h->last_stream = s;
  if (h->is_static) return MSK_OK;  // status read by msk_synchronize
  if (hipMemcpyAsync(h->err_host, h->ws + L.err, 4, hipMemcpyDeviceToHost, s) != hipSuccess)
    return fail(h, MSK_E_HIP, "hipMemcpyAsync of the error word failed");
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return fail(h, MSK_E_HIP, "hipStreamIsCapturing failed");
  if (cs == hipStreamCaptureStatusNone) {
    if (hipEventRecord(h->done, s) != hipSuccess) return fail(h, MSK_E_HIP, "hipEventRecord failed");
    h->done_pending = true;
  }
  return MSK_OK;
}

}  // namespace

namespace {

// Pointer to request r0's slice of a [R][nkv][cap][d] cache.
uint16_t* cache_at(uint16_t* base, int r0, const msk_config& c) {
  return base + (size_t)r0 * c.n_kv_heads * c.kv_capacity * c.head_dim;
}

msk::LayerW layer_for_pass(const msk_layer_desc& d, int r0, const msk_config& c) {
  msk::LayerW w = to_w(d);
  w.k_cache = cache_at(d.k_cache, r0, c);
  w.v_cache = cache_at(d.v_cache, r0, c);
  return w;
}

// Enqueues one verify call: layers [l0, l1) of the step (one launch each; the
// first launch also projects its own layer's QKV), run for the requests in
// passes of at most 16 tokens. Pass outputs go to the requests' own rows.
msk_status run_call(msk_handle h, int l0, int l1, const msk_io* io, hipStream_t s, bool debug) {
  const msk_config& c = h->cfg;
  const Layout& L = h->lay;
  const int T = io->n_tokens, R = io->n_requests, NT_all = R * T, K = c.top_k, H = c.hidden;
  const int rpp = requests_per_pass(T);
  const int n = l1 - l0;
  if ((io->debug || io->trace) && R > rpp)
    return fail(h, MSK_E_INVALID, "debug dumps and the trace need all tokens of the call in one 16-token pass");
  float* hb[2] = {reinterpret_cast<float*>(h->ws + L.hbuf0), reinterpret_cast<float*>(h->ws + L.hbuf1)};
  // residual leaving launch i of pass r0 (the last launch writes h_out)
  auto resid = [&](int i, int r0) -> float* {
    if (io->layer_out) return io->layer_out + (size_t)i * NT_all * H + (size_t)r0 * T * H;
    return hb[i & 1];
  };
  if (msk_launch_reset(reinterpret_cast<uint32_t*>(h->ws + L.bar), reinterpret_cast<int32_t*>(h->ws + L.err),
                       h->clear_err, s) != hipSuccess)
    return fail(h, MSK_E_HIP, "reset launch failed");
  h->clear_err = false;
  uint32_t base = 0;
  for (int r0 = 0; r0 < R; r0 += rpp) {
    const int nr = std::min(rpp, R - r0);
    for (int i = 0; i < n; ++i) {
      const int l = l0 + i;
      msk::Params p = base_params(h, io);
      p.R = nr;
      p.NT = nr * T;
      p.r0 = r0;
      p.mode = (i == 0 ? msk::kModeQkvOwn : 0u) | (i + 1 < n ? msk::kModeQkvNext : 0u);
      p.layer = l;
      p.bar_base = base;
      p.cur = layer_for_pass(h->layers[l], r0, c);
      p.nxt = (i + 1 < n) ? layer_for_pass(h->layers[l + 1], r0, c) : p.cur;
      p.h_in = (i == 0) ? io->h_in + (size_t)r0 * T * H : resid(i - 1, r0);
      p.h_out = (i == n - 1) ? io->h_out + (size_t)r0 * T * H : resid(i, r0);
      const size_t row0 = (size_t)i * NT_all * K + (size_t)r0 * T * K;
      p.out_ids = io->expert_ids ? io->expert_ids + row0 : nullptr;
      p.out_gates = io->gates ? io->gates + row0 : nullptr;
      // the speculative prefetch runs in the first pass, from the previous call's counts
      p.n_prefetch = r0 == 0 ? c.expert_prefetch : 0;
      p.out_prefetch = (r0 == 0 && io->prefetch_ids) ? io->prefetch_ids + (size_t)i * c.expert_prefetch : nullptr;
      p.hist_add = r0 > 0;
      p.trace = io->trace;
      p.trace_launch = i;
      if (debug) {
        const msk_debug& d = *io->debug;
        p.dbg = msk::Debug{d.q, d.k_new, d.v_new, d.attn, d.h1, d.n2, d.logits, d.p, d.acc,
                           d.dq_expert, d.dq_gate_up, d.dq_down, d.act, d.act_codes, d.act_scales,
                           d.act_codes_all, d.act_scales_all};
      }
      hipError_t e = msk_launch_layer(p, h->grid, debug, s);
      if (e != hipSuccess) return fail(h, MSK_E_HIP, std::string("layer launch failed: ") + hipGetErrorString(e));
      base += barriers_of(p.mode);
    }
  }
  if (io->layer_out &&
      hipMemcpyAsync(io->layer_out + (size_t)(n - 1) * NT_all * H, io->h_out, (size_t)NT_all * H * sizeof(float),
                     hipMemcpyDeviceToDevice, s) != hipSuccess)
    return fail(h, MSK_E_HIP, "hipMemcpyAsync of the last layer's residual failed");
  h->calls += 1;
  return finish(h, s);
}

}  // namespace

extern "C" msk_status msk_verify_layer(msk_handle h, int32_t layer, const msk_io* io, void* stream) {
  if (!h) return fail(nullptr, MSK_E_INVALID, "handle is NULL");
  if (layer < 0 || layer >= h->cfg.n_layers) return fail(h, MSK_E_INVALID, "layer out of range");
  if (!h->loaded[layer]) return fail(h, MSK_E_STATE, "layer not loaded");
  msk_status st = check_io(h, io, (hipStream_t)stream);
  if (st != MSK_OK) return st;
  return run_call(h, layer, layer + 1, io, (hipStream_t)stream, io->debug != nullptr);
}

extern "C" msk_status msk_verify_step(msk_handle h, const msk_io* io, void* stream) {
  if (!h) return fail(nullptr, MSK_E_INVALID, "handle is NULL");
  for (int l = 0; l < h->cfg.n_layers; ++l)
    if (!h->loaded[l]) return fail(h, MSK_E_STATE, "not every layer is loaded");
  msk_status st = check_io(h, io, (hipStream_t)stream);
  if (st != MSK_OK) return st;
  if (io->debug) return fail(h, MSK_E_INVALID, "debug dumps are honoured by msk_verify_layer only");
  return run_call(h, 0, h->cfg.n_layers, io, (hipStream_t)stream, false);
}

extern "C" msk_status msk_synchronize(msk_handle h) {
  if (!h) return fail(nullptr, MSK_E_INVALID, "handle is NULL");
  return poll_device_status(h, true);
}

extern "C" msk_status msk_destroy(msk_handle h) {
  if (!h) return fail(nullptr, MSK_E_INVALID, "handle is NULL");
  if (h->done) (void)hipEventDestroy(h->done);
  if (h->err_host) (void)hipHostFree(h->err_host);
  delete h;
  return MSK_OK;
}

extern "C" size_t msk_down_scale_bytes(int32_t n_experts, int32_t pool_dim, int32_t expert_inter) {
  if (n_experts <= 0 || pool_dim <= 0 || pool_dim % 16 != 0 || expert_inter <= 0 || expert_inter % 32 != 0) return 0;
  return (size_t)n_experts * pool_dim * msk::dn_scale_slices(expert_inter) * 8;
}

extern "C" msk_status msk_pack_down_scale(const void* src, void* dst, int32_t n_experts, int32_t pool_dim,
                                          int32_t expert_inter, void* stream) {
  if (!src || !dst) return fail(nullptr, MSK_E_INVALID, "src and dst are required");
  if (!aligned16(src) || !aligned16(dst)) return fail(nullptr, MSK_E_ALIGN, "src and dst must be 16-byte aligned");
  if (msk_down_scale_bytes(n_experts, pool_dim, expert_inter) == 0)
    return fail(nullptr, MSK_E_SHAPE, "n_experts > 0, pool_dim a multiple of 16, expert_inter a multiple of 32 required");
  const hipError_t e = msk_launch_pack_down_scale(static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), n_experts,
                                                  pool_dim, expert_inter, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(nullptr, MSK_E_HIP, std::string("scale packing launch failed: ") + hipGetErrorString(e));
  return MSK_OK;
}

extern "C" const char* msk_last_error(msk_handle h) {
  if (!h) return g_create_error.c_str();
  return h->last_error.c_str();
}
