// C ABI of the MoE expert layer (declared in include/moe.h): argument
// validation, workspace layout and kernel launches.  No call allocates,
// frees, copies to the host or synchronises.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "kernels.hpp"
#include "tuning.hpp"

using namespace moe;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace sections (byte offsets).
struct Layout {
  size_t chunk_counts, chunk_base, mtiles, n_mtiles, bands, bands2, first_tile, flags, split, total;
  int mt_bound;
};

Layout layout(const moe_dims* d) {
  Layout L;
  const size_t nchunk = (size_t)route_nchunk(d->T);
  const size_t mt = (size_t)mtile_bound(d->T, d->K, d->E, d->n_shared, kMinTileM);
  size_t off = 0;
  L.chunk_counts = off; off = align_up(off + nchunk * d->E * 4);
  L.chunk_base = off;   off = align_up(off + nchunk * d->E * 4);
  L.mtiles = off;       off = align_up(off + mt * 16);
  L.n_mtiles = off;     off = align_up(off + 16);
  L.bands = off;        off = align_up(off + mt * 8);
  L.bands2 = off;       off = align_up(off + mt * 8);
  L.first_tile = off;   off = align_up(off + (size_t)(d->E + d->n_shared) * 4);
  // row-tile counters, then the task cursors, then the split counters
  L.flags = off;        off = align_up(off + (mt + kFusedCursors + kXcds * kSplitWr) * 4);
  // partial tiles of the k-split tails (bf16 GEMMs: 256 x 256 f32 each)
  L.split = off;
  if (d->dtype == MOE_BF16) off = align_up(off + (size_t)kXcds * kSplitSlots * 256 * 256 * 4);
  L.total = off;
  L.mt_bound = (int)mt;
  return L;
}

template <typename T>
T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_dims(const moe_dims* d) {
  if (!d) return fail(MOE_EINVAL, "dims is NULL");
  if (d->T < 1) return fail(MOE_EINVAL, "T must be >= 1 (got %d)", d->T);
  if (d->E < 1 || d->E > kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "E must be in [1, %d] (got %d)", kMaxExperts, d->E);
  if (d->K < 1 || d->K > d->E)
    return fail(MOE_EUNSUPPORTED, "K must be in [1, E] (got K=%d, E=%d)", d->K, d->E);
  if (d->H <= 0 || d->H % 8)
    return fail(MOE_EUNSUPPORTED, "H must be a positive multiple of 8 (got %d)", d->H);
  if (d->I <= 0 || d->I % 8)
    return fail(MOE_EUNSUPPORTED, "I must be a positive multiple of 8 (got %d)", d->I);
  if (d->n_shared < 0 || d->n_shared > kMaxShared)
    return fail(MOE_EUNSUPPORTED, "n_shared must be in [0, %d] (got %d)", kMaxShared, d->n_shared);
  if (d->n_shared > 0 && d->I_shared != d->I)
    return fail(MOE_EUNSUPPORTED,
                "shared experts must have the routed experts' intermediate dim (I_shared=%d, I=%d)",
                d->I_shared, d->I);
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16)
    return fail(MOE_EUNSUPPORTED, "dtype must be MOE_F32 or MOE_BF16 (got %d)", d->dtype);
  const int64_t ra = (int64_t)d->T * d->K + (int64_t)d->n_shared * d->T;
  if (ra >= (int64_t)1 << 31) return fail(MOE_EUNSUPPORTED, "R + n_shared*T must be < 2^31");
  return MOE_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(MOE_EINVAL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16) return fail(MOE_EINVAL, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

int check_ws(const moe_dims* d, const void* ws, size_t ws_bytes) {
  const size_t need = layout(d).total;
  if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(MOE_EWORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
  return MOE_OK;
}

#define MOE_TRY(expr)            \
  do {                           \
    const int _s = (expr);       \
    if (_s != MOE_OK) return _s; \
  } while (0)

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Debug settings, read from the environment by moe_init only (never at a
// launch): the bound of the in-kernel waits in ticks of the 100 MHz clock
// (20 s, or MOE_WAIT_LIMIT_US microseconds), MOE_DEBUG_UNREACHABLE_WAITS=1
// (every wait's target one more than can happen: exercises the timeout
// record), MOE_DEBUG_PERTURB_SEED=n (seeded claim order and delays in the
// persistent GEMM launches; results must not change) and MOE_FUSED_WORKERS=n
// (persistent workers of the fused calls; results must not change).
struct DebugSettings {
  uint64_t wait_ticks = 20ull * 100000000ull;
  int wait_extra = 0;
  uint32_t perturb = 0;
  int fused_workers = 0;   // 0: one per CU
  moe_tuning tune = {0, 0, 0, 0, 0, 0, 0, -1};   // MOE_TUNE overrides (0 / -1: the shape's choice)
};
std::mutex g_debug_mu;
DebugSettings g_debug;

DebugSettings debug_settings() {
  std::lock_guard<std::mutex> lk(g_debug_mu);
  return g_debug;
}

// MOE_TUNE="key=value,...": schedule-knob overrides (keys as in moe_tuning).
// Returns false for a malformed string or a value outside the knob's range.
bool parse_tune(const char* e, moe_tuning* t) {
  *t = moe_tuning{0, 0, 0, 0, 0, 0, 0, -1};
  std::string s(e);
  size_t pos = 0;
  while (pos < s.size()) {
    size_t end = s.find(',', pos);
    if (end == std::string::npos) end = s.size();
    const std::string item = s.substr(pos, end - pos);
    pos = end + 1;
    if (item.empty()) continue;
    const size_t eq = item.find('=');
    if (eq == std::string::npos) return false;
    const std::string key = item.substr(0, eq);
    char* stop = nullptr;
    const long v = strtol(item.c_str() + eq + 1, &stop, 10);
    if (stop == item.c_str() + eq + 1 || *stop) return false;
    int32_t* slot = key == "band_up" ? &t->band_up : key == "band_act" ? &t->band_act
                  : key == "small_group" ? &t->small_group : key == "band_wgrad_up" ? &t->band_wgrad_up
                  : key == "band_wgrad_down" ? &t->band_wgrad_down
                  : key == "combine_tokens" ? &t->combine_tokens
                  : key == "copy_tokens" ? &t->copy_tokens
                  : key == "copy_in_tiles" ? &t->copy_in_tiles : nullptr;
    if (!slot) return false;
    const bool tokens = slot == &t->combine_tokens || slot == &t->copy_tokens;
    if (slot == &t->copy_in_tiles) {
      if (v < 0 || v > 1) return false;
    } else if (v < 1 || v > (tokens ? kMaxTaskTokens : kMaxBand)) {
      return false;
    }
    *slot = (int32_t)v;
  }
  return true;
}

bool read_debug_settings() {
  DebugSettings s;
  if (const char* e = getenv("MOE_TUNE")) {
    if (!parse_tune(e, &s.tune)) return false;
  }
  if (const char* e = getenv("MOE_WAIT_LIMIT_US")) {
    char* end = nullptr;
    const unsigned long long us = strtoull(e, &end, 10);
    if (end != e) s.wait_ticks = us * 100ull;
  }
  const char* u = getenv("MOE_DEBUG_UNREACHABLE_WAITS");
  s.wait_extra = (u && u[0] == '1') ? 1 : 0;
  if (const char* e = getenv("MOE_DEBUG_PERTURB_SEED")) s.perturb = (uint32_t)strtoul(e, nullptr, 10);
  if (const char* e = getenv("MOE_FUSED_WORKERS")) {
    const int n = atoi(e);
    s.fused_workers = n > 0 ? n : 0;
  }
  std::lock_guard<std::mutex> lk(g_debug_mu);
  g_debug = s;
  return true;
}

// The schedule knobs for these dims: the shape's choice (choose_tuning), then
// any MOE_TUNE override.
Tuning tuning_for(const moe_dims* d) {
  moe_tuning t = choose_tuning(d->T, d->H, d->E, d->K, d->I, d->n_shared);
  const moe_tuning o = debug_settings().tune;
  if (o.band_up) t.band_up = o.band_up;
  if (o.band_act) t.band_act = o.band_act;
  if (o.small_group) t.small_group = o.small_group;
  if (o.band_wgrad_up) t.band_wgrad_up = o.band_wgrad_up;
  if (o.band_wgrad_down) t.band_wgrad_down = o.band_wgrad_down;
  if (o.combine_tokens) t.combine_tokens = o.combine_tokens;
  if (o.copy_tokens) t.copy_tokens = o.copy_tokens;
  if (o.copy_in_tiles >= 0) t.copy_in_tiles = o.copy_in_tiles;
  Tuning u;
  u.band_up = t.band_up; u.band_act = t.band_act; u.small_group = t.small_group;
  u.band_wg_up = t.band_wgrad_up; u.band_wg_down = t.band_wgrad_down;
  u.combine_tokens = t.combine_tokens; u.copy_tokens = t.copy_tokens;
  u.copy_in_tiles = t.copy_in_tiles;
  return u;
}

void wait_bounds(GemmArgs& a) {
  const DebugSettings s = debug_settings();
  a.wait_ticks = s.wait_ticks;
  a.wait_extra = s.wait_extra;
  a.perturb = s.perturb;
}

GemmArgs base_args(const moe_dims* d, const int32_t* offsets, void* ws) {
  GemmArgs a{};
  wait_bounds(a);
  a.T = d->T; a.H = d->H; a.E = d->E; a.K = d->K; a.I = d->I; a.Ns = d->n_shared;
  a.R = d->T * d->K;
  a.offsets = offsets;
  if (d->dtype == MOE_BF16 && ws) {
    const Layout L = layout(d);
    a.split_part = ws_at<float>(ws, L.split);
    a.split_cnt = ws_at<int32_t>(ws, L.flags) + L.mt_bound + kFusedCursors;
    a.split_wr = kSplitWr;
  }
  return a;
}

int current_cu_count(int* out);

// Plain GEMM launch; the bf16 workers use the tile cursors of the fused
// kernels' section (never in use by two launches at once: both are ordered on
// the caller's stream).
int gemm(const moe_dims* d, int kind, const GemmArgs& a, void* ws, hipStream_t st, const char* what) {
  const Layout L = layout(d);
  int workers = 0;
  MOE_TRY(current_cu_count(&workers));
  int32_t* cursors = ws_at<int32_t>(ws, L.flags) + L.mt_bound + 1;
  return hip_status(launch_gemm(d->dtype == MOE_BF16, kind, a, tuning_for(d), ws_at<int4>(ws, L.mtiles),
                                ws_at<int32_t>(ws, L.n_mtiles), ws_at<int2>(ws, L.bands),
                                cursors, workers, st),
                    what);
}

struct DeviceCache {
  std::mutex mu;
  int cu_count[64] = {0};
};
DeviceCache g_dev;

// CU count of the current device (cached).
int current_cu_count(int* out) {
  int dev = 0;
  MOE_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= 64) return fail(MOE_EINVAL, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev.mu);
  if (!g_dev.cu_count[dev]) {
    int n = 0;
    MOE_TRY(hip_status(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev),
                       "hipDeviceGetAttribute"));
    g_dev.cu_count[dev] = n;
  }
  *out = g_dev.cu_count[dev];
  return MOE_OK;
}

// Workspace sections of the fused kernels; one persistent worker per CU
// (each uses most of a CU's LDS).
int fused_ws(const moe_dims* d, void* ws, FusedWs* w) {
  const Layout L = layout(d);
  w->mtiles = ws_at<int4>(ws, L.mtiles);
  w->n_mtiles = ws_at<int32_t>(ws, L.n_mtiles);
  w->first_tile = ws_at<int32_t>(ws, L.first_tile);
  w->bands = ws_at<int2>(ws, L.bands);
  w->bands2 = ws_at<int2>(ws, L.bands2);
  w->flags = ws_at<int32_t>(ws, L.flags);
  w->cursor = w->flags + L.mt_bound;
  w->mt_bound = L.mt_bound;
  MOE_TRY(current_cu_count(&w->workers));
  // debug: this many persistent workers instead, to check that results do not
  // depend on how many workers share the tasks
  const int n = debug_settings().fused_workers;
  if (n > 0) w->workers = n;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_init(int device) {
  if (device < 0 || device >= 64) return fail(MOE_EINVAL, "device index %d out of range", device);
  if (!read_debug_settings())
    return fail(MOE_EINVAL, "MOE_TUNE must be key=value[,key=value...] with keys band_up, band_act, "
                "small_group, band_wgrad_up, band_wgrad_down (1..%d), combine_tokens, copy_tokens "
                "(1..%d)", kMaxBand, kMaxTaskTokens);
  // device address of moe_route_noalloc's fixed scratch on this device
  MOE_TRY(hip_status(route_scratch_prepare(device), "moe_init (route scratch)"));
  std::lock_guard<std::mutex> lk(g_dev.mu);
  if (g_dev.cu_count[device]) return MOE_OK;
  int n = 0;
  MOE_TRY(hip_status(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device),
                     "hipDeviceGetAttribute"));
  g_dev.cu_count[device] = n;
  return MOE_OK;
}

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE";
    case MOE_EHIP: return "MOE_EHIP";
    case MOE_ETIMEOUT: return "MOE_ETIMEOUT";
    default: return "MOE_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int moe_get_tuning(const moe_dims* d, moe_tuning* out) {
  MOE_TRY(check_dims(d));
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  const Tuning u = tuning_for(d);
  out->band_up = u.band_up; out->band_act = u.band_act; out->small_group = u.small_group;
  out->band_wgrad_up = u.band_wg_up; out->band_wgrad_down = u.band_wg_down;
  out->combine_tokens = u.combine_tokens; out->copy_tokens = u.copy_tokens;
  out->copy_in_tiles = u.copy_in_tiles;
  return MOE_OK;
}

double moe_tuning_predict(const moe_dims* d, const char* knob, int value) {
  if (check_dims(d) != MOE_OK || !knob || value < 1 || value > kMaxBand) return -1.0;
  const Tuning u = tuning_for(d);
  const std::string k(knob);
  auto pred = [&](bool act, int band, int small) {
    return predict_traffic(d->T, d->H, d->E, d->K, d->I, d->n_shared, act, band, small);
  };
  if (k == "band_up") return pred(false, value, u.small_group);
  if (k == "band_act") return pred(true, value, u.small_group);
  if (k == "small_group") return pred(false, u.band_up, value) + pred(true, u.band_act, value);
  return -1.0;
}

size_t moe_workspace_bytes(const moe_dims* d) {
  if (check_dims(d) != MOE_OK) return 0;
  return layout(d).total;
}

int moe_route(const moe_dims* d, const float* logits, int32_t* topk_idx, float* topk_w,
              int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* slot_src, void* ws,
              size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(counts, "counts"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(slot_src, "slot_src"));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  const Layout L = layout(d);
  return hip_status(launch_route(logits, d->T, d->E, d->K, topk_idx, topk_w, counts, offsets, slot,
                                 slot_src, ws_at<int32_t>(ws, L.chunk_counts),
                                 ws_at<int32_t>(ws, L.chunk_base), as_stream(stream)),
                    "moe_route");
}

int moe_route_noalloc(const moe_dims* d, const float* logits, int32_t* topk_idx, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* slot_src,
                      void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(logits, "logits"));
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(counts, "counts"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(slot_src, "slot_src"));
  if (!route_scratch_fits(d->T, d->E))
    return fail(MOE_EUNSUPPORTED,
                "moe_route_noalloc: ceil(T/64)*E = %lld exceeds the fixed scratch (%lld); "
                "use moe_route with a workspace",
                (long long)route_nchunk(d->T) * d->E, (long long)kRouteScratchInts / 2);
  int32_t* sc = nullptr;
  MOE_TRY(hip_status(route_scratch_current(&sc), "moe_route_noalloc (scratch address)"));
  const size_t half = (size_t)route_nchunk(d->T) * d->E;
  return hip_status(launch_route(logits, d->T, d->E, d->K, topk_idx, topk_w, counts, offsets, slot,
                                 slot_src, sc, sc + half, as_stream(stream)),
                    "moe_route_noalloc");
}

size_t moe_route_ranks_workspace_bytes(const moe_dims* d, int G) {
  if (check_dims(d) != MOE_OK || G < 1 || G > d->T) return 0;
  const size_t nmax = (size_t)route_ranks_nchunk(d->T, G);
  return align_up((2 * nmax * d->E + (nmax + 1) + (size_t)(G + 1)) * 4);
}

int moe_route_ranks(const moe_dims* d, const int32_t* topk_idx, int G, int32_t* rank_counts,
                    int32_t* rank_base, int32_t* counts, int32_t* offsets, int32_t* slot,
                    int32_t* slot_src, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  if (G < 1 || G > d->T) return fail(MOE_EINVAL, "G must be in [1, T] (got G=%d, T=%d)", G, d->T);
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(rank_counts, "rank_counts"));
  MOE_TRY(check_ptr(rank_base, "rank_base"));
  MOE_TRY(check_ptr(counts, "counts"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(slot_src, "slot_src"));
  const size_t need = moe_route_ranks_workspace_bytes(d, G);
  if (!ws) return fail(MOE_EWORKSPACE, "workspace is NULL");
  if (ws_bytes < need)
    return fail(MOE_EWORKSPACE, "workspace too small: %zu bytes, need %zu", ws_bytes, need);
  const size_t nmax = (size_t)route_ranks_nchunk(d->T, G);
  int32_t* w = static_cast<int32_t*>(ws);
  int32_t* chunk_counts = w;
  int32_t* chunk_base = chunk_counts + nmax * d->E;
  int32_t* chunk_t0 = chunk_base + nmax * d->E;
  int32_t* rank_chunk = chunk_t0 + nmax + 1;
  return hip_status(launch_route_ranks(topk_idx, d->T, d->E, d->K, G, rank_counts, rank_base, counts,
                                       offsets, slot, slot_src, chunk_counts, chunk_base, chunk_t0,
                                       rank_chunk, as_stream(stream)),
                    "moe_route_ranks");
}

int moe_dispatch(const moe_dims* d, const void* x, const int32_t* slot, void* x_perm, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(x_perm, "x_perm"));
  return hip_status(launch_dispatch(d->dtype == MOE_BF16, x, slot, x_perm, d->T, d->H, d->K,
                                    as_stream(stream)),
                    "moe_dispatch");
}

int moe_expert_ffn_up(const moe_dims* d, const void* x_perm, const void* x, const int32_t* offsets,
                      const void* w1, const void* w3, const void* ws1, const void* ws3, void* ab,
                      void* h, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(x_perm, "x_perm"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(w1, "w1"));
  MOE_TRY(check_ptr(w3, "w3"));
  MOE_TRY(check_ptr(ab, "ab"));
  MOE_TRY(check_ptr(h, "h"));
  if (d->n_shared) {
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(ws1, "ws1"));
    MOE_TRY(check_ptr(ws3, "ws3"));
  }
  MOE_TRY(check_ws(d, ws, ws_bytes));
  GemmArgs a = base_args(d, offsets, ws);
  a.x_perm = x_perm; a.x = x; a.w1 = w1; a.w3 = w3; a.ws1 = ws1; a.ws3 = ws3;
  a.o_ab = ab; a.o_h = h;
  return gemm(d, kUp, a, ws, as_stream(stream), "moe_expert_ffn_up");
}

int moe_expert_ffn_down(const moe_dims* d, const void* h, const int32_t* offsets, const void* w2,
                        const void* ws2, void* y, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(h, "h"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(w2, "w2"));
  MOE_TRY(check_ptr(y, "y"));
  if (d->n_shared) MOE_TRY(check_ptr(ws2, "ws2"));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  GemmArgs a = base_args(d, offsets, ws);
  a.h = h; a.w2 = w2; a.ws2 = ws2; a.o_y = y;
  return gemm(d, kDown, a, ws, as_stream(stream), "moe_expert_ffn_down");
}

int moe_expert_ffn(const moe_dims* d, const void* x_perm, const void* x, const int32_t* offsets,
                   const void* w1, const void* w3, const void* w2, const void* ws1,
                   const void* ws3, const void* ws2, void* ab, void* h, void* y, void* ws,
                   size_t ws_bytes, void* stream) {
  MOE_TRY(moe_expert_ffn_up(d, x_perm, x, offsets, w1, w3, ws1, ws3, ab, h, ws, ws_bytes, stream));
  return moe_expert_ffn_down(d, h, offsets, w2, ws2, y, ws, ws_bytes, stream);
}

int moe_combine(const moe_dims* d, const void* y, const int32_t* slot, const float* topk_w,
                void* out, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(y, "y"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(out, "out"));
  return hip_status(launch_combine(d->dtype == MOE_BF16, y, slot, topk_w, out, d->T, d->H, d->K,
                                   d->n_shared, as_stream(stream)),
                    "moe_combine");
}

int moe_dispatch_ffn(const moe_dims* d, const void* x, const int32_t* slot_src,
                     const int32_t* slot, const int32_t* offsets, const void* w1, const void* w3,
                     const void* ws1, const void* ws3, void* x_perm, void* ab, void* h, void* ws,
                     size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(x, "x"));
  MOE_TRY(check_ptr(slot_src, "slot_src"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(w1, "w1"));
  MOE_TRY(check_ptr(w3, "w3"));
  MOE_TRY(check_ptr(x_perm, "x_perm"));
  MOE_TRY(check_ptr(ab, "ab"));
  MOE_TRY(check_ptr(h, "h"));
  if (d->n_shared) {
    MOE_TRY(check_ptr(ws1, "ws1"));
    MOE_TRY(check_ptr(ws3, "ws3"));
  }
  MOE_TRY(check_ws(d, ws, ws_bytes));
  const hipStream_t st = as_stream(stream);
  // f32 has no persistent kernel, the bf16 one reads token rows with 32-bit
  // byte offsets and its copy tasks hold at most 64 pairs per token: otherwise
  // a plain gather and the plain GEMM launch give the same result
  if (d->dtype != MOE_BF16 || (int64_t)d->T * d->H * 2 > 0x7FFF0000LL || d->K > 64) {
    MOE_TRY(hip_status(launch_gather(d->dtype == MOE_BF16, x, slot_src, x_perm, d->T * d->K, d->H, st),
                       "moe_dispatch_ffn (gather)"));
    return moe_expert_ffn_up(d, x_perm, x, offsets, w1, w3, ws1, ws3, ab, h, ws, ws_bytes, stream);
  }
  GemmArgs a = base_args(d, offsets, ws);
  a.x_perm = x_perm; a.o_x_perm = x_perm; a.x = x; a.w1 = w1; a.w3 = w3; a.ws1 = ws1; a.ws3 = ws3;
  a.o_ab = ab; a.o_h = h;
  FusedWs w;
  MOE_TRY(fused_ws(d, ws, &w));
  return hip_status(launch_dispatch_ffn(a, tuning_for(d), slot_src, slot, w, st), "moe_dispatch_ffn");
}

int moe_ffn_combine(const moe_dims* d, const void* h, const int32_t* offsets, const void* w2,
                    const void* ws2, const int32_t* slot, const float* topk_w, void* y, void* out,
                    void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(h, "h"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(w2, "w2"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(y, "y"));
  MOE_TRY(check_ptr(out, "out"));
  if (d->n_shared) MOE_TRY(check_ptr(ws2, "ws2"));
  MOE_TRY(check_ws(d, ws, ws_bytes));
  const hipStream_t st = as_stream(stream);
  if (d->dtype != MOE_BF16 || d->K > 64) {
    // f32 has no persistent kernel, and the bf16 one's combine tasks hold at
    // most 64 pairs per token: the two plain launches give the same result
    MOE_TRY(moe_expert_ffn_down(d, h, offsets, w2, ws2, y, ws, ws_bytes, stream));
    return moe_combine(d, y, slot, topk_w, out, stream);
  }
  GemmArgs a = base_args(d, offsets, ws);
  a.h = h; a.w2 = w2; a.ws2 = ws2; a.o_y = y; a.o_out = out;
  FusedWs w;
  MOE_TRY(fused_ws(d, ws, &w));
  return hip_status(launch_ffn_combine(a, tuning_for(d), slot, topk_w, w, st), "moe_ffn_combine");
}

int moe_combine_bwd(const moe_dims* d, const void* dout, const void* y, const int32_t* slot,
                    const float* topk_w, void* dy, float* dtopk_w, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(dout, "dout"));
  MOE_TRY(check_ptr(y, "y"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(dy, "dy"));
  MOE_TRY(check_ptr(dtopk_w, "dtopk_w"));
  return hip_status(launch_combine_bwd(d->dtype == MOE_BF16, dout, y, slot, topk_w, dy, dtopk_w,
                                       d->T, d->H, d->K, as_stream(stream)),
                    "moe_combine_bwd");
}

int moe_expert_ffn_bwd_act(const moe_dims* d, const void* dy, const void* dout,
                           const int32_t* offsets, const void* w2, const void* ws2,
                           const void* ab, void* dab, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(dy, "dy"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(w2, "w2"));
  MOE_TRY(check_ptr(ab, "ab"));
  MOE_TRY(check_ptr(dab, "dab"));
  if (d->n_shared) {
    MOE_TRY(check_ptr(dout, "dout"));
    MOE_TRY(check_ptr(ws2, "ws2"));
  }
  MOE_TRY(check_ws(d, ws, ws_bytes));
  GemmArgs a = base_args(d, offsets, ws);
  a.dy = dy; a.dout = dout; a.w2 = w2; a.ws2 = ws2; a.ab = ab; a.o_dab = dab;
  return gemm(d, kBwdUp, a, ws, as_stream(stream), "moe_expert_ffn_bwd_act");
}

int moe_expert_ffn_bwd_input(const moe_dims* d, const void* dab, const int32_t* offsets,
                             const void* w1, const void* w3, const void* ws1, const void* ws3,
                             void* dx_rows, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(dab, "dab"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(w1, "w1"));
  MOE_TRY(check_ptr(w3, "w3"));
  MOE_TRY(check_ptr(dx_rows, "dx_rows"));
  if (d->n_shared) {
    MOE_TRY(check_ptr(ws1, "ws1"));
    MOE_TRY(check_ptr(ws3, "ws3"));
  }
  MOE_TRY(check_ws(d, ws, ws_bytes));
  GemmArgs a = base_args(d, offsets, ws);
  a.dab = dab; a.w1 = w1; a.w3 = w3; a.ws1 = ws1; a.ws3 = ws3; a.o_dx = dx_rows;
  return gemm(d, kBwdDown, a, ws, as_stream(stream), "moe_expert_ffn_bwd_input");
}

int moe_expert_ffn_bwd_data(const moe_dims* d, const void* dy, const void* dout,
                            const int32_t* offsets, const void* w1, const void* w3,
                            const void* w2, const void* ws1, const void* ws3, const void* ws2,
                            const void* ab, void* dab, void* dx_rows, void* ws, size_t ws_bytes,
                            void* stream) {
  MOE_TRY(moe_expert_ffn_bwd_act(d, dy, dout, offsets, w2, ws2, ab, dab, ws, ws_bytes, stream));
  return moe_expert_ffn_bwd_input(d, dab, offsets, w1, w3, ws1, ws3, dx_rows, ws, ws_bytes, stream);
}

int moe_expert_ffn_bwd_weight_gate_up(const moe_dims* d, const void* x_perm, const void* x,
                                      const void* dab, const int32_t* offsets, float* dw1,
                                      float* dw3, float* dws1, float* dws3, void* ws,
                                      size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(x_perm, "x_perm"));
  MOE_TRY(check_ptr(dab, "dab"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(dw1, "dw1"));
  MOE_TRY(check_ptr(dw3, "dw3"));
  if (d->n_shared) {
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(dws1, "dws1"));
    MOE_TRY(check_ptr(dws3, "dws3"));
  }
  MOE_TRY(check_ws(d, ws, ws_bytes));
  GemmArgs a = base_args(d, offsets, ws);
  a.x_perm = x_perm; a.x = x; a.dab = dab;
  a.o_dw1 = dw1; a.o_dw3 = dw3; a.o_dws1 = dws1; a.o_dws3 = dws3;
  return gemm(d, kWgUp, a, ws, as_stream(stream), "moe_expert_ffn_bwd_weight_gate_up");
}

int moe_expert_ffn_bwd_weight_down(const moe_dims* d, const void* h, const void* dy,
                                   const void* dout, const int32_t* offsets, float* dw2,
                                   float* dws2, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(h, "h"));
  MOE_TRY(check_ptr(dy, "dy"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(dw2, "dw2"));
  if (d->n_shared) {
    MOE_TRY(check_ptr(dout, "dout"));
    MOE_TRY(check_ptr(dws2, "dws2"));
  }
  MOE_TRY(check_ws(d, ws, ws_bytes));
  GemmArgs a = base_args(d, offsets, ws);
  a.h = h; a.dy = dy; a.dout = dout; a.o_dw2 = dw2; a.o_dws2 = dws2;
  return gemm(d, kWgDown, a, ws, as_stream(stream), "moe_expert_ffn_bwd_weight_down");
}

int moe_expert_ffn_bwd_weight(const moe_dims* d, const void* x_perm, const void* x,
                              const void* h, const void* dy, const void* dout, const void* dab,
                              const int32_t* offsets, float* dw1, float* dw3, float* dw2,
                              float* dws1, float* dws3, float* dws2, void* ws, size_t ws_bytes,
                              void* stream) {
  MOE_TRY(moe_expert_ffn_bwd_weight_gate_up(d, x_perm, x, dab, offsets, dw1, dw3, dws1, dws3, ws,
                                            ws_bytes, stream));
  return moe_expert_ffn_bwd_weight_down(d, h, dy, dout, offsets, dw2, dws2, ws, ws_bytes, stream);
}

int moe_expert_ffn_bwd(const moe_dims* d, const void* dy, const void* dout,
                       const int32_t* offsets, const void* w1, const void* w3, const void* w2,
                       const void* ws1, const void* ws3, const void* ws2, const void* ab,
                       const void* x_perm, const void* x, const void* h, void* dab,
                       void* dx_rows, float* dw1, float* dw3, float* dw2, float* dws1,
                       float* dws3, float* dws2, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(d));
  if (d->dtype != MOE_BF16) {
    // f32 has no persistent kernel: the plain calls give the same result
    MOE_TRY(moe_expert_ffn_bwd_data(d, dy, dout, offsets, w1, w3, w2, ws1, ws3, ws2, ab, dab,
                                    dx_rows, ws, ws_bytes, stream));
    return moe_expert_ffn_bwd_weight(d, x_perm, x, h, dy, dout, dab, offsets, dw1, dw3, dw2, dws1,
                                     dws3, dws2, ws, ws_bytes, stream);
  }
  MOE_TRY(check_ptr(dy, "dy"));
  MOE_TRY(check_ptr(offsets, "offsets"));
  MOE_TRY(check_ptr(w1, "w1"));
  MOE_TRY(check_ptr(w3, "w3"));
  MOE_TRY(check_ptr(w2, "w2"));
  MOE_TRY(check_ptr(ab, "ab"));
  MOE_TRY(check_ptr(x_perm, "x_perm"));
  MOE_TRY(check_ptr(h, "h"));
  MOE_TRY(check_ptr(dab, "dab"));
  MOE_TRY(check_ptr(dx_rows, "dx_rows"));
  MOE_TRY(check_ptr(dw1, "dw1"));
  MOE_TRY(check_ptr(dw3, "dw3"));
  MOE_TRY(check_ptr(dw2, "dw2"));
  if (d->n_shared) {
    MOE_TRY(check_ptr(dout, "dout"));
    MOE_TRY(check_ptr(x, "x"));
    MOE_TRY(check_ptr(ws1, "ws1"));
    MOE_TRY(check_ptr(ws3, "ws3"));
    MOE_TRY(check_ptr(ws2, "ws2"));
    MOE_TRY(check_ptr(dws1, "dws1"));
    MOE_TRY(check_ptr(dws3, "dws3"));
    MOE_TRY(check_ptr(dws2, "dws2"));
  }
  MOE_TRY(check_ws(d, ws, ws_bytes));
  GemmArgs a = base_args(d, offsets, ws);
  a.dy = dy; a.dout = dout; a.w1 = w1; a.w3 = w3; a.w2 = w2; a.ws1 = ws1; a.ws3 = ws3; a.ws2 = ws2;
  a.ab = ab; a.x_perm = x_perm; a.x = x; a.h = h; a.dab = dab;
  a.o_dab = dab; a.o_dx = dx_rows;
  a.o_dw1 = dw1; a.o_dw3 = dw3; a.o_dw2 = dw2; a.o_dws1 = dws1; a.o_dws3 = dws3; a.o_dws2 = dws2;
  FusedWs w;
  MOE_TRY(fused_ws(d, ws, &w));
  return hip_status(launch_ffn_bwd(a, tuning_for(d), w, as_stream(stream)), "moe_expert_ffn_bwd");
}

int moe_sync_status(void* stream) {
  MOE_TRY(hip_status(hipStreamSynchronize(as_stream(stream)), "moe_sync_status"));
  uint32_t any = 0;
  hipError_t (*const take[])(uint32_t*) = {take_wait_error_gemm, take_wait_error_fused,
                                           take_wait_error_bwd};
  for (auto f : take) {
    uint32_t v = 0;
    MOE_TRY(hip_status(f(&v), "moe_sync_status"));
    any |= v;
  }
  if (any) return fail(MOE_ETIMEOUT, "a bounded wait inside a kernel gave up; results are invalid");
  return MOE_OK;
}

int moe_dispatch_bwd(const moe_dims* d, const void* dx_rows, const int32_t* slot, void* dx,
                     void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(dx_rows, "dx_rows"));
  MOE_TRY(check_ptr(slot, "slot"));
  MOE_TRY(check_ptr(dx, "dx"));
  return hip_status(launch_dispatch_bwd(d->dtype == MOE_BF16, dx_rows, slot, dx, d->T, d->H, d->K,
                                        d->n_shared, as_stream(stream)),
                    "moe_dispatch_bwd");
}

int moe_route_bwd(const moe_dims* d, const float* dtopk_w, const float* topk_w,
                  const int32_t* topk_idx, float* dlogits, void* stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(check_ptr(dtopk_w, "dtopk_w"));
  MOE_TRY(check_ptr(topk_w, "topk_w"));
  MOE_TRY(check_ptr(topk_idx, "topk_idx"));
  MOE_TRY(check_ptr(dlogits, "dlogits"));
  return hip_status(launch_route_bwd(dtopk_w, topk_w, topk_idx, dlogits, d->T, d->E, d->K,
                                     as_stream(stream)),
                    "moe_route_bwd");
}

}  // extern "C"
