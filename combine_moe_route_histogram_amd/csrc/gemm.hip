// Plain (one launch per GEMM kind) grouped expert-FFN GEMMs and the row-tile
// planner.  Tile code lives in gemm_tile.hpp.
//
// Padding-free grouped GEMM (UniEP article, section 1.2): the rows of expert
// e are offsets[e]..offsets[e+1] of the expert-contiguous buffer; the row tiles
// of every group are listed by a one-wave planner straight from the device
// offsets, so the host never reads a count back.  Tiles never straddle two
// experts; the last tile of an expert is partial.
#include <algorithm>

#include "gemm_tile.hpp"

namespace moe {

// Row-tile table: per group (E routed experts, then Ns shared experts over
// all T tokens) ceil(rows / bm) entries {group, first row, rows, 0}, groups in
// order; n_mtiles[0] = number of entries.  Band table: a group of at most
// `small` row tiles is one band, a larger one runs of `big` row tiles
// (group_bands); bands[tm] = {first row tile, row tiles} of the band holding
// row tile tm (so a worker finds a tile's band with one load), n_mtiles[1] =
// number of bands; bands2 (if not null) likewise with small2, big2 and
// n_mtiles[2].  Wave 0 places the groups: each lane owns a contiguous run of
// groups, and wave scans give each group its first table index (kept in LDS).
// Then every thread writes table entries: entry i's group is the last one
// whose first index is <= i (a binary search in LDS).
constexpr int kPlanThreads = 256;
__global__ __launch_bounds__(kPlanThreads) void plan_mtiles_kernel(
    const int32_t* __restrict__ offsets, int E, int Ns, int T, int R, int bm, int small, int big,
    int4* __restrict__ mtiles, int32_t* __restrict__ n_mtiles, int32_t* __restrict__ first_tile,
    int2* __restrict__ bands, int2* __restrict__ bands2, int small2, int big2,
    int32_t* __restrict__ clear, int n_clear) {
  __shared__ int off_s[kMaxExperts + 1];
  __shared__ int first_s[kMaxExperts + kMaxShared + 1];   // per group, then the entry count
  const int tid = threadIdx.x;
  const int G = E + Ns;
  for (int e = tid; e <= E; e += kPlanThreads) off_s[e] = offsets[e];   // all loads in flight at once
  for (int i = tid; i < n_clear; i += kPlanThreads) clear[i] = 0;
  __syncthreads();
  auto group_rows = [&](int grp, int& row0, int& rows) {
    if (grp < E) {
      row0 = off_s[grp];
      rows = off_s[grp + 1] - row0;
    } else {
      row0 = R + (grp - E) * T;
      rows = T;
    }
  };
  if (tid < kWave) {
    const int lane = tid;
    const int per = (G + kWave - 1) / kWave;
    const int g_begin = min(G, lane * per), g_end = min(G, g_begin + per);
    int mine = 0, mine_b = 0, mine_b2 = 0;
    for (int grp = g_begin; grp < g_end; ++grp) {
      int row0, rows;
      group_rows(grp, row0, rows);
      const int mt = (rows + bm - 1) / bm;
      mine += mt;
      mine_b += group_bands(mt, small, big);
      if (bands2) mine_b2 += group_bands(mt, small2, big2);
    }
    int incl = mine, incl_b = mine_b, incl_b2 = mine_b2;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      const int yb = __shfl_up(incl_b, o, kWave);
      const int yb2 = __shfl_up(incl_b2, o, kWave);
      if (lane >= o) {
        incl += y;
        incl_b += yb;
        incl_b2 += yb2;
      }
    }
    int idx = incl - mine;
    for (int grp = g_begin; grp < g_end; ++grp) {
      int row0, rows;
      group_rows(grp, row0, rows);
      first_s[grp] = idx;
      if (first_tile) first_tile[grp] = idx;
      idx += (rows + bm - 1) / bm;
    }
    if (lane == kWave - 1) {
      first_s[G] = incl;
      n_mtiles[0] = incl;
      n_mtiles[1] = incl_b;
      if (bands2) n_mtiles[2] = incl_b2;
    }
  }
  __syncthreads();
  const int n_mt = first_s[G];
  for (int i = tid; i < n_mt; i += kPlanThreads) {
    int lo = 0, hi = G;   // first_s[lo] <= i < first_s[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (first_s[mid] <= i) lo = mid; else hi = mid;
    }
    const int f = first_s[lo], mt = first_s[lo + 1] - f, j = i - f;
    int row0, rows;
    group_rows(lo, row0, rows);
    mtiles[i] = make_int4(lo, row0 + j * bm, min(bm, rows - j * bm), 0);
    const int step = mt <= small ? small : big;
    const int c = j / step * step;
    bands[i] = make_int2(f + c, min(step, mt - c));
    if (bands2) {
      const int step2 = mt <= small2 ? small2 : big2;
      const int c2 = j / step2 * step2;
      bands2[i] = make_int2(f + c2, min(step2, mt - c2));
    }
  }
}

hipError_t launch_plan(const int32_t* offsets, int E, int Ns, int T, int R, int bm, int small,
                       int big, int4* mtiles, int32_t* n_mtiles, int32_t* first_tile,
                       int2* bands, int32_t* clear, int n_clear, hipStream_t st,
                       int2* bands2, int small2, int big2) {
  plan_mtiles_kernel<<<1, kPlanThreads, 0, st>>>(offsets, E, Ns, T, R, bm, small, big, mtiles, n_mtiles,
                                       first_tile, bands, bands2, small2, big2, clear, n_clear);
  return hipGetLastError();
}

// k length of the forward-shaped kinds (the same for every tile).
template <int KIND>
inline int64_t kind_k_len(const GemmArgs& a) {
  switch (KIND) {
    case kUp: return a.H;
    case kDown: return a.I;
    case kBwdUp: return a.H;
    case kBwdDown: return 2 * (int64_t)a.I;
    default: return 1;   // weight gradient: not split
  }
}

// Persistent workers over per-XCD tile ranges (see for_tasks_xcd_ranges).
// Forward kinds read the number of row tiles from the planner's device output,
// so the tile count is exact; weight-gradient kinds have a fixed tile grid.
template <class C, bool R>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::NW / 4, C::NW / 4)))
void gemm_bf16_kernel(GemmArgs g, int mt_fixed, int nt_count, int32_t* cursors, int max_parts) {
  MOE_LDS_RING(C, ring);
  __shared__ int task_slot;
  const int mt_count = KindTraits<C::KIND>::kWgrad ? mt_fixed : *g.n_mtiles;
  for_tasks_xcd_ranges(cursors, mt_count * nt_count, g.split_wr, max_parts, &task_slot,
                       [&](const TaskPart& tp) {
    int tm, tn;
    if constexpr (KindTraits<C::KIND>::kWgrad)
      band_order(tp.L, mt_count, nt_count, g.wg_band, tm, tn);
    else
      band_order_groups(tp.L, nt_count, g.bands, tm, tn);
    const TileDesc<uint16_t> d = decode_tile<uint16_t, C::KIND, C::BM, C::BN>(g, tm, tn);
    if (!d.skip) run_tile_bf16<C, false, R>(g, d, ring, tp);
  }, g.perturb);
}

__global__ __launch_bounds__(64) void clear_i32_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0;
}

template <int KIND>
__global__ __launch_bounds__(kF32NT) void gemm_f32_kernel(GemmArgs g, int mt_count, int nt_count) {
  __shared__ float smem_f[kF32LdsFloats];
  const int L = blockIdx.x;
  if (L >= mt_count * nt_count) return;
  const int tm = L % mt_count, tn = L / mt_count;
  const TileDesc<float> d = decode_tile<float, KIND, kF32BM, kF32BN>(g, tm, tn);
  if (d.skip) return;
  run_tile_f32<KIND>(g, d, smem_f);
}

template <int KIND>
static hipError_t launch_kind(bool is_bf16, GemmArgs a, const Tuning& tu, int4* mtiles_ws,
                              int32_t* n_ws, int2* bands_ws, int32_t* cursors, int workers,
                              hipStream_t st) {
  using C = typename BfPick<KIND>::C;
  const int BM = is_bf16 ? C::BM : kF32BM;
  const int BN = is_bf16 ? C::BN : kF32BN;
  int mt_count;
  if constexpr (!KindTraits<KIND>::kWgrad) {
    // bands: fixed for the kinds with split tails, else the tuned heights
    const int small = KindTraits<KIND>::kSplit ? kSplitSmall : tu.small_group;
    const int big = KindTraits<KIND>::kSplit ? split_kind_band(KIND)
                    : KIND == kUp ? tu.band_up : tu.band_act;
    // clears the tile cursors and, kFusedCursors - 1 ints on, the split counters
    const hipError_t e = launch_plan(a.offsets, a.E, a.Ns, a.T, a.R, BM, small, big, mtiles_ws, n_ws,
                                     nullptr, bands_ws, cursors,
                                     is_bf16 ? (kFusedCursors - 1) + kXcds * kSplitWr : 0, st);
    if (e != hipSuccess) return e;
    a.mtiles = mtiles_ws;
    a.n_mtiles = n_ws;
    a.bands = bands_ws;
    mt_count = (int)mtile_bound(a.T, a.K, a.E, a.Ns, BM);
    a.mt_max = mt_count;
  } else {
    mt_count = (a.E + a.Ns) * wgrad_mtiles<KIND>(a.H, a.I, BM);
    a.wg_band = KIND == kWgUp ? tu.band_wg_up : tu.band_wg_down;
    a.split_wr = 0;   // many tiles per launch: no tail split
    if (is_bf16) clear_i32_kernel<<<1, 64, 0, st>>>(cursors, kXcds);
  }
  if (!KindTraits<KIND>::kSplit) a.split_wr = 0;
  const int nt_count = gemm_ntiles<KIND>(a.H, a.I, BN);
  const int64_t tiles = (int64_t)mt_count * nt_count;
  if (tiles <= 0) return hipSuccess;
  if (tiles > INT_MAX - 8) return hipErrorInvalidValue;
  if (is_bf16) {
    const int grid = (int)std::min<int64_t>(tiles * kMaxSplit, workers);
    const int max_parts = (int)((kind_k_len<KIND>(a) + C::BK - 1) / C::BK);
    // H or I not a whole number of k slices: the instantiation with ragged k
    if (ragged_k(a.H, a.I, C::BK))
      gemm_bf16_kernel<C, true><<<grid, C::NT, 0, st>>>(a, mt_count, nt_count, cursors, max_parts);
    else
      gemm_bf16_kernel<C, false><<<grid, C::NT, 0, st>>>(a, mt_count, nt_count, cursors, max_parts);
  } else {
    gemm_f32_kernel<KIND><<<(int)tiles, kF32NT, 0, st>>>(a, mt_count, nt_count);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(bool is_bf16, int kind, const GemmArgs& a, const Tuning& tu,
                       int4* mtiles_ws, int32_t* n_mtiles_ws, int2* bands_ws, int32_t* cursors,
                       int workers, hipStream_t st) {
#define MOE_KIND(K) launch_kind<K>(is_bf16, a, tu, mtiles_ws, n_mtiles_ws, bands_ws, cursors, workers, st)
  switch (kind) {
    case kUp: return MOE_KIND(kUp);
    case kDown: return MOE_KIND(kDown);
    case kBwdUp: return MOE_KIND(kBwdUp);
    case kBwdDown: return MOE_KIND(kBwdDown);
    case kWgUp: return MOE_KIND(kWgUp);
    case kWgDown: return MOE_KIND(kWgDown);
    default: return hipErrorInvalidValue;
  }
#undef MOE_KIND
}

hipError_t take_wait_error_gemm(uint32_t* out) { return take_wait_error(out); }

}  // namespace moe
