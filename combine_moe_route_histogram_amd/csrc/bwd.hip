// Expert-FFN backward in one persistent launch, with the weight-gradient
// ("W") tiles scheduled into the gaps of the data-gradient ("B") chain.
//
// ZB2P's split of the backward (GraphPP article, section on zero-bubble
// pipeline schedules): the input gradient needs only the activation gradient,
// the weight gradients can run whenever their operands exist, so they fill
// the bubbles of the data-gradient chain.  On one GPU the bubbles of four
// separate launches are the tails of each launch (the last partial round of
// tiles) and the full stop between the activation gradient and the input
// gradient that reads it.  Here one set of persistent workers runs four
// phases of tiles, each phase in per-XCD ranges with stealing as in the plain
// launches:
//   1. activation gradient: dh = dY W2^T, SwiGLU backward -> da | db
//   2. dW2 = h^T dY            (needs nothing from phase 1)
//   3. input gradient: dx = [da db] [W1 W3]^T   (reads phase 1's output)
//   4. dW1 | dW3 = X^T [da db]                  (reads phase 1's output)
// A worker moves to the next phase when the current phase has no unclaimed
// tile, so phase 2 tiles fill the tail of phase 1, phase 3 tiles the tail of
// phase 2, and so on.
//
// Visibility of phase 1's output: every worker, on leaving phase 1, waits for
// its own stores, takes one agent-scope release (one write-back of its XCD's
// L2) and adds the number of phase-1 tiles it finished to a counter.  Before
// its first phase-3 tile a worker waits until that counter reaches the number
// of phase-1 tiles and takes one acquire; phases 3 and 4 then read da | db
// without further synchronisation.  One release and one acquire per worker,
// instead of one per tile: an acquire invalidates the XCD's L2, which per tile
// would throw away the operands that the XCD's other tiles are sharing.
//
// Deadlock freedom: the only waits are that one (on phase-1 tiles, which
// never wait and were all claimed by running workers before any worker can
// reach phase 3) and the split-tail owners of phase 3 (on their helpers,
// claimed before them; as in the plain launch).  Every wait ends whatever the
// number of resident workers.
//
// Determinism: each tile runs the tile code of the plain launch with the same
// operands, and phase 3 splits its tail exactly as the plain input-gradient
// launch does (the split depends only on the tile count), so every output is
// bit-identical to moe_expert_ffn_bwd_data followed by moe_expert_ffn_bwd_weight.
#include "gemm_tile.hpp"

namespace moe {

using BuCfg = BfPick<kBwdUp>::C;
using BdCfg = BfPick<kBwdDown>::C;
using WuCfg = BfPick<kWgUp>::C;
using WdCfg = BfPick<kWgDown>::C;
static_assert(BuCfg::NT == BdCfg::NT && BuCfg::NT == WuCfg::NT && BuCfg::NT == WdCfg::NT,
              "one workgroup size for every phase");
static_assert(BuCfg::STAGE_BYTES == BdCfg::STAGE_BYTES && BuCfg::STAGE_BYTES == WuCfg::STAGE_BYTES &&
                  BuCfg::STAGE_BYTES == WdCfg::STAGE_BYTES && BuCfg::STAGES == BdCfg::STAGES &&
                  BuCfg::STAGES == WuCfg::STAGES && BuCfg::STAGES == WdCfg::STAGES,
              "one LDS ring for every phase");
static_assert(BuCfg::BM == BdCfg::BM, "both data-gradient phases use one row-tile table");

template <bool R>
__global__ __launch_bounds__(BuCfg::NT) __attribute__((amdgpu_waves_per_eu(BuCfg::NW / 4, BuCfg::NW / 4)))
void ffn_bwd_kernel(GemmArgs g, FusedWs w, int band_wg_down, int band_wg_up) {
  MOE_LDS_RING(BuCfg, ring);
  __shared__ int task_slot;
  const int n_mt = *g.n_mtiles;
  const int nt_bu = gemm_ntiles<kBwdUp>(g.H, g.I, BuCfg::BN);
  const int nt_bd = gemm_ntiles<kBwdDown>(g.H, g.I, BdCfg::BN);
  const int mt_wd = (g.E + g.Ns) * wgrad_mtiles<kWgDown>(g.H, g.I, WdCfg::BM);
  const int nt_wd = gemm_ntiles<kWgDown>(g.H, g.I, WdCfg::BN);
  const int mt_wu = (g.E + g.Ns) * wgrad_mtiles<kWgUp>(g.H, g.I, WuCfg::BM);
  const int nt_wu = gemm_ntiles<kWgUp>(g.H, g.I, WuCfg::BN);
  int32_t* const p1_done = &w.cursor[0];
  int32_t* const cur = &w.cursor[1];

  // phase 1: activation gradient
  int mine = 0;
  for_tasks_xcd_ranges(cur, n_mt * nt_bu, 0, 1, &task_slot, [&](const TaskPart& tp) {
    int tm, tn;
    band_order_groups(tp.L, nt_bu, g.bands, tm, tn);
    const TileDesc<uint16_t> d = decode_tile<uint16_t, kBwdUp, BuCfg::BM, BuCfg::BN>(g, tm, tn);
    if (!d.skip) run_tile_bf16<BuCfg, false, R>(g, d, ring, tp);
    ++mine;
  }, g.perturb);
  // publish this worker's phase-1 rows: own stores complete, one release,
  // then the count
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (mine) __hip_atomic_fetch_add(p1_done, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // phase 2: dW2
  for_tasks_xcd_ranges(cur + kXcds, mt_wd * nt_wd, 0, 1, &task_slot, [&](const TaskPart& tp) {
    int tm, tn;
    band_order(tp.L, mt_wd, nt_wd, band_wg_down, tm, tn);
    const TileDesc<uint16_t> d = decode_tile<uint16_t, kWgDown, WdCfg::BM, WdCfg::BN>(g, tm, tn);
    if (!d.skip) run_tile_bf16<WdCfg, false, R>(g, d, ring, tp);
  }, g.perturb);

  // phases 3 and 4 read phase 1's output
  wait_count(g, p1_done, n_mt * nt_bu);

  // phase 3: input gradient, tail split as in the plain launch
  for_tasks_xcd_ranges(cur + 2 * kXcds, n_mt * nt_bd, g.split_wr, (2 * g.I + BdCfg::BK - 1) / BdCfg::BK,
                       &task_slot, [&](const TaskPart& tp) {
    int tm, tn;
    band_order_groups(tp.L, nt_bd, g.bands2, tm, tn);
    const TileDesc<uint16_t> d = decode_tile<uint16_t, kBwdDown, BdCfg::BM, BdCfg::BN>(g, tm, tn);
    if (!d.skip) run_tile_bf16<BdCfg, false, R>(g, d, ring, tp);
  }, g.perturb);

  // phase 4: dW1 | dW3
  for_tasks_xcd_ranges(cur + 3 * kXcds, mt_wu * nt_wu, 0, 1, &task_slot, [&](const TaskPart& tp) {
    int tm, tn;
    band_order(tp.L, mt_wu, nt_wu, band_wg_up, tm, tn);
    const TileDesc<uint16_t> d = decode_tile<uint16_t, kWgUp, WuCfg::BM, WuCfg::BN>(g, tm, tn);
    if (!d.skip) run_tile_bf16<WuCfg, false, R>(g, d, ring, tp);
  }, g.perturb);
}

hipError_t launch_ffn_bwd(const GemmArgs& a0, const Tuning& tu, const FusedWs& w, hipStream_t st) {
  GemmArgs a = a0;
  a.mtiles = w.mtiles;
  a.n_mtiles = w.n_mtiles;
  a.bands = w.bands;     // activation gradient: tuned bands
  a.bands2 = w.bands2;   // input gradient: the fixed bands of its plain launch (split tails)
  a.mt_max = w.mt_bound;
  // row tiles, both band tables, and every counter and cursor of the launch cleared
  hipError_t e = launch_plan(a.offsets, a.E, a.Ns, a.T, a.R, BuCfg::BM, tu.small_group, tu.band_act,
                             w.mtiles, w.n_mtiles, nullptr, w.bands, w.flags,
                             w.mt_bound + kFusedCursors + kXcds * kSplitWr, st, w.bands2, kSplitSmall,
                             split_kind_band(kBwdDown));
  if (e != hipSuccess) return e;
  const int64_t mt = mtile_bound(a.T, a.K, a.E, a.Ns, BuCfg::BM);
  const int64_t tiles = mt * gemm_ntiles<kBwdUp>(a.H, a.I, BuCfg::BN) +
                        mt * gemm_ntiles<kBwdDown>(a.H, a.I, BdCfg::BN) +
                        (int64_t)(a.E + a.Ns) * wgrad_mtiles<kWgDown>(a.H, a.I, WdCfg::BM) *
                            gemm_ntiles<kWgDown>(a.H, a.I, WdCfg::BN) +
                        (int64_t)(a.E + a.Ns) * wgrad_mtiles<kWgUp>(a.H, a.I, WuCfg::BM) *
                            gemm_ntiles<kWgUp>(a.H, a.I, WuCfg::BN);
  if (tiles > INT_MAX - 8) return hipErrorInvalidValue;
  if (ragged_k(a.H, a.I, BuCfg::BK))
    ffn_bwd_kernel<true><<<w.workers, BuCfg::NT, 0, st>>>(a, w, tu.band_wg_down, tu.band_wg_up);
  else
    ffn_bwd_kernel<false><<<w.workers, BuCfg::NT, 0, st>>>(a, w, tu.band_wg_down, tu.band_wg_up);
  return hipGetLastError();
}

hipError_t take_wait_error_bwd(uint32_t* out) { return take_wait_error(out); }

}  // namespace moe
