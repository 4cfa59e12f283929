// Fused persistent kernels: Dispatch+GroupGEMM and GroupGEMM+Combine.
//
// UniEP article, section 2.1/2.2: one launch per fused stage, a fixed set of
// persistent workers that take tasks from global atomic cursors, and a
// scoreboard in global memory that a task polls before it may start.
//
// Dispatch+GroupGEMM.  On one GPU the "communication" of dispatch is the
// gather of token rows into the expert-contiguous order.  MI355X difference
// from a gather task that GEMM tiles wait for: the direct-to-LDS operand
// loads take a byte offset per lane, so a tile reads its routed rows straight
// from the token rows through the slot map; the gather costs nothing extra
// and no tile waits.  The expert-contiguous copy x_perm (the backward reads
// it) is written by tasks after the tiles, on workers the tile tail leaves
// idle, token by token (each token row read once, written to its K slots).
//
// GroupGEMM+Combine.  Combine tasks come after the GEMM tiles; each completed
// tile adds one to its row tile's counter, and a token is combined once the
// row tiles of all its rows are complete.  The tiles write their output rows
// with agent-coherent stores and publish without a release fence (see
// publish_add); a combine task takes one acquire after its polls.
//
// MI355X difference from the single cursor of the article: the GEMM tiles are
// split into 8 contiguous ranges in the plain launch's tile order, one per XCD
// (workers are handed to the XCDs round robin, worker b to XCD b % 8), each
// with its own cursor; a worker takes tiles from its XCD's range, then steals
// from the others.  Tiles that share weight columns and token rows then run
// on one XCD and share its L2, as in the plain launch.
//
// Deadlock freedom: combine tasks wait on GEMM tiles, and the owner of a
// split tail tile waits on its helper parts.  A worker takes combine tasks
// only once every tile has been claimed, and a split tile's helpers are
// claimed before its owner; helpers and whole tiles never wait, so every wait
// is on work that a running worker has already claimed and will finish,
// whatever the number of resident workers.  (Each wait is also bounded in
// time; one that gives up is recorded for moe_sync_status.)
//
// Determinism: every GEMM tile runs the same tile code with the same operands
// as the plain launch and every combine row the same combine code, so the
// outputs are bit-identical to the unfused calls whatever order the workers
// take the tasks in.
#include "gemm_tile.hpp"
#include "rows.hpp"

namespace moe {

using UpCfg = BfPick<kUp>::C;
using DownCfg = BfPick<kDown>::C;


// kCopyInTiles: x_perm is written by the GEMM tiles from the gathered rows in
// LDS (run_tile_bf16's kCopyA) instead of by copy tasks after the tiles.
template <bool R, bool kCopyInTiles>
__global__ __launch_bounds__(UpCfg::NT) void dispatch_ffn_kernel(GemmArgs g,
                                                                  const int32_t* __restrict__ slot,
                                                                  FusedWs w, int nt_count) {
  using C = UpCfg;
  MOE_LDS_RING(C, ring);
  __shared__ int task_slot;
  const int n_mt = *w.n_mtiles;
  // phase 1: GEMM tiles; the routed rows' A operand is gathered from the token
  // rows as it is loaded (g.a_rows = slot_src), so no tile waits for anything
  for_tasks_xcd_ranges(w.cursor + 1, n_mt * nt_count, 0, 1,
                       &task_slot, [&](const TaskPart& tp) {
    int tm, tn;
    band_order_groups(tp.L, nt_count, w.bands, tm, tn);
    const TileDesc<uint16_t> d = decode_tile<uint16_t, kUp, C::BM, C::BN>(g, tm, tn);
    run_tile_bf16<C, false, R, kCopyInTiles>(g, d, ring, tp);
  }, g.perturb);
  if constexpr (kCopyInTiles) return;
  // phase 2: the permuted copy x_perm (an output the backward reads), token
  // by token as the plain dispatch does it: each token row is read once and
  // written to its K slots (a copy by destination row would read every token
  // row K times).  Tasks of g.task_tokens tokens, one wave per token, fill the
  // workers that the tile tail leaves idle.
  const int n_copy = (g.T + g.task_tokens - 1) / g.task_tokens;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  for (;;) {
    const int task = claim_task(&w.cursor[0], &task_slot);
    if (task >= n_copy) break;
    const int t1 = min(g.T, (task + 1) * g.task_tokens);
    for (int t = task * g.task_tokens + wave; t < t1; t += C::NW)
      dispatch_row<uint16_t, 4, false>(static_cast<const uint16_t*>(g.x), slot,
                                       static_cast<uint16_t*>(g.o_x_perm), t, g.H, g.K, lane);
  }
}

// Row tile of all-rows index `row`: the group from the expert offsets (or the
// shared block), then the tile inside the group.
__device__ __forceinline__ int tile_of_row(int64_t row, const GemmArgs& g, const int32_t* first_tile,
                                          int bm) {
  if (row >= g.R) {
    const int64_t sh = (row - g.R) / g.T;
    return first_tile[g.E + sh] + (int)((row - g.R - sh * g.T) / bm);
  }
  int lo = 0, hi = g.E;  // largest e with offsets[e] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.offsets[mid] <= row) lo = mid; else hi = mid;
  }
  return first_tile[lo] + (int)((row - g.offsets[lo]) / bm);
}


template <bool R>
__global__ __launch_bounds__(DownCfg::NT) void ffn_combine_kernel(GemmArgs g,
                                                                   const int32_t* __restrict__ slot,
                                                                   const float* __restrict__ topk_w,
                                                                   FusedWs w, int nt_count) {
  using C = DownCfg;
  MOE_LDS_RING(C, ring);
  __shared__ int task_slot;
  const int n_mt = *w.n_mtiles;
  const int n_comb = (g.T + g.task_tokens - 1) / g.task_tokens;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  // phase 1: GEMM tiles; each completed tile counts towards its row tile
  for_tasks_xcd_ranges(w.cursor + 1, n_mt * nt_count, g.split_wr, (g.I + C::BK - 1) / C::BK,
                       &task_slot, [&](const TaskPart& tp) {
    int tm, tn;
    band_order_groups(tp.L, nt_count, w.bands, tm, tn);
    const TileDesc<uint16_t> d = decode_tile<uint16_t, kDown, C::BM, C::BN>(g, tm, tn);
    run_tile_bf16<C, true, R>(g, d, ring, tp);
    if (tp.part == tp.parts - 1)   // the tile is complete
      publish_add(&w.flags[tm], &w.cursor[kTilesDone]);
  }, g.perturb);
  // phase 2: combine tasks, each token once all its rows' tiles are done.
  // A worker that finds every tile published takes one acquire and then runs
  // all its remaining tasks without polls or further acquires (an agent-scope
  // acquire invalidates the XCD's whole L2, so one per task would cost the
  // tiles still running there their operands).
  __shared__ int all_done_s;
  bool all_done = false;   // uniform over the workgroup
  const int n_tiles = n_mt * nt_count;
  for (;;) {
    const int task = claim_task(&w.cursor[0], &task_slot);
    if (task >= n_comb) break;
    const int t0 = task * g.task_tokens;
    const int t1 = min(g.T, t0 + g.task_tokens);
    if (!all_done) {
      // wave 0: unless every tile is published, wait until the row tiles
      // holding the task's routed rows (q < K) and shared-expert rows (q >= K)
      // are complete; then one acquire
      if (wave == 0) {
        int done = 0;
        if (lane == 0)
          done = __hip_atomic_load(&w.cursor[kTilesDone], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) >= n_tiles + g.wait_extra;
        done = __builtin_amdgcn_readfirstlane(done);
        if (!done) {
          const int nq = g.K + g.Ns;
          for (int i = lane; i < (t1 - t0) * nq; i += kWave) {
            const int t = t0 + i / nq, q = i - (i / nq) * nq;
            const int64_t row = q < g.K ? (int64_t)slot[(int64_t)t * g.K + q]
                                        : g.R + (int64_t)(q - g.K) * g.T + t;
            const int tile = tile_of_row(row, g, w.first_tile, C::BM);
            poll_at_least(g, &w.flags[tile], nt_count);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (lane == 0) all_done_s = done;
      }
      __syncthreads();
      all_done = __builtin_amdgcn_readfirstlane(all_done_s) != 0;
    }
    for (int t = t0 + wave; t < t1; t += C::NW)
      combine_row<uint16_t, 4, 4, false>(static_cast<const uint16_t*>(g.o_y), slot, topk_w,
                            static_cast<uint16_t*>(g.o_out), t, g.T, g.H, g.K, g.Ns, lane);
  }
}

hipError_t launch_dispatch_ffn(const GemmArgs& a0, const Tuning& tu, const int32_t* slot_src,
                               const int32_t* slot, const FusedWs& w, hipStream_t st) {
  GemmArgs a = a0;
  a.mtiles = w.mtiles;
  a.n_mtiles = w.n_mtiles;
  a.bands = w.bands;
  a.a_rows = slot_src;
  a.task_tokens = tu.copy_tokens;
  hipError_t e = launch_plan(a.offsets, a.E, a.Ns, a.T, a.R, UpCfg::BM, tu.small_group, tu.band_up,
                             w.mtiles, w.n_mtiles, w.first_tile, w.bands, w.flags,
                             w.mt_bound + kFusedCursors + kXcds * kSplitWr, st);
  if (e != hipSuccess) return e;
  const int nt = gemm_ntiles<kUp>(a.H, a.I, UpCfg::BN);
  const bool rk = ragged_k(a.H, a.I, UpCfg::BK);
  if (tu.copy_in_tiles) {
    if (rk) dispatch_ffn_kernel<true, true><<<w.workers, UpCfg::NT, 0, st>>>(a, slot, w, nt);
    else dispatch_ffn_kernel<false, true><<<w.workers, UpCfg::NT, 0, st>>>(a, slot, w, nt);
  } else {
    if (rk) dispatch_ffn_kernel<true, false><<<w.workers, UpCfg::NT, 0, st>>>(a, slot, w, nt);
    else dispatch_ffn_kernel<false, false><<<w.workers, UpCfg::NT, 0, st>>>(a, slot, w, nt);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_combine(const GemmArgs& a0, const Tuning& tu, const int32_t* slot,
                              const float* topk_w, const FusedWs& w, hipStream_t st) {
  GemmArgs a = a0;
  a.mtiles = w.mtiles;
  a.n_mtiles = w.n_mtiles;
  a.bands = w.bands;
  a.task_tokens = tu.combine_tokens;
  // the down projection splits its tail tiles: fixed bands, as in the plain launch
  hipError_t e = launch_plan(a.offsets, a.E, a.Ns, a.T, a.R, DownCfg::BM, kSplitSmall,
                             split_kind_band(kDown), w.mtiles, w.n_mtiles, w.first_tile, w.bands,
                             w.flags, w.mt_bound + kFusedCursors + kXcds * kSplitWr, st);
  if (e != hipSuccess) return e;
  const int nt = gemm_ntiles<kDown>(a.H, a.I, DownCfg::BN);
  if (ragged_k(a.H, a.I, DownCfg::BK))
    ffn_combine_kernel<true><<<w.workers, DownCfg::NT, 0, st>>>(a, slot, topk_w, w, nt);
  else
    ffn_combine_kernel<false><<<w.workers, DownCfg::NT, 0, st>>>(a, slot, topk_w, w, nt);
  return hipGetLastError();
}

hipError_t take_wait_error_fused(uint32_t* out) { return take_wait_error(out); }

}  // namespace moe
