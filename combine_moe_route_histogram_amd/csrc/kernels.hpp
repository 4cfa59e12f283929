// Host-side launchers of the HIP kernels (internal; the public ABI is moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Tokens per routing chunk: one histogram row and one slot-ranking wave each
// (short chunks: the ranking is a chain of dependent ballots per 64 pairs,
// so more, shorter chains keep more of the GPU busy).
constexpr int kChunkTokens = 64;

// Largest number of routed experts (the routing kernels keep one LDS word per
// expert; the planner stages E + 1 offsets in LDS).
constexpr int kMaxExperts = 256;
constexpr int kMaxShared = 8;      // shared experts per layer at most

inline int route_nchunk(int T) { return (T + kChunkTokens - 1) / kChunkTokens; }

hipError_t launch_route(const float* logits, int T, int E, int K, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* slot_src,
                        int32_t* chunk_counts, int32_t* chunk_base, hipStream_t st);

// Fixed device scratch of the routing variant that allocates nothing (for
// callers that cannot allocate): one array per device, 1 MiB, holding the
// per-chunk expert counts and bases (route_nchunk(T) * E ints each).
constexpr int64_t kRouteScratchInts = 1 << 18;
inline bool route_scratch_fits(int T, int E) {
  return 2 * (int64_t)route_nchunk(T) * E <= kRouteScratchInts;
}
// Device address of the scratch array on `device`, looked up once per device
// (the device is made current for the lookup) and cached.
hipError_t route_scratch_prepare(int device);
// The cached address for the current device (looked up on first use).
hipError_t route_scratch_current(int32_t** out);

// Row kernels; is_bf16 selects the storage type (bf16 or f32).
hipError_t launch_dispatch(bool is_bf16, const void* x, const int32_t* slot, void* x_perm, int T,
                           int H, int K, hipStream_t st);
hipError_t launch_gather(bool is_bf16, const void* x, const int32_t* slot_src, void* x_perm,
                         int64_t R, int H, hipStream_t st);
hipError_t launch_combine(bool is_bf16, const void* y, const int32_t* slot, const float* w,
                          void* out, int T, int H, int K, int Ns, hipStream_t st);
hipError_t launch_combine_bwd(bool is_bf16, const void* dout, const void* y, const int32_t* slot,
                              const float* w, void* dy, float* dw, int T, int H, int K,
                              hipStream_t st);
hipError_t launch_dispatch_bwd(bool is_bf16, const void* dx_rows, const int32_t* slot, void* dx,
                               int T, int H, int K, int Ns, hipStream_t st);
// Algorithm 1 with G explicit ranks (route.hip); chunk scratch sized by
// route_ranks_nchunk(T, G) chunks.
int route_ranks_nchunk(int T, int G);
hipError_t launch_route_ranks(const int32_t* topk_idx, int T, int E, int K, int G,
                              int32_t* rank_counts, int32_t* rank_base, int32_t* counts,
                              int32_t* offsets, int32_t* slot, int32_t* slot_src, int32_t* chunk_counts,
                              int32_t* chunk_base, int32_t* chunk_t0, int32_t* rank_chunk,
                              hipStream_t st);
hipError_t launch_route_bwd(const float* dw, const float* w, const int32_t* idx, float* dl, int T,
                            int E, int K, hipStream_t st);

// Grouped GEMM kinds of the expert FFN.
enum GemmKind : int {
  kUp = 0,       // a|b = X [W1|W3], h = silu(a) b      (forward, first GEMM)
  kDown = 1,     // y = h W2                            (forward, second GEMM)
  kBwdUp = 2,    // dh = dY W2^T, SwiGLU backward -> da|db
  kBwdDown = 3,  // dx = [da db] [W1 W3]^T
  kWgUp = 4,     // dW1 = X^T da, dW3 = X^T db          (transposed, over rows)
  kWgDown = 5,   // dW2 = h^T dY
};

// Schedule knobs (the auto-tuning space): each changes which tiles run
// together on an XCD or how the fused kernels cut their row tasks, never the
// arithmetic of an output element, so every choice gives the same bits.  The
// GEMM kinds whose tail tiles are split along k (down projection, input
// gradient) keep fixed bands: their split tiles are the last ones of each
// XCD range in tile order, so a different order would split other tiles.
struct Tuning {
  int band_up;         // row tiles per band of a large group: gate/up projection
  int band_act;        // the same for the activation gradient
  int small_group;     // groups of at most this many row tiles are one band (those two kinds)
  int band_wg_up;      // H blocks per band: dW1/dW3
  int band_wg_down;    // I blocks per band: dW2
  int combine_tokens;  // tokens per combine task of the fused down+combine
  int copy_tokens;     // tokens per x_perm copy task of the fused dispatch+up
  int copy_in_tiles;   // 1: the fused dispatch+up writes x_perm from its GEMM tiles instead
};

// Fixed bands of the split kinds: groups of at most kSplitSmall row tiles are
// one band, larger ones run in bands of split_kind_band(kind).
constexpr int kSplitSmall = 8;
__host__ __device__ constexpr int split_kind_band(int kind) { return kind == kDown ? 8 : 4; }

struct GemmArgs {
  int T, H, E, K, I, Ns, R;
  const int32_t* offsets;  // [E+1] routed row ranges
  const int4* mtiles;      // per M-tile {group, first row (all-rows index), rows, 0}
  const int32_t* n_mtiles; // [0] valid entries in mtiles, [1] bands in `bands`, [2] in `bands2`
  const int2* bands;       // per M-tile: {first M-tile, M-tiles} of the band holding it
  const int2* bands2;      // second band table over the same M-tiles (the one-launch backward's
                           // input-gradient phase), or null
  int mt_max;              // host bound on the number of M-tiles
  int wg_band;             // weight-gradient kinds: M tiles per band
  int task_tokens;         // fused kernels: tokens per combine or copy task
  const void* x_perm;
  const void* x;
  const void* w1;
  const void* w3;
  const void* w2;
  const void* ws1;
  const void* ws3;
  const void* ws2;
  const void* ab;
  const void* h;
  const void* dy;
  const void* dout;
  const void* dab;
  const int32_t* a_rows;  // kUp: token of each routed row, A read from x through it (fused
                          // dispatch); nullptr: A read from x_perm
  void* o_x_perm;  // fused dispatch: gather target (same buffer as x_perm)
  void* o_out;     // fused combine: token outputs
  void* o_ab;
  void* o_h;
  void* o_y;
  void* o_dab;
  void* o_dx;
  float* o_dw1;
  float* o_dw3;
  float* o_dw2;
  float* o_dws1;
  float* o_dws3;
  float* o_dws2;
  // k split of each XCD range's tail tiles (bf16 forward-shaped kinds)
  float* split_part;       // [kXcds * kSplitSlots] partial tiles of BM x BN f32
  int32_t* split_cnt;      // [kXcds * kSplitWr] finished helper parts per split tile
  int split_wr;            // nominal workers per XCD (0: no split)
  // bounded in-kernel waits: give up after wait_ticks of the 100 MHz clock;
  // wait_extra (debug, 0 or 1) is added to every wait's target
  uint64_t wait_ticks;
  int wait_extra;
  // debug (determinism tests): nonzero = persistent workers claim each
  // range's whole tiles in a seeded order and sleep a seeded time before
  // every claim; results must not change
  uint32_t perturb;
};

// Bounded-wait records, one error word per code object (.hip file): take
// (read and clear) the word of each.
hipError_t take_wait_error_gemm(uint32_t* out);
hipError_t take_wait_error_fused(uint32_t* out);
hipError_t take_wait_error_bwd(uint32_t* out);

// Tail split constants: kSplitWr nominal workers per XCD (256 CUs / 8 XCDs
// on MI355X; a plan constant, so results do not depend on how many workers
// actually run), at most kMaxSplit parts per tile, kSplitSlots partial tiles
// per range = max over rem in [1, kSplitWr) of rem * (parts(rem) - 1).
constexpr int kSplitWr = 32;
constexpr int kMaxSplit = 4;
constexpr int split_parts(int rem, int wr, int max_parts) {
  return rem <= 0 ? 1 : (wr / rem < max_parts ? wr / rem : max_parts);
}
constexpr int split_slots_max() {
  int m = 0;
  for (int rem = 1; rem < kSplitWr; ++rem) {
    const int p = split_parts(rem, kSplitWr, kMaxSplit);
    if (p >= 2 && rem * (p - 1) > m) m = rem * (p - 1);
  }
  return m;
}
constexpr int kSplitSlots = split_slots_max();

// Upper bound on the number of row tiles of height bm over all groups.
inline int64_t mtile_bound(int64_t T, int64_t K, int64_t E, int64_t Ns, int bm) {
  return (T * K + bm - 1) / bm + E + Ns * ((T + bm - 1) / bm);
}

// Smallest row-tile height used by any GEMM configuration (the f32 tiles are
// 64 rows); sizes the row-tile tables in the workspace.
constexpr int kMinTileM = 64;

// bf16: `workers` persistent workgroups take the tiles through the kXcds
// cursors at `cursors` (cleared by the launch itself); f32: one workgroup per
// tile.
hipError_t launch_gemm(bool is_bf16, int kind, const GemmArgs& a, const Tuning& tu,
                       int4* mtiles_ws, int32_t* n_mtiles_ws, int2* bands_ws, int32_t* cursors,
                       int workers, hipStream_t st);

// Row-tile planner (one block): table of bm-row tiles per group, the first
// table index of every group (if first_tile), the band table (a group of at
// most `small` row tiles is one band, a larger one runs of `big`; per row
// tile, the first row tile and the height of its band) and, if bands2, a
// second one with (small2, big2), and n_clear ints of `clear` set to zero
// (flags and cursors of the fused kernels).
hipError_t launch_plan(const int32_t* offsets, int E, int Ns, int T, int R, int bm, int small,
                       int big, int4* mtiles, int32_t* n_mtiles, int32_t* first_tile,
                       int2* bands, int32_t* clear, int n_clear, hipStream_t st,
                       int2* bands2 = nullptr, int small2 = 0, int big2 = 0);

// Fused persistent kernels (bf16).  ws_* are workspace sections.
// Task cursors of a fused launch: [0] the x_perm copy (dispatch_ffn) or combine
// (ffn_combine) tasks, or the finished first-phase tiles (ffn_bwd); then
// kXcds tile cursors per GEMM phase (one phase in the forward kernels, four
// in ffn_bwd); last, [kTilesDone]: GEMM tiles published so far (ffn_combine).
constexpr int kXcds = 8;
constexpr int kMaxPhases = 4;
constexpr int kFusedCursors = 2 + kMaxPhases * kXcds;
constexpr int kTilesDone = kFusedCursors - 1;
struct FusedWs {
  int4* mtiles;
  int32_t* n_mtiles;
  int32_t* first_tile;  // [E + Ns]
  int2* bands;          // [mt bound]
  int2* bands2;         // [mt bound]
  int32_t* flags;       // [mt bound]: done counters of the row tiles (ffn_combine)
  int32_t* cursor;      // [kFusedCursors], right after the flags
  int mt_bound;
  int workers;          // persistent workgroups to launch
};
hipError_t launch_dispatch_ffn(const GemmArgs& a, const Tuning& tu, const int32_t* slot_src,
                               const int32_t* slot, const FusedWs& w, hipStream_t st);
hipError_t launch_ffn_combine(const GemmArgs& a, const Tuning& tu, const int32_t* slot,
                              const float* topk_w, const FusedWs& w, hipStream_t st);
// Expert-FFN backward in one persistent launch (bwd.hip): activation-gradient
// tiles, then dW2 tiles, then input-gradient tiles, then dW1/dW3 tiles.
hipError_t launch_ffn_bwd(const GemmArgs& a, const Tuning& tu, const FusedWs& w, hipStream_t st);

}  // namespace moe
