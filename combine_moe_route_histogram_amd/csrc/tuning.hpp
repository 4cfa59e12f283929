// Schedule knobs of the grouped GEMMs and fused kernels chosen per shape
// (auto-tuning), host side.
#pragma once

#include "../../include/moe.h"

namespace moe {

constexpr int kMaxBand = 64;          // largest band height a knob may take
constexpr int kMaxTaskTokens = 1024;  // largest combine / copy task

// The knobs the library uses for a layer shape, from the analytical traffic
// model in tuning.hip (no MOE_TUNE override applied).
moe_tuning choose_tuning(int T, int H, int E, int K, int I, int Ns);

// Predicted operand bytes fetched from beyond L2 per flop for one GEMM kind
// run in bands of `band` row tiles (M tiles for the weight gradient) over
// groups of `rows` rows, `n_tiles` column tiles of `bn` columns and a k depth
// of `k_len` (the model behind choose_tuning; exposed for the tests).
double band_traffic_per_flop(double rows, int bm, int bn, int n_tiles, double k_len, int band,
                             int small_group);

// Predicted bytes beyond L2 per flop of the gate/up projection (act = false)
// or the activation gradient (act = true) with the given band knobs.
double predict_traffic(int T, int H, int E, int K, int I, int Ns, bool act, int band, int small);

}  // namespace moe
