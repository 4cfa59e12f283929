// Auto-tuning of the schedule knobs (host side).
//
// The UniEP article names an auto-tuning stage -- an optimisation space, an
// analytical performance model and priority token scheduling (its section 3,
// of which only the table of contents survives).  Here the space is the set
// of knobs that change the schedule but never the arithmetic of an output
// element (Tuning in kernels.hpp: band heights, the small-group threshold,
// fused task sizes), so every choice gives the same bits and the choice can
// follow the shape freely.
//
// Model for the band heights of the forward-shaped kinds that are not split
// along k (gate/up projection, activation gradient).  One XCD runs W = 32
// persistent workers that take consecutive tiles of the band order, so the
// tiles in flight together are h row tiles x W/h column tiles of one band.
// Each k slice of those tiles is fetched into the XCD's L2 once and shared.
// Across the band's column windows, the band's token rows (h * BM rows * k)
// are fetched once if they stay in L2 (h * BM * k * 2 bytes <= kL2Share of
// the 4 MiB, the rest being taken by the streaming weights), else once per
// window (ceil(n_tiles * h / W) windows); the weight columns are fetched once
// per band.  Operand bytes fetched beyond L2 per flop of a band:
//     rows:    passes / (n_tiles * BN)        weights:  1 / (h * BM)
// A fetch beyond L2 is served by the 256 MiB Infinity Cache when the operand's
// footprint fits in half of it (the token rows: the routed tokens' rows; the
// weights: the experts the 8 XCDs work on at once), else by HBM; an Infinity
// Cache fetch costs kMallCost of an HBM fetch.  The flop-weighted cost over
// the groups decides: the band height with the lowest cost, and the
// small-group threshold below the first group size for which cutting a group
// into bands costs less (grown up to 16 row tiles while one band costs less).
// A change from the measured defaults (bands of 4, groups of up to 8 row tiles
// as one band) needs a predicted gain of kMargin.  Measured on MI355X over the
// five layer sizes: the model picks the fastest band height of the gate/up
// projection and of the activation gradient within 1 % except for the gate/up
// projection at the DeepSeek-like size (2 % behind 4).
//
// The weight-gradient band heights and the fused task sizes are measured
// choices: the traffic model mispredicts the weight gradient of small groups,
// whose tiles are dominated by their float32 output stores, and combine tasks
// of 8 tokens were never slower than 16 (2.6 % faster at the DeepSeek-like
// size, 4 per worker or more everywhere), while copy tasks of 16-128 tokens
// were all within noise.
#include <cmath>

#include "gemm_tile.hpp"
#include "tuning.hpp"

namespace moe {

namespace {

constexpr int kWorkersPerXcd = 32;           // 256 CUs / 8 XCDs
constexpr int kXcdsModel = 8;
constexpr double kL2Share = 3.0 * 1024 * 1024;  // of a 4 MiB L2, for one band's token rows
constexpr double kMallBytes = 256.0 * 1024 * 1024;
constexpr double kMallCost = 0.3;               // cost of an Infinity Cache fetch vs HBM
const int kBandChoices[] = {2, 4, 8, 16};

struct OperandCost {
  double rows, weights;   // cost of a byte of token rows / weights fetched beyond L2
};

// Bytes beyond L2 per flop for one band of h row tiles, weighted by where
// each operand is served from (see the file comment).
double band_cost(int h, int bm, int bn, int n_tiles, double k_len, const OperandCost& oc) {
  const double a_band = (double)h * bm * k_len * 2.0;
  const double windows = std::ceil((double)n_tiles * h / kWorkersPerXcd);
  const double passes = a_band <= kL2Share ? 1.0 : windows;
  return oc.rows * passes / ((double)n_tiles * bn) + oc.weights / ((double)h * bm);
}

double band_traffic(double rows, int bm, int bn, int n_tiles, double k_len, int band, int small_group,
                    const OperandCost& oc) {
  const int mt = (int)std::ceil(rows / bm);
  if (mt <= 0) return 0.0;
  if (mt <= small_group) return band_cost(mt, bm, bn, n_tiles, k_len, oc);
  // bands of `band`, the last one shorter; flop-weighted
  double cost = 0.0;
  for (int c = 0; c < mt; c += band) {
    const int h = mt - c < band ? mt - c : band;
    cost += band_cost(h, bm, bn, n_tiles, k_len, oc) * h;
  }
  return cost / mt;
}

}  // namespace

double band_traffic_per_flop(double rows, int bm, int bn, int n_tiles, double k_len, int band,
                             int small_group) {
  return band_traffic(rows, bm, bn, n_tiles, k_len, band, small_group, OperandCost{1.0, 1.0});
}

namespace {

// Flop-weighted cost of one kind over the routed groups (about R/E rows each)
// and the shared groups (T rows each).
double kind_traffic(int T, int E, int K, int Ns, int bn, int n_tiles, double k_len, int band,
                    int small, const OperandCost& oc) {
  const double routed = (double)T * K / E;
  const double w_routed = (double)T * K, w_shared = (double)T * Ns;
  double c = w_routed * band_traffic(routed, 256, bn, n_tiles, k_len, band, small, oc);
  if (Ns) c += w_shared * band_traffic(T, 256, bn, n_tiles, k_len, band, small, oc);
  return c / (w_routed + w_shared);
}

double served_cost(double footprint) { return footprint <= kMallBytes / 2 ? kMallCost : 1.0; }

// Where the operands of the two modelled kinds come from.  Gate/up: the token
// rows x (the fused launch gathers them from x), the experts' W1|W3.
// Activation gradient: the routed rows' output gradients dy and W2.
OperandCost operand_cost(int T, int H, int E, int K, int I, bool act) {
  const double active = (double)(E < kXcdsModel ? E : kXcdsModel);
  if (!act) return {served_cost((double)T * H * 2), served_cost(active * H * 2.0 * I * 2)};
  return {served_cost((double)T * K * H * 2), served_cost(active * (double)I * H * 2)};
}

// The model's choices move off the measured defaults (bands of 4, groups of
// up to 8 row tiles as one band) only where it predicts at least kMargin less
// traffic: its estimates are coarse, ties are common, and a change that it
// cannot tell apart from the default is not worth a different schedule.
constexpr double kMargin = 0.02;

void choose_bands(int T, int E, int K, int Ns, int bn, int n_tiles, double k_len,
                  const OperandCost& oc, int& band, int& small) {
  band = 4;
  double best = kind_traffic(T, E, K, Ns, bn, n_tiles, k_len, 4, 8, oc);
  for (int h : kBandChoices) {
    const double c = kind_traffic(T, E, K, Ns, bn, n_tiles, k_len, h, 8, oc);
    if (c < best * (1.0 - kMargin)) {
      best = c;
      band = h;
    }
  }
  auto one = [&](int m) { return band_traffic((double)m * 256, 256, bn, n_tiles, k_len, band, m, oc); };
  auto cut = [&](int m) { return band_traffic((double)m * 256, 256, bn, n_tiles, k_len, band, 0, oc); };
  small = 8;
  for (int m = band + 1; m <= 8; ++m) {
    if (one(m) > cut(m) * (1.0 + kMargin)) {
      small = m - 1;
      return;
    }
  }
  for (int m = 9; m <= 16 && one(m) < cut(m) * (1.0 - kMargin); ++m) small = m;
}

}  // namespace

double predict_traffic(int T, int H, int E, int K, int I, int Ns, bool act, int band, int small) {
  const int n_tiles = act ? (I + 255) / 256 : (I + 127) / 128;
  return kind_traffic(T, E, K, Ns, 256, n_tiles, H, band, small, operand_cost(T, H, E, K, I, act));
}

moe_tuning choose_tuning(int T, int H, int E, int K, int I, int Ns) {
  moe_tuning t;
  int small_up = 8, small_act = 8;
  // gate/up projection: N = I (paired: 128 of W1 and 128 of W3 per tile), k = H
  choose_bands(T, E, K, Ns, 256, (I + 127) / 128, H, operand_cost(T, H, E, K, I, false), t.band_up,
               small_up);
  // activation gradient: N = I, k = H
  choose_bands(T, E, K, Ns, 256, (I + 255) / 256, H, operand_cost(T, H, E, K, I, true), t.band_act,
               small_act);
  // one threshold serves both kinds (the one-launch backward and the fused
  // forward share it): the smaller of the two
  t.small_group = small_up < small_act ? small_up : small_act;
  // measured (see the file comment)
  t.band_wgrad_up = 4;
  t.band_wgrad_down = 8;
  t.combine_tokens = 8;
  t.copy_tokens = 32;
  // x_perm of the fused dispatch+up: copy tasks re-read the token rows x,
  // cheap while x fits in half of the Infinity Cache; beyond that, writing it
  // from the rows the tiles already gathered into LDS saves the HBM re-read
  t.copy_in_tiles = (double)T * H * 2 > kMallBytes / 2 ? 1 : 0;
  return t;
}

}  // namespace moe
