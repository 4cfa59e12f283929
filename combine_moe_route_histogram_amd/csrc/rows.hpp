// Row-level device functions shared by the plain row kernels and the fused
// persistent kernels (so both produce identical bits).
#pragma once

#include "common.hpp"

namespace moe {

// out[t] = sum_k w[t,k] y[slot[t,k]] + sum_s y[R + s*T + t]; one rounding.
// Each lane takes U 16-byte column vectors per round (U loads of one row in
// flight at a time); every element still sums k in ascending order, then the
// shared rows, so the bits do not depend on U.  w == nullptr: unit weights
// (plain sums: the dispatch backward).
template <typename S>
__device__ __forceinline__ void combine_row(const S* __restrict__ y, const int32_t* __restrict__ slot,
                                            const float* __restrict__ w, S* __restrict__ out,
                                            int t, int T, int H, int K, int Ns, int lane) {
  constexpr int P = Elem<S>::kPerVec;
  constexpr int U = 8;
  const bool weighted = w != nullptr;
  const int my_slot = lane < K ? slot[(int64_t)t * K + lane] : 0;
  const float my_w = (weighted && lane < K) ? w[(int64_t)t * K + lane] : 0.f;
  const int64_t R = (int64_t)T * K;
  const int nvec = H / P;
  for (int v0 = lane; v0 < nvec; v0 += kWave * U) {
    float acc[U][P];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < P; ++j) acc[u][j] = 0.f;
    for (int k = 0; k < K + Ns; ++k) {
      const S* row;
      float wk = 1.f;
      if (k < K) {
        row = y + (int64_t)lane_int(my_slot, k) * H;
        wk = lane_float(my_w, k);
      } else {
        row = y + (R + (int64_t)(k - K) * T + t) * H;
      }
      u32x4 r[U];
#pragma unroll
      for (int u = 0; u < U; ++u)   // a lane past the row's end reloads its last vector
        r[u] = ld16(reinterpret_cast<const char*>(row) + (int64_t)min(v0 + u * kWave, nvec - 1) * 16);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float f[P];
        Elem<S>::unpack(r[u], f);
        if (k < K && weighted) {
#pragma unroll
          for (int j = 0; j < P; ++j) acc[u][j] = fmaf(wk, f[j], acc[u][j]);
        } else {
#pragma unroll
          for (int j = 0; j < P; ++j) acc[u][j] += f[j];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * kWave;
      if (v < nvec) st16(reinterpret_cast<char*>(out + (int64_t)t * H) + (int64_t)v * 16, Elem<S>::pack(acc[u]));
    }
  }
}

}  // namespace moe
