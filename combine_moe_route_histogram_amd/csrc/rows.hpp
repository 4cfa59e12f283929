// Row-level device functions shared by the plain row kernels and the fused
// persistent kernels (so both produce identical bits).
#pragma once

#include "common.hpp"

namespace moe {

// out[t] = sum_k w[t,k] y[slot[t,k]] + sum_s y[R + s*T + t]; one rounding.
template <typename S>
__device__ __forceinline__ void combine_row(const S* __restrict__ y, const int32_t* __restrict__ slot,
                                            const float* __restrict__ w, S* __restrict__ out,
                                            int t, int T, int H, int K, int Ns, int lane) {
  constexpr int P = Elem<S>::kPerVec;
  const int my_slot = lane < K ? slot[(int64_t)t * K + lane] : 0;
  const float my_w = lane < K ? w[(int64_t)t * K + lane] : 0.f;
  const int64_t R = (int64_t)T * K;
  const int nvec = H / P;
  for (int v = lane; v < nvec; v += kWave) {
    float acc[P];
#pragma unroll
    for (int j = 0; j < P; ++j) acc[j] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int s = __shfl(my_slot, k, kWave);
      const float wk = __shfl(my_w, k, kWave);
      float f[P];
      Elem<S>::unpack(ld16(reinterpret_cast<const char*>(y + (int64_t)s * H) + (int64_t)v * 16), f);
#pragma unroll
      for (int j = 0; j < P; ++j) acc[j] = fmaf(wk, f[j], acc[j]);
    }
    for (int sh = 0; sh < Ns; ++sh) {
      float f[P];
      Elem<S>::unpack(ld16(reinterpret_cast<const char*>(y + (R + (int64_t)sh * T + t) * H) +
                           (int64_t)v * 16), f);
#pragma unroll
      for (int j = 0; j < P; ++j) acc[j] += f[j];
    }
    st16(reinterpret_cast<char*>(out + (int64_t)t * H) + (int64_t)v * 16, Elem<S>::pack(acc));
  }
}

}  // namespace moe
