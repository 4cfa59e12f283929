// Row-level device functions shared by the plain row kernels and the fused
// persistent kernels (so both produce identical bits).
#pragma once

#include "common.hpp"

namespace moe {

// 16-byte vector load / store; NT marks data that is touched once (streamed
// rows): non-temporal, so it does not displace lines that are still wanted
// and dirty lines it would evict do not have to be written back first.
template <bool NT>
__device__ __forceinline__ u32x4 ld16_hint(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  else return ld16(p);
}
template <bool NT>
__device__ __forceinline__ void st16_hint(void* p, const u32x4& v) {
  if constexpr (NT) __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
  else st16(p, v);
}

// out[t] = sum_k w[t,k] y[slot[t,k]] + sum_s y[R + s*T + t]; one rounding.
// Each lane takes U 16-byte column vectors of a row per round, and the loads
// of RB rows are issued together (U*RB loads in flight per lane); every
// element still sums k in ascending order, then the shared rows, so the bits
// depend on neither U nor RB.  w == nullptr: unit weights (plain sums: the
// dispatch backward).  NT: non-temporal loads and stores (plain launches,
// whose rows stream through once); the fused kernel reads rows written by
// other workgroups of the same launch and keeps ordinary loads.
// NC: chunks of 64 pairs per token (K <= 64 NC).
template <typename S, int U, int RB, bool NT, int NC = 1>
__device__ __forceinline__ void combine_row(const S* __restrict__ y, const int32_t* __restrict__ slot,
                                            const float* __restrict__ w, S* __restrict__ out,
                                            int t, int T, int H, int K, int Ns, int lane) {
  constexpr int P = Elem<S>::kPerVec;
  const bool weighted = w != nullptr;
  PairVals<int, NC> my_slot;
  PairVals<float, NC> my_w;
  my_slot.load(slot + (int64_t)t * K, K, lane, 0);
  if (weighted) my_w.load(w + (int64_t)t * K, K, lane, 0.f);
  const int64_t R = (int64_t)T * K;
  const int nvec = H / P;
  const int nrows = K + Ns;
  for (int v0 = lane; v0 < nvec; v0 += kWave * U) {
    float acc[U][P];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < P; ++j) acc[u][j] = 0.f;
    for (int k0 = 0; k0 < nrows; k0 += RB) {
      u32x4 r[RB][U];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int k = k0 + rb;
        if (k < nrows) {
          const int64_t row = k < K ? (int64_t)my_slot.at(k) : R + (int64_t)(k - K) * T + t;
          const char* base = reinterpret_cast<const char*>(y + row * H);
#pragma unroll
          for (int u = 0; u < U; ++u)   // a lane past the row's end reloads its last vector
            r[rb][u] = ld16_hint<NT>(base + (int64_t)min(v0 + u * kWave, nvec - 1) * 16);
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int k = k0 + rb;
        if (k < nrows) {
          const float wk = (weighted && k < K) ? my_w.at(k) : 0.f;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float f[P];
            Elem<S>::unpack(r[rb][u], f);
            if (k < K && weighted) {
#pragma unroll
              for (int j = 0; j < P; ++j) acc[u][j] = fmaf(wk, f[j], acc[u][j]);
            } else {
#pragma unroll
              for (int j = 0; j < P; ++j) acc[u][j] += f[j];
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * kWave;
      if (v < nvec)
        st16_hint<NT>(reinterpret_cast<char*>(out + (int64_t)t * H) + (int64_t)v * 16, Elem<S>::pack(acc[u]));
    }
  }
}

// x_perm[slot[t,k]] = x[t] for k = 0..K-1: the token row is read once (U
// 16-byte vectors per lane per round) and written to its K slots.  NT:
// non-temporal loads (the plain launch, where nothing reads the row again).
template <typename S, int U, bool NT, int NC = 1>
__device__ __forceinline__ void dispatch_row(const S* __restrict__ x, const int32_t* __restrict__ slot,
                                             S* __restrict__ x_perm, int t, int H, int K, int lane) {
  PairVals<int, NC> my_slot;
  my_slot.load(slot + (int64_t)t * K, K, lane, 0);
  const int nvec = H / Elem<S>::kPerVec;
  const char* src = reinterpret_cast<const char*>(x + (int64_t)t * H);
  for (int v0 = lane; v0 < nvec; v0 += U * kWave) {
    u32x4 val[U];
#pragma unroll
    for (int u = 0; u < U; ++u)   // a lane past the row's end reloads its last vector
      val[u] = ld16_hint<NT>(src + (int64_t)min(v0 + u * kWave, nvec - 1) * 16);
    for (int k = 0; k < K; ++k) {
      char* dst = reinterpret_cast<char*>(x_perm + (int64_t)my_slot.at(k) * H);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * kWave;
        if (v < nvec) st16(dst + (int64_t)v * 16, val[u]);
      }
    }
  }
}

}  // namespace moe
