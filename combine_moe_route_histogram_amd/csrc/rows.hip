// Row kernels of the MoE layer: dispatch (permute into expert-contiguous
// rows), combine (gate-weighted sum back to token order), and the backward of
// both plus the gate softmax backward.  All are HBM-bound copies/reductions:
// one wave per token row, 16-byte vector loads and stores, fixed summation
// order (k = 0..K-1, then shared experts), float32 accumulation.
//
// UniEP article, section 1.1: tokens are reordered to their experts
// (dispatch) and the expert outputs are weighted by the gate scores and summed
// (combine); the backward mirrors the forward.
#include "common.hpp"
#include "kernels.hpp"
#include "rows.hpp"

namespace moe {

constexpr int kRowBlock = 256;               // 4 waves -> 4 tokens per block
constexpr int kRowsPerBlock = kRowBlock / kWave;

// x_perm[slot[t,k]] = x[t]: each x row is read once (non-temporal: nothing
// reads it again in this launch) and written K times.
template <typename S, int NC>
__global__ __launch_bounds__(kRowBlock) void dispatch_kernel(const S* __restrict__ x,
                                                             const int32_t* __restrict__ slot,
                                                             S* __restrict__ x_perm, int T, int H,
                                                             int K) {
  const int t = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  dispatch_row<S, 4, true, NC>(x, slot, x_perm, t, H, K, threadIdx.x & (kWave - 1));
}

// x_perm[s] = x[slot_src[s]]: the same rows as dispatch, indexed by destination.
template <typename S>
__global__ __launch_bounds__(kRowBlock) void gather_kernel(const S* __restrict__ x,
                                                           const int32_t* __restrict__ slot_src,
                                                           S* __restrict__ x_perm, int64_t R, int H) {
  const int64_t s = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (s >= R) return;
  const char* src = reinterpret_cast<const char*>(x + (int64_t)slot_src[s] * H);
  char* dst = reinterpret_cast<char*>(x_perm + s * H);
  const int nvec = H / Elem<S>::kPerVec;
  for (int v = lane; v < nvec; v += kWave) st16(dst + (int64_t)v * 16, ld16(src + (int64_t)v * 16));
}

template <typename S, int NC>
__global__ __launch_bounds__(kRowBlock) void combine_kernel(const S* __restrict__ y,
                                                            const int32_t* __restrict__ slot,
                                                            const float* __restrict__ w,
                                                            S* __restrict__ out, int T, int H,
                                                            int K, int Ns) {
  const int t = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  combine_row<S, 4, 4, true, NC>(y, slot, w, out, t, T, H, K, Ns, threadIdx.x & (kWave - 1));
}

// dy[slot[t,k]] = w[t,k] dout[t];  dw[t,k] = <dout[t], y[slot[t,k]]>.
// The dot product: per-lane partial sums in vector order, then a fixed
// butterfly across the wave.  The k rows go in batches of RB: per round a
// lane loads U vectors of dout and U of each of the batch's y rows together
// ((RB+1)*U loads in flight), non-temporal; the order of each partial sum is
// unchanged, so the bits do not depend on U or RB.
template <typename S, int NC>
__global__ __launch_bounds__(kRowBlock) void combine_bwd_kernel(const S* __restrict__ dout,
                                                                const S* __restrict__ y,
                                                                const int32_t* __restrict__ slot,
                                                                const float* __restrict__ w,
                                                                S* __restrict__ dy,
                                                                float* __restrict__ dw, int T,
                                                                int H, int K) {
  constexpr int P = Elem<S>::kPerVec;
  constexpr int U = 4, RB = 4;
  const int t = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (t >= T) return;
  PairVals<int, NC> my_slot;
  PairVals<float, NC> my_w;
  my_slot.load(slot + (int64_t)t * K, K, lane, 0);
  my_w.load(w + (int64_t)t * K, K, lane, 0.f);
  const int nvec = H / P;
  const char* g_row = reinterpret_cast<const char*>(dout + (int64_t)t * H);
  for (int k0 = 0; k0 < K; k0 += RB) {
    float part[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) part[rb] = 0.f;
    for (int v0 = lane; v0 < nvec; v0 += kWave * U) {
      u32x4 gr[U], yr[RB][U];
#pragma unroll
      for (int u = 0; u < U; ++u)   // a lane past the row's end reloads its last vector
        gr[u] = ld16_hint<true>(g_row + (int64_t)min(v0 + u * kWave, nvec - 1) * 16);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (k0 + rb < K) {
          const char* y_row = reinterpret_cast<const char*>(y + (int64_t)my_slot.at(k0 + rb) * H);
#pragma unroll
          for (int u = 0; u < U; ++u)
            yr[rb][u] = ld16_hint<true>(y_row + (int64_t)min(v0 + u * kWave, nvec - 1) * 16);
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (k0 + rb < K) {
          const float wk = my_w.at(k0 + rb);
          char* dy_row = reinterpret_cast<char*>(dy + (int64_t)my_slot.at(k0 + rb) * H);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int v = v0 + u * kWave;
            if (v < nvec) {
              float g[P], f[P], o[P];
              Elem<S>::unpack(gr[u], g);
              Elem<S>::unpack(yr[rb][u], f);
#pragma unroll
              for (int jj = 0; jj < P; ++jj) {
                part[rb] = fmaf(g[jj], f[jj], part[rb]);
                o[jj] = wk * g[jj];
              }
              st16_hint<true>(dy_row + (int64_t)v * 16, Elem<S>::pack(o));
            }
          }
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (k0 + rb < K) {
        const float p = wave_sum(part[rb]);
        if (lane == 0) dw[(int64_t)t * K + k0 + rb] = p;
      }
    }
  }
}

// dx[t] = sum_k dx_rows[slot[t,k]] + sum_s dx_rows[R + s*T + t]; one rounding
// (the combine row with unit weights).
template <typename S, int NC>
__global__ __launch_bounds__(kRowBlock) void dispatch_bwd_kernel(const S* __restrict__ dx_rows,
                                                                 const int32_t* __restrict__ slot,
                                                                 S* __restrict__ dx, int T, int H,
                                                                 int K, int Ns) {
  const int t = blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (t >= T) return;
  combine_row<S, 4, 4, true, NC>(dx_rows, slot, nullptr, dx, t, T, H, K, Ns, threadIdx.x & (kWave - 1));
}

// dl[t, e_k] = w_k (dw_k - sum_j w_j dw_j), zero for unselected experts.
// A block owns kRouteBwdFloats / E consecutive tokens, whose rows of dl are
// one contiguous run: it builds them in LDS (zeros, then one thread per token
// sums w_j dw_j over j = 0..K-1 in that order and places its K values), then
// writes the run with 16-byte stores.  Every value is written once, so the
// dense dl costs one pass at the write bandwidth.
constexpr int kRouteBwdFloats = 4096;   // 16 KiB of LDS per block

__global__ __launch_bounds__(256) void route_bwd_kernel(const float* __restrict__ dw,
                                                        const float* __restrict__ w,
                                                        const int32_t* __restrict__ idx,
                                                        float* __restrict__ dl, int T, int E,
                                                        int K, int tok_per_block) {
  __shared__ __align__(16) float rows[kRouteBwdFloats];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * tok_per_block;
  const int nt = (int)min<int64_t>(tok_per_block, T - t0);
  const int n = nt * E;   // floats of this block's run
  for (int i = tid; i < n; i += 256) rows[i] = 0.f;
  __syncthreads();
  for (int j = tid; j < nt; j += 256) {
    const int64_t t = t0 + j;
    float inner = 0.f;
    for (int k = 0; k < K; ++k) inner = fmaf(w[t * K + k], dw[t * K + k], inner);
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      if ((unsigned)e < (unsigned)E) rows[j * E + e] = w[t * K + k] * (dw[t * K + k] - inner);
    }
  }
  __syncthreads();
  float* dst = dl + t0 * E;
  // the run starts at a multiple of tok_per_block * E floats; 16-byte stores
  // where the run is 16-byte aligned (E % 4 == 0), else one float each
  if ((E & 3) == 0) {
    for (int i = tid; i < n / 4; i += 256)
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(rows + 4 * i),
                                  reinterpret_cast<f32x4*>(dst) + i);
  } else {
    for (int i = tid; i < n; i += 256) __builtin_nontemporal_store(rows[i], dst + i);
  }
}

static inline dim3 row_grid(int T) { return dim3((T + kRowsPerBlock - 1) / kRowsPerBlock); }

hipError_t launch_dispatch(bool is_bf16, const void* x, const int32_t* slot, void* x_perm, int T,
                           int H, int K, hipStream_t st) {
  const bool wide = pair_chunks(K) > 1;
#define MOE_LAUNCH(S, NC)                                                              \
  dispatch_kernel<S, NC><<<row_grid(T), kRowBlock, 0, st>>>(                           \
      static_cast<const S*>(x), slot, static_cast<S*>(x_perm), T, H, K)
  if (is_bf16) {
    if (wide) MOE_LAUNCH(uint16_t, 4); else MOE_LAUNCH(uint16_t, 1);
  } else {
    if (wide) MOE_LAUNCH(float, 4); else MOE_LAUNCH(float, 1);
  }
#undef MOE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gather(bool is_bf16, const void* x, const int32_t* slot_src, void* x_perm,
                         int64_t R, int H, hipStream_t st) {
  const dim3 grid((unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock));
  if (is_bf16)
    gather_kernel<uint16_t><<<grid, kRowBlock, 0, st>>>(static_cast<const uint16_t*>(x), slot_src,
                                                        static_cast<uint16_t*>(x_perm), R, H);
  else
    gather_kernel<float><<<grid, kRowBlock, 0, st>>>(static_cast<const float*>(x), slot_src,
                                                     static_cast<float*>(x_perm), R, H);
  return hipGetLastError();
}

hipError_t launch_combine(bool is_bf16, const void* y, const int32_t* slot, const float* w,
                          void* out, int T, int H, int K, int Ns, hipStream_t st) {
  const bool wide = pair_chunks(K) > 1;
#define MOE_LAUNCH(S, NC)                                                              \
  combine_kernel<S, NC><<<row_grid(T), kRowBlock, 0, st>>>(                            \
      static_cast<const S*>(y), slot, w, static_cast<S*>(out), T, H, K, Ns)
  if (is_bf16) {
    if (wide) MOE_LAUNCH(uint16_t, 4); else MOE_LAUNCH(uint16_t, 1);
  } else {
    if (wide) MOE_LAUNCH(float, 4); else MOE_LAUNCH(float, 1);
  }
#undef MOE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_combine_bwd(bool is_bf16, const void* dout, const void* y, const int32_t* slot,
                              const float* w, void* dy, float* dw, int T, int H, int K,
                              hipStream_t st) {
  const bool wide = pair_chunks(K) > 1;
#define MOE_LAUNCH(S, NC)                                                              \
  combine_bwd_kernel<S, NC><<<row_grid(T), kRowBlock, 0, st>>>(                        \
      static_cast<const S*>(dout), static_cast<const S*>(y), slot, w, static_cast<S*>(dy), dw, T, H, K)
  if (is_bf16) {
    if (wide) MOE_LAUNCH(uint16_t, 4); else MOE_LAUNCH(uint16_t, 1);
  } else {
    if (wide) MOE_LAUNCH(float, 4); else MOE_LAUNCH(float, 1);
  }
#undef MOE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_dispatch_bwd(bool is_bf16, const void* dx_rows, const int32_t* slot, void* dx,
                               int T, int H, int K, int Ns, hipStream_t st) {
  const bool wide = pair_chunks(K) > 1;
#define MOE_LAUNCH(S, NC)                                                              \
  dispatch_bwd_kernel<S, NC><<<row_grid(T), kRowBlock, 0, st>>>(                       \
      static_cast<const S*>(dx_rows), slot, static_cast<S*>(dx), T, H, K, Ns)
  if (is_bf16) {
    if (wide) MOE_LAUNCH(uint16_t, 4); else MOE_LAUNCH(uint16_t, 1);
  } else {
    if (wide) MOE_LAUNCH(float, 4); else MOE_LAUNCH(float, 1);
  }
#undef MOE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_route_bwd(const float* dw, const float* w, const int32_t* idx, float* dl, int T,
                            int E, int K, hipStream_t st) {
  const int tpb = kRouteBwdFloats / E;   // E <= 256: at least 16 tokens per block
  route_bwd_kernel<<<(T + tpb - 1) / tpb, 256, 0, st>>>(dw, w, idx, dl, T, E, K, tpb);
  return hipGetLastError();
}

}  // namespace moe
