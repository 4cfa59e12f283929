// One output tile of the grouped expert-FFN GEMMs, shared by the plain
// launches and by the fused persistent kernels so that both produce the same
// bits.
//
// The expert FFN is the SwiGLU MLP of the GraphPP article (sections 5.1/5.2:
// gate projection w1, up projection w3, SiLU, gate product, down projection
// w2; grad_w2 = h^T grad_out, grad_w1/3 from x^T and the intermediate
// gradients, grad_x the sum of two paths), run per expert over the
// expert-contiguous, padding-free rows of the UniEP article (section 1.2:
// ragged per-expert row ranges handled by pointer arithmetic, no padding).
//
// Six GEMM kinds (see GemmKind).  Every kind computes C[m][n] = sum_k A[m][k]
// B[k][n] for one BM x BN tile with float32 accumulation; the K loop always
// runs in ascending k, so a tile's result does not depend on which worker
// computes it or when.
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16.  Both operands are staged in LDS
// K-contiguous ([row][k], 64 k per row, 16-byte chunks XOR-swizzled by row
// so that the 16-byte MFMA operand reads of 16 consecutive rows hit distinct
// banks).  Operands that are K-contiguous in memory are copied with 16-byte
// loads; operands that are MN-contiguous (weights in the forward, every
// operand of the weight gradient) are read as 8(k) x 4(mn) blocks of 8-byte
// loads and transposed in registers with v_perm before the LDS store.
// Double-buffered LDS: the global loads of tile k+1 are in flight while the
// MFMAs of tile k run.
//
// f32 path: plain LDS-tiled FMA kernel (the MI355X fp32 vector and fp32
// matrix peaks are equal, so VALU FMA loses nothing for fp32).
#pragma once

#include <climits>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kBK = 64;  // k per LDS stage (bf16)

template <typename S>
struct TileDesc {
  const S* a;          // A(m,k) = a[m*a_sm + k*a_sk]
  int64_t a_sm, a_sk;
  const S* b0;         // B(k,n) = b[k*b_sk + n*b_sn]; paired kinds: n < BN/2 from b0,
  const S* b1;         //   else b1 at n - BN/2; split-K kinds: k >= ksplit from b1 at k - ksplit
  int64_t b_sn, b_sk;
  int ksplit;
  int m_valid, n_valid, k_len;  // n_valid counts per half for paired kinds
  int64_t row0;        // forward kinds: first output row (all-rows index); wgrad: first dW row
  int col0;            // first output column (per half for paired kinds)
  int group;           // expert (>= E: shared expert group - E)
  bool skip;
};

template <int KIND>
struct KindTraits {
  static constexpr bool kPaired = (KIND == kUp || KIND == kWgUp);
  static constexpr bool kWgrad = (KIND == kWgUp || KIND == kWgDown);
  static constexpr bool kAMn = kWgrad;                        // A is MN-contiguous
  static constexpr bool kBMn = (KIND == kUp || KIND == kDown || kWgrad);  // B is N-contiguous
};

// Number of N-tiles (per M-tile) and of M-tiles per group for wgrad kinds.
template <int KIND>
__host__ __device__ inline int gemm_ntiles(int H, int I, int BN) {
  switch (KIND) {
    case kUp: return (I + BN / 2 - 1) / (BN / 2);
    case kDown: return (H + BN - 1) / BN;
    case kBwdUp: return (I + BN - 1) / BN;
    case kBwdDown: return (H + BN - 1) / BN;
    case kWgUp: return (I + BN / 2 - 1) / (BN / 2);
    default: return (H + BN - 1) / BN;  // kWgDown
  }
}
template <int KIND>
__host__ __device__ inline int wgrad_mtiles(int H, int I, int BM) {
  return KIND == kWgUp ? (H + BM - 1) / BM : (I + BM - 1) / BM;
}

// Operand pointers and extents of tile (tm, tn).  Forward kinds: tm indexes
// the row-tile table built from the expert offsets; wgrad kinds: tm indexes
// (group, m-tile) over the fixed weight shapes and K runs over the group's rows.
template <typename S, int KIND, int BM, int BN>
__device__ inline TileDesc<S> decode_tile(const GemmArgs& g, int tm, int tn) {
  TileDesc<S> d;
  d.skip = false;
  d.ksplit = INT_MAX;
  d.b1 = nullptr;
  const int64_t H = g.H, I = g.I, T = g.T, R = g.R;
  if constexpr (!KindTraits<KIND>::kWgrad) {
    if (tm >= *g.n_mtiles) {
      d.skip = true;
      return d;
    }
    const int4 mt = g.mtiles[tm];
    const int grp = mt.x;
    const int64_t row0 = mt.y;
    const bool shared = grp >= g.E;
    const int64_t sidx = grp - g.E;
    const int64_t tok0 = shared ? row0 - R - sidx * T : 0;
    d.group = grp;
    d.row0 = row0;
    d.m_valid = mt.z;
    if constexpr (KIND == kUp) {
      d.a = shared ? static_cast<const S*>(g.x) + tok0 * H : static_cast<const S*>(g.x_perm) + row0 * H;
      d.a_sm = H; d.a_sk = 1;
      const S* W1 = shared ? static_cast<const S*>(g.ws1) + sidx * H * I : static_cast<const S*>(g.w1) + (int64_t)grp * H * I;
      const S* W3 = shared ? static_cast<const S*>(g.ws3) + sidx * H * I : static_cast<const S*>(g.w3) + (int64_t)grp * H * I;
      d.col0 = tn * (BN / 2);
      d.b0 = W1 + d.col0; d.b1 = W3 + d.col0;
      d.b_sk = I; d.b_sn = 1;
      d.n_valid = (int)min<int64_t>(BN / 2, I - d.col0);
      d.k_len = (int)H;
    } else if constexpr (KIND == kDown) {
      d.a = static_cast<const S*>(g.h) + row0 * I;
      d.a_sm = I; d.a_sk = 1;
      const S* W2 = shared ? static_cast<const S*>(g.ws2) + sidx * I * H : static_cast<const S*>(g.w2) + (int64_t)grp * I * H;
      d.col0 = tn * BN;
      d.b0 = W2 + d.col0;
      d.b_sk = H; d.b_sn = 1;
      d.n_valid = (int)min<int64_t>(BN, H - d.col0);
      d.k_len = (int)I;
    } else if constexpr (KIND == kBwdUp) {
      d.a = shared ? static_cast<const S*>(g.dout) + tok0 * H : static_cast<const S*>(g.dy) + row0 * H;
      d.a_sm = H; d.a_sk = 1;
      const S* W2 = shared ? static_cast<const S*>(g.ws2) + sidx * I * H : static_cast<const S*>(g.w2) + (int64_t)grp * I * H;
      d.col0 = tn * BN;
      d.b0 = W2 + (int64_t)d.col0 * H;   // B(k=h, n=i) = W2[i][h]
      d.b_sn = H; d.b_sk = 1;
      d.n_valid = (int)min<int64_t>(BN, I - d.col0);
      d.k_len = (int)H;
    } else {  // kBwdDown
      d.a = static_cast<const S*>(g.dab) + row0 * 2 * I;
      d.a_sm = 2 * I; d.a_sk = 1;
      const S* W1 = shared ? static_cast<const S*>(g.ws1) + sidx * H * I : static_cast<const S*>(g.w1) + (int64_t)grp * H * I;
      const S* W3 = shared ? static_cast<const S*>(g.ws3) + sidx * H * I : static_cast<const S*>(g.w3) + (int64_t)grp * H * I;
      d.col0 = tn * BN;
      d.b0 = W1 + (int64_t)d.col0 * I;   // B(k=i, n=h) = W1[h][i] for k < I, W3[h][k-I] after
      d.b1 = W3 + (int64_t)d.col0 * I;
      d.b_sn = I; d.b_sk = 1;
      d.ksplit = (int)I;
      d.n_valid = (int)min<int64_t>(BN, H - d.col0);
      d.k_len = (int)(2 * I);
    }
  } else {
    const int mtg = wgrad_mtiles<KIND>(g.H, g.I, BM);
    const int grp = tm / mtg;
    const int mti = tm - grp * mtg;
    const bool shared = grp >= g.E;
    const int64_t sidx = grp - g.E;
    int64_t r0, rows;
    const S* X;
    const S* DY;
    if (!shared) {
      r0 = g.offsets[grp];
      rows = g.offsets[grp + 1] - r0;
      X = static_cast<const S*>(g.x_perm) + r0 * H;
      DY = static_cast<const S*>(g.dy) + r0 * H;
    } else {
      r0 = R + sidx * T;
      rows = T;
      X = static_cast<const S*>(g.x);
      DY = static_cast<const S*>(g.dout);
    }
    d.group = grp;
    d.k_len = (int)rows;
    const int64_t m0 = (int64_t)mti * BM;
    d.row0 = m0;
    if constexpr (KIND == kWgUp) {
      d.a = X + m0;                       // A(m=h, k=r) = X[r][h]
      d.a_sm = 1; d.a_sk = H;
      d.m_valid = (int)min<int64_t>(BM, H - m0);
      d.col0 = tn * (BN / 2);
      d.b0 = static_cast<const S*>(g.dab) + r0 * 2 * I + d.col0;  // da(k=r, n=i)
      d.b1 = d.b0 + I;                                             // db
      d.b_sk = 2 * I; d.b_sn = 1;
      d.n_valid = (int)min<int64_t>(BN / 2, I - d.col0);
    } else {
      d.a = static_cast<const S*>(g.h) + r0 * I + m0;  // A(m=i, k=r) = h[r][i]
      d.a_sm = 1; d.a_sk = I;
      d.m_valid = (int)min<int64_t>(BM, I - m0);
      d.col0 = tn * BN;
      d.b0 = DY + d.col0;                 // B(k=r, n=h) = dY[r][h]
      d.b_sk = H; d.b_sn = 1;
      d.n_valid = (int)min<int64_t>(BN, H - d.col0);
    }
  }
  return d;
}

// Store one output element (m, n) of a tile; v2 is the paired value (b for
// kUp, dW3 for kWgUp).
template <typename S, int KIND>
__device__ __forceinline__ void emit(const GemmArgs& g, const TileDesc<S>& d, int m, int n, float v,
                                     float v2) {
  const int64_t H = g.H, I = g.I;
  const int64_t r = d.row0 + m;
  const int64_t c = d.col0 + n;
  if constexpr (KIND == kUp) {
    Elem<S>::store1(g.o_ab, r * 2 * I + c, v);
    Elem<S>::store1(g.o_ab, r * 2 * I + I + c, v2);
    Elem<S>::store1(g.o_h, r * I + c, silu_f(v) * v2);
  } else if constexpr (KIND == kDown) {
    Elem<S>::store1(g.o_y, r * H + c, v);
  } else if constexpr (KIND == kBwdUp) {
    const float a = Elem<S>::load1(g.ab, r * 2 * I + c);
    const float b = Elem<S>::load1(g.ab, r * 2 * I + I + c);
    const float s = sigmoid_f(a);
    Elem<S>::store1(g.o_dab, r * 2 * I + c, v * b * s * (1.0f + a * (1.0f - s)));
    Elem<S>::store1(g.o_dab, r * 2 * I + I + c, v * a * s);
  } else if constexpr (KIND == kBwdDown) {
    Elem<S>::store1(g.o_dx, r * H + c, v);
  } else if constexpr (KIND == kWgUp) {
    const bool shared = d.group >= g.E;
    const int64_t e = shared ? d.group - g.E : d.group;
    float* w1 = (shared ? g.o_dws1 : g.o_dw1) + e * H * I;
    float* w3 = (shared ? g.o_dws3 : g.o_dw3) + e * H * I;
    __builtin_nontemporal_store(v, w1 + r * I + c);
    __builtin_nontemporal_store(v2, w3 + r * I + c);
  } else {  // kWgDown
    const bool shared = d.group >= g.E;
    const int64_t e = shared ? d.group - g.E : d.group;
    float* w2 = (shared ? g.o_dws2 : g.o_dw2) + e * I * H;
    __builtin_nontemporal_store(v, w2 + r * H + c);
  }
}

// ----------------------------------------------------------------- bf16 ----

// LDS element offset of (row, k): rows of kBK bf16, 16-byte chunks swizzled.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// K-contiguous operand: BMN rows x 64 k, 16-byte chunks.
template <int BMN, int NT>
struct LoadKC {
  static constexpr int kN = BMN * (kBK / 8) / NT;
  static_assert(kN >= 1 && BMN * (kBK / 8) % NT == 0, "tile/threads mismatch");
  u32x4 r[kN];
  // p points at element (mn = 0, k = k0) of the tile's rows; s_mn = row stride.
  __device__ __forceinline__ void load(const uint16_t* p, int64_t s_mn, int mn_valid, int tid) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int id = tid + i * NT;
      const int mn = id >> 3, ch = id & 7;
      if (mn < mn_valid)
        r[i] = ld16(p + (int64_t)mn * s_mn + ch * 8);
      else
        r[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int id = tid + i * NT;
      st16(s + lds_off(id >> 3, id & 7), r[i]);
    }
  }
};

// MN-contiguous operand: 64 k rows x BMN columns, read as 8(k) x 4(mn)
// blocks of 8-byte loads, transposed in registers, stored K-contiguous.
template <int BMN, int NT, bool PAIRED>
struct LoadMN {
  static constexpr int kBlocksMN = BMN / 4;
  static constexpr int kNB = (kBK / 8) * kBlocksMN / NT;
  static_assert(kNB >= 1 && (kBK / 8) * kBlocksMN % NT == 0, "tile/threads mismatch");
  u32x2 r[kNB][8];
  // p0 (and p1 for paired) point at element (k = k0, mn = 0); s_k = k stride.
  // mn_valid counts per half when PAIRED; k_valid = valid k rows from k0.
  __device__ __forceinline__ void load(const uint16_t* p0, const uint16_t* p1, int64_t s_k,
                                       int mn_valid, int k_valid, int tid) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int id = tid + b * NT;
      const int kb = id / kBlocksMN, mb = id - kb * kBlocksMN;
      int mn = mb * 4;
      const uint16_t* p = p0;
      if constexpr (PAIRED) {
        if (mn >= BMN / 2) {
          p = p1;
          mn -= BMN / 2;
        }
      }
      const bool mn_ok = mn < mn_valid;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = kb * 8 + j;
        if (mn_ok && k < k_valid)
          r[b][j] = *reinterpret_cast<const u32x2*>(p + (int64_t)k * s_k + mn);
        else
          r[b][j] = u32x2{0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int id = tid + b * NT;
      const int kb = id / kBlocksMN, mb = id - kb * kBlocksMN;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = __builtin_amdgcn_perm(r[b][2 * q + 1][n >> 1], r[b][2 * q][n >> 1], sel);
        st16(s + lds_off(mb * 4 + n, kb), o);
      }
    }
  }
};

template <int KIND_, int BM_, int BN_, int WGM_, int WGN_>
struct BfCfg {
  static constexpr int KIND = KIND_, BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int NT = WGM * WGN * kWave;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  static constexpr bool PAIRED = KindTraits<KIND>::kPaired;
  static constexpr int LDS_BYTES = 2 * (BM + BN) * kBK * 2;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be made of 32x32 blocks");
  static_assert(!PAIRED || (NJ % 2 == 0), "paired kinds need an even number of N blocks");
};

// B-tile LDS row of the first column of wave wn's N-block j.  Paired kinds
// keep gate columns in rows [0, BN/2) and up columns in [BN/2, BN); block j and
// block j + NJ/2 of a wave then cover the same output column.
template <class C>
__device__ __forceinline__ int b_row(int wn, int j) {
  if constexpr (C::PAIRED) {
    constexpr int HJ = C::NJ / 2;
    return (j / HJ) * (C::BN / 2) + wn * (C::WN / 2) + 32 * (j % HJ);
  } else {
    return wn * C::WN + 32 * j;
  }
}

// The whole tile: K loop over LDS double buffers, then the epilogue.
template <class C>
__device__ void run_tile_bf16(const GemmArgs& g, const TileDesc<uint16_t>& d, uint16_t* smem) {
  constexpr int BM = C::BM, BN = C::BN, NT = C::NT, MI = C::MI, NJ = C::NJ;
  using TA = KindTraits<C::KIND>;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  uint16_t* sA[2] = {smem, smem + BM * kBK};
  uint16_t* sB[2] = {smem + 2 * BM * kBK, smem + 2 * BM * kBK + BN * kBK};

  typename std::conditional<TA::kAMn, LoadMN<BM, NT, false>, LoadKC<BM, NT>>::type la;
  typename std::conditional<TA::kBMn, LoadMN<BN, NT, C::PAIRED>, LoadKC<BN, NT>>::type lb;

  auto load = [&](int kt) {
    const int k0 = kt * kBK;
    if constexpr (TA::kAMn)
      la.load(d.a + (int64_t)k0 * d.a_sk, nullptr, d.a_sk, d.m_valid, d.k_len - k0, tid);
    else
      la.load(d.a + k0, d.a_sm, d.m_valid, tid);
    if constexpr (TA::kBMn) {
      lb.load(d.b0 + (int64_t)k0 * d.b_sk, C::PAIRED ? d.b1 + (int64_t)k0 * d.b_sk : nullptr,
              d.b_sk, d.n_valid, d.k_len - k0, tid);
    } else {
      const uint16_t* p = k0 < d.ksplit ? d.b0 + k0 : d.b1 + (k0 - d.ksplit);
      lb.load(p, d.b_sn, d.n_valid, tid);
    }
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (d.k_len + kBK - 1) / kBK;
  if (nk > 0) {
    load(0);
    la.store(sA[0], tid);
    lb.store(sB[0], tid);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
    const uint16_t* a_s = sA[cur];
    const uint16_t* b_s = sB[cur];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      bf16x8 av[MI], bv[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        av[i] = *reinterpret_cast<const bf16x8*>(a_s + lds_off(wm * C::WM + 32 * i + (lane & 31), ch));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bv[j] = *reinterpret_cast<const bf16x8*>(b_s + lds_off(b_row<C>(wn, j) + (lane & 31), ch));
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      la.store(sA[cur ^ 1], tid);
      lb.store(sB[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane & 31) and
  // rows 8*(r/4) + 4*(lane/32) + (r%4), r = 0..15.
  const int ncol = lane & 31;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    if constexpr (C::PAIRED) {
      constexpr int HJ = NJ / 2;
#pragma unroll
      for (int j = 0; j < HJ; ++j) {
        const int n = wn * (C::WN / 2) + 32 * j + ncol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * C::WM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (m < d.m_valid && n < d.n_valid)
            emit<uint16_t, C::KIND>(g, d, m, n, acc[i][j][r], acc[i][j + HJ][r]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int n = wn * C::WN + 32 * j + ncol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = wm * C::WM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (m < d.m_valid && n < d.n_valid)
            emit<uint16_t, C::KIND>(g, d, m, n, acc[i][j][r], 0.f);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ f32 ----

constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 16, kF32NT = 256;

template <int KIND>
__device__ void run_tile_f32(const GemmArgs& g, const TileDesc<float>& d, float* smem) {
  constexpr bool PAIRED = KindTraits<KIND>::kPaired;
  float (*sA)[kF32BM + 4] = reinterpret_cast<float (*)[kF32BM + 4]>(smem);
  float (*sB)[kF32BN + 4] = reinterpret_cast<float (*)[kF32BN + 4]>(smem + kF32BK * (kF32BM + 4));
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  auto col_of = [&](int jj) { return PAIRED ? (jj < 2 ? 2 * tx + jj : 32 + 2 * tx + (jj - 2)) : 4 * tx + jj; };
  for (int k0 = 0; k0 < d.k_len; k0 += kF32BK) {
#pragma unroll
    for (int i = 0; i < kF32BM * kF32BK / kF32NT; ++i) {
      const int id = tid + i * kF32NT;
      const int m = id % kF32BM, k = id / kF32BM;
      const int kk = k0 + k;
      sA[k][m] = (m < d.m_valid && kk < d.k_len) ? d.a[(int64_t)m * d.a_sm + (int64_t)kk * d.a_sk] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kF32BN * kF32BK / kF32NT; ++i) {
      const int id = tid + i * kF32NT;
      const int n = id % kF32BN, k = id / kF32BN;
      int kk = k0 + k;
      const float* p = d.b0;
      int nl = n;
      if (PAIRED && n >= kF32BN / 2) {
        p = d.b1;
        nl = n - kF32BN / 2;
      }
      if (kk >= d.ksplit) {
        p = d.b1;
        kk -= d.ksplit;
      }
      const bool ok = nl < d.n_valid && (k0 + k) < d.k_len;
      sB[k][n] = ok ? p[(int64_t)kk * d.b_sk + (int64_t)nl * d.b_sn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kF32BK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sA[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = sB[k][col_of(j)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty * 4 + i;
    if (PAIRED) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = 2 * tx + j;
        if (m < d.m_valid && n < d.n_valid) emit<float, KIND>(g, d, m, n, acc[i][j], acc[i][j + 2]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = 4 * tx + j;
        if (m < d.m_valid && n < d.n_valid) emit<float, KIND>(g, d, m, n, acc[i][j], 0.f);
      }
    }
  }
}

constexpr int kF32LdsFloats = kF32BK * (kF32BM + 4) + kF32BK * (kF32BN + 4);

}  // namespace moe
