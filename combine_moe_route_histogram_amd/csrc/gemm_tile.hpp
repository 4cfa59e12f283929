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
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16.  Operands move global -> LDS
// with buffer loads that write LDS directly (no register staging), each
// operand in the layout it has in memory: K-contiguous operands as [row][64 k]
// with 16-byte chunks XOR-swizzled by row, read back with ds_read_b128;
// MN-contiguous operands (weights in the forward, both operands of the weight
// gradient) as [k][columns] with a chunk XOR of 4 (k mod 4), read back with
// the gfx950 LDS transpose read ds_read_b64_tr_b16, which hands each MFMA
// lane its 8 consecutive k directly.  A ring of LDS k slices: the loads of
// the next slice are in flight while the MFMAs of the current one run.
//
// f32 path: plain LDS-tiled FMA kernel (the MI355X fp32 vector and fp32
// matrix peaks are equal, so VALU FMA loses nothing for fp32).
#pragma once

#include <climits>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kBK = 64;  // default k per LDS slice (bf16)

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
  const int32_t* a_rows;  // non-null: row m of A is row a_rows[m] of a (gathered rows)
  bool skip;
};

template <int KIND>
struct KindTraits {
  static constexpr bool kPaired = (KIND == kUp || KIND == kWgUp);
  static constexpr bool kWgrad = (KIND == kWgUp || KIND == kWgDown);
  static constexpr bool kAMn = kWgrad;                        // A is MN-contiguous
  static constexpr bool kBMn = (KIND == kUp || KIND == kDown || kWgrad);  // B is N-contiguous
  // k split of tail tiles: the kinds with a long k and few column tiles (the
  // down projection and the input gradient); the others run many rounds of
  // tiles per launch, where the tail is a small share
  static constexpr bool kSplit = (KIND == kDown || KIND == kBwdDown);
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
  d.a_rows = nullptr;
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
      if (shared) {
        d.a = static_cast<const S*>(g.x) + tok0 * H;
      } else if (g.a_rows) {   // dispatch folded into the operand load
        d.a = static_cast<const S*>(g.x);
        d.a_rows = g.a_rows + row0;
      } else {
        d.a = static_cast<const S*>(g.x_perm) + row0 * H;
      }
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
//
// LDS layouts (one stage; a stage holds one 64-deep k slice of both operands):
//  K-contiguous operand ("KC"): rows = m (or n), 64 k per row = 128 bytes;
//    16-byte chunk c of row r is stored at chunk c ^ ((r >> 1) & 7).  A wave's
//    16-byte fragment reads of 16 consecutive rows then hit 16 distinct bank
//    groups.
//  MN-contiguous operand ("MN"): rows = k (64 of them), the m (or n) columns
//    contiguous, in one or two sub-tiles of >= 128 columns (paired kinds keep
//    their two source tensors in separate sub-tiles); 16-byte chunk c of row k
//    is stored at chunk c ^ (4 * (k % 4)), which keeps the transposed reads
//    below free of bank conflicts.
// Operands move global -> LDS with buffer loads that write LDS directly (lane
// l of an instruction fills bytes [16 l, 16 l + 16) of a 1 KiB LDS block), so
// no register staging or VALU work is spent on the copy.  Rows or k outside
// the valid range use an out-of-range buffer offset and land as zeros.
// Fragment reads: KC operands with ds_read_b128 (8 consecutive k of one row);
// MN operands with two ds_read_b64_tr_b16 (gfx950 LDS transpose read: in each
// 16-lane group, lanes 4j..4j+3 point at 16 consecutive columns of k row j and
// lane i receives column i of the 4 rows), giving the same 8 consecutive k.

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_t;

constexpr uint32_t kBufRecords = 0x7FFFFFF0u;
constexpr uint32_t kBufInvalid = 0x80000000u;
constexpr int kBufDword3 = 0x00020000;  // raw buffer, 32-bit data (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, kBufRecords, kBufDword3);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, void* lds_block, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t)lds_block, 16, voff, 0, 0, 0);
}

// Byte offset of (row, 16-byte chunk) inside a KC slice of BK k per row.  A
// 256-byte bank row holds 16 / (BK/8) tile rows; the chunk index is XORed with
// the bank-row index so 16 consecutive rows' same chunk hit 16 bank groups.
template <int BK>
__device__ __forceinline__ uint32_t kc_off(int row, int chunk) {
  constexpr int kCpr = BK / 8, kRpb = 16 / kCpr;
  return (uint32_t)(row * BK * 2 + ((chunk ^ ((row / kRpb) & (kCpr - 1))) << 4));
}
// Byte offset of (k, column) inside an MN sub-tile of `cols` columns.
__device__ __forceinline__ uint32_t mn_off(int k, int col, int cols) {
  return (uint32_t)(k * cols * 2 + ((((col >> 3) ^ (4 * (k & 3)))) << 4) + (col & 7) * 2);
}

// Global -> LDS copy of one operand stage.
//  KC: rows BMN, 8 rows per 1 KiB instruction.
//  MN: NH sub-tiles of HMN columns, 64 k rows, 1024 / (2 HMN) rows per instruction.
template <int BMN, int NW, bool MN, int NH, bool RAGGED_K, int BK>
struct DmaOperand {
  static constexpr int kHMN = BMN / NH;
  static constexpr int kCpr = BK / 8;                       // 16-byte chunks per KC row
  static constexpr int kInstr = BMN * BK * 2 / 1024;        // 1 KiB instructions per slice
  static constexpr int kPerWave = kInstr / NW;
  static_assert(kInstr % NW == 0, "stage copy must split evenly over the waves");
  static_assert(!MN || kHMN >= 128, "MN sub-tiles need >= 128 columns");
  static_assert(MN || NH == 1, "KC operands have one source");
  uint32_t off[kPerWave];   // per-lane byte offset (relative to the k slice start) or invalid
  int krow[RAGGED_K ? kPerWave : 1];  // ragged K: k of this lane's load within the slice
                                      // (MN: its k row; KC: its chunk's first k)
  // s = row stride (KC) or k stride (MN) in elements; mn_valid per sub-tile;
  // rows (KC only, may be null): source row of each tile row, for gathered
  // operands (the host keeps every such byte offset below 2^31).
  __device__ __forceinline__ void init(int64_t s, int mn_valid, int wave, int lane,
                                       const int32_t* rows = nullptr) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int q = wave + NW * i;                           // instruction index in the stage
      if constexpr (!MN) {
        constexpr int kRpi = 1024 / (BK * 2);                 // rows per instruction
        const int r = kRpi * q + lane / kCpr;
        const int c = (lane % kCpr) ^ ((r / (16 / kCpr)) & (kCpr - 1));
        if (r < mn_valid) {
          const int64_t src = rows ? (int64_t)rows[r] : (int64_t)r;
          off[i] = (uint32_t)(src * s * 2 + c * 16);
        } else {
          off[i] = kBufInvalid;
        }
        if constexpr (RAGGED_K) krow[i] = c * 8;
      } else {
        constexpr int kQHalf = kHMN * BK * 2 / 1024;         // instructions per sub-tile
        const int qh = q % kQHalf;
        const int byte = qh * 1024 + 16 * lane;
        const int k = byte / (2 * kHMN);
        const int p = (byte % (2 * kHMN)) / 16;
        const int col = (p ^ (4 * (k & 3))) * 8;
        off[i] = col < mn_valid ? (uint32_t)(k * s * 2 + col * 2) : kBufInvalid;
        if constexpr (RAGGED_K) krow[i] = k;
      }
    }
  }
  // Issue the copy of one k slice.  src0/src1: operand at (k slice start,
  // column 0) of sub-tile 0/1 (KC: row 0 at k0); k_valid: valid k of the
  // slice (used with RAGGED_K; loads past it are zero-filled); live false:
  // the slice lies past the end of k and is filled with zeros.
  __device__ __forceinline__ void issue(uint8_t* stage, const uint16_t* src0, const uint16_t* src1,
                                        int k_valid, bool live, int wave) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int q = wave + NW * i;
      const uint16_t* src = src0;
      if constexpr (NH == 2) {
        constexpr int kQHalf = kHMN * BK * 2 / 1024;
        if (q >= kQHalf) src = src1;
      }
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(src);
      uint32_t o = live ? off[i] : kBufInvalid;
      if constexpr (RAGGED_K) o = krow[i] < k_valid ? o : kBufInvalid;
      dma16(rs, stage + q * 1024, o);
    }
  }
};

template <int KIND_, int BM_, int BN_, int WGM_, int WGN_, int STAGES_, int BK_ = kBK>
struct BfCfg {
  static constexpr int KIND = KIND_, BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, STAGES = STAGES_;
  static constexpr int BK = BK_;
  static_assert(BK == 32 || BK == 64, "k slice of 32 or 64");
  static constexpr int NW = WGM * WGN, NT = NW * kWave;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  static constexpr bool PAIRED = KindTraits<KIND>::kPaired;
  static constexpr bool A_MN = KindTraits<KIND>::kAMn, B_MN = KindTraits<KIND>::kBMn;
  static constexpr int B_NH = PAIRED ? 2 : 1;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be made of 32x32 blocks");
  static_assert(!PAIRED || (NJ % 2 == 0), "paired kinds need an even number of N blocks");
  static_assert(STAGES >= 2, "at least double buffering");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Fragment reads.  kc_frag: 8 consecutive k (16-byte chunk ch) of row `row`.
template <int BK>
__device__ __forceinline__ bf16x8 kc_frag(const uint8_t* tile, int row, int ch) {
  return *reinterpret_cast<const bf16x8*>(tile + kc_off<BK>(row, ch));
}
// mn_frag: for MFMA lane l, column col0 + (l % 32) and k rows 8 * (l / 32) +
// 16 * ks .. + 8 of an MN sub-tile of `cols` columns.
__device__ __forceinline__ bf16x8 mn_frag(const uint8_t* tile, int cols, int col0, int ks, int lane) {
  const int h = lane >> 4, i = lane & 15;
  const int k = 16 * ks + 8 * (h >> 1) + (i >> 2);
  const int col = col0 + 16 * (h & 1) + 4 * (i & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t)(tile + mn_off(k, col, cols)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t)(tile + mn_off(k + 4, col, cols)));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// First column (within its B sub-tile) of wave wn's N-block j, and the sub-tile.
// Paired kinds: block j and block j + NJ/2 cover the same output column, from
// the first and the second source tensor.
template <class C>
__device__ __forceinline__ void b_block(int wn, int j, int& sub, int& col) {
  if constexpr (C::PAIRED) {
    constexpr int HJ = C::NJ / 2;
    sub = j / HJ;
    col = wn * (C::WN / 2) + 32 * (j % HJ);
  } else {
    sub = 0;
    col = wn * C::WN + 32 * j;
  }
}

// Scheduling pattern for one k step: NM MFMAs, each followed by its share of
// the ND LDS fragment reads and the NV global->LDS loads, so the matrix pipe
// is fed while reads and loads issue instead of waiting behind a burst of them.
template <int T, int NM, int ND, int NV>
__device__ __forceinline__ void interleave_step() {
  if constexpr (T < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    constexpr int nd = ND * (T + 1) / NM - ND * T / NM;
    constexpr int nv = NV * (T + 1) / NM - NV * T / NM;
    if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nd, 0);   // LDS reads
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);   // VMEM loads
    interleave_step<T + 1, NM, ND, NV>();
  }
}

// f(std::integral_constant<int, n>) for a run-time n in [0, N].
template <int N, class F>
__device__ __forceinline__ void with_count(int n, F&& f) {
  if constexpr (N >= 0) {
    if (n == N) {
      f(std::integral_constant<int, N>{});
      return;
    }
    with_count<N - 1>(n, f);
  }
}

template <int IMM>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt with vmcnt = IMM, expcnt and lgkmcnt left at their maximum
  static_assert(IMM >= 0 && IMM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((IMM & 0xF) | ((IMM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that orders LDS accesses around it without making the
// compiler drain the outstanding global->LDS loads (the ring waits for those
// itself, slice by slice).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), visible to the compiler's wait tracking
  asm volatile("s_barrier" ::: "memory");
}

// The LDS slices of one tile worker: separate LDS objects, so the compiler can
// tell the loads into one slice from the fragment reads of another.
#define MOE_LDS_RING(C, name)                                                       \
  __shared__ __align__(16) uint8_t name##0[C::STAGE_BYTES];                         \
  __shared__ __align__(16) uint8_t name##1[C::STAGE_BYTES];                         \
  __shared__ __align__(16) uint8_t name##2[C::STAGES > 2 ? C::STAGE_BYTES : 16];    \
  __shared__ __align__(16) uint8_t name##3[C::STAGES > 3 ? C::STAGE_BYTES : 16];    \
  uint8_t* const name[4] = {name##0, name##1, name##2, name##3}

// Block (wm, wn) of the tile that wave `wave` computes.  Normally wm = wave /
// WGN, wn = wave % WGN.  The waves of a workgroup run on the CU's four SIMDs in
// turn (wave w on SIMD w % 4), so with the 2 x 4 layout the waves of one wn
// share a SIMD pair; a tile with at most half of its columns valid (the last
// column tile when N is an odd multiple of BN/2, e.g. I = 1408 for 256-wide
// tiles) would then leave two SIMDs with no MFMA work and the other two with
// two waves each.  Such a tile takes wm = wave % WGM, wn = wave / WGM instead,
// so its active waves (wn < WGN/2) are one per SIMD.  Which wave computes a
// block does not change the block's arithmetic.
template <class C>
__device__ __forceinline__ void wave_block(const TileDesc<uint16_t>& d, int wave, int& wm, int& wn) {
  constexpr bool kCanSpread = !C::PAIRED && C::WGM == 2 && C::WGN == 4;
  if (kCanSpread && d.n_valid <= C::BN / 2 && d.m_valid > C::BM / 2) {
    wm = wave % C::WGM;
    wn = wave / C::WGM;
  } else {
    wm = wave / C::WGN;
    wn = wave % C::WGN;
  }
}

// Epilogue of one tile.  Each wave owns a WM x WN block of the tile; it moves
// its accumulators, 32 rows x 64 columns (two 32x32 blocks) at a time, through
// its own LDS region (row pitch 72 floats so the scattered writes of the 32x32
// accumulator layout and the row reads below are both free of bank
// conflicts), then every lane handles 4 consecutive columns of one row:
// 8-byte bf16 or 16-byte f32 stores, 8-byte loads of the saved activations.
// Paired kinds keep the two values of an output column in region columns c and
// c + 32 (blocks j and j + NJ/2).
constexpr int kEpiPitch = 72;                      // floats per region row
constexpr int kEpiRegionBytes = 32 * kEpiPitch * 4;

__device__ __forceinline__ void st_bf16x4(void* p, const float* v) {
  u32x2 w;
  w[0] = pack_bf16x2(v[0], v[1]);
  w[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(p) = w;
}
// The same with a non-temporal store: for the activation gradient's da | db,
// which no tile of the launch reads back soon and which exceed the Infinity
// Cache at the long-sequence size (one-launch backward 16.08 -> 16.02 ms
// there, equal at the Mixtral-like size; non-temporal a | b, h or dx_rows
// stores were slower or equal).
__device__ __forceinline__ void st_bf16x4_nt(void* p, const float* v) {
  u32x2 w;
  w[0] = pack_bf16x2(v[0], v[1]);
  w[1] = pack_bf16x2(v[2], v[3]);
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}
// Stores that other workgroups of the same launch read (the down
// projection's output rows, which the fused combine reads, and split-k
// partial sums): relaxed agent-scope atomic stores.  Each is coherent at
// device scope once it completes (the per-XCD L2 writes it through), so a
// publish only has to wait for the wave's stores; a release fence would write
// back the whole L2 of the XCD at every publish.
__device__ __forceinline__ void st_agent_u64(void* p, uint64_t v) {
  __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_bf16x4(void* p, const float* v) {
  const uint64_t lo = pack_bf16x2(v[0], v[1]);
  const uint64_t hi = pack_bf16x2(v[2], v[3]);
  st_agent_u64(p, lo | (hi << 32));
}
// Split-k partial tiles: in each 64-float row of a staging block, columns
// 4j, 4j+1 sit at 2j and columns 4j+2, 4j+3 at 32 + 2j, so each 8-byte store
// instruction of 16 lanes covers one whole 128-byte line.
__device__ __forceinline__ void st_part4(float* row, int c4, const f32x4& v) {
  const int j = c4 >> 2;
  st_agent_u64(row + 2 * j, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32));
  st_agent_u64(row + 32 + 2 * j, (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32));
}
__device__ __forceinline__ f32x4 ld_part4(const float* row, int c4) {
  const int j = c4 >> 2;
  const f32x2 lo = *reinterpret_cast<const f32x2*>(row + 2 * j);
  const f32x2 hi = *reinterpret_cast<const f32x2*>(row + 32 + 2 * j);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}
__device__ __forceinline__ void ld_bf16x4(const void* p, float* v) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  v[0] = __uint_as_float(w[0] << 16); v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
  v[2] = __uint_as_float(w[1] << 16); v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
}
// sigmoid(a) = 1 / (1 + e^-a) with the hardware exponential and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp each; the argument of the reciprocal is
// >= 1, so no denormal or overflow case: e^-a = inf gives 0).  A correctly
// rounded reciprocal expands to a division sequence of about ten
// instructions, which the gate/up and activation-gradient epilogues would run
// 64 times per lane per tile.
__device__ __forceinline__ float fast_sigmoid(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// k-split parts: part_out (a helper) receives the tile's partial sums instead
// of the outputs; part_in[0 .. n_in) (the owner's helpers) are added, in that
// order, before the outputs are formed.  A partial tile holds, per wave and
// 32 x 64 staging block, the block's rows of 64 f32 -- the same elements, in
// the same places, that the epilogue reads back from its LDS region.
template <class C, bool kCoherentY>
__device__ __forceinline__ void epilogue_bf16(const GemmArgs& g, const TileDesc<uint16_t>& d,
                                              const f32x16 (&acc)[C::MI][C::NJ],
                                              uint8_t* const (&stages)[4], int wave, int lane,
                                              float* part_out, const float* part_in, int n_in,
                                              int64_t part_floats) {
  constexpr int MI = C::MI, NJ = C::NJ, KIND = C::KIND;
  static_assert(NJ % 2 == 0, "the region takes two 32-column blocks at a time");
  constexpr int kRps = C::STAGE_BYTES / kEpiRegionBytes;   // regions per LDS slice
  static_assert(kRps >= 1 && (C::NW + kRps - 1) / kRps <= C::STAGES, "epilogue regions fit in the slices");
  int wm, wn;
  wave_block<C>(d, wave, wm, wn);
  const int rs = wave / kRps;
  uint8_t* const rbase = rs == 0 ? stages[0] : rs == 1 ? stages[1] : rs == 2 ? stages[2] : stages[3];
  float* reg = reinterpret_cast<float*>(rbase + (wave - rs * kRps) * kEpiRegionBytes);
  const int64_t H = g.H, I = g.I;
  // output column of the wave's first column (paired: of both values)
  const int ncol0 = C::PAIRED ? wn * (C::WN / 2) : wn * C::WN;
  // activation gradient: the saved a, b of the lane's 8 row pieces of a
  // 32 x 64 block, loaded one block ahead so that only the first block waits
  // on a global round trip (a load issued after a block's stores would wait
  // for them too: stores count in vmcnt)
  constexpr bool kLoadAB = (KIND == kBwdUp);
  u32x2 ab_buf[2][8][2];
  auto load_ab = [&](int i, int hc, u32x2 (&buf)[8][2]) {
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      // unconditional loads (a branch per load would make the compiler's
      // wait tracking conservative); a lane outside the tile's valid part
      // reads the tile's first element instead, and its result is not stored
      int m = wm * C::WM + 32 * i + pass * 4 + (lane >> 4);
      int n = ncol0 + 64 * hc + 4 * (lane & 15);
      const bool ok = m < d.m_valid && n < d.n_valid;
      m = ok ? m : 0;
      n = ok ? n : 0;
      const uint16_t* ab = static_cast<const uint16_t*>(g.ab) + (d.row0 + m) * 2 * I + d.col0 + n;
      buf[pass][0] = *reinterpret_cast<const u32x2*>(ab);
      buf[pass][1] = *reinterpret_cast<const u32x2*>(ab + I);
    }
  };
  if constexpr (kLoadAB) load_ab(0, 0, ab_buf[0]);
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int hc = 0; hc < NJ / 2; ++hc) {
      const int blk = i * (NJ / 2) + hc;
      if constexpr (kLoadAB) {
        if (blk + 1 < MI * (NJ / 2))
          load_ab((blk + 1) / (NJ / 2), (blk + 1) % (NJ / 2), ab_buf[(blk + 1) & 1]);
      }
      // two accumulator blocks -> region columns 0..31 and 32..63: paired
      // kinds take block hc and its partner hc + NJ/2 (same output columns),
      // others two neighbouring blocks
      const int j0 = C::PAIRED ? hc : 2 * hc;
      const int j1 = C::PAIRED ? hc + NJ / 2 : 2 * hc + 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        reg[row * kEpiPitch + (lane & 31)] = acc[i][j0][r];
        reg[row * kEpiPitch + 32 + (lane & 31)] = acc[i][j1][r];
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's own region is written
      const int m_base = wm * C::WM + 32 * i;
      const int64_t pblk = (int64_t)((wave * MI + i) * (NJ / 2) + hc) * (32 * 64);
      if (KindTraits<KIND>::kSplit && part_out) {   // helper: the block's rows, as staged, to the partial tile
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
          const int q = pass * 4 + (lane >> 4);
          const int c4 = 4 * (lane & 15);
          st_part4(part_out + pblk + q * 64, c4, *reinterpret_cast<const f32x4*>(reg + q * kEpiPitch + c4));
        }
      } else if constexpr (C::PAIRED) {
        // 8 lanes per row, 4 columns of both values each; 8 rows per pass
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
          const int q = pass * 8 + (lane >> 3);
          const int c4 = 4 * (lane & 7);
          const int m = m_base + q, n = ncol0 + 32 * hc + c4;
          float v[4], w[4];
          const float4 va = *reinterpret_cast<const float4*>(reg + q * kEpiPitch + c4);
          const float4 vb = *reinterpret_cast<const float4*>(reg + q * kEpiPitch + 32 + c4);
          v[0] = va.x; v[1] = va.y; v[2] = va.z; v[3] = va.w;
          w[0] = vb.x; w[1] = vb.y; w[2] = vb.z; w[3] = vb.w;
          for (int t = 0; t < (KindTraits<KIND>::kSplit ? n_in : 0); ++t) {
            const float* pin = part_in + t * part_floats + pblk + q * 64;
            const f32x4 pa = ld_part4(pin, c4);
            const f32x4 pb = ld_part4(pin, 32 + c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] += pa[e];
              w[e] += pb[e];
            }
          }
          if (m < d.m_valid && n < d.n_valid) {
            const int64_t row = d.row0 + m, col = d.col0 + n;
            if constexpr (KIND == kUp) {
              uint16_t* ab = static_cast<uint16_t*>(g.o_ab) + row * 2 * I;
              st_bf16x4(ab + col, v);
              st_bf16x4(ab + I + col, w);
              float h[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) h[e] = v[e] * fast_sigmoid(v[e]) * w[e];
              st_bf16x4(static_cast<uint16_t*>(g.o_h) + row * I + col, h);
            } else {  // kWgUp: dW1 | dW3 columns of expert / shared group
              const bool shared = d.group >= g.E;
              const int64_t e = shared ? d.group - g.E : d.group;
              float* w1 = (shared ? g.o_dws1 : g.o_dw1) + e * H * I + row * I + col;
              float* w3 = (shared ? g.o_dws3 : g.o_dw3) + e * H * I + row * I + col;
              __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(v), reinterpret_cast<f32x4*>(w1));
              __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(w), reinterpret_cast<f32x4*>(w3));
            }
          }
        }
      } else {
        // 16 lanes per row, 4 columns each; 4 rows per pass
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
          const int q = pass * 4 + (lane >> 4);
          const int c4 = 4 * (lane & 15);
          const int m = m_base + q, n = ncol0 + 64 * hc + c4;
          const float4 va = *reinterpret_cast<const float4*>(reg + q * kEpiPitch + c4);
          float v[4] = {va.x, va.y, va.z, va.w};
          for (int t = 0; t < (KindTraits<KIND>::kSplit ? n_in : 0); ++t) {
            const f32x4 pa = ld_part4(part_in + t * part_floats + pblk + q * 64, c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += pa[e];
          }
          if (m < d.m_valid && n < d.n_valid) {
            const int64_t row = d.row0 + m, col = d.col0 + n;
            if constexpr (KIND == kDown) {
              if constexpr (kCoherentY)   // read by other workgroups of the launch
                st_agent_bf16x4(static_cast<uint16_t*>(g.o_y) + row * H + col, v);
              else
                st_bf16x4(static_cast<uint16_t*>(g.o_y) + row * H + col, v);
            } else if constexpr (KIND == kBwdDown) {
              st_bf16x4(static_cast<uint16_t*>(g.o_dx) + row * H + col, v);
            } else if constexpr (KIND == kBwdUp) {
              float a[4], b[4], da[4], db[4];
              ld_bf16x4(&ab_buf[blk & 1][pass][0], a);
              ld_bf16x4(&ab_buf[blk & 1][pass][1], b);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float sg = fast_sigmoid(a[e]);
                da[e] = v[e] * b[e] * sg * (1.0f + a[e] * (1.0f - sg));
                db[e] = v[e] * a[e] * sg;
              }
              uint16_t* dab = static_cast<uint16_t*>(g.o_dab) + row * 2 * I;
              st_bf16x4_nt(dab + col, da);
              st_bf16x4_nt(dab + I + col, db);
            } else {  // kWgDown
              const bool shared = d.group >= g.E;
              const int64_t e = shared ? d.group - g.E : d.group;
              float* w2 = (shared ? g.o_dws2 : g.o_dw2) + e * I * H + row * H + col;
              __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(v), reinterpret_cast<f32x4*>(w2));
            }
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // region reads done before it is rewritten
    }
  }
  __syncthreads();  // regions free for the next tile of a persistent worker
}

// One task of the tile scheduler: a whole tile, or part `part` of `parts`
// of a tile split along k (see for_tasks_xcd_ranges).
struct TaskPart {
  int L;            // logical tile
  int part, parts;  // parts == 1: the whole tile
  int slot;         // split tiles: the tile's index among its range's split tiles
  int range;        // XCD range
};

// Publish data written with agent-coherent stores (st_agent_*): every wave
// waits until its stores have completed (vmcnt 0: each is then coherent at
// device scope), then thread 0 counts the publish with an agent-scope atomic
// (on a second counter as well, if one is given).
// No release fence: the data a reader of this counter consumes is coherent
// already, and a release would write back the XCD's whole L2.  Readers poll
// the counter and then take one agent-scope acquire (which invalidates their
// L2's non-coherent lines) before reading.  The trailing barrier keeps thread
// 0's publish and a following claim in separate convergent regions, so the
// compiler cannot merge them across a loop edge into a thread-0-only path.
__device__ __forceinline__ void publish_add(int32_t* counter, int32_t* counter2 = nullptr) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (counter2) __hip_atomic_fetch_add(counter2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// Record of a bounded wait that gave up: one word per code object (each
// .hip file including this header has its own copy, taken by the host
// through take_wait_error_*), set with a vector atomic.
static __device__ uint32_t g_wait_error;

// Poll until *counter >= n + g.wait_extra, giving up (and recording it) after
// g.wait_ticks of the 100 MHz clock.  The caller's lanes may poll different
// counters.
__device__ __forceinline__ void poll_at_least(const GemmArgs& g, const int32_t* counter, int n) {
  const int target = n + g.wait_extra;
  if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return;
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (wall_clock64() - t0 >= g.wait_ticks) {
      __hip_atomic_fetch_or(&g_wait_error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Wait until *counter >= n (thread 0 polls with relaxed loads), then one
// agent-scope acquire in wave 0; the barrier orders the whole workgroup after
// it.  (An acquiring load per poll would invalidate the L2 at every poll.)
__device__ __forceinline__ void wait_count(const GemmArgs& g, const int32_t* counter, int n) {
  if (threadIdx.x < kWave) {
    if (threadIdx.x == 0) poll_at_least(g, counter, n);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Host: read and clear this code object's wait record.
static inline hipError_t take_wait_error(uint32_t* out) {
  hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_wait_error), sizeof(uint32_t), 0,
                                     hipMemcpyDeviceToHost);
  if (e != hipSuccess || *out == 0) return e;
  const uint32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_wait_error), &zero, sizeof(uint32_t), 0,
                           hipMemcpyHostToDevice);
}

// H or I is not a whole number of k slices (both are multiples of 8): the
// forward-shaped kinds then run the instantiation that zero-fills past the
// end of k.
inline bool ragged_k(int H, int I, int bk) { return (H % bk) != 0 || (I % bk) != 0; }

// Copy of half of a k slice's A operand from LDS to global rows (the fused
// dispatch+up writes the expert-contiguous rows x_perm this way): wave w
// takes tile rows [32 w, 32 w + 32), lane l chunk l % 8 (8 k) of rows
// l / 8 + 8 j, j = 2 half .. 2 half + 1.  Rows past m_valid and chunks past
// k_valid (zero-filled in LDS) are not stored.  Non-temporal stores: nothing
// in the launch reads x_perm back, so its lines should not take L2 space from
// the tiles' operands (the fused dispatch+up at the long-sequence size: 5.76
// -> 5.69 ms).
template <class C>
__device__ __forceinline__ void copy_a_half(const uint8_t* stage, uint16_t* dst, int64_t ld, int k0,
                                            int k_valid, int m_valid, int wave, int lane, int half) {
  constexpr int kCpr = C::BK / 8;
  static_assert(!C::A_MN && C::BM == 32 * C::NW && kCpr == 8, "one 32-row block per wave");
  const int c = lane % kCpr;
#pragma unroll
  for (int j = 2 * half; j < 2 * half + 2; ++j) {
    const int r = 32 * wave + lane / kCpr + 8 * j;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + kc_off<C::BK>(r, c));
    if (r < m_valid && c * 8 < k_valid)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + (int64_t)r * ld + k0 + c * 8));
  }
}

// The whole tile: a ring of LDS k slices filled by direct loads, MFMA over
// each slice with the next k step's fragments in flight, then the epilogue.
// kCopyA (the fused dispatch+up): the first column tile of a routed row tile
// also writes each A slice it has gathered from the token rows to x_perm.
// A split tile's helper part stores its partial sums and publishes them; the
// owner part (the last) waits for its helpers, adds their partials in part
// order (a fixed order, so the bits do not depend on timing) and runs the
// epilogue.
template <class C, bool kCoherentY = false, bool kRaggedK = false, bool kCopyA = false>
__device__ void run_tile_bf16(const GemmArgs& g, const TileDesc<uint16_t>& d,
                              uint8_t* const (&stages)[4], const TaskPart& tp) {
  constexpr int MI = C::MI, NJ = C::NJ;
  static_assert(C::STAGES >= 2 && C::STAGES <= 4, "2 to 4 LDS slices");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  int wm, wn;
  wave_block<C>(d, wave, wm, wn);

  // the weight gradient's k range (an expert's rows) is not a whole number
  // of slices; kRaggedK: neither is H or I (multiples of 8, not of the slice)
  constexpr bool kRagged = KindTraits<C::KIND>::kWgrad || kRaggedK;
  DmaOperand<C::BM, C::NW, C::A_MN, 1, kRagged, C::BK> da;
  DmaOperand<C::BN, C::NW, C::B_MN, C::B_NH, kRagged, C::BK> db;
  if constexpr (C::A_MN) da.init(d.a_sk, d.m_valid, wave, lane); else da.init(d.a_sm, d.m_valid, wave, lane, d.a_rows);
  if constexpr (C::B_MN) db.init(d.b_sk, d.n_valid, wave, lane); else db.init(d.b_sn, d.n_valid, wave, lane);

  constexpr int BK = C::BK;
  constexpr bool kSplit = KindTraits<C::KIND>::kSplit;
  const int parts = kSplit ? tp.parts : 1;
  const int part = kSplit ? tp.part : 0;
  // The input gradient's k runs over [da | db] against [W1 | W3]: two
  // segments of ksplit = I each, every segment a whole number of slices (the
  // last slice of a segment partial when I is not a multiple of BK).
  const bool two_seg = d.ksplit != INT_MAX;
  const int nk_seg = two_seg ? (d.ksplit + BK - 1) / BK : 0;
  const int nk_all = two_seg ? 2 * nk_seg : (d.k_len + BK - 1) / BK;
  const int kb = parts > 1 ? (int)((int64_t)nk_all * part / parts) : 0;   // this part's slices
  const int nk = parts > 1 ? (int)((int64_t)nk_all * (part + 1) / parts) - kb : nk_all;
  // kCopyA: gathered routed rows of the first column tile go to x_perm too
  const bool copy_a = kCopyA && d.a_rows != nullptr && d.col0 == 0;
  uint16_t* const xperm_rows = kCopyA ? static_cast<uint16_t*>(g.o_x_perm) + d.row0 * d.a_sm : nullptr;
  auto issue = [&](uint8_t* st, int kt) {   // kt: slice index within the part
    int ks = (kb + kt) * BK;                 // k of the slice within its segment
    int seg = 0;
    if (two_seg && kb + kt >= nk_seg) {
      seg = 1;
      ks -= nk_seg * BK;
    }
    const int k_valid = (two_seg ? d.ksplit : d.k_len) - ks;
    const bool live = kt < nk;   // kt < nk_pad always; zero-filled past nk
    if constexpr (C::A_MN)
      da.issue(st, d.a + (int64_t)ks * d.a_sk, nullptr, k_valid, live, wave);
    else
      da.issue(st, d.a + (seg ? d.ksplit : 0) + ks, nullptr, k_valid, live, wave);
    if constexpr (C::B_MN)
      db.issue(st + C::A_BYTES, d.b0 + (int64_t)ks * d.b_sk,
               C::PAIRED ? d.b1 + (int64_t)ks * d.b_sk : nullptr, k_valid, live, wave);
    else
      db.issue(st + C::A_BYTES, (seg ? d.b1 : d.b0) + ks, nullptr, k_valid, live, wave);
  };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  int a_row[MI], b_sub[NJ], b_col[NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i) a_row[i] = wm * C::WM + 32 * i;
#pragma unroll
  for (int j = 0; j < NJ; ++j) b_block<C>(wn, j, b_sub[j], b_col[j]);
  constexpr int kBSubBytes = C::B_BYTES / C::B_NH;
  constexpr int kBCols = C::BN / C::B_NH;

  // Ring of S slices: slice kt lives in stage kt % S; the loads of S-1
  // slices are in flight.  Fragments run one k step ahead of the MFMAs: step
  // ks's fragments are read while the MFMAs of the step before it are issued,
  // one MFMA, then a share of the reads and loads, and so on (scheduling
  // groups keep that order); the step before slice kt's first one is the
  // previous slice's last, whose fragments were read before the barrier that
  // opened slice kt.  So each slice starts, right after its barrier, with the
  // refill of the stage the previous slice freed, its first fragment reads
  // and MFMAs that need no wait; a barrier closes the slice once this wave's
  // loads of the next slice are in.  Nothing is in flight in LDS across the
  // loop edge.  The slice count is padded to a multiple of S with zero-filled
  // slices (they add exact zeros), so the loop has a single exit and the
  // accumulators stay in place across it.
  //
  // NA = the wave's 32-row blocks that hold valid rows (the last row tile of
  // an expert is partial): blocks past it issue neither fragment reads nor
  // MFMAs, which leaves the matrix pipe to the other wave of the SIMD.  The
  // wave still does its share of the copies and barriers.  Results of the
  // valid rows do not depend on NA.
  constexpr int S = C::STAGES;
  constexpr int KS = BK / 16;
  static_assert(KS % 2 == 0, "fragment buffers alternate by k step");
  constexpr int kLoads = decltype(da)::kPerWave + decltype(db)::kPerWave;
  const int nk_pad = (nk + S - 1) / S * S;
  auto wait_slices = [&](int pending) {   // at most `pending` later slices outstanding
    if (S >= 4 && pending >= 2) wait_vmcnt<(S >= 4 ? 2 : 0) * kLoads>();
    else if (S >= 3 && pending >= 1) wait_vmcnt<(S >= 3 ? 1 : 0) * kLoads>();
    else wait_vmcnt<0>();
  };
#pragma unroll
  for (int i = 0; i < S - 1; ++i) issue(stages[i], i);

  auto ring = [&](auto na_c) {
    constexpr int NA = decltype(na_c)::value;
    constexpr int kReads = NA == 0 ? 0 : NA * (C::A_MN ? 2 : 1) + NJ * (C::B_MN ? 2 : 1);
    // Reads in the order the MFMAs of a step (i outer, j inner) first need
    // them: B block 0, A block 0, the other B blocks, the other A blocks.
    auto frags = [&](const uint8_t* st, int ks, bf16x8 (&av)[MI], bf16x8 (&bv)[NJ]) {
      if constexpr (NA > 0) {
        const uint8_t* ta = st;
        const uint8_t* tb = st + C::A_BYTES;
        auto fa = [&](int i) {
          if constexpr (C::A_MN)
            av[i] = mn_frag(ta, C::BM, a_row[i], ks, lane);
          else
            av[i] = kc_frag<BK>(ta, a_row[i] + (lane & 31), 2 * ks + (lane >> 5));
        };
        auto fb = [&](int j) {
          if constexpr (C::B_MN)
            bv[j] = mn_frag(tb + b_sub[j] * kBSubBytes, kBCols, b_col[j], ks, lane);
          else
            bv[j] = kc_frag<BK>(tb, b_col[j] + (lane & 31), 2 * ks + (lane >> 5));
        };
        fb(0);
        fa(0);
#pragma unroll
        for (int j = 1; j < NJ; ++j) fb(j);
#pragma unroll
        for (int i = 1; i < NA; ++i) fa(i);
      }
    };
    auto mfma_step = [&](const bf16x8 (&av)[MI], const bf16x8 (&bv)[NJ]) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    };
    bf16x8 av[2][MI], bv[2][NJ];
    const bf16x8 zero = {};
#pragma unroll
    for (int i = 0; i < MI; ++i) av[1][i] = zero;   // "previous step" of slice 0: adds zeros
#pragma unroll
    for (int j = 0; j < NJ; ++j) bv[1][j] = zero;
    wait_slices(S - 2);
    lds_barrier();
    for (int kt0 = 0; kt0 < nk_pad; kt0 += S) {
#pragma unroll
      for (int i = 0; i < S; ++i) {
        const int kt = kt0 + i;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          frags(stages[i], ks, av[ks & 1], bv[ks & 1]);
          // slices past the end are zero-filled; the last wait of the loop
          // drains them before the epilogue reuses the stages
          if (ks == 0) issue(stages[(i + S - 1) % S], kt + S - 1);
          mfma_step(av[(ks + 1) & 1], bv[(ks + 1) & 1]);
          if (ks == 0)
            interleave_step<0, NA * NJ, kReads, kLoads>();
          else
            interleave_step<0, NA * NJ, kReads, 0>();
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kCopyA) {
            // the slice stays in its stage until the barrier that closes it
            if (copy_a && ks < 2 && kt < nk) {
              copy_a_half<C>(stages[i], xperm_rows, d.a_sm, (kb + kt) * BK, d.k_len - (kb + kt) * BK,
                             d.m_valid, wave, lane, ks);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        wait_slices(min(S - 2, nk_pad - 2 - kt));
        lds_barrier();
      }
    }
    mfma_step(av[1], bv[1]);   // last step of the last slice
  };
  const int col_first = C::PAIRED ? wn * (C::WN / 2) : wn * C::WN;
  const int na = col_first >= d.n_valid ? 0 : max(0, min(MI, (d.m_valid - wm * C::WM + 31) / 32));
  with_count<MI>(__builtin_amdgcn_readfirstlane(na), ring);
  __syncthreads();  // LDS free for the next tile of a persistent worker

  const int64_t tile_floats = (int64_t)C::BM * C::BN;
  float* part_out = nullptr;
  const float* part_in = nullptr;
  int n_in = 0;
  int32_t* cnt = nullptr;
  if (kSplit && parts > 1) {
    float* pbase = g.split_part + (int64_t)(tp.range * kSplitSlots + tp.slot * (parts - 1)) * tile_floats;
    cnt = g.split_cnt + tp.range * kSplitWr + tp.slot;
    if (part < parts - 1) {   // helper
      part_out = pbase + part * tile_floats;
    } else {                  // owner: wait for the helpers' partials
      wait_count(g, cnt, parts - 1);
      part_in = pbase;
      n_in = parts - 1;
    }
  }
  epilogue_bf16<C, kCoherentY>(g, d, acc, stages, wave, lane, part_out, part_in, n_in, tile_floats);
  if (kSplit && part_out) publish_add(cnt);
}

// ------------------------------------------------------------------ f32 ----

constexpr int kF32BM = 64, kF32BN = 64, kF32BK = 64, kF32NT = 256;

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
  // The next k step's operands are loaded into registers while the current
  // step computes, and stored to LDS after its trailing barrier; every output
  // still accumulates in ascending k.
  constexpr int kLa = kF32BM * kF32BK / kF32NT, kLb = kF32BN * kF32BK / kF32NT;
  float ra[kLa], rb[kLb];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kLa; ++i) {
      const int id = tid + i * kF32NT;
      const int m = id % kF32BM, k = id / kF32BM;
      const int kk = k0 + k;
      ra[i] = (m < d.m_valid && kk < d.k_len) ? d.a[(int64_t)m * d.a_sm + (int64_t)kk * d.a_sk] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kLb; ++i) {
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
      rb[i] = ok ? p[(int64_t)kk * d.b_sk + (int64_t)nl * d.b_sn] : 0.f;
    }
  };
  load(0);
  for (int k0 = 0; k0 < d.k_len; k0 += kF32BK) {
#pragma unroll
    for (int i = 0; i < kLa; ++i) {
      const int id = tid + i * kF32NT;
      sA[id / kF32BM][id % kF32BM] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < kLb; ++i) {
      const int id = tid + i * kF32NT;
      sB[id / kF32BN][id % kF32BN] = rb[i];
    }
    __syncthreads();
    if (k0 + kF32BK < d.k_len) load(k0 + kF32BK);
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

// Logical tile -> (row tile, column tile).  Row tiles are taken in bands (the
// forward and input-gradient kinds: over each group's row tiles, from the
// planner's band table; the weight-gradient kinds: over their fixed grid of
// (group, M tile), whose M tiles are H blocks for dW1/dW3 and I blocks for
// dW2, GemmArgs::wg_band high); inside a band the column tiles advance
// slowest, so the tiles an XCD runs at the same time form a band x
// (concurrent / band) block: each operand slice they load is shared by
// several of them through L2.  The heights are schedule knobs (Tuning).
__host__ __device__ inline int group_bands(int mt, int small, int big) {
  return mt <= 0 ? 0 : mt <= small ? 1 : (mt + big - 1) / big;
}
__device__ __forceinline__ void band_order(int L, int mt_count, int nt_count, int kB, int& tm, int& tn) {
  const int band_tiles = kB * nt_count;
  const int band = L / band_tiles;
  const int rem = L - band * band_tiles;
  const int rows = min(kB, mt_count - band * kB);
  tn = rem / rows;
  tm = band * kB + (rem - tn * rows);
}

// ------------------------------------------------------- tile scheduling ----
//
// Persistent workers (one per CU) take tiles from per-XCD ranges: the tiles,
// in band order, are split into kXcds contiguous ranges with a cursor each;
// worker b starts on range b % kXcds (workgroups are handed to the XCDs round
// robin, so that is its own XCD's range: tiles sharing operands share an L2)
// and then steals from the other ranges, which evens out the tail.  The
// claimed index is identical in every thread.

// The claimed index is broadcast with readfirstlane so the compiler sees it
// as uniform: every loop around a claim then has a uniform exit.  Otherwise
// the compiler may treat the exit as divergent and restructure the loop so
// that thread 0 (which publishes and claims) leaves it while the other lanes
// go round again on the old index -- a livelock across the barriers.
__device__ __forceinline__ int claim_task(int32_t* cursor, int* slot) {
  if (threadIdx.x == 0) *slot = atomicAdd(cursor, 1);
  __syncthreads();
  const int task = __builtin_amdgcn_readfirstlane(*slot);
  __syncthreads();
  return task;
}

// Tail split.  A range of n_r < 4 wr tiles worked by wr workers per XCD ends
// with rem = n_r mod wr tiles that would leave most of the XCD idle; they are
// split along k into P = min(kMaxSplit, wr / rem, slices) parts when P >= 2,
// so the range's last round has about as many tasks as workers.  A split
// tile's parts are consecutive in the range's task order, helpers first and
// the owner last, so when the owner is claimed every helper has been claimed
// by a running worker that never waits: the owner's wait always ends.
struct RangePlan {
  int lo, hi;        // tiles [lo, hi)
  int split_from;    // tiles [split_from, hi) are split
  int parts;
};
__device__ __forceinline__ RangePlan range_plan(int r, int n, int wr, int max_parts) {
  RangePlan p;
  p.lo = (int)((int64_t)n * r / kXcds);
  p.hi = (int)((int64_t)n * (r + 1) / kXcds);
  p.split_from = p.hi;
  p.parts = 1;
  if (wr > 0 && p.hi - p.lo < 4 * wr) {   // only ranges of few rounds
    const int rem = (p.hi - p.lo) % wr;
    const int P = split_parts(rem, wr, min(max_parts, kMaxSplit));
    if (P >= 2) {
      p.split_from = p.hi - rem;
      p.parts = P;
    }
  }
  return p;
}

// Debug perturbation of the schedule (GemmArgs::perturb, determinism tests).
__device__ __forceinline__ uint32_t perturb_hash(uint32_t x) {
  x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
  return x;
}
// Sleep 0..7 x 32 x 64 clocks, chosen by (seed, worker, claim count).
__device__ __forceinline__ void perturb_delay(uint32_t seed, uint32_t claims) {
  const uint32_t h = perturb_hash(seed ^ perturb_hash(blockIdx.x * 0x9E3779B1u + claims));
  for (uint32_t i = 0; i < (h & 7u); ++i) __builtin_amdgcn_s_sleep(32);
}
// Affine bijection t -> (a t + c) mod n of [0, n): a seeded multiplier made
// coprime to n.
__device__ __forceinline__ void perturb_affine(uint32_t seed, int r, int n, int& a, int& c) {
  a = 1; c = 0;
  if (n <= 1) return;
  const uint32_t h = perturb_hash(seed * 0x85EBCA77u + (uint32_t)r);
  c = (int)(h % (uint32_t)n);
  a = (int)(perturb_hash(h) % (uint32_t)n) | 1;
  for (;;) {   // smallest a' >= a with gcd(a', n) = 1 (a' = n + 1 at the latest)
    int x = a, y = n;
    while (y) { const int z = x % y; x = y; y = z; }
    if (x == 1) break;
    ++a;
  }
}

// Run every task of the ranges, own XCD's range first.  wr = 0: whole tiles
// only; otherwise tail tiles are split as above (max_parts: slices per tile).
// perturb (debug, nonzero): each range's whole tiles are claimed in a seeded
// order and every claim is preceded by a seeded sleep; split tails keep their
// order (helpers before owners), so every wait still ends.
template <class F>
__device__ __forceinline__ void for_tasks_xcd_ranges(int32_t* cursors, int n, int wr, int max_parts,
                                                     int* slot, F&& task, uint32_t perturb = 0) {
  const int home = blockIdx.x % kXcds;
  uint32_t claims = 0;
  for (int q = 0; q < kXcds; ++q) {
    const int r = (home + q) % kXcds;
    const RangePlan p = range_plan(r, n, wr, max_parts);
    const int whole = p.split_from - p.lo;
    const int total = whole + (p.hi - p.split_from) * p.parts;
    int pa = 1, pc = 0;
    if (perturb) perturb_affine(perturb, r, whole, pa, pc);
    for (;;) {
      if (perturb) perturb_delay(perturb, claims++);
      const int t = claim_task(&cursors[r], slot);
      if (t >= total) break;
      TaskPart tp;
      tp.range = r;
      if (t < whole) {
        tp.L = p.lo + (perturb ? (int)(((int64_t)t * pa + pc) % whole) : t);
        tp.part = 0;
        tp.parts = 1;
        tp.slot = 0;
      } else {
        const int u = t - whole;
        tp.slot = u / p.parts;
        tp.L = p.split_from + tp.slot;
        tp.part = u - tp.slot * p.parts;
        tp.parts = p.parts;
      }
      task(tp);
    }
  }
}

// Logical tile -> (row tile, column tile) over the planner's bands (a group's
// row tiles in runs): bands in order, inside a band the column tiles advance
// slowest.  Tiles running at the same time on an XCD then belong to one or two
// experts, so they share weight columns as well as token rows through L2.
// Band b covers logical tiles [first_b * nt, (first_b + rows_b) * nt), so row
// tile L / nt lies in the band holding L, and its band-table entry gives the
// band with one load (a search over the band starts would be a chain of
// dependent loads at the start of every tile).
__device__ __forceinline__ void band_order_groups(int L, int nt_count, const int2* bands, int& tm,
                                                  int& tn) {
  const int2 b = bands[L / nt_count];
  const int rem = L - b.x * nt_count;
  tn = rem / b.y;
  tm = b.x + (rem - tn * b.y);
}

// bf16 tile configurations per kind: BM, BN, waves along M, waves along N,
// LDS k slices.  The fused kernels use the same ones, so their tiles are
// computed exactly as by the plain launches.
#ifndef MOE_CFG_UP
#define MOE_CFG_UP 256, 256, 2, 4, 2
#endif
#ifndef MOE_CFG_DOWN
#define MOE_CFG_DOWN 256, 256, 2, 4, 2
#endif
#ifndef MOE_CFG_BWD_UP
#define MOE_CFG_BWD_UP 256, 256, 2, 4, 2
#endif
#ifndef MOE_CFG_BWD_DOWN
#define MOE_CFG_BWD_DOWN 256, 256, 2, 4, 2
#endif
#ifndef MOE_CFG_WG_UP
#define MOE_CFG_WG_UP 256, 256, 2, 4, 2
#endif
#ifndef MOE_CFG_WG_DOWN
#define MOE_CFG_WG_DOWN 256, 256, 2, 4, 2
#endif
template <int KIND> struct BfPick;
template <> struct BfPick<kUp> { using C = BfCfg<kUp, MOE_CFG_UP>; };
template <> struct BfPick<kDown> { using C = BfCfg<kDown, MOE_CFG_DOWN>; };
template <> struct BfPick<kBwdUp> { using C = BfCfg<kBwdUp, MOE_CFG_BWD_UP>; };
template <> struct BfPick<kBwdDown> { using C = BfCfg<kBwdDown, MOE_CFG_BWD_DOWN>; };
template <> struct BfPick<kWgUp> { using C = BfCfg<kWgUp, MOE_CFG_WG_UP>; };
template <> struct BfPick<kWgDown> { using C = BfCfg<kWgDown, MOE_CFG_WG_DOWN>; };
// the workspace holds k-split partial tiles of at most 256 x 256 f32
static_assert(BfPick<kUp>::C::BM * BfPick<kUp>::C::BN <= 256 * 256 &&
                  BfPick<kDown>::C::BM * BfPick<kDown>::C::BN <= 256 * 256 &&
                  BfPick<kBwdUp>::C::BM * BfPick<kBwdUp>::C::BN <= 256 * 256 &&
                  BfPick<kBwdDown>::C::BM * BfPick<kBwdDown>::C::BN <= 256 * 256,
              "partial tile size");


}  // namespace moe
