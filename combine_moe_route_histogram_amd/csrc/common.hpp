// Device-side helpers shared by the HIP kernels of the MoE expert layer.
// gfx950 (CDNA4) only: wave64, bf16 MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 storage is the upper half of an IEEE float32.
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float32 -> bf16, round to nearest, ties to even (inputs are finite).
// f32 -> bf16, round to nearest even, with gfx950's conversion instruction
// (v_cvt_pk_bf16_f32: two values per instruction).  For finite inputs it
// gives the same bits as adding 0x7FFF plus the lowest kept bit and dropping
// the low half (checked over 2^24 values including ties and denormals).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const float __attribute__((ext_vector_type(2))) f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Elements of a storage type in one 16-byte vector.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;
  __device__ static __forceinline__ void unpack(const u32x4& v, float* f) {
    f[0] = __uint_as_float(v[0]); f[1] = __uint_as_float(v[1]);
    f[2] = __uint_as_float(v[2]); f[3] = __uint_as_float(v[3]);
  }
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    u32x4 v;
    v[0] = __float_as_uint(f[0]); v[1] = __float_as_uint(f[1]);
    v[2] = __float_as_uint(f[2]); v[3] = __float_as_uint(f[3]);
    return v;
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static __forceinline__ void store1(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <> struct Elem<uint16_t> {  // bf16
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ void unpack(const u32x4& v, float* f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = __uint_as_float(v[j] << 16);
      f[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
    }
  }
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(f[2 * j], f[2 * j + 1]);
    return v;
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ static __forceinline__ void store1(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16(v);
  }
};

// Lane k's value of v, for a wave-uniform k; unlike a shuffle it also reads
// lanes that are inactive at this point (e.g. lanes past the end of a row).
__device__ __forceinline__ int lane_int(int v, int k) { return __builtin_amdgcn_readlane(v, k); }
__device__ __forceinline__ float lane_float(float v, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}
// A token's K per-pair values (slot, gate weight, ...) spread over a wave:
// lane l holds pairs l, l + 64, ... (NC chunks of 64: K <= 64 NC), loaded
// while every lane is active.  at(k) reads pair k's value for a wave-uniform
// k from whichever lane holds it.  The chunk is chosen AFTER the lane read,
// among uniform values: at() is called inside loops where only some lanes
// are active, and a per-lane select done there would leave the inactive
// lanes' copies unwritten -- the very lanes a read of pair k may address.
template <typename V, int NC>
struct PairVals {
  V v[NC];
  __device__ __forceinline__ void load(const V* p, int K, int lane, V fill) {
#pragma unroll
    for (int c = 0; c < NC; ++c) v[c] = lane + kWave * c < K ? p[lane + kWave * c] : fill;
  }
  __device__ __forceinline__ static V read(V x, int l) {
    if constexpr (__is_same(V, float)) return lane_float(x, l);
    else return lane_int(x, l);
  }
  __device__ __forceinline__ V at(int k) const {
    const int l = k & (kWave - 1);
    V x = read(v[0], l);
#pragma unroll
    for (int c = 1; c < NC; ++c)
      if (k >= kWave * c) x = read(v[c], l);
    return x;
  }
};
// Chunks of 64 pairs needed for K pairs per token (the kernels are
// instantiated for 1 and 4, i.e. K <= 64 and K <= 256).
inline int pair_chunks(int K) { return K <= kWave ? 1 : 4; }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *static_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *static_cast<u32x4*>(p) = v; }

// Deterministic wave-wide sum: fixed butterfly order, every lane gets the result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + expf(-a)); }
__device__ __forceinline__ float sigmoid_f(float a) { return 1.0f / (1.0f + expf(-a)); }

}  // namespace moe
