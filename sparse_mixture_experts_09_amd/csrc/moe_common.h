// Internal helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Storage-type tags. A 16-byte vector holds kVec elements.
struct BF16 {
  typedef uint16_t elem;
  static constexpr int kVec = 8;
};
struct F32 {
  typedef float elem;
  static constexpr int kVec = 4;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even: the hardware's packed conversion (one
// instruction for two values); lo in the low half of the result.
typedef __bf16 bf16x2_vec __attribute__((ext_vector_type(2)));
typedef float f32x2_vec __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_vec v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_vec));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

// Unpack a 16-byte vector into kVec floats.
__device__ __forceinline__ void unpack16(BF16, const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(v[i]);
    f[2 * i + 1] = bf16_hi(v[i]);
  }
}
__device__ __forceinline__ void unpack16(F32, const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}
// Pack kVec floats (rounded to the storage type) into a 16-byte vector.
__device__ __forceinline__ u32x4 pack16(BF16, const float* f) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}
__device__ __forceinline__ u32x4 pack16(F32, const float* f) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
  return v;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Raw buffer access: the record count ends the buffer, and a load past it
// returns zeros without touching memory. The base and the count must be
// wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// AUX: the cache policy bits (2: nontemporal, for data read once)
template <int AUX = 0>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, AUX));
}

// A store at or past the record count is dropped.
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t voff, const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Sum of V values over the 64 lanes of a wave, spread so that lane L ends up
// holding the total of value index (L >> (6 - log2 V)) in v[0] (V <= 64, a
// power of two). Each exchange step halves the values a lane keeps, so the
// whole reduction costs V - 1 + (6 - log2 V) shuffles instead of 6 V.
template <int V>
__device__ __forceinline__ void wave_transpose_sum(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V must be a power of two <= 64");
  int n = V;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    if (n > 1) {
      const bool upper = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < V / 2; ++i) {
        if (i < n / 2) {
          const float a = v[i], b = v[i + n / 2];
          const float send = upper ? a : b;
          const float keep = upper ? b : a;
          v[i] = keep + __shfl_xor(send, o);
        }
      }
      n >>= 1;
    } else {
      v[0] += __shfl_xor(v[0], o);
    }
  }
}

template <int V>
struct Log2 {
  static constexpr int value = 1 + Log2<V / 2>::value;
};
template <>
struct Log2<1> {
  static constexpr int value = 0;
};

}  // namespace moe
