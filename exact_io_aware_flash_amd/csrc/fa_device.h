// fa_device.h -- device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA conventions used throughout (32x32 tiles, one wave = 64 lanes, lane = 32*h + n):
//   A operand (M x K):  lane n + 32*h holds row n and the K-slice owned by half h;
//   B operand (K x N):  lane n + 32*h holds column n and the same K-slice of half h;
//   result (M x N):     lane n + 32*h, register g holds row 8*(g/4) + 4*h + (g%4), column n.
// For bf16/f16 (v_mfma_f32_32x32x16_*) the K-slice is 8 elements (half h: k = 8h..8h+7);
// for f32 (v_mfma_f32_32x32x2_f32) it is one element (k = h). A and B always share the
// K-slice mapping, so any consistent relabelling of K on both operands gives the same
// product; the kernels use this to feed probabilities straight from the result registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Element-type traits: 16-bit types go through the 32x32x16 MFMA, float through 32x32x2.
template <typename T> struct Elt;

template <> struct Elt<__bf16> {
  static constexpr int kBytes = 2;
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two floats -> two bf16 (round to nearest even) packed low|high
  __device__ static inline uint32_t pack2(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
};

template <> struct Elt<_Float16> {
  static constexpr int kBytes = 2;
  __device__ static inline f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
};

template <> struct Elt<float> {
  static constexpr int kBytes = 4;
  __device__ static inline f32x16 mma1(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Result-register helpers for the 32x32 layout.
__device__ constexpr int res_row(int g, int h) { return 8 * (g / 4) + 4 * h + (g % 4); }

// Cross-half exchange: value held by lane l ^ 32 (the other half of the same column).
__device__ inline float xhalf(float v) { return __shfl_xor(v, 32, 64); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// 16-byte global load/store through plain vector accesses.
__device__ inline u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void stg8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// LDS accessors (byte offsets into a __shared__ char array).
__device__ inline u32x4 lds_ld16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ inline void lds_st16(char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}
__device__ inline void lds_st8(char* base, int off, u32x2 v) {
  *reinterpret_cast<u32x2*>(base + off) = v;
}
__device__ inline void lds_st4(char* base, int off, uint32_t v) {
  *reinterpret_cast<uint32_t*>(base + off) = v;
}

// Byte permute: result byte k = byte sel_k of the 8-byte value {hi:lo}.
__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low 16-bit halves of two words, packed (a.lo | b.lo << 16); high halves likewise.
__device__ inline uint32_t pack_lo(uint32_t a, uint32_t b) { return perm(b, a, 0x05040100u); }
__device__ inline uint32_t pack_hi(uint32_t a, uint32_t b) { return perm(b, a, 0x07060302u); }

}  // namespace fa
