// Device helpers shared by the paged-KV kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---- debug builds: bounds checks of device-resident indices ----------------------------------
// Built with PKV_DEBUG_CHECKS, the kernels check every index they take from device memory (slots,
// block ids, copy pairs, ragged row offsets) before using it. A bad index is skipped or replaced
// by a safe one, and the kernel stores 1 into the matching error word of its translation unit
// (plain stores: concurrent writers store the same value). Release builds compile the checks out.
enum : int { DBG_SLOT = 0, DBG_BLOCK = 1, DBG_RAGGED = 2, DBG_PAIR = 3, DBG_WORDS = 4 };
#ifdef PKV_DEBUG_CHECKS
constexpr bool kDebugChecks = true;
#else
constexpr bool kDebugChecks = false;
#endif

// Defines the translation unit's error words, debug_flag(word), and the host accessor
// debug_words_<unit> (declared in internal.hpp).
#ifdef PKV_DEBUG_CHECKS
#define PKV_DEBUG_UNIT(unit)                                                                        \
  static __device__ uint32_t g_debug_words[DBG_WORDS];                                              \
  static __device__ __forceinline__ void debug_flag(int w) { g_debug_words[w] = 1u; }               \
  int debug_words_##unit(uint32_t* out, bool clear) {                                               \
    if (hipDeviceSynchronize() != hipSuccess) return -1;                                            \
    if (hipMemcpyFromSymbol(out, HIP_SYMBOL(g_debug_words), sizeof(uint32_t) * DBG_WORDS, 0,        \
                            hipMemcpyDeviceToHost) != hipSuccess)                                   \
      return -1;                                                                                    \
    if (clear) {                                                                                    \
      const uint32_t zero[DBG_WORDS] = {0, 0, 0, 0};                                                \
      if (hipMemcpyToSymbol(HIP_SYMBOL(g_debug_words), zero, sizeof(zero), 0,                       \
                            hipMemcpyHostToDevice) != hipSuccess)                                   \
        return -1;                                                                                  \
    }                                                                                               \
    return 0;                                                                                       \
  }
#else
#define PKV_DEBUG_UNIT(unit)                                                                        \
  static __device__ __forceinline__ void debug_flag(int) {}                                         \
  int debug_words_##unit(uint32_t* out, bool) {                                                     \
    for (int i = 0; i < DBG_WORDS; ++i) out[i] = 0;                                                 \
    return 0;                                                                                       \
  }
#endif

// Storage type of each element type (bf16 is kept as raw 16-bit patterns).
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { using T = float; };
template <> struct Elem<DT_F16> { using T = _Float16; };
template <> struct Elem<DT_BF16> { using T = uint16_t; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two packed 16-bit elements of one 32-bit word -> two floats.
template <int DT> __device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi);
template <> __device__ __forceinline__ void unpack2<DT_BF16>(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xffff0000u);
}
template <> __device__ __forceinline__ void unpack2<DT_F16>(uint32_t w, float& lo, float& hi) {
  f16x2 h = __builtin_bit_cast(f16x2, w);
  lo = (float)h[0];
  hi = (float)h[1];
}

// acc + a·b over the two packed elements of each 32-bit word (products exact in fp32).
template <int DT> __device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float acc);
template <> __device__ __forceinline__ float dot2_acc<DT_BF16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}
template <> __device__ __forceinline__ float dot2_acc<DT_F16>(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
}

// Dot product of two 16-byte chunks (8 x 16-bit or 4 x fp32 elements).
template <int DT> __device__ __forceinline__ float dot16B(const u32x4& a, const u32x4& b, float acc) {
  if constexpr (DT == DT_F32) {
    acc = __builtin_fmaf(__uint_as_float(a[0]), __uint_as_float(b[0]), acc);
    acc = __builtin_fmaf(__uint_as_float(a[1]), __uint_as_float(b[1]), acc);
    acc = __builtin_fmaf(__uint_as_float(a[2]), __uint_as_float(b[2]), acc);
    acc = __builtin_fmaf(__uint_as_float(a[3]), __uint_as_float(b[3]), acc);
  } else {
    acc = dot2_acc<DT>(a[0], b[0], acc);
    acc = dot2_acc<DT>(a[1], b[1], acc);
    acc = dot2_acc<DT>(a[2], b[2], acc);
    acc = dot2_acc<DT>(a[3], b[3], acc);
  }
  return acc;
}

// ---- cross-lane reductions -------------------------------------------------------------------
// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the total.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  return x;
}

// Over lanes l, l^16, l^32, l^48 (the wave's four 16-lane rows), in VALU: a row swap of a value
// with itself leaves the two partners' values in the two results (gfx950 permlane swaps).
__device__ __forceinline__ float max_rows4(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float sum_rows4(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Whole-wave max / sum, every lane gets the result: DPP within each 16-lane row (pairs, quads,
// half-row mirror, row mirror), then the row swaps above. No LDS traffic.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  return max_rows4(x);
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return sum_rows4(x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Store one fp32 value as the output element type.
__device__ __forceinline__ void store_out(void* base, size_t idx, float v, int out_dt) {
  if (out_dt == DT_F32) {
    reinterpret_cast<float*>(base)[idx] = v;
  } else if (out_dt == DT_F16) {
    reinterpret_cast<_Float16*>(base)[idx] = (_Float16)v;
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
  }
}

// Store four consecutive fp32 values (idx a multiple of 4) as the output element type.
__device__ __forceinline__ void store_out4(void* base, size_t idx, float __attribute__((ext_vector_type(4))) v,
                                           int out_dt) {
  if (out_dt == DT_F32) {
    *reinterpret_cast<float __attribute__((ext_vector_type(4)))*>(reinterpret_cast<float*>(base) + idx) = v;
  } else if (out_dt == DT_F16) {
    const uint32_t lo = __builtin_bit_cast(uint32_t, f16x2{(_Float16)v[0], (_Float16)v[1]});
    const uint32_t hi = __builtin_bit_cast(uint32_t, f16x2{(_Float16)v[2], (_Float16)v[3]});
    *reinterpret_cast<u32x2*>(reinterpret_cast<_Float16*>(base) + idx) = u32x2{lo, hi};
  } else {
    const uint32_t lo = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    const uint32_t hi = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + idx) = u32x2{lo, hi};
  }
}

}  // namespace pkv
