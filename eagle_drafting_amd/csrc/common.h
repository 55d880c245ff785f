// Device helpers shared by the gfx950 kernels of the P-EAGLE draft / verify path.
#pragma once
#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

#define PE_WAVE 64

// device flag bits (mirrors pe_device_flags)
#define PE_FLAG_TOKEN 1
#define PE_FLAG_SLOT 2
#define PE_FLAG_POS 4

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
typedef __bf16 hw_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float hw_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// two values in one instruction: a in the low half, b in the high half
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((hw_f32x2_t){a, b}, hw_bf16x2_t));
}

// eight E4M3 codes (one 8-byte fragment lane) as the bf16 MFMA operand; every E4M3 value is exact in bf16
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint2 w) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, true);
  const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false), d = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, true);
  const u32x4_t pk = {f32x2_to_bf16x2(a[0], a[1]), f32x2_to_bf16x2(b[0], b[1]), f32x2_to_bf16x2(c[0], c[1]),
                      f32x2_to_bf16x2(d[0], d[1])};
  return __builtin_bit_cast(bf16x8_t, pk);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ void raise_flag(int* flags, int bit) {
  __hip_atomic_fetch_or(flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// (value, index) pair ordering of the argmax: larger value wins, equal values go to the lower index
__device__ __forceinline__ bool am_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Reductions over aligned groups of W lanes (W = 2 .. 64) with register-to-register lane moves instead of
// LDS permutes (whose latency a chain of them pays in full): DPP quad permutations (lane ^ 1, lane ^ 2), the
// half-row and row mirrors (lane i of each 8 / 16 lanes meets lane 7 - i / 15 - i), v_permlane16_swap
// between the 16-lane rows of a 32-lane half and v_permlane32_swap between the halves. Every step combines
// a lane with a partner that holds the partner group's result, so each lane of the group ends with the
// same value. The (value, index) maximum uses a total order (larger value, then lower index), so its
// result does not depend on the pairing.
// f(std::integral_constant<int, T>()) for T = B .. E - 1 (compile-time lane and control indices)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}
template <int CTRL>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int W, typename Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
  static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "group of 2 .. 64 lanes");
  v = op(v, __int_as_float(dpp_move<0xB1>(__float_as_int(v))));                  // quad_perm [1, 0, 3, 2]
  if (W >= 4) v = op(v, __int_as_float(dpp_move<0x4E>(__float_as_int(v))));      // quad_perm [2, 3, 0, 1]
  if (W >= 8) v = op(v, __int_as_float(dpp_move<0x141>(__float_as_int(v))));     // row_half_mirror
  if (W >= 16) v = op(v, __int_as_float(dpp_move<0x140>(__float_as_int(v))));    // row_mirror
  if (W >= 32) {
    // both results of a swap: the even row's and the odd row's value, in that order in both lanes
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  if (W >= 64) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  return v;
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  return group_reduce<W>(v, [](float x, float y) { return x + y; });
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
  return group_reduce<W>(v, [](float x, float y) { return fmaxf(x, y); });
}
template <int W>
__device__ __forceinline__ void am_group_reduce(float& v, int& i) {
  static_assert(W >= 32 && (W == 32 || W == 64), "half-wave or wave groups");
  auto step = [&](float ov, int oi) {
    if (am_better(ov, oi, v, i)) { v = ov; i = oi; }
  };
  step(__int_as_float(dpp_move<0xB1>(__float_as_int(v))), dpp_move<0xB1>(i));
  step(__int_as_float(dpp_move<0x4E>(__float_as_int(v))), dpp_move<0x4E>(i));
  step(__int_as_float(dpp_move<0x141>(__float_as_int(v))), dpp_move<0x141>(i));
  step(__int_as_float(dpp_move<0x140>(__float_as_int(v))), dpp_move<0x140>(i));
  {  // value and index of the same lane in the same result slot
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const auto b = __builtin_amdgcn_permlane16_swap((uint32_t)i, (uint32_t)i, false, false);
    v = __uint_as_float(a[0]);
    i = (int)b[0];
    step(__uint_as_float(a[1]), (int)b[1]);
  }
  if (W == 64) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const auto b = __builtin_amdgcn_permlane32_swap((uint32_t)i, (uint32_t)i, false, false);
    v = __uint_as_float(a[0]);
    i = (int)b[0];
    step(__uint_as_float(a[1]), (int)b[1]);
  }
}

// Reductions across the four 16-lane rows of a wave without LDS traffic: v_permlane16_swap exchanges
// rows 0<->1 and 2<->3, v_permlane32_swap the two wave halves; both operands are v, so the two results are
// the values of lane l and of its partner, in lane-independent order.
__device__ __forceinline__ float rows_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// sum over a block of NT threads (NT multiple of 64, <= 1024); every thread gets the total.
// Fixed reduction order, so results are bit-reproducible.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / PE_WAVE, l = threadIdx.x % PE_WAVE;
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < NT / PE_WAVE; ++k) t += red[k];
  __syncthreads();
  return t;
}
