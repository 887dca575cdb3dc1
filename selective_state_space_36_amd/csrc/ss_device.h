// ss_device.h -- device-side helpers shared by the gfx950 prefill and decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element access for the two io dtypes.  bf16 is carried as raw 16-bit patterns: widening is a
// 16-bit shift (exact); narrowing uses the hardware round-to-nearest-even conversion.
struct F32 {
  using elem = float;
  static __device__ __forceinline__ float load(const elem* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ float widen(elem e) { return e; }
  static __device__ __forceinline__ elem from_float(float f) { return f; }
};
struct BF16 {
  using elem = uint16_t;
  static __device__ __forceinline__ float load(const elem* p, int64_t i) { return widen(p[i]); }
  static __device__ __forceinline__ float widen(elem e) {
    return __uint_as_float(static_cast<uint32_t>(e) << 16);
  }
  static __device__ __forceinline__ elem from_float(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  }
};

// 2^x and log2(x) on the hardware transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(s) = max(s, 0) + log1p(e^{-|s|}).  log1p(e) for e in (0, 1] is evaluated as
// log(w) + (e - (w - 1)) with w = fl(1 + e): the second term restores the part of e lost when
// forming w, so the result keeps full relative precision when e is tiny (small step sizes).
__device__ __forceinline__ float softplus_f(float s) {
  const float e = exp2_hw(-fabsf(s) * kLog2e);
  const float w = 1.0f + e;
  const float l = log2_hw(w) * kLn2;
  const float c = e - (w - 1.0f);
  // max(s, 0) as a median (no NaN canonicalisation, one instruction)
  return __builtin_amdgcn_fmed3f(s, 0.0f, __builtin_inff()) + (l + c);
}

// (2^y - 1) / y, given u = 2^y; it tends to ln 2 at y = 0.  This is the exact zero-order-hold
// input gain in base 2: (exp(x) - 1) / x = (2^y - 1) / (y ln 2) for x = y ln 2.  For |y| < 1/2
// it is the Taylor series sum_k ln2^(k+1) y^k / (k+1)! cut after y^7 (the rest is below
// 1e-9 relative there), which avoids the cancellation in 2^y - 1; elsewhere (u - 1) / y, where
// |u - 1| >= 0.29 keeps that difference accurate.  u == 0 (large negative y) gives -1 / y.
__device__ __forceinline__ float zoh_gain(float u, float y) {
  float p = 1.3215486660556053e-06f;
  p = fmaf(p, y, 1.5252733646775596e-05f);
  p = fmaf(p, y, 0.0001540352968731895f);
  p = fmaf(p, y, 0.0013333557872101665f);
  p = fmaf(p, y, 0.009618128649890423f);
  p = fmaf(p, y, 0.05550410971045494f);
  p = fmaf(p, y, 0.24022650718688965f);
  p = fmaf(p, y, 0.6931471824645996f);
  return fabsf(y) < 0.5f ? p : (u - 1.0f) * rcp_hw(y);
}

// Exact-hold input gain (exp(dt A) - 1) / A for one update of the prefill, from e = 2^y with
// y = dt A log2(e) and ia = 1 / A (0 where A = 0).  For |y| < 1/8 it is dt R(y),
// R(y) = (2^y - 1) / (y ln 2) = sum_k (y ln 2)^k / (k + 1)! cut after k = 4 (the rest is below
// 7e-9 relative there): no cancellation in 2^y - 1 and no division.  Elsewhere it is (e - 1) / A
// as one fused multiply-add; there |e - 1| >= 0.083, so the 1-ulp error of e is at most 1.5e-6
// of the difference.  e = 0 (large negative y) gives -1 / A; A = 0 gives dt.
__device__ __forceinline__ float hold_gain(float e, float y, float dt, float ia) {
  float q = 1.9236258e-3f;
  q = fmaf(q, y, 1.3876027e-2f);
  q = fmaf(q, y, 8.0075502e-2f);
  q = fmaf(q, y, 3.4657359e-1f);
  q = fmaf(q, y, 1.0f);
  return fabsf(y) < 0.125f ? dt * q : fmaf(e, ia, -ia);
}

// Derivative of that gain g = (exp(dt A) - 1) / A in A, (dt e - g) / A, with the same inputs.
// For |y| < 1/8 it is dt^2 S(x), x = dt A = y ln 2, S(x) = sum_k (k + 1) x^k / (k + 2)! =
// 1/2 + x/3 + x^2/8 + x^3/30 + x^4/144 (the rest is below 1e-8 relative there): the difference
// dt e - g cancels as x -> 0 and tends to dt^2 / 2.  Elsewhere (dt e - (e - 1) / A) / A, where
// the difference keeps all but about 5 bits.
__device__ __forceinline__ float hold_gain_da(float e, float y, float dt, float ia) {
  const float x = y * kLn2;
  float q = 1.0f / 144.0f;
  q = fmaf(q, x, 1.0f / 30.0f);
  q = fmaf(q, x, 0.125f);
  q = fmaf(q, x, 1.0f / 3.0f);
  q = fmaf(q, x, 0.5f);
  return fabsf(y) < 0.125f ? (dt * dt) * q : fmaf(dt, e, -fmaf(e, ia, -ia)) * ia;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^{-z}).
__device__ __forceinline__ float silu_f(float z) {
  return z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// Value of `x` held by lane SRC of this lane's 16-lane row (DPP row_newbcast).  When the result
// feeds a multiply the compiler folds the broadcast into the multiply itself.  Every lane has
// its source, so bound_ctrl never applies; set, it spares the move that would clear the
// destination of a broadcast kept as a move (one feeding a fused multiply-add).
template <int SRC>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(SRC >= 0 && SRC < 16, "row lane");
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + SRC, 0xf, 0xf, true));
}

// Raw buffer resource over `bytes` bytes at `base` (stride 0).  The hardware range check makes
// loads at byte offsets >= bytes return 0 and drops stores there; offsets are per-lane bytes.
// `base` must be uniform over the wavefront (the resource lives in scalar registers).
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kOffNone = 0x80000000u;  // an offset past every range used here
__device__ __forceinline__ rsrc_t make_buf(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
template <class T>
__device__ __forceinline__ T buf_load(rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ uint4 buf_load<uint4>(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <>
__device__ __forceinline__ uint2 buf_load<uint2>(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
template <>
__device__ __forceinline__ float4 buf_load<float4>(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <>
__device__ __forceinline__ uint16_t buf_load<uint16_t>(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
template <>
__device__ __forceinline__ float buf_load<float>(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store(uint4 v, rsrc_t r, uint32_t off) {
  using v4u = __attribute__((ext_vector_type(4))) unsigned int;
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store(float4 v, rsrc_t r, uint32_t off) {
  buf_store(__builtin_bit_cast(uint4, v), r, off);
}
__device__ __forceinline__ void buf_store(uint16_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store(float v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// Value of `x` held by lane (k - S) mod 16 of this lane's 16-lane row, k being this lane's
// index in the row (DPP row_ror:S).  Every lane has a source in its row, so bound_ctrl never
// applies; set, it tells the compiler that no lane keeps the old value (no move to clear it).
template <int S>
__device__ __forceinline__ float row_ror(float x) {
  static_assert(S >= 1 && S < 16, "rotation");
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + S, 0xf, 0xf, true));
}

// Make this wavefront's LDS writes visible to all of its lanes (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait until this wave's outstanding LDS reads have returned.  A workgroup barrier orders LDS
// writes but does not wait for reads still in flight, so a read whose value is consumed only
// after a barrier, of memory that other waves overwrite after it, needs this before the barrier.
__device__ __forceinline__ void lds_reads_done() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
}

// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).  Remap the hardware
// workgroup index so that each XCD receives one contiguous range of logical indices: logical
// neighbours (which share cache lines of the inputs) then meet in the same L2.  A bijection on
// [0, n) for any n.
__device__ __forceinline__ int64_t xcd_remap(int64_t hw, int64_t n) {
  const int64_t q = n >> 3, rem = n & 7;
  const int64_t x = hw & 7, j = hw >> 3;
  return x < rem ? x * (q + 1) + j : rem * (q + 1) + (x - rem) * q + j;
}

}  // namespace ss
