// ss_state_update.hip -- gfx950 single-token decode of the selective scan.
//
// One call advances the resident float32 state (batch, d_inner, d_state) by one token, in place:
//     dt = softplus(delta + bias),  h[n] <- exp(dt A[d,n]) h[n] + dt B[n] u,
//     y = C . h + D u,  out = y * silu(z).
// With ZOH the input term is the exact zero-order-hold one, (exp(dt A) - 1) / A * B u (reading
// guide, "Método"), in place of dt B u.
// (Mamba reading guide, "Perguntas": generation keeps only a fixed d_inner x d_state state per
// layer and costs O(1) per token; "Método" for the recurrence.)
//
// The step is bound by memory: every state element is read once and written once, with a
// handful of operations each.  Layout: each channel's d_state floats are split over a
// power-of-two group of lanes, 4 consecutive states per lane, so that a wave reads and writes one
// contiguous run of the state with 16-byte accesses.  Each thread handles several such 4-state
// items and issues all their loads before any arithmetic, to keep enough bytes in flight to cover
// the memory latency.  The group reduces C . h with cross-lane shuffles; its first lane finishes
// the element (skip, gate, store).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kDecodeThreads = 256;

template <class IO>
struct Vec4In;  // four consecutive io elements
template <>
struct Vec4In<F32> {
  using raw = float4;
  static __device__ __forceinline__ raw load(const float* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  static __device__ __forceinline__ float get(const raw& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
  }
};
template <>
struct Vec4In<BF16> {
  using raw = uint2;
  static __device__ __forceinline__ raw load(const uint16_t* p) {
    return *reinterpret_cast<const uint2*>(p);
  }
  static __device__ __forceinline__ float get(const raw& v, int i) {
    const uint32_t w = (i < 2) ? v.x : v.y;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

// Vector path: d_state % 4 == 0, 16-byte aligned state and A, ITEMS 4-state items per thread.
template <class IO, bool GATE, bool ZOH, int ITEMS>
__global__ void __launch_bounds__(kDecodeThreads) decode_vec4_kernel(DecodeArgs a) {
  using elem = typename IO::elem;
  using V = Vec4In<IO>;
  const int G = a.lanes_per_chan;
  const int N = a.d_state;
  const int64_t nch = a.batch * a.d_inner;
  const elem* up = static_cast<const elem*>(a.u);
  const elem* dp = static_cast<const elem*>(a.delta);
  const elem* zp = static_cast<const elem*>(a.z);
  const elem* Bp = static_cast<const elem*>(a.B);
  const elem* Cp = static_cast<const elem*>(a.C);

  int64_t ch[ITEMS];
  int q[ITEMS];
  bool act[ITEMS];
  float4 hv[ITEMS], av[ITEMS];
  typename V::raw bv[ITEMS], cv[ITEMS];
  elem xr[ITEMS], dr[ITEMS], zr[ITEMS];
  float bias[ITEMS], dsk[ITEMS];
  // issue every load first
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int64_t item = (static_cast<int64_t>(blockIdx.x) * ITEMS + i) * kDecodeThreads +
                         threadIdx.x;
    ch[i] = item / G;
    q[i] = static_cast<int>(item - ch[i] * G);
    act[i] = ch[i] < nch && q[i] * 4 < N;
    const int64_t c = ch[i] < nch ? ch[i] : nch - 1;  // clamped: always a valid address
    const int n0 = (q[i] * 4 < N) ? q[i] * 4 : 0;
    const int64_t b = c / a.d_inner, d = c - b * a.d_inner;
    hv[i] = *reinterpret_cast<const float4*>(a.state + c * N + n0);
    av[i] = *reinterpret_cast<const float4*>(a.A + d * N + n0);
    bv[i] = V::load(Bp + b * N + n0);
    cv[i] = V::load(Cp + b * N + n0);
    xr[i] = up[c];
    dr[i] = dp[c];
    if (GATE) zr[i] = zp[c];
    bias[i] = a.delta_bias ? a.delta_bias[d] : 0.0f;
    dsk[i] = a.D ? a.D[d] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const float x = IO::widen(xr[i]);
    const float s = IO::widen(dr[i]) + bias[i];
    const float dt = a.softplus ? softplus_f(s) : s;
    const float du = dt * x;
    float hh[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
    const float aa[4] = {av[i].x, av[i].y, av[i].z, av[i].w};
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float y = dt * (aa[j] * kLog2e);
      const float e = exp2_hw(y);
      const float inc = du * V::get(bv[i], j);
      hh[j] = fmaf(e, hh[j], ZOH ? inc * (zoh_gain(e, y) * (1.0f / kLn2)) : inc);
      p = fmaf(V::get(cv[i], j), hh[j], p);
    }
    if (act[i])
      *reinterpret_cast<float4*>(a.state + ch[i] * N + q[i] * 4) =
          make_float4(hh[0], hh[1], hh[2], hh[3]);
    p = act[i] ? p : 0.0f;
    for (int m = G >> 1; m >= 1; m >>= 1) p += __shfl_xor(p, m, G);
    if (ch[i] < nch && q[i] == 0) {
      float y = fmaf(dsk[i], x, p);
      if (GATE) y *= silu_f(IO::widen(zr[i]));
      static_cast<elem*>(a.out)[ch[i]] = IO::from_float(y);
    }
  }
}

// Generic path: any d_state in 1..64 and any alignment; one 4-state item per thread.
template <class IO, bool GATE, bool ZOH>
__global__ void __launch_bounds__(kDecodeThreads) decode_generic_kernel(DecodeArgs a) {
  using elem = typename IO::elem;
  const int G = a.lanes_per_chan;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kDecodeThreads + threadIdx.x;
  const int64_t ch = gid / G;  // (b, d) row
  const int q = static_cast<int>(gid - ch * G);
  const bool active = ch < a.batch * a.d_inner;
  const int64_t b = active ? ch / a.d_inner : 0;
  const int64_t d = active ? ch - b * a.d_inner : 0;
  const int N = a.d_state;
  const int n0 = q * 4;

  float x = 0.f, dt = 0.f, zv = 0.f, p = 0.f;
  if (active) {
    x = IO::load(static_cast<const elem*>(a.u), ch);
    const float s = IO::load(static_cast<const elem*>(a.delta), ch) +
                    (a.delta_bias ? a.delta_bias[d] : 0.0f);
    dt = a.softplus ? softplus_f(s) : s;
    if (GATE) zv = IO::load(static_cast<const elem*>(a.z), ch);
  }
  const float du = dt * x;
  const elem* Bp = static_cast<const elem*>(a.B);
  const elem* Cp = static_cast<const elem*>(a.C);
  if (active && n0 < N) {
    float* st = a.state + ch * N + n0;
    const float* Ar = a.A + d * N + n0;
    const int64_t bc = b * N + n0;
    for (int i = 0; i < 4 && n0 + i < N; ++i) {
      const float y = dt * (Ar[i] * kLog2e);
      const float e = exp2_hw(y);
      const float inc = du * IO::load(Bp, bc + i);
      const float hn = fmaf(e, st[i], ZOH ? inc * (zoh_gain(e, y) * (1.0f / kLn2)) : inc);
      st[i] = hn;
      p = fmaf(IO::load(Cp, bc + i), hn, p);
    }
  }
  for (int m = G >> 1; m >= 1; m >>= 1) p += __shfl_xor(p, m, G);
  if (active && q == 0) {
    float y = p + (a.D ? a.D[d] : 0.0f) * x;
    if (GATE) y *= silu_f(zv);
    static_cast<elem*>(a.out)[ch] = IO::from_float(y);
  }
}

constexpr int kItems = 4;

template <class IO, bool GATE, bool ZOH>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const int64_t lanes = a.batch * a.d_inner * a.lanes_per_chan;
  if (a.vec4) {
    const int64_t per_block = int64_t(kDecodeThreads) * kItems;
    const dim3 grid(static_cast<unsigned>((lanes + per_block - 1) / per_block));
    hipLaunchKernelGGL((decode_vec4_kernel<IO, GATE, ZOH, kItems>), grid, dim3(kDecodeThreads),
                       0, stream, a);
  } else {
    const dim3 grid(static_cast<unsigned>((lanes + kDecodeThreads - 1) / kDecodeThreads));
    hipLaunchKernelGGL((decode_generic_kernel<IO, GATE, ZOH>), grid, dim3(kDecodeThreads), 0,
                       stream, a);
  }
  return hipGetLastError();
}

template <bool ZOH>
hipError_t launch_z(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  if (bf16)
    return a.z ? launch_g<BF16, true, ZOH>(a, stream) : launch_g<BF16, false, ZOH>(a, stream);
  return a.z ? launch_g<F32, true, ZOH>(a, stream) : launch_g<F32, false, ZOH>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  return a.zoh ? launch_z<true>(a, bf16, stream) : launch_z<false>(a, bf16, stream);
}

}  // namespace ss
