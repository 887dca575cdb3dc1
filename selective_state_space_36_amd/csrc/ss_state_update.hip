// ss_state_update.hip -- gfx950 single-token decode of the selective scan.
//
// One call advances the resident float32 state (batch, d_inner, d_state) by one token, in place:
//     dt = softplus(delta + bias),  h[n] <- exp(dt A[d,n]) h[n] + dt B[n] u,
//     y = C . h + D u,  out = y * silu(z).
// (Mamba reading guide, "Perguntas": generation keeps only a fixed d_inner x d_state state per
// layer and costs O(1) per token; "Método" for the recurrence.)
//
// The step is bound by HBM: every state element is read once and written once, and the arithmetic
// per element is a handful of operations.  Layout: each channel's d_state floats are split over
// a power-of-two group of lanes, 4 consecutive states per lane, so that one wave reads and writes
// one contiguous run of the state with 16-byte accesses.  The group reduces C . h with
// cross-lane shuffles; its first lane finishes the element (skip, gate, store).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kDecodeThreads = 256;

template <class IO, bool GATE, bool VEC4>
__global__ void __launch_bounds__(kDecodeThreads) decode_kernel(DecodeArgs a) {
  using elem = typename IO::elem;
  const int G = a.lanes_per_chan;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kDecodeThreads + threadIdx.x;
  const int64_t ch = gid / G;              // (b, d) row
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
    if (VEC4) {
      float4 hv = *reinterpret_cast<const float4*>(st);
      const float4 av = *reinterpret_cast<const float4*>(Ar);
      float hh[4] = {hv.x, hv.y, hv.z, hv.w};
      const float aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = exp2_hw(dt * (aa[i] * kLog2e));
        hh[i] = fmaf(e, hh[i], du * IO::load(Bp, bc + i));
        p = fmaf(IO::load(Cp, bc + i), hh[i], p);
      }
      *reinterpret_cast<float4*>(st) = make_float4(hh[0], hh[1], hh[2], hh[3]);
    } else {
      for (int i = 0; i < 4 && n0 + i < N; ++i) {
        const float e = exp2_hw(dt * (Ar[i] * kLog2e));
        const float hn = fmaf(e, st[i], du * IO::load(Bp, bc + i));
        st[i] = hn;
        p = fmaf(IO::load(Cp, bc + i), hn, p);
      }
    }
  }
  // reduce the partial dot products over the channel's lane group (G is a power of two <= 16)
  for (int m = G >> 1; m >= 1; m >>= 1) p += __shfl_xor(p, m, G);
  if (active && q == 0) {
    float y = p + (a.D ? a.D[d] : 0.0f) * x;
    if (GATE) y *= silu_f(zv);
    static_cast<elem*>(a.out)[ch] = IO::from_float(y);
  }
}

template <class IO, bool GATE>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const int64_t lanes = a.batch * a.d_inner * a.lanes_per_chan;
  const dim3 grid(static_cast<unsigned>((lanes + kDecodeThreads - 1) / kDecodeThreads));
  if (a.vec4)
    hipLaunchKernelGGL((decode_kernel<IO, GATE, true>), grid, dim3(kDecodeThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<IO, GATE, false>), grid, dim3(kDecodeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream) {
  if (bf16) return a.z ? launch_g<BF16, true>(a, stream) : launch_g<BF16, false>(a, stream);
  return a.z ? launch_g<F32, true>(a, stream) : launch_g<F32, false>(a, stream);
}

}  // namespace ss
