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
// contiguous run of the state with 16-byte accesses.  Each thread handles its 4-state slice in
// several batch rows and issues all their loads before any arithmetic, to keep enough bytes in
// flight to cover the memory latency.  The group reduces C . h with cross-lane DPP adds; its first lane finishes
// the element (skip, gate, store).  Address arithmetic is kept to a few 32-bit operations per
// item: with this little work per byte, index math alone would otherwise bound the kernel.
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
  static __device__ __forceinline__ float get(const raw& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
  }
};
template <>
struct Vec4In<BF16> {
  using raw = uint2;
  static __device__ __forceinline__ float get(const raw& v, int i) {
    const uint32_t w = (i < 2) ? v.x : v.y;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

// Value of x held by lane J of this lane's quad (DPP quad_perm broadcast).  Quad permutations
// always have a source lane, so bound_ctrl never applies; set, it tells the compiler that no lane
// keeps the old value (no move to clear it).
template <int J>
__device__ __forceinline__ float quad_bcast(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), J * 0x55, 0xf, 0xf, true));
}

// Sum of x over aligned groups of G lanes (G a power of two <= 64), the result in every lane of
// the group.  Groups of up to 4 use DPP quad permutations (no LDS traffic).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if (G >= 2)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, true));
  if (G >= 4)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, true));
  for (int m = 4; m < G; m <<= 1) x += __shfl_xor(x, m, G);
  return x;
}

// Vector path: d_state % 4 == 0, 16-byte aligned state and A, and a group of BI batch rows of
// the state under 2^31 bytes.  Grid: x over the lanes of one batch row (G lanes per channel, 4
// consecutive states per lane), y over groups of BI batch rows (strided when there are more
// groups than the grid holds).  A thread keeps one (channel, 4-state slice) and walks the BI rows
// of its group: the channel's A, bias and D are loaded once for all of them (A's 16 bytes per
// lane were as much L2 traffic as the state itself), and the BI rows' state loads are all issued
// before the thread needs any row's u, delta or z.  When those inputs sit on pages the GPU has
// not translated yet (a decode loop reading each step's inputs from fresh memory), the first
// vector access to such a page stalls the CU's memory pipeline for a page-table walk; with
// several rows per thread more of the state stream is already in flight when it does.
// Arrays are raw buffers based at the group's first row with 32-bit lane offsets; lanes past the
// row and rows past the batch get offsets beyond every range, so their loads return 0 and their
// stores are dropped by the hardware range check.
template <class IO, bool GATE, bool ZOH, bool CONV, int G, int BI>
__global__ void __launch_bounds__(kDecodeThreads) decode_vec4_kernel(DecodeArgs a) {
  using elem = typename IO::elem;
  using raw4 = typename Vec4In<IO>::raw;  // four io elements
  using V = Vec4In<IO>;
  constexpr int ES = sizeof(elem);
  constexpr int LOG_G = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : 4;
  static_assert((1 << LOG_G) == G && G <= 16, "lanes per channel");
  const int N = a.d_state;
  const int D = static_cast<int>(a.d_inner);
  const uint32_t st_bytes = static_cast<uint32_t>(D) * N * 4;  // one batch row of the state
  const rsrc_t rA = make_buf(a.A, st_bytes);

  // Per-channel inputs.  With G >= 4 the four lanes of a quad (one channel) split them: lane 0
  // of the quad loads u, lane 1 delta, lane 2 z, and lanes 0/1 also delta_bias/D; DPP quad
  // broadcasts then hand them to the whole quad.  That is 2 narrow loads per lane instead of 5,
  // and the narrow loads are what the memory pipeline spends the most instructions on.
  constexpr bool QUAD = G >= 4;
  static_assert(!CONV || QUAD, "the front end needs a quad per channel");
  const int qq = threadIdx.x & 3;
  // With the front end (CONV) the quad's lanes load delta / z instead, lane 2 the conv bias, and
  // every lane one element of the 4-wide input window [conv_state (K-1 entries), x] with its tap
  // weight; the window sum is a quad reduction.
  const elem* aux_base =
      CONV ? static_cast<const elem*>(qq == 0 ? a.delta : (GATE && qq == 1 ? a.z : a.delta))
           : static_cast<const elem*>(qq == 0 ? a.u
                                              : (qq == 1 ? a.delta
                                                         : (GATE && qq == 2 ? a.z : a.u)));
  const float* f_src = qq == 0 ? a.delta_bias : ((CONV && qq == 2) ? a.conv_b : a.D);
  const bool f_ok = f_src != nullptr;
  const float* f_base = f_ok ? f_src : a.A;  // any valid address; the value is then zeroed

  const uint32_t l = blockIdx.x * kDecodeThreads + threadIdx.x;  // lane within a batch row
  const uint32_t d = l >> LOG_G, q = l & (G - 1);
  const bool act = d < static_cast<uint32_t>(D) && q * 4 < static_cast<uint32_t>(N);
  const uint32_t dcl = d < static_cast<uint32_t>(D) ? d : D - 1;  // channel clamped into the row
  const uint32_t so = act ? (d * N + q * 4) * 4 : kOffNone;       // state and A, within a row
  const uint32_t io = act ? d * ES : kOffNone;                    // u, delta, z, within a row
  const uint32_t bo = act ? q * 4 * ES : kOffNone;                // B, C, within a row
  const uint32_t oo = act && q == 0 ? d * ES : kOffNone;          // out (first lane of the group)

  // the channel's own values, shared by the rows of every group
  const float4 av = buf_load<float4>(rA, so);
  float fv = 0.0f, bias_c = 0.0f, dsk_c = 0.0f, wt = 0.0f;
  if (QUAD) {
    fv = f_base[dcl];  // delta_bias, D or the conv bias by lane of the quad
  } else {
    const uint32_t fo = act ? d * 4 : kOffNone;
    bias_c = buf_load<float>(make_buf(a.delta_bias, a.delta_bias ? D * 4u : 0u), fo);
    dsk_c = buf_load<float>(make_buf(a.D, a.D ? D * 4u : 0u), fo);
  }
  const int K = CONV ? a.conv_k : 0;
  const int jw = qq - (4 - K);  // this lane's window slot as a tap index (< 0: unused)
  if (CONV) {                   // tap weight (unused slots: a valid address, the value zeroed)
    const float wv = a.conv_w[int64_t(dcl) * K + (jw >= 0 ? jw : 0)];
    wt = jw >= 0 ? wv : 0.0f;
  }

  for (int64_t b0 = int64_t(blockIdx.y) * BI; b0 < a.batch; b0 += int64_t(gridDim.y) * BI) {
    const int nb = a.batch - b0 < BI ? static_cast<int>(a.batch - b0) : BI;
    const rsrc_t rs = make_buf(a.state + b0 * D * N, nb * st_bytes);
    const rsrc_t rB = make_buf(static_cast<const elem*>(a.B) + b0 * N, nb * N * ES);
    const rsrc_t rC = make_buf(static_cast<const elem*>(a.C) + b0 * N, nb * N * ES);
    const rsrc_t ro = make_buf(static_cast<elem*>(a.out) + b0 * D, nb * D * ES);
    const uint32_t xb = QUAD ? 0u : nb * D * ES;
    const rsrc_t ru = make_buf(QUAD ? nullptr : static_cast<const elem*>(a.u) + b0 * D, xb);
    const rsrc_t rd = make_buf(QUAD ? nullptr : static_cast<const elem*>(a.delta) + b0 * D, xb);
    const rsrc_t rz = make_buf(QUAD || !GATE ? nullptr : static_cast<const elem*>(a.z) + b0 * D,
                               QUAD || !GATE ? 0u : xb);
    float4 hv[BI];
    raw4 bv[BI], cv[BI];
    elem xr[BI], dr[BI], zr[BI], wn[BI];
    // the state stream first: every row's 16 bytes in flight before any narrow input returns
#pragma unroll
    for (int i = 0; i < BI; ++i) hv[i] = buf_load<float4>(rs, so + i * st_bytes);
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int64_t bi = b0 + (i < nb ? i : nb - 1);  // row clamped into the batch
      bv[i] = buf_load<raw4>(rB, bo + i * N * ES);
      cv[i] = buf_load<raw4>(rC, bo + i * N * ES);
      if (CONV) {  // window element of this lane (unused slots: a valid address, value zeroed)
        const bool from_x = qq == 3 || jw < 0;
        const elem* src = from_x ? static_cast<const elem*>(a.u) + bi * D + dcl
                                 : static_cast<const elem*>(a.conv_state) +
                                       (bi * (K - 1) + jw) * D + dcl;
        const elem v = *src;
        wn[i] = jw >= 0 ? v : elem{};
      }
      if (QUAD) {
        xr[i] = aux_base[bi * D + dcl];  // u, delta or z by lane of the quad
      } else {
        xr[i] = buf_load<elem>(ru, io + i * D * ES);
        dr[i] = buf_load<elem>(rd, io + i * D * ES);
        if (GATE) zr[i] = buf_load<elem>(rz, io + i * D * ES);
      }
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      float x, s, zv = 0.0f, dskip;
      if (CONV) {
        const float w = IO::widen(xr[i]);
        const float f = f_ok ? fv : 0.0f;
        const float win = IO::widen(wn[i]);
        x = silu_f(group_sum<4>(wt * win) + quad_bcast<2>(f));
        s = quad_bcast<0>(w) + quad_bcast<0>(f);
        if (GATE) zv = quad_bcast<1>(w);
        dskip = quad_bcast<1>(f);
        // shift the window: slot j of the new state is the old slot j + 1 (the last one is x);
        // the first quad of the channel writes, for rows inside the batch
        const int pos = jw - 1;
        if (pos >= 0 && (l & (G - 1)) < 4 && d < static_cast<uint32_t>(D) && i < nb)
          static_cast<elem*>(a.conv_state)[((b0 + i) * (K - 1) + pos) * D + dcl] = wn[i];
      } else if (QUAD) {
        const float w = IO::widen(xr[i]);
        const float f = f_ok ? fv : 0.0f;
        x = quad_bcast<0>(w);
        s = quad_bcast<1>(w) + quad_bcast<0>(f);
        if (GATE) zv = quad_bcast<2>(w);
        dskip = quad_bcast<1>(f);
      } else {
        x = IO::widen(xr[i]);
        s = IO::widen(dr[i]) + bias_c;
        if (GATE) zv = IO::widen(zr[i]);
        dskip = dsk_c;
      }
      const float dt = a.softplus ? softplus_f(s) : s;
      const float du = dt * x;
      float hh[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
      const float aa[4] = {av.x, av.y, av.z, av.w};
      float p = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = dt * (aa[j] * kLog2e);
        const float e = exp2_hw(y);
        const float inc = du * V::get(bv[i], j);
        hh[j] = fmaf(e, hh[j], ZOH ? inc * (zoh_gain(e, y) * (1.0f / kLn2)) : inc);
        p = fmaf(V::get(cv[i], j), hh[j], p);  // inactive lanes: C reads 0, p stays 0
      }
      buf_store(make_float4(hh[0], hh[1], hh[2], hh[3]), rs, so + i * st_bytes);
      p = group_sum<G>(p);
      float y = fmaf(dskip, x, p);
      if (GATE) y *= silu_f(zv);
      buf_store(IO::from_float(y), ro, oo + i * D * ES);
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

template <class IO, bool GATE, bool ZOH, int G, bool CONV = false>
void launch_vec(const DecodeArgs& a, hipStream_t stream) {
  const int64_t row_lanes = a.d_inner * G;
  const int64_t groups = (a.batch + kDecodeRows - 1) / kDecodeRows;
  const dim3 grid(static_cast<unsigned>((row_lanes + kDecodeThreads - 1) / kDecodeThreads),
                  static_cast<unsigned>(groups < 65535 ? groups : 65535));
  hipLaunchKernelGGL((decode_vec4_kernel<IO, GATE, ZOH, CONV, G, kDecodeRows>), grid,
                     dim3(kDecodeThreads), 0, stream, a);
}

template <class IO, bool GATE, bool ZOH>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  if (a.conv_w) {  // the host admits the front end only on the vector path with G >= 4
    switch (a.lanes_per_chan) {
      case 4: launch_vec<IO, GATE, ZOH, 4, true>(a, stream); break;
      case 8: launch_vec<IO, GATE, ZOH, 8, true>(a, stream); break;
      default: launch_vec<IO, GATE, ZOH, 16, true>(a, stream); break;
    }
    return hipGetLastError();
  }
  if (a.vec4) {
    switch (a.lanes_per_chan) {
      case 1: launch_vec<IO, GATE, ZOH, 1>(a, stream); break;
      case 2: launch_vec<IO, GATE, ZOH, 2>(a, stream); break;
      case 4: launch_vec<IO, GATE, ZOH, 4>(a, stream); break;
      case 8: launch_vec<IO, GATE, ZOH, 8>(a, stream); break;
      default: launch_vec<IO, GATE, ZOH, 16>(a, stream); break;
    }
  } else {
    const int64_t lanes = a.batch * a.d_inner * a.lanes_per_chan;
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
