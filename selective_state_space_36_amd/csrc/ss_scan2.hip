// ss_scan2.hip -- gfx950 multi-head selective scan with a scalar transition per head (the
// Mamba-2 form: IBM explainer, Mamba-2 heads with B and C shared by groups of heads; Cartesia
// Mamba-3 post: the diagonal transition reduced to a scalar times the identity).  For batch b,
// head h of group g, state n and head channel p:
//     dt_t = softplus(dt + dt_bias[h]),  S_t[n,p] = exp(dt_t A[h]) S_{t-1}[n,p] + dt_t B_t[n] x_t[p]
//     y_t[p] = sum_n C_t[n] S_t[n,p] + D[h] x_t[p],  out = y_t[p] silu(z_t[p]).
// The decay is one number per (token, head), so an update is a multiply and two FMAs with no
// exponential.
//
// Work layout: one workgroup per (batch row, head, block of 16 head channels) -- channels of a
// head are independent, which gives the 80-head layers enough workgroups.  Lane p of a 16-lane
// row owns head channel p of the block; the 16 rows of the workgroup (4 per wave) own 16 slices
// of NPT states each, so a thread keeps NPT state values in registers.  Per step a thread updates
// its NPT states, forms its share of y, and the wave's four rows are summed by row swaps; the four
// waves' sums meet in LDS and are finished (skip, gate, store) after each 16-step chunk.  B and C
// of a chunk are staged in LDS as float32 and read by all lanes of a row at once; the next
// chunk's global loads are issued before the current chunk is computed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "ss_device.h"
#include "ss_scan2.h"

namespace ss {
namespace {

constexpr int kT = kScan2Chunk;
constexpr int kPB = kScan2PBlock;

__device__ __forceinline__ float sum_rows4(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <class IO, int NPT, bool GATE>
struct Scan2Kernel {
  using elem = typename IO::elem;
  static constexpr int NP = 16 * NPT;                  // padded state count
  static constexpr int BC_PER_THREAD = kT * NP / kScan2Threads;  // = NPT

  struct alignas(16) Smem {
    float b[kT][NP];         // B_t[n] of the chunk
    float c[kT][NP];         // C_t[n]
    float x[kT][kPB];        // x_t[p] of the block
    float z[kT][kPB];        // z_t[p]
    float dt[kT], e[kT];     // dt_t and exp(dt_t A) of the head
    float y[4][kT][kPB];     // per wave: y summed over the wave's state slices
  };

  static __device__ __forceinline__ void run(const Scan2Args& a) {
    __shared__ Smem sm;
    const int64_t H = a.nheads, P = a.headdim, G = a.ngroups, L = a.seqlen;
    const int N = a.d_state;
    int64_t blk = blockIdx.x;
    const int64_t pb = __builtin_amdgcn_readfirstlane(static_cast<int>(blk % a.n_pblk));
    blk /= a.n_pblk;
    const int64_t h = __builtin_amdgcn_readfirstlane(static_cast<int>(blk % H));
    const int64_t b = __builtin_amdgcn_readfirstlane(static_cast<int>(blk / H));
    const int64_t g = h / (H / G);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int pl = lane & 15;                      // head channel within the block
    const int ns = wave * 4 + (lane >> 4);         // state slice
    const int64_t p = pb * kPB + pl;
    const bool p_ok = p < P;
    const float A2 = a.A[h] * kLog2e;
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float dskip = a.D ? a.D[h] : 0.0f;

    float S[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int n = ns * NPT + j;
      S[j] = (a.h0 && p_ok && n < N) ? a.h0[((b * H + h) * N + n) * P + p] : 0.0f;
    }

    // cooperative loads: thread -> (step, channel) of x and z, (step) of dt, and NPT (step, state)
    // elements of B and C; raw buffers sized to the chunk's valid steps return 0 past the end.
    const int nchunks = static_cast<int>((L + kT - 1) / kT);
    const int last_valid = static_cast<int>(L - int64_t(nchunks - 1) * kT);
    auto nvalid_of = [&](int c) { return c == nchunks - 1 ? last_valid : kT; };
    const int xt = tid >> 4, xp = tid & 15;
    const uint32_t x_off = (pb * kPB + xp < P)
                               ? static_cast<uint32_t>((xt * H * P + xp) * sizeof(elem))
                               : kOffNone;
    const uint32_t dt_off = tid < kT ? static_cast<uint32_t>(tid * H * sizeof(elem)) : kOffNone;
    uint32_t bc_off[BC_PER_THREAD];
    int bc_t[BC_PER_THREAD], bc_n[BC_PER_THREAD];
#pragma unroll
    for (int i = 0; i < BC_PER_THREAD; ++i) {
      const int idx = tid + i * kScan2Threads;
      bc_t[i] = idx / NP;
      bc_n[i] = idx - bc_t[i] * NP;
      bc_off[i] = bc_n[i] < N ? static_cast<uint32_t>((bc_t[i] * G * N + bc_n[i]) * sizeof(elem))
                              : kOffNone;
    }
    elem rx, rz = elem{}, rdt;
    elem rb[BC_PER_THREAD], rc[BC_PER_THREAD];
    auto issue = [&](int c) {
      const int nv = nvalid_of(c);
      const int64_t t0 = int64_t(c) * kT;
      const char* xb = static_cast<const char*>(a.x) +
                       (((b * L + t0) * H + h) * P + pb * kPB) * sizeof(elem);
      const uint32_t xbytes = static_cast<uint32_t>(((nv - 1) * H * P + (P - pb * kPB)) *
                                                    sizeof(elem));
      rx = buf_load<elem>(make_buf(xb, xbytes), x_off);
      if (GATE) {
        const char* zb = static_cast<const char*>(a.z) +
                         (((b * L + t0) * H + h) * P + pb * kPB) * sizeof(elem);
        rz = buf_load<elem>(make_buf(zb, xbytes), x_off);
      }
      const char* db = static_cast<const char*>(a.dt) + ((b * L + t0) * H + h) * sizeof(elem);
      rdt = buf_load<elem>(make_buf(db, static_cast<uint32_t>(((nv - 1) * H + 1) * sizeof(elem))),
                           dt_off);
      const int64_t bco = ((b * L + t0) * G + g) * N * sizeof(elem);
      const uint32_t bcbytes = static_cast<uint32_t>(((nv - 1) * G * N + N) * sizeof(elem));
      const rsrc_t rbb = make_buf(static_cast<const char*>(a.B) + bco, bcbytes);
      const rsrc_t rcc = make_buf(static_cast<const char*>(a.C) + bco, bcbytes);
#pragma unroll
      for (int i = 0; i < BC_PER_THREAD; ++i) {
        rb[i] = buf_load<elem>(rbb, bc_off[i]);
        rc[i] = buf_load<elem>(rcc, bc_off[i]);
      }
    };
    auto stage = [&](int c) {
      const int nv = nvalid_of(c);
      sm.x[xt][xp] = IO::widen(rx);
      if (GATE) sm.z[xt][xp] = IO::widen(rz);
#pragma unroll
      for (int i = 0; i < BC_PER_THREAD; ++i) {
        sm.b[bc_t[i]][bc_n[i]] = IO::widen(rb[i]);
        sm.c[bc_t[i]][bc_n[i]] = IO::widen(rc[i]);
      }
      if (tid < kT) {
        const float s = IO::widen(rdt) + bias;
        float d = a.softplus ? softplus_f(s) : s;
        d = tid < nv ? d : 0.0f;  // steps past the end leave the state unchanged
        sm.dt[tid] = d;
        sm.e[tid] = exp2_hw(d * A2);
      }
    };

    if (nchunks > 0) {
      issue(0);
      stage(0);
      __syncthreads();
    }
    for (int c = 0; c < nchunks; ++c) {
      if (c + 1 < nchunks) issue(c + 1);
      float dtv[kT], ev[kT];
#pragma unroll
      for (int i = 0; i < kT; i += 4) {
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dt[i]);
        const float4 e4 = *reinterpret_cast<const float4*>(&sm.e[i]);
        dtv[i] = d4.x; dtv[i + 1] = d4.y; dtv[i + 2] = d4.z; dtv[i + 3] = d4.w;
        ev[i] = e4.x; ev[i + 1] = e4.y; ev[i + 2] = e4.z; ev[i + 3] = e4.w;
      }
      steps(std::make_integer_sequence<int, kT>{}, sm, dtv, ev, S, ns, pl, wave, lane);
      __syncthreads();  // y shares of all waves are in LDS
      {
        const int t = tid >> 4, q = tid & 15;
        const int64_t pp = pb * kPB + q;
        if (t < nvalid_of(c) && pp < P) {
          float y = sm.y[0][t][q] + sm.y[1][t][q] + sm.y[2][t][q] + sm.y[3][t][q];
          const float xv = sm.x[t][q];
          y = fmaf(dskip, xv, y);
          if (GATE) y *= silu_f(sm.z[t][q]);
          static_cast<elem*>(a.out)[((b * L + int64_t(c) * kT + t) * H + h) * P + pp] =
              IO::from_float(y);
        }
      }
      __syncthreads();  // the chunk's tiles have been read
      if (c + 1 < nchunks) {
        stage(c + 1);
        __syncthreads();
      }
    }
    if (a.h_last && p_ok) {
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        const int n = ns * NPT + j;
        if (n < N) a.h_last[((b * H + h) * N + n) * P + p] = S[j];
      }
    }
  }

  // Step T: S <- e_T S + (dt_T x_T[p]) B_T[n] for this thread's NPT states, y share C_T . S.
  template <int T>
  static __device__ __forceinline__ void step(Smem& sm, const float (&dtv)[kT],
                                              const float (&ev)[kT], float (&S)[NPT], int ns,
                                              int pl, int wave, int lane) {
    const float xdt = dtv[T] * sm.x[T][pl];
    const float e = ev[T];
    const float* bp = &sm.b[T][ns * NPT];
    const float* cp = &sm.c[T][ns * NPT];
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      S[j] = fmaf(e, S[j], xdt * bp[j]);
      y = fmaf(cp[j], S[j], y);
    }
    y = sum_rows4(y);
    if (lane < 16) sm.y[wave][T][pl] = y;
  }
  template <int... TS>
  static __device__ __forceinline__ void steps(std::integer_sequence<int, TS...>, Smem& sm,
                                               const float (&dtv)[kT], const float (&ev)[kT],
                                               float (&S)[NPT], int ns, int pl, int wave,
                                               int lane) {
    (step<TS>(sm, dtv, ev, S, ns, pl, wave, lane), ...);
  }
};

template <class IO, int NPT, bool GATE>
__global__ void __launch_bounds__(kScan2Threads) scan2_kernel(Scan2Args a) {
  Scan2Kernel<IO, NPT, GATE>::run(a);
}

template <class IO, int NPT>
void launch_n(const Scan2Args& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.batch * a.nheads * a.n_pblk)), block(kScan2Threads);
  if (a.z)
    hipLaunchKernelGGL((scan2_kernel<IO, NPT, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((scan2_kernel<IO, NPT, false>), grid, block, 0, stream, a);
}

template <class IO>
void launch_io(const Scan2Args& a, hipStream_t stream) {
  const int npt = (a.d_state + 15) / 16;
  if (npt <= 1) launch_n<IO, 1>(a, stream);
  else if (npt <= 2) launch_n<IO, 2>(a, stream);
  else if (npt <= 4) launch_n<IO, 4>(a, stream);
  else if (npt <= 8) launch_n<IO, 8>(a, stream);
  else launch_n<IO, 16>(a, stream);
}

}  // namespace

hipError_t launch_scan2(const Scan2Args& a, bool bf16, hipStream_t stream) {
  if (a.batch * a.nheads * a.n_pblk == 0) return hipSuccess;
  if (bf16) launch_io<BF16>(a, stream);
  else launch_io<F32>(a, stream);
  return hipGetLastError();
}

}  // namespace ss
