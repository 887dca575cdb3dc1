// ss_scan_fwd.hip -- gfx950 prefill kernels of the selective scan.
//
// What is computed (per batch row b, channel d, state n; see the Mamba reading guide, sections
// "Método" and "O Mecanismo de Seleção (S6)"):
//     dt_t = softplus(delta + bias),  h_t = exp(dt_t A) h_{t-1} + dt_t B_t u_t,
//     y_t = C_t . h_t + D u_t,  out = y_t * silu(z_t).
// The (batch, L, d_inner, d_state) state never leaves registers; only y reaches HBM ("Expansão
// de Estado Ciente de Hardware").
//
// Work layout (chosen for CDNA4, not taken from the pages' GPU design):
//   * One channel = one 16-lane DPP row; lane k of the row owns states n = k, k+16, k+32, k+48.
//     A wave holds 4 channels, a workgroup 16.  A cfg like (4, 4096, 5120, 16) thus yields
//     5 waves per SIMD with no ragged wave count, which a channel-per-lane layout cannot.
//   * Time runs in 16-step sub-chunks.  Lane k also owns the element work (softplus, dt*u,
//     skip, gate, store) of step k of each sub-chunk; the per-step dt and dt*u reach the other
//     lanes of the row through DPP row broadcasts folded into the multiplies that consume them.
//   * B_t and C_t (shared by all channels) are staged per 32-step tile in LDS as float pairs.
//   * The row's 16 partial sums C_t[n] h_t[n] go through a per-wave LDS tile; the owner lane of
//     step t adds them up.  No atomics: results are bitwise reproducible.
//   * Long sequences with few channels are cut into time segments.  A summary pass computes each
//     segment's end state from a zero start and the sum of its dt; the output pass then starts
//     segment s from h0 carried through segments 0..s-1 with h <- exp(A sum dt) h + h_end, the
//     blockwise form of the associative recurrence (reading guide: parallel associative scan;
//     IBM explainer: blocks combined hierarchically).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kWaves = kPrefillThreads / 64;
constexpr int kSub = 16;                 // steps per sub-chunk = lanes per row
constexpr int kTileStride = kChunk + 2;  // float2 slots per state row of the B/C tile (padding)
constexpr int kPRow = 336;               // floats per channel row of the partial tile (padding)
constexpr int kPTau = 20;                // floats per step of the partial tile (padding)

template <class IO, int NL, bool GATE, bool SUMMARY>
struct ScanKernel {
  using elem = typename IO::elem;
  static constexpr int NP = 16 * NL;  // padded state count

  struct alignas(16) Smem {
    float2 bc[2][NP][kTileStride];      // (B_t[n], C_t[n]) for the current and next tile
    float p[kWaves][4 * kPRow];         // per-wave partial sums, [row][step][lane]
  };

  static __device__ __forceinline__ void run(const ScanArgs& a) {
    __shared__ Smem sm;
    const int64_t ncb_total = a.batch * a.n_cblk;
    const int64_t lg = xcd_remap(blockIdx.x, a.n_wg);
    const int64_t seg = lg / ncb_total;
    const int64_t cb = lg - seg * ncb_total;
    const int64_t b = cb / a.n_cblk;
    const int64_t d0 = (cb - b * a.n_cblk) * kChanPerWG;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane >> 4;   // channel within the wave
    const int k = lane & 15;   // lane within the row
    const int64_t d = d0 + wave * 4 + r;
    const bool chan_ok = d < a.d_inner;
    const int64_t row = b * a.d_inner + d;  // (b, d) row index
    const int64_t t_begin = seg * a.seg_len;
    const int64_t t_end = (t_begin + a.seg_len < a.seqlen) ? t_begin + a.seg_len : a.seqlen;

    const elem* __restrict__ u = static_cast<const elem*>(a.u);
    const elem* __restrict__ dl = static_cast<const elem*>(a.delta);
    const elem* __restrict__ zz = static_cast<const elem*>(a.z);
    const elem* __restrict__ Bp = static_cast<const elem*>(a.B);
    const elem* __restrict__ Cp = static_cast<const elem*>(a.C);
    elem* __restrict__ outp = static_cast<elem*>(a.out);

    // Per-lane constants: A scaled by log2(e) so that exp(dt A) = 2^(dt A2).
    float A2[NL], h[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int n = k + 16 * j;
      const bool ok = chan_ok && n < a.d_state;
      A2[j] = ok ? a.A[d * a.d_state + n] * kLog2e : 0.0f;
      h[j] = 0.0f;
    }
    const float bias = (chan_ok && a.delta_bias) ? a.delta_bias[d] : 0.0f;
    const float dskip = (!SUMMARY && chan_ok && a.D) ? a.D[d] : 0.0f;

    if (!SUMMARY) {
      // Initial state of this segment: h0 carried through the summaries of segments 0..seg-1.
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int n = k + 16 * j;
        if (a.h0 && chan_ok && n < a.d_state) h[j] = a.h0[row * a.d_state + n];
      }
      for (int64_t s = 0; s < seg; ++s) {
        const int64_t srow = s * a.batch * a.d_inner + row;
        const float dsum = chan_ok ? a.seg_dt[srow] : 0.0f;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int n = k + 16 * j;
          const float he = (chan_ok && n < a.d_state) ? a.seg_h[srow * a.d_state + n] : 0.0f;
          h[j] = fmaf(exp2_hw(A2[j] * dsum), h[j], he);
        }
      }
    }

    // ---- B/C tile staging: NP states x kChunk steps ----
    // Loads go to registers as raw elements at clamped (always valid) addresses and are only
    // widened and masked when written to LDS, so that they stay in flight while the current tile
    // is being processed.
    constexpr int kTilePairs = NP * kChunk;
    constexpr int kPerThread = (kTilePairs + kPrefillThreads - 1) / kPrefillThreads;
    elem tb[kPerThread], tc[kPerThread];
    auto tile_load = [&](int64_t t0) {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        const int idx = threadIdx.x + i * kPrefillThreads;
        const int tau = idx / NP, n = idx - (idx / NP) * NP;
        const int64_t t = (t0 + tau < t_end) ? t0 + tau : t_end - 1;
        const int nc = n < a.d_state ? n : a.d_state - 1;
        const int64_t off = (b * a.seqlen + t) * a.d_state + nc;
        tb[i] = Bp[off];
        tc[i] = Cp[off];
      }
    };
    auto tile_store = [&](int buf, int64_t t0) {
#pragma unroll
      for (int i = 0; i < kPerThread; ++i) {
        const int idx = threadIdx.x + i * kPrefillThreads;
        if (idx < kTilePairs) {
          const int tau = idx / NP, n = idx - (idx / NP) * NP;
          const bool ok = t0 + tau < t_end && n < a.d_state;
          sm.bc[buf][n][tau] = ok ? make_float2(IO::widen(tb[i]), IO::widen(tc[i]))
                                  : make_float2(0.0f, 0.0f);
        }
      }
    };

    // ---- own-element inputs of a sub-chunk: step t0 + k of channel d (raw, clamped) ----
    const int64_t d_c = chan_ok ? d : a.d_inner - 1;
    elem own_u, own_d, own_z{};
    auto own_load = [&](int64_t t0, elem& ou, elem& od, elem& oz) {
      const int64_t t = (t0 + k < t_end) ? t0 + k : t_end - 1;
      const int64_t off = (b * a.seqlen + t) * a.d_inner + d_c;
      ou = u[off];
      od = dl[off];
      if (GATE && !SUMMARY) oz = zz[off];
    };

    float dt_acc = 0.0f;  // summary pass: this lane's share of sum(dt) over the segment

    tile_load(t_begin);
    tile_store(0, t_begin);
    own_load(t_begin, own_u, own_d, own_z);
    __syncthreads();

    int buf = 0;
    for (int64_t tcb = t_begin; tcb < t_end; tcb += kChunk) {
      const bool has_next = tcb + kChunk < t_end;
      if (has_next) tile_load(tcb + kChunk);
#pragma unroll
      for (int q = 0; q < kChunk / kSub; ++q) {
        const int64_t t0 = tcb + q * kSub;
        if (t0 < t_end) {
          // prefetch the next sub-chunk's own inputs (clamped: always a valid address)
          elem nu, nd, nz{};
          own_load(t0 + kSub, nu, nd, nz);

          const bool own_ok = chan_ok && (t0 + k) < t_end;
          const float xu = IO::widen(own_u);
          const float s = IO::widen(own_d) + bias;
          float dt = a.softplus ? softplus_f(s) : s;
          dt = own_ok ? dt : 0.0f;                  // steps past the end leave h unchanged
          const float du = own_ok ? dt * xu : 0.0f;
          if (SUMMARY) dt_acc += dt;

          sub_chunk(sm, buf, q * kSub, dt, du, A2, h, wave, r, k);

          if (!SUMMARY) {
            wave_lds_sync();
            const float* pr = &sm.p[wave][r * kPRow + k * kPTau];
            const float4 q0 = *reinterpret_cast<const float4*>(pr + 0);
            const float4 q1 = *reinterpret_cast<const float4*>(pr + 4);
            const float4 q2 = *reinterpret_cast<const float4*>(pr + 8);
            const float4 q3 = *reinterpret_cast<const float4*>(pr + 12);
            wave_lds_sync();
            float y = (((q0.x + q0.y) + (q0.z + q0.w)) + ((q1.x + q1.y) + (q1.z + q1.w))) +
                      (((q2.x + q2.y) + (q2.z + q2.w)) + ((q3.x + q3.y) + (q3.z + q3.w)));
            y = fmaf(dskip, xu, y);
            if (GATE) y *= silu_f(IO::widen(own_z));
            if (own_ok) outp[(b * a.seqlen + t0 + k) * a.d_inner + d] = IO::from_float(y);
          }
          own_u = nu;
          own_d = nd;
          own_z = nz;
        }
      }
      if (has_next) tile_store(buf ^ 1, tcb + kChunk);
      __syncthreads();
      buf ^= 1;
    }

    if (SUMMARY) {
      // segment summary: local end state and the row's total dt
      float sdt = dt_acc;
      sdt += __shfl_xor(sdt, 1, 16);
      sdt += __shfl_xor(sdt, 2, 16);
      sdt += __shfl_xor(sdt, 4, 16);
      sdt += __shfl_xor(sdt, 8, 16);
      if (chan_ok) {
        const int64_t srow = seg * a.batch * a.d_inner + row;
        if (k == 0) a.seg_dt[srow] = sdt;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int n = k + 16 * j;
          if (n < a.d_state) a.seg_h[srow * a.d_state + n] = h[j];
        }
      }
    } else if (a.h_last && chan_ok && seg == a.nseg - 1) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int n = k + 16 * j;
        if (n < a.d_state) a.h_last[row * a.d_state + n] = h[j];
      }
    }
  }

  // One recurrence step (TAU of the sub-chunk) for this lane's states.  bcv holds the sub-chunk's
  // (B, C) pairs for this lane's states, two steps per float4.
  template <int TAU>
  static __device__ __forceinline__ void step(Smem& sm, const float4 (&bcv)[NL][kSub / 2],
                                              float dt, float du, const float (&A2)[NL],
                                              float (&h)[NL], int wave, int r, int k) {
    const float dtb = row_bcast<TAU>(dt);
    const float dub = row_bcast<TAU>(du);
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const float4 v = bcv[j][TAU / 2];
      const float bb = (TAU & 1) ? v.z : v.x;
      const float cc = (TAU & 1) ? v.w : v.y;
      const float e = exp2_hw(dtb * A2[j]);
      h[j] = fmaf(e, h[j], dub * bb);
      p = (j == 0) ? cc * h[j] : fmaf(cc, h[j], p);
    }
    if (!SUMMARY) sm.p[wave][r * kPRow + TAU * kPTau + k] = p;
  }

  template <int... TAUS>
  static __device__ __forceinline__ void steps(std::integer_sequence<int, TAUS...>, Smem& sm,
                                               const float4 (&bcv)[NL][kSub / 2], float dt,
                                               float du, const float (&A2)[NL], float (&h)[NL],
                                               int wave, int r, int k) {
    (step<TAUS>(sm, bcv, dt, du, A2, h, wave, r, k), ...);
  }

  // 16 recurrence steps of one sub-chunk.  toff: offset of the sub-chunk inside the B/C tile.
  // The tile reads are issued together up front (16-byte reads, two steps each) so that the
  // steps themselves are pure VALU work.
  static __device__ __forceinline__ void sub_chunk(Smem& sm, int buf, int toff, float dt,
                                                   float du, const float (&A2)[NL],
                                                   float (&h)[NL], int wave, int r, int k) {
    float4 bcv[NL][kSub / 2];
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
      for (int i = 0; i < kSub / 2; ++i)
        bcv[j][i] = *reinterpret_cast<const float4*>(&sm.bc[buf][k + 16 * j][toff + 2 * i]);
    steps(std::make_integer_sequence<int, kSub>{}, sm, bcv, dt, du, A2, h, wave, r, k);
  }
};

template <class IO, int NL, bool GATE, bool SUMMARY>
__global__ void __launch_bounds__(kPrefillThreads) scan_kernel(ScanArgs a) {
  ScanKernel<IO, NL, GATE, SUMMARY>::run(a);
}

__global__ void __launch_bounds__(256) copy_state_kernel(float* dst, const float* src, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src ? src[i] : 0.0f;
}

template <class IO, int NL, bool GATE>
hipError_t launch3(const ScanArgs& a, bool summary, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.n_wg)), block(kPrefillThreads);
  if (summary)
    hipLaunchKernelGGL((scan_kernel<IO, NL, GATE, true>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((scan_kernel<IO, NL, GATE, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <class IO, int NL>
hipError_t launch2(const ScanArgs& a, bool summary, hipStream_t stream) {
  // the gate never matters in the summary pass
  if (a.z != nullptr && !summary) return launch3<IO, NL, true>(a, summary, stream);
  return launch3<IO, NL, false>(a, summary, stream);
}

template <class IO>
hipError_t launch1(const ScanArgs& a, bool summary, hipStream_t stream) {
  switch ((a.d_state + 15) / 16) {
    case 1: return launch2<IO, 1>(a, summary, stream);
    case 2: return launch2<IO, 2>(a, summary, stream);
    case 3: return launch2<IO, 3>(a, summary, stream);
    default: return launch2<IO, 4>(a, summary, stream);
  }
}

}  // namespace

hipError_t launch_scan(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream) {
  return bf16 ? launch1<BF16>(a, summary, stream) : launch1<F32>(a, summary, stream);
}

hipError_t launch_copy_state(float* dst, const float* src, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(copy_state_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, dst, src, n);
  return hipGetLastError();
}

}  // namespace ss
