// ss_scan_fwd.hip -- gfx950 prefill kernels of the selective scan.
//
// What is computed (per batch row b, channel d, state n; Mamba reading guide, sections "Método"
// and "O Mecanismo de Seleção (S6)"):
//     dt_t = softplus(delta + bias),  h_t = exp(dt_t A) h_{t-1} + dt_t B_t u_t,
//     y_t = C_t . h_t + D u_t,  out = y_t * silu(z_t).
// The (batch, L, d_inner, d_state) state never leaves registers; only y reaches HBM (reading
// guide, "Expansão de Estado Ciente de Hardware").
//
// Work layout (chosen for CDNA4, not taken from the pages' GPU design):
//   * One channel = one 16-lane DPP row; lane k of the row owns states n = k, k+16, k+32, k+48.
//     A wave holds 4 channels, a workgroup 16.  A layer like (4, 4096, 5120, 16) thus yields
//     1280 workgroups = 5 per CU and 5 waves per SIMD, with no ragged last round.
//   * Time runs in 16-step chunks.  Lane k also owns the element work (softplus, dt*u, skip,
//     gate) of step k of each chunk; the per-step dt and dt*u reach the other lanes of the row
//     through DPP row broadcasts that the compiler folds into the multiplies consuming them.
//   * Global memory is touched only by cooperative 16-byte loads and stores of whole tiles
//     (u, delta, z and out as 16 steps x 16 channels; B and C as 16 steps x d_state), staged
//     through LDS and double-buffered so that the next chunk's loads are in flight while the
//     current chunk is computed.
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
constexpr int kT = kChunk;               // steps per chunk (= lanes per row)
constexpr int kTileStride = kT + 2;      // float2 slots per state row of the B/C tile (padding)
constexpr int kPRow = 336;               // floats per channel row of the partial tile (padding)
constexpr int kPTau = 20;                // floats per step of the partial tile (padding)
static_assert(kT == 16, "one chunk step per row lane");

template <class IO, int NL, bool GATE, bool SUMMARY, bool VEC>
struct ScanKernel {
  using elem = typename IO::elem;
  static constexpr int NP = 16 * NL;                         // padded state count
  static constexpr int ES = sizeof(elem);                    // io element bytes
  static constexpr int NTEN = SUMMARY ? 2 : (GATE ? 3 : 2);  // streamed inputs: u, delta, (z)
  static constexpr int PIECES = kChanPerWG * ES / 16;        // 16-byte pieces per tile row
  static constexpr int IN_PIECES = NTEN * kT * PIECES;       // per chunk
  static constexpr int OUT_PIECES = kT * PIECES;
  static_assert(IN_PIECES <= kPrefillThreads, "one 16-byte input piece per thread");
  static constexpr int BC_PER_THREAD = (kT * NP + kPrefillThreads - 1) / kPrefillThreads;

  struct alignas(16) Smem {
    float2 bc[2][NP][kTileStride];  // (B_t[n], C_t[n]) per chunk
    uint4 in[2][NTEN][kT][PIECES];  // raw u, delta, z tiles per chunk
    uint4 out[2][kT][PIECES];       // raw output tile per chunk
    float p[kWaves][4 * kPRow];     // per-wave partial sums [row][step][lane]
  };

  static __device__ __forceinline__ void run(const ScanArgs& a) {
    __shared__ Smem sm;
    const int64_t ncb_total = a.batch * a.n_cblk;
    const int64_t lg = xcd_remap(blockIdx.x, a.n_wg);
    const int64_t seg = lg / ncb_total;
    const int64_t cb = lg - seg * ncb_total;
    const int64_t b = cb / a.n_cblk;
    const int64_t d0 = (cb - b * a.n_cblk) * kChanPerWG;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r = lane >> 4;      // channel within the wave
    const int k = lane & 15;      // lane within the row = owned step of each chunk
    const int cl = wave * 4 + r;  // channel within the workgroup
    const int64_t d = d0 + cl;
    const bool chan_ok = d < a.d_inner;
    const int64_t row = b * a.d_inner + d;  // (b, d) row index
    const int64_t t_begin = seg * a.seg_len;
    const int64_t t_end = (t_begin + a.seg_len < a.seqlen) ? t_begin + a.seg_len : a.seqlen;

    const elem* __restrict__ Bp = static_cast<const elem*>(a.B);
    const elem* __restrict__ Cp = static_cast<const elem*>(a.C);
    const elem* __restrict__ up = static_cast<const elem*>(a.u);
    const elem* __restrict__ dp = static_cast<const elem*>(a.delta);
    const elem* __restrict__ zp = static_cast<const elem*>(a.z);
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

    // ---- cooperative tile traffic ----
    // Thread roles: B/C element(s) (tau, n) with consecutive threads on consecutive n (contiguous
    // in memory); one 16-byte piece (tensor, step row, piece) of the u/delta/z tiles; one 16-byte
    // piece (step row, piece) of the output tile.  Global loads for chunk i+1 are issued before
    // chunk i is computed and written to LDS after it.  All loads are unconditional, at running
    // pointers advanced by one chunk per call; only the last, partial chunk clamps its rows.
    const int64_t D = a.d_inner, N = a.d_state;
    const int64_t row0 = b * a.seqlen + t_begin;  // (b, t_begin) row of u/delta/z/out, B/C
    const int in_ten_raw = tid / (kT * PIECES);
    const int in_ten = in_ten_raw < NTEN ? in_ten_raw : NTEN - 1;
    const int in_row = (tid / PIECES) % kT;
    const int in_pc = tid % PIECES;
    const int64_t in_col = d0 + in_pc * (16 / ES);  // first channel of this thread's piece
    // a select, not an array of pointers: keeps the loads in the global address space
    const elem* __restrict__ in_src = in_ten == 0 ? up : (in_ten == 1 ? dp : zp);
    const elem* in_ld = in_src + (row0 + in_row) * D + in_col;
    int bc_tau[BC_PER_THREAD], bc_n[BC_PER_THREAD];
    bool bc_ok[BC_PER_THREAD];
    const elem* b_ld[BC_PER_THREAD];
    const elem* c_ld[BC_PER_THREAD];
#pragma unroll
    for (int i = 0; i < BC_PER_THREAD; ++i) {
      const int idx = tid + i * kPrefillThreads;
      bc_tau[i] = idx / NP;
      bc_n[i] = idx - bc_tau[i] * NP;
      bc_ok[i] = idx < kT * NP && bc_n[i] < N;
      const int64_t nc = bc_n[i] < N ? bc_n[i] : N - 1;
      const int64_t tau = bc_tau[i] < kT ? bc_tau[i] : kT - 1;
      b_ld[i] = Bp + (row0 + tau) * N + nc;
      c_ld[i] = Cp + (row0 + tau) * N + nc;
    }
    const int orow = tid / PIECES, opc = tid % PIECES;
    const int64_t out_col = d0 + opc * (16 / ES);
    elem* out_st = outp + (row0 + orow) * D + out_col;
    const int64_t nchunks = (t_end - t_begin + kT - 1) / kT;
    const bool partial = (t_end - t_begin) % kT != 0;  // the last chunk is cut short

    struct Pre {
      elem rb[BC_PER_THREAD], rc[BC_PER_THREAD];
      uint4 rin;
    } pre;

    auto load_piece = [&](const elem* src) -> uint4 {
      if (VEC) return *reinterpret_cast<const uint4*>(src);  // whole aligned block (host-checked)
      elem tmp[16 / ES];
#pragma unroll
      for (int e = 0; e < 16 / ES; ++e) tmp[e] = src[in_col + e < D ? e : D - 1 - in_col];
      return *reinterpret_cast<const uint4*>(tmp);
    };
    // valid steps of chunk ci (kT except for a partial last chunk); uniform over the workgroup
    const int last_valid = static_cast<int>(t_end - t_begin - (nchunks - 1) * kT);
    auto nvalid_of = [&](int64_t ci) { return ci == nchunks - 1 ? last_valid : kT; };

    auto load_chunk = [&](int64_t ci) {
      // Rows past the end of the sequence re-read the last valid row (their values are masked
      // when staged).  Only pointers are adjusted inside the (uniform) branch; the loads follow
      // the join, so no wait is forced there.
      const elem* pb[BC_PER_THREAD];
      const elem* pc[BC_PER_THREAD];
      const elem* pin = in_ld;
#pragma unroll
      for (int i = 0; i < BC_PER_THREAD; ++i) {
        pb[i] = b_ld[i];
        pc[i] = c_ld[i];
      }
      if (partial && ci == nchunks - 1) {
        const int vr = last_valid - 1;
#pragma unroll
        for (int i = 0; i < BC_PER_THREAD; ++i) {
          const int over = bc_tau[i] < kT ? max(bc_tau[i] - vr, 0) : 0;
          pb[i] -= over * N;
          pc[i] -= over * N;
        }
        pin -= static_cast<int64_t>(max(in_row - vr, 0)) * D;
      }
#pragma unroll
      for (int i = 0; i < BC_PER_THREAD; ++i) {
        pre.rb[i] = *pb[i];
        pre.rc[i] = *pc[i];
        b_ld[i] += kT * N;
        c_ld[i] += kT * N;
      }
      pre.rin = load_piece(pin);
      in_ld += kT * D;
    };
    auto stage_chunk = [&](int buf, int64_t ci) {
      const int nv = nvalid_of(ci);
#pragma unroll
      for (int i = 0; i < BC_PER_THREAD; ++i) {
        if (bc_tau[i] < kT) {
          float2 v = make_float2(IO::widen(pre.rb[i]), IO::widen(pre.rc[i]));
          if (NL * 16 != 16 || nv != kT) {  // masks needed only for padded states / a cut chunk
            if (!(bc_ok[i] && bc_tau[i] < nv)) v = make_float2(0.0f, 0.0f);
          } else if (!bc_ok[i]) {
            v = make_float2(0.0f, 0.0f);
          }
          sm.bc[buf][bc_n[i]][bc_tau[i]] = v;
        }
      }
      if (tid < IN_PIECES) {
        uint4 v = pre.rin;
        if (nv != kT && in_row >= nv) v = uint4{0, 0, 0, 0};
        if (!VEC) {
          elem tmp[16 / ES];
          *reinterpret_cast<uint4*>(tmp) = v;
#pragma unroll
          for (int e = 0; e < 16 / ES; ++e)
            if (in_col + e >= D) tmp[e] = elem{};
          v = *reinterpret_cast<const uint4*>(tmp);
        }
        sm.in[buf][in_ten][in_row][in_pc] = v;
      }
    };
    // The registers of the last output store are kept live (hold_store) until the next chunk's
    // compute is done: otherwise the allocator reuses them at once and the write to them has to
    // wait for the store to complete.
    uint4 st_val{0, 0, 0, 0};
    uint64_t st_ptr = 0;
    auto hold_store = [&]() {
      if (VEC && !SUMMARY)
        asm volatile("" ::"v"(st_val.x), "v"(st_val.y), "v"(st_val.z), "v"(st_val.w),
                     "v"(st_ptr));
    };
    auto store_out = [&](int buf, int64_t ci) {
      if (!SUMMARY && tid < OUT_PIECES) {
        if (orow < nvalid_of(ci)) {
          const uint4 v = sm.out[buf][orow][opc];
          if (VEC) {
            st_val = v;
            st_ptr = reinterpret_cast<uint64_t>(out_st);
            *reinterpret_cast<uint4*>(out_st) = v;
          } else {
            elem tmp[16 / ES];
            *reinterpret_cast<uint4*>(tmp) = v;
#pragma unroll
            for (int e = 0; e < 16 / ES; ++e)
              if (out_col + e < D) out_st[e] = tmp[e];
          }
        }
        out_st += kT * D;
      }
    };
    auto own_in = [&](int buf, int ten) -> float {
      const elem* t = reinterpret_cast<const elem*>(&sm.in[buf][ten][k][0]);
      return IO::widen(t[cl]);
    };

    float dt_acc = 0.0f;  // summary pass: this lane's share of sum(dt) over the segment

    load_chunk(0);
    stage_chunk(0, 0);
    __syncthreads();

    // Waves of different workgroups sharing a SIMD would otherwise be served oldest first, so
    // some finish early and the SIMD runs the end of the kernel with few waves.  A wave lowers
    // its issue priority as it progresses, which keeps the waves of a SIMD close together.
    int prio = 3;
    __builtin_amdgcn_s_setprio(3);
    const int64_t q1 = nchunks / 4, q2 = nchunks / 2, q3 = (3 * nchunks) / 4;

    int buf = 0;
    for (int64_t ci = 0; ci < nchunks; ++ci) {
      const bool has_next = ci + 1 < nchunks;
      if (has_next) load_chunk(ci + 1);

      if (ci == q1 || ci == q2 || ci == q3) {  // uniform
        --prio;
        if (prio == 2) __builtin_amdgcn_s_setprio(2);
        else if (prio == 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }

      const bool own_ok = chan_ok && k < nvalid_of(ci);
      const float xu = own_in(buf, 0);
      const float sv = own_in(buf, 1) + bias;
      float dt = a.softplus ? softplus_f(sv) : sv;
      dt = own_ok ? dt : 0.0f;  // steps past the end leave h unchanged
      const float du = own_ok ? dt * xu : 0.0f;
      if (SUMMARY) dt_acc += dt;

      chunk_steps(sm, buf, dt, du, A2, h, wave, r, k);

      if (!SUMMARY) {
        wave_lds_sync();
        const float* pr = &sm.p[wave][r * kPRow + k * kPTau];
        const float4 q0 = *reinterpret_cast<const float4*>(pr + 0);
        const float4 q1v = *reinterpret_cast<const float4*>(pr + 4);
        const float4 q2v = *reinterpret_cast<const float4*>(pr + 8);
        const float4 q3v = *reinterpret_cast<const float4*>(pr + 12);
        wave_lds_sync();
        float y = (((q0.x + q0.y) + (q0.z + q0.w)) + ((q1v.x + q1v.y) + (q1v.z + q1v.w))) +
                  (((q2v.x + q2v.y) + (q2v.z + q2v.w)) + ((q3v.x + q3v.y) + (q3v.z + q3v.w)));
        y = fmaf(dskip, xu, y);
        if (GATE) y *= silu_f(own_in(buf, 2));
        reinterpret_cast<elem*>(&sm.out[buf][k][0])[cl] = IO::from_float(y);
      }
      hold_store();
      if (has_next) stage_chunk(buf ^ 1, ci + 1);
      __syncthreads();
      store_out(buf, ci);
      buf ^= 1;
    }
    __builtin_amdgcn_s_setprio(0);

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

  // One recurrence step (TAU of the chunk) for this lane's states.  bcv holds the chunk's
  // (B, C) pairs for this lane's states, two steps per float4.
  template <int TAU>
  static __device__ __forceinline__ void step(Smem& sm, const float4 (&bcv)[NL][kT / 2],
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
                                               const float4 (&bcv)[NL][kT / 2], float dt,
                                               float du, const float (&A2)[NL], float (&h)[NL],
                                               int wave, int r, int k) {
    (step<TAUS>(sm, bcv, dt, du, A2, h, wave, r, k), ...);
  }

  // The 16 recurrence steps of one chunk.  The B/C tile reads are issued together up front
  // (16-byte reads, two steps each) so that the steps themselves are pure VALU work.
  static __device__ __forceinline__ void chunk_steps(Smem& sm, int buf, float dt, float du,
                                                     const float (&A2)[NL], float (&h)[NL],
                                                     int wave, int r, int k) {
    float4 bcv[NL][kT / 2];
#pragma unroll
    for (int j = 0; j < NL; ++j)
#pragma unroll
      for (int i = 0; i < kT / 2; ++i)
        bcv[j][i] = *reinterpret_cast<const float4*>(&sm.bc[buf][k + 16 * j][2 * i]);
    steps(std::make_integer_sequence<int, kT>{}, sm, bcv, dt, du, A2, h, wave, r, k);
  }
};

template <class IO, int NL, bool GATE, bool SUMMARY, bool VEC>
__global__ void __launch_bounds__(kPrefillThreads) scan_kernel(ScanArgs a) {
  ScanKernel<IO, NL, GATE, SUMMARY, VEC>::run(a);
}

__global__ void __launch_bounds__(256) copy_state_kernel(float* dst, const float* src, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src ? src[i] : 0.0f;
}

template <class IO, int NL, bool VEC>
hipError_t launch3(const ScanArgs& a, bool summary, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.n_wg)), block(kPrefillThreads);
  if (summary)
    hipLaunchKernelGGL((scan_kernel<IO, NL, false, true, VEC>), grid, block, 0, stream, a);
  else if (a.z != nullptr)
    hipLaunchKernelGGL((scan_kernel<IO, NL, true, false, VEC>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((scan_kernel<IO, NL, false, false, VEC>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <class IO, int NL>
hipError_t launch2(const ScanArgs& a, bool summary, hipStream_t stream) {
  return a.vec_io ? launch3<IO, NL, true>(a, summary, stream)
                  : launch3<IO, NL, false>(a, summary, stream);
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
