// ss_scan_bwd.hip -- gfx950 backward of the prefill scan (first-order input term dt B u).
//
// Gradients by reverse-mode differentiation of the recurrence (Mamba reading guide, "Método":
// h_t = exp(dt_t A) h_{t-1} + dt_t B_t u_t, y_t = C_t h_t; IBM explainer: D term and gate), with
// the states recomputed instead of stored (reading guide, "Expansão de Estado Ciente de
// Hardware": intermediate states are recomputed in the backward pass).  For one channel and
// state n, with e_t = exp(dt_t a_n) and gy_t = dout_t silu(z_t):
//     lam_t   = gy_t C_t + e_{t+1} lam_{t+1}                  (adjoint of h_t, run backwards)
//     ddt_t   = sum_n lam_t (a_n e_t h_{t-1} + B_t u_t),  du_t = gy_t D + dt_t sum_n lam_t B_t
//     dB_t   += lam_t dt_t u_t,  dC_t += gy_t h_t             (summed over channels)
//     dA     += lam_t dt_t e_t h_{t-1},  dD += gy_t u_t,  dz_t = dout_t y_t silu'(z_t)
//     ddelta_t = ddt_t sigmoid(delta_t + bias) (softplus'),  dbias += ddelta_t,  dh0 = e_0 lam_0.
//
// Work layout (as in the forward kernel): one channel per 16-lane DPP row, lane k owns state k
// and the element work of step k of each 16-step chunk; 16 channels per 256-thread workgroup,
// one workgroup per (16 channels, batch row); the next chunk's global loads are in flight while a
// chunk is computed (LDS tiles double-buffered).  The kernel starts from the chunk-end states in
// the workspace (4 d_state bytes per channel and chunk), saved by the caller's forward
// (ss_scan_fwd_states) or, before this launch, by the prefill kernel's states-only pass.  It
// walks the chunks backwards: it recomputes the chunk's 16 states and decays from the stored
// state into registers, computes y for the gate's derivative, then runs the adjoint backwards
// through the 16 steps.  Sums over a channel's states go through per-wave LDS tiles (summed by
// the owner lane of the step, as in the forward); sums over channels (dB, dC) are reduced over
// row pairs by a row swap (dB and dC in one swap) and over the eight pairs in LDS, then added to
// global memory with one atomic per (step, state) and workgroup; dA, dD and dbias likewise once
// per workgroup.  The atomic sums make dA, dB, dC, dD and dbias reproducible only up to rounding
// order.  u/delta/z/dout tiles move as 16-byte pieces when the channel blocks are whole, with
// the pieces of each tile row permuted by step against LDS bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "ss_bwd.h"
#include "ss_device.h"

namespace ss {
namespace {

constexpr int kT = kBwdChunk;

// Sums over the row pairs (0, 1) and (2, 3) of the wave of two quantities at once: x in rows 0
// and 2 of the result, y in rows 1 and 3.  v_permlane16_swap exchanges the odd rows of its first
// operand with the even rows of its second, leaving (x0, y0, x2, y2) and (x1, y1, x3, y3).
__device__ __forceinline__ float sum_row_pairs2(float x, float y) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                  false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Partial tiles: channel row r at r * kPRow, step slot s at s * kPTau, lane k at k; odd rows keep
// step t in slot t ^ kPSwap.  With this layout the owners' 16-byte reads and the paired 4-byte
// writes of two steps are both free of LDS bank conflicts on gfx950 (measured with the
// bank-conflict counter; rows 336 floats apart conflict on the reads, rows 320 apart without the
// swap on the writes).
constexpr int kPRow = 320;  // floats per channel row of a partial tile
constexpr int kPTau = 20;   // floats per step slot of a partial tile (padding)
constexpr int kPSwap = 12;  // odd rows: step t in slot t ^ kPSwap
// Offset of step TAU's slot from slot TAU, for a row of parity ODD.
template <int TAU>
__device__ __forceinline__ int pslot_shift(int odd) {
  return ((TAU ^ kPSwap) - TAU) * kPTau * odd;
}
// Once the owner lanes of a wave have read their sums, the wave's partial tiles hold its dB and dC
// tiles: per row pair (rows 0-1, 2-3) kBwdChunk steps x 16 states, dB at pair * 256 and dC
// kGcOff further (16 floats past a multiple of 32, so that rows 0 and 1, which write dB and dC
// with one instruction, use different LDS banks).  Sharing the space keeps the workgroup at
// 49.7 KB of LDS: three workgroups per CU.
constexpr int kGcOff = 2 * kBwdChunk * 16 + 16;

template <class IO, bool GATE, bool VEC>
struct BwdKernel {
  using elem = typename IO::elem;
  static constexpr int ES = sizeof(elem);
  static constexpr int PIECE_E = 16 / ES;        // elements per 16-byte piece
  static constexpr int PIECES = 16 / PIECE_E;    // pieces per 16-channel tile row
  // The 16-byte pieces of row (step) k of an input tile are stored XOR-permuted by
  // (k / (8 / PIECES)) mod PIECES, so that the owner lanes of steps 4 (bf16) or 2 (fp32) apart
  // do not read the same LDS banks (32 banks of 4 bytes; rows are 32 or 64 bytes).
  static __device__ __forceinline__ int pswz(int row) {
    return (row / (8 / PIECES)) & (PIECES - 1);
  }

  struct alignas(16) Smem {
    float2 bc[2][16][kT + 2];       // (B_t[n], C_t[n]) of the chunk, double-buffered
    elem in[2][4][kT][16];          // u, delta, z, dout tiles [buf][tensor][step][channel]
    // per wave: partial sums over states, p (y, then ddt) at 0 and q (du) at 4 * kPRow; after
    // the owner sums, the dB and dC tiles of the wave's row pairs
    float pq[4][2 * 4 * kPRow];
  };
  static_assert(kGcOff + 2 * kT * 16 <= 2 * 4 * kPRow, "dB/dC tiles inside the partial tiles");

  static __device__ __forceinline__ void run(const BwdArgs& a) {
    __shared__ Smem sm;
    const int64_t b = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x / a.n_cblk));
    const int64_t d0 = __builtin_amdgcn_readfirstlane(
        static_cast<int>((blockIdx.x - b * a.n_cblk) * 16));
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int r = lane >> 4, k = lane & 15;
    const int cl = wave * 4 + r;
    const int64_t D = a.d_inner, N = a.d_state, L = a.seqlen;
    const int64_t d = d0 + cl;
    const bool chan_ok = d < D;
    const bool lane_ok = chan_ok && k < N;
    const int64_t row = b * D + d;
    const int nchunks = static_cast<int>((L + kT - 1) / kT);
    const int last_valid = static_cast<int>(L - int64_t(nchunks - 1) * kT);
    auto nvalid_of = [&](int c) { return c == nchunks - 1 ? last_valid : kT; };

    const float a_n = lane_ok ? a.A[d * N + k] : 0.0f;
    const float A2 = a_n * kLog2e;
    const float bias = (chan_ok && a.delta_bias) ? a.delta_bias[d] : 0.0f;
    const float dskip = (chan_ok && a.D) ? a.D[d] : 0.0f;
    const int64_t row0 = b * L;  // (b, 0) row of u/delta/z/dout and of B/C

    // ---- tile loads: wave w loads tensor w of (u, delta, z, dout), element by element through
    // a raw buffer sized to the chunk's valid steps (loads past the end read 0; channels past
    // d_inner read the next row or 0 and are not used); every thread loads one (step, state) of
    // B and C.
    const void* tens[4] = {a.u, a.delta, a.z, a.dout};
    const int tl_row = lane / PIECES, tl_pc = lane % PIECES;
    const bool tl_on = lane < kT * PIECES;
    const uint32_t tl_off =
        tl_on ? static_cast<uint32_t>((tl_row * D + tl_pc * PIECE_E) * ES) : kOffNone;
    const int bc_tau = tid >> 4, bc_n = tid & 15;
    const uint32_t bc_off = bc_n < N ? static_cast<uint32_t>((bc_tau * N + bc_n) * ES) : kOffNone;

    // Global loads of chunk c go to registers (issued before the current chunk is computed) and
    // are written to LDS buffer `buf` after it.
    elem pv[PIECE_E];
    uint4 pvv{0, 0, 0, 0};
    float pbv = 0.0f, pcv = 0.0f;
    auto issue = [&](int c) {
      const int nv = nvalid_of(c);
      const int64_t t0 = int64_t(c) * kT;
      const uint32_t io_bytes = static_cast<uint32_t>((nv * D - d0) * ES);
      if (GATE || wave_u != 2) {  // uniform: z only with the gate
        const rsrc_t rt = make_buf(
            static_cast<const char*>(tens[wave_u]) + ((row0 + t0) * D + d0) * ES, io_bytes);
        if (VEC) {
          pvv = buf_load<uint4>(rt, tl_off);
        } else {
#pragma unroll
          for (int e = 0; e < PIECE_E; ++e) pv[e] = buf_load<elem>(rt, tl_off + e * ES);
        }
      }
      const uint32_t bc_bytes = static_cast<uint32_t>(nv * N * ES);
      const rsrc_t rb = make_buf(static_cast<const char*>(a.B) + (row0 + t0) * N * ES, bc_bytes);
      pbv = IO::widen(buf_load<elem>(rb, bc_off));
      const rsrc_t rc = make_buf(static_cast<const char*>(a.C) + (row0 + t0) * N * ES, bc_bytes);
      pcv = IO::widen(buf_load<elem>(rc, bc_off));
    };
    auto stage = [&](int buf) {
      if ((GATE || wave_u != 2) && tl_on) {
        elem* dst = &sm.in[buf][wave_u][tl_row][(tl_pc ^ pswz(tl_row)) * PIECE_E];
        if (VEC) {
          *reinterpret_cast<uint4*>(dst) = pvv;
        } else {
#pragma unroll
          for (int e = 0; e < PIECE_E; ++e) dst[e] = pv[e];
        }
      }
      sm.bc[buf][bc_n][bc_tau] = make_float2(pbv, pcv);
    };
    const int own_col = ((cl / PIECE_E) ^ pswz(k)) * PIECE_E + cl % PIECE_E;
    auto own = [&](int buf, int ten) -> float { return IO::widen(sm.in[buf][ten][k][own_col]); };

    // chunk-end states, (batch, chunk, d_inner, d_state): the wave's four channels of a chunk are
    // 256 contiguous bytes
    const float* ck_lane = a.ck + ((b * nchunks) * D + d) * N + k;
    const int64_t ck_chunk = D * N;
    int buf = 0;
    if (nchunks > 0) {  // the last chunk first
      issue(nchunks - 1);
      stage(0);
      __syncthreads();
    }

    // ---- pass 2: chunks backwards
    float lam = (a.dh_last && lane_ok) ? a.dh_last[row * N + k] : 0.0f;
    float e_next = 1.0f;
    float ga = 0.0f, gd_acc = 0.0f, gb_acc = 0.0f;
    for (int c = nchunks - 1; c >= 0; --c) {
      if (c > 0) issue(c - 1);
      const int nv = nvalid_of(c);
      const bool own_ok = chan_ok && k < nv;
      const float xu = own(buf, 0);
      const float sv = own(buf, 1) + bias;
      float dt = a.softplus ? softplus_f(sv) : sv;
      dt = own_ok ? dt : 0.0f;
      const float du = own_ok ? dt * xu : 0.0f;
      float hprev;
      if (c > 0) hprev = lane_ok ? ck_lane[int64_t(c - 1) * ck_chunk] : 0.0f;
      else hprev = (a.h0 && lane_ok) ? a.h0[row * N + k] : 0.0f;

      float4 bcv[kT / 2];
#pragma unroll
      for (int i = 0; i < kT / 2; ++i)
        bcv[i] = *reinterpret_cast<const float4*>(&sm.bc[buf][k][2 * i]);
      // recompute the chunk: states, decays and the partial sums C.h of y
      float hh[kT], ee[kT];
      float* pw = &sm.pq[wave][r * kPRow + k];
      rec_steps(std::make_integer_sequence<int, kT>{}, bcv, dt, du, A2, hprev, hh, ee, pw, r & 1);
      wave_lds_sync();
      float y = 0.0f;
      {
        const float* pr = &sm.pq[wave][r * kPRow + (k ^ (kPSwap * (r & 1))) * kPTau];
#pragma unroll
        for (int i = 0; i < 16; ++i) y += pr[i];
      }
      wave_lds_sync();
      y = fmaf(dskip, xu, y);
      const float g = own_ok ? own(buf, 3) : 0.0f;
      float gy = g, gz = 0.0f;
      if (GATE) {
        const float zv = own(buf, 2);
        const float sg = rcp_hw(1.0f + exp2_hw(-zv * kLog2e));
        gy = g * zv * sg;
        gz = g * y * sg * fmaf(zv, 1.0f - sg, 1.0f);
      }
      gd_acc = fmaf(gy, xu, gd_acc);

      // the adjoint backwards through the chunk
      float* qw = &sm.pq[wave][4 * kPRow + r * kPRow + k];
      float* gbc_w = &sm.pq[wave][(r & 1) * kGcOff + (r >> 1) * kT * 16];
      float xb[kT], yc[kT];
      rev_steps(std::make_integer_sequence<int, kT>{}, bcv, dt, du, xu, gy, a_n, hprev, hh, ee,
                lam, e_next, ga, pw, qw, xb, yc, r & 1);
      // dB and dC of each step, summed over channel pairs (independent of one another, so the
      // row swaps of different steps overlap); stored below, over the partial tiles
      float gpair[kT];
#pragma unroll
      for (int t = 0; t < kT; ++t) gpair[t] = sum_row_pairs2(xb[t], yc[t]);
      wave_lds_sync();
      float gdt = 0.0f, gx = 0.0f;
      {
        const int own_slot = r * kPRow + (k ^ (kPSwap * (r & 1))) * kPTau;
        const float* pr = &sm.pq[wave][own_slot];
        const float* qr = &sm.pq[wave][4 * kPRow + own_slot];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          gdt += pr[i];
          gx += qr[i];
        }
        gdt = fmaf(xu, gx, gdt);  // + u_t sum_n lam B, the input term of ddt
      }
      wave_lds_sync();  // every lane of the wave has its sums: the tiles take dB and dC
#pragma unroll
      for (int t = 0; t < kT; ++t) gbc_w[t * 16 + k] = gpair[t];
      // the next chunk's tiles first: its wait for the loads would also wait for the stores below
      if (c > 0) stage(buf ^ 1);
      if (own_ok) {
        const float gdelta = a.softplus ? gdt * rcp_hw(1.0f + exp2_hw(-sv * kLog2e)) : gdt;
        gb_acc += gdelta;
        const int64_t e = (row0 + int64_t(c) * kT + k) * D + d;
        static_cast<elem*>(a.du)[e] = IO::from_float(fmaf(gx, dt, gy * dskip));
        static_cast<elem*>(a.ddelta)[e] = IO::from_float(gdelta);
        if (GATE) static_cast<elem*>(a.dz)[e] = IO::from_float(gz);
      }
      __syncthreads();  // the wave tiles of dB and dC, and the next chunk's tiles, are complete
      {
        const int tau = tid >> 4, n = tid & 15;
        float sb = 0.0f, sc = 0.0f;
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {
          sb += sm.pq[pr >> 1][((pr & 1) * kT + tau) * 16 + n];
          sc += sm.pq[pr >> 1][kGcOff + ((pr & 1) * kT + tau) * 16 + n];
        }
        if (tau < nv && n < N) {
          const int64_t o = (row0 + int64_t(c) * kT + tau) * N + n;
          atomicAdd(a.dB + o, sb);
          atomicAdd(a.dC + o, sc);
        }
      }
      __syncthreads();  // the dB and dC tiles are rewritten by the next chunk
      buf ^= 1;
    }
    if (lane_ok) {
      atomicAdd(a.dA + d * N + k, ga);
      if (a.dh0) a.dh0[row * N + k] = e_next * lam;
    }
    // sums over the row's 16 owner lanes
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      gd_acc += __shfl_xor(gd_acc, m, 16);
      gb_acc += __shfl_xor(gb_acc, m, 16);
    }
    if (chan_ok && k == 0) {
      if (a.dD) atomicAdd(a.dD + d, gd_acc);
      if (a.ddelta_bias) atomicAdd(a.ddelta_bias + d, gb_acc);
    }
  }

  // Recompute step: keep the state and the decay of every step, and the partial sum C.h.
  template <int TAU>
  static __device__ __forceinline__ void rec_step(const float4 (&bcv)[kT / 2], float dt, float du,
                                                  float A2, float& h, float (&hh)[kT],
                                                  float (&ee)[kT], float* pw, int odd) {
    const float4 v = bcv[TAU / 2];
    const float bb = (TAU & 1) ? v.z : v.x;
    const float cc = (TAU & 1) ? v.w : v.y;
    const float e = exp2_hw(row_bcast<TAU>(dt) * A2);
    h = fmaf(e, h, row_bcast<TAU>(du) * bb);
    hh[TAU] = h;
    ee[TAU] = e;
    pw[TAU * kPTau + pslot_shift<TAU>(odd)] = cc * h;
  }
  template <int... TAUS>
  static __device__ __forceinline__ void rec_steps(std::integer_sequence<int, TAUS...>,
                                                   const float4 (&bcv)[kT / 2], float dt,
                                                   float du, float A2, float hprev,
                                                   float (&hh)[kT], float (&ee)[kT], float* pw,
                                                   int odd) {
    float h = hprev;
    (rec_step<TAUS>(bcv, dt, du, A2, h, hh, ee, pw, odd), ...);
  }

  // Adjoint step TAU (taken in decreasing TAU): lam <- gy C + e_next lam, then the step's
  // contributions.  Partial sums over states go to the wave tiles pw (the A e h_prev part of ddt)
  // and qw (lam B, which gives du and the u B part of ddt); dB and dC are summed over each pair of
  // the wave's channels (rows) after the chain (xb, yc), rows 0 and 2 storing dB and rows 1
  // and 3 dC.
  template <int TAU>
  static __device__ __forceinline__ void rev_step(const float4 (&bcv)[kT / 2], float dt, float du,
                                                  float xu, float gy, float a_n, float hprev,
                                                  const float (&hh)[kT], const float (&ee)[kT],
                                                  float& lam, float& e_next, float& ga, float* pw,
                                                  float* qw, float (&xb)[kT], float (&yc)[kT],
                                                  int odd) {
    const float4 v = bcv[TAU / 2];
    const float bb = (TAU & 1) ? v.z : v.x;
    const float cc = (TAU & 1) ? v.w : v.y;
    const float gyb = row_bcast<TAU>(gy);
    lam = fmaf(e_next, lam, gyb * cc);
    const float hp = TAU > 0 ? hh[TAU > 0 ? TAU - 1 : 0] : hprev;
    const float rr = lam * ee[TAU] * hp;
    ga = fmaf(row_bcast<TAU>(dt), rr, ga);
    const float qq = lam * bb;
    pw[TAU * kPTau + pslot_shift<TAU>(odd)] = a_n * rr;
    qw[TAU * kPTau + pslot_shift<TAU>(odd)] = qq;
    xb[TAU] = lam * row_bcast<TAU>(du);  // this channel's dB and dC terms, summed over
    yc[TAU] = gyb * hh[TAU];             // channel pairs after the chain
    e_next = ee[TAU];
  }
  template <int... TAUS>
  static __device__ __forceinline__ void rev_steps(std::integer_sequence<int, TAUS...>,
                                                   const float4 (&bcv)[kT / 2], float dt,
                                                   float du, float xu, float gy, float a_n,
                                                   float hprev, const float (&hh)[kT],
                                                   const float (&ee)[kT], float& lam,
                                                   float& e_next, float& ga, float* pw, float* qw,
                                                   float (&xb)[kT], float (&yc)[kT], int odd) {
    // fold over the steps in decreasing order
    (rev_step<kT - 1 - TAUS>(bcv, dt, du, xu, gy, a_n, hprev, hh, ee, lam, e_next, ga, pw, qw,
                             xb, yc, odd),
     ...);
  }
};

template <class IO, bool GATE, bool VEC>
__global__ void __launch_bounds__(kBwdThreads) scan_bwd_kernel(BwdArgs a) {
  BwdKernel<IO, GATE, VEC>::run(a);
}

__global__ void __launch_bounds__(256) zero_kernel(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    p[i] = 0.0f;
}

hipError_t zero(float* p, int64_t n, hipStream_t stream) {
  if (!p || n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256 < 2048 ? (n + 255) / 256 : 2048;
  hipLaunchKernelGGL(zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p,
                     n);
  return hipGetLastError();
}

template <class IO>
void launch_io(const BwdArgs& a, hipStream_t stream) {
  if (a.batch * a.n_cblk == 0) return;  // nothing but the zeroed sums
  const dim3 grid(static_cast<unsigned>(a.batch * a.n_cblk)), block(kBwdThreads);
  if (a.vec_io) {
    if (a.z)
      hipLaunchKernelGGL((scan_bwd_kernel<IO, true, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((scan_bwd_kernel<IO, false, true>), grid, block, 0, stream, a);
  } else {
    if (a.z)
      hipLaunchKernelGGL((scan_bwd_kernel<IO, true, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((scan_bwd_kernel<IO, false, false>), grid, block, 0, stream, a);
  }
}

}  // namespace

hipError_t launch_scan_bwd(const BwdArgs& a, bool bf16, hipStream_t stream) {
  const int64_t N = a.d_state;
  hipError_t e;
  if ((e = zero(a.dA, a.d_inner * N, stream)) != hipSuccess) return e;
  if ((e = zero(a.dB, a.batch * a.seqlen * N, stream)) != hipSuccess) return e;
  if ((e = zero(a.dC, a.batch * a.seqlen * N, stream)) != hipSuccess) return e;
  if ((e = zero(a.dD, a.d_inner, stream)) != hipSuccess) return e;
  if ((e = zero(a.ddelta_bias, a.d_inner, stream)) != hipSuccess) return e;
  if (bf16) launch_io<BF16>(a, stream);
  else launch_io<F32>(a, stream);
  return hipGetLastError();
}

}  // namespace ss
