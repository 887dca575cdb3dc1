// ss_scan2_mfma.hip -- the multi-head scalar-transition scan (ss_scan2.hip states the
// recurrence) in its chunked dual form on the gfx950 matrix cores.
//
// With one decay per (token, head) the recurrence over a chunk of Q steps starting from state
// S_in is a set of dense products (the quadratic "dual" form: IBM explainer, Mamba-2 and its
// link between state-space models and attention; Cartesia Mamba-3 post, the scalar transition).
// With a_t = dt_t A (log decay) and c_t = a_0 + ... + a_t inside the chunk:
//     Y      = (L o (C B^T)) diag(dt) X  +  diag(e^{c}) C S_in       (L[t,s] = e^{c_t - c_s}, s <= t)
//     S_out  = e^{c_{Q-1}} S_in  +  B^T diag(w) X,   w_s = dt_s e^{c_{Q-1} - c_s}
// (rows of X, Y: steps; columns: head channels p; S: d_state x headdim).  All four products run
// as v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  x, B and C are bf16 inputs and enter the
// products exactly; the three fp32 operands (the masked decayed C B^T, the state S_in and the
// weighted w o X) are split into bf16 high and low parts, v = hi + lo to about 16 significant
// bits, and each takes two products, so the result keeps close to fp32 accuracy.
//
// Work layout: one workgroup (4 waves) per (batch row, head) walks the chunks in order and keeps
// the state in registers; wave w owns head channels 16w..16w+15 (one 16-column tile of S, X and
// Y), so the state never leaves the wave.  The 10 causal 16x16 tiles of C B^T are shared: each
// wave computes some of them, applies the mask and decays, and writes the split products to LDS.
// Per chunk the workgroup stages B (row-major and transposed), C and x (transposed) in LDS from
// 16-byte / 8-byte global loads issued one chunk ahead; each wave transposes its own z tile into
// LDS once the B tile is free, and writes its outputs through an LDS tile as 16-byte stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_device.h"
#include "ss_scan2.h"

namespace ss {
namespace {

using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using f32x4 = float __attribute__((ext_vector_type(4)));

constexpr int kQ = kScan2MfmaChunk;  // chunk length = wave width
constexpr int kP = 64;               // head channels (headdim) handled by the workgroup
constexpr int kTP = kQ + 8;          // bf16 per row of the (p, s) and (t, s) tiles

struct Op {  // one MFMA operand: 8 bf16 in 4 dwords
  uint32_t w[4];
};

__device__ __forceinline__ f32x4 mfma(const Op& a, const Op& b, f32x4 c) {
  using u4 = uint32_t __attribute__((ext_vector_type(4)));
  const u4 av = {a.w[0], a.w[1], a.w[2], a.w[3]};
  const u4 bv = {b.w[0], b.w[1], b.w[2], b.w[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                 __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
}

// Two floats to two bf16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  using b2 = __bf16 __attribute__((ext_vector_type(2)));
  const b2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float lo_f(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_f(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Split (a, b) into high and low bf16 pairs: a = hi + lo to about 2^-17 relative.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - lo_f(hi), b - hi_f(hi));
}

// The low 16 bits of a and of b, as (a_lo, b_lo); the high halves, as (a_hi, b_hi).
__device__ __forceinline__ uint32_t lows(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t highs(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// LDS of one workgroup: 80 KB at d_state 128, so that two workgroups share a CU.  Two regions
// are reused within a chunk: once every wave is past the C B^T tiles and the state update, the
// B tile holds each wave's z tile (p, t); and once a wave has read its x for the epilogue, its
// own 16 rows of the x tile hold its output tile (t, p).
// Column of element s in row r of a transposed tile ((p, s) for x, (n, s) for B): the eight
// 16-byte groups of a row are XOR-permuted by (r / 8) mod 8.  The transposed stores write rows
// 4 or 8 apart from neighbouring lanes, which would otherwise land on the same LDS banks; the
// MFMA operand reads (16 bytes of 8 consecutive s) stay contiguous and conflict-free.
__device__ __forceinline__ int swz(int r, int s) {
  return (((s >> 3) ^ ((r >> 3) & 7)) << 3) | (s & 7);
}

template <int N>
struct alignas(16) Smem2 {
  uint16_t b[kQ][N + 8];        // B of the chunk, (s, n); later: per-wave z tiles
  uint16_t bt[N][kTP];          // B transposed, (n, s) (swizzled)
  uint16_t c[kQ][N + 8];        // C, (t, n)
  uint16_t xt[kP][kTP];         // x transposed, (p, s) (swizzled); later: per-wave output tiles
  uint16_t mhi[kQ][kTP];        // masked, decayed and dt-scaled C B^T, (t, s): high part
  uint16_t mlo[kQ][kTP];        // low part
  float ac[kQ];                 // c_t, the chunk's cumulative log2 decay
  float dtv[kQ];                // dt_t (0 past the sequence end)
  float e[kQ];                  // 2^{c_t}
  float w[kQ];                  // dt_t 2^{c_{Q-1} - c_t}
};

// Inclusive prefix sum over the 64 lanes of the wave: Hillis-Steele steps inside each 16-lane
// row by DPP row shifts (lanes shifted in from outside the row read 0), then the totals of the
// rows below added from scalar lane reads.
__device__ __forceinline__ float wave_prefix_sum(float x, int lane) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  const int row = lane >> 4;
  const float below = row == 0 ? 0.0f : row == 1 ? r0 : row == 2 ? r0 + r1 : (r0 + r1) + r2;
  return x + below;
}

template <int N, bool GATE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
scan2_mfma_kernel(Scan2Args a) {
  constexpr int NT = N / 16;         // 16-row tiles of the state
  constexpr int KB = N / 32;         // 32-wide K blocks over the states
  constexpr int UNITS = 2 * N;       // (4-row, 8-state) pieces of a B or C tile
  constexpr int UPT = (UNITS + 255) / 256;
  static_assert(N % 32 == 0 && N <= 128, "state tile");
  __shared__ Smem2<N> sm;

  const int tid = threadIdx.x;
  const int wv = tid >> 6, l = tid & 63, l16 = l & 15, g4 = l >> 4;
  const int64_t H = a.nheads, L = a.seqlen, G = a.ngroups;
  const int64_t bh = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = bh / H, h = bh - b * H;
  const int64_t grp = h / (H / G);
  const float A2 = a.A[h] * kLog2e;
  const float Dh = a.D ? a.D[h] : 0.0f;
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;

  // Byte strides between consecutive steps.
  const uint32_t xrow = static_cast<uint32_t>(H * kP * 2);
  const uint32_t bcrow = static_cast<uint32_t>(G * N * 2);
  const uint32_t dtrow = static_cast<uint32_t>(H * 2);
  const uint16_t* xg = static_cast<const uint16_t*>(a.x) + (b * L * H + h) * kP;
  const uint16_t* zg = GATE ? static_cast<const uint16_t*>(a.z) + (b * L * H + h) * kP : nullptr;
  uint16_t* og = static_cast<uint16_t*>(a.out) + (b * L * H + h) * kP;
  const uint16_t* dtg = static_cast<const uint16_t*>(a.dt) + b * L * H + h;
  const uint16_t* bg = static_cast<const uint16_t*>(a.B) + (b * L * G + grp) * N;
  const uint16_t* cg = static_cast<const uint16_t*>(a.C) + (b * L * G + grp) * N;

  // Staging roles.  x and z: 4 rows x 4 channels per thread; B and C: 4 rows x 8 states per unit.
  const int xq = tid >> 4, xp = tid & 15;
  uint32_t xoff[4], zoff[4], boff[UPT][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    xoff[r] = (4 * xq + r) * xrow + 8 * xp;
    // z: each wave loads its own 16 channels, 4 steps x 4 channels per lane
    zoff[r] = (4 * (l >> 2) + r) * xrow + (16 * wv + 4 * (l & 3)) * 2;
  }
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u = tid + 256 * k;
    const int rq = u / (N / 8), nb = u % (N / 8);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      boff[k][r] = u < UNITS ? (4 * rq + r) * bcrow + 16 * nb : kOffNone;
  }

  uint2 xr[4], zr[4];
  uint4 br[UPT][4], cr[UPT][4];
  uint16_t dtr;
  // Loads of the chunk at t0 into registers.  Each tile is a buffer over the chunk's valid steps
  // (none past the sequence end: then every load returns 0 and touches no memory).
  auto fetch = [&](int64_t t0) {
    const int64_t left = L - t0;
    const uint32_t nv = static_cast<uint32_t>(left <= 0 ? 0 : left < kQ ? left : kQ);
    auto bytes = [nv](uint32_t row, uint32_t last) { return nv ? (nv - 1) * row + last : 0u; };
    const rsrc_t rx = make_buf(xg + t0 * H * kP, bytes(xrow, kP * 2));
    const rsrc_t rb = make_buf(bg + t0 * G * N, bytes(bcrow, N * 2));
    const rsrc_t rc = make_buf(cg + t0 * G * N, bytes(bcrow, N * 2));
    const rsrc_t rd = make_buf(dtg + t0 * H, bytes(dtrow, 2));
    dtr = buf_load<uint16_t>(rd, l * dtrow);  // first: it is the first value the chunk needs
#pragma unroll
    for (int r = 0; r < 4; ++r) xr[r] = buf_load<uint2>(rx, xoff[r]);
#pragma unroll
    for (int k = 0; k < UPT; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        br[k][r] = buf_load<uint4>(rb, boff[k][r]);
        cr[k][r] = buf_load<uint4>(rc, boff[k][r]);
      }
  };

  // State tile of this wave: S[nt][r] = state (n = 16 nt + 4 g4 + r, p = 16 wv + l16).
  f32x4 S[NT];
  const int p = 16 * wv + l16;
  if (a.h0) {
    const float* h0 = a.h0 + bh * N * kP;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[nt][r] = h0[(16 * nt + 4 * g4 + r) * kP + p];
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) S[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Tiles of C B^T above the diagonal blocks are never written: zero them once.
  {
    uint4* m = reinterpret_cast<uint4*>(&sm.mhi[0][0]);
    constexpr int n16 = 2 * kQ * kTP * 2 / 16;
    for (int i = tid; i < n16; i += 256) m[i] = make_uint4(0, 0, 0, 0);
  }

  // z of the chunk at t0: needed only by that chunk's epilogue, so it is loaded at the chunk's
  // start (as far ahead as the next chunk's other inputs).
  auto fetch_z = [&](int64_t t0) {
    if (GATE) {
      const int64_t left = L - t0;
      const uint32_t nv = static_cast<uint32_t>(left < kQ ? left : kQ);
      const rsrc_t rz = make_buf(zg + t0 * H * kP, (nv - 1) * xrow + kP * 2);
#pragma unroll
      for (int r = 0; r < 4; ++r) zr[r] = buf_load<uint2>(rz, zoff[r]);
    }
  };

  // Output tile of the previous chunk, stored at the start of the next one: stores issued right
  // after the next chunk's loads would make the wait for those loads wait for the stores too.
  uint4 pend[2];
  rsrc_t pend_r = make_buf(og, 0);
  auto store_pending = [&]() {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int t = 32 * it + (l >> 1), piece = l & 1;
      buf_store(pend[it], pend_r, t * xrow + (16 * wv + 8 * piece) * 2);
    }
  };

  const int64_t nchunks = (L + kQ - 1) / kQ;
  fetch(0);
  for (int64_t ch = 0; ch < nchunks; ++ch) {
    const int64_t t0 = ch * kQ;
    const int nv = static_cast<int>(L - t0 < kQ ? L - t0 : kQ);
    __syncthreads();  // the previous chunk's LDS reads are done
    // ---- stage the chunk in LDS
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {  // x transposed: (p, 4 consecutive steps) per write
      const int w = cc >> 1;
      uint32_t r4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) r4[r] = w == 0 ? xr[r].x : xr[r].y;
      const uint2 v = (cc & 1) ? make_uint2(highs(r4[0], r4[1]), highs(r4[2], r4[3]))
                               : make_uint2(lows(r4[0], r4[1]), lows(r4[2], r4[3]));
      *reinterpret_cast<uint2*>(&sm.xt[4 * xp + cc][swz(4 * xp + cc, 4 * xq)]) = v;
    }
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = tid + 256 * k;
      if (UNITS % 256 == 0 || u < UNITS) {
        const int rq = u / (N / 8), nb = u % (N / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *reinterpret_cast<uint4*>(&sm.b[4 * rq + r][8 * nb]) = br[k][r];
          *reinterpret_cast<uint4*>(&sm.c[4 * rq + r][8 * nb]) = cr[k][r];
        }
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          uint32_t r4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint4 q = br[k][r];
            r4[r] = (cc >> 1) == 0 ? q.x : (cc >> 1) == 1 ? q.y : (cc >> 1) == 2 ? q.z : q.w;
          }
          const uint2 v = (cc & 1) ? make_uint2(highs(r4[0], r4[1]), highs(r4[2], r4[3]))
                                   : make_uint2(lows(r4[0], r4[1]), lows(r4[2], r4[3]));
          *reinterpret_cast<uint2*>(&sm.bt[8 * nb + cc][swz(8 * nb + cc, 4 * rq)]) = v;
        }
      }
    }
    // ---- step sizes and decays of the chunk (every wave keeps its own copy)
    float acEnd;
    {
      const float s = BF16::widen(dtr) + bias;
      float dv = a.softplus ? softplus_f(s) : s;
      dv = l < nv ? dv : 0.0f;
      const float c = wave_prefix_sum(dv * A2, l);
      acEnd = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
      if (wv == 0) {  // every wave has the same values; one copy in LDS
        sm.ac[l] = c;
        sm.dtv[l] = dv;
        sm.e[l] = exp2_hw(c);
        sm.w[l] = exp2_hw(acEnd - c) * dv;
      }
    }
    if (ch > 0) store_pending();
    fetch(t0 + kQ);  // past the end on the last chunk: no memory is touched
    fetch_z(t0);
    __syncthreads();  // staged tiles visible

    // ---- the causal tiles of C B^T owned by this wave -> masked, decayed, split, to LDS.  The
    // 10 tiles (s-tile ti <= t-tile tj) in the order (0,0) (0,1) (1,1) (0,2) ... (3,3) are dealt
    // to the waves round-robin (3, 3, 2, 2 tiles).
    for (int k = wv; k < 10; k += 4) {
      const int tj = (k >= 1) + (k >= 3) + (k >= 6);
      const int ti = k - tj * (tj + 1) / 2;
      f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const Op ab = *reinterpret_cast<const Op*>(&sm.b[16 * ti + l16][32 * kb + 8 * g4]);
        const Op bc = *reinterpret_cast<const Op*>(&sm.c[16 * tj + l16][32 * kb + 8 * g4]);
        g = mfma(ab, bc, g);  // g[r] = sum_n B[s, n] C[t, n], s = 16 ti + 4 g4 + r, t = 16 tj + l16
      }
      const int t = 16 * tj + l16, s0 = 16 * ti + 4 * g4;
      const float act = sm.ac[t];
      const float4 acs = *reinterpret_cast<const float4*>(&sm.ac[s0]);
      const float4 dts = *reinterpret_cast<const float4*>(&sm.dtv[s0]);
      const float as[4] = {acs.x, acs.y, acs.z, acs.w};
      const float ds[4] = {dts.x, dts.y, dts.z, dts.w};
      float m[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = g[r] * exp2_hw(act - as[r]) * ds[r];
        m[r] = (ti < tj || s0 + r <= t) ? v : 0.0f;
      }
      uint32_t h0w, h1w, l0w, l1w;
      split2(m[0], m[1], h0w, l0w);
      split2(m[2], m[3], h1w, l1w);
      *reinterpret_cast<uint2*>(&sm.mhi[t][s0]) = make_uint2(h0w, h1w);
      *reinterpret_cast<uint2*>(&sm.mlo[t][s0]) = make_uint2(l0w, l1w);
    }

    // ---- Y = diag(e^c) C S_in, with S_in split into bf16 high and low parts
    f32x4 Y[4];
    {
      Op shi[KB], slo[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        split2(S[2 * kb][0], S[2 * kb][1], shi[kb].w[0], slo[kb].w[0]);
        split2(S[2 * kb][2], S[2 * kb][3], shi[kb].w[1], slo[kb].w[1]);
        split2(S[2 * kb + 1][0], S[2 * kb + 1][1], shi[kb].w[2], slo[kb].w[2]);
        split2(S[2 * kb + 1][2], S[2 * kb + 1][3], shi[kb].w[3], slo[kb].w[3]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          // K order matching the state operand: n = 32 kb + 4 g4 + (0..3), then + 16
          const uint2 c0 = *reinterpret_cast<const uint2*>(&sm.c[16 * j + l16][32 * kb + 4 * g4]);
          const uint2 c1 =
              *reinterpret_cast<const uint2*>(&sm.c[16 * j + l16][32 * kb + 16 + 4 * g4]);
          const Op ca = {{c0.x, c0.y, c1.x, c1.y}};
          acc = mfma(ca, shi[kb], acc);
          acc = mfma(ca, slo[kb], acc);
        }
        const float4 ev = *reinterpret_cast<const float4*>(&sm.e[16 * j + 4 * g4]);
        acc[0] *= ev.x;
        acc[1] *= ev.y;
        acc[2] *= ev.z;
        acc[3] *= ev.w;
        Y[j] = acc;
      }
    }

    // ---- S_out = e^{c_end} S_in + B^T (w o X)
    Op xop[2];
    {
      const float eEnd = exp2_hw(acEnd);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S[nt] *= eEnd;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        xop[kb] = *reinterpret_cast<const Op*>(&sm.xt[p][swz(p, 32 * kb + 8 * g4)]);
        const float4 w0 = *reinterpret_cast<const float4*>(&sm.w[32 * kb + 8 * g4]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sm.w[32 * kb + 8 * g4 + 4]);
        const float ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        Op whi, wlo;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          split2(lo_f(xop[kb].w[q]) * ww[2 * q], hi_f(xop[kb].w[q]) * ww[2 * q + 1], whi.w[q],
                 wlo.w[q]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const Op bt = *reinterpret_cast<const Op*>(
              &sm.bt[16 * nt + l16][swz(16 * nt + l16, 32 * kb + 8 * g4)]);
          S[nt] = mfma(bt, whi, S[nt]);
          S[nt] = mfma(bt, wlo, S[nt]);
        }
      }
    }
    __syncthreads();  // every wave's tiles of C B^T are in LDS

    // ---- Y += M X over the causal blocks, then skip, gate and store
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int kb = 0; kb <= (j >> 1); ++kb) {
        const Op mh = *reinterpret_cast<const Op*>(&sm.mhi[16 * j + l16][32 * kb + 8 * g4]);
        const Op ml = *reinterpret_cast<const Op*>(&sm.mlo[16 * j + l16][32 * kb + 8 * g4]);
        Y[j] = mfma(mh, xop[kb], Y[j]);
        Y[j] = mfma(ml, xop[kb], Y[j]);
      }
    }
    // this wave's z tile, transposed to (p, t), in the B tile (free after the barrier above)
    uint16_t(*zt)[kTP] = reinterpret_cast<uint16_t(*)[kTP]>(&sm.b[0][0]) + 16 * wv;
    if (GATE) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        uint32_t r4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) r4[r] = (cc >> 1) == 0 ? zr[r].x : zr[r].y;
        const uint2 v = (cc & 1) ? make_uint2(highs(r4[0], r4[1]), highs(r4[2], r4[3]))
                                 : make_uint2(lows(r4[0], r4[1]), lows(r4[2], r4[3]));
        *reinterpret_cast<uint2*>(&zt[4 * (l & 3) + cc][4 * (l >> 2)]) = v;
      }
      wave_lds_sync();
    }
    float xs[4][4], zs[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tb = 16 * j + 4 * g4;
      const uint2 xv = *reinterpret_cast<const uint2*>(&sm.xt[p][swz(p, tb)]);
      xs[j][0] = lo_f(xv.x);
      xs[j][1] = hi_f(xv.x);
      xs[j][2] = lo_f(xv.y);
      xs[j][3] = hi_f(xv.y);
      if (GATE) {
        const uint2 zv = *reinterpret_cast<const uint2*>(&zt[l16][tb]);
        zs[j][0] = lo_f(zv.x);
        zs[j][1] = hi_f(zv.x);
        zs[j][2] = lo_f(zv.y);
        zs[j][3] = hi_f(zv.y);
      }
    }
    // the wave's output tile (t, 16 channels) over its own rows of the x tile, read above
    uint16_t* ot = &sm.xt[16 * wv][0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tb = 16 * j + 4 * g4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float y = fmaf(Dh, xs[j][r], Y[j][r]);
        if (GATE) y *= silu_f(zs[j][r]);
        ot[(tb + r) * 16 + l16] = BF16::from_float(y);
      }
    }
    wave_lds_sync();
    pend_r = make_buf(og + t0 * H * kP, static_cast<uint32_t>(nv - 1) * xrow + kP * 2);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int t = 32 * it + (l >> 1), piece = l & 1;
      pend[it] = *reinterpret_cast<const uint4*>(&ot[t * 16 + 8 * piece]);
    }
    lds_reads_done();  // the next chunk's staging overwrites these rows after the barrier
  }
  if (nchunks > 0) store_pending();

  if (a.h_last) {
    float* hl = a.h_last + bh * N * kP;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) hl[(16 * nt + 4 * g4 + r) * kP + p] = S[nt][r];
  }
}

template <int N>
void launch_n(const Scan2Args& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.batch * a.nheads));
  if (a.z)
    hipLaunchKernelGGL((scan2_mfma_kernel<N, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((scan2_mfma_kernel<N, false>), grid, dim3(256), 0, stream, a);
}

}  // namespace

bool scan2_mfma_supported(const Scan2Args& a, bool bf16) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.out) |
                       reinterpret_cast<uintptr_t>(a.B) | reinterpret_cast<uintptr_t>(a.C) |
                       reinterpret_cast<uintptr_t>(a.z);
  return bf16 && a.headdim == kP && (a.d_state == 64 || a.d_state == 128) && (al & 15) == 0 &&
         int64_t(kQ) * a.nheads * kP * 2 < (int64_t(1) << 31) &&
         int64_t(kQ) * a.ngroups * a.d_state * 2 < (int64_t(1) << 31) &&
         a.batch * a.nheads <= int64_t(0x7fffffff);
}

hipError_t launch_scan2_mfma(const Scan2Args& a, hipStream_t stream) {
  if (a.batch * a.nheads == 0 || a.seqlen == 0) return hipSuccess;
  if (a.d_state == 64) launch_n<64>(a, stream);
  else launch_n<128>(a, stream);
  return hipGetLastError();
}

}  // namespace ss
