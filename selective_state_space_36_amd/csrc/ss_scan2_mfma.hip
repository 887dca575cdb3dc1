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
// the state in registers (with more pairs than CUs but fewer than two per CU, some pairs are cut
// into time pieces instead; see launch_n); wave w owns head channels 16w..16w+15 (one 16-column
// tile of S, X and Y), so the state never leaves the wave.  The 10 causal 16x16 tiles of C B^T are shared: each
// wave computes some of them, applies the mask and decays, and writes the split products to LDS.
// Per chunk the workgroup stages B, C and x in LDS as loaded (16-byte / 8-byte global loads
// issued one chunk ahead) and reads the operands that need a transpose with the LDS transpose
// read.  The outputs are formed transposed (rows: channels, columns: steps), which leaves each
// lane 4 adjacent channels of one step, as x, z and out lie in memory: z is loaded straight into
// that layout, and the outputs leave straight from registers as 8-byte stores.
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
constexpr int kTP = kQ + 8;          // bf16 per row of the (t, s) tiles
// bf16 per row of the x tile (s, p): 160 bytes, so that the four rows a transpose read covers
// start 8 banks apart and the read is free of bank conflicts
constexpr int kXS = kP + 16;

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
// 8-byte store through a buffer resource (dropped past its range).
__device__ __forceinline__ void store8(uint2 v, rsrc_t r, uint32_t off) {
  using v2u = __attribute__((ext_vector_type(2))) unsigned int;
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v), r, off, 0, 0);
}
__device__ __forceinline__ float lo_f(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_f(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Four bf16 of column n0 + l16 (l16 = lane % 16) in rows s0 .. s0 + 3 of a row-major LDS tile
// of `stride` elements per row, as (rows s0, s0 + 1) and (s0 + 2, s0 + 3) pairs: an MFMA operand
// half with K running down a column.  The gfx950 LDS transpose read (ds_read_b64_tr_b16) hands
// lane i of each 16-lane group element i % 4 of the 8 bytes read by lanes i / 4 + 4 m of the
// group, m = 0..3 (lane layout checked on the MI355X); so lane j reads the 4 elements of row
// s0 + j / 4 starting at column n0 + 4 (j % 4).
// The same from a tile whose rows hold their 8-byte units (4 bf16) XOR-permuted by `key`
// (uniform over rows s0 .. s0 + 3): lane j reads logical columns n0 + 4 (j % 4) .. + 3 where the
// permutation put them.
__device__ __forceinline__ uint2 tr_read4_swz(const uint16_t* tile, int stride, int s0, int n0,
                                              int l16, int key) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef v4s __attribute__((address_space(3)))* lds_v4s;
  const int unit = (n0 >> 2) + (l16 & 3);
  const uint16_t* q = tile + (s0 + (l16 >> 2)) * stride + 4 * (unit ^ key);
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(q)));
}
__device__ __forceinline__ uint2 tr_read4(const uint16_t* tile, int stride, int s0, int n0,
                                          int l16) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef v4s __attribute__((address_space(3)))* lds_v4s;
  const uint16_t* q = tile + (s0 + (l16 >> 2)) * stride + n0 + 4 * (l16 & 3);
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(q)));
}

// Split (a, b) into high and low bf16 pairs: a = hi + lo to about 2^-17 relative.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(a - lo_f(hi), b - hi_f(hi));
}

// LDS of one workgroup: 64 KB at d_state 128.  B, C and x are staged as loaded (row-major);
// the operands that run K down a column (B^T for the state update, x for the products and the
// epilogue) come from them by LDS transpose reads (tr_read4).
template <int N>
struct alignas(16) Smem2 {
  uint16_t b[kQ][N + 16];       // B of the chunk, (s, n) (rows start 8 banks apart for the
                                // transpose reads)
  uint16_t c[kQ][N + 4];        // C, (t, n): rows 2 banks apart, so the 8-byte operand reads
                                // of S_in^T C^T (16 rows, one per lane) are free of conflicts;
                                // staged and read by the C B^T tiles 8 bytes at a time
  uint16_t x[kQ][kXS];          // x, (s, p); in row s the 8-byte units (4 channels) are
                                // XOR-permuted by (s / 4) mod 4, so that the epilogue's 8-byte
                                // reads of 16 rows are free of bank conflicts
  uint16_t mhi[kQ][kTP];        // masked, decayed and dt-scaled C B^T, (t, s): high part
  uint16_t mlo[kQ][kTP];        // low part
  float ac[kQ];                 // c_t, the chunk's cumulative log2 decay
  float dtv[kQ];                // dt_t (0 past the sequence end)
  float e[kQ];                  // 2^{c_t}
  float w[kQ];                  // dt_t 2^{c_{Q-1} - c_t}
};

// Inclusive prefix sum over the 64 lanes of the wave: Hillis-Steele steps inside each 16-lane
// row by DPP row shifts (lanes shifted in from outside the row read 0), then the row totals
// carried across rows by the GFX9 row broadcasts: lane 15 of rows 0 and 2 added to rows 1 and 3,
// then lane 31 (the total of rows 0 and 1) to rows 2 and 3 (rows left out of a row mask add 0).
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, false));
  return x;
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
  // Workgroups 0 .. n_whole - 1 take whole (batch row, head) pairs; the rest take the remaining
  // pairs in q_split pieces each, piece k the chunks [piece_beg[k], piece_beg[k + 1]), after
  // running the state alone over the chunks before it (see launch_n).
  const int64_t nchunks = (L + kQ - 1) / kQ;
  int64_t bh, cbeg = 0, cend = nchunks;
  if (int64_t(blockIdx.x) < a.n_whole) {
    bh = xcd_remap(blockIdx.x, a.n_whole);
  } else {
    const int64_t np = int64_t(gridDim.x) - a.n_whole;
    const int64_t pc = xcd_remap(blockIdx.x - a.n_whole, np);
    const int k = static_cast<int>(pc % a.q_split);
    bh = a.n_whole + pc / a.q_split;
    cbeg = a.piece_beg[k];
    cend = a.piece_beg[k + 1];
  }
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
    // z: each wave loads its own 16 channels in the layout of its outputs: for step
    // 16 r + l16, the 4 channels 16 wv + 4 g4 .. + 3
    zoff[r] = (16 * r + l16) * xrow + (16 * wv + 4 * g4) * 2;
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
  auto fetch = [&](int64_t t0, bool with_c) {
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
        if (with_c) cr[k][r] = buf_load<uint4>(rc, boff[k][r]);
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

  // Outputs of the previous chunk, stored at the start of the next one: stores issued right
  // after the next chunk's loads would make the wait for those loads wait for the stores too.
  // Each lane stores its 4 channels of each of its 4 steps (8 bytes, at z's offsets); the four
  // waves fill the 128 bytes of a step's row.
  uint2 pend[4] = {make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0), make_uint2(0, 0)};
  rsrc_t pend_r = make_buf(og, 0);
  auto store_pending = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) store8(pend[j], pend_r, zoff[j]);
  };

  // S_out = e^{c_end} S_in + B^T (w o X) for the chunk staged in LDS; leaves this wave's x
  // operand (K = steps) in xop for the chunk's M X
  auto update_state = [&](Op (&xop)[2], float acEnd) {
    const float eEnd = exp2_hw(acEnd);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) S[nt] *= eEnd;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      {  // x of channel p, K = s = 32 kb + 8 g4 + 0..7, down a column of the x tile
        const uint2 k03 =
            tr_read4_swz(&sm.x[0][0], kXS, 32 * kb + 8 * g4, 16 * wv, l16, (2 * g4) & 3);
        const uint2 k47 =
            tr_read4_swz(&sm.x[0][0], kXS, 32 * kb + 8 * g4 + 4, 16 * wv, l16, (2 * g4 + 1) & 3);
        xop[kb] = Op{{k03.x, k03.y, k47.x, k47.y}};
      }
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
        // B^T rows n = 16 nt + l16, K = s = 32 kb + 8 g4 + 0..7, read from the row-major tile
        const uint2 k03 = tr_read4(&sm.b[0][0], N + 16, 32 * kb + 8 * g4, 16 * nt, l16);
        const uint2 k47 = tr_read4(&sm.b[0][0], N + 16, 32 * kb + 8 * g4 + 4, 16 * nt, l16);
        const Op bt = {{k03.x, k03.y, k47.x, k47.y}};
        S[nt] = mfma(bt, whi, S[nt]);
        S[nt] = mfma(bt, wlo, S[nt]);
      }
    }
  };

  // ---- the state alone over the chunks before this workgroup's range: staging of B and x,
  // the decays and the state update (no outputs)
  auto decays = [&](uint16_t dcur, int nv, float& acEnd) {
    const float s = BF16::widen(dcur) + bias;
    float dv = a.softplus ? softplus_f(s) : s;
    dv = l < nv ? dv : 0.0f;
    const float c = wave_prefix_sum(dv * A2);
    acEnd = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 63));
    // every wave has the same values and writes them: identical bits to the same place
    sm.ac[l] = c;
    sm.dtv[l] = dv;
    sm.e[l] = exp2_hw(c);
    sm.w[l] = exp2_hw(acEnd - c) * dv;
  };
  fetch(0, cbeg == 0);
  for (int64_t ch = 0; ch < cbeg; ++ch) {
    const int64_t t0 = ch * kQ;
    __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<uint2*>(&sm.x[4 * xq + r][4 * (xp ^ (xq & 3))]) = xr[r];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = tid + 256 * k;
      if (UNITS % 256 == 0 || u < UNITS) {
        const int rq = u / (N / 8), nb = u % (N / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<uint4*>(&sm.b[4 * rq + r][8 * nb]) = br[k][r];
      }
    }
    const uint16_t dcur = dtr;
    fetch(t0 + kQ, ch + 1 == cbeg);  // the range's first chunk needs C as well
    float acEnd;
    decays(dcur, static_cast<int>(L - t0 < kQ ? L - t0 : kQ), acEnd);
    __syncthreads();  // staged tiles visible
    Op xop[2];
    update_state(xop, acEnd);
  }

  for (int64_t ch = cbeg; ch < cend; ++ch) {
    const int64_t t0 = ch * kQ;
    const int nv = static_cast<int>(L - t0 < kQ ? L - t0 : kQ);
    __syncthreads();  // the previous chunk's LDS reads are done
    // ---- stage the chunk in LDS
#pragma unroll
    for (int r = 0; r < 4; ++r)  // x as loaded: 4 channels of a step per write
      *reinterpret_cast<uint2*>(&sm.x[4 * xq + r][4 * (xp ^ (xq & 3))]) = xr[r];
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u = tid + 256 * k;
      if (UNITS % 256 == 0 || u < UNITS) {
        const int rq = u / (N / 8), nb = u % (N / 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *reinterpret_cast<uint4*>(&sm.b[4 * rq + r][8 * nb]) = br[k][r];
          {
            uint2* cp = reinterpret_cast<uint2*>(&sm.c[4 * rq + r][8 * nb]);
            cp[0] = make_uint2(cr[k][r].x, cr[k][r].y);
            cp[1] = make_uint2(cr[k][r].z, cr[k][r].w);
          }
        }
      }
    }
    // the chunk's dt, before the loads below replace it with the next chunk's
    const uint16_t dcur = dtr;
    // the output stores and the next chunk's loads go out first: they are what the chunk's
    // arithmetic hides
    store_pending();  // on the first chunk pend_r covers no bytes: nothing is written
    fetch(t0 + kQ, true);  // past the end on the last chunk: no memory is touched
    fetch_z(t0);
    // ---- step sizes and decays of the chunk (every wave keeps its own copy)
    float acEnd;
    decays(dcur, nv, acEnd);
    __syncthreads();  // staged tiles visible

    // ---- the causal tiles of C B^T owned by this wave -> masked, decayed, split, to LDS.  The
    // 10 tiles (s-tile ti <= t-tile tj) in the order (0,0) (0,1) (1,1) (0,2) ... (3,3) are dealt
    // to the waves round-robin; waves 2 and 3, which own two, repeat tile 0 or 1 as their third,
    // writing the same bits to the same place as its owner, so that every wave runs the same
    // three tiles without a branch and their products and the S_in split can interleave.
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int kk = wv + 4 * i;
      const int k = kk < 10 ? kk : kk - 10;
      const int tj = (k >= 1) + (k >= 3) + (k >= 6);
      const int ti = k - tj * (tj + 1) / 2;
      f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const Op ab = *reinterpret_cast<const Op*>(&sm.b[16 * ti + l16][32 * kb + 8 * g4]);
        const uint2* cq = reinterpret_cast<const uint2*>(&sm.c[16 * tj + l16][32 * kb + 8 * g4]);
        const uint2 bc0 = cq[0], bc1 = cq[1];
        const Op bc = {{bc0.x, bc0.y, bc1.x, bc1.y}};
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

    // ---- Y = diag(e^c) C S_in, with S_in split into bf16 high and low parts.  Y is formed
    // transposed, Y[j][r] = Y(t = 16 j + l16, p = 16 wv + 4 g4 + r): each lane then holds 4
    // adjacent channels of one step, the layout of x, z and out in memory.
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
          // S_in^T C^T: rows are channels, columns steps
          acc = mfma(shi[kb], ca, acc);
          acc = mfma(slo[kb], ca, acc);
        }
        const float ev = sm.e[16 * j + l16];
        acc[0] *= ev;
        acc[1] *= ev;
        acc[2] *= ev;
        acc[3] *= ev;
        Y[j] = acc;
      }
    }

    // ---- S_out = e^{c_end} S_in + B^T (w o X)
    Op xop[2];
    update_state(xop, acEnd);
    __syncthreads();  // every wave's tiles of C B^T are in LDS

    // ---- Y += M X over the causal blocks (as X^T M^T), then skip, gate and store
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int kb = 0; kb <= (j >> 1); ++kb) {
        const Op mh = *reinterpret_cast<const Op*>(&sm.mhi[16 * j + l16][32 * kb + 8 * g4]);
        const Op ml = *reinterpret_cast<const Op*>(&sm.mlo[16 * j + l16][32 * kb + 8 * g4]);
        Y[j] = mfma(xop[kb], mh, Y[j]);
        Y[j] = mfma(xop[kb], ml, Y[j]);
      }
    }
    // skip and gate: lane (l16, g4) owns step 16 j + l16, channels 16 wv + 4 g4 .. + 3, and reads
    // its x in the x tile
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 xv = *reinterpret_cast<const uint2*>(
          &sm.x[16 * j + l16][4 * ((4 * wv + g4) ^ ((l16 >> 2) & 3))]);
      const float xs[4] = {lo_f(xv.x), hi_f(xv.x), lo_f(xv.y), hi_f(xv.y)};
      float y[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = fmaf(Dh, xs[r], Y[j][r]);
      if (GATE) {
        const float zs[4] = {lo_f(zr[j].x), hi_f(zr[j].x), lo_f(zr[j].y), hi_f(zr[j].y)};
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] *= silu_f(zs[r]);
      }
      pend[j] = make_uint2(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]));
    }
    pend_r = make_buf(og + t0 * H * kP, static_cast<uint32_t>(nv - 1) * xrow + kP * 2);
    lds_reads_done();  // the next chunk's staging overwrites the x tile after the barrier
  }
  if (cend > cbeg) store_pending();

  if (a.h_last && cend == nchunks) {
    float* hl = a.h_last + bh * N * kP;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) hl[(16 * nt + 4 * g4 + r) * kP + p] = S[nt][r];
  }
}

// Relative cost of a chunk run for the state alone (B, x, decays and the state update) against a
// full chunk, measured on the 80-head layer at batch 1 (three pieces per pair: 142.5 us against
// 266 us whole).
constexpr double kPreludeCost = 0.30;
// Time of a chunk when two workgroups share a CU, against one alone (same layer, batch 4).
constexpr double kSharedSlowdown = 1.385;

// Boundaries of q pieces over n chunks with equal work: piece k runs P_k earlier chunks for the
// state alone and its own l_k chunks, l_k + r P_k equal for all k, so l_{k+1} = (1 - r) l_k and
// the pieces shrink geometrically.  Rounded to whole chunks, every piece at least one chunk.
void piece_bounds(int64_t n, int q, int32_t* beg) {
  double sum = 0.0, len = 1.0;
  for (int k = 0; k < q; ++k, len *= 1.0 - kPreludeCost) sum += len;
  double acc = 0.0;
  len = 1.0;
  beg[0] = 0;
  for (int k = 1; k < q; ++k, len *= 1.0 - kPreludeCost) {
    acc += len;
    int64_t b = static_cast<int64_t>(double(n) * acc / sum + 0.5);
    if (b < beg[k - 1] + 1) b = beg[k - 1] + 1;
    if (b > n - (q - k)) b = n - (q - k);
    beg[k] = static_cast<int32_t>(b);
  }
  beg[q] = static_cast<int32_t>(n);
}

// Longest piece's work, in whole-pair units, when a pair is cut into q equal-work pieces.
double piece_work(int q) {
  double sum = 0.0, len = 1.0;
  for (int k = 0; k < q; ++k, len *= 1.0 - kPreludeCost) sum += len;
  return 1.0 / sum;
}

// Each (batch row, head) pair is a sequential walk over the chunks, two of which share a CU.
// With more pairs than CUs but fewer than two per CU, the CUs given two whole pairs would set the
// time while the others idle half of it.  So when the pairs number between one and two per CU,
// one pair per CU runs whole and each remaining pair is cut into q time pieces (q = CUs / extra
// pairs, at most 4), one workgroup each: every CU then holds one whole pair and one piece.  With
// at most one pair per CU, every pair is cut (below).  A piece first runs the state alone (B, x
// and the decays; no C, no outputs) over the chunks before its own, about a third of a chunk's
// work each, so the pieces are cut to equal work rather than equal length.
template <int N>
void launch_n(const Scan2Args& a0, hipStream_t stream) {
  Scan2Args a = a0;
  const int64_t pairs = a.batch * a.nheads;
  const int64_t nchunks = (a.seqlen + kQ - 1) / kQ;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 0;
  a.n_whole = pairs;
  a.q_split = 1;
  int64_t q = 1;
  if (cus > 0 && pairs > 0 && pairs <= cus) {
    // At most one pair per CU: cut every pair into the q pieces (1..4) that minimise the longest
    // piece's work, slowed by kSharedSlowdown when the pieces outnumber the CUs and two share
    // one; never more pieces than two per CU.
    double best = 1.0;
    for (int64_t qq = 2; qq <= kScan2MaxPieces && qq <= nchunks; ++qq) {
      if (pairs * qq > 2 * int64_t(cus)) break;
      const double work = piece_work(static_cast<int>(qq)) *
                          (pairs * qq > cus ? kSharedSlowdown : 1.0);
      if (work < best) {
        best = work;
        q = qq;
      }
    }
  } else if (cus > 0 && pairs > cus && pairs < 2 * int64_t(cus)) {
    q = cus / (pairs - cus);
    if (q > kScan2MaxPieces) q = kScan2MaxPieces;
    if (q > nchunks) q = nchunks;
  }
  if (q >= 2 && nchunks < (int64_t(1) << 31)) {
    a.q_split = static_cast<int32_t>(q);
    a.n_whole = pairs <= cus ? 0 : cus;
    piece_bounds(nchunks, static_cast<int>(q), a.piece_beg);
  }
  const dim3 grid(static_cast<unsigned>(a.n_whole + (pairs - a.n_whole) * a.q_split));
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
