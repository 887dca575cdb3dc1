// ss_scan_kernel.h -- gfx950 prefill kernel template of the selective scan, instantiated by
// ss_scan_fwd.hip (first-order input term) and ss_scan_zoh.hip (exact zero-order hold).
//
// What is computed (per batch row b, channel d, state n; Mamba reading guide, sections "Método"
// and "O Mecanismo de Seleção (S6)"):
//     dt_t = softplus(delta + bias),  h_t = exp(dt_t A) h_{t-1} + dt_t B_t u_t,
//     y_t = C_t . h_t + D u_t,  out = y_t * silu(z_t).
// With ZOH the input term is the exact zero-order-hold one, (exp(dt_t A) - 1) / A * B_t u_t
// (reading guide, "Método"), in place of the first-order dt_t B_t u_t.
// With CONV the kernel reads the block's x instead of u and forms u itself (IBM explainer,
// Mamba-block walk-through: x passes a 1-D convolution, then SiLU):
//     u_t = silu(conv_b + sum_{j<k} conv_w[j] x_{t-k+1+j}),   k <= 4, causal, per channel,
// so u never makes a round trip through HBM.  The owner lane of step t holds x_t; the earlier
// taps come from the lanes of steps t-1..t-3 by DPP row rotations, from the previous chunk's
// values for the first three steps of a chunk.
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
//     current chunk is computed.  The tiles are addressed as raw buffers sized to the valid
//     steps, so the hardware range check handles the sequence tail.
//   * The output sum over states goes through a per-wave LDS tile: with d_state <= 16 the lanes
//     store their states h_t[n] and the owner lane of step t forms C_t . h_t itself (16 FMAs,
//     C_t read as a row of the C tile); with wider states the lanes store partial sums over
//     their own states and the owner adds them up.  No atomics: results are bitwise
//     reproducible.
//   * Long sequences with few channels are cut into time segments.  A summary pass computes each
//     segment's end state from a zero start and the sum of its dt; the output pass then starts
//     segment s from h0 carried through segments 0..s-1 with h <- exp(A sum dt) h + h_end, the
//     blockwise form of the associative recurrence (reading guide: parallel associative scan;
//     IBM explainer: blocks combined hierarchically).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "ss_device.h"
#include "ss_launch.h"

namespace ss {
namespace {

constexpr int kWaves = kPrefillThreads / 64;
constexpr int kT = kChunk;               // steps per chunk (= lanes per row)
constexpr int kTileStride = kT + 2;      // float2 slots per state row of the B/C tile (padding)
// Per-wave tile of the values the lanes hand to the owner lanes: channel row r at r * kPRow,
// step slot s at s * kPTau, lane k at k; odd rows keep step t in slot t ^ kPSwap.  Chosen by
// measurement on gfx950 (LDS bank-conflict counter over the tile's own access patterns): with
// this layout both the owners' 16-byte reads and the paired 4-byte writes of two steps are
// conflict-free, while rows 336 floats apart (no swap) conflict on the reads and rows 320 apart
// conflict on the writes (swap 0 or 4) or on the reads (swap 4).
constexpr int kPRow = 320;               // floats per channel row of the partial tile
constexpr int kPSwap = 12;               // odd rows: step t in slot t ^ kPSwap
constexpr int kPTau = 20;                // floats per step slot of the partial tile (padding)
constexpr int kSRow = 20;                // floats per row of the split B and C tiles (padding)
static_assert(kT == 16, "one chunk step per row lane");

template <class IO, int NL, bool GATE, bool SUMMARY, bool VEC, bool ZOH, bool CONV>
struct ScanKernel {
  using elem = typename IO::elem;
  static constexpr int NP = 16 * NL;                         // padded state count
  static constexpr int ES = sizeof(elem);                    // io element bytes
  static constexpr int NTEN = SUMMARY ? 2 : (GATE ? 3 : 2);  // streamed inputs: u, delta, (z)
  static constexpr int PIECES = kChanPerWG * ES / 16;        // 16-byte pieces per tile row
  static_assert(kT * PIECES <= 64, "one 16-byte piece of a tile per lane of a wave");
  static_assert(NTEN < kWaves, "a wave left over for the output tile");
  static constexpr int BC_PER_THREAD = kT * NP / kPrefillThreads;
  // d_state <= 16 (one state per lane): the lanes hand their states h_t[n] to the owner lane of
  // step t, which forms C_t . h_t with 16 FMAs, instead of each lane multiplying by C_t[n] and
  // the owner adding 16 products (31 instructions per chunk -> 17).  Wider states keep the
  // per-lane partial sums: their states would not fit the per-wave tile.
  static constexpr bool FOLD = NL == 1 && !SUMMARY;
  // B in a tile of its own, four steps per 16-byte read: with one state per lane (C then in a
  // tile of its own as well, read as rows by the owner lanes) and in every summary pass, which
  // never forms C . h and so neither loads nor stages C.
  static constexpr bool SPLIT = NL == 1 || SUMMARY;
  // The 16-byte pieces of row (step) k of a u/delta/z/out tile are stored XOR-permuted by
  // (k / (8 / PIECES)) mod PIECES.  The owner lanes of steps 4 (bf16) or 2 (fp32) apart read the
  // same column of rows that share LDS banks (rows are 32 or 64 bytes; LDS has 32 banks of 4
  // bytes); the permutation moves half of them to the other bank set.
  static __device__ __forceinline__ int pswz(int row) {
    return (row / (8 / PIECES)) & (PIECES - 1);
  }

  struct PairTile {
    float2 bc[2][NP][kTileStride];  // (B_t[n], C_t[n]) per chunk
  };
  struct SplitTile {
    float b[2][kT][kSRow];  // B_t[n] per chunk, row n (read by the lane of state n)
    float c[2][kT][kSRow];  // C_t[n] per chunk, row t (read by the owner lane of step t)
  };
  struct BTile {
    float b[2][NP][kSRow];  // B_t[n] per chunk, row n (summary passes)
  };
  struct alignas(16) Smem {
    std::conditional_t<FOLD, SplitTile, std::conditional_t<SUMMARY, BTile, PairTile>> bt;
    uint4 in[2][NTEN][kT][PIECES];  // raw u, delta, z tiles per chunk
    uint4 out[2][kT][PIECES];       // raw output tile per chunk
    float p[kWaves][4 * kPRow];     // per-wave partial sums or states [row][step][lane]
  };

  static __device__ __forceinline__ void run(const ScanArgs& a) {
    __shared__ Smem sm;
    // Workgroup coordinates (all below 2^31: the host bounds the grid and d_inner); kept in
    // scalar registers so that everything derived from them is scalar work.
    const int64_t ncb_total = a.batch * a.n_cblk;
    const int64_t lg = xcd_remap(blockIdx.x, a.n_wg);
    const int64_t seg = __builtin_amdgcn_readfirstlane(static_cast<int>(lg / ncb_total));
    const int64_t cb = lg - seg * ncb_total;
    const int64_t b = __builtin_amdgcn_readfirstlane(static_cast<int>(cb / a.n_cblk));
    const int64_t d0 =
        __builtin_amdgcn_readfirstlane(static_cast<int>((cb - b * a.n_cblk) * kChanPerWG));
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

    // Per-lane constants: A scaled by log2(e) so that exp(dt A) = 2^(dt A2), and (exact hold
    // only) 1 / A, 0 where A = 0.
    float A2[NL], ia[NL], h[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int n = k + 16 * j;
      const bool ok = chan_ok && n < a.d_state;
      const float an = ok ? a.A[d * a.d_state + n] : 0.0f;
      A2[j] = an * kLog2e;
      ia[j] = (ZOH && an != 0.0f) ? 1.0f / an : 0.0f;
      h[j] = 0.0f;
    }
    const float bias = (chan_ok && a.delta_bias) ? a.delta_bias[d] : 0.0f;
    const float dskip = (!SUMMARY && chan_ok && a.D) ? a.D[d] : 0.0f;
    // saved chunk-end states, (batch, chunk, d_inner, d_state): this lane's state n = k of
    // channel d, from the segment's first chunk on (the output pass carries the true state across
    // segments).  The four channels of a wave fill 256 contiguous bytes per chunk.
    const int64_t st_chunk = a.d_inner * a.d_state;  // floats per chunk
    // the states-only pass (a summary launch without segment buffers) saves them as well
    const bool states_only = SUMMARY && a.seg_h == nullptr;
    float* st_lane = ((!SUMMARY || states_only) && a.states && chan_ok)
                         ? a.states + ((b * a.states_chunks + t_begin / kT) * a.d_inner + d) *
                                          a.d_state + k
                         : nullptr;

    // Front end (CONV): tap weights of a 4-wide window ending at this lane's step (cw[s - 1]
    // for the step t - s), and the lane's x of the previous chunk (for the first chunk, x before
    // the segment: from x itself, from the caller's history x_prev before t = 0, or 0).
    float cw_own = 0.0f, cbias = 0.0f, cw[3] = {0.0f, 0.0f, 0.0f};
    float xprev = 0.0f;
    if (CONV && chan_ok) {
      const int K = a.conv_k;
#pragma unroll
      for (int s = 1; s <= 3; ++s)  // tap at step t - s
        cw[s - 1] = s < K ? a.conv_w[d * K + (K - 1 - s)] : 0.0f;
      cw_own = a.conv_w[d * K + (K - 1)];
      cbias = a.conv_b ? a.conv_b[d] : 0.0f;
      const int64_t tp = t_begin - kT + k;  // the step this lane held in the "previous chunk"
      if (tp >= 0)
        xprev = IO::load(static_cast<const elem*>(a.u), (b * a.seqlen + tp) * a.d_inner + d);
      else if (a.x_prev && tp >= -(K - 1))
        xprev = IO::load(static_cast<const elem*>(a.x_prev),
                         (b * (K - 1) + (K - 1) + tp) * a.d_inner + d);
    }

    if (!SUMMARY || states_only) {
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
    // Tiles are addressed through raw buffer resources whose base moves by one chunk per call and
    // whose size covers only the chunk's valid steps: loads past the end of the sequence return 0
    // and stores past it are dropped by the hardware range check.  Each thread's byte offset
    // inside a tile is therefore fixed for the whole loop, and no load or store needs a mask or an
    // address update of its own.
    // Roles: every thread loads element(s) (tau, n) of the B and C tiles, consecutive threads on
    // consecutive n (contiguous in memory); wave w < NTEN loads tile w of (u, delta, z), one
    // 16-byte piece (step row, piece) per lane; wave NTEN stores the output tile.  Global loads for
    // chunk i+1 are issued before chunk i is computed and written to LDS after it.
    const int64_t D = a.d_inner, N = a.d_state;
    const int64_t row0 = b * a.seqlen + t_begin;  // (b, t_begin) row of u/delta/z/out, B/C
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int tl_row = lane / PIECES, tl_pc = lane % PIECES;  // piece of a u/delta/z/out tile
    const bool tl_on = lane < kT * PIECES;
    const uint32_t tl_off =
        tl_on ? static_cast<uint32_t>((tl_row * D + tl_pc * (16 / ES)) * ES) : kOffNone;
    // wave w < NTEN loads tensor w; the other waves get a valid base they never load from
    const char* in_base = static_cast<const char*>(
        wave_u == 0 ? a.u : (wave_u == 1 ? a.delta : (wave_u == 2 && NTEN == 3 ? a.z : a.u)));
    const int64_t io_chunk_bytes = kT * D * ES;
    const int64_t io_off0 = (row0 * D + d0) * ES;  // byte offset of chunk 0's tiles
    int bc_tau[BC_PER_THREAD], bc_n[BC_PER_THREAD];
    uint32_t bc_off[BC_PER_THREAD];
#pragma unroll
    for (int i = 0; i < BC_PER_THREAD; ++i) {
      const int idx = tid + i * kPrefillThreads;  // < kT * NP
      bc_tau[i] = idx / NP;
      bc_n[i] = idx - bc_tau[i] * NP;
      bc_off[i] = bc_n[i] < N ? static_cast<uint32_t>((bc_tau[i] * N + bc_n[i]) * ES) : kOffNone;
    }
    static_assert(BC_PER_THREAD * kPrefillThreads == kT * NP, "B/C tile split over threads");
    int ncols = static_cast<int>(D - (d0 + tl_pc * (16 / ES)));  // valid channels of the piece
    ncols = ncols < 0 ? 0 : (ncols > 16 / ES ? 16 / ES : ncols);
    // chunk counters are 32-bit (scalar compares; the host bounds seqlen below 2^31)
    const int nchunks = static_cast<int>((t_end - t_begin + kT - 1) / kT);

    struct Pre {
      elem rb[BC_PER_THREAD], rc[BC_PER_THREAD];
      uint4 rin;
    } pre;

    // valid steps of chunk ci (kT except for a partial last chunk); uniform over the workgroup
    const int last_valid = static_cast<int>(t_end - t_begin - int64_t(nchunks - 1) * kT);
    auto nvalid_of = [&](int ci) { return ci == nchunks - 1 ? last_valid : kT; };
    // Tile bases advance by a fixed stride per chunk: running pointers in scalar registers, one
    // add per chunk, rather than each chunk's 64-bit offsets recomputed from its index (some 40
    // scalar instructions per chunk on every wave's critical path).  The io ranges end with the
    // chunk's last valid row: channels past d_inner in that row (reached only by the element
    // path) read 0 and are not written.
    const int64_t bc_chunk_bytes = int64_t(kT) * N * ES;
    const uint32_t bc_bytes_full = static_cast<uint32_t>(kT * N * ES);
    const uint32_t bc_bytes_last = static_cast<uint32_t>(last_valid * N * ES);
    const uint32_t io_bytes_full = static_cast<uint32_t>((kT * D - d0) * ES);
    const uint32_t io_bytes_last = static_cast<uint32_t>((last_valid * D - d0) * ES);
    const char* b_next = static_cast<const char*>(a.B) + row0 * N * ES;  // next chunk to load
    const char* c_next = static_cast<const char*>(a.C) + row0 * N * ES;
    const char* in_next = in_base + io_off0;
    const char* out_next = SUMMARY ? nullptr : static_cast<const char*>(a.out) + io_off0;

    auto load_chunk = [&](int ci) {
      const bool last = ci == nchunks - 1;
      const uint32_t bc_bytes = last ? bc_bytes_last : bc_bytes_full;
      const rsrc_t rb = make_buf(b_next, bc_bytes);
      const rsrc_t rc = make_buf(c_next, bc_bytes);
      b_next += bc_chunk_bytes;
      c_next += bc_chunk_bytes;
#pragma unroll
      for (int i = 0; i < BC_PER_THREAD; ++i) {
        pre.rb[i] = buf_load<elem>(rb, bc_off[i]);
        if constexpr (!SUMMARY) pre.rc[i] = buf_load<elem>(rc, bc_off[i]);
      }
      const char* in_cur = in_next;
      in_next += io_chunk_bytes;
      if (wave_u < NTEN) {  // uniform
        const rsrc_t ri = make_buf(in_cur, last ? io_bytes_last : io_bytes_full);
        if (VEC) {
          pre.rin = buf_load<uint4>(ri, tl_off);
        } else {
          // element loads; channels past d_inner read the next row or 0 and are never used
          elem tmp[16 / ES];
#pragma unroll
          for (int e = 0; e < 16 / ES; ++e) tmp[e] = buf_load<elem>(ri, tl_off + e * ES);
          pre.rin = *reinterpret_cast<const uint4*>(tmp);
        }
      }
    };
    auto stage_chunk = [&](int buf) {
#pragma unroll
      for (int i = 0; i < BC_PER_THREAD; ++i) {
        if constexpr (SPLIT) {
          sm.bt.b[buf][bc_n[i]][bc_tau[i]] = IO::widen(pre.rb[i]);
          if constexpr (FOLD) sm.bt.c[buf][bc_tau[i]][bc_n[i]] = IO::widen(pre.rc[i]);
        } else {
          sm.bt.bc[buf][bc_n[i]][bc_tau[i]] =
              make_float2(IO::widen(pre.rb[i]), IO::widen(pre.rc[i]));
        }
      }
      if (wave_u < NTEN && tl_on) sm.in[buf][wave_u][tl_row][tl_pc ^ pswz(tl_row)] = pre.rin;
    };
    // The data registers of the last output store are kept live (hold_store) until the next
    // chunk's compute is done: otherwise the allocator reuses them at once and the write to them
    // has to wait for the store to complete.
    uint4 st_val{0, 0, 0, 0};
    auto hold_store = [&]() {
      if (VEC && !SUMMARY)
        asm volatile("" ::"v"(st_val.x), "v"(st_val.y), "v"(st_val.z), "v"(st_val.w));
    };
    auto store_out = [&](int buf, int ci) {
      const char* out_cur = out_next;
      out_next += io_chunk_bytes;
      if (!SUMMARY && wave_u == NTEN && tl_on) {
        const rsrc_t ro = make_buf(out_cur, ci == nchunks - 1 ? io_bytes_last : io_bytes_full);
        const uint4 v = sm.out[buf][tl_row][tl_pc ^ pswz(tl_row)];
        if (VEC) {
          st_val = v;
          buf_store(v, ro, tl_off);
        } else {
          elem tmp[16 / ES];
          *reinterpret_cast<uint4*>(tmp) = v;
#pragma unroll
          for (int e = 0; e < 16 / ES; ++e)
            if (e < ncols) buf_store(tmp[e], ro, tl_off + e * ES);
        }
      }
    };
    // column of channel cl in row k of a tile (pieces permuted by pswz)
    const int own_col = ((cl / (16 / ES)) ^ pswz(k)) * (16 / ES) + cl % (16 / ES);
    auto own_in = [&](int buf, int ten) -> float {
      const elem* t = reinterpret_cast<const elem*>(&sm.in[buf][ten][k][0]);
      return IO::widen(t[own_col]);
    };

    float dt_acc = 0.0f;  // summary pass: this lane's share of sum(dt) over the segment

    load_chunk(0);
    stage_chunk(0);
    __syncthreads();

    // One chunk: issue the loads of the next chunk, compute this one from LDS buffer BUF, stage
    // the next chunk into the other buffer, then store this chunk's output tile.  BUF is a
    // compile-time constant so that every LDS address is a register plus an immediate.
    auto chunk = [&](int ci, auto bufc) {
      constexpr int buf = decltype(bufc)::value;
      const bool has_next = ci + 1 < nchunks;
      if (has_next) load_chunk(ci + 1);

      // Every LDS read of the chunk is issued here, in the order the results are needed (LDS
      // returns them in order): this lane's u and delta for the element work, the B column of its
      // states for the steps, z for the gate, the C row of its step for the output sum.
      float xu = own_in(buf, 0);
      const float sraw = own_in(buf, 1);
      float4 bcv[NL][kT / 2];
      read_b(sm, buf, k, bcv);
      const float zraw = (GATE && !SUMMARY) ? own_in(buf, 2) : 0.0f;
      float4 cv[4];
      if constexpr (FOLD) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          cv[i] = *reinterpret_cast<const float4*>(&sm.bt.c[buf][k][4 * i]);
      }

      const bool own_ok = chan_ok && k < nvalid_of(ci);
      if (CONV) {  // xu holds x_t here; u_t = silu(conv)
        const float xc = xu;
        // x_{t-s} is in lane k - s of this chunk for k >= s and in lane k - s + 16 of the
        // previous one otherwise: each source lane j offers this chunk's x if j < 16 - s, else
        // the previous chunk's, and one row rotation by s delivers it
        float acc = fmaf(cw_own, xc, cbias);
        acc = fmaf(cw[0], row_ror<1>(k < 15 ? xc : xprev), acc);
        acc = fmaf(cw[1], row_ror<2>(k < 14 ? xc : xprev), acc);
        acc = fmaf(cw[2], row_ror<3>(k < 13 ? xc : xprev), acc);
        xprev = xc;
        xu = silu_f(acc);
      }
      const float sv = sraw + bias;
      const float sp = softplus_f(sv);  // computed either way: a select, not a branch
      float dt = a.softplus ? sp : sv;
      dt = own_ok ? dt : 0.0f;  // steps past the end leave h unchanged
      // exact hold: the input term is u B_t[n] times the gain of hold_gain
      const float du = own_ok ? (ZOH ? xu : dt * xu) : 0.0f;
      if (SUMMARY) dt_acc += dt;

      steps(std::make_integer_sequence<int, kT>{}, sm, bcv, dt, du, A2, ia, h, wave, r, k);
      if constexpr (SUMMARY) {
        // The summary's steps store nothing, so the compiler would sink their arithmetic past
        // the next chunk's staging (a branch) while the row broadcasts, which cannot move across
        // control flow, stay above it; in different blocks the broadcasts are not folded into
        // the multiplies (32 extra moves per chunk).  Using the states here keeps them together.
#pragma unroll
        for (int j = 0; j < NL; ++j) asm volatile("" ::"v"(h[j]));
      }

      if (!SUMMARY) {
        wave_lds_sync();
        const float* pr = &sm.p[wave][r * kPRow + (k ^ (kPSwap * (r & 1))) * kPTau];
        const float4 q0 = *reinterpret_cast<const float4*>(pr + 0);
        const float4 q1 = *reinterpret_cast<const float4*>(pr + 4);
        const float4 q2 = *reinterpret_cast<const float4*>(pr + 8);
        const float4 q3 = *reinterpret_cast<const float4*>(pr + 12);
        float y;
        if constexpr (FOLD) {
          // q holds h_t[0..15] of this lane's step t = k; cv is C_t (row k of the C tile; the four
          // channels of the wave read the same row)
          const float4 c0 = cv[0], c1 = cv[1], c2 = cv[2], c3 = cv[3];
          wave_lds_sync();
          float y0 = c0.x * q0.x, y1 = c2.x * q2.x;
          y0 = fmaf(c0.y, q0.y, y0);
          y1 = fmaf(c2.y, q2.y, y1);
          y0 = fmaf(c0.z, q0.z, y0);
          y1 = fmaf(c2.z, q2.z, y1);
          y0 = fmaf(c0.w, q0.w, y0);
          y1 = fmaf(c2.w, q2.w, y1);
          y0 = fmaf(c1.x, q1.x, y0);
          y1 = fmaf(c3.x, q3.x, y1);
          y0 = fmaf(c1.y, q1.y, y0);
          y1 = fmaf(c3.y, q3.y, y1);
          y0 = fmaf(c1.z, q1.z, y0);
          y1 = fmaf(c3.z, q3.z, y1);
          y0 = fmaf(c1.w, q1.w, y0);
          y1 = fmaf(c3.w, q3.w, y1);
          y = y0 + y1;
        } else {
          wave_lds_sync();
          y = (((q0.x + q0.y) + (q0.z + q0.w)) + ((q1.x + q1.y) + (q1.z + q1.w))) +
              (((q2.x + q2.y) + (q2.z + q2.w)) + ((q3.x + q3.y) + (q3.z + q3.w)));
        }
        y = fmaf(dskip, xu, y);
        if (GATE) y *= silu_f(zraw);
        reinterpret_cast<elem*>(&sm.out[buf][k][0])[own_col] = IO::from_float(y);
      }
      hold_store();
      if (has_next) stage_chunk(buf ^ 1);
      // The chunk-end state goes out after the staging: a wait for the next chunk's loads also
      // waits for stores issued before it, and this one then has a whole chunk to complete.
      if ((!SUMMARY || states_only) && a.states && st_lane) {
        float* p = st_lane + int64_t(ci) * st_chunk;
#pragma unroll
        for (int j = 0; j < NL; ++j)
          if (k + 16 * j < a.d_state) p[16 * j] = h[j];
      }
      __syncthreads();
      store_out(buf, ci);
    };
    using Buf0 = std::integral_constant<int, 0>;
    using Buf1 = std::integral_constant<int, 1>;

    // Waves of different workgroups sharing a SIMD would otherwise be served oldest first, so
    // some finish early and the SIMD runs the end of the kernel with few waves.  A wave lowers
    // its issue priority by one at each quarter of its chunks, which keeps the waves of a SIMD
    // close together.  Quarter boundaries are even, so chunk pairs always start on buffer 0.
    int ci = 0;
    for (int qi = 0; qi < 4; ++qi) {
      switch (qi) {
        case 0: __builtin_amdgcn_s_setprio(3); break;
        case 1: __builtin_amdgcn_s_setprio(2); break;
        case 2: __builtin_amdgcn_s_setprio(1); break;
        default: __builtin_amdgcn_s_setprio(0); break;
      }
      const int c_end = qi == 3 ? nchunks : (((qi + 1) * nchunks) / 4) & ~1;
      for (; ci + 1 < c_end; ci += 2) {
        chunk(ci, Buf0{});
        chunk(ci + 1, Buf1{});
      }
      if (ci < c_end) {  // odd chunk count: the last chunk, on buffer 0
        chunk(ci, Buf0{});
        ++ci;
      }
    }
    __builtin_amdgcn_s_setprio(0);

    if (SUMMARY && !states_only) {
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
  // (B, C) pairs for this lane's states, two steps per float4 (with one state per lane and in
  // summary passes: B only, four steps per float4; with FOLD the lane stores its new state
  // instead of C_t[n] h_t[n]).
  template <int TAU>
  static __device__ __forceinline__ void step(Smem& sm, const float4 (&bcv)[NL][kT / 2],
                                              float dt, float du, const float (&A2)[NL],
                                              const float (&ia)[NL], float (&h)[NL], int wave,
                                              int r, int k) {
    const float dtb = row_bcast<TAU>(dt);
    const float dub = row_bcast<TAU>(du);
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      float bb, cc = 0.0f;
      if constexpr (SPLIT) {
        const float4 v = bcv[j][TAU / 4];
        bb = (TAU & 3) == 0 ? v.x : ((TAU & 3) == 1 ? v.y : ((TAU & 3) == 2 ? v.z : v.w));
      } else {
        const float4 v = bcv[j][TAU / 2];
        bb = (TAU & 1) ? v.z : v.x;
        cc = (TAU & 1) ? v.w : v.y;
      }
      const float y = dtb * A2[j];
      const float e = exp2_hw(y);
      const float inc = ZOH ? (dub * bb) * hold_gain(e, y, dtb, ia[j]) : dub * bb;
      h[j] = fmaf(e, h[j], inc);
      if constexpr (FOLD)
        p = h[j];
      else if constexpr (!SUMMARY)
        p = (j == 0) ? cc * h[j] : fmaf(cc, h[j], p);
    }
    if (!SUMMARY) {
      // slot TAU ^ kPSwap on odd rows
      const int flip = ((TAU ^ kPSwap) - TAU) * (r & 1) * kPTau;
      sm.p[wave][r * kPRow + k + flip + TAU * kPTau] = p;
    }
  }

  template <int... TAUS>
  static __device__ __forceinline__ void steps(std::integer_sequence<int, TAUS...>, Smem& sm,
                                               const float4 (&bcv)[NL][kT / 2], float dt,
                                               float du, const float (&A2)[NL],
                                               const float (&ia)[NL], float (&h)[NL], int wave,
                                               int r, int k) {
    (step<TAUS>(sm, bcv, dt, du, A2, ia, h, wave, r, k), ...);
  }

  // The B (one state per lane) or (B, C) tile entries of this lane's states for the 16 steps of
  // a chunk, read as 16-byte pieces so that the steps themselves are pure VALU work.
  static __device__ __forceinline__ void read_b(const Smem& sm, int buf, int k,
                                                float4 (&bcv)[NL][kT / 2]) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      if constexpr (SPLIT) {
#pragma unroll
        for (int i = 0; i < kT / 4; ++i)
          bcv[j][i] = *reinterpret_cast<const float4*>(&sm.bt.b[buf][k + 16 * j][4 * i]);
      } else {
#pragma unroll
        for (int i = 0; i < kT / 2; ++i)
          bcv[j][i] = *reinterpret_cast<const float4*>(&sm.bt.bc[buf][k + 16 * j][2 * i]);
      }
    }
  }
};

template <class IO, int NL, bool GATE, bool SUMMARY, bool VEC, bool ZOH, bool CONV>
__global__ void __launch_bounds__(kPrefillThreads) scan_kernel(ScanArgs a) {
  ScanKernel<IO, NL, GATE, SUMMARY, VEC, ZOH, CONV>::run(a);
}

template <class IO, int NL, bool VEC, bool ZOH, bool CONV>
hipError_t launch3(const ScanArgs& a, bool summary, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.n_wg)), block(kPrefillThreads);
  if (summary)
    hipLaunchKernelGGL((scan_kernel<IO, NL, false, true, VEC, ZOH, CONV>), grid, block, 0, stream,
                       a);
  else if (a.z != nullptr)
    hipLaunchKernelGGL((scan_kernel<IO, NL, true, false, VEC, ZOH, CONV>), grid, block, 0, stream,
                       a);
  else
    hipLaunchKernelGGL((scan_kernel<IO, NL, false, false, VEC, ZOH, CONV>), grid, block, 0,
                       stream, a);
  return hipGetLastError();
}

template <class IO, int NL, bool ZOH, bool CONV>
hipError_t launch2(const ScanArgs& a, bool summary, hipStream_t stream) {
  return a.vec_io ? launch3<IO, NL, true, ZOH, CONV>(a, summary, stream)
                  : launch3<IO, NL, false, ZOH, CONV>(a, summary, stream);
}

// Instance selection for one discretisation and front end: io dtype, state registers per lane
// (NL), 16-byte tile path, gate and pass.
template <bool ZOH, bool CONV>
hipError_t launch_scan_instances(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream) {
  const int nl = (a.d_state + 15) / 16;
  if (bf16) {
    switch (nl) {
      case 1: return launch2<BF16, 1, ZOH, CONV>(a, summary, stream);
      case 2: return launch2<BF16, 2, ZOH, CONV>(a, summary, stream);
      case 3: return launch2<BF16, 3, ZOH, CONV>(a, summary, stream);
      default: return launch2<BF16, 4, ZOH, CONV>(a, summary, stream);
    }
  }
  switch (nl) {
    case 1: return launch2<F32, 1, ZOH, CONV>(a, summary, stream);
    case 2: return launch2<F32, 2, ZOH, CONV>(a, summary, stream);
    case 3: return launch2<F32, 3, ZOH, CONV>(a, summary, stream);
    default: return launch2<F32, 4, ZOH, CONV>(a, summary, stream);
  }
}

}  // namespace
}  // namespace ss
