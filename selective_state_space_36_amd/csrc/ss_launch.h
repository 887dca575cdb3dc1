// ss_launch.h -- host-side launch interface between the C-ABI layer (ss_api.hip) and the kernel
// translation units.  Argument validation happens before these are called; they only pick the
// kernel instance and enqueue it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

// Geometry of the prefill kernels: 16 lanes (one DPP row) per channel, 4 channels per wave,
// 4 waves (16 channels) per workgroup, time processed in 16-step chunks.
constexpr int kPrefillThreads = 256;
constexpr int kChanPerWG = 16;
constexpr int kChunk = 16;

struct ScanArgs {
  const void* u;
  const void* delta;
  const void* z;       // nullptr: no gate
  const void* B;
  const void* C;
  const float* A;
  const float* D;      // nullptr: 0
  const float* delta_bias;  // nullptr: 0
  const float* h0;     // nullptr: zeros
  float* h_last;       // nullptr: not written
  void* out;
  // summary pass: (nseg-1, batch, d_inner, d_state) local end state and (nseg-1, batch, d_inner)
  // sum of dt of each segment; seg_h == nullptr selects the states-only pass instead (one
  // segment, from h0, writing every chunk-end state to `states` and nothing else)
  float* seg_h;
  float* seg_dt;
  int64_t batch, seqlen, d_inner;
  int64_t seg_len;     // multiple of kChunk
  int64_t n_cblk;      // channel blocks per batch row = ceil(d_inner / kChanPerWG)
  int64_t n_wg;        // workgroups of the launch
  int32_t d_state;
  int32_t nseg;
  int32_t softplus;
  int32_t vec_io;      // whole 16-channel blocks with 16-byte aligned rows of u, delta, z, out
  int32_t zoh;         // exact zero-order-hold input term instead of dt * B
  // front end (conv_w != nullptr): u holds the block's x; u = silu(causal conv of x + conv_b)
  const float* conv_w;  // (d_inner, conv_k)
  const float* conv_b;  // (d_inner), nullptr: 0
  const void* x_prev;   // (batch, conv_k - 1, d_inner) io dtype: x before t = 0; nullptr: 0
  int32_t conv_k;       // 1..4
  // chunk-end states: (batch, states_chunks, d_inner, d_state); nullptr: none
  float* states;
  int64_t states_chunks;  // ceil(seqlen / kChunk)
};

// Batch rows each thread of the decode step's vector path walks (a group of rows of the state
// is addressed with 32-bit byte offsets, so the host admits that path only when kDecodeRows
// rows of the state stay under 2^31 bytes).
#ifndef SS_DECODE_ROWS
#define SS_DECODE_ROWS 8
#endif
constexpr int kDecodeRows = SS_DECODE_ROWS;

struct DecodeArgs {
  float* state;
  const void* u;
  const void* delta;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* D;
  const float* delta_bias;
  void* out;
  int64_t batch, d_inner;
  int32_t d_state;
  int32_t lanes_per_chan;  // power of two >= ceil(d_state / 4)
  int32_t softplus;
  int32_t vec4;            // d_state % 4 == 0 and 16-byte aligned state/A
  int32_t zoh;             // exact zero-order-hold input term instead of dt * B
  // front end (conv_w != nullptr, vector path with lanes_per_chan >= 4 only): u holds the
  // block's x; u = silu(causal conv over [conv_state, x] + conv_b), conv_state shifted in place
  void* conv_state;        // (batch, conv_k - 1, d_inner) io dtype
  const float* conv_w;     // (d_inner, conv_k)
  const float* conv_b;     // (d_inner), nullptr: 0
  int32_t conv_k;          // 1..4
};

// Prefill passes.  `summary` selects the first pass of a time-split scan (segments 0..nseg-2,
// local end states and dt sums into seg_h/seg_dt); otherwise the output pass over all segments.
hipError_t launch_scan(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream);
hipError_t launch_scan_zoh(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream);
hipError_t launch_scan_conv(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream);
hipError_t launch_scan_conv_zoh(const ScanArgs& a, bool bf16, bool summary, hipStream_t stream);

// Fill h_last with h0 (or zeros) when the sequence is empty.
hipError_t launch_copy_state(float* dst, const float* src, int64_t n, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, bool bf16, hipStream_t stream);

}  // namespace ss
