// ss_bwd.h -- host-side launch interface of the backward scan kernels (ss_scan_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

// Backward geometry: like the prefill, 16 lanes (one DPP row) per channel and 16 channels per
// 256-thread workgroup, time in 16-step chunks; d_state <= 16.
constexpr int kBwdThreads = 256;
constexpr int kBwdChunk = 16;

struct BwdArgs {
  const void* u;
  const void* delta;
  const void* z;         // nullptr: no gate
  const void* B;
  const void* C;
  const void* dout;      // upstream gradient of out, io dtype
  const float* A;
  const float* D;        // nullptr: 0
  const float* delta_bias;
  const float* h0;       // nullptr: zeros
  const float* dh_last;  // nullptr: 0
  void* du;              // io dtype
  void* ddelta;          // io dtype
  void* dz;              // io dtype, required with z
  float* dA;             // accumulated (zeroed by the launch)
  float* dB;             // (batch, seqlen, d_state), accumulated
  float* dC;             // (batch, seqlen, d_state), accumulated
  float* dD;             // nullptr: not computed; accumulated
  float* ddelta_bias;    // nullptr: not computed; accumulated
  float* dh0;            // nullptr: not written
  const float* ck;       // workspace: (batch, nchunks, d_inner, d_state) chunk-end states
  int64_t batch, seqlen, d_inner;
  int64_t n_cblk;        // channel blocks of 16 per batch row
  int32_t d_state;
  int32_t softplus;
  int32_t vec_io;        // whole 16-channel blocks with 16-byte aligned rows of u, delta, z, dout
};

// Zero the accumulated outputs, then run the reverse pass (one workgroup per 16 channels of a
// batch row) from the chunk-end states in ck.
hipError_t launch_scan_bwd(const BwdArgs& a, bool bf16, hipStream_t stream);

}  // namespace ss
