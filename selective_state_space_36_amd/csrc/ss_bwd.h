// ss_bwd.h -- host-side launch interface of the backward scan kernels (ss_scan_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

// Backward geometry: like the prefill, 16 lanes (one DPP row) per channel and 16 channels per
// 256-thread workgroup, time in 16-step chunks; d_state <= 64 as 1, 2 or 4 groups of 16 states
// per lane.
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
  float* dA;             // (d_inner, d_state): sum over batch rows
  float* dB;             // (batch, seqlen, d_state): sum over channels
  float* dC;             // (batch, seqlen, d_state): sum over channels
  float* dD;             // nullptr: not computed; sum over batch rows and steps
  float* ddelta_bias;    // nullptr: not computed; sum over batch rows and steps
  float* dh0;            // nullptr: not written
  const float* ck;       // workspace: (batch, nchunks, d_inner, d_state) chunk-end states
  // Per-workgroup partial sums in the workspace, added in a fixed order by the reduction
  // kernels (no atomics: the summed gradients are bit-reproducible):
  float* part_bc;        // (batch, nchunks, n_cblk, kBwdChunk, np, 2): dB, dC of 16 channels,
                         // np = bwd_states_padded(d_state)
  float* part_a;         // (batch, d_inner, d_state): dA of one batch row
  float* part_d;         // (batch, d_inner): dD of one batch row
  float* part_b;         // (batch, d_inner): ddelta_bias of one batch row
  int64_t batch, seqlen, d_inner;
  int64_t n_cblk;        // channel blocks of 16 per batch row
  int32_t d_state;
  int32_t softplus;
  int32_t zoh;           // exact zero-order-hold input term instead of dt B u
  int32_t vec_io;        // whole 16-channel blocks with 16-byte aligned rows of u, delta, z, dout
};

// States per channel as the backward kernel lays them out: 16, 32 or 64.
inline int bwd_states_padded(int64_t d_state) { return d_state <= 16 ? 16 : d_state <= 32 ? 32 : 64; }

// Workspace of the backward: the chunk-end states, then the partial sums (256-byte aligned).
struct BwdLayout {
  size_t states, bc, a, d, b, total;  // byte offsets (states at 0) and the total size
};
inline BwdLayout bwd_layout(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const int64_t nch = (seqlen + kBwdChunk - 1) / kBwdChunk, ncb = (d_inner + 15) / 16;
  BwdLayout l{};
  l.states = 0;
  l.bc = up(size_t(batch) * nch * d_inner * d_state * 4);
  l.a = up(l.bc + size_t(batch) * nch * ncb * kBwdChunk * bwd_states_padded(d_state) * 2 * 4);
  l.d = up(l.a + size_t(batch) * d_inner * d_state * 4);
  l.b = up(l.d + size_t(batch) * d_inner * 4);
  l.total = up(l.b + size_t(batch) * d_inner * 4);
  return l;
}

// Run the reverse pass (one workgroup per 16 channels of a batch row) from the chunk-end states
// in ck, then add the partial sums into dA, dB, dC, dD and ddelta_bias.
hipError_t launch_scan_bwd(const BwdArgs& a, bool bf16, hipStream_t stream);

}  // namespace ss
