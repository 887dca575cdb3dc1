// ss_scan2.h -- host-side launch interface of the multi-head scalar-transition scan
// (ss_scan2.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr int kScan2Threads = 256;
constexpr int kScan2Chunk = 16;
constexpr int kScan2PBlock = 16;  // head channels per workgroup
constexpr int kScan2MaxPieces = 4;  // time pieces a (batch row, head) pair is cut into, at most

struct Scan2Args {
  const void* x;         // (batch, seqlen, nheads, headdim) io dtype
  const void* dt;        // (batch, seqlen, nheads) io dtype
  const void* z;         // (batch, seqlen, nheads, headdim) io dtype; nullptr: no gate
  const void* B;         // (batch, seqlen, ngroups, d_state) io dtype
  const void* C;
  const float* A;        // (nheads)
  const float* D;        // (nheads); nullptr: 0
  const float* dt_bias;  // (nheads); nullptr: 0
  const float* h0;       // (batch, nheads, d_state, headdim); nullptr: zeros
  float* h_last;         // (batch, nheads, d_state, headdim); nullptr: not written
  void* out;             // (batch, seqlen, nheads, headdim) io dtype
  int64_t batch, seqlen, nheads, headdim, ngroups;
  int64_t n_pblk;        // ceil(headdim / kScan2PBlock)
  int32_t d_state;
  int32_t softplus;
  // chunked kernel only (set by its launcher): the first n_whole (batch row, head) pairs run
  // whole, each of the others in q_split time pieces, piece k over the chunks
  // [piece_beg[k], piece_beg[k + 1])
  int64_t n_whole;
  int32_t q_split;
  int32_t piece_beg[kScan2MaxPieces + 1];
};

hipError_t launch_scan2(const Scan2Args& a, bool bf16, hipStream_t stream);

// The chunked form on the matrix cores (ss_scan2_mfma.hip): bf16 io, headdim 64, d_state 64 or
// 128, 16-byte aligned x, z, out, B and C.
constexpr int kScan2MfmaChunk = 64;
bool scan2_mfma_supported(const Scan2Args& a, bool bf16);
hipError_t launch_scan2_mfma(const Scan2Args& a, hipStream_t stream);

}  // namespace ss
