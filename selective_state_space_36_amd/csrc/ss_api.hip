// ss_api.hip -- the C ABI of libssscan.so (declared in include/ss_scan.h): argument checking,
// choice of the time split, workspace layout and kernel dispatch.  No allocation, no
// synchronisation, no printing: errors come back as status codes with a thread-local message.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "ss_scan.h"
#include "ss_bwd.h"
#include "ss_launch.h"
#include "ss_scan2.h"

// Scratch of ss_scan_fwd_noalloc: the time split's segment end states and step sums.  Each GPU
// holds its own copy from the library's first use on it until the process ends.  Host code never
// passes this name to a kernel (on the host it is only a stand-in); it uses the device address
// looked up once per device below.
static __device__ __align__(256) unsigned char scratch[SS_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

ss_status fail(ss_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ss_status fail(ss_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

ss_status ok() {
  g_err[0] = '\0';
  return SS_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* p, int64_t elems, int64_t esize) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + static_cast<uintptr_t>(elems * esize) : lo};
}

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of the current device's copy of `scratch`, looked up on first use.
ss_status static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SS_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SS_ERR_UNSUPPORTED, "device %d above the %d devices the static scratch serves",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SS_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return SS_OK;
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Automatic time split.  A shape with at least 2 waves per SIMD without a split runs unsplit:
// the summary pass would add most of a pass's work for little occupancy.  Fewer channels than
// that (long sequences, small batches) are cut into segments of >= 256 steps, enough for ~24
// waves per SIMD (about five rounds of the 5 workgroups per CU the kernel holds, which evens out
// the workgroups' finishing times; measured on the 2^20-step layer: 8 segments 13.9 ms, 13 12.6,
// 40 12.2, 64 11.9).
int32_t auto_nseg(int64_t batch, int64_t seqlen, int64_t d_inner) {
  if (batch <= 0 || seqlen <= 0 || d_inner <= 0) return 1;
  const int64_t simds = 4ll * cu_count();
  const int64_t waves_per_seg = batch * ((d_inner + ss::kChanPerWG - 1) / ss::kChanPerWG) * 4;
  if (waves_per_seg >= 2 * simds) return 1;
  int64_t nseg = (24 * simds + waves_per_seg - 1) / waves_per_seg;
  nseg = std::min<int64_t>(nseg, std::max<int64_t>(1, seqlen / 256));
  nseg = std::min<int64_t>(nseg, 4096);
  return static_cast<int32_t>(std::max<int64_t>(nseg, 1));
}

// Segment length (a multiple of the B/C tile) and the effective segment count for a request.
void segments(int64_t seqlen, int32_t want, int64_t* seg_len, int32_t* nseg) {
  if (want <= 1 || seqlen <= ss::kChunk) {
    *seg_len = std::max<int64_t>(seqlen, 1);
    *seg_len = (*seg_len + ss::kChunk - 1) / ss::kChunk * ss::kChunk;
    *nseg = 1;
    return;
  }
  int64_t len = (seqlen + want - 1) / want;
  len = (len + ss::kChunk - 1) / ss::kChunk * ss::kChunk;
  *seg_len = len;
  *nseg = static_cast<int32_t>((seqlen + len - 1) / len);
}

size_t ws_bytes(int64_t batch, int64_t d_inner, int64_t d_state, int32_t nseg) {
  if (nseg <= 1) return 0;
  const int64_t rows = batch * d_inner;
  const int64_t per = rows * d_state + rows;  // floats per summarised segment
  return static_cast<size_t>((nseg - 1) * per) * sizeof(float) + 256;
}

ss_status check_dtype(ss_dtype dt, int64_t* esize) {
  if (dt == SS_F32) { *esize = 4; return SS_OK; }
  if (dt == SS_BF16) { *esize = 2; return SS_OK; }
  return fail(SS_ERR_UNSUPPORTED, "unknown dtype %d", static_cast<int>(dt));
}

ss_status check_flags(uint32_t flags, uint32_t allowed = SS_FLAG_ZOH_EXACT) {
  if (flags & ~allowed)
    return fail(SS_ERR_UNSUPPORTED, "flag bits 0x%x not taken here", flags & ~allowed);
  return SS_OK;
}

ss_status scan_impl(const void* u, const void* delta, const float* A, const void* B,
                    const void* C, const float* D, const void* z, const float* delta_bias,
                    int delta_softplus, const float* h0, float* h_last, void* out, int64_t batch,
                    int64_t seqlen, int64_t d_inner, int64_t d_state, ss_dtype dtype,
                    void* workspace, size_t workspace_bytes, int32_t nseg_req, bool forced,
                    uint32_t flags, void* stream, const float* conv_w = nullptr,
                    const float* conv_b = nullptr, const void* x_prev = nullptr,
                    int32_t conv_k = 0, float* states = nullptr,
                    bool use_static_scratch = false) {
  int64_t es = 0;
  if (check_dtype(dtype, &es) != SS_OK) return SS_ERR_UNSUPPORTED;
  if (check_flags(flags) != SS_OK) return SS_ERR_UNSUPPORTED;
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 0)
    return fail(SS_ERR_INVALID_ARG, "negative size (batch=%lld seqlen=%lld d_inner=%lld "
                "d_state=%lld)", (long long)batch, (long long)seqlen, (long long)d_inner,
                (long long)d_state);
  if (d_state < 1 || d_state > 64)
    return fail(SS_ERR_UNSUPPORTED, "d_state=%lld outside 1..64", (long long)d_state);
  if (nseg_req < 0) return fail(SS_ERR_INVALID_ARG, "nseg=%d is negative", nseg_req);
  if (conv_w && (conv_k < 1 || conv_k > 4))
    return fail(SS_ERR_UNSUPPORTED, "conv_k=%d outside 1..4", conv_k);
  int64_t rows, elems, bc_elems, st_elems;
  if (!mul_ok(batch, d_inner, &rows) || !mul_ok(rows, seqlen, &elems) ||
      !mul_ok(batch * seqlen, d_state, &bc_elems) || !mul_ok(rows, d_state, &st_elems) ||
      !mul_ok(elems, 8, &elems) || !mul_ok(bc_elems, 8, &bc_elems))
    return fail(SS_ERR_INVALID_ARG, "sizes overflow 64-bit byte offsets");
  elems /= 8;
  bc_elems /= 8;
  // tiles of 16 steps are addressed with 32-bit byte offsets (16 * d_inner * 4 bytes < 2^31)
  // and chunks are counted in 32 bits
  if (d_inner > (int64_t(1) << 24))
    return fail(SS_ERR_UNSUPPORTED, "d_inner=%lld above 16777216", (long long)d_inner);
  if (seqlen > int64_t(0x7fffffff))
    return fail(SS_ERR_UNSUPPORTED, "seqlen=%lld above 2147483647", (long long)seqlen);
  if (batch == 0 || d_inner == 0) return ok();
  if (seqlen == 0) {
    if (h_last) {
      if (h0 && overlap(range("h0", h0, st_elems, 4), range("h_last", h_last, st_elems, 4)) &&
          h0 != h_last)
        return fail(SS_ERR_INVALID_ARG, "h_last overlaps h0");
      if (h0 != h_last) {
        const hipError_t e = ss::launch_copy_state(h_last, h0, st_elems,
                                                   static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(SS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
      }
    }
    return ok();
  }
  if (!u || !delta || !A || !B || !C || !out)
    return fail(SS_ERR_INVALID_ARG, "required pointer is NULL (u, delta, A, B, C and out are "
                "required)");
  const void* io_ptrs[] = {u, delta, B, C, z, out, x_prev};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es))
      return fail(SS_ERR_UNSUPPORTED, "io pointer %p not aligned to its %lld-byte element", p,
                  (long long)es);
  const void* f_ptrs[] = {A, D, delta_bias, h0, h_last, conv_w, conv_b};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return fail(SS_ERR_UNSUPPORTED, "float pointer %p misaligned", p);
  if (int64_t(d_inner) * d_state > (int64_t(1) << 40))
    return fail(SS_ERR_INVALID_ARG, "A too large");

  const Range ins[] = {range("u", u, elems, es), range("delta", delta, elems, es),
                       range("z", z, elems, es), range("B", B, bc_elems, es),
                       range("C", C, bc_elems, es), range("A", A, d_inner * d_state, 4),
                       range("D", D, d_inner, 4), range("delta_bias", delta_bias, d_inner, 4),
                       range("h0", h0, st_elems, 4),
                       range("conv_w", conv_w, d_inner * conv_k, 4),
                       range("conv_b", conv_w ? conv_b : nullptr, d_inner, 4),
                       range("x_prev", conv_w ? x_prev : nullptr, batch * (conv_k - 1) * d_inner, es)};
  const Range ro = range("out", out, elems, es);
  const Range rh = range("h_last", h_last, st_elems, 4);
  for (const Range& in : ins) {
    if (overlap(ro, in)) return fail(SS_ERR_INVALID_ARG, "out overlaps %s", in.name);
    if (overlap(rh, in)) return fail(SS_ERR_INVALID_ARG, "h_last overlaps %s", in.name);
  }
  if (overlap(ro, rh)) return fail(SS_ERR_INVALID_ARG, "out overlaps h_last");
  const int64_t nct = (seqlen + ss::kChunk - 1) / ss::kChunk;
  int64_t st_count = 0;
  if (states) {
    if (!aligned(states, 4)) return fail(SS_ERR_UNSUPPORTED, "states pointer misaligned");
    if (!mul_ok(rows, nct, &st_count) || !mul_ok(st_count, d_state * 4, &st_count))
      return fail(SS_ERR_INVALID_ARG, "states size overflows");
    st_count /= 4;
    const Range rs = range("states", states, st_count, 4);
    for (const Range& in : ins)
      if (overlap(rs, in)) return fail(SS_ERR_INVALID_ARG, "states overlaps %s", in.name);
    if (overlap(rs, ro) || overlap(rs, rh))
      return fail(SS_ERR_INVALID_ARG, "states overlaps out or h_last");
  }

  // time split
  int32_t want = forced && nseg_req > 0 ? nseg_req : auto_nseg(batch, seqlen, d_inner);
  int64_t seg_len = 0;
  int32_t nseg = 1;
  segments(seqlen, want, &seg_len, &nseg);
  if (forced && nseg_req > 0) {
    if (ws_bytes(batch, d_inner, d_state, nseg) > workspace_bytes || (nseg > 1 && !workspace))
      return fail(SS_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu bytes "
                  "needed for nseg=%d", workspace_bytes, ws_bytes(batch, d_inner, d_state, nseg),
                  nseg);
  } else {
    if (use_static_scratch) {
      // the allocation-free entry point: the automatic split must fit the static scratch
      const size_t need = ws_bytes(batch, d_inner, d_state, nseg);
      if (need > SS_NOALLOC_SCRATCH_BYTES)
        return fail(SS_ERR_INVALID_ARG, "the time split of this shape needs %zu bytes of "
                    "scratch, above the %u bytes of ss_scan_fwd_noalloc's static scratch (use "
                    "ss_scan_fwd with a workspace)", need, SS_NOALLOC_SCRATCH_BYTES);
      if (nseg > 1) {
        const ss_status s = static_scratch(&workspace);
        if (s != SS_OK) return s;
        workspace_bytes = SS_NOALLOC_SCRATCH_BYTES;
      }
    }
    // split only as far as the workspace allows
    while (nseg > 1 && (!workspace || ws_bytes(batch, d_inner, d_state, nseg) > workspace_bytes)) {
      want = std::max<int32_t>(1, want / 2);
      segments(seqlen, want, &seg_len, &nseg);
      if (want == 1) break;
    }
    if (nseg > 1 && (!workspace || ws_bytes(batch, d_inner, d_state, nseg) > workspace_bytes))
      segments(seqlen, 1, &seg_len, &nseg);
  }

  ss::ScanArgs a{};
  a.u = u; a.delta = delta; a.z = z; a.B = B; a.C = C; a.A = A; a.D = D;
  a.delta_bias = delta_bias; a.h0 = h0; a.h_last = h_last; a.out = out;
  a.batch = batch; a.seqlen = seqlen; a.d_inner = d_inner;
  a.seg_len = seg_len;
  a.n_cblk = (d_inner + ss::kChanPerWG - 1) / ss::kChanPerWG;
  a.d_state = static_cast<int32_t>(d_state);
  a.nseg = nseg;
  a.softplus = delta_softplus ? 1 : 0;
  a.zoh = (flags & SS_FLAG_ZOH_EXACT) ? 1 : 0;
  if (conv_w) {
    a.conv_w = conv_w;
    a.conv_b = conv_b;
    a.x_prev = conv_k > 1 ? x_prev : nullptr;
    a.conv_k = conv_k;
  }
  // 16-byte tile accesses need whole 16-channel blocks and 16-byte aligned rows
  a.vec_io = (d_inner % ss::kChanPerWG == 0 && (d_inner * es) % 16 == 0 && aligned(u, 16) &&
              aligned(delta, 16) && (!z || aligned(z, 16)) && aligned(out, 16)) ? 1 : 0;
  if (nseg > 1) {
    uintptr_t base = (reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255);
    a.seg_h = reinterpret_cast<float*>(base);
    a.seg_dt = a.seg_h + (nseg - 1) * rows * d_state;
    const Range rw = range("workspace", workspace, static_cast<int64_t>(workspace_bytes), 1);
    for (const Range& in : ins)
      if (overlap(rw, in)) return fail(SS_ERR_INVALID_ARG, "workspace overlaps %s", in.name);
    if (overlap(rw, ro) || overlap(rw, rh))
      return fail(SS_ERR_INVALID_ARG, "workspace overlaps an output");
    if (states && overlap(rw, range("states", states, st_count, 4)))
      return fail(SS_ERR_INVALID_ARG, "workspace overlaps states");
  }
  a.states = states;
  a.states_chunks = nct;
  const int64_t ncb = batch * a.n_cblk;
  if (ncb * nseg > int64_t(0x7fffffff))
    return fail(SS_ERR_INVALID_ARG, "too many workgroups (batch * d_inner too large)");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == SS_BF16;
  if (nseg > 1) {
    a.n_wg = ncb * (nseg - 1);
    const hipError_t e = ss::launch_scan(a, bf16, /*summary=*/true, st);
    if (e != hipSuccess) return fail(SS_ERR_HIP, "summary launch failed: %s", hipGetErrorString(e));
  }
  a.n_wg = ncb * nseg;
  const hipError_t e = ss::launch_scan(a, bf16, /*summary=*/false, st);
  if (e != hipSuccess) return fail(SS_ERR_HIP, "scan launch failed: %s", hipGetErrorString(e));
  return ok();
}

ss_status decode_impl(float* state, const void* u, const void* delta, const float* A,
                      const void* B, const void* C, const float* D, const void* z,
                      const float* delta_bias, int delta_softplus, void* out, int64_t batch,
                      int64_t d_inner, int64_t d_state, ss_dtype dtype, uint32_t flags,
                      void* stream, void* conv_state = nullptr, const float* conv_w = nullptr,
                      const float* conv_b = nullptr, int32_t conv_k = 0) {
  int64_t es = 0;
  if (check_dtype(dtype, &es) != SS_OK) return SS_ERR_UNSUPPORTED;
  if (check_flags(flags) != SS_OK) return SS_ERR_UNSUPPORTED;
  if (batch < 0 || d_inner < 0 || d_state < 0)
    return fail(SS_ERR_INVALID_ARG, "negative size");
  if (conv_w && (conv_k < 1 || conv_k > 4))
    return fail(SS_ERR_UNSUPPORTED, "conv_k=%d outside 1..4", conv_k);
  if (d_state < 1 || d_state > 64)
    return fail(SS_ERR_UNSUPPORTED, "d_state=%lld outside 1..64", (long long)d_state);
  int64_t rows, st_elems;
  if (!mul_ok(batch, d_inner, &rows) || !mul_ok(rows, d_state, &st_elems) ||
      !mul_ok(st_elems, 64, &st_elems))
    return fail(SS_ERR_INVALID_ARG, "sizes overflow");
  st_elems /= 64;
  if (rows == 0) return ok();
  if (!state || !u || !delta || !A || !B || !C || !out)
    return fail(SS_ERR_INVALID_ARG, "required pointer is NULL (state, u, delta, A, B, C, out)");
  if (conv_w && conv_k > 1 && !conv_state)
    return fail(SS_ERR_INVALID_ARG, "conv_state is NULL");
  const void* io_ptrs[] = {u, delta, B, C, z, out, conv_w ? conv_state : nullptr};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es)) return fail(SS_ERR_UNSUPPORTED, "io pointer %p misaligned", p);
  const void* f_ptrs[] = {state, A, D, delta_bias, conv_w, conv_b};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return fail(SS_ERR_UNSUPPORTED, "float pointer %p misaligned", p);
  const Range ins[] = {range("u", u, rows, es), range("delta", delta, rows, es),
                       range("z", z, rows, es), range("B", B, batch * d_state, es),
                       range("C", C, batch * d_state, es), range("A", A, d_inner * d_state, 4),
                       range("D", D, d_inner, 4), range("delta_bias", delta_bias, d_inner, 4),
                       range("conv_w", conv_w, d_inner * conv_k, 4),
                       range("conv_b", conv_w ? conv_b : nullptr, d_inner, 4)};
  const Range rs = range("state", state, st_elems, 4);
  const Range ro = range("out", out, rows, es);
  const Range rcs = range("conv_state", conv_w && conv_k > 1 ? conv_state : nullptr,
                          batch * (conv_k - 1) * d_inner, es);
  for (const Range& in : ins) {
    if (overlap(rs, in)) return fail(SS_ERR_INVALID_ARG, "state overlaps %s", in.name);
    if (overlap(ro, in)) return fail(SS_ERR_INVALID_ARG, "out overlaps %s", in.name);
    if (overlap(rcs, in)) return fail(SS_ERR_INVALID_ARG, "conv_state overlaps %s", in.name);
  }
  if (overlap(ro, rs)) return fail(SS_ERR_INVALID_ARG, "out overlaps state");
  if (overlap(rcs, rs) || overlap(rcs, ro))
    return fail(SS_ERR_INVALID_ARG, "conv_state overlaps state or out");

  ss::DecodeArgs a{};
  a.state = state; a.u = u; a.delta = delta; a.z = z; a.B = B; a.C = C; a.A = A; a.D = D;
  a.delta_bias = delta_bias; a.out = out;
  a.batch = batch; a.d_inner = d_inner; a.d_state = static_cast<int32_t>(d_state);
  int g = 1;
  while (g * 4 < d_state) g <<= 1;
  a.lanes_per_chan = g;
  a.softplus = delta_softplus ? 1 : 0;
  a.zoh = (flags & SS_FLAG_ZOH_EXACT) ? 1 : 0;
  const int64_t bc_align = dtype == SS_BF16 ? 8 : 16;  // four io elements of B and C
  // the vector path addresses a group of kDecodeRows batch rows of the state with 32-bit byte
  // offsets
  a.vec4 = (d_state % 4 == 0 && d_inner * d_state * 4 * ss::kDecodeRows < (int64_t(1) << 31) &&
            aligned(state, 16) && aligned(A, 16) && aligned(B, bc_align) &&
            aligned(C, bc_align)) ? 1 : 0;
  if (conv_w) {
    if (!a.vec4 || g < 4)
      return fail(SS_ERR_UNSUPPORTED, "the fused decode front end needs d_state a multiple of 4 "
                  "in 12..64 with 16-byte aligned state and A");
    a.conv_state = conv_k > 1 ? conv_state : nullptr;
    a.conv_w = conv_w;
    a.conv_b = conv_b;
    a.conv_k = conv_k;
  }
  if ((rows * g + 255) / 256 > int64_t(0x7fffffff))
    return fail(SS_ERR_INVALID_ARG, "too many rows");
  const hipError_t e = ss::launch_decode(a, dtype == SS_BF16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SS_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Backward workspace: the chunk-end states, then the per-workgroup partial sums of dB, dC and
// the per-batch-row partials of dA, dD, ddelta_bias (ss::bwd_layout).  0 for an empty problem
// (nothing to sum) or an unsupported d_state.
size_t bwd_ws_bytes(int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state) {
  if (batch <= 0 || seqlen <= 0 || d_inner <= 0 || d_state < 1 || d_state > 64) return 0;
  const int64_t nchunks = (seqlen + ss::kBwdChunk - 1) / ss::kBwdChunk;
  int64_t n;  // a bound on every term of the layout, in bytes
  if (!mul_ok(batch * (d_inner + 16), nchunks + 1, &n) || !mul_ok(n, 1024 * 8, &n)) return 0;
  return ss::bwd_layout(batch, seqlen, d_inner, d_state).total;
}

ss_status bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, int delta_softplus,
                   const float* h0, const void* dout, const float* dh_last, void* du,
                   void* ddelta, void* dz, float* dA, float* dB, float* dC, float* dD,
                   float* ddelta_bias, float* dh0, int64_t batch, int64_t seqlen,
                   int64_t d_inner, int64_t d_state, ss_dtype dtype, void* workspace,
                   size_t workspace_bytes, uint32_t flags, void* stream) {
  int64_t es = 0;
  if (check_dtype(dtype, &es) != SS_OK) return SS_ERR_UNSUPPORTED;
  if (check_flags(flags, SS_FLAG_ZOH_EXACT | SS_FLAG_STATES_GIVEN) != SS_OK)
    return SS_ERR_UNSUPPORTED;
  if ((flags & SS_FLAG_ZOH_EXACT) && (flags & SS_FLAG_STATES_GIVEN))
    return fail(SS_ERR_UNSUPPORTED, "SS_FLAG_STATES_GIVEN takes the first-order states of "
                "ss_scan_fwd_states; the exact-hold backward recomputes its own");
  if (batch < 0 || seqlen < 0 || d_inner < 0 || d_state < 0)
    return fail(SS_ERR_INVALID_ARG, "negative size");
  if (d_state < 1 || d_state > 64)
    return fail(SS_ERR_UNSUPPORTED, "backward: d_state=%lld outside 1..64", (long long)d_state);
  int64_t rows, elems, bc_elems, st_elems;
  if (!mul_ok(batch, d_inner, &rows) || !mul_ok(rows, seqlen, &elems) ||
      !mul_ok(batch * seqlen, d_state, &bc_elems) || !mul_ok(rows, d_state, &st_elems) ||
      !mul_ok(elems, 8, &elems) || !mul_ok(bc_elems, 8, &bc_elems))
    return fail(SS_ERR_INVALID_ARG, "sizes overflow 64-bit byte offsets");
  elems /= 8;
  bc_elems /= 8;
  if (d_inner > (int64_t(1) << 24))
    return fail(SS_ERR_UNSUPPORTED, "d_inner=%lld above 16777216", (long long)d_inner);
  if (seqlen > int64_t(0x7fffffff))
    return fail(SS_ERR_UNSUPPORTED, "seqlen=%lld above 2147483647", (long long)seqlen);
  if (!u || !delta || !A || !B || !C || !dout || !du || !ddelta || !dA || !dB || !dC)
    return fail(SS_ERR_INVALID_ARG, "required pointer is NULL (u, delta, A, B, C, dout, du, "
                "ddelta, dA, dB, dC are required)");
  if (z && !dz) return fail(SS_ERR_INVALID_ARG, "dz is required when z is given");
  const void* io_ptrs[] = {u, delta, B, C, z, dout, du, ddelta, dz};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es))
      return fail(SS_ERR_UNSUPPORTED, "io pointer %p not aligned to its %lld-byte element", p,
                  (long long)es);
  const void* f_ptrs[] = {A, D, delta_bias, h0, dh_last, dA, dB, dC, dD, ddelta_bias, dh0};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return fail(SS_ERR_UNSUPPORTED, "float pointer %p misaligned", p);
  const size_t need = bwd_ws_bytes(batch, seqlen, d_inner, d_state);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SS_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu bytes the "
                "backward needs (ss_scan_bwd_workspace_bytes)", workspace_bytes, need);
  if (need > 0 && !aligned(workspace, 16))
    return fail(SS_ERR_UNSUPPORTED, "workspace pointer %p not 16-byte aligned", workspace);
  const Range ins[] = {range("u", u, elems, es), range("delta", delta, elems, es),
                       range("z", z, elems, es), range("B", B, bc_elems, es),
                       range("C", C, bc_elems, es), range("A", A, d_inner * d_state, 4),
                       range("D", D, d_inner, 4), range("delta_bias", delta_bias, d_inner, 4),
                       range("h0", h0, st_elems, 4), range("dout", dout, elems, es),
                       range("dh_last", dh_last, st_elems, 4)};
  const Range outs[] = {range("du", du, elems, es), range("ddelta", ddelta, elems, es),
                        range("dz", z ? dz : nullptr, elems, es),
                        range("dA", dA, d_inner * d_state, 4), range("dB", dB, bc_elems, 4),
                        range("dC", dC, bc_elems, 4), range("dD", dD, d_inner, 4),
                        range("ddelta_bias", ddelta_bias, d_inner, 4),
                        range("dh0", dh0, st_elems, 4),
                        range("workspace", need ? workspace : nullptr,
                              static_cast<int64_t>(need), 1)};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return fail(SS_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name,
                                            in.name);
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j]))
        return fail(SS_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  ss::BwdArgs a{};
  a.u = u; a.delta = delta; a.z = z; a.B = B; a.C = C; a.dout = dout; a.A = A; a.D = D;
  a.delta_bias = delta_bias; a.h0 = h0; a.dh_last = dh_last; a.du = du; a.ddelta = ddelta;
  a.dz = z ? dz : nullptr; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD;
  a.ddelta_bias = ddelta_bias; a.dh0 = dh0; a.ck = static_cast<float*>(workspace);
  if (need > 0) {
    const ss::BwdLayout lay = ss::bwd_layout(batch, seqlen, d_inner, d_state);
    char* ws = static_cast<char*>(workspace);
    a.part_bc = reinterpret_cast<float*>(ws + lay.bc);
    a.part_a = reinterpret_cast<float*>(ws + lay.a);
    a.part_d = reinterpret_cast<float*>(ws + lay.d);
    a.part_b = reinterpret_cast<float*>(ws + lay.b);
  }
  a.batch = batch; a.seqlen = seqlen; a.d_inner = d_inner;
  a.n_cblk = (d_inner + 15) / 16;
  a.d_state = static_cast<int32_t>(d_state);
  a.softplus = delta_softplus ? 1 : 0;
  a.zoh = (flags & SS_FLAG_ZOH_EXACT) ? 1 : 0;
  // 16-byte tile loads of u, delta, z, dout and 16-byte tile stores of du, ddelta, dz
  a.vec_io = (d_inner % 16 == 0 && (d_inner * es) % 16 == 0 && aligned(u, 16) &&
              aligned(delta, 16) && aligned(dout, 16) && (!z || aligned(z, 16)) &&
              aligned(du, 16) && aligned(ddelta, 16) && (!dz || aligned(dz, 16))) ? 1 : 0;
  if (batch * a.n_cblk > int64_t(0x7fffffff))
    return fail(SS_ERR_INVALID_ARG, "too many workgroups (batch * d_inner too large)");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!(flags & SS_FLAG_STATES_GIVEN) && batch * seqlen * d_inner > 0) {
    // The forward pass that stores the chunk-end states runs as the prefill kernel's summary
    // instance in its states-only form (no segment buffers): the same recurrence at the
    // prefill's occupancy, five waves per SIMD against the backward kernel's three.
    ss::ScanArgs f{};
    f.u = u; f.delta = delta; f.B = B; f.C = C; f.A = A; f.delta_bias = delta_bias; f.h0 = h0;
    f.batch = batch; f.seqlen = seqlen; f.d_inner = d_inner;
    segments(seqlen, 1, &f.seg_len, &f.nseg);
    f.n_cblk = (d_inner + ss::kChanPerWG - 1) / ss::kChanPerWG;
    f.d_state = static_cast<int32_t>(d_state);
    f.softplus = a.softplus;
    f.zoh = a.zoh;
    f.vec_io = (d_inner % ss::kChanPerWG == 0 && (d_inner * es) % 16 == 0 && aligned(u, 16) &&
                aligned(delta, 16)) ? 1 : 0;
    f.states = static_cast<float*>(workspace);
    f.states_chunks = (seqlen + ss::kChunk - 1) / ss::kChunk;
    f.n_wg = batch * f.n_cblk;
    const hipError_t ef = ss::launch_scan(f, dtype == SS_BF16, /*summary=*/true, st);
    if (ef != hipSuccess)
      return fail(SS_ERR_HIP, "backward forward-pass launch failed: %s", hipGetErrorString(ef));
  }
  const hipError_t e = ss::launch_scan_bwd(a, dtype == SS_BF16, st);
  if (e != hipSuccess) return fail(SS_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

ss_status scan2_impl(const void* x, const void* dt, const float* A, const void* B,
                     const void* C, const float* D, const void* z, const float* dt_bias,
                     int dt_softplus, const float* h0, float* h_last, void* out, int64_t batch,
                     int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                     int64_t d_state, ss_dtype dtype, void* stream) {
  int64_t es = 0;
  if (check_dtype(dtype, &es) != SS_OK) return SS_ERR_UNSUPPORTED;
  if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 0 || ngroups < 0 || d_state < 0)
    return fail(SS_ERR_INVALID_ARG, "negative size");
  if (d_state < 1 || d_state > 256)
    return fail(SS_ERR_UNSUPPORTED, "d_state=%lld outside 1..256", (long long)d_state);
  if (nheads > 0 && (ngroups < 1 || nheads % ngroups != 0))
    return fail(SS_ERR_INVALID_ARG, "nheads=%lld is not a multiple of ngroups=%lld",
                (long long)nheads, (long long)ngroups);
  int64_t rows, elems, dt_elems, bc_elems, st_elems;
  if (!mul_ok(batch, nheads, &rows) || !mul_ok(rows * seqlen, headdim, &elems) ||
      !mul_ok(batch * seqlen, nheads, &dt_elems) ||
      !mul_ok(batch * seqlen * ngroups, d_state, &bc_elems) ||
      !mul_ok(rows * d_state, headdim, &st_elems) || !mul_ok(elems, 8, &elems))
    return fail(SS_ERR_INVALID_ARG, "sizes overflow 64-bit byte offsets");
  elems /= 8;
  if (batch == 0 || seqlen == 0 || nheads == 0 || headdim == 0) {
    if (h_last && st_elems > 0) {
      if (h0 && h0 != h_last &&
          overlap(range("h0", h0, st_elems, 4), range("h_last", h_last, st_elems, 4)))
        return fail(SS_ERR_INVALID_ARG, "h_last overlaps h0");
      if (h0 != h_last) {
        const hipError_t e =
            ss::launch_copy_state(h_last, h0, st_elems, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(SS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
      }
    }
    return ok();
  }
  // a 16-step tile of one head is addressed with 32-bit byte offsets
  if (int64_t(ss::kScan2Chunk) * nheads * headdim * 4 >= (int64_t(1) << 31) ||
      int64_t(ss::kScan2Chunk) * ngroups * d_state * 4 >= (int64_t(1) << 31) ||
      seqlen > int64_t(0x7fffffff))
    return fail(SS_ERR_UNSUPPORTED, "a 16-step tile exceeds 2 GiB (nheads * headdim or ngroups "
                "* d_state too large) or seqlen above 2147483647");
  if (!x || !dt || !A || !B || !C || !out)
    return fail(SS_ERR_INVALID_ARG, "required pointer is NULL (x, dt, A, B, C and out are "
                "required)");
  const void* io_ptrs[] = {x, dt, B, C, z, out};
  for (const void* p : io_ptrs)
    if (p && !aligned(p, es))
      return fail(SS_ERR_UNSUPPORTED, "io pointer %p not aligned to its %lld-byte element", p,
                  (long long)es);
  const void* f_ptrs[] = {A, D, dt_bias, h0, h_last};
  for (const void* p : f_ptrs)
    if (p && !aligned(p, 4)) return fail(SS_ERR_UNSUPPORTED, "float pointer %p misaligned", p);
  const Range ins[] = {range("x", x, elems, es), range("dt", dt, dt_elems, es),
                       range("z", z, elems, es), range("B", B, bc_elems, es),
                       range("C", C, bc_elems, es), range("A", A, nheads, 4),
                       range("D", D, nheads, 4), range("dt_bias", dt_bias, nheads, 4),
                       range("h0", h0, st_elems, 4)};
  const Range ro = range("out", out, elems, es);
  const Range rh = range("h_last", h_last, st_elems, 4);
  for (const Range& in : ins) {
    if (overlap(ro, in)) return fail(SS_ERR_INVALID_ARG, "out overlaps %s", in.name);
    if (overlap(rh, in)) return fail(SS_ERR_INVALID_ARG, "h_last overlaps %s", in.name);
  }
  if (overlap(ro, rh)) return fail(SS_ERR_INVALID_ARG, "out overlaps h_last");
  ss::Scan2Args a{};
  a.x = x; a.dt = dt; a.z = z; a.B = B; a.C = C; a.A = A; a.D = D; a.dt_bias = dt_bias;
  a.h0 = h0; a.h_last = h_last; a.out = out;
  a.batch = batch; a.seqlen = seqlen; a.nheads = nheads; a.headdim = headdim;
  a.ngroups = ngroups;
  a.n_pblk = (headdim + ss::kScan2PBlock - 1) / ss::kScan2PBlock;
  a.d_state = static_cast<int32_t>(d_state);
  a.softplus = dt_softplus ? 1 : 0;
  if (batch * nheads * a.n_pblk > int64_t(0x7fffffff))
    return fail(SS_ERR_INVALID_ARG, "too many workgroups");
  const bool bf16 = dtype == SS_BF16;
  const hipError_t e = ss::scan2_mfma_supported(a, bf16)
                           ? ss::launch_scan2_mfma(a, static_cast<hipStream_t>(stream))
                           : ss::launch_scan2(a, bf16, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

ss_status ss_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      int delta_softplus, const float* h0, float* h_last, void* out,
                      int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                      ss_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return scan_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, h_last, out, batch,
                   seqlen, d_inner, d_state, dtype, workspace, workspace_bytes, 0, false, 0,
                   stream);
}

ss_status ss_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                              const void* C, const float* D, const void* z,
                              const float* delta_bias, int delta_softplus, const float* h0,
                              float* h_last, void* out, int64_t batch, int64_t seqlen,
                              int64_t d_inner, int64_t d_state, ss_dtype dtype, void* stream) {
  return scan_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, h_last, out, batch,
                   seqlen, d_inner, d_state, dtype, nullptr, 0, 0, false, 0, stream, nullptr,
                   nullptr, nullptr, 0, nullptr, /*use_static_scratch=*/true);
}

size_t ss_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                   int64_t d_state, ss_dtype dtype) {
  (void)dtype;
  if (batch <= 0 || seqlen <= 0 || d_inner <= 0 || d_state < 1 || d_state > 64) return 0;
  int64_t seg_len;
  int32_t nseg;
  segments(seqlen, auto_nseg(batch, seqlen, d_inner), &seg_len, &nseg);
  return ws_bytes(batch, d_inner, d_state, nseg);
}

ss_status ss_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D, const void* z, const float* delta_bias,
                         int delta_softplus, const float* h0, float* h_last, void* out,
                         int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                         ss_dtype dtype, void* workspace, size_t workspace_bytes, int32_t nseg,
                         uint32_t flags, void* stream) {
  return scan_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, h_last, out, batch,
                   seqlen, d_inner, d_state, dtype, workspace, workspace_bytes, nseg, true, flags,
                   stream);
}

size_t ss_scan_fwd_ex_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                      int64_t d_state, ss_dtype dtype, int32_t nseg) {
  (void)dtype;
  if (batch <= 0 || seqlen <= 0 || d_inner <= 0 || d_state < 1 || d_state > 64) return 0;
  int64_t seg_len;
  int32_t n;
  segments(seqlen, nseg > 0 ? nseg : auto_nseg(batch, seqlen, d_inner), &seg_len, &n);
  return ws_bytes(batch, d_inner, d_state, n);
}

ss_status ss_scan_fwd_states(const void* u, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z,
                             const float* delta_bias, int delta_softplus, const float* h0,
                             float* h_last, void* out, float* states, int64_t batch,
                             int64_t seqlen, int64_t d_inner, int64_t d_state, ss_dtype dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!states && batch > 0 && seqlen > 0 && d_inner > 0)
    return fail(SS_ERR_INVALID_ARG, "states is NULL");
  return scan_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, h_last, out, batch,
                   seqlen, d_inner, d_state, dtype, workspace, workspace_bytes, 0, false, 0,
                   stream, nullptr, nullptr, nullptr, 0, states);
}

size_t ss_scan_fwd_states_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                int64_t d_state) {
  if (batch <= 0 || seqlen <= 0 || d_inner <= 0 || d_state < 1 || d_state > 64) return 0;
  int64_t n;
  if (!mul_ok(batch * d_inner, (seqlen + ss::kChunk - 1) / ss::kChunk, &n) ||
      !mul_ok(n, d_state * 4, &n))
    return 0;
  return static_cast<size_t>(n);
}

ss_status ss_scan_fwd_conv(const void* x, const float* conv_weight, const float* conv_bias,
                           const void* x_prev, int32_t conv_k, const void* delta, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* delta_bias, int delta_softplus, const float* h0,
                           float* h_last, void* out, int64_t batch, int64_t seqlen,
                           int64_t d_inner, int64_t d_state, ss_dtype dtype, void* workspace,
                           size_t workspace_bytes, int32_t nseg, uint32_t flags, void* stream) {
  if (!conv_weight) return fail(SS_ERR_INVALID_ARG, "conv_weight is NULL");
  return scan_impl(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, h_last, out, batch,
                   seqlen, d_inner, d_state, dtype, workspace, workspace_bytes, nseg, true, flags,
                   stream, conv_weight, conv_bias, x_prev, conv_k);
}

ss_status ss_state_update(float* state, const void* u, const void* delta, const float* A,
                          const void* B, const void* C, const float* D, const void* z,
                          const float* delta_bias, int delta_softplus, void* out,
                          int64_t batch, int64_t d_inner, int64_t d_state, ss_dtype dtype,
                          void* stream) {
  return decode_impl(state, u, delta, A, B, C, D, z, delta_bias, delta_softplus, out, batch,
                     d_inner, d_state, dtype, 0, stream);
}

ss_status ss_state_update_ex(float* state, const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D, const void* z,
                             const float* delta_bias, int delta_softplus, void* out,
                             int64_t batch, int64_t d_inner, int64_t d_state, ss_dtype dtype,
                             uint32_t flags, void* stream) {
  return decode_impl(state, u, delta, A, B, C, D, z, delta_bias, delta_softplus, out, batch,
                     d_inner, d_state, dtype, flags, stream);
}

size_t ss_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                   int64_t d_state, ss_dtype dtype) {
  (void)dtype;
  return bwd_ws_bytes(batch, seqlen, d_inner, d_state);
}

ss_status ss_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      int delta_softplus, const float* h0, const void* dout,
                      const float* dh_last, void* du, void* ddelta, void* dz, float* dA,
                      float* dB, float* dC, float* dD, float* ddelta_bias, float* dh0,
                      int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                      ss_dtype dtype, void* workspace, size_t workspace_bytes, uint32_t flags,
                      void* stream) {
  return bwd_impl(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, dout, dh_last, du,
                  ddelta, dz, dA, dB, dC, dD, ddelta_bias, dh0, batch, seqlen, d_inner, d_state,
                  dtype, workspace, workspace_bytes, flags, stream);
}

ss_status ss_scan2_fwd(const void* x, const void* dt, const float* A, const void* B,
                       const void* C, const float* D, const void* z, const float* dt_bias,
                       int dt_softplus, const float* h0, float* h_last, void* out,
                       int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t ngroups, int64_t d_state, ss_dtype dtype, void* stream) {
  return scan2_impl(x, dt, A, B, C, D, z, dt_bias, dt_softplus, h0, h_last, out, batch, seqlen,
                    nheads, headdim, ngroups, d_state, dtype, stream);
}

ss_status ss_state_update_conv(float* state, void* conv_state, const void* x,
                               const float* conv_weight, const float* conv_bias, int32_t conv_k,
                               const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias,
                               int delta_softplus, void* out, int64_t batch, int64_t d_inner,
                               int64_t d_state, ss_dtype dtype, uint32_t flags, void* stream) {
  if (!conv_weight) return fail(SS_ERR_INVALID_ARG, "conv_weight is NULL");
  return decode_impl(state, x, delta, A, B, C, D, z, delta_bias, delta_softplus, out, batch,
                     d_inner, d_state, dtype, flags, stream, conv_state, conv_weight, conv_bias,
                     conv_k);
}

const char* ss_status_string(ss_status s) {
  switch (s) {
    case SS_OK: return "ok";
    case SS_ERR_INVALID_ARG: return "invalid argument";
    case SS_ERR_UNSUPPORTED: return "unsupported argument";
    case SS_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* ss_last_error(void) { return g_err; }

int ss_version(void) { return 101; }

}  // extern "C"
