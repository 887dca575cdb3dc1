/*
 * ss_scan.h -- C ABI of the MI355X (gfx950) selective state-space scan library (libssscan.so).
 *
 * The operation (Mamba's selective SSM, "S6"), for every batch row b and channel d:
 *
 *     dt_t    = softplus(delta[b,t,d] + delta_bias[d])      (or the raw sum, softplus off)
 *     h_t[n]  = exp(dt_t * A[d,n]) * h_{t-1}[n] + dt_t * B[b,t,n] * u[b,t,d]
 *     y_t     = sum_n C[b,t,n] * h_t[n] + D[d] * u[b,t,d]
 *     out     = y_t * silu(z[b,t,d])                        (when z is given)
 *
 * Sources (web pages; cited by title and section):
 *   - "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" reading guide
 *     (xyznot.com): "Método" (continuous SSM, ZOH discretisation Abar = exp(dt A), the
 *     recurrence and y_t = C h_t), "O Mecanismo de Seleção (S6)" (B_t, C_t and dt_t depend on the
 *     input; dt = softplus(Parameter + s(x))), "Expansão de Estado Ciente de Hardware" (the
 *     (batch, L, d_inner, d_state) state is never written to HBM; the output is contracted with C
 *     first), "Perguntas" (decode keeps a fixed d_inner x d_state state per layer, O(1) per token).
 *   - "O que é um modelo Mamba?" (ibm.com): the output equation with the D term, the diagonal A,
 *     and the Mamba block in which the SSM output is multiplied by the activated gate z.
 *   - "Как работает Mamba" (aivaro.ru), section 3 "Selective Scan": the function shape
 *     selective_scan(u, delta, A, B, C, D) with u, delta [batch, length, d_in] and B, C
 *     [batch, length, d_state], and the first-order input term B_bar = delta * B.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller; arrays are contiguous and row-major.
 *     The library allocates no device memory and keeps no state between calls (the one
 *     exception: the static scratch array of ss_scan_fwd_noalloc, described there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls only enqueue
 *     work and return; they never synchronise, print or throw.
 *   - Argument errors are detected before anything is launched and leave all outputs untouched.
 *     A launch failure is reported as SS_ERR_HIP.  ss_last_error() gives a thread-local message.
 *   - All index arithmetic is 64-bit.  Calls are thread-safe.
 *   - Element types: SS_F32 (float) or SS_BF16 (bfloat16 bits) for u, delta, z, B, C and out;
 *     A, D, delta_bias, the state, h0 and h_last are always float32.  Arithmetic and the state
 *     are float32; out is rounded to its dtype with round-to-nearest-even.
 */
#ifndef SS_SCAN_H
#define SS_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SS_OK = 0,
  SS_ERR_INVALID_ARG = 1, /* NULL required pointer, negative or inconsistent size, aliasing */
  SS_ERR_UNSUPPORTED = 2, /* d_state outside 1..64, unknown dtype or flag, misaligned element */
  SS_ERR_HIP = 3          /* the HIP runtime reported an error while launching */
} ss_status;

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

/*
 * Option bits (an entry point given a bit it does not take -> SS_ERR_UNSUPPORTED).
 *   SS_FLAG_ZOH_EXACT (prefill and decode): the input term uses the exact zero-order-hold
 *     discretisation of the continuous system (reading guide, "Método": B_bar =
 *     (dt A)^-1 (exp(dt A) - I) dt B, which for the diagonal A is B_bar[n] =
 *     (exp(dt A[d,n]) - 1) / A[d,n] * B[n], and dt * B[n] where A[d,n] == 0) in place of the
 *     first-order dt * B[n] of the default (aivaro.ru, section 3).  A_bar = exp(dt A) either
 *     way.  It costs a few more operations per state update.
 *   SS_FLAG_STATES_GIVEN (ss_scan_bwd only): the workspace already begins with the chunk-end
 *     states of these inputs, as written by ss_scan_fwd_states; the backward then skips its own
 *     forward pass.
 */
enum { SS_FLAG_ZOH_EXACT = 1, SS_FLAG_STATES_GIVEN = 2 };

/*
 * Prefill: the whole sequence in one call.
 *
 *   u, delta, z, out : (batch, seqlen, d_inner), io dtype.  z == NULL: no gate.
 *   B, C             : (batch, seqlen, d_state), io dtype, shared by all channels.
 *   A                : (d_inner, d_state) float32, the diagonal of each channel's A.
 *   D                : (d_inner) float32, skip weight; NULL means 0.
 *   delta_bias       : (d_inner) float32, added to delta before softplus; NULL means 0.
 *   delta_softplus   : nonzero -> dt = softplus(delta + bias); zero -> dt = delta + bias.
 *   h0               : (batch, d_inner, d_state) float32 initial state; NULL means zeros.
 *   h_last           : (batch, d_inner, d_state) float32 final state, written if non-NULL.
 *   workspace        : optional device scratch for splitting long sequences in time.  Size it
 *                      with ss_scan_fwd_workspace_bytes(); with less (or NULL/0) the library
 *                      splits less (or not at all): the result is the same up to rounding,
 *                      only slower on shapes with few channels.
 * out and h_last must not overlap any input or each other (SS_ERR_INVALID_ARG).
 * d_state outside 1..64, d_inner above 2^24 or seqlen above 2^31 - 1 -> SS_ERR_UNSUPPORTED.
 * batch == 0, seqlen == 0 or d_inner == 0 is a no-op returning SS_OK (with seqlen == 0 and
 * h_last given, h_last receives h0, or zeros).
 */
ss_status ss_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      int delta_softplus, const float* h0, float* h_last, void* out,
                      int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                      ss_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes ss_scan_fwd can use for this shape (0 when it would not split in time). */
size_t ss_scan_fwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                   int64_t d_state, ss_dtype dtype);

/*
 * Prefill that allocates nothing, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The same operation,
 * arguments and results as ss_scan_fwd, without the workspace: when the automatic time split
 * is used (shapes with few channels and long sequences), its segment end states and step sums
 * live in a static device array of SS_NOALLOC_SCRATCH_BYTES bytes inside the library, one per
 * GPU, held from its first use on that GPU until the process ends.
 *   - The array of the calling thread's current device is used; `stream` must belong to that
 *     device.  Its address is looked up once per device (hipGetSymbolAddress) and cached.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 *     different streams, or from several threads) race on it and give wrong results.  Calls
 *     ordered on one stream are safe; nothing in the array needs to start at zero.
 *   - 8 MiB holds the automatic split of every shape with d_state <= 16 on a 256-CU MI355X
 *     (the split targets about 24 waves per SIMD with 4 channels per wave, so its carries stay
 *     below 98304 rows of d_state + 1 floats, 6.7 MB).  A shape whose split needs more (d_state
 *     above 16 with few channels and long sequences) -> SS_ERR_INVALID_ARG before any launch;
 *     ss_scan_fwd with a workspace takes every shape.
 *   - No hipMalloc, hipFree or other allocating call is made.
 */
#define SS_NOALLOC_SCRATCH_BYTES (8u << 20)
ss_status ss_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                              const void* C, const float* D, const void* z,
                              const float* delta_bias, int delta_softplus, const float* h0,
                              float* h_last, void* out, int64_t batch, int64_t seqlen,
                              int64_t d_inner, int64_t d_state, ss_dtype dtype, void* stream);

/*
 * Prefill with an explicit time split and options.  nseg > 0 forces the sequence to be cut into
 * that many segments (each scanned from a carried state; the carries come from a first summary
 * pass over the segments, the blockwise associative decomposition of the recurrence); nseg == 0
 * chooses automatically.  Used to check that the result does not depend on the split.  With
 * nseg > 1 the workspace must hold ss_scan_fwd_ex_workspace_bytes(..., nseg) bytes
 * (SS_ERR_INVALID_ARG otherwise).  flags: SS_FLAG_* bits (0 = the ss_scan_fwd operation).
 */
ss_status ss_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D, const void* z, const float* delta_bias,
                         int delta_softplus, const float* h0, float* h_last, void* out,
                         int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                         ss_dtype dtype, void* workspace, size_t workspace_bytes, int32_t nseg,
                         uint32_t flags, void* stream);

size_t ss_scan_fwd_ex_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                      int64_t d_state, ss_dtype dtype, int32_t nseg);

/*
 * Prefill that also saves the state after every 16-step chunk, for a later backward (the
 * reading guide, "Expansão de Estado Ciente de Hardware", keeps intermediate states out of
 * memory and recomputes them in the backward pass; the chunk-end states are the points the
 * recomputation restarts from).  As ss_scan_fwd (first-order input term), plus:
 *   states : (batch, ceil(seqlen / 16), d_inner, d_state) float32, written: states[b,c,d,:] is
 *            the state after step min(16 c + 15, seqlen - 1).  Caller-owned, of
 *            ss_scan_fwd_states_bytes() bytes; it must not overlap the inputs, out, h_last or
 *            the workspace.  It is exactly the first part of the workspace
 *            ss_scan_bwd takes with SS_FLAG_STATES_GIVEN: a training step points `states` at the
 *            start of a buffer of ss_scan_bwd_workspace_bytes() bytes and passes that buffer to
 *            the backward.
 */
ss_status ss_scan_fwd_states(const void* u, const void* delta, const float* A, const void* B,
                             const void* C, const float* D, const void* z,
                             const float* delta_bias, int delta_softplus, const float* h0,
                             float* h_last, void* out, float* states, int64_t batch,
                             int64_t seqlen, int64_t d_inner, int64_t d_state, ss_dtype dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the states ss_scan_fwd_states writes for this shape (0 for an empty problem). */
size_t ss_scan_fwd_states_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                int64_t d_state);

/*
 * Prefill with the block's front end fused in: instead of u the call takes the block's x and
 * forms the SSM input itself (IBM explainer, Mamba-block walk-through: x_proj passes a
 * one-dimensional convolution, then SiLU, and the result feeds the SSM):
 *
 *     u[b,t,d] = silu( conv_bias[d] + sum_{j<conv_k} conv_weight[d,j] * x[b, t-conv_k+1+j, d] )
 *
 * a causal (step t sees x up to t), depthwise (one kernel per channel) convolution of width
 * conv_k in 1..4 (the pages give no width; 4 is the usual choice).  u is kept in float32 and
 * never written to memory.  Everything else is ss_scan_fwd_ex with u replaced by:
 *   x            : (batch, seqlen, d_inner), io dtype.
 *   conv_weight  : (d_inner, conv_k) float32, required.
 *   conv_bias    : (d_inner) float32; NULL means 0.
 *   x_prev       : (batch, conv_k - 1, d_inner), io dtype: the conv_k - 1 inputs that came
 *                  before t = 0 (oldest first), e.g. the end of the previous call's x; NULL
 *                  means zeros.
 * conv_k outside 1..4 -> SS_ERR_UNSUPPORTED; conv_weight NULL -> SS_ERR_INVALID_ARG.
 */
ss_status ss_scan_fwd_conv(const void* x, const float* conv_weight, const float* conv_bias,
                           const void* x_prev, int32_t conv_k, const void* delta, const float* A,
                           const void* B, const void* C, const float* D, const void* z,
                           const float* delta_bias, int delta_softplus, const float* h0,
                           float* h_last, void* out, int64_t batch, int64_t seqlen,
                           int64_t d_inner, int64_t d_state, ss_dtype dtype, void* workspace,
                           size_t workspace_bytes, int32_t nseg, uint32_t flags, void* stream);

/*
 * Decode: advance a resident state by ONE token (the recurrence above for a single t).
 *
 *   state        : (batch, d_inner, d_state) float32, read and overwritten IN PLACE.
 *   u, delta, z  : (batch, d_inner), io dtype; z == NULL: no gate.
 *   B, C         : (batch, d_state), io dtype.
 *   out          : (batch, d_inner), io dtype.
 *   A, D, delta_bias, delta_softplus, dtype, stream: as for ss_scan_fwd.
 * out must not overlap state or the inputs.
 */
ss_status ss_state_update(float* state, const void* u, const void* delta, const float* A,
                          const void* B, const void* C, const float* D, const void* z,
                          const float* delta_bias, int delta_softplus, void* out,
                          int64_t batch, int64_t d_inner, int64_t d_state, ss_dtype dtype,
                          void* stream);

/* Decode with options: flags are SS_FLAG_* bits (0 = the ss_state_update operation). */
ss_status ss_state_update_ex(float* state, const void* u, const void* delta, const float* A,
                             const void* B, const void* C, const float* D, const void* z,
                             const float* delta_bias, int delta_softplus, void* out,
                             int64_t batch, int64_t d_inner, int64_t d_state, ss_dtype dtype,
                             uint32_t flags, void* stream);

/*
 * Backward of the prefill (first-order or exact-hold input term): given dout = dL/d out (and optionally
 * dh_last = dL/d h_last), the gradients of every input.  Reverse-mode differentiation of the
 * recurrence above (reading guide, "Método"), with the states recomputed from stored chunk-end
 * states rather than kept (reading guide, "Expansão de Estado Ciente de Hardware": recomputation
 * in the backward pass):
 *     lam_t[n] = gy_t C_t[n] + exp(dt_{t+1} A[d,n]) lam_{t+1}[n],  gy_t = dout_t silu(z_t)
 *     du_t = gy_t D + dt_t sum_n lam_t B_t,  ddt_t = sum_n lam_t (A e_t h_{t-1} + B_t u_t)
 *     ddelta_t = ddt_t sigmoid(delta_t + bias) (softplus') or ddt_t,  dz_t = dout_t y_t silu'(z_t)
 *     dB_t += lam_t dt_t u_t,  dC_t += gy_t h_t (over channels),  dA += lam_t dt_t e_t h_{t-1},
 *     dD += gy_t u_t,  ddelta_bias += ddelta_t,  dh0 = e_0 lam_0.
 *
 *   inputs            : exactly as given to ss_scan_fwd (u, delta, A, B, C, D, z, delta_bias,
 *                       delta_softplus, h0, sizes, dtype).
 *   dout              : (batch, seqlen, d_inner) io dtype, required.
 *   dh_last           : (batch, d_inner, d_state) float32; NULL means 0.
 *   du, ddelta        : (batch, seqlen, d_inner) io dtype, required, overwritten.
 *   dz                : (batch, seqlen, d_inner) io dtype, required iff z is given.
 *   dA                : (d_inner, d_state) float32, required, overwritten.
 *   dB, dC            : (batch, seqlen, d_state) float32, required, overwritten.
 *   dD, ddelta_bias   : (d_inner) float32, overwritten when non-NULL (the gradient at the given
 *                       D / bias, also when D or delta_bias is NULL, i.e. 0).
 *   dh0               : (batch, d_inner, d_state) float32, written when non-NULL.
 *   workspace         : 16-byte aligned device scratch of ss_scan_bwd_workspace_bytes() bytes,
 *                       required when that is non-zero (SS_ERR_INVALID_ARG if smaller): first
 *                       the chunk-end states, (batch, ceil(seqlen / 16), d_inner, d_state)
 *                       floats, then the partial sums of dB and dC per 16-channel block and of
 *                       dA, dD, ddelta_bias per batch row.  Without SS_FLAG_STATES_GIVEN the
 *                       call first writes the states there with a forward pass (a launch of its
 *                       own on the stream), then runs the reverse pass and two reductions.
 * dA, dB, dC, dD and ddelta_bias are sums over channels or batch rows: each workgroup writes its
 * partial sum and a second kernel adds the partials in a fixed order, so every output is
 * bit-for-bit reproducible.  flags: SS_FLAG_ZOH_EXACT gives the gradients of the exact-hold
 * input term g_t B_t u_t, g_t = (exp(dt_t A) - 1) / A (then ddt_t = sum_n lam_t e_t (A h_{t-1} +
 * B_t u_t), du_t = gy_t D + sum_n lam_t g_t B_t, dB_t += lam_t g_t u_t and dA adds
 * lam_t (dt e_t - g_t) / A B_t u_t); SS_FLAG_STATES_GIVEN as below, not together with the exact
 * hold (ss_scan_fwd_states saves first-order states): SS_ERR_UNSUPPORTED.  d_state above 64 ->
 * SS_ERR_UNSUPPORTED.
 * Outputs must not overlap inputs, each other or the workspace.
 */
ss_status ss_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      int delta_softplus, const float* h0, const void* dout,
                      const float* dh_last, void* du, void* ddelta, void* dz, float* dA,
                      float* dB, float* dC, float* dD, float* ddelta_bias, float* dh0,
                      int64_t batch, int64_t seqlen, int64_t d_inner, int64_t d_state,
                      ss_dtype dtype, void* workspace, size_t workspace_bytes, uint32_t flags,
                      void* stream);

/* Workspace bytes ss_scan_bwd needs for this shape (0 for an empty problem or d_state > 64).
 * With flags SS_FLAG_STATES_GIVEN the states part of the workspace is read, not written: it
 * must hold the states ss_scan_fwd_states wrote for the same u, delta, A, B, delta_bias,
 * delta_softplus, h0, sizes and dtype (C, D and z do not enter the states). */
size_t ss_scan_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t d_inner,
                                   int64_t d_state, ss_dtype dtype);

/*
 * Multi-head scan with a scalar transition per head (the Mamba-2 form: IBM explainer, the
 * Mamba-2 block split into heads like multi-head attention, with B and C shared by groups of
 * heads as in grouped-query attention; Cartesia Mamba-3 post, the diagonal transition reduced to
 * a scalar times the identity).  For batch b, head h in group g = h / (nheads / ngroups), state n
 * and head channel p:
 *
 *     dt_t      = softplus(dt[b,t,h] + dt_bias[h])          (or the raw sum, softplus off)
 *     S_t[n,p]  = exp(dt_t * A[h]) * S_{t-1}[n,p] + dt_t * B[b,t,g,n] * x[b,t,h,p]
 *     y_t[p]    = sum_n C[b,t,g,n] * S_t[n,p] + D[h] * x[b,t,h,p]
 *     out       = y_t[p] * silu(z[b,t,h,p])                (when z is given)
 *
 *   x, z, out : (batch, seqlen, nheads, headdim), io dtype; z == NULL: no gate.
 *   dt        : (batch, seqlen, nheads), io dtype.
 *   B, C      : (batch, seqlen, ngroups, d_state), io dtype.
 *   A         : (nheads) float32, one transition per head.  D, dt_bias: (nheads) float32, NULL 0.
 *   h0, h_last: (batch, nheads, d_state, headdim) float32; NULL: zeros / not written.
 * nheads must be a multiple of ngroups (SS_ERR_INVALID_ARG); d_state outside 1..256 ->
 * SS_ERR_UNSUPPORTED.  Empty sizes are a no-op (h_last <- h0 or zeros).  out and h_last must not
 * overlap the inputs or each other.
 */
ss_status ss_scan2_fwd(const void* x, const void* dt, const float* A, const void* B,
                       const void* C, const float* D, const void* z, const float* dt_bias,
                       int dt_softplus, const float* h0, float* h_last, void* out,
                       int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                       int64_t ngroups, int64_t d_state, ss_dtype dtype, void* stream);

/*
 * Decode with the block's front end fused in (the one-token form of ss_scan_fwd_conv): takes
 * the block's x for this token and forms u = silu(conv_bias + sum_j conv_weight[d,j] *
 * window[j]) over the window [conv_state (the conv_k - 1 previous inputs, oldest first), x];
 * conv_state is then shifted in place (oldest dropped, x appended).
 *   conv_state   : (batch, conv_k - 1, d_inner) io dtype, read and overwritten IN PLACE
 *                  (required when conv_k > 1).
 *   x            : (batch, d_inner) io dtype.
 *   conv_weight, conv_bias, conv_k : as for ss_scan_fwd_conv.
 *   the rest     : as for ss_state_update_ex.
 * Needs d_state a multiple of 4 in 12..64 with 16-byte aligned state and A
 * (SS_ERR_UNSUPPORTED otherwise).  conv_state must not overlap state, out or the inputs.
 */
ss_status ss_state_update_conv(float* state, void* conv_state, const void* x,
                               const float* conv_weight, const float* conv_bias, int32_t conv_k,
                               const void* delta, const float* A, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias,
                               int delta_softplus, void* out, int64_t batch, int64_t d_inner,
                               int64_t d_state, ss_dtype dtype, uint32_t flags, void* stream);

/* Static description of a status code. */
const char* ss_status_string(ss_status s);

/* Thread-local detail of the last non-OK status returned on this thread ("" if none). */
const char* ss_last_error(void);

/* Library ABI version (major * 100 + minor). */
int ss_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SS_SCAN_H */
