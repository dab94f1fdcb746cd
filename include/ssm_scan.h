/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) fused selective scan: the
 * forward and its backward (ssm_selective_scan_bwd, further below).
 *
 * The operation (Mamba's selective state-space scan).  For every
 * batch row b, channel d and state n, with A = -exp(A_log[d,n]):
 *
 *     delta_t = softplus(delta_raw[b,t,d])            (optional; then optional clip)
 *     Abar_t  = exp(delta_t * A)                      in (0, 1)
 *     h_t     = Abar_t * h_{t-1} + delta_t * B[b,t,n] * x[b,t,d],   h_{-1} = 0
 *     y[b,t,d] = sum_n C[b,t,n] * h_t[n] + D[d] * x[b,t,d]
 *     h_last[b,d,n] = h after the last valid step of row b
 *
 * Sources: the recurrence and readout are those of the pwwt.cn article
 * (section 1.1, "the recursion"); the parameterisation A = -exp(A_log),
 * softplus(delta) > 0 and Abar = exp(delta*A) is its section 2.4; the clip of
 * delta after softplus is its section 3.3; padding folded in as the identity
 * pair (a, b) = (1, 0) is its section 2.3; the state after the last step is
 * what the chunked scan of the bjdmk.com.cn article (section 4.2) carries out.
 * The input term is delta*B*x (not the exact zero-order-hold B), and B and C
 * are shared by all channels of a batch row.
 *
 * Layouts (all row-major, contiguous, no strides):
 *   x, delta, y : [batch, seqlen, dim]       io dtype (fp32 or bf16), dim fastest
 *   B, C        : [batch, seqlen, dstate]    io dtype, dstate fastest
 *   A_log       : [dim, dstate]              fp32
 *   D           : [dim]                      fp32, may be NULL (no skip term)
 *   valid_len   : [batch]                    int32, may be NULL (every row has seqlen steps)
 *   h_last      : [batch, dim, dstate]       fp32, may be NULL (not written)
 * Every pointer is a device pointer on the handle's device.  The caller owns
 * all memory; the library allocates nothing per call.
 *
 * Padding: steps t >= valid_len[b] are the identity (the state is carried
 * unchanged), y there is written as +0.0, and the values of x, delta, B and C
 * there never reach any output (NaN or Inf included).  valid_len outside
 * [0, seqlen] is clamped into it.  Padding is on the right only.
 *
 * Arithmetic is fp32 throughout (bf16 inputs convert exactly); y is rounded to
 * the io dtype with round-to-nearest-even.  Results are bitwise reproducible
 * run to run for the same inputs and dims.
 *
 * Streams and graphs: a call only enqueues kernels on the caller's stream (no
 * copies, memsets, allocations or synchronisation), so it may be captured
 * into a HIP graph; a replay computes what the call would compute with the
 * buffers' contents at replay time.
 *
 * Errors: every entry point returns SSM_OK (0) or a negative SSM_ERR_* code and
 * never throws.  Argument checks happen on the host before anything is
 * enqueued; a failed check enqueues nothing.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ssm_scan_handle_s* ssm_scan_t;

enum ssm_io_dtype { SSM_IO_F32 = 0, SSM_IO_BF16 = 1 };

enum ssm_status {
  SSM_OK = 0,
  SSM_ERR_INVALID_ARG = -1,     /* NULL required pointer or handle, negative dim, bad flag or clip bounds */
  SSM_ERR_UNSUPPORTED = -2,     /* dstate not 16/32/64, dim not a multiple of 16, misaligned pointer, wrong GPU,
                                   one batch row of x, delta, B or C spanning 2 GiB or more, or a grid too
                                   large */
  SSM_ERR_ALIAS = -3,           /* y or h_last overlaps an input, or y overlaps h_last */
  SSM_ERR_HIP = -4,             /* a HIP runtime or launch error */
  SSM_ERR_NO_DEVICE = -5,       /* no usable GPU at the requested ordinal */
  SSM_ERR_DEVICE_MISMATCH = -6, /* the calling thread's current device is not the handle's device */
  SSM_ERR_SCRATCH = -7          /* ssm_selective_scan_fwd_noalloc: the time split asked for needs more than
                                   SSM_SCAN_NOALLOC_SCRATCH_BYTES */
};

/* Size of the static device scratch behind ssm_selective_scan_fwd_noalloc
 * (16 MiB per GPU the library runs on, held until the process ends). */
#define SSM_SCAN_NOALLOC_SCRATCH_BYTES (16u << 20)

typedef struct ssm_scan_dims {
  int64_t batch;          /* number of rows b */
  int64_t seqlen;         /* L (the padded length when valid_len is given); 0 is a valid no-op */
  int64_t dim;            /* D channels: multiple of 16 */
  int64_t dstate;         /* N states per channel: 16, 32 or 64 */
  int32_t io_dtype;       /* enum ssm_io_dtype for x, delta, B, C and y */
  int32_t delta_softplus; /* 1: delta = softplus(delta_raw); 0: delta is used as given */
  int32_t delta_clamp;    /* 1: delta = min(max(delta, delta_min), delta_max) after softplus */
  float delta_min;        /* used when delta_clamp = 1; must satisfy 0 <= delta_min <= delta_max */
  float delta_max;
} ssm_scan_dims;

/* Create a handle bound to GPU `device_ordinal` (HIP numbering).  Loads nothing
 * lazily later: after this returns SSM_OK the handle is immutable, so one
 * handle may serve concurrent calls on different streams.  *out is set to NULL
 * on failure.  Errors: SSM_ERR_INVALID_ARG (out NULL), SSM_ERR_NO_DEVICE,
 * SSM_ERR_UNSUPPORTED (not a gfx950 device), SSM_ERR_HIP. */
int ssm_scan_create(ssm_scan_t* out, int device_ordinal);

/* Enqueue the forward on `stream` (a hipStream_t; NULL = the default stream)
 * and return without waiting.  The calling thread's current device must be the
 * handle's device.  Inputs must stay valid and unmodified, and outputs
 * untouched, until the stream reaches the end of this work.  Pointer
 * alignment: natural for the element type.  batch == 0, dim == 0 or
 * seqlen == 0 are valid (for seqlen == 0, h_last is written with zeros). */
int ssm_selective_scan_fwd(ssm_scan_t handle, const void* x, const void* delta, const float* A_log, const void* B,
                           const void* C, const float* D, const int32_t* valid_len, void* y, float* h_last,
                           const ssm_scan_dims* dims, void* stream);

/* Optional inputs and outputs of the forward (any field may be NULL/0).
 *
 *  h0           [batch, dim, dstate] fp32: the state before step 0 instead of
 *               zeros (continuing a sequence processed in pieces: the split
 *               run equals the whole run, pwwt.cn section 4.2 and
 *               bjdmk.com.cn section 2.4 carry the state between chunks).
 *               h0 may be the same buffer as h_last (in-place update; the
 *               scan then runs unsplit, whatever time_parts asks); any other
 *               overlap with an output is rejected.
 *  delta_bias   [dim] fp32: added to delta before softplus and the clip (the
 *               dt bias of the fused kernel body in the nxbn.cn article,
 *               section 3).
 *  z            [batch, seqlen, dim], io dtype: output gate, y <- y * silu(z)
 *               with silu(v) = v / (1 + e^-v), applied to the whole readout
 *               C.h + D*x at valid steps (the same article and section).
 *  chunk_states [batch, ceil(seqlen / chunk_len), dim, dstate] fp32: the state
 *               after the last step of every chunk of chunk_len steps (the last
 *               chunk may be shorter; past valid_len the state no longer
 *               changes) -- the boundary states kept for recomputation in the
 *               pwwt.cn article, section 3.4.
 *  chunk_len    when chunk_states is set: a multiple of 4 that divides
 *               ssm_scan_chunk_len(dstate) (that value itself, the kernel's
 *               time tile, is the coarsest choice), else SSM_ERR_INVALID_ARG.
 *
 *  time_parts, workspace, workspace_bytes: cut the time axis into parts that
 *               run on different workgroups (the multi-block chunked scan of
 *               the pwwt.cn article, sections 3.1 and 4.2: each block folds its
 *               chunk, the chunk carries are combined in order, each chunk is
 *               then rescanned from its incoming state), for batches too small
 *               to fill the GPU with (row, channel) work alone.  Two kernels
 *               run on the stream: the fold of the first P-1 parts, then every
 *               part.  time_parts = 0 lets the library choose
 *               (ssm_scan_auto_time_parts) and falls back to no split when the
 *               workspace is NULL or smaller than ssm_scan_workspace_bytes for
 *               that choice; 1 never splits; P >= 2 asks for at most P parts
 *               of whole chunks and needs at least
 *               ssm_scan_workspace_bytes(dims, P) bytes of device workspace
 *               (else SSM_ERR_INVALID_ARG).  The workspace is caller-owned
 *               scratch (4-byte aligned, overlapping nothing else) that the
 *               call overwrites; it must not be shared by calls that may run
 *               at the same time.  With two parts the results are bitwise those
 *               of the unsplit scan; with more, the states entering parts 2 and
 *               later are composed from per-part sums and may differ from
 *               them by rounding.
 *  combine      how the sub-chunks of a time tile are joined (the second and
 *               third levels of the pwwt.cn article, section 3.1):
 *               SSM_COMBINE_WALK (0, the default and the faster on gfx950):
 *               one lane per (channel, state) carries the state serially
 *               through every sub-chunk's (a_prod, b_total) in LDS;
 *               SSM_COMBINE_WAVE_SCAN (1): a log-depth Hillis-Steele scan of
 *               the pairs across each wave's sub-chunks by cross-lane
 *               permutes (its section 2.2), then the serial carry through the
 *               wave totals only.  Equal in exact arithmetic (the combine is
 *               associative), within rounding otherwise.  Other values:
 *               SSM_ERR_INVALID_ARG.  The fold kernel of a time split always
 *               walks. */
enum ssm_combine { SSM_COMBINE_WALK = 0, SSM_COMBINE_WAVE_SCAN = 1 };

typedef struct ssm_scan_fwd_extras {
  const float* h0;
  const float* delta_bias;
  const void* z;
  float* chunk_states;
  int64_t chunk_len;
  int32_t time_parts;
  void* workspace;
  int64_t workspace_bytes;
  int32_t combine;
} ssm_scan_fwd_extras;

/* The kernel's time tile for this dstate -- the coarsest chunk_len of
 * chunk_states: 128, 64 or 32 for dstate 16, 32 or 64; 0 for an unsupported
 * dstate. */
int64_t ssm_scan_chunk_len(int64_t dstate);

/* The number of time parts the library picks for these dims on the handle's
 * GPU when time_parts = 0 (1 = no split): it splits only while the
 * (row, 16-channel) workgroups would leave CUs idle (at most three quarters
 * as many of them as CUs), into about four workgroups per resident slot and
 * parts of at least 512 steps.  Returns 1 for a NULL handle or dims, or
 * invalid sizes. */
int32_t ssm_scan_auto_time_parts(ssm_scan_t handle, const ssm_scan_dims* dims);

/* Bytes of workspace a split into (at most) time_parts parts needs for these
 * dims (0 when that split is no split); -1 for NULL dims, a negative size or
 * time_parts, or an unsupported dstate. */
int64_t ssm_scan_workspace_bytes(const ssm_scan_dims* dims, int32_t time_parts);

/* ssm_selective_scan_fwd with the optional extras above (extras may be NULL,
 * which is ssm_selective_scan_fwd).  Same ordering, asynchrony and errors;
 * additionally SSM_ERR_INVALID_ARG for a chunk_len that does not match, and
 * SSM_ERR_ALIAS for an extra output overlapping an input or another output. */
int ssm_selective_scan_fwd_ex(ssm_scan_t handle, const void* x, const void* delta, const float* A_log, const void* B,
                              const void* C, const float* D, const int32_t* valid_len, void* y, float* h_last,
                              const ssm_scan_dims* dims, const ssm_scan_fwd_extras* extras, void* stream);

/* ssm_selective_scan_fwd_ex for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, the same kernels and bitwise the same
 * results, but the time split's carries live in a static device array of
 * SSM_SCAN_NOALLOC_SCRATCH_BYTES that every GPU holds for the life of the
 * process, so the call allocates nothing (and, like every entry point,
 * enqueues no copy or memset).  extras may be NULL; its workspace must be
 * NULL and workspace_bytes 0 (else SSM_ERR_INVALID_ARG).  time_parts = 0
 * picks the split as ssm_selective_scan_fwd_ex would and runs unsplit if
 * its carries would not fit the scratch (the automatic split never needs
 * more than 12 MiB); an explicit time_parts >= 2 whose
 * ssm_scan_workspace_bytes exceeds SSM_SCAN_NOALLOC_SCRATCH_BYTES returns
 * SSM_ERR_SCRATCH.  Nothing in the scratch needs to start at zero: each call
 * writes every carry before reading it.  The scratch is shared by every call
 * on the same GPU (whatever the handle): calls that may overlap in time on
 * one GPU (different streams, or graphs replayed concurrently) race on it
 * and must be serialised by the caller.  Other errors as
 * ssm_selective_scan_fwd_ex. */
int ssm_selective_scan_fwd_noalloc(ssm_scan_t handle, const void* x, const void* delta, const float* A_log,
                                   const void* B, const void* C, const float* D, const int32_t* valid_len, void* y,
                                   float* h_last, const ssm_scan_dims* dims, const ssm_scan_fwd_extras* extras,
                                   void* stream);

/* ---- backward --------------------------------------------------------
 *
 * Gradients of the forward for the loss sum(dy * y) + sum(dh_last * h_last),
 * by reverse-mode differentiation of the recurrence: the adjoint of the state
 * runs backwards in time (the same affine scan on flipped time, pwwt.cn
 * sections 2.1 and 3.1), and the forward states are recomputed tile by tile
 * from the chunk-boundary states the forward saved (its section 3.4).  x,
 * delta, A_log, B, C, D, valid_len, dims and the extras (h0, delta_bias, z;
 * the other extras fields are ignored) must be those of the forward.
 *
 *  dy            [batch, seqlen, dim] io dtype: gradient of y (the gated y
 *                when z is given).
 *  dh_last       [batch, dim, dstate] fp32 or NULL (zero).
 *  chunk_states  the forward's chunk_states with chunk_len =
 *                ssm_scan_bwd_chunk_len(dstate) (only the first
 *                ceil(seqlen / chunk_len) - 1 are read; NULL allowed when
 *                seqlen <= chunk_len).
 *  dx, ddelta    [batch, seqlen, dim] io dtype: gradients of x and of the raw
 *                delta (before bias, softplus and clip); +0 at padded steps.
 *  dz            [batch, seqlen, dim] io dtype, required when z is given.
 *  dA_log        [dim, dstate] fp32.
 *  dB, dC        [batch, seqlen, dstate] fp32; zero at padded steps.
 *  dD, ddelta_bias [dim] fp32 or NULL.
 *  dh0           [batch, dim, dstate] fp32 or NULL: gradient of the initial
 *                state.
 *  workspace     at least ssm_scan_bwd_workspace_bytes(dims) bytes of device
 *                scratch (4-byte aligned), overwritten; it holds per channel
 *                group partial sums of dB and dC that a second kernel adds in
 *                a fixed order, so the result is deterministic.
 * No output may overlap an input or another output. */
typedef struct ssm_scan_bwd_io {
  const void* dy;
  const float* dh_last;
  const float* chunk_states;
  void* dx;
  void* ddelta;
  void* dz;
  float* dA_log;
  float* dB;
  float* dC;
  float* dD;
  float* ddelta_bias;
  float* dh0;
  void* workspace;
  int64_t workspace_bytes;
} ssm_scan_bwd_io;

/* The backward's time tile for this dstate (32, 16 or 8 for dstate 16, 32 or
 * 64; 0 if unsupported): the chunk_len the forward must save chunk_states at. */
int64_t ssm_scan_bwd_chunk_len(int64_t dstate);

/* Workspace bytes of ssm_selective_scan_bwd for these dims: 4 * (2 * (dim/16)
 * * batch * seqlen * dstate + 31 * batch * dim * dstate + 47 * batch * dim)
 * (dB/dC partials per channel group, and per-part partials for a time split
 * into up to 16 parts, which the library uses when the batch is too small to
 * fill the GPU); -1 for NULL or invalid dims. */
int64_t ssm_scan_bwd_workspace_bytes(const ssm_scan_dims* dims);

/* Enqueue the backward on `stream` (the main kernel and the reduction of the
 * partial sums; with a time split a fold kernel first; for seqlen == 0 only
 * small fill kernels).  Same conventions as the
 * forward: host-side checks first (SSM_ERR_INVALID_ARG also for a missing
 * required output, chunk_states or workspace, or a workspace that is too
 * small), nothing enqueued on failure, bitwise reproducible results. */
int ssm_selective_scan_bwd(ssm_scan_t handle, const void* x, const void* delta, const float* A_log, const void* B,
                           const void* C, const float* D, const int32_t* valid_len, const ssm_scan_dims* dims,
                           const ssm_scan_fwd_extras* extras, const ssm_scan_bwd_io* io, void* stream);

/* Release the handle.  NULL is accepted.  The caller must ensure no work
 * enqueued with the handle is still to be launched. */
int ssm_scan_destroy(ssm_scan_t handle);

/* A static, human-readable string for a status code (never NULL). */
const char* ssm_scan_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
