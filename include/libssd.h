/*
 * libssd -- the Mamba-2 SSD (structured state space duality) scan on AMD
 * Instinct MI355X (gfx950), behind a plain C ABI.
 *
 * The operation.  For every batch b and head h (group g = h / (H / G)), with a
 * state S of P x N numbers per (b, h), starting from init_state (zero when
 * absent):
 *
 *   alpha_t = exp(dt[b,t,h] * A[h])
 *   S      <- alpha_t * S + dt[b,t,h] * x[b,t,h,:] (outer) Bm[b,t,g,:]
 *   y[b,t,h,p] = sum_n S[p,n] * Cm[b,t,g,n] + D[h] * x[b,t,h,p]
 *
 * and final_state is S after the last token.  This is the selective SSM
 * recurrence h_t = A_t h_{t-1} + B_t x_t, y_t = C_t^T h_t with a scalar decay
 * A_t = a_t I (the "Mamba-2" note, sections "writing the SSM as a matrix" and
 * "reducing A to a number"), the decay discretised as exp(dt A) ("Mamba"
 * reading notes, section 2.2) and the input term as dt B, with multi-head
 * inputs sharing B and C within a group ("Mamba-2" note, section "Mamba-2
 * block", item 2) and a D skip connection.
 *
 * ssd_chunk_scan_fwd evaluates it in blocks of chunk_size tokens, the
 * two-way split of the "Mamba-2" note (section "taking each path half way")
 * and of the "Mamba-2 model walkthrough" (sections 6.1-6.2): a quadratic,
 * attention-like product inside each block, (Cm Bm^T masked by the segment-sum
 * decay) times dt x, plus states passed from block to block.  The result does
 * not depend on chunk_size except through rounding.  ssd_step applies the
 * recurrence to one token.
 *
 * Conventions shared by every call:
 *
 *  - Memory.  Every tensor argument is a DEVICE pointer to dense, row-major
 *    memory in the shape stated, owned by the caller.  The library allocates
 *    nothing at run time and keeps no state between calls (the one exception,
 *    ssd_chunk_scan_fwd_noalloc, keeps its scratch in a static device array).
 *    Every pointer must be 16-byte aligned, else SSD_ERR_INVALID_ARG.
 *  - Device.  `stream` belongs to the current device (0 = its null stream);
 *    per-device set-up is done for the current device.
 *  - Types.  dt, A, D and all states are float32.  x, Bm, Cm and y are
 *    float32 (SSD_DTYPE_F32) or bfloat16 (SSD_DTYPE_BF16).  Arithmetic
 *    accumulates in float32; products inside a block may use bfloat16 operands
 *    in SSD_DTYPE_BF16 mode.
 *  - Execution.  Calls validate their arguments on the host, enqueue kernels
 *    on `stream` (0 = the null stream) and return without waiting.  Argument
 *    errors are returned before anything is enqueued.  A launch error is
 *    returned as SSD_ERR_HIP.  No exception crosses the ABI.
 *  - Values.  Inputs are not inspected.  The method assumes A <= 0 and dt >= 0
 *    (the decay lies in [0, 1]); other values are computed as written and may
 *    overflow.
 *  - Support.  P in {16, 32, 64, 128}; N in {16, 32, 64, 128, 256};
 *    chunk_size in {64, 128, 256}; H % G == 0; B, L >= 0 (L need not be a
 *    multiple of chunk_size); B * H <= 65535 for the chunk scan.  Other shapes
 *    return SSD_ERR_UNSUPPORTED.
 */
#ifndef LIBSSD_H
#define LIBSSD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, negative size, H % G != 0 */
    SSD_ERR_UNSUPPORTED = 2,   /* shape, chunk size, dtype or algorithm not supported */
    SSD_ERR_WORKSPACE = 3,     /* workspace missing or smaller than the query says */
    SSD_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
    SSD_ERR_TOO_LARGE = 5      /* more scratch than ssd_chunk_scan_fwd_noalloc holds */
} ssd_status;

typedef enum {
    SSD_DTYPE_F32 = 0,
    SSD_DTYPE_BF16 = 1
} ssd_dtype;

/* Which kernel sequence evaluates the chunk scan.  All give the same result
 * up to rounding.  SSD_ALGO_AUTO picks by shape and dtype: SSD_ALGO_PIPE
 * wherever it covers the shape (bfloat16, P in {64, 128}, N in {64, 128,
 * 256}), else SSD_ALGO_STAGED where it does (bfloat16, P == 64), else
 * SSD_ALGO_REFERENCE. */
typedef enum {
    SSD_ALGO_AUTO = 0,
    SSD_ALGO_REFERENCE = 1,   /* float32 vector arithmetic, three kernels, every supported shape */
    SSD_ALGO_STAGED = 2,      /* bf16 matrix cores: block states, state pass, block outputs */
    SSD_ALGO_PIPE = 3         /* bf16 matrix cores, one workgroup walks each (batch, head) sequence */
} ssd_algo;

/* Human-readable name of a status code (static storage). */
const char *ssd_status_string(ssd_status status);

/* Library version string (static storage). */
const char *ssd_version(void);

/*
 * Bytes of device workspace ssd_chunk_scan_fwd needs for this shape: that of
 * the algorithm SSD_ALGO_AUTO runs (ssd_chunk_scan_workspace_size_algo with
 * SSD_ALGO_AUTO).  Returns 0 when the shape is not supported.
 */
size_t ssd_chunk_scan_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                     int64_t N, int64_t chunk_size, ssd_dtype dtype);

/*
 * Bytes of device workspace ssd_chunk_scan_fwd_algo needs with `algo`, 0 when
 * `algo` does not cover the shape or dtype.  The workspace is scratch that
 * every call writes before it reads: SSD_ALGO_PIPE keeps the Cm.Bm^T tiles of
 * every 64-token sub-block (B*G*ceil(L/64)*64*64 bfloat16) and the states of
 * the time segments it cuts sequences into (at most 256 of P*N + 1 floats);
 * SSD_ALGO_STAGED and SSD_ALGO_REFERENCE keep the state and decay of every
 * block (B*ceil(L/chunk_size)*H*(P*N + 1) floats), SSD_ALGO_STAGED also the
 * Cm.Bm^T tiles.  It needs no initialisation.  Calls that share a workspace
 * must be ordered (one stream, or synchronised): two calls in flight on one
 * workspace race.
 */
size_t ssd_chunk_scan_workspace_size_algo(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                          int64_t N, int64_t chunk_size, ssd_dtype dtype,
                                          ssd_algo algo);

/*
 * Chunked SSD scan, forward.
 *
 *   x            [B, L, H, P]   dtype        inputs
 *   dt           [B, L, H]      float32      step sizes (>= 0)
 *   A            [H]            float32      per-head decay rate (<= 0)
 *   Bm           [B, L, G, N]   dtype        input projections ("B")
 *   Cm           [B, L, G, N]   dtype        output projections ("C")
 *   D            [H]            float32      skip weights
 *   init_state   [B, H, P, N]   float32      state before token 0, or NULL for zeros
 *   y            [B, L, H, P]   dtype        output (written); must not alias an input
 *   final_state  [B, H, P, N]   float32      state after token L-1, or NULL to skip;
 *                                            may alias init_state
 *   workspace    device memory of at least ssd_chunk_scan_workspace_size(...) bytes
 *                (contents need no initialisation and are not kept)
 *
 * Errors: SSD_ERR_INVALID_ARG for a null required pointer, a misaligned
 * pointer or a negative size; SSD_ERR_UNSUPPORTED outside the support matrix;
 * SSD_ERR_WORKSPACE when the workspace is NULL or too small; SSD_ERR_HIP when a
 * launch fails.  L == 0 or B == 0 copies init_state (or zeros) to final_state.
 */
ssd_status ssd_chunk_scan_fwd(const void *x, const float *dt, const float *A,
                              const void *Bm, const void *Cm, const float *D,
                              const float *init_state, void *y, float *final_state,
                              void *workspace, size_t workspace_bytes,
                              int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                              int64_t chunk_size, ssd_dtype dtype, hipStream_t stream);

/*
 * As ssd_chunk_scan_fwd, with the kernel sequence chosen by the caller and a
 * workspace of ssd_chunk_scan_workspace_size_algo(..., algo) bytes.  An
 * algorithm that does not cover the shape or dtype returns
 * SSD_ERR_UNSUPPORTED: SSD_ALGO_STAGED and SSD_ALGO_PIPE need SSD_DTYPE_BF16
 * and N in {64, 128, 256}; SSD_ALGO_STAGED takes P == 64, SSD_ALGO_PIPE P in
 * {64, 128} (a head of 128 channels is scanned as two heads of 64 sharing
 * dt, A and D).  SSD_ALGO_PIPE walks every (batch, head) sequence in 64-token
 * sub-blocks whatever chunk_size is (the result is the same up to rounding)
 * and spreads sequences over the device's compute units in time segments
 * when there are fewer of them than compute units, or fewer than twice as many.
 */
ssd_status ssd_chunk_scan_fwd_algo(const void *x, const float *dt, const float *A,
                                   const void *Bm, const void *Cm, const float *D,
                                   const float *init_state, void *y, float *final_state,
                                   void *workspace, size_t workspace_bytes,
                                   int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                   int64_t N, int64_t chunk_size, ssd_dtype dtype,
                                   ssd_algo algo, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * forward scan of ssd_chunk_scan_fwd (SSD_ALGO_AUTO) with no workspace
 * argument.  Its scratch is a static device array of
 * SSD_NOALLOC_SCRATCH_BYTES per device, created with the library's code
 * object on that device and held until the process ends; the call allocates
 * nothing (no hipMalloc, no library allocation).  A shape whose workspace
 * (ssd_chunk_scan_workspace_size) exceeds that size returns SSD_ERR_TOO_LARGE
 * before anything is enqueued.  Every call on one device shares that
 * device's array, which keeps the last call's contents (nothing in it needs
 * to start at zero): calls that overlap on one device (two streams, or two
 * host threads) race and give wrong results; order them.  Arguments, layouts
 * and other errors as ssd_chunk_scan_fwd; the caller passes y and
 * final_state.  The first call on a device looks up the array's address.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

ssd_status ssd_chunk_scan_fwd_noalloc(const void *x, const float *dt, const float *A,
                                      const void *Bm, const void *Cm, const float *D,
                                      const float *init_state, void *y, float *final_state,
                                      int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                      int64_t N, int64_t chunk_size, ssd_dtype dtype,
                                      hipStream_t stream);

/*
 * Packed rows of independent sequences ("Mamba" reading notes, section 3.5:
 * boundary resetting, so that sequences concatenated into one row do not leak
 * into one another).  seq_idx: device int32 [B, L]; token t of row b starts a
 * new sequence when t > 0 and seq_idx[b][t] != seq_idx[b][t-1].  Each
 * sequence is scanned as if it stood alone: the first sequence of a row
 * starts from init_state (or zero), every later one from zero; y is written
 * for every token and final_state (nullable) is the state after the row's
 * last token, that of its last sequence.  Other arguments and layouts as
 * ssd_chunk_scan_fwd; dt must be non-negative (its magnitude is used).
 * Covered: bfloat16, P = 64 or 128, N = 64 or 128 (else SSD_ERR_UNSUPPORTED).
 * The workspace (size from ssd_chunk_scan_varlen_workspace_size: that of
 * SSD_ALGO_PIPE plus B*L*H floats) is owned by the caller;
 * asynchronous on `stream`; no allocation.
 */
size_t ssd_chunk_scan_varlen_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                            int64_t N, int64_t chunk_size, ssd_dtype dtype);

ssd_status ssd_chunk_scan_fwd_varlen(const void *x, const float *dt, const float *A,
                                     const void *Bm, const void *Cm, const float *D,
                                     const float *init_state, const int32_t *seq_idx, void *y,
                                     float *final_state, void *workspace, size_t workspace_bytes,
                                     int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                     int64_t N, int64_t chunk_size, ssd_dtype dtype,
                                     hipStream_t stream);

/*
 * The step before the scan in a Mamba-2 block ("Mamba-2" note, section
 * "Mamba-2 block": one parallel projection yields z, X, B, C and dt).
 * zxbcdt: bfloat16 [B, L, 2HP + 2GN + H], each token's row laid out
 * [z (HP) | x (HP) | Bm (GN) | Cm (GN) | dt_raw (H)].  The C = HP + 2GN
 * middle channels go through a causal depthwise convolution of width W
 * (conv_w fp32 [C, W], tap W-1 on the current token, zero input before
 * token 0; conv_b fp32 [C] or NULL) and SiLU, and are written to x
 * [B, L, H, P], Bm and Cm [B, L, G, N] (bfloat16); dt fp32 [B, L, H] =
 * softplus(dt_raw + dt_bias) (dt_bias fp32 [H] or NULL).  z stays in place
 * for ssd_gated_norm.  Covered: bfloat16, 1 <= W <= 4, HP, GN and the row
 * length multiples of 8 (else SSD_ERR_UNSUPPORTED).  Device pointers,
 * caller-owned, 16-byte aligned for the bfloat16 arrays; asynchronous.
 */
ssd_status ssd_block_prologue(const void *zxbcdt, const float *conv_w, const float *conv_b,
                              const float *dt_bias, void *x, void *Bm, void *Cm, float *dt,
                              int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                              int64_t W, ssd_dtype dtype, hipStream_t stream);

/*
 * The step after the scan: the gate and the normalisation ("Mamba-2" note,
 * section "Mamba-2 block"; a GroupNorm per the "Mamba-2" walkthrough,
 * section 7.2).  For each of T tokens: v = y * SiLU(z) over its D channels;
 * each of `ngroups` equal groups of channels is normalised (center = 1: minus
 * its mean, over the root of its variance + eps; center = 0: over the root of
 * its mean square + eps); out = that * weight (+ bias).  y, out bfloat16
 * [T, D]; z bfloat16 with row stride z_stride elements (D for a [T, D] tensor,
 * or the projection row length to read z straight out of zxbcdt); weight,
 * bias fp32 [D] (bias may be NULL).  Covered: bfloat16, D a multiple of 8 up
 * to 8192, 1 <= ngroups <= 8 with D / ngroups a multiple of 8, z_stride a
 * multiple of 8 (else SSD_ERR_UNSUPPORTED); weight and bias 16-byte aligned.
 * Deterministic; asynchronous.
 */
ssd_status ssd_gated_norm(const void *y, const void *z, int64_t z_stride, const float *weight,
                          const float *bias, void *out, int64_t T, int64_t D, int64_t ngroups,
                          float eps, int center, ssd_dtype dtype, hipStream_t stream);

/*
 * Mamba-1 selective scan with diagonal A ("Mamba" reading notes, section 2.2:
 * h_t = Abar h_{t-1} + Bbar x_t, y_t = C h_t, zero-order hold
 * Abar = exp(dt A), Bbar = (dt A)^-1 (exp(dt A) - I) dt B; section 3.2: dt,
 * B, C depend on the token).  Per channel d and state n:
 *   h[d][n] = exp(dt[d] A[d][n]) h[d][n] + bbar x[d],
 *   y[d] = sum_n Cm[n] h[d][n] + D[d] x[d],
 * with bbar = (exp(dt A) - 1) / A[d][n] * Bm[n] (zoh = 1; dt Bm[n] where A is
 * 0) or bbar = dt[d] Bm[n] (zoh = 0).  Layouts: x, dt, y bfloat16
 * [B, L, Dch] (dt the step, already positive); A fp32 [Dch, N]; Bm, Cm
 * bfloat16 [B, L, G, N], channel d reading group d / (Dch / G); D fp32 [Dch]
 * or NULL; init_state and final_state fp32 [B, Dch, N] or NULL.  Covered:
 * bfloat16, N = 8, 16 or 32, Dch / G a multiple of 64 (else
 * SSD_ERR_UNSUPPORTED).  Device pointers, caller-owned, 16-byte aligned for
 * the bfloat16 arrays; no workspace; asynchronous on `stream`.
 */
ssd_status ssd_selective_scan(const void *x, const void *dt, const float *A, const void *Bm,
                              const void *Cm, const float *D, const float *init_state, void *y,
                              float *final_state, int64_t B, int64_t L, int64_t Dch, int64_t G,
                              int64_t N, int zoh, ssd_dtype dtype, hipStream_t stream);

/*
 * Bytes of device workspace ssd_chunk_scan_bwd needs for this shape: the
 * state entering every 64-token sub-block and the gradient of the state
 * leaving it (two bfloat16 arrays of B*H*ceil(L/64)*P*N), plus float32
 * parts of dA and dD per (batch row, head, sub-block).
 * Returns 0 when the backward does not cover the shape or dtype.  No
 * zero-filling is needed; calls sharing a workspace must be ordered on one
 * stream.
 */
size_t ssd_chunk_scan_bwd_workspace_size(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G,
                                         int64_t N, int64_t chunk_size, ssd_dtype dtype);

/*
 * Chunked SSD scan, backward: the gradients of the scalar
 *     <dy, y> + <dfinal, final_state>
 * with respect to every input of ssd_chunk_scan_fwd, i.e. the adjoint of the
 * recurrence of the "Mamba-2" note (section "writing the SSM as a matrix")
 * evaluated block by block as in the block decomposition of the "Mamba-2
 * model walkthrough" (section 6.1).  The forward states are recomputed, not
 * taken from a forward call.
 *
 *   x, dt, A, Bm, Cm, D, init_state   as for ssd_chunk_scan_fwd (init_state nullable)
 *   dy       [B, L, H, P]   dtype    gradient of y
 *   dfinal   [B, H, P, N]   float32  gradient of the final state, or NULL for zeros
 *   dx       [B, L, H, P]   dtype    written
 *   ddt      [B, L, H]      float32  written
 *   dA       [H]            float32  written (summed over batch rows and tokens)
 *   dBm      [B, L, G, N]   dtype    written (summed over the heads of each group)
 *   dCm      [B, L, G, N]   dtype    written (summed over the heads of each group)
 *   dD       [H]            float32  written
 *   dinit    [B, H, P, N]   float32  gradient of init_state, or NULL to skip
 *   workspace  device memory of at least ssd_chunk_scan_bwd_workspace_size(...) bytes
 *
 * Supported: dtype SSD_DTYPE_BF16, P == 64 or 128, N == 64 or 128, chunk_size
 * as for the forward (the result does not depend on it beyond rounding);
 * anything else returns SSD_ERR_UNSUPPORTED.  Products run on the matrix cores with
 * bfloat16 operands and float32 accumulation.  Outputs must not alias inputs.
 * Errors as for ssd_chunk_scan_fwd.  L == 0 or B == 0 writes dA = dD = 0 and
 * dinit = dfinal (or zeros).
 */
ssd_status ssd_chunk_scan_bwd(const void *x, const float *dt, const float *A, const void *Bm,
                              const void *Cm, const float *D, const float *init_state, const void *dy,
                              const float *dfinal, void *dx, float *ddt, float *dA, void *dBm, void *dCm,
                              float *dD, float *dinit, void *workspace, size_t workspace_bytes, int64_t B,
                              int64_t L, int64_t H, int64_t P, int64_t G, int64_t N, int64_t chunk_size,
                              ssd_dtype dtype, hipStream_t stream);

/*
 * One recurrent decode step: the update above for a single token, in place.
 *
 *   state  [B, H, P, N]  float32  read and overwritten with the updated state
 *   x      [B, H, P]     dtype
 *   dt     [B, H]        float32
 *   A      [H]           float32
 *   Bm     [B, G, N]     dtype
 *   Cm     [B, G, N]     dtype
 *   D      [H]           float32
 *   y      [B, H, P]     dtype    y = Cm . (updated state) + D x
 *
 * This is the recurrent path of the "Mamba-2" note (four-token section): it
 * carries only the fixed-size state from token to token.  Errors as for
 * ssd_chunk_scan_fwd; B == 0 is a no-op.
 */
ssd_status ssd_step(float *state, const void *x, const float *dt, const float *A,
                    const void *Bm, const void *Cm, const float *D, void *y,
                    int64_t B, int64_t H, int64_t P, int64_t G, int64_t N,
                    ssd_dtype dtype, hipStream_t stream);

/*
 * A plain device-to-device copy of `bytes` bytes: the bandwidth reference of
 * the benchmark (what a kernel with no arithmetic streams on this device).
 * src and dst are device pointers, 16-byte aligned, not overlapping; bytes a
 * multiple of 16 (else SSD_ERR_INVALID_ARG).  Streamed in 4 KB pieces per
 * workgroup with non-temporal loads and stores; asynchronous on `stream`.
 */
ssd_status ssd_stream_copy(void *dst, const void *src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_H */
