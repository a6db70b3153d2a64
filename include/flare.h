/*
 * libflare: FLARE / FLARE++ low-rank attention routing, forward pass, on one
 * AMD Instinct MI355X (gfx950).
 *
 * Operator (per batch item b and head h; heads are independent and each owns
 * its own latent slice, FLARE arXiv abstract):
 *   logits   l[m][n] = s * <Q[h][m], K[b][h][n]>,  s = 1/sqrt(D)
 *   encode   Z[m]    = sum_n softmax_n(l[m][.])[n] * V[b][h][n]
 *            (latents attend to tokens: FLARE skill page, "2. Implement
 *             Encode Stage")
 *   decode   Y[n]    = sum_m softmax_m(l[.][n])[m] * Z[m]
 *            (tokens attend back through the transposed logits; the
 *             encode-decode factorization of the FLARE arXiv abstract)
 *   FLARE++  Q' = Q + encode(Q, K, V), then encode and decode with Q'
 *            (FLARE++ arXiv abstract: the encoder's output corrects the
 *             learned queries)
 *
 * Conventions shared by every entry point
 *   Layout    Q is [H][M][D] (one latent set per head, shared over the batch).
 *             K, V and Y are [B][H][N][D] (the *_ex variants also take them
 *             token-major, [B][N][H][D]). Z is [B][H][M][D]. All row-major,
 *             contiguous, D innermost.
 *   Memory    All tensor pointers are device pointers on the current HIP
 *             device, 16-byte aligned. The caller owns every tensor; the
 *             library neither frees nor retains them.
 *   Types     dtype selects the element type of Q, K, V, Z and Y alike.
 *             FLARE_F32 computes in fp32 throughout. FLARE_BF16 feeds bf16
 *             MFMA and keeps every accumulator, softmax statistic and Z in
 *             fp32; probabilities, Z and Q' are rounded to nearest-even bf16
 *             where they become MFMA operands, and outputs are rounded to
 *             nearest-even bf16.
 *   Sizes     B, H, N, M, D >= 1, B*H <= 65535, N <= 2^30. Supported:
 *             FLARE_F32 with D in {8, 16, 24, 32, 48, 64, 96, 128} and
 *             M <= 4096; FLARE_BF16 with D in {32, 64, 128} and M <= 512.
 *             Other sizes return FLARE_ERR_UNSUPPORTED.
 *   Async     Work is enqueued on `stream` (0 = the legacy default stream)
 *             and the call returns; inputs must stay unchanged until the
 *             stream passes the call. Device faults surface at the caller's
 *             next synchronisation.
 *   Errors    A call returns FLARE_OK or an error status and never aborts.
 *             Arguments are validated before any launch, so an error status
 *             other than FLARE_ERR_HIP means nothing was enqueued.
 *             flare_last_error() describes the last failure of the calling
 *             thread.
 *   Workspace The plain entry points allocate stream-ordered scratch memory
 *             (hipMallocAsync/hipFreeAsync on `stream`). The *_ws variants
 *             take caller-owned scratch memory of at least
 *             flare_workspace_size() bytes instead; concurrent calls must not
 *             share one workspace.
 */
#ifndef LIBFLARE_FLARE_H
#define LIBFLARE_FLARE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerated argument types below are fixed 32-bit integers with named
 * values (not C enums), so that a caller passing a value outside the named
 * ones gets FLARE_ERR_INVALID_ARG rather than undefined behaviour. */
typedef int32_t flare_dtype;
enum { FLARE_F32 = 0, FLARE_BF16 = 1 };

typedef int32_t flare_status;
enum {
    FLARE_OK = 0,
    FLARE_ERR_INVALID_ARG = 1, /* null pointer, size < 1, misaligned or aliased tensors, small workspace */
    FLARE_ERR_UNSUPPORTED = 2, /* (dtype, D, M) outside the supported set */
    FLARE_ERR_NO_MEMORY = 3,   /* scratch allocation failed */
    FLARE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
};

typedef int32_t flare_op;
enum {
    FLARE_OP_ENCODE = 0,
    FLARE_OP_DECODE = 1,
    FLARE_OP_FORWARD = 2,
    FLARE_OP_PP_FORWARD = 3,
    FLARE_OP_BACKWARD = 4,   /* flare_backward (workspace sizing only) */
    FLARE_OP_PP_BACKWARD = 5, /* flare_pp_backward (workspace sizing only) */
    FLARE_OP_PP_QUERIES = 6   /* flare_pp_queries */
};

/* Encode: Y := Z[B][H][M][D] = softmax_n(s Q K^T) V for every (b, h).
 * FLARE skill page, "2. Implement Encode Stage"; encode half of step 4.
 * Inputs Q [H][M][D], K and V [B][H][N][D]; output Y is the Z tensor. */
flare_status flare_encode(const void* Q, const void* K, const void* V, void* Y,
                          int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                          flare_dtype dtype, hipStream_t stream);

/* Decode: Y[B][H][N][D] = softmax_m(s K Q^T) Z for every (b, h), with the
 * latents Z passed in the V argument as [B][H][M][D]. The decode half of the
 * FLARE encode-decode factorization (FLARE arXiv abstract). K is [B][H][N][D]. */
flare_status flare_decode(const void* Q, const void* K, const void* V, void* Y,
                          int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                          flare_dtype dtype, hipStream_t stream);

/* FLARE forward: Y = decode(Q, K, encode(Q, K, V)). Z stays fp32 between the
 * two stages and is rounded once when it becomes an MFMA operand, so the
 * result equals flare_decode(flare_encode(.)) for the same shapes.
 * FLARE skill page, step 4; FLARE arXiv abstract ("two SDPA calls"). */
flare_status flare_forward(const void* Q, const void* K, const void* V, void* Y,
                           int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                           flare_dtype dtype, hipStream_t stream);

/* FLARE++ forward: Q'[b][h] = Q[h] + encode(Q, K, V)[b][h] (rounded to dtype),
 * then Y = decode(Q', K, encode(Q', K, V)). FLARE++ skill page, "Core
 * Mechanism"; FLARE++ arXiv abstract. */
flare_status flare_pp_forward(const void* Q, const void* K, const void* V, void* Y,
                              int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                              flare_dtype dtype, hipStream_t stream);

/* FLARE++ corrected queries alone: Qp[b][h] = Q[h] + encode(Q, K, V)[b][h],
 * rounded to nearest-even in dtype, as [B][H][M][D]. These are the dynamic,
 * input-conditioned latent queries of the FLARE++ skill page ("Core
 * Mechanism", "Mathematical Formulation"), with the residual of the FLARE++
 * arXiv abstract (the encoder's output corrects the learned queries). The
 * values are bit for bit the Q' that flare_pp_forward computes for the same
 * inputs and then uses in its second encode and its decode (same kernels,
 * same split of the tokens), so flare_pp_forward at B = 1 equals
 * flare_forward with Q = Qp[0]. Inputs Q [H][M][D], K and V [B][H][N][D];
 * output Qp [B][H][M][D] (may not overlap an input). The _ws variant takes
 * flare_workspace_size(FLARE_OP_PP_QUERIES, ...) bytes of scratch memory. */
flare_status flare_pp_queries(const void* Q, const void* K, const void* V, void* Qp,
                              int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                              flare_dtype dtype, hipStream_t stream);
flare_status flare_pp_queries_ws(const void* Q, const void* K, const void* V, void* Qp,
                                 int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                 flare_dtype dtype, hipStream_t stream, void* workspace, size_t ws_bytes);

/* FLARE forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and result as flare_forward (bit for bit), but the
 * workspace is a static device array of FLARE_STATIC_SCRATCH_BYTES inside the
 * library, one per GPU, held from the library's load until the process ends;
 * nothing is allocated. Sizes whose forward workspace
 * (flare_workspace_size(FLARE_OP_FORWARD, ...)) exceeds it return
 * FLARE_ERR_UNSUPPORTED before anything is enqueued. Every call on one GPU
 * uses that GPU's one array: calls that overlap in time on a GPU (other
 * streams, other threads) race and must be serialised by the caller; calls
 * in order on one stream are safe. */
#define FLARE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
flare_status flare_forward_noalloc(const void* Q, const void* K, const void* V, void* Y,
                                   int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                   flare_dtype dtype, hipStream_t stream);

/* Scratch bytes the *_ws variant of `op` needs for these sizes (0 when the
 * sizes or type are invalid or unsupported). */
size_t flare_workspace_size(flare_op op, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                            flare_dtype dtype);

/* Variants taking caller-owned scratch memory (device pointer, 256-byte
 * aligned, at least flare_workspace_size(op, ...) bytes). Same results as the
 * plain entry points; nothing is allocated. */
flare_status flare_encode_ws(const void* Q, const void* K, const void* V, void* Y,
                             int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                             flare_dtype dtype, hipStream_t stream, void* workspace, size_t ws_bytes);
flare_status flare_decode_ws(const void* Q, const void* K, const void* V, void* Y,
                             int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                             flare_dtype dtype, hipStream_t stream, void* workspace, size_t ws_bytes);
flare_status flare_forward_ws(const void* Q, const void* K, const void* V, void* Y,
                              int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                              flare_dtype dtype, hipStream_t stream, void* workspace, size_t ws_bytes);
flare_status flare_pp_forward_ws(const void* Q, const void* K, const void* V, void* Y,
                                 int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                 flare_dtype dtype, hipStream_t stream, void* workspace, size_t ws_bytes);

/* Layout of the token tensors K, V and Y. Q stays [H][M][D], and Z (the
 * output of flare_encode, the V argument of flare_decode) stays [B][H][M][D].
 *   FLARE_LAYOUT_BHND  [B][H][N][D], as everywhere else in this header.
 *   FLARE_LAYOUT_BNHD  [B][N][H][D]: token-major, i.e. a projection's
 *                      (B, N, H*D) output read in place, without the head
 *                      transpose the FLARE skill page applies after its
 *                      projections and undoes before its output projection
 *                      ("4. Combine Encode-Decode into Attention Layer"). */
typedef int32_t flare_layout;
enum { FLARE_LAYOUT_BHND = 0, FLARE_LAYOUT_BNHD = 1 };

/* The four operations with a layout argument. workspace == NULL with
 * ws_bytes == 0 allocates scratch memory as the plain entry points do;
 * otherwise it is caller-owned as for the *_ws variants. Results are those
 * of the plain entry points on the same values (the layout changes only
 * where elements live). A layout other than the two above returns
 * FLARE_ERR_INVALID_ARG. */
flare_status flare_encode_ex(const void* Q, const void* K, const void* V, void* Y,
                             int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                             flare_dtype dtype, flare_layout layout, hipStream_t stream,
                             void* workspace, size_t ws_bytes);
flare_status flare_decode_ex(const void* Q, const void* K, const void* V, void* Y,
                             int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                             flare_dtype dtype, flare_layout layout, hipStream_t stream,
                             void* workspace, size_t ws_bytes);
flare_status flare_forward_ex(const void* Q, const void* K, const void* V, void* Y,
                              int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                              flare_dtype dtype, flare_layout layout, hipStream_t stream,
                              void* workspace, size_t ws_bytes);
flare_status flare_pp_forward_ex(const void* Q, const void* K, const void* V, void* Y,
                                 int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                 flare_dtype dtype, flare_layout layout, hipStream_t stream,
                                 void* workspace, size_t ws_bytes);

/* Token-query decode of the FLARE skill page ("3. Implement Decode Stage";
 * the decode half of "4. Combine Encode-Decode into Attention Layer"): each
 * token's own query attends to the latent states, which serve as keys and
 * values,
 *   Y[b][h][n] = sum_m softmax_m(s * <q[b][h][n], Z[b][h][m]>) * Z[b][h][m].
 * q and Y are [B][H][N][D] or, with FLARE_LAYOUT_BNHD, [B][N][H][D]; Z is
 * [B][H][M][D] (e.g. the output of flare_encode). Same types, sizes and
 * conventions as flare_decode; no workspace is needed. The page's layer is
 * then flare_encode(latents, k, v) followed by flare_attend(q, Z). */
flare_status flare_attend(const void* q, const void* Z, void* Y,
                          int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                          flare_dtype dtype, flare_layout layout, hipStream_t stream);

/* Backward of flare_forward: the gradients of Q, K and V for an upstream
 * gradient dY of Y. The FLARE pages train their models end to end (FLARE
 * skill page, "5. Scale to Million-Point Sequences": gradient checkpointing
 * for long inputs); this is the chain rule through the encode and decode
 * softmaxes of the operator above (with l = s Q K^T, A = softmax_n(l),
 * Bt = softmax_m(l)^T, Z = A V, Y = Bt Z):
 *   dZ = Bt^T dY,  dV = A^T dZ,
 *   dl[m][n] = A[m][n] (<dZ[m],V[n]> - <dZ[m],Z[m]>)
 *            + Bt[n][m] (<dY[n],Z[m]> - <dY[n],Y[n]>),
 *   dQ = s dl K (summed over the batch, Q being shared),  dK = s dl^T Q.
 * Inputs Q [H][M][D], K, V, dY [B][H][N][D]; outputs dQ [H][M][D], dK, dV
 * [B][H][N][D], in the operator dtype. Precision follows the forward's:
 * FLARE_F32 computes in fp32 throughout; FLARE_BF16 heads at D = 32, at
 * D = 64 (above 256 latents over latent ranges of at most 256) and at
 * D = 128 (above 128 latents over ranges of at most 128) run on bf16 MFMA
 * with fp32 accumulation, the probabilities, dl and the staged
 * Q, Z and dZ being rounded to nearest-even bf16 where they become MFMA
 * operands (where the dZ partials are formed with the token statistics,
 * D = 32 with M <= 128 or D = 64 with M <= 64, also dY scaled by the
 * token's inverse decode sum).
 * It recomputes the forward's encode internally; nothing N x M is stored.
 * Supported for D in {8, 16, 24, 32, 48, 64, 96, 128} (bf16: 32, 64 and
 * 128) with the forward's M range; otherwise FLARE_ERR_UNSUPPORTED. Outputs
 * may not overlap inputs or each other. The _ws variant takes
 * flare_workspace_size(FLARE_OP_BACKWARD, ...) bytes of caller-owned
 * scratch memory. */
flare_status flare_backward(const void* Q, const void* K, const void* V, const void* dY,
                            void* dQ, void* dK, void* dV,
                            int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                            flare_dtype dtype, hipStream_t stream);
flare_status flare_backward_ws(const void* Q, const void* K, const void* V, const void* dY,
                               void* dQ, void* dK, void* dV,
                               int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                               flare_dtype dtype, hipStream_t stream, void* workspace, size_t ws_bytes);

/* flare_backward with a token layout: K, V, dY, dK and dV are [B][H][N][D]
 * (FLARE_LAYOUT_BHND) or token-major [B][N][H][D] (FLARE_LAYOUT_BNHD); Q
 * and dQ stay [H][M][D]. Same kernels with token rows addressed through the
 * layout's stride, so the gradients equal flare_backward's on the same
 * values bit for bit. workspace == NULL with ws_bytes == 0: the library
 * allocates (stream-ordered); otherwise flare_workspace_size(
 * FLARE_OP_BACKWARD, ...) bytes, as for flare_backward_ws. */
flare_status flare_backward_ex(const void* Q, const void* K, const void* V, const void* dY,
                               void* dQ, void* dK, void* dV,
                               int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                               flare_dtype dtype, flare_layout layout, hipStream_t stream,
                               void* workspace, size_t ws_bytes);

/* Backward of flare_pp_forward (FLARE++ skill page, "Core Mechanism"; FLARE++
 * abstract: Q' = Q + encode(Q, K, V), then the FLARE forward with Q'). The
 * chain rule through the two stages: the FLARE backward at Q' (one batch
 * entry at a time, Q' being per entry) gives dQ' and the second stage's dK,
 * dV; the encode's backward for dZ = dQ' (dV += A^T dQ', dl = A (dQ' V^T -
 * <dQ', Z>), dQ += s dl K, dK += s dl^T Q, with A, Z of the first encode)
 * gives the first stage's; dQ = sum over the batch of dQ' plus the first
 * stage's. Same arguments, layouts, dtypes, support range and error
 * behaviour as flare_backward; the stages' gradients are summed in fp32 and
 * rounded once (dQ' and the second stage's dK, dV are rounded to the
 * operator dtype first). The _ws variant takes flare_workspace_size(
 * FLARE_OP_PP_BACKWARD, ...) bytes. */
flare_status flare_pp_backward(const void* Q, const void* K, const void* V, const void* dY,
                               void* dQ, void* dK, void* dV,
                               int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                               flare_dtype dtype, hipStream_t stream);
flare_status flare_pp_backward_ws(const void* Q, const void* K, const void* V, const void* dY,
                                  void* dQ, void* dK, void* dV,
                                  int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                  flare_dtype dtype, hipStream_t stream,
                                  void* workspace, size_t workspace_bytes);
/* flare_pp_backward with a token layout, as flare_backward_ex (workspace:
 * flare_workspace_size(FLARE_OP_PP_BACKWARD, ...) bytes, or NULL and 0). */
flare_status flare_pp_backward_ex(const void* Q, const void* K, const void* V, const void* dY,
                                  void* dQ, void* dK, void* dV,
                                  int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                  flare_dtype dtype, flare_layout layout, hipStream_t stream,
                                  void* workspace, size_t ws_bytes);

/* Static text for a status code. */
const char* flare_status_string(flare_status s);

/* Detail of the calling thread's last non-OK status ("" if none). The
 * pointer stays valid until the thread's next libflare call. */
const char* flare_last_error(void);

/* --------------------------------------------------------------- tuning
 * Process-wide overrides of the launch plan, for tests and measurement
 * sweeps. They change how the work is split across workgroups, never what is
 * computed: results differ at most by rounding. A value of 0 restores the
 * library's own choice; negative values and unknown keys return
 * FLARE_ERR_INVALID_ARG. Overrides apply to calls that start after the set. */
typedef int32_t flare_tune;
enum {
    FLARE_TUNE_CHUNKS = 0,      /* encode: token chunks per (b, h) (capped at N) */
    FLARE_TUNE_ENC_MBW = 1,     /* bf16 encode shape: latent blocks of 32 per wave, */
    FLARE_TUNE_ENC_WM = 2,      /*   waves over latent blocks (0: one wave owns them all), */
    FLARE_TUNE_ENC_WT = 3,      /*   waves over tokens. Used together when MBW > 0 and they
                                 *   cover M; a shape that is not built fails the launch
                                 *   with FLARE_ERR_HIP. */
    FLARE_TUNE_DEC_TB = 4,      /* bf16 decode: 32-token blocks per wave and step (1; 2 at
                                 *   D <= 64 and M <= 256) */
    FLARE_TUNE_DEC_GROUPS = 5,  /* decode: workgroups per (b, h) */
    FLARE_TUNE_FAIL_ALLOC = 6,  /* 1: the allocating entry points fail with
                                 *   FLARE_ERR_NO_MEMORY (error-path tests) */
    FLARE_TUNE_DEC_HEADS = 7,   /* bf16 decode, token-major layout: heads per workgroup
                                 *   (1, 2 or 4, a divisor of H, where built) */
    FLARE_TUNE_KEYS = 8
};

flare_status flare_set_tuning(flare_tune key, int64_t value);

/* ---------------------------------------------------------- measurement
 * Kernel timing with HIP events recorded on the launch stream around every
 * kernel the library enqueues. Kernel kinds: 0 = encode partial (split-N
 * online softmax), 1 = combine, 2 = decode, 3 = backward kernels. */
#define FLARE_KERNEL_KINDS 4

/* Turn event recording on (1) or off (0) for the calling process, and drop
 * every recorded event. While it is on, each kernel is launched with
 * hipExtLaunchKernel and an event pair bound to its dispatch, so the elapsed
 * time of a pair is the kernel's own execution time (as a kernel trace
 * reports it), without the launch gaps. */
flare_status flare_timing_enable(int on);

/* Wait for the recorded events, add the elapsed milliseconds of each kernel
 * kind into ms[kind] and the number of launches into count[kind] (arrays of
 * FLARE_KERNEL_KINDS entries), then drop them. */
flare_status flare_timing_read(double* ms, int64_t* count);

/* Plain device-to-device copy of `bytes` bytes (multiple of 16, 16-byte
 * aligned pointers) on `stream`: a kernel of known traffic, used to scale
 * hardware memory counters to bytes. */
flare_status flare_copy_kernel(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Peak probes for measurement: fixed instruction streams of known size,
 * launched over the whole chip (four waves per SIMD on 256 compute units)
 * on `stream`, for the caller to time with events; their rate is what the
 * GPU sustains at its clock of the moment.
 *   FLARE_PROBE_MFMA_BF16: each wave issues iters x 4 independent
 *     v_mfma_f32_32x32x16_bf16 (32768 flops each);
 *   FLARE_PROBE_EXP: each lane evaluates iters x 16 independent v_exp_f32.
 * `out` (device memory, at least flare_probe_lanes() floats) receives one
 * value per lane so that nothing is elided. *work (host) receives the work
 * launched: flops, or exponentials. 1 <= iters <= 2^20, else
 * FLARE_ERR_INVALID_ARG; an unknown kind is FLARE_ERR_INVALID_ARG. */
typedef int32_t flare_probe;
enum { FLARE_PROBE_MFMA_BF16 = 0, FLARE_PROBE_EXP = 1 };
size_t flare_probe_lanes(void);
flare_status flare_probe_peak(flare_probe kind, int64_t iters, float* out, size_t out_floats, double* work,
                              hipStream_t stream);

/* Streaming read of `bytes` bytes (multiple of 16, 16-byte aligned) by a
 * grid of flare_probe_lanes() lanes, each folding what it reads into one
 * float of `out` (at least flare_probe_lanes() floats): a read-only kernel
 * of known traffic, to calibrate streaming-read bandwidth. */
flare_status flare_read_kernel(const void* src, size_t bytes, float* out, size_t out_floats, hipStream_t stream);

/* Launch plan the library would use (for logs): writes a short text into
 * buf (up to len bytes incl. the terminator). */
flare_status flare_describe_plan(flare_op op, int64_t B, int64_t H, int64_t N, int64_t M, int64_t D,
                                 flare_dtype dtype, char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* LIBFLARE_FLARE_H */
