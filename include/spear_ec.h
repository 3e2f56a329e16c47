/*
 * spear_ec.h -- C ABI of libspear_ec, the error-compensated 4-bit linear layer
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (SPEAR summary, "SPEAR: A System for Post-Quantization
 * Error-Adaptive Recovery Enabling Efficient Low-Bit LLM Serving", section
 * 2.1 A, input-adaptive error compensators) multiplies each token x by the
 * effective weight
 *
 *     W~ + alpha * B * diag(gamma(A x)) * A
 *
 * where W~ is the dequantized int4 weight, A (rank x d_in) projects x to a
 * low rank, gamma is a per-token gate on that projection and B (d_out x rank)
 * projects back.  The gate is fixed to the elementwise form
 * gamma(u) = sigmoid(g (.) u + b) with learned vectors g and b (the pages
 * describe a lightweight gate without giving a formula).  Computed in the
 * factored form
 *
 *     y[t,n] = sum_k W~[n,k] x[t,k] + alpha * sum_j B[n,j] v[t,j],
 *     u[t,j] = sum_k A[j,k] x[t,k],   v[t,j] = sigmoid(g[j] u[t,j] + b[j]) u[t,j].
 *
 * Data formats (all row-major, contiguous, 16-byte aligned device memory):
 *   x       bf16   [tokens][d_in]
 *   wq      uint32 [d_out][d_in/8]   code of column k in bits 4*(k%8) of word k/8
 *   scales  fp16   [d_out][d_in/group_size]
 *   zeros   uint32 [d_out][ceil(G/8)] zero-point of group j in bits 4*(j%8) of
 *           word j/8; NULL means symmetric codes with implicit zero-point 8
 *   A       bf16   [rank][d_in]
 *   B       bf16   [d_out][rank]
 *   g, b    fp32   [rank]
 *   y       bf16   [tokens][d_out], written once per call (round to nearest even)
 * Dequantization: W~[n,k] = (c[n,k] - z[n,k/g]) * s[n,k/g], exact in fp32.
 *
 * Conventions shared by every entry point:
 *   - All pointers are caller-owned device pointers; the library keeps none
 *     of them after the call returns and allocates nothing.
 *   - Calls are asynchronous on `stream` (NULL = the default stream); there is
 *     no host synchronisation inside a call.
 *   - Every argument is validated before any HIP call; on a validation error
 *     nothing is launched and the status code says why.  No C++ exception
 *     crosses this interface.  spear_ec_last_error() gives a thread-local text
 *     for the last failure.
 *   - `y` must not alias any input.
 */
#ifndef SPEAR_EC_H
#define SPEAR_EC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEAR_EC_VERSION 1

/* Status codes. */
#define SPEAR_EC_OK 0
#define SPEAR_EC_ERR_INVALID_ARGUMENT 1 /* NULL required pointer, negative size, bad desc */
#define SPEAR_EC_ERR_UNSUPPORTED 2      /* shape or format outside the supported set      */
#define SPEAR_EC_ERR_MISALIGNED 3       /* a pointer is not 16-byte aligned                */
#define SPEAR_EC_ERR_WORKSPACE 4        /* workspace NULL or smaller than required         */
#define SPEAR_EC_ERR_HIP 5              /* HIP launch / runtime error (see last_error)     */

/* desc.flags */
#define SPEAR_EC_ZEROS 1      /* asymmetric codes: `zeros` is present and required */
#define SPEAR_EC_PER_TENSOR 2 /* one symmetric scale for the whole tensor (stored per row) */
#define SPEAR_EC_OUT_F32 4    /* diagnostic: y is fp32 [tokens][d_out], the fp32 accumulation
                                 stored as it is instead of rounded to bf16 (same kernels;
                                 layer calls only, ignored by the quantizer and dequantizer) */

/* Error bits of a workspace (spear_ec_workspace_status). */
#define SPEAR_EC_WS_WAIT_TIMEOUT 1 /* a decode workgroup gave up waiting for the gated
                                      projection; the rows it finished hold NaN */

/* Largest token count the decode path accepts (decode = 1..32 tokens). */
#define SPEAR_EC_DECODE_MAX_TOKENS 32

/*
 * Shapes and weight format of one layer.  Supported set:
 *   d_in       multiple of 128, 128 .. 131072
 *   d_out      multiple of 16, 16 .. 131072
 *   rank       0 (plain W4, no compensator) or a multiple of 16 up to 128
 *   group_size d_in (per-output-channel scales) or 128
 *   flags      0, SPEAR_EC_ZEROS, or SPEAR_EC_PER_TENSOR (with group_size ==
 *              d_in and no zeros: the symmetric per-tensor format of the
 *              Quasar verify pass, summary "Targeted quantization"; it is
 *              stored as per-channel scales that are all equal, so the layer
 *              calls treat it as per-channel and only the quantizer differs),
 *              each optionally with SPEAR_EC_OUT_F32
 * Passed by pointer and read during the call only.
 */
typedef struct spear_ec_desc {
  int32_t d_in;
  int32_t d_out;
  int32_t rank;
  int32_t group_size;
  int32_t flags;
} spear_ec_desc;

/*
 * Bytes of scratch device memory one call with up to `max_tokens` tokens
 * needs (either path, and spear_ec_linear_serq).  The workspace holds the
 * rank-r projections, per-block
 * sums of x, split-K partial sums and a few arrival counters.  Its first use
 * requires it to be zero-filled by the caller (hipMemset once after
 * allocation); every call leaves the counters at zero again.  One workspace
 * per stream: calls that overlap on one workspace race.  Returns 0 for an
 * invalid desc or max_tokens < 0.
 */
size_t spear_ec_workspace_bytes(const spear_ec_desc* desc, int32_t max_tokens);

/*
 * Read and clear the error word of a workspace.  The decode kernel never
 * blocks without bound: where it gives up (a wait for the rank-r projection
 * that does not end) it writes NaN into the affected outputs and sets a bit
 * here, and the layer call itself has already returned SPEAR_EC_OK.  This call synchronizes `stream`, stores the
 * bits seen since the last call (SPEAR_EC_WS_*; 0 = none) in *error_bits and
 * clears them.  workspace is a device pointer of at least 16 bytes that the
 * layer calls use; error_bits a host pointer.  Returns SPEAR_EC_OK,
 * SPEAR_EC_ERR_INVALID_ARGUMENT (NULL pointer), SPEAR_EC_ERR_WORKSPACE
 * (workspace_bytes < 16) or SPEAR_EC_ERR_HIP.
 */
int spear_ec_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream,
                              int32_t* error_bits);

/*
 * Phase-aware dispatch (SPEAR summary, section 2.2 A, phase-aware adaptive
 * kernel fusion dispatch: memory-bound decode fuses the compensator into the
 * low-bit GEMM epilogue; compute-bound prefill takes the GEMM path).
 * tokens <= SPEAR_EC_DECODE_MAX_TOKENS runs spear_ec_linear_decode, larger
 * batches run spear_ec_linear_prefill.  tokens == 0 returns SPEAR_EC_OK and
 * launches nothing.  With rank == 0, A, B, g and b may be NULL and alpha is
 * ignored.
 */
int spear_ec_linear(const spear_ec_desc* desc, int32_t tokens, const void* x,
                    const uint32_t* wq, const void* scales, const uint32_t* zeros,
                    const void* A, const void* B, const float* g, const float* b,
                    float alpha, void* y, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * spear_ec_linear without a workspace argument, for callers that cannot
 * allocate memory (code under stream capture into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc): the call runs on the library's own
 * scratch, a file-scope device array of 64 MiB on each device the library
 * runs on (held until the process ends; its address is looked up and its
 * counters cleared on the device's first call).  It allocates nothing and
 * calls no allocating routine.  All calls on one device share that scratch:
 * calls that overlap on a device (several streams or threads at once) race.
 * The decode kernel's error word lives in that scratch and is not reported
 * (an output that a failed wait could not finish still holds NaN).  Same
 * arguments, dispatch and status codes as spear_ec_linear otherwise; a call
 * that needs more than 64 MiB of scratch (spear_ec_workspace_bytes of its
 * shape and token count) returns SPEAR_EC_ERR_WORKSPACE, before any HIP call.
 */
int spear_ec_linear_static(const spear_ec_desc* desc, int32_t tokens, const void* x,
                           const uint32_t* wq, const void* scales, const uint32_t* zeros,
                           const void* A, const void* B, const float* g, const float* b,
                           float alpha, void* y, hipStream_t stream);

/*
 * Decode path, 1..32 tokens (memory-bound: streams the packed weights once;
 * the rank-r projection is computed once per token and the gated B term is
 * added in registers before the single store of y).  tokens > 32 returns
 * SPEAR_EC_ERR_UNSUPPORTED.  Same arguments as spear_ec_linear.
 */
int spear_ec_linear_decode(const spear_ec_desc* desc, int32_t tokens, const void* x,
                           const uint32_t* wq, const void* scales, const uint32_t* zeros,
                           const void* A, const void* B, const float* g, const float* b,
                           float alpha, void* y, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Prefill path, any token count >= 1 (compute-bound: matrix-core GEMM on
 * exact integer codes with the scales applied in fp32; the gated B term is a
 * small matrix-core product added to the same accumulators before the
 * store).  Same arguments as spear_ec_linear.
 */
int spear_ec_linear_prefill(const spear_ec_desc* desc, int32_t tokens, const void* x,
                            const uint32_t* wq, const void* scales, const uint32_t* zeros,
                            const void* A, const void* B, const float* g, const float* b,
                            float alpha, void* y, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * The same layer with the gate as the bottleneck MLP the SPEAR summary
 * (section 2.1 A) names: gamma(u) = sigmoid(W2 relu(W1 u + b1) + b2), so
 * V = gamma(U) (.) U with U = X A^T, and Y = X W~^T + alpha V B^T.  hidden
 * (1 .. 128) is the bottleneck width h; w1 fp32 [h][rank], b1 fp32 [h],
 * w2 fp32 [rank][h], b2 fp32 [rank] (device pointers, 16-byte aligned,
 * caller-owned; required when rank > 0, ignored with rank 0).  Every other
 * argument, the dispatch (T <= 32 decode kernel, else prefill), the workspace
 * and the status codes are those of spear_ec_linear; an unsupported hidden is
 * SPEAR_EC_ERR_UNSUPPORTED.  relu is the reading of the bottleneck's
 * activation (the pages give no formula).
 */
int spear_ec_linear_mlp_gate(const spear_ec_desc* desc, int32_t tokens, const void* x,
                             const uint32_t* wq, const void* scales, const uint32_t* zeros,
                             const void* A, const void* B, int32_t hidden, const float* w1,
                             const float* b1, const float* w2, const float* b2, float alpha,
                             void* y, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * SERQ single-matrix reconstruction ("SERQ: Saliency-Aware Low-Rank Error
 * Reconstruction for LLM Quantization", section 2 on the single matrix and the
 * offline permutation): the salient input channels, contiguous after the
 * offline permutation, are x[:, s0 .. s0 + k) with s0 = salient_begin and
 * k = desc.rank; one matrix R reconstructs their quantization error,
 *     y[t, n] = sum_k W~[n, k] x[t, k] + sum_{j<k} R[n, j] x[t, s0 + j],
 * with no projection, no gate and no intermediate quantization.  R is bf16
 * [d_out][k] (row n holds output n's k weights, B's layout); x, wq, scales,
 * zeros, y, workspace and the token-count dispatch are as for
 * spear_ec_linear.  Requires k > 0 (a multiple of 16 up to 128), salient_begin
 * a multiple of 8 and salient_begin + k <= d_in, else
 * SPEAR_EC_ERR_INVALID_ARGUMENT / SPEAR_EC_ERR_UNSUPPORTED.
 */
int spear_ec_linear_serq(const spear_ec_desc* desc, int32_t tokens, const void* x,
                         const uint32_t* wq, const void* scales, const uint32_t* zeros,
                         int32_t salient_begin, const void* R, void* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * Round-to-nearest int4 quantization of fp32 weights w [d_out][d_in] into the
 * packed format above (offline preparation; SPEAR summary, section 3.1: RTN
 * with per-channel scales is the hardest setting the compensators target).
 * Without SPEAR_EC_ZEROS: symmetric, s = RN_fp16(max|W|/7), codes
 * clamp(rint(W/s), -8, 7) + 8.  With SPEAR_EC_ZEROS: asymmetric over the range
 * widened to include 0, s = RN_fp16((hi - lo)/15), z = clamp(rint(-lo/s), 0, 15),
 * codes clamp(rint(W/s) + z, 0, 15).  Ratios are formed in double, rint rounds
 * half to even, a scale that rounds to 0 becomes 1, and fp16 rounding of a
 * scale saturates at 65504.  `zeros` is written only with SPEAR_EC_ZEROS.
 * With SPEAR_EC_PER_TENSOR one scale s = RN_fp16(max|W| / 7) over the whole
 * tensor (written to every row's scale), codes as in the symmetric case.
 * desc.rank is ignored.
 */
int spear_ec_quantize_rtn(const spear_ec_desc* desc, const float* w, uint32_t* wq,
                          void* scales, uint32_t* zeros, hipStream_t stream);

/*
 * Dequantize the packed weights to fp32 w_out [d_out][d_in]:
 * (c - z) * s, exact.  Used to check the unpack path bit for bit.
 */
int spear_ec_dequant_f32(const spear_ec_desc* desc, const uint32_t* wq, const void* scales,
                         const uint32_t* zeros, float* w_out, hipStream_t stream);

/*
 * EC-aware chunk selection (SPEAR summary, section 2.2 C: a latency-aware
 * scheduler reads a precomputed table of kernel latencies and picks the
 * largest prefill chunk that still meets the inter-token latency target, for
 * the current compensator placement and decode load).  Host only.
 *
 * A step makes, per layer, one dispatcher call on the decode tokens and one
 * on the prefill chunk.  Layers of one kind (shape and rank, e.g. with and
 * without a compensator) share a table: us[i] is the latency of one call with
 * tokens[i] tokens (ascending, >= 1), and `count` is how many calls of that
 * kind one step makes per token group (its number of layers).  Between table
 * points the latency is interpolated linearly over the table's running
 * maximum; below the first point it is the first point's value, above the
 * last it grows in proportion to the tokens; zero tokens cost nothing.
 */
typedef struct spear_ec_lut_kind {
  int32_t n;              /* table points */
  const int32_t* tokens;  /* [n], strictly ascending, >= 1 */
  const float* us;        /* [n], finite, >= 0 */
  int32_t count;          /* calls of this kind per token group in one step */
} spear_ec_lut_kind;

/* Latency (us) of a step with `decode_tokens` and a prefill chunk of
 * `chunk_tokens`: overhead_us + sum_kinds count * (t(decode) + t(chunk)).
 * Returns -1 for an invalid table or a negative token count. */
float spear_ec_step_latency_us(const spear_ec_lut_kind* kinds, int32_t n_kinds,
                               int32_t decode_tokens, int32_t chunk_tokens, float overhead_us);

/* The largest multiple of `granule` up to `max_chunk` whose step latency, as
 * spear_ec_step_latency_us returns it (fp32), is at most itl_us; 0 when even
 * the decode tokens alone miss it (no prefill this step).  Returns -1 for an invalid table, decode_tokens < 0, max_chunk < 0,
 * granule < 1 or a non-finite itl_us. */
int32_t spear_ec_pick_chunk(const spear_ec_lut_kind* kinds, int32_t n_kinds, int32_t decode_tokens,
                            float itl_us, float overhead_us, int32_t max_chunk, int32_t granule);

/*
 * Measure one kind's table on the device: for each of the n token counts,
 * one untimed call of spear_ec_linear, then `reps` calls timed between two
 * HIP events on `stream`, averaged into us_out[i].  x and y must hold
 * max(tokens) rows; the other arguments are spear_ec_linear's.  Synchronizes
 * the stream; creates and destroys two events.
 */
int spear_ec_lut_measure(const spear_ec_desc* desc, const int32_t* tokens, int32_t n, int32_t reps,
                         const void* x, const uint32_t* wq, const void* scales,
                         const uint32_t* zeros, const void* A, const void* B, const float* g,
                         const float* b, float alpha, void* y, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, float* us_out);

/* Static text for a status code. */
const char* spear_ec_status_string(int status);

/* Thread-local text describing the last failure on this thread ("" if none). */
const char* spear_ec_last_error(void);

/* SPEAR_EC_VERSION of the built library. */
int spear_ec_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPEAR_EC_H */
