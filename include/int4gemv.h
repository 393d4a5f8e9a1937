/*
 * int4gemv.h -- C ABI of the int4 group-quantized matrix-vector library for
 * MI355X (gfx950).
 *
 * Sources (four gerbil diff pages; every entry point cites the passage that
 * defines its operation):
 *   [P1] gerbil 1.11.4 -> 1.13.0, page 9   (index type declarations: Executor docs)
 *   [P2] gerbil 1.12.0 -> 1.13.0, page 8   (gpu module: Gepard backbone graph, addLinearOp)
 *   [P3] gerbil 1.0.0-rc.9 -> 1.0.0, page 17 (gpu module: dequantizeMLXProjection)
 *   [P4] gerbil 1.12.0 -> 1.13.0, page 12  (kernel registry: WGSL_QUAD_MATVEC_INT4,
 *        WGSL_NORM_MATVEC_INT4 and their dispatch specs; Executor fusion passes)
 *
 * Quantized weight matrix with N output columns over K inputs, group size gs
 * ([P2] addLinearOp: the {w}.q / {w}.scales / {w}.zeros triplet; [P4]
 * fuseMambaFrontDecodeEntries doc: column-major, one column contiguous):
 *   q      uint32 [N][K/8]   eight 4-bit codes per word; the code of input k of
 *                            column n sits at bits 4*(k%8) of q[n*K/8 + k/8]
 *                            (low nibble first: [P1]/[P3] dequantizeMLXProjection)
 *   scales float  [N][K/gs]  scale of group g = k/gs of column n at [n*K/gs + g]
 *   zeros  float  [N][K/gs]  zero point, an integer value in [0, 15]
 *   w[n][k] = (code - zero) * scale            ([P4] WGSL_QUAD_MATVEC_INT4 dequant)
 * Every kernel forms code - zero exactly, so a term whose code equals its
 * zero point contributes exactly 0 (an output made only of such terms is 0),
 * and each dot-product output is within 1e-4 * sum_k |x_k * w[n][k]| + 1e-6
 * of the exact sum for any codes, any scales and any integer zero points.
 * Activations and outputs are fp32, row-major: X[m][k] at X[m*K + k],
 * Y[m][n] at Y[m*N + n].
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE pointers on the current HIP device, owned
 *     by the caller.  The library allocates nothing, keeps no pointer after
 *     the call returns and holds no state between calls (int4_mlp keeps its
 *     call counter in the caller's workspace).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; the call never synchronizes.  A kernel fault surfaces at
 *     the caller's next synchronization.
 *   - Shapes: K >= gs, K % gs == 0, gs % 32 == 0 (a 32-code, 16-byte load
 *     never straddles a group).  N >= 0; N == 0 writes nothing (see norm).
 *   - Alignment: q, X (and every other input vector, and W) must be 16-byte aligned;
 *     scales, zeros and outputs 4-byte aligned.
 *   - Outputs must not overlap any input or each other ([P4]
 *     fuseNormMatVecDecodeEntries / fuseMambaFrontDecodeEntries alias rules).
 *   - Arguments are validated before anything is enqueued; on any error
 *     nothing is written and no kernel is launched.  int4_last_error()
 *     returns a message for the last failed call on the calling thread.
 *   - Calls are reentrant; concurrent calls on different streams are allowed.
 */
#ifndef INT4GEMV_H
#define INT4GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum int4_status {
    INT4_OK = 0,
    INT4_ERR_NULL = 1,   /* a required pointer is NULL                          */
    INT4_ERR_SHAPE = 2,  /* K / gs / M / N outside the supported set            */
    INT4_ERR_ALIGN = 3,  /* a pointer is not aligned as required                */
    INT4_ERR_ALIAS = 4,  /* an output overlaps an input or another output       */
    INT4_ERR_ARG = 5,    /* split points out of order, eps negative or not finite */
    INT4_ERR_HIP = 6     /* the HIP runtime refused a query or a launch         */
} int4_status;

/* Static, human-readable name of a status code. */
const char* int4_status_str(int status);

/* Message describing the last failed call on the calling thread ("" if none). */
const char* int4_last_error(void);

/*
 * Asymmetric per-group min/max quantization and packing of W (fp32 [N][K],
 * row n = output column n).  The pages import the quantizer but do not show
 * its body ([P4] module imports of quantizeInt4; [P1] quantizeKaniBackbone
 * doc); the reading implemented, per group of gs inputs of one column, in
 * IEEE binary32 with round-to-nearest-even and no flushing of subnormals:
 *   scale = (max - min) / 15            (a constant group c != 0: |c| / 15)
 *   zero  = clamp(rint(-min / scale), 0, 15)
 *   code  = clamp(rint(w / scale) + zero, 0, 15)
 * A group whose scale is 0 (all zero, or the range underflows) stores
 * scale = 0, zero = +0 and codes 0.  Inputs must be finite.
 * Outputs: q [N][K/8], scales [N][K/gs], zeros [N][K/gs].
 */
int int4_quantize_pack(const float* W, int64_t N, int64_t K, int32_t group_size,
                       uint32_t* q, float* scales, float* zeros, void* stream);

/*
 * Y[m][n] = sum_k X[m][k] * w[n][k] for M decode lanes, 0 <= M <= 8
 * (M == 0 writes nothing).  The weights are read from memory once per call
 * for all lanes; lanes never interact ([P1] lockstep batch decode: linear
 * layers run the batched INT4 GEMM; [P4] MATVEC_INT4 K-parallel matvec for
 * the single-lane case).  Limits of the per-block local data share (160 KiB
 * on gfx950), else INT4_ERR_SHAPE: for M = 1, K * 4 bytes must fit it
 * (K <= 40960); for M >= 2 it holds the scales and zero points of 16
 * columns (2 * 16 * (K/gs + at most 25) words) beside about 54 KiB of
 * staging, which allows K/gs up to about 820.  At M >= 2 every lane's outputs are
 * bit-identical whatever the other lanes hold; they need not be bit-identical
 * to the M = 1 call (both are within the tolerance).
 */
int int4_matvec(const float* X, int32_t M, const uint32_t* q, const float* scales,
                const float* zeros, int64_t N, int64_t K, int32_t group_size,
                float* Y, void* stream);

/*
 * One matvec over N column-concatenated outputs, routed into up to four
 * buffers ([P4] WGSL_QUAD_MATVEC_INT4 routing, QUAD_MATVEC_INT4_SPEC params
 * [K, N, gs, n0, n1, n2], fuseMambaFrontDecodeEntries doc):
 *   column n -> out0[n] (n < n0), out1[n-n0] (n < n1), out2[n-n1] (n < n2),
 *               out3[n-n2] otherwise.
 * Requires 0 <= n0 <= n1 <= n2 <= N (else INT4_ERR_ARG).  out_j may be NULL
 * only when its range is empty.  Per-column arithmetic is the same as
 * int4_matvec's, so the routed values equal int4_matvec over the same
 * concatenated matrix bit for bit.
 */
int int4_matvec_split4(const float* x, const uint32_t* q, const float* scales,
                       const float* zeros, int64_t N, int64_t K, int32_t group_size,
                       int64_t n0, int64_t n1, int64_t n2,
                       float* out0, float* out1, float* out2, float* out3, void* stream);

/*
 * SiLU-gated gate/up matvec ([P1] fuseSwiGLUDecodeEntries: gate_proj +
 * up_proj + SwiGLU in one dispatch; the activation is silu(gate) * up):
 *   g[n] = x . w_gate[n],  u[n] = x . w_up[n],  h[n] = g / (1 + exp(-g)) * u.
 * Both matrices share N, K and gs.  g and u are bit-identical to
 * int4_matvec's outputs for the same weights.
 */
int int4_matvec_gated(const float* x,
                      const uint32_t* q_gate, const float* s_gate, const float* z_gate,
                      const uint32_t* q_up, const float* s_up, const float* z_up,
                      int64_t N, int64_t K, int32_t group_size, float* h, void* stream);

/*
 * The SiLU-gated gate/up matvec for M decode lanes in one launch ([P1]
 * fuseBatchSwiGLUMLPEntries: gate + up + SwiGLU as one fused batched GEMM
 * of the lockstep batch decode):
 *   H[m][n] = silu(X[m] . w_gate[n]) * (X[m] . w_up[n]),  0 <= M <= 8.
 * X [M][K], H [M][N].  M = 1 is int4_matvec_gated.  For M >= 2 the gate and
 * up sums are bit-identical to int4_matvec at the same M; the scale and
 * zero-point tables of both matrices share the local data share, so K/gs
 * is limited to about half of int4_matvec's M >= 2 limit.
 */
int int4_matvec_gated_lanes(const float* X, int32_t M,
                            const uint32_t* q_gate, const float* s_gate, const float* z_gate,
                            const uint32_t* q_up, const float* s_up, const float* z_up,
                            int64_t N, int64_t K, int32_t group_size, float* H, void* stream);

/*
 * The whole decode MLP block in one launch: the gated gate/up matvec, then
 * the down projection of its output ([P2] generateGepardBackboneGraph: the
 * layer's gate and up MatMulInt4 nodes, the SwiGLU node and the down
 * MatMulInt4 node; [P1] fuseSwiGLUDecodeEntries fuses the first three):
 *   h[f] = silu(x . w_gate[f]) * (x . w_up[f]),   0 <= f < F,
 *   y[d] = h . w_down[d],                         0 <= d < D.
 * x [D], h [F] (written), y [D].  w_gate and w_up are F columns of D
 * inputs, w_down is D columns of F inputs; all three use group_size, which
 * must divide both D and F.  h is bit-identical to int4_matvec_gated and y
 * to int4_matvec on that h.  h must be 16-byte aligned (it is the down
 * projection's input).
 *
 * workspace: at least int4_mlp_workspace_bytes() bytes of device memory,
 * 16-byte aligned, owned by the caller, all ZERO before its first use and
 * then left as the calls leave it: word 0 counts the completed fused calls,
 * word 1 is the timeout flag, and one flag per block follows, through which
 * the down projection waits until every part of h is written.  Calls that
 * share a workspace must not overlap in time.  The wait assumes the
 * launch's blocks are all resident at once (the grid is one block per
 * compute unit, and nothing else may occupy the device meanwhile); a block
 * that waits about a second gives up and sets word 1.  The outputs of that
 * call are then undefined, and every later fused call with that workspace
 * writes NaN to all of h and y and does nothing else, until the caller
 * zeroes the workspace again; int4_mlp_timed_out reads word 1.  Shapes the
 * fused launch does not cover (very small F or D, or K beyond the one-lane
 * register kernel) run as the two separate calls, with the same results,
 * and neither read nor write the workspace.
 */
size_t int4_mlp_workspace_bytes(void);
int int4_mlp(const float* x,
             const uint32_t* q_gate, const float* s_gate, const float* z_gate,
             const uint32_t* q_up, const float* s_up, const float* z_up,
             const uint32_t* q_down, const float* s_down, const float* z_down,
             int64_t D, int64_t F, int32_t group_size, float* h, float* y,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Whether a fused int4_mlp wait on `workspace` has timed out (word 1 of the
 * workspace is set): *timed_out = 1 if so, else 0.  Waits for `stream`
 * (every call enqueued on it before this one) to finish, then reads the
 * word; allocates nothing.  After a timeout, zero the workspace before
 * using it again.
 */
int int4_mlp_timed_out(const void* workspace, int32_t* timed_out, void* stream);

/*
 * Residual-add + RMSNorm prefixed matvec ([P4] WGSL_NORM_MATVEC_INT4,
 * NORM_MATVEC_INT4_SPEC with params [K, N, gs, eps]):
 *   r[k]   = a_a[k] + a_b[k]                          (binary32)
 *   inv    = 1 / sqrt(sum_k r[k]^2 / K + eps)
 *   x[k]   = r[k] * inv * w_norm[k]
 *   y[n]   = sum_k x[k] * w[n][k]
 * inv is one factor of the whole input, so the library computes
 * y[n] = inv * sum_k (r[k] * w_norm[k]) * w[n][k] and writes
 * norm_out[k] = (r[k] * w_norm[k]) * inv, each product rounded to binary32
 * (within the dot-product tolerance of the definition above; residual_out
 * is exact).  residual_out (r) and norm_out (x) are optional (NULL = not
 * written) and are written once per call.  eps must be finite and >= 0 (the pages default to
 * 1e-6).  N == 0 still writes residual_out / norm_out when they are given.
 * K * 4 bytes must fit the per-block local data share.
 */
int int4_matvec_norm(const float* a_a, const float* a_b, const float* w_norm, float eps,
                     const uint32_t* q, const float* scales, const float* zeros,
                     int64_t N, int64_t K, int32_t group_size,
                     float* y, float* residual_out, float* norm_out, void* stream);

/*
 * Dual matvec: two projections that share one input and the same N, K and
 * gs, in one call that reads the input once ([P4]
 * fuseDualMatVecDecodeEntries, DualMatVecInt4: q_proj + gate_proj or
 * k_proj + v_proj of full-attention decode; [P1] fuseBatchDualMatVecEntries,
 * its port to M decode lanes):
 *   y0[m][n] = X[m] . w0[n],  y1[m][n] = X[m] . w1[n],  0 <= M <= 8.
 * X [M][K], y0 and y1 [M][N].  Each output is bit-identical to int4_matvec
 * at the same M for its own matrix; limits as int4_matvec.
 */
int int4_matvec_dual(const float* X, int32_t M,
                     const uint32_t* q0, const float* s0, const float* z0,
                     const uint32_t* q1, const float* s1, const float* z1,
                     int64_t N, int64_t K, int32_t group_size,
                     float* y0, float* y1, void* stream);

/*
 * Sigmoid-gated input matvec ([P4] fuseGatedOProjDecodeEntries: the
 * attention SigmoidGate, attn_out * sigmoid(gate), recomputed inside the
 * o_proj matvec's input load, GatedMatVecInt4; [P1]
 * fuseBatchGatedProjEntries "sigmoid", its port to M decode lanes):
 *   xg[m][k] = a[m][k] * sigmoid(gate[m][k]),  sigmoid(t) = 1 / (1 + exp(-t)),
 *   y[m][n]  = xg[m] . w[n],  0 <= M <= 8.
 * a, gate [M][K] (16-byte aligned), y [M][N].  The gate is evaluated in
 * binary32 (with exp(-|t|), so it never overflows); y is within the
 * dot-product tolerance of the fp64 definition.  Limits as int4_matvec.
 */
int int4_matvec_sigmoid_gated(const float* a, const float* gate, int32_t M,
                              const uint32_t* q, const float* scales, const float* zeros,
                              int64_t N, int64_t K, int32_t group_size,
                              float* y, void* stream);

/*
 * SwiGLU-gated input matvec ([P4] fuseSwiGLUGatedProjDecodeEntries: a
 * standalone SwiGLU feeding an int4 projection, e.g. the linear-attention
 * block's silu(z) * norm_out into out_proj, SwiGLUGatedMatVecInt4; [P1]
 * fuseBatchGatedProjEntries "swiglu", its port to M decode lanes):
 *   xg[m][k] = silu(gate[m][k]) * up[m][k],  silu(t) = t / (1 + exp(-t)),
 *   y[m][n]  = xg[m] . w[n],  0 <= M <= 8.
 * Layouts, evaluation and limits as int4_matvec_sigmoid_gated.
 */
int int4_matvec_swiglu_gated(const float* gate, const float* up, int32_t M,
                             const uint32_t* q, const float* scales, const float* zeros,
                             int64_t N, int64_t K, int32_t group_size,
                             float* y, void* stream);

/*
 * RMSNorm-prefixed SwiGLU front of a decode MLP in one call ([P4]
 * fuseNormSwiGLUDecodeEntries, NormSwiGLUMatVec: ResidualRMSNorm + gate
 * matvec + up matvec + SwiGLU; block 0 keeps the residual sum for the
 * residual chain):
 *   r, inv, x as int4_matvec_norm;  g[n] = x . w_gate[n],  u[n] = x . w_up[n],
 *   h[n] = silu(g[n]) * u[n].
 * g and u are bit-identical to int4_matvec_norm's y for each matrix;
 * residual_out (r, exact in binary32) is optional (NULL = not written).
 * eps must be finite and >= 0.  N == 0 still writes residual_out when given.
 * K * 4 bytes must fit the per-block local data share.
 */
int int4_matvec_norm_swiglu(const float* a_a, const float* a_b, const float* w_norm, float eps,
                            const uint32_t* q_gate, const float* s_gate, const float* z_gate,
                            const uint32_t* q_up, const float* s_up, const float* z_up,
                            int64_t N, int64_t K, int32_t group_size,
                            float* h, float* residual_out, void* stream);

/*
 * Int4 embedding row gather and dequant ([P1] EmbeddingInt4, the first
 * kernel of a forward pass, and the per-layer-embedding rows gathered and
 * dequantized for the input tokens only; [P3] the embed_tokens .q / .scales
 * / .zeros triplet).  The table [N][K] is stored like a weight matrix (row n
 * = "column" n above):
 *   out[t][k] = (code(ids[t], k) - zero) * scale,   0 <= t < T,
 * in binary32 with one rounding, so the rows are bit-identical to the
 * definition.  ids is an int32 device array of T token ids; an id outside
 * [0, N) writes a row of zeros.  out is [T][K] fp32, 16-byte aligned.
 * T == 0 writes nothing; N == 0 (an empty table) writes zeros.
 */
int int4_embedding_gather(const int32_t* ids, int64_t T, const uint32_t* q, const float* scales,
                          const float* zeros, int64_t N, int64_t K, int32_t group_size,
                          float* out, void* stream);

/*
 * The same gather with the table kept in page-locked host memory
 * ([P1] setPleSource / streamPleRows: the per-layer-embedding table,
 * [vocab, L*256] int4 and about 1.2 GB for its model, stays off the GPU, and
 * each step only the rows of the input tokens are gathered and dequantized).
 * q, scales and zeros are host pointers into memory allocated with
 * hipHostMalloc (mapped for the device); the kernel reads the T rows over
 * the host link and dequantizes them on the GPU, so only T * (K/2 +
 * (K/gs) * 8) bytes cross it, and no host thread dequantizes anything.
 * ids (int32, T) and out ([T][K] fp32, 16-byte aligned) are device memory.
 * Results are bit-identical to int4_embedding_gather on the same table.
 * Table pointers that are not page-locked host memory are refused with
 * INT4_ERR_ARG before any launch (a kernel cannot read pageable memory).
 */
int int4_embedding_gather_host(const int32_t* ids, int64_t T, const uint32_t* q, const float* scales,
                               const float* zeros, int64_t N, int64_t K, int32_t group_size, float* out,
                               void* stream);

/*
 * Prefill GEMM: Y[t][n] = sum_k X[t][k] * w[n][k] for T tokens at once
 * ([P1] the prefill path runs a tiled matmul for any number of rows, decode
 * the K-parallel matvec).  Same weights, layouts and tolerance as
 * int4_matvec (X [T][K], Y [T][N] row-major; any T >= 0).  Runs on the
 * matrix cores with the activations split into two fp16 halves, so each
 * output is within 1e-4 * sum_k |x w| + 1e-6 of the exact sum.
 *
 * workspace: device memory of at least int4_gemm_workspace_bytes(T, N, K,
 * group_size) bytes, 256-byte aligned, owned by the caller; its contents are
 * scratch (overwritten, not read back across calls).  Two calls that share
 * a workspace must not overlap in time.  Requires N * K / 2 < 2^31.
 */
size_t int4_gemm_workspace_bytes(int64_t T, int64_t N, int64_t K, int32_t group_size);
int int4_gemm(const float* X, int64_t T, const uint32_t* q, const float* scales,
              const float* zeros, int64_t N, int64_t K, int32_t group_size, float* Y,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The prefill GEMM for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): int4_gemm with its workspace taken from a scratch array that
 * the library holds in device memory, INT4_GEMM_NOALLOC_SCRATCH_BYTES
 * (64 MiB) on each GPU it runs on, from the library's load until the
 * process ends.  The call allocates nothing.  A problem whose workspace
 * (int4_gemm_workspace_bytes(T, N, K, group_size)) exceeds that size
 * returns INT4_ERR_SHAPE with nothing launched (e.g. at K = 4096 up to
 * about T = 3968).  The scratch holds nothing across calls, but every call
 * on one GPU uses the same array: two calls that overlap in time on one GPU
 * (other streams or other host threads) race and give undefined results;
 * calls ordered on one stream are safe.  Arguments, validation and
 * results are those of int4_gemm, bit for bit.
 */
#define INT4_GEMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int int4_gemm_noalloc(const float* X, int64_t T, const uint32_t* q, const float* scales,
                      const float* zeros, int64_t N, int64_t K, int32_t group_size, float* Y,
                      void* stream);

/*
 * Measurement, not part of the method: one plain streaming read of `bytes`
 * bytes of `buf` (16-byte aligned, a multiple of 16), the ceiling that the
 * matvec calls' effective bandwidth is compared with.  `blocks` blocks of
 * `waves` waves (1..16) each read one contiguous slice with `unroll` (1, 2
 * or 4) 16-byte loads per lane in flight, and write the XOR of every 32-bit
 * word of their slice to sink[block] (`blocks` words).  Returns INT4_ERR_NULL,
 * _ALIGN, _SHAPE (a slice of 2 GiB or more) or _ARG (unroll) on bad
 * arguments, _HIP on a launch failure; asynchronous on `stream`.
 */
int int4_probe_stream_read(const void* buf, size_t bytes, int32_t blocks, int32_t waves,
                           int32_t unroll, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* INT4GEMV_H */
