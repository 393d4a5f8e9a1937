/*
 * oracle.c -- plain, slow CPU oracle for the int4 group-quantized matvec family.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke entry point and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never links, imports or calls it, and
 * this file shares no code, header, table or constant with that path.
 *
 * Sources (the four gerbil diff pages):
 *   [P1] gerbil 1.11.4 -> 1.13.0, page 9  (index type declarations)
 *   [P2] gerbil 1.12.0 -> 1.13.0, page 8  (gpu module, Gepard backbone graph)
 *   [P3] gerbil 1.0.0-rc.9 -> 1.0.0, page 17 (gpu module)
 *   [P4] gerbil 1.12.0 -> 1.13.0, page 12 (kernel registry + Executor)
 *
 * Storage of one quantized weight matrix (N output columns, K inputs):
 *   q      u32 [N][K/8]  column n contiguous, eight 4-bit codes per word,
 *                        code of input k at bits 4*(k%8) of word k/8
 *                        ([P2] addLinearOp tensor triplet; [P4] fuseMambaFront
 *                        doc: column-major, one column contiguous; [P1]/[P3]
 *                        dequantizeMLXProjection: low nibble first)
 *   scales f32 [N][K/gs], zeros f32 [N][K/gs], group g covers k in [g*gs,(g+1)*gs)
 *   dequantized weight  w = (f32(code) - zero) * scale   ([P4] WGSL_QUAD_MATVEC_INT4)
 *
 * Every floating-point dot product here accumulates in fp64, sequentially in k.
 * Build with -ffp-contract=off and without -ffast-math: the quantizer must be
 * the exact IEEE binary32 sequence written below.
 *
 * Parity pins live in tests/test_oracle_*.py; no function here is unpinned.
 * Loops over independent output columns (or groups, or rows) are shared out
 * over OpenMP threads; nothing within one output depends on the thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* Output columns are independent, so the loops over them run on OpenMP
 * threads; each column is still computed by one thread in exactly the order
 * written, so the results do not depend on the thread count. */
void oracle_set_threads(int32_t n) { omp_set_num_threads(n > 0 ? n : 1); }
int32_t oracle_max_threads(void) { return (int32_t)omp_get_max_threads(); }

/* ---------------------------------------------------------------- helpers */

/* Code of input k of column n: nibble k%8 of word k/8, low nibble first. */
static unsigned code_at(const uint32_t* q, int64_t K, int64_t n, int64_t k) {
    uint32_t word = q[n * (K / 8) + k / 8];
    return (unsigned)((word >> (4 * (k % 8))) & 15u);
}

/* Dequantized weight of (n, k) in binary32: (code - zero) * scale.  The
 * subtraction of two small integers is exact, the product rounds once. */
static float dq_at(const uint32_t* q, const float* scales, const float* zeros,
                   int64_t K, int32_t gs, int64_t n, int64_t k) {
    int64_t gidx = n * (K / gs) + k / gs;
    float diff = (float)code_at(q, K, n, k) - zeros[gidx];
    return diff * scales[gidx];
}

/* Clamp of a binary32 value to [0, 15]; NaN and both zeros map to +0. */
static float clamp_0_15(float v) {
    if (!(v > 0.0f)) return 0.0f;
    if (v > 15.0f) return 15.0f;
    return v;
}

/* ------------------------------------------------------------- quantizer */

/*
 * Asymmetric per-group min/max quantization and packing.
 *
 * The pages import the quantizer (quantizeInt4, quantizeBackboneInt4) but do
 * not show its body ([P4] module imports; [P1] quantizeKaniBackbone docs).
 * The reading taken, for each group of gs consecutive inputs of one column,
 * all in binary32 with round-to-nearest-even:
 *   lo, hi = min, max of the group
 *   scale  = (hi - lo) / 15                       if hi > lo
 *            |c| / 15                             if the group is constant c != 0
 *   zero   = clamp(rint(-lo / scale), 0, 15)
 *   code   = clamp(rint(w / scale) + zero, 0, 15)
 * A constant-zero group, or one whose scale underflows to 0, stores
 * scale = 0, zero = 0 and all codes 0.  The clamp is applied in binary32
 * before the conversion to an integer.
 */
void oracle_quantize_pack(const float* W, int64_t N, int64_t K, int32_t gs,
                          uint32_t* q, float* scales, float* zeros) {
    int64_t groups = K / gs;
#pragma omp parallel
    {
    unsigned* cbuf = (unsigned*)malloc(sizeof(unsigned) * (size_t)gs);
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < groups; ++g) {
            const float* w = W + n * K + g * gs;
            float lo = w[0], hi = w[0];
            for (int32_t j = 1; j < gs; ++j) {
                if (w[j] < lo) lo = w[j];
                if (w[j] > hi) hi = w[j];
            }
            float scale;
            if (hi > lo) {
                float range = hi - lo;
                scale = range / 15.0f;
            } else {
                scale = fabsf(hi) / 15.0f;
            }
            float zero = 0.0f;
            if (scale == 0.0f) {
                scale = 0.0f;
                for (int32_t j = 0; j < gs; ++j) cbuf[j] = 0;
            } else {
                float neg_lo = -lo;
                zero = clamp_0_15(rintf(neg_lo / scale));
                for (int32_t j = 0; j < gs; ++j) {
                    float t = rintf(w[j] / scale);
                    float c = clamp_0_15(t + zero);
                    cbuf[j] = (unsigned)c;
                }
            }
            scales[n * groups + g] = scale;
            zeros[n * groups + g] = zero;
            /* Eight codes per u32, the first input of the eight in bits 0..3. */
            for (int32_t j = 0; j < gs; j += 8) {
                uint32_t word = 0;
                for (int t = 0; t < 8; ++t) word |= (uint32_t)cbuf[j + t] << (4 * t);
                q[n * (K / 8) + (g * gs + j) / 8] = word;
            }
        }
    }
    free(cbuf);
    }
}

/* Dequantized matrix, binary32 [N][K]: dq[n][k] = (code - zero) * scale. */
void oracle_dequant(const uint32_t* q, const float* scales, const float* zeros,
                    int64_t N, int64_t K, int32_t gs, float* dq) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            dq[n * K + k] = dq_at(q, scales, zeros, K, gs, n, k);
}

/* ------------------------------------------------------------- matvec */

/*
 * Y[m][n] = sum_k X[m][k] * dq[n][k]   (fp64, k ascending)
 * B[m][n] = sum_k |X[m][k] * dq[n][k]| (fp64), the scale of the error bound.
 * M decode lanes share one weight matrix; rows never interact
 * ([P1] batched INT4 GEMM of the lockstep batch decode path).
 */
void oracle_matvec(const float* X, int32_t M, const uint32_t* q, const float* scales,
                   const float* zeros, int64_t N, int64_t K, int32_t gs,
                   double* Y, double* B) {
    for (int32_t m = 0; m < M; ++m) {
        const float* x = X + (int64_t)m * K;
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)x[k] * (double)dq_at(q, scales, zeros, K, gs, n, k);
                acc += p;
                mag += fabs(p);
            }
            Y[(int64_t)m * N + n] = acc;
            B[(int64_t)m * N + n] = mag;
        }
    }
}

/*
 * The same dot product accumulated naively in binary32 (k ascending).  Used
 * only to check that the error bound admits an ordinary fp32 implementation.
 */
void oracle_matvec_f32(const float* X, int32_t M, const uint32_t* q, const float* scales,
                       const float* zeros, int64_t N, int64_t K, int32_t gs, float* Y) {
    for (int32_t m = 0; m < M; ++m) {
        const float* x = X + (int64_t)m * K;
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float p = x[k] * dq_at(q, scales, zeros, K, gs, n, k);
                acc = acc + p;
            }
            Y[(int64_t)m * N + n] = acc;
        }
    }
}

/*
 * Split-4 routing ([P4] WGSL_QUAD_MATVEC_INT4 output routing and the
 * fuseMambaFrontDecodeEntries doc): one matvec over the column-concatenated
 * matrix, column n written to
 *   out0[n] (n < n0), out1[n-n0] (n < n1), out2[n-n1] (n < n2), out3[n-n2].
 * B follows the same routing.  Requires 0 <= n0 <= n1 <= n2 <= N.
 */
void oracle_split4(const float* x, const uint32_t* q, const float* scales, const float* zeros,
                   int64_t N, int64_t K, int32_t gs, int64_t n0, int64_t n1, int64_t n2,
                   double* out0, double* out1, double* out2, double* out3,
                   double* b0, double* b1, double* b2, double* b3) {
    double* y = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* b = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    oracle_matvec(x, 1, q, scales, zeros, N, K, gs, y, b);
    for (int64_t n = 0; n < N; ++n) {
        if (n < n0) { out0[n] = y[n]; b0[n] = b[n]; }
        else if (n < n1) { out1[n - n0] = y[n]; b1[n - n0] = b[n]; }
        else if (n < n2) { out2[n - n1] = y[n]; b2[n - n1] = b[n]; }
        else { out3[n - n2] = y[n]; b3[n - n2] = b[n]; }
    }
    free(y);
    free(b);
}

/*
 * SiLU-gated gate/up matvec: h[n] = silu(g[n]) * u[n] with g = x . Wg[n],
 * u = x . Wu[n] and silu(t) = t / (1 + exp(-t))
 * ([P1] fuseSwiGLUDecodeEntries / SwiGLUGatedProj docs: "silu(gate) * up").
 * g, u and their bounds Bg, Bu are returned too (fp64).
 */
void oracle_gated(const float* x,
                  const uint32_t* q_gate, const float* s_gate, const float* z_gate,
                  const uint32_t* q_up, const float* s_up, const float* z_up,
                  int64_t N, int64_t K, int32_t gs,
                  double* h, double* g, double* u, double* bg, double* bu) {
    oracle_matvec(x, 1, q_gate, s_gate, z_gate, N, K, gs, g, bg);
    oracle_matvec(x, 1, q_up, s_up, z_up, N, K, gs, u, bu);
    for (int64_t n = 0; n < N; ++n) {
        double silu = g[n] / (1.0 + exp(-g[n]));
        h[n] = silu * u[n];
    }
}

/*
 * Residual-add + RMSNorm prefixed matvec ([P4] WGSL_NORM_MATVEC_INT4 and
 * NORM_MATVEC_INT4_SPEC):
 *   r[k]     = a_a[k] + a_b[k]                   (binary32; the residual output)
 *   inv_rms  = 1 / sqrt(sum_k r[k]^2 / K + eps)  (fp64)
 *   nrm[k]   = r[k] * inv_rms * w_norm[k]        (fp64; the norm output)
 *   y[n]     = sum_k nrm[k] * dq[n][k], B[n] = sum_k |nrm[k] * dq[n][k]|
 * The norm gain multiplies as stored ([P4] loader bakes any +1 offset into it).
 */
void oracle_norm(const float* a_a, const float* a_b, const float* w_norm, float eps,
                 const uint32_t* q, const float* scales, const float* zeros,
                 int64_t N, int64_t K, int32_t gs,
                 double* y, double* B, float* residual, double* normed) {
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        float r = a_a[k] + a_b[k];
        residual[k] = r;
        ss += (double)r * (double)r;
    }
    double inv_rms = 1.0 / sqrt(ss / (double)K + (double)eps);
    for (int64_t k = 0; k < K; ++k)
        normed[k] = (double)residual[k] * inv_rms * (double)w_norm[k];
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = normed[k] * (double)dq_at(q, scales, zeros, K, gs, n, k);
            acc += p;
            mag += fabs(p);
        }
        y[n] = acc;
        B[n] = mag;
    }
}

/* ------------------------------------------------------ next-row variants */

/*
 * Dual matvec ([P4] fuseDualMatVecDecodeEntries / DualMatVecInt4, and the
 * [P1] batch port fuseBatchDualMatVecEntries): two matrices with the same N,
 * K and group size read one shared input; each output is the plain matvec of
 * its own matrix, nothing else changes.
 */
void oracle_dual(const float* x,
                 const uint32_t* q0, const float* s0, const float* z0,
                 const uint32_t* q1, const float* s1, const float* z1,
                 int64_t N, int64_t K, int32_t gs,
                 double* y0, double* b0, double* y1, double* b1) {
    oracle_matvec(x, 1, q0, s0, z0, N, K, gs, y0, b0);
    oracle_matvec(x, 1, q1, s1, z1, N, K, gs, y1, b1);
}

/*
 * Input-gated matvec: the elementwise gate is applied to the input vector,
 * then the plain matvec runs on the gated vector.
 *   kind 0 ([P4] fuseGatedOProjDecodeEntries, GatedMatVecInt4 fed by the
 *          attention SigmoidGate):  xg[k] = a[k] * sigma(b[k]),
 *          sigma(t) = 1 / (1 + exp(-t))
 *   kind 1 ([P4] fuseSwiGLUGatedProjDecodeEntries, SwiGLUGatedMatVecInt4):
 *          xg[k] = silu(a[k]) * b[k],  silu(t) = t / (1 + exp(-t))
 * The gate is evaluated in fp64 from the binary32 inputs; y[n] = sum_k
 * xg[k] * dq[n][k] and B[n] = sum_k |xg[k] * dq[n][k]| (fp64, k ascending).
 */
void oracle_input_gated(int32_t kind, const float* a, const float* b,
                        const uint32_t* q, const float* scales, const float* zeros,
                        int64_t N, int64_t K, int32_t gs,
                        double* y, double* B, double* xg) {
    for (int64_t k = 0; k < K; ++k) {
        double ak = (double)a[k], bk = (double)b[k];
        if (kind == 0)
            xg[k] = ak * (1.0 / (1.0 + exp(-bk)));
        else
            xg[k] = (ak / (1.0 + exp(-ak))) * bk;
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = xg[k] * (double)dq_at(q, scales, zeros, K, gs, n, k);
            acc += p;
            mag += fabs(p);
        }
        y[n] = acc;
        B[n] = mag;
    }
}

/*
 * RMSNorm-prefixed SwiGLU front ([P4] fuseNormSwiGLUDecodeEntries /
 * NormSwiGLUMatVec): the residual-add + RMSNorm prologue of oracle_norm,
 * then the gate and up matvecs of the normalized vector and
 * h[n] = silu(g[n]) * u[n] as in oracle_gated.  residual = a_a + a_b in
 * binary32 (the one side output the pages keep).
 */
void oracle_norm_swiglu(const float* a_a, const float* a_b, const float* w_norm, float eps,
                        const uint32_t* q_gate, const float* s_gate, const float* z_gate,
                        const uint32_t* q_up, const float* s_up, const float* z_up,
                        int64_t N, int64_t K, int32_t gs,
                        double* h, double* g, double* u, double* bg, double* bu,
                        float* residual) {
    double* normed = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    oracle_norm(a_a, a_b, w_norm, eps, q_gate, s_gate, z_gate, N, K, gs, g, bg, residual, normed);
    oracle_norm(a_a, a_b, w_norm, eps, q_up, s_up, z_up, N, K, gs, u, bu, residual, normed);
    for (int64_t n = 0; n < N; ++n) {
        double silu = g[n] / (1.0 + exp(-g[n]));
        h[n] = silu * u[n];
    }
    free(normed);
}

/*
 * Int4 embedding row gather ([P1] EmbeddingInt4, the first kernel of a
 * forward pass, and the per-layer-embedding rows gathered and dequantized
 * for the input tokens; [P3] the embed_tokens .q/.scales/.zeros triplet):
 *   out[t][k] = dq[ids[t]][k] = (code - zero) * scale   (binary32)
 * A row of the table is stored like a weight column.  Ids outside [0, N)
 * give a row of zeros (the reading taken for an out-of-range token).
 */
void oracle_embedding(const int32_t* ids, int64_t T, const uint32_t* q, const float* scales,
                      const float* zeros, int64_t N, int64_t K, int32_t gs, float* out) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        int64_t n = ids[t];
        for (int64_t k = 0; k < K; ++k)
            out[t * K + k] = (n >= 0 && n < N) ? dq_at(q, scales, zeros, K, gs, n, k) : 0.0f;
    }
}
