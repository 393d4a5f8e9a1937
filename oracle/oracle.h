/*
 * oracle.h -- declarations of the CPU oracle (test infrastructure only).
 * Host pointers, row-major arrays, sizes in elements.  See oracle.c for the
 * definition each function follows and the passage of the pages it cites.
 */
#ifndef INT4_ORACLE_H
#define INT4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

void oracle_quantize_pack(const float* W, int64_t N, int64_t K, int32_t gs,
                          uint32_t* q, float* scales, float* zeros);
void oracle_dequant(const uint32_t* q, const float* scales, const float* zeros,
                    int64_t N, int64_t K, int32_t gs, float* dq);
void oracle_matvec(const float* X, int32_t M, const uint32_t* q, const float* scales,
                   const float* zeros, int64_t N, int64_t K, int32_t gs,
                   double* Y, double* B);
void oracle_matvec_f32(const float* X, int32_t M, const uint32_t* q, const float* scales,
                       const float* zeros, int64_t N, int64_t K, int32_t gs, float* Y);
void oracle_split4(const float* x, const uint32_t* q, const float* scales, const float* zeros,
                   int64_t N, int64_t K, int32_t gs, int64_t n0, int64_t n1, int64_t n2,
                   double* out0, double* out1, double* out2, double* out3,
                   double* b0, double* b1, double* b2, double* b3);
void oracle_gated(const float* x,
                  const uint32_t* q_gate, const float* s_gate, const float* z_gate,
                  const uint32_t* q_up, const float* s_up, const float* z_up,
                  int64_t N, int64_t K, int32_t gs,
                  double* h, double* g, double* u, double* bg, double* bu);
void oracle_norm(const float* a_a, const float* a_b, const float* w_norm, float eps,
                 const uint32_t* q, const float* scales, const float* zeros,
                 int64_t N, int64_t K, int32_t gs,
                 double* y, double* B, float* residual, double* normed);
void oracle_dual(const float* x,
                 const uint32_t* q0, const float* s0, const float* z0,
                 const uint32_t* q1, const float* s1, const float* z1,
                 int64_t N, int64_t K, int32_t gs,
                 double* y0, double* b0, double* y1, double* b1);
void oracle_input_gated(int32_t kind, const float* a, const float* b,
                        const uint32_t* q, const float* scales, const float* zeros,
                        int64_t N, int64_t K, int32_t gs,
                        double* y, double* B, double* xg);
void oracle_norm_swiglu(const float* a_a, const float* a_b, const float* w_norm, float eps,
                        const uint32_t* q_gate, const float* s_gate, const float* z_gate,
                        const uint32_t* q_up, const float* s_up, const float* z_up,
                        int64_t N, int64_t K, int32_t gs,
                        double* h, double* g, double* u, double* bg, double* bu,
                        float* residual);
void oracle_embedding(const int32_t* ids, int64_t T, const uint32_t* q, const float* scales,
                      const float* zeros, int64_t N, int64_t K, int32_t gs, float* out);

/* Threads the column loops use (OpenMP); results do not depend on it. */
void oracle_set_threads(int32_t n);
int32_t oracle_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
