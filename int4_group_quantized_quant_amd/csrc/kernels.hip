// kernels.hip -- HIP kernels for gfx950 (CDNA4, wave64): the int4 group-quantized
// streaming matvec family and the quantize/pack kernel.
//
// Sources: [P4] gerbil 1.12.0 -> 1.13.0, page 12 (WGSL_QUAD_MATVEC_INT4,
// WGSL_NORM_MATVEC_INT4: layout, dequant (code - zero) * scale, routing, norm
// prologue); [P1] gerbil 1.11.4 -> 1.13.0, page 9 (SwiGLU fusion, batched INT4
// GEMM for decode lanes).  The WGSL kernels give 16 lanes per column with a
// shared-memory lane sum; the design here is CDNA-native instead:
//
//  * A column's K/32 sixteen-byte units are spread over the 64 lanes of a wave
//    (lane l takes units l, l+64, ...), so every global_load_dwordx4 of a wave
//    is one contiguous 1 KiB piece of one column.  A wave walks a contiguous
//    range of columns NCOL at a time and prefetches the next step's units
//    while it computes the current one.
//  * The activation vector(s) are staged once per block into LDS, transposed
//    so that lane l reads unit l's 32 inputs with conflict-free ds_read_b128.
//  * Dequant-dot without zero-point folding and without int->float converts:
//    a nibble masked into the low bits of an fp16 half is the subnormal
//    code * 2^-24 (exactly); v_pk_add_f16 subtracts zero * 2^-24 exactly,
//    and v_fma_mix_f32 multiplies the fp32 activation by that fp16 (q - zero).
//    Odd inputs use the nibble 4 bits higher (value 16 * code * 2^-24), so
//    their activations are pre-scaled by 2^-4 in LDS.  One unit costs 1 shift,
//    16 AND, 16 packed-f16 subtractions and 32 mixed FMAs per 32 weights.
//    Each unit's sum is rescaled by 2^24 and multiplied by its group's scale.
//  * Cross-lane sums use DPP (quad perms, row mirrors, row broadcasts) in a
//    fixed order, so a column's result depends only on K, its weights and x:
//    split-4 routing, the gated streams and every lane count give the same
//    bits as the plain matvec over the same column.
//  * No MFMA: at one to eight lanes the work is a bandwidth-bound stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "internal.h"

namespace int4gemv {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxBlockThreads = 256;
constexpr float kTwo24 = 16777216.0f;  // undoes the 2^-24 of the fp16 subnormal codes

__device__ __forceinline__ half2_t as_half2(uint32_t b) { return __builtin_bit_cast(half2_t, b); }

__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Lane-shuffled copy of v through DPP; lanes in rows outside ROW_MASK read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes of a wave, returned as a wave-uniform value.  The
// order of the additions is fixed: pairs, quads, half rows, rows (all DPP
// within a 16-lane row), then row 0+1 and 2+3 via row_bcast15, then the two
// halves via row_bcast31; lane 63 ends with the total.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_move<0x140, 0xF>(v);  // row_mirror
  v += dpp_move<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// ------------------------------------------------------------ LDS staging

// The activation row of lane m is stored as float4 xl[m][j][u] = inputs
// 32u + 4j .. 32u + 4j + 3, with every odd input multiplied by 2^-4 (exact).
__device__ __forceinline__ float4 lds_scale_odd(float4 v) {
  v.y *= 0.0625f;
  v.w *= 0.0625f;
  return v;
}

template <int M>
__device__ __forceinline__ void stage_x(const float* __restrict__ X, int K, int U, float4* xl) {
  const int n4 = K >> 2;
  for (int m = 0; m < M; ++m) {
    const float4* src = reinterpret_cast<const float4*>(X + (size_t)m * K);
    for (int i = threadIdx.x; i < n4; i += blockDim.x) {
      const float4 v = src[i];
      xl[(m * 8 + (i & 7)) * U + (i >> 3)] = lds_scale_odd(v);
    }
  }
}

// Residual add + RMSNorm prologue ([P4] WGSL_NORM_MATVEC_INT4): every block
// computes the same inv_rms in the same order; block 0 writes residual_out
// and norm_out.  `red` is LDS scratch of one float per wave.
__device__ __forceinline__ void stage_norm(const GemvArgs& a, float4* xl, float* red) {
  const int n4 = a.K >> 2;
  const int U = a.U;
  const float4* aa = reinterpret_cast<const float4*>(a.x);
  const float4* ab = reinterpret_cast<const float4*>(a.x2);
  const float4* wn = reinterpret_cast<const float4*>(a.w_norm);
  float ss = 0.0f;
  for (int i = threadIdx.x; i < n4; i += blockDim.x) {
    const float4 x1 = aa[i];
    const float4 x2 = ab[i];
    float4 r;
    r.x = x1.x + x2.x;
    r.y = x1.y + x2.y;
    r.z = x1.z + x2.z;
    r.w = x1.w + x2.w;
    ss = fmaf(r.x, r.x, ss);
    ss = fmaf(r.y, r.y, ss);
    ss = fmaf(r.z, r.z, ss);
    ss = fmaf(r.w, r.w, ss);
    xl[(i & 7) * U + (i >> 3)] = r;  // unscaled residual for the second pass
  }
  const float wsum = wave_sum(ss);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = wsum;
  __syncthreads();
  float total = red[0];
  const int nw = blockDim.x >> 6;
  for (int w = 1; w < nw; ++w) total += red[w];
  const float inv_rms = 1.0f / sqrtf(total / (float)a.K + a.eps);
  const bool writer = blockIdx.x == 0;
  float4* res_out = reinterpret_cast<float4*>(a.residual_out);
  float4* nrm_out = reinterpret_cast<float4*>(a.norm_out);
  for (int i = threadIdx.x; i < n4; i += blockDim.x) {
    const int idx = (i & 7) * U + (i >> 3);
    const float4 r = xl[idx];
    const float4 g = wn[i];
    float4 x;
    x.x = r.x * inv_rms * g.x;
    x.y = r.y * inv_rms * g.y;
    x.z = r.z * inv_rms * g.z;
    x.w = r.w * inv_rms * g.w;
    if (writer) {
      if (res_out) res_out[i] = r;
      if (nrm_out) nrm_out[i] = x;
    }
    xl[idx] = lds_scale_odd(x);
  }
}

// ------------------------------------------------------------ streaming core

template <int NSLOT>
struct Step {
  u32x4 q[NSLOT];
  float s[NSLOT];
  float z[NSLOT];
};

// Issue the loads of step (n, ch): for each slot, unit ch*64 + lane of column
// n + slot/NSTREAM in weight stream slot%NSTREAM, with its scale and zero.
template <int NCOL, int NSTREAM>
__device__ __forceinline__ void load_step(const GemvArgs& a, int64_t n, int ch, int64_t c_end,
                                          int lane, Step<NCOL * NSTREAM>& r) {
  const int u = ch * kWave + lane;
  const bool active = u < a.U;
  const int g = (int)(((uint64_t)u * a.g_magic) >> 40);
#pragma unroll
  for (int c = 0; c < NCOL * NSTREAM; ++c) {
    const int st = c % NSTREAM;
    const int64_t col = n + c / NSTREAM;
    if (col < c_end && active) {
      r.q[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.q[st]) + col * a.U + u);
      r.s[c] = a.s[st][col * a.G + g];
      r.z[c] = a.z[st][col * a.G + g];
    } else {
      r.q[c] = u32x4{0u, 0u, 0u, 0u};
      r.s[c] = 0.0f;
      r.z[c] = 0.0f;
    }
  }
}

// (code - zero) for the 32 inputs of one unit as 16 fp16 pairs, scaled by
// 2^-24 (even inputs) or 2^-20 (odd inputs).  Pair 4i+t holds inputs
// 8i+t' and 8i+t'+4 with t' = (0, 1, 2, 3)[t].
__device__ __forceinline__ void unit_codes(u32x4 w, float zero, half2_t (&d)[16]) {
  const uint32_t zi = (uint32_t)zero;
  const uint32_t zlo_bits = zi | (zi << 16);
  const half2_t zlo = as_half2(zlo_bits);
  const half2_t zhi = as_half2(zlo_bits << 4);
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = words[i];
    const uint32_t hi = words[i] >> 8;
    d[4 * i + 0] = as_half2(lo & 0x000F000Fu) - zlo;
    d[4 * i + 1] = as_half2(lo & 0x00F000F0u) - zhi;
    d[4 * i + 2] = as_half2(hi & 0x000F000Fu) - zlo;
    d[4 * i + 3] = as_half2(hi & 0x00F000F0u) - zhi;
  }
}

// 2^-24 * sum of x[k] * (code_k - zero) over one unit, k ascending.
__device__ __forceinline__ float unit_dot(const float (&x)[32], const half2_t (&d)[16]) {
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t = fmaf(x[8 * i + 0], (float)d[4 * i + 0].x, t);
    t = fmaf(x[8 * i + 1], (float)d[4 * i + 1].x, t);
    t = fmaf(x[8 * i + 2], (float)d[4 * i + 2].x, t);
    t = fmaf(x[8 * i + 3], (float)d[4 * i + 3].x, t);
    t = fmaf(x[8 * i + 4], (float)d[4 * i + 0].y, t);
    t = fmaf(x[8 * i + 5], (float)d[4 * i + 1].y, t);
    t = fmaf(x[8 * i + 6], (float)d[4 * i + 2].y, t);
    t = fmaf(x[8 * i + 7], (float)d[4 * i + 3].y, t);
  }
  return t;
}

template <int M, int NSLOT>
__device__ __forceinline__ void compute_step(const float4* xl, int U, int ch, int lane,
                                             const Step<NSLOT>& r, float (&acc)[M][NSLOT]) {
  const int u = ch * kWave + lane;
  const bool active = u < U;
  half2_t d[NSLOT][16];
#pragma unroll
  for (int c = 0; c < NSLOT; ++c) unit_codes(r.q[c], r.z[c], d[c]);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float x[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 v = active ? xl[(m * 8 + j) * U + u] : make_float4(0.f, 0.f, 0.f, 0.f);
      x[4 * j + 0] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
    }
#pragma unroll
    for (int c = 0; c < NSLOT; ++c) {
      const float t = unit_dot(x, d[c]);
      acc[m][c] = fmaf(r.s[c], t * kTwo24, acc[m][c]);
    }
  }
}

template <int M, int NCOL, int MODE>
__device__ __forceinline__ void finish_group(const GemvArgs& a, int64_t n, int64_t c_end, int lane,
                                             float (&acc)[M][NCOL * (MODE == kGated ? 2 : 1)]) {
  constexpr int NSTREAM = MODE == kGated ? 2 : 1;
  constexpr int NSLOT = NCOL * NSTREAM;
  float tot[M][NSLOT];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int c = 0; c < NSLOT; ++c) {
      tot[m][c] = wave_sum(acc[m][c]);
      acc[m][c] = 0.0f;
    }
  if (lane != 0) return;
#pragma unroll
  for (int cc = 0; cc < NCOL; ++cc) {
    const int64_t col = n + cc;
    if (col >= c_end) break;
    if (MODE == kPlain) {
#pragma unroll
      for (int m = 0; m < M; ++m) a.out[0][(int64_t)m * a.N + col] = tot[m][cc];
    } else if (MODE == kNorm) {
      a.out[0][col] = tot[0][cc];
    } else if (MODE == kSplit4) {
      const float v = tot[0][cc];
      if (col < a.n0) a.out[0][col] = v;
      else if (col < a.n1) a.out[1][col - a.n0] = v;
      else if (col < a.n2) a.out[2][col - a.n1] = v;
      else a.out[3][col - a.n2] = v;
    } else {  // kGated: slot 2cc is the gate column, 2cc+1 the up column
      const float g = tot[0][2 * cc];
      const float u = tot[0][2 * cc + 1];
      a.out[0][col] = g / (1.0f + expf(-g)) * u;
    }
  }
}

template <int M, int NCOL, int MODE>
__global__ __launch_bounds__(kMaxBlockThreads) void gemv_int4_kernel(GemvArgs a) {
  constexpr int NSTREAM = MODE == kGated ? 2 : 1;
  constexpr int NSLOT = NCOL * NSTREAM;
  extern __shared__ float4 xl[];

  if (MODE == kNorm) {
    float* red = reinterpret_cast<float*>(xl + (size_t)8 * a.U);
    stage_norm(a, xl, red);
  } else {
    stage_x<M>(a.x, a.K, a.U, xl);
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_int(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  const int64_t c_begin = gw * a.N / a.total_waves;
  const int64_t c_end = (gw + 1) * a.N / a.total_waves;
  if (c_begin >= c_end) return;

  float acc[M][NSLOT];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int c = 0; c < NSLOT; ++c) acc[m][c] = 0.0f;

  const int nch = a.nch;
  Step<NSLOT> ra, rb;
  int64_t n = c_begin;
  int ch = 0;
  load_step<NCOL, NSTREAM>(a, n, ch, c_end, lane, ra);
  // Two-stage software pipeline, unrolled twice so the register sets ping-pong
  // instead of being copied.
  while (true) {
    int ch2 = ch + 1;
    int64_t n2 = n;
    if (ch2 == nch) { ch2 = 0; n2 += NCOL; }
    bool more = n2 < c_end;
    if (more) load_step<NCOL, NSTREAM>(a, n2, ch2, c_end, lane, rb);
    compute_step<M, NSLOT>(xl, a.U, ch, lane, ra, acc);
    if (ch == nch - 1) finish_group<M, NCOL, MODE>(a, n, c_end, lane, acc);
    if (!more) break;
    n = n2;
    ch = ch2;

    ch2 = ch + 1;
    n2 = n;
    if (ch2 == nch) { ch2 = 0; n2 += NCOL; }
    more = n2 < c_end;
    if (more) load_step<NCOL, NSTREAM>(a, n2, ch2, c_end, lane, ra);
    compute_step<M, NSLOT>(xl, a.U, ch, lane, rb, acc);
    if (ch == nch - 1) finish_group<M, NCOL, MODE>(a, n, c_end, lane, acc);
    if (!more) break;
    n = n2;
    ch = ch2;
  }
}

// ------------------------------------------------------------ quantize + pack

// Clamp to [0, 15] in binary32; NaN and both zeros give +0.
__device__ __forceinline__ float clamp_code(float v) {
  if (!(v > 0.0f)) return 0.0f;
  if (v > 15.0f) return 15.0f;
  return v;
}

// One block handles `gpb` groups of gs consecutive floats; `tpg` threads share
// a group, each thread owning whole 8-code words.  Min/max meet in LDS, one
// thread per group derives scale and zero, then every thread packs its words.
__global__ __launch_bounds__(256) void quantize_pack_kernel(const float* __restrict__ W,
                                                            int64_t total_groups, int gs, int tpg,
                                                            int gpb, uint32_t* __restrict__ q,
                                                            float* __restrict__ scales,
                                                            float* __restrict__ zeros) {
  __shared__ float lo_s[256];
  __shared__ float hi_s[256];
  __shared__ float sc_s[64];
  __shared__ float zr_s[64];
  const int t = threadIdx.x;
  const int lg = t / tpg;
  const int part = t - lg * tpg;
  const int64_t grp = (int64_t)blockIdx.x * gpb + lg;
  const bool valid = lg < gpb && grp < total_groups;
  const int wpg = gs >> 3;
  const float* wg = W + grp * gs;

  float lo = INFINITY, hi = -INFINITY;
  if (valid) {
    for (int wi = part; wi < wpg; wi += tpg) {
      const float4 v0 = reinterpret_cast<const float4*>(wg)[2 * wi];
      const float4 v1 = reinterpret_cast<const float4*>(wg)[2 * wi + 1];
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (v[e] < lo) lo = v[e];
        if (v[e] > hi) hi = v[e];
      }
    }
  }
  lo_s[t] = lo;
  hi_s[t] = hi;
  __syncthreads();
  if (valid && part == 0) {
    for (int p = 1; p < tpg; ++p) {
      if (lo_s[t + p] < lo) lo = lo_s[t + p];
      if (hi_s[t + p] > hi) hi = hi_s[t + p];
    }
    float scale;
    if (hi > lo) {
      const float range = hi - lo;
      scale = range / 15.0f;
    } else {
      scale = fabsf(hi) / 15.0f;
    }
    float zero = 0.0f;
    if (scale == 0.0f) {
      scale = 0.0f;
    } else {
      const float neg_lo = -lo;
      zero = clamp_code(rintf(neg_lo / scale));
    }
    sc_s[lg] = scale;
    zr_s[lg] = zero;
    scales[grp] = scale;
    zeros[grp] = zero;
  }
  __syncthreads();
  if (!valid) return;
  const float scale = sc_s[lg];
  const float zero = zr_s[lg];
  for (int wi = part; wi < wpg; wi += tpg) {
    const float4 v0 = reinterpret_cast<const float4*>(wg)[2 * wi];
    const float4 v1 = reinterpret_cast<const float4*>(wg)[2 * wi + 1];
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t word = 0u;
    if (scale != 0.0f) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float code = clamp_code(rintf(v[e] / scale) + zero);
        word |= (uint32_t)code << (4 * e);
      }
    }
    q[grp * wpg + wi] = word;
  }
}

// ------------------------------------------------------------ dispatch tables

template <int MODE, int M, int NCOL>
hipError_t launch_one(const GemvArgs& a, const LaunchShape& s, hipStream_t stream) {
  auto kern = gemv_int4_kernel<M, NCOL, MODE>;
  // Dynamic LDS beyond 64 KiB must be allowed per kernel; do it once, for the
  // device maximum, before the first large launch of this instantiation.
  static std::atomic<bool> lds_raised{false};
  if (s.lds_bytes > 65536 && !lds_raised.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)s.lds_max);
    if (e != hipSuccess) return e;
    lds_raised.store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(kern, dim3(s.grid), dim3(s.block_threads), s.lds_bytes, stream, a);
  return hipGetLastError();
}

template <int MODE, int M>
hipError_t launch_ncol(const GemvArgs& a, const LaunchShape& s, hipStream_t stream) {
  switch (s.ncol) {
    case 1: return launch_one<MODE, M, 1>(a, s, stream);
    case 2: return launch_one<MODE, M, 2>(a, s, stream);
    default: return launch_one<MODE, M, (M <= 2 ? 4 : 2)>(a, s, stream);
  }
}

}  // namespace

int max_ncol(Mode mode, int M) {
  if (mode == kGated) return 2;
  return M <= 2 ? 4 : 2;
}

hipError_t launch_gemv(Mode mode, const GemvArgs& a, const LaunchShape& s, hipStream_t stream) {
  switch (mode) {
    case kSplit4: return launch_ncol<kSplit4, 1>(a, s, stream);
    case kNorm: return launch_ncol<kNorm, 1>(a, s, stream);
    case kGated:
      return s.ncol == 1 ? launch_one<kGated, 1, 1>(a, s, stream)
                         : launch_one<kGated, 1, 2>(a, s, stream);
    case kPlain:
    default:
      switch (a.M) {
        case 1: return launch_ncol<kPlain, 1>(a, s, stream);
        case 2: return launch_ncol<kPlain, 2>(a, s, stream);
        case 3: return launch_ncol<kPlain, 3>(a, s, stream);
        case 4: return launch_ncol<kPlain, 4>(a, s, stream);
        case 5: return launch_ncol<kPlain, 5>(a, s, stream);
        case 6: return launch_ncol<kPlain, 6>(a, s, stream);
        case 7: return launch_ncol<kPlain, 7>(a, s, stream);
        default: return launch_ncol<kPlain, 8>(a, s, stream);
      }
  }
}

hipError_t launch_quantize(const float* W, int64_t total_groups, int32_t gs, uint32_t* q,
                           float* scales, float* zeros, hipStream_t stream) {
  const int wpg = gs / 8;
  const int tpg = wpg < 256 ? wpg : 256;
  const int gpb = 256 / tpg < 64 ? 256 / tpg : 64;
  const int64_t grid = (total_groups + gpb - 1) / gpb;
  hipLaunchKernelGGL(quantize_pack_kernel, dim3((unsigned)grid), dim3(256), 0, stream, W,
                     total_groups, gs, tpg, gpb, q, scales, zeros);
  return hipGetLastError();
}

}  // namespace int4gemv
