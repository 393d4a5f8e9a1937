// kernels.hip -- HIP kernels for gfx950 (CDNA4, wave64): the int4 group-quantized
// streaming matvec family and the quantize/pack kernel.
//
// Sources: [P4] gerbil 1.12.0 -> 1.13.0, page 12 (WGSL_QUAD_MATVEC_INT4,
// WGSL_NORM_MATVEC_INT4: layout, dequant (code - zero) * scale, routing, norm
// prologue); [P1] gerbil 1.11.4 -> 1.13.0, page 9 (SwiGLU fusion, batched INT4
// GEMM for decode lanes).  The WGSL kernels give 16 lanes per column with a
// shared-memory lane sum; the design here is CDNA-native instead.
//
// The one-lane kernels (gemv_reg_kernel, gemv_lds_kernel):
//  * A column's K/32 sixteen-byte code units are spread over the 64 lanes of
//    a wave, so one buffer_load_dwordx4 of a wave is one contiguous piece of
//    one column (up to 1 KiB).  Each wave addresses its columns through
//    buffer resources (scalar base, 32-bit lane offsets), and the loads of
//    the next step are issued before the current step is computed.
//  * Dequant-dot with no int->float converts: a nibble masked into the low
//    bits of an fp16 half is the subnormal code * 2^-24 (exact), and
//    v_fma_mix_f32 multiplies the fp32 activation by it.  Odd inputs use the
//    nibble 4 bits higher (16 * code * 2^-24).  The activations are held
//    pre-scaled by 2^24 (even inputs) and 2^20 (odd inputs), exact
//    power-of-two scalings, so a unit's chain is sum x * code.  The zero
//    point is constant over a unit, so sum x * (code - zero) is that chain
//    minus zero * sum x, with the unit's activation sum computed once per
//    lane.  Per 32 weights: 4 shifts, 16 AND, 32 mixed FMAs, then one FMA
//    for the zero point and one multiply by the group's scale.
//  * Cross-lane sums are butterflies in the fixed order xor 32, xor 16 (lane
//    swaps across wave halves / row pairs), then xor 8, 4, 2, 1 (DPP row
//    rotations).  Several values are reduced at once by pairing them in the
//    swap steps; every value still sees exactly the single-value tree.
//
// gemv_reg_kernel (one lane, K <= 16384; every fused variant): K is cut into nch chunks
// of at most 64 units.  A block holds P rows of nch waves (about 8 waves);
// the block stages the activations once in LDS, then wave (p, c) keeps the
// inputs of chunk c in registers, streams the columns of row p NCOL at a
// time with the loads DEPTH steps ahead, and writes one partial per (column,
// chunk) to an LDS table.  After one barrier the block sums each column's
// partials in chunk order and runs the epilogue (routing, SiLU gate, norm
// scale, plain store).  Blocks are persistent: one per CU.
//
// gemv_lds_kernel (one lane, longer K): the activation row is staged in
// LDS, transposed so lane l reads unit l's inputs with conflict-free
// ds_read_b128; each wave walks whole columns chunk by chunk (the register
// kernel's nch chunks of cw units), reducing every chunk across the wave and
// summing the chunk totals in chunk order -- the register kernel's order.
//
// gemv_slice_kernel (two to eight lanes): the matrix cores, with K sliced
// over the waves of a block (described at the kernel).
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
constexpr float kEvenScale = 16777216.0f;  // 2^24: undoes the 2^-24 of even-input codes
constexpr float kOddScale = 1048576.0f;    // 2^20: undoes the 2^-20 of odd-input codes

__device__ __forceinline__ half2_t as_half2(uint32_t b) { return __builtin_bit_cast(half2_t, b); }
__device__ __forceinline__ uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bitsf(uint32_t v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }
// A wave-uniform 64-bit value moved to scalar registers (the 64-bit division
// that produces row bounds runs on the vector unit).
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ------------------------------------------------------------ reductions

// DPP move within 16-lane rows (row_ror:N = 0x120 + N).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return bitsf(__builtin_amdgcn_update_dpp(0u, fbits(v), CTRL, 0xF, 0xF, false));
}

// Levels xor 8, 4, 2, 1 inside each row.  row_ror by 2^j pairs lane i with a
// lane that differs from i ^ 2^j only in higher bits, whose value the
// previous levels already made equal.
__device__ __forceinline__ float row_allreduce(float v) {
  v += dpp_move<0x128>(v);
  v += dpp_move<0x124>(v);
  v += dpp_move<0x122>(v);
  v += dpp_move<0x121>(v);
  return v;
}

// Level xor 32 for two values: lower half of the result = a[l] + a[l+32],
// upper half = b[l-32] + b[l].
__device__ __forceinline__ float add_swap32(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(fbits(a), fbits(b), false, false);
  return bitsf(r[0]) + bitsf(r[1]);
}

// Level xor 16 for two values: rows of the result = a0+a1, b0+b1, a2+a3, b2+b3.
__device__ __forceinline__ float add_swap16(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(fbits(a), fbits(b), false, false);
  return bitsf(r[0]) + bitsf(r[1]);
}

// All-reduce of V values (V = 1, 2, 4 or 8).  Register j of z holds, in every
// lane of row r, the total of value reduced_index<V>(j, r).
template <int V>
__device__ __forceinline__ void wave_reduce(const float (&v)[V], float (&z)[(V + 3) / 4]) {
  static_assert(V == 1 || V == 2 || V == 4 || V == 8, "V must be 1, 2, 4 or 8");
  if constexpr (V == 1) {
    const float w = add_swap32(v[0], v[0]);
    z[0] = row_allreduce(add_swap16(w, w));
  } else if constexpr (V == 2) {
    const float w = add_swap32(v[0], v[1]);
    z[0] = row_allreduce(add_swap16(w, w));
  } else {
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      const float w0 = add_swap32(v[4 * j + 0], v[4 * j + 1]);
      const float w1 = add_swap32(v[4 * j + 2], v[4 * j + 3]);
      z[j] = row_allreduce(add_swap16(w0, w1));
    }
  }
}

template <int V>
__device__ __forceinline__ int reduced_index(int j, int row) {
  if constexpr (V == 1) return 0;
  if constexpr (V == 2) return row >> 1;
  return 4 * j + (((row & 1) << 1) | (row >> 1));
}

// Total over the wave, wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
  const float one[1] = {v};
  float z[1];
  wave_reduce<1>(one, z);
  return bitsf(__builtin_amdgcn_readfirstlane(fbits(z[0])));
}

// Wave-uniform totals of V values (any V): batches of 4, then 2, then 1, each
// value reduced with the single-value butterfly tree.
template <int V>
__device__ __forceinline__ void wave_totals(const float (&v)[V], float (&t)[V]) {
  auto lane_value = [](float z, int l) {
    return bitsf(__builtin_amdgcn_readlane(fbits(z), l));
  };
#pragma unroll
  for (int i = 0; i + 4 <= V; i += 4) {
    const float b[4] = {v[i], v[i + 1], v[i + 2], v[i + 3]};
    float z[1];
    wave_reduce<4>(b, z);
    t[i + 0] = lane_value(z[0], 0);
    t[i + 2] = lane_value(z[0], 16);
    t[i + 1] = lane_value(z[0], 32);
    t[i + 3] = lane_value(z[0], 48);
  }
  constexpr int r = V % 4;
  constexpr int i0 = V - r;
  if constexpr (r >= 2) {
    const float b[2] = {v[i0], v[i0 + 1]};
    float z[1];
    wave_reduce<2>(b, z);
    t[i0] = lane_value(z[0], 0);
    t[i0 + 1] = lane_value(z[0], 32);
  }
  if constexpr (r == 1 || r == 3) t[V - 1] = wave_sum(v[V - 1]);
}

// ------------------------------------------------------------ dequant-dot

template <int NSLOT>
struct Step {
  u32x4 q[NSLOT];
  float s[NSLOT];
  float z[NSLOT];
};

// The codes of the 32 inputs of one unit as 16 fp16 pairs, scaled by 2^-24
// (even inputs) or 2^-20 (odd inputs): each nibble is masked in place into
// the mantissa of a subnormal half, so the value is exact with no
// conversion.  Pair 4i+t holds inputs 8i+t and 8i+t+4.
__device__ __forceinline__ void unit_codes(u32x4 w, half2_t (&d)[16]) {
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = words[i];
    const uint32_t hi = words[i] >> 8;
    d[4 * i + 0] = as_half2(lo & 0x000F000Fu);
    d[4 * i + 1] = as_half2(lo & 0x00F000F0u);
    d[4 * i + 2] = as_half2(hi & 0x000F000Fu);
    d[4 * i + 3] = as_half2(hi & 0x00F000F0u);
  }
}

// sum_k x[k] * (code_k - zero) over one unit (x pre-scaled, xs the unit's
// activation sum from unit_xsum): the code products are accumulated k
// ascending with one rounding each, then the zero point's term -zero * xs is
// added with one fused rounding.  The zero point is constant over the unit
// (a group spans whole units), so this is the dequantized dot product with
// the subtraction moved out of the per-input work.
__device__ __forceinline__ float unit_dot(const float (&x)[32], const half2_t (&d)[16], float xs,
                                          float zero) {
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
  return fmaf(-zero, xs, t);
}

// Sum of one unit's 32 activations, k ascending, from the pre-scaled values
// (multiplying by 2^-24 or 2^-20 undoes the scaling exactly).
__device__ __forceinline__ float unit_xsum(const float (&x)[32]) {
  float t = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) t += x[k] * ((k & 1) ? (1.0f / kOddScale) : (1.0f / kEvenScale));
  return t;
}

// Activations of one unit: float4 v holds inputs 4j..4j+3.  Even inputs are
// scaled by 2^24 and odd inputs by 2^20 (exact power-of-two scalings), so the
// products with the fp16 codes code * 2^-24 / code * 2^-20 are plain
// x * code and a unit's sum needs no rescaling.
__device__ __forceinline__ float4 prescale4(float4 v) {
  return make_float4(v.x * kEvenScale, v.y * kOddScale, v.z * kEvenScale, v.w * kOddScale);
}

__device__ __forceinline__ void put4(float (&x)[32], int j, float4 v) {
  const float4 p = prescale4(v);
  x[4 * j + 0] = p.x;
  x[4 * j + 1] = p.y;
  x[4 * j + 2] = p.z;
  x[4 * j + 3] = p.w;
}

// Buffer resources of one wave's weight streams (scalar registers): each
// starts at the wave's first column, so every offset below is 32-bit.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit dwords (gfx9 family)
constexpr int kLoadNonTemporal = 2;       // cache policy: streamed, no reuse expected

struct StreamBufs {
  __amdgpu_buffer_rsrc_t q[2], s[2], z[2];
};

template <int NSTREAM>
__device__ __forceinline__ StreamBufs make_stream_bufs(const GemvArgs& a, int64_t c_begin, int64_t c_end) {
  StreamBufs b;
  const int64_t ncols = c_end > c_begin ? c_end - c_begin : 0;
  const int64_t qbytes = (int64_t)a.U * 16, gbytes = (int64_t)a.G * 4;
#pragma unroll
  for (int st = 0; st < NSTREAM; ++st) {
    b.q[st] = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.q[st]) + c_begin * qbytes), (short)0,
        (int)(ncols * qbytes), kBufferWord3);
    b.s[st] = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.s[st]) + c_begin * gbytes), (short)0,
        (int)(ncols * gbytes), kBufferWord3);
    b.z[st] = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.z[st]) + c_begin * gbytes), (short)0,
        (int)(ncols * gbytes), kBufferWord3);
  }
  return b;
}

// Issue the loads of one step: for slot c, the unit at byte offset `qoff` of
// column rel + c/NSTREAM (relative to the wave's first column) in weight
// stream c%NSTREAM, and the scale and zero at byte offset `soff` of that
// column's group table.  Column offsets are wave-uniform scalars and the lane
// offsets 32-bit vector registers, so each load is one buffer instruction
// with no 64-bit address arithmetic.  A column past the last one (`last`)
// reads column `last`; its result is never stored.  An inactive lane reads
// unit 0 of the column, and since its activations are 0 it adds exactly 0.
// The loads are unconditional and nothing here uses a loaded value, so the
// compiler's wait counts stay exact and the next step's loads overlap the
// current step's arithmetic.
template <int NCOL, int NSTREAM>
__device__ __forceinline__ void load_units(const GemvArgs& a, const StreamBufs& b, uint32_t rel,
                                           uint32_t last, uint32_t qoff, uint32_t soff,
                                           Step<NCOL * NSTREAM>& r) {
  const uint32_t qbytes = (uint32_t)a.U * 16u, gbytes = (uint32_t)a.G * 4u;
#pragma unroll
  for (int c = 0; c < NCOL * NSTREAM; ++c) {
    const int st = c % NSTREAM;
    const uint32_t col0 = rel + (uint32_t)(c / NSTREAM);
    const uint32_t col = col0 < last ? col0 : last;
    r.q[c] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(b.q[st], qoff, col * qbytes, kLoadNonTemporal));
    r.s[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(b.s[st], soff, col * gbytes, 0));
    r.z[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(b.z[st], soff, col * gbytes, 0));
  }
}

__device__ __forceinline__ int unit_group(const GemvArgs& a, int u) {
  return (int)(((uint64_t)u * a.g_magic) >> 40);
}

// ------------------------------------------------------------ RMSNorm prologue

// inv_rms = 1 / sqrt(sum_k (a_a + a_b)^2 / K + eps) ([P4] WGSL_NORM_MATVEC_INT4),
// identical in every block: per-thread strided partials, wave butterflies,
// waves summed in index order.  `scratch` holds one float per wave.
__device__ __forceinline__ float block_inv_rms(const GemvArgs& a, float* scratch) {
  const int n4 = a.K >> 2;
  const float4* aa = reinterpret_cast<const float4*>(a.x);
  const float4* ab = reinterpret_cast<const float4*>(a.x2);
  float ss = 0.0f;
  for (int i = threadIdx.x; i < n4; i += blockDim.x) {
    const float4 x1 = aa[i];
    const float4 x2 = ab[i];
    const float r0 = x1.x + x2.x, r1 = x1.y + x2.y, r2 = x1.z + x2.z, r3 = x1.w + x2.w;
    ss = fmaf(r0, r0, ss);
    ss = fmaf(r1, r1, ss);
    ss = fmaf(r2, r2, ss);
    ss = fmaf(r3, r3, ss);
  }
  const float wsum = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = wsum;
  __syncthreads();
  float total = scratch[0];
  const int nw = blockDim.x >> 6;
  for (int w = 1; w < nw; ++w) total += scratch[w];
  return 1.0f / sqrtf(total / (float)a.K + a.eps);
}

// r = a_a + a_b and x = r * w_norm for float4 i (binary32).  The matvec runs
// on x; inv_rms is a single factor of the whole input, applied to each
// finished column sum, so the reduction over K never delays the weight stream.
__device__ __forceinline__ void norm_in4(const GemvArgs& a, int i, float4& r, float4& x) {
  const float4 x1 = reinterpret_cast<const float4*>(a.x)[i];
  const float4 x2 = reinterpret_cast<const float4*>(a.x2)[i];
  const float4 g = reinterpret_cast<const float4*>(a.w_norm)[i];
  r = make_float4(x1.x + x2.x, x1.y + x2.y, x1.z + x2.z, x1.w + x2.w);
  x = make_float4(r.x * g.x, r.y * g.y, r.z * g.z, r.w * g.w);
}

// Block 0 writes residual_out = r and norm_out = (r * w_norm) * inv_rms
// (optional outputs, once per call).
__device__ __forceinline__ void write_norm_outputs(const GemvArgs& a, float inv) {
  if (blockIdx.x != 0 || (a.residual_out == nullptr && a.norm_out == nullptr)) return;
  float4* res = reinterpret_cast<float4*>(a.residual_out);
  float4* nrm = reinterpret_cast<float4*>(a.norm_out);
  for (int i = threadIdx.x; i < (a.K >> 2); i += blockDim.x) {
    float4 r, x;
    norm_in4(a, i, r, x);
    if (res) res[i] = r;
    if (nrm) nrm[i] = make_float4(x.x * inv, x.y * inv, x.z * inv, x.w * inv);
  }
}

// ------------------------------------------------------------ elementwise gates

// sigmoid(t) = 1 / (1 + e^-t) and silu(t) = t * sigmoid(t) in binary32, with
// e = e^-|t| so that the exponential never overflows: for negative t,
// sigmoid(t) = e / (1 + e).  ([P1] SwiGLU: silu(gate) * up; [P4] SigmoidGate
// feeding GatedMatVecInt4: attn_out * sigmoid(gate).)
__device__ __forceinline__ float sigmoid_f32(float t) {
  const float e = expf(-fabsf(t));
  return t >= 0.0f ? 1.0f / (1.0f + e) : e / (1.0f + e);
}
__device__ __forceinline__ float silu_f32(float t) {
  const float e = expf(-fabsf(t));
  return t >= 0.0f ? t / (1.0f + e) : (t * e) / (1.0f + e);
}

// Gated input ([P4] GatedMatVecInt4 / SwiGLUGatedMatVecInt4: the
// elementwise gate is rebuilt inside the matvec's input load) of one float4
// of p = a / gate and r = gate / up: kSigIn x = a * sigmoid(gate), kSwiIn
// x = silu(gate) * up.  gated_in4 takes float4 i of the rows x and x2.
template <int MODE>
__device__ __forceinline__ float4 gate4(float4 p, float4 r) {
  if constexpr (MODE == kSigIn)
    return make_float4(p.x * sigmoid_f32(r.x), p.y * sigmoid_f32(r.y), p.z * sigmoid_f32(r.z),
                       p.w * sigmoid_f32(r.w));
  else
    return make_float4(silu_f32(p.x) * r.x, silu_f32(p.y) * r.y, silu_f32(p.z) * r.z,
                       silu_f32(p.w) * r.w);
}
template <int MODE>
__device__ __forceinline__ float4 gated_in4(const GemvArgs& a, int i) {
  return gate4<MODE>(reinterpret_cast<const float4*>(a.x)[i], reinterpret_cast<const float4*>(a.x2)[i]);
}

// Column epilogue shared by both kernels: `tot[st][m]` are the finished sums
// of column `col` (stream st: 0 = the weights / gate / first projection,
// 1 = up / second projection).  `inv` is inv_rms for the norm modes and
// unused otherwise.
template <int M, int MODE>
__device__ __forceinline__ void store_column(const GemvArgs& a, int64_t col,
                                             const float (&tot)[mode_streams(MODE)][M],
                                             float inv) {
  if constexpr (MODE == kPlain) {
#pragma unroll
    for (int m = 0; m < M; ++m) a.out[0][(int64_t)m * a.N + col] = tot[0][m];
  } else if constexpr (MODE == kNorm) {
    a.out[0][col] = tot[0][0] * inv;
  } else if constexpr (MODE == kSplit4) {
    const float v = tot[0][0];
    if (col < a.n0) a.out[0][col] = v;
    else if (col < a.n1) a.out[1][col - a.n0] = v;
    else if (col < a.n2) a.out[2][col - a.n1] = v;
    else a.out[3][col - a.n2] = v;
  } else if constexpr (MODE == kDual) {
    a.out[0][col] = tot[0][0];
    a.out[1][col] = tot[1][0];
  } else if constexpr (MODE == kSigIn || MODE == kSwiIn) {
    a.out[0][col] = tot[0][0];
  } else if constexpr (MODE == kNormSwi) {
    // g and u are the int4_matvec_norm values of the two streams.
    const float g = tot[0][0] * inv;
    const float u = tot[1][0] * inv;
    a.out[0][col] = silu_f32(g) * u;
  } else {
    a.out[0][col] = silu_f32(tot[0][0]) * tot[1][0];
  }
}

// ------------------------------------------------------------ register kernel


template <int M, int NCOL, int MODE, int DEPTH>
__global__ __launch_bounds__(512) void gemv_reg_kernel(GemvArgs a) {
  constexpr int NSTREAM = mode_streams(MODE);
  constexpr int NSLOT = NCOL * NSTREAM;
  constexpr int V = M * NSLOT;
  constexpr int NZ = (V + 3) / 4;
  // [cols of the block][NSTREAM][M][nch], one float per wave, then the
  // staged activations (x_lds_offset)
  extern __shared__ float part[];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_int(threadIdx.x >> 6);
  const int nch = a.nch;
  const int P = a.rows_per_block;
  const int p = wave / nch;
  const int c = wave - p * nch;
  const int64_t R = (int64_t)gridDim.x * P;
  const int64_t blk_begin = uniform_i64((int64_t)blockIdx.x * P * a.N / R);
  const int64_t blk_end = uniform_i64(((int64_t)blockIdx.x * P + P) * a.N / R);
  const int64_t row = (int64_t)blockIdx.x * P + p;
  const int64_t c_begin = uniform_i64(row * a.N / R);
  const int64_t c_end = uniform_i64((row + 1) * a.N / R);
  const int u = c * a.cw + lane;
  const bool active = lane < a.cw && u < a.U;
  const uint32_t qoff = (uint32_t)(active ? u : 0) * 16u;
  const uint32_t soff = (uint32_t)(active ? unit_group(a, u) : 0) * 4u;
  float* scratch = part + a.part_floats;

  // Activations: the block stages the M rows once in LDS (coalesced; for
  // the norm, x = (a_a + a_b) * w_norm and block 0 writes residual_out; for
  // a gated input, the gated vector), then each lane keeps its unit's 32
  // inputs in registers for the sweep.
  float4* xl = reinterpret_cast<float4*>(part + x_lds_offset(a.part_floats));
  const int n4 = a.K >> 2;
  if constexpr (mode_has_norm(MODE)) {
    // Per-thread share of sum_k r_k^2, then the wave's total in its slot.
    float ssq = 0.0f;
    for (int i = threadIdx.x; i < n4; i += blockDim.x) {
      float4 r, v;
      norm_in4(a, i, r, v);
      ssq = fmaf(r.x, r.x, ssq);
      ssq = fmaf(r.y, r.y, ssq);
      ssq = fmaf(r.z, r.z, ssq);
      ssq = fmaf(r.w, r.w, ssq);
      if (blockIdx.x == 0 && a.residual_out) reinterpret_cast<float4*>(a.residual_out)[i] = r;
      xl[(i & 7) * a.U + (i >> 3)] = v;
    }
    const float wsum = wave_sum(ssq);
    if (lane == 0) scratch[wave] = wsum;
  } else if constexpr (mode_gates_input(MODE)) {
    for (int i = threadIdx.x; i < n4; i += blockDim.x) xl[(i & 7) * a.U + (i >> 3)] = gated_in4<MODE>(a, i);
  } else {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4* src = reinterpret_cast<const float4*>(a.x + (int64_t)m * a.K);
      for (int i = threadIdx.x; i < n4; i += blockDim.x) xl[(m * 8 + (i & 7)) * a.U + (i >> 3)] = src[i];
    }
  }
  // Ring of DEPTH + 1 register sets: the loads of step i + DEPTH are issued
  // before step i is computed.  The first weight loads go out once the
  // activation loads have returned (the memory counter is in order, so the
  // staging would otherwise wait for them) and overlap the barrier.
  // Every load is unconditional: steps past the wave's last column re-read
  // that column, and a wave without columns has an empty buffer range, whose
  // loads return 0 without touching memory.
  const StreamBufs bufs = make_stream_bufs<NSTREAM>(a, c_begin, c_end);
  const uint32_t last = c_end > c_begin ? (uint32_t)(c_end - c_begin - 1) : 0u;
  Step<NSLOT> s0, s1, s2;
  load_units<NCOL, NSTREAM>(a, bufs, 0u, last, qoff, soff, s0);
  if constexpr (DEPTH == 2) load_units<NCOL, NSTREAM>(a, bufs, (uint32_t)NCOL, last, qoff, soff, s1);
  __syncthreads();
  float x[M][32];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int j = 0; j < 8; ++j) put4(x[m], j, active ? xl[(m * 8 + j) * a.U + u] : make_float4(0.f, 0.f, 0.f, 0.f));

  float xs[M];
#pragma unroll
  for (int m = 0; m < M; ++m) xs[m] = unit_xsum(x[m]);

  const bool writer = V >= 4 ? (lane & 15) == 0 : (V == 2 ? (lane & 31) == 0 : lane == 0);
  auto step = [&](int64_t n, const Step<NSLOT>& r) {
    float vals[V];
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) {
      half2_t d[16];
      unit_codes(r.q[sl], d);
#pragma unroll
      for (int m = 0; m < M; ++m) vals[m * NSLOT + sl] = r.s[sl] * unit_dot(x[m], d, xs[m], r.z[sl]);
    }
    float z[NZ];
    wave_reduce<V>(vals, z);
    if (writer) {
      const int rrow = lane >> 4;
#pragma unroll
      for (int j = 0; j < NZ; ++j) {
        const int vi = reduced_index<V>(j, rrow);
        const int m = vi / NSLOT;
        const int sl = vi - m * NSLOT;
        const int64_t col = n + sl / NSTREAM;
        if (col < c_end)
          part[(((col - blk_begin) * NSTREAM + sl % NSTREAM) * M + m) * nch + c] = z[j];
      }
    }
  };

  // One pipeline stage: issue the loads DEPTH steps ahead into `far` (past
  // the last column they re-read it), then compute `cur` (columns n..).  No
  // load sits behind a branch, so the compiler's wait counts stay exact and
  // every step, the last ones included, overlaps the next loads.
  auto stage = [&](int64_t n, const Step<NSLOT>& cur, Step<NSLOT>& far) {
    load_units<NCOL, NSTREAM>(a, bufs, (uint32_t)(n - c_begin) + DEPTH * NCOL, last, qoff, soff, far);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
    step(n, cur);
  };
  if (c_begin < c_end) {
    int64_t n = c_begin;
    if constexpr (DEPTH == 1) {
      while (true) {
        stage(n, s0, s1);
        if ((n += NCOL) >= c_end) break;
        stage(n, s1, s0);
        if ((n += NCOL) >= c_end) break;
      }
    } else {
      while (true) {
        stage(n, s0, s2);
        if ((n += NCOL) >= c_end) break;
        stage(n, s1, s0);
        if ((n += NCOL) >= c_end) break;
        stage(n, s2, s1);
        if ((n += NCOL) >= c_end) break;
      }
    }
  }
  __syncthreads();

  // inv_rms = 1 / sqrt(sum_k r_k^2 / K + eps) ([P4] WGSL_NORM_MATVEC_INT4),
  // from the wave totals in wave order: the same value in every block.
  // Block 0 writes norm_out = x * inv_rms from the staged x.
  float inv = 1.0f;
  if constexpr (mode_has_norm(MODE)) {
    float ss = scratch[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) ss += scratch[w];
    inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
    if (blockIdx.x == 0 && a.norm_out) {
      for (int i = threadIdx.x; i < n4; i += blockDim.x) {
        const float4 v = xl[(i & 7) * a.U + (i >> 3)];
        reinterpret_cast<float4*>(a.norm_out)[i] = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
      }
    }
  }

  // Each column's chunk partials, summed in chunk order.
  const int64_t ncols = blk_end - blk_begin;
  for (int64_t j = threadIdx.x; j < ncols; j += blockDim.x) {
    float tot[NSTREAM][M];
#pragma unroll
    for (int st = 0; st < NSTREAM; ++st)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float* pp = part + ((j * NSTREAM + st) * M + m) * nch;
        float s = pp[0];
        for (int cc = 1; cc < nch; ++cc) s += pp[cc];
        tot[st][m] = s;
      }
    store_column<M, MODE>(a, blk_begin + j, tot, inv);
  }
}

// ------------------------------------------------------------ LDS kernel

// Activation row m is stored as float4 xl[m][j][u] = inputs 32u+4j .. 32u+4j+3,
// pre-scaled like the register kernel's activations (prescale4).
template <int M>
__device__ __forceinline__ void stage_x(const float* __restrict__ X, int K, int U, float4* xl) {
  const int n4 = K >> 2;
  for (int m = 0; m < M; ++m) {
    const float4* src = reinterpret_cast<const float4*>(X + (size_t)m * K);
    for (int i = threadIdx.x; i < n4; i += blockDim.x)
      xl[(m * 8 + (i & 7)) * U + (i >> 3)] = prescale4(src[i]);
  }
}

template <int M, int NCOL, int MODE>
__global__ __launch_bounds__(256) void gemv_lds_kernel(GemvArgs a) {
  constexpr int NSTREAM = mode_streams(MODE);
  constexpr int NSLOT = NCOL * NSTREAM;
  extern __shared__ float4 xl[];
  float inv = 1.0f;  // inv_rms (norm modes)

  if constexpr (mode_has_norm(MODE)) {
    float* scratch = reinterpret_cast<float*>(xl + (size_t)8 * a.U);
    inv = block_inv_rms(a, scratch);
    for (int i = threadIdx.x; i < (a.K >> 2); i += blockDim.x) {
      float4 r, v;
      norm_in4(a, i, r, v);
      xl[(i & 7) * a.U + (i >> 3)] = prescale4(v);
    }
    write_norm_outputs(a, inv);
  } else if constexpr (mode_gates_input(MODE)) {
    for (int i = threadIdx.x; i < (a.K >> 2); i += blockDim.x)
      xl[(i & 7) * a.U + (i >> 3)] = prescale4(gated_in4<MODE>(a, i));
  } else {
    stage_x<M>(a.x, a.K, a.U, xl);
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_int(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
  const int64_t c_begin = uniform_i64(gw * a.N / a.total_waves);
  const int64_t c_end = uniform_i64((gw + 1) * a.N / a.total_waves);
  if (c_begin >= c_end) return;

  // acc[m][sl]: the column's chunk partials summed in chunk order, the same
  // order as the register kernel's epilogue (wave-uniform values).
  float acc[M][NSLOT];
  const int nch = a.nch;
  auto compute = [&](int ch, const Step<NSLOT>& r) {
    const int u = ch * a.cw + lane;
    const bool active = lane < a.cw && u < a.U;
    half2_t d[NSLOT][16];
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) unit_codes(r.q[sl], d[sl]);
    float vals[M * NSLOT];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float x[32];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 v = active ? xl[(m * 8 + j) * a.U + u] : make_float4(0.f, 0.f, 0.f, 0.f);
        x[4 * j + 0] = v.x;
        x[4 * j + 1] = v.y;
        x[4 * j + 2] = v.z;
        x[4 * j + 3] = v.w;
      }
      const float xs = unit_xsum(x);
#pragma unroll
      for (int sl = 0; sl < NSLOT; ++sl)
        vals[m * NSLOT + sl] = r.s[sl] * unit_dot(x, d[sl], xs, r.z[sl]);
    }
    float tot[M * NSLOT];
    wave_totals<M * NSLOT>(vals, tot);
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int sl = 0; sl < NSLOT; ++sl)
        acc[m][sl] = ch == 0 ? tot[m * NSLOT + sl] : acc[m][sl] + tot[m * NSLOT + sl];
  };
  auto finish = [&](int64_t n) {
    if (lane != 0) return;
#pragma unroll
    for (int cc = 0; cc < NCOL; ++cc) {
      const int64_t col = n + cc;
      if (col >= c_end) break;
      float t[NSTREAM][M];
#pragma unroll
      for (int st = 0; st < NSTREAM; ++st)
#pragma unroll
        for (int m = 0; m < M; ++m) t[st][m] = acc[m][cc * NSTREAM + st];
      store_column<M, MODE>(a, col, t, inv);
    }
  };
  const StreamBufs bufs = make_stream_bufs<NSTREAM>(a, c_begin, c_end);
  const uint32_t last = (uint32_t)(c_end - c_begin - 1);
  auto load = [&](int64_t n, int ch, Step<NSLOT>& r) {
    const int u = ch * a.cw + lane;
    const bool active = lane < a.cw && u < a.U;
    load_units<NCOL, NSTREAM>(a, bufs, (uint32_t)(n - c_begin), last, (uint32_t)(active ? u : 0) * 16u,
                              (uint32_t)(active ? unit_group(a, u) : 0) * 4u, r);
  };

  Step<NSLOT> ra, rb;
  int64_t n = c_begin;
  int ch = 0;
  load(n, ch, ra);
  while (true) {
    int ch2 = ch + 1;
    int64_t n2 = n;
    if (ch2 == nch) { ch2 = 0; n2 += NCOL; }
    bool more = n2 < c_end;
    if (more) load(n2, ch2, rb);
    compute(ch, ra);
    if (ch == nch - 1) finish(n);
    if (!more) break;
    n = n2;
    ch = ch2;

    ch2 = ch + 1;
    n2 = n;
    if (ch2 == nch) { ch2 = 0; n2 += NCOL; }
    more = n2 < c_end;
    if (more) load(n2, ch2, ra);
    compute(ch, rb);
    if (ch == nch - 1) finish(n);
    if (!more) break;
    n = n2;
    ch = ch2;
  }
}

// ------------------------------------------------------------ embedding gather

// out[t][k] = (code - zero) * scale of row ids[t] of a table stored like the
// weight columns ([P1] EmbeddingInt4 and the per-layer-embedding row gather).
// One lane per 32-bit code word: a 4-byte load, eight values, two 16-byte
// stores, so a wave reads 256 contiguous bytes and writes 2 KiB.  The value
// is rounded once, as the definition states.  Ids outside [0, N) write zeros.
__global__ __launch_bounds__(256) void embedding_gather_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                               const uint32_t* __restrict__ q,
                                                               const float* __restrict__ scales,
                                                               const float* __restrict__ zeros, int64_t N,
                                                               int32_t K, int32_t gs, float* __restrict__ out) {
  const int64_t wpr = K >> 3;  // code words per row
  const int64_t total = T * wpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t t = i / wpr;
    const int64_t w = i - t * wpr;
    const int64_t n = ids[t];
    float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
    if (n >= 0 && n < N) {
      const uint32_t word = q[n * wpr + w];
      const int64_t g = n * (K / gs) + (w * 8) / gs;
      const float sc = scales[g], zp = zeros[g];
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ((float)((word >> (4 * j)) & 15u) - zp) * sc;
      lo = make_float4(v[0], v[1], v[2], v[3]);
      hi = make_float4(v[4], v[5], v[6], v[7]);
    }
    float4* dst = reinterpret_cast<float4*>(out + t * (int64_t)K + w * 8);
    dst[0] = lo;
    dst[1] = hi;
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
// Wave-level quantizer: a group of gs inputs (gs/8 words) lives on TPG
// consecutive lanes of one wave (TPG the power of two >= gs/8, at most 64),
// each lane holding WPT words (8 inputs each) in registers; min and max are
// all-reduced across the group's lanes with xor shuffles, so the group is
// read once and no LDS or barrier is involved.  The arithmetic is the same
// binary32 sequence as quantize_pack_kernel (min/max are exact in any
// order; a +0/-0 tie cannot change scale or zero).
template <int WPT>
__global__ __launch_bounds__(256) void quantize_pack_wave_kernel(const float* __restrict__ W,
                                                                 int64_t total_groups, int gs, int tpg,
                                                                 uint32_t* __restrict__ q,
                                                                 float* __restrict__ scales,
                                                                 float* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int gpw = 64 / tpg;  // groups per wave
  const int64_t grp = ((int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)) * gpw + lane / tpg;
  const int part = lane & (tpg - 1);
  const int wpg = gs >> 3;
  const bool live = grp < total_groups;
  const float* wg = W + (live ? grp : 0) * gs;

  float v[WPT][8];
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int wi = part + j * tpg;
    const bool has = live && wi < wpg;
    const int wc = has ? wi : 0;
    const float4 a0 = reinterpret_cast<const float4*>(wg)[2 * wc];
    const float4 a1 = reinterpret_cast<const float4*>(wg)[2 * wc + 1];
    v[j][0] = a0.x; v[j][1] = a0.y; v[j][2] = a0.z; v[j][3] = a0.w;
    v[j][4] = a1.x; v[j][5] = a1.y; v[j][6] = a1.z; v[j][7] = a1.w;
    if (has) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (v[j][e] < lo) lo = v[j][e];
        if (v[j][e] > hi) hi = v[j][e];
      }
    }
  }
  for (int o = tpg >> 1; o >= 1; o >>= 1) {
    const float lo2 = __shfl_xor(lo, o, 64);
    const float hi2 = __shfl_xor(hi, o, 64);
    if (lo2 < lo) lo = lo2;
    if (hi2 > hi) hi = hi2;
  }
  if (!live) return;
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
  if (part == 0) {
    scales[grp] = scale;
    zeros[grp] = zero;
  }
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int wi = part + j * tpg;
    if (wi < wpg) {
      uint32_t word = 0u;
      if (scale != 0.0f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float code = clamp_code(rintf(v[j][e] / scale) + zero);
          word |= (uint32_t)code << (4 * e);
        }
      }
      q[grp * wpg + wi] = word;
    }
  }
}

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

// ------------------------------------------------------------ dispatch

// ------------------------------------------------------------ matrix-core lanes kernel

// Two to eight decode lanes on the matrix cores, v_mfma_f32_16x16x32_f16:
// D[i][col] = sum_k A[i][k] * B[k][col] over the 32 inputs of one unit.
//  * B[k][col] = (code - zero) * 2^-24 for the even nibbles of a word and
//    (code - zero) * 2^-20 for the odd ones: each nibble is masked in place
//    into an fp16 subnormal (the odd ones four bits up) and the zero point,
//    shifted the same way, subtracted; all exact (the matrix cores keep fp16
//    subnormal inputs).
//  * A row i < 8 holds hi and row 8 + i holds lo for activation row m = i:
//    y = x[m][k] * 2^e (times 2^-4 for the odd-nibble inputs) is split into
//    hi = fp16(y) and lo = fp16(y - hi), both rounded toward zero; e is a
//    power of two per (row, slice) that puts the slice's largest |x| just
//    below 2^14.  One MFMA yields the hi and the lo products of every row;
//    they are added once per tile.
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and
// D[4*(l/16) .. +3][l%16].  Slot 8g + 2v of a unit is input 8g + v and slot
// 8g + 2v + 1 is input 8g + v + 4, the order the nibble masks produce.
//
// Work split.  Block b owns columns [b*N/B, (b+1)*N/B) in tiles of 16
// columns.  K is cut into slices of SU units; the block's W <= 8 waves (two
// per SIMD) take slices w, w + W, ..., keep the A operand of the slice in
// 4*SU registers and stream every tile of the block over it, DEPTH tiles of
// loads in flight.  A tile's codes load as 64 consecutive 16-byte units per
// instruction (SU units of each column in a row, so each column's bytes are
// contiguous); each lane also loads SZW scale and zero-point words of its
// column.  The tile passes through the wave's LDS stage to reach the matrix
// layout (lane (g, col) reads word g of every unit of column col).  Each
// unit's D is scaled by its group's scale into four accumulators; at the end
// of the tile the lo rows are added to the hi rows, multiplied by 2^(24 - e)
// and written to the block's partial table.  After a round of tiles, the
// block adds the waves' partials in wave order and stores Y.  Every row's
// arithmetic reads only that row's activations, so a lane's outputs never
// depend on the other lanes.

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 2^e as a float, e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return bitsf((uint32_t)(e + 127) << 23); }

// e for a row slice whose largest magnitude is amax: amax * 2^e < 2^14.
__device__ __forceinline__ int row_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int biased = (int)((fbits(amax) >> 23) & 0xFFu);
  const int E = biased == 0 ? -126 : biased - 126;  // amax < 2^E
  const int e = 14 - E;
  return e < -100 ? -100 : (e > 100 ? 100 : e);
}

// One tile of one slice in flight: SU/4 x 16 bytes of codes.
template <int SU>
struct SliceTile {
  u32x4 c[SU / 4];
};

// MODE: kPlain; kDual (the first half of the blocks runs stream 0 into
// out[0], the second half stream 1 into out[1]); kSigIn / kSwiIn (each
// lane's input is the elementwise gate of rows x and x2); kGated (each block
// runs both streams over its columns: a round's tiles of stream 0, then of
// stream 1, and the round's outputs are silu(g) * u).
template <int SU, int GS, int DEPTH, int MODE>
__global__ __launch_bounds__(64 * kSliceMaxWaves) void gemv_slice_kernel(GemvArgs a) {
  extern __shared__ float4 lds4[];
  constexpr int NJ = SU / 4;  // load instructions per tile
  constexpr int CS = slice_code_stride(SU);
  constexpr int kStage = slice_stage_words(SU);
  constexpr int H = SU / 2;  // units each half of a row's lanes converts
  constexpr int NB = 5;      // table chunks per thread loaded ahead of the activations
  static_assert(DEPTH == 2 || DEPTH == 3, "the ring below holds two or three tiles");
  constexpr int NV = MODE == kGated ? 2 : 1;  // weight streams per column tile
  const int M = a.M;
  const int K = a.K;
  const int U = a.U;
  const int G = a.G;
  const int GP = slice_table_stride(G, SU, GS);
  const int gsu = U / G;
  const int64_t N = a.N;
  const int lane = threadIdx.x & 63;
  const int hi4 = lane >> 4;   // matrix layout: k group / D row group
  const int lo16 = lane & 15;  // matrix layout: column
  const int wave = uniform_int(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int nsl = (U + SU - 1) / SU;
  const int nbk = MODE == kDual ? (int)gridDim.x / 2 : (int)gridDim.x;
  const int stream = MODE == kDual && (int)blockIdx.x >= nbk ? 1 : 0;
  const int64_t bk = (int64_t)blockIdx.x - (int64_t)stream * nbk;
  const int64_t cb = uniform_i64(bk * N / nbk);
  const int64_t ce = uniform_i64((bk + 1) * N / nbk);
  const int ntile = (int)((ce - cb + 15) >> 4);
  const int RT = a.rt;

  uint32_t* lds = reinterpret_cast<uint32_t*>(lds4);
  uint32_t* stage = lds + wave * kStage;
  float* part = reinterpret_cast<float*>(lds + W * kStage);
  // Tables of stream v: s_tab + v * RT * 16 * GP (and z_tab likewise).
  uint32_t* s_tab = lds + W * kStage + NV * RT * W * 128;
  uint32_t* z_tab = s_tab + NV * RT * 16 * GP;
  auto qbase = [&](int v) { return reinterpret_cast<const char*>(a.q[NV == 2 ? v : stream]); };
  auto sbase = [&](int v) { return reinterpret_cast<const char*>(a.s[NV == 2 ? v : stream]); };
  auto zbase = [&](int v) { return reinterpret_cast<const char*>(a.z[NV == 2 ? v : stream]); };
  float* const yout = a.out[NV == 2 ? 0 : stream];

  // Load layout: instruction j, lane l carries unit t of column col, where
  // 64j + l = SU*col + t.  The same unit goes to stage dword col*CS + 4t.
  uint32_t ld_unit[NJ], st_off[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = 64 * j + lane;
    const int col = c / SU;
    const int t = c - col * SU;
    ld_unit[j] = (uint32_t)(col * U + t);
    st_off[j] = (uint32_t)(col * CS + 4 * t);
  }

  for (int r0 = 0; r0 < ntile; r0 += RT) {
    const int rn = ntile - r0 < RT ? ntile - r0 : RT;

    // The round's scales and zero points.  Its columns [c_lo, c_lo + ncr)
    // are consecutive rows of the [N][G] arrays, so each array is one
    // contiguous range of ncr*G words, copied in 16-byte chunks by the whole
    // block (whole cache lines) into [column][GP] tables; the zero points
    // are stored as fp16 subnormal pairs, and the GP - G entries after a
    // column's groups are zero (groups named by units past K, whose
    // activations are zero).
    const int64_t c_lo = cb + 16 * (int64_t)r0;
    const int ncr = (int)((ce < c_lo + 16 * rn ? ce : c_lo + 16 * rn) - c_lo);
    const int nel = ncr * G;
    const int nchunk = (nel + 3) >> 2;
    const int vn = NV * rn;  // tiles of the round over all streams
    auto table_rsrc = [&](const char* base) {
      return __builtin_amdgcn_make_buffer_rsrc((void*)(base + c_lo * (int64_t)G * 4), (short)0, nel * 4,
                                               kBufferWord3);
    };
    const auto rs = table_rsrc(sbase(0));
    const auto rz = table_rsrc(zbase(0));
    auto table_put = [&](int c, u32x4 sv, u32x4 zv, int v = 0) {
      uint32_t* st_ = s_tab + v * RT * 16 * GP;
      uint32_t* zt_ = z_tab + v * RT * 16 * GP;
      if (c >= nchunk) return;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = 4 * c + k;
        if (e < nel) {
          // col = e / G: high word of e * ceil(2^32 / G), one step too
          // large at most.
          int col = a.g_recip ? (int)__umulhi((uint32_t)e, a.g_recip) : e;
          int g = e - col * G;
          if (g < 0) {
            col -= 1;
            g += G;
          }
          const uint32_t zi = (uint32_t)bitsf(zv[k]);
          st_[col * GP + g] = sv[k];
          zt_[col * GP + g] = zi | (zi << 16);
        }
      }
    };
    u32x4 tsv[NB], tzv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint32_t off = (uint32_t)(threadIdx.x + b * blockDim.x) * 16u;
      tsv[b] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kLoadNonTemporal));
      tzv[b] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, off, 0, kLoadNonTemporal));
    }
#pragma unroll
    for (int v = 0; v < NV; ++v)
      for (int col = wave; col < ncr; col += W)
        if (lane < GP - G) {
          s_tab[v * RT * 16 * GP + col * GP + G + lane] = 0u;
          z_tab[v * RT * 16 * GP + col * GP + G + lane] = 0u;
        }

    bool first_pass = true;
    for (int sl = wave; sl < nsl; sl += W) {
      const int u0 = SU * sl;
      const int h0 = u0 / gsu;

      // Activations of the slice for lane (g, i): row m = i & 7, units
      // H*half .. H*half + H - 1 (half = i >> 3), inputs 8g .. 8g+7 of each.
      const int m = lo16 & 7;
      const int half = lo16 >> 3;
      const bool row_live = m < M;
      float4 xp[H], xq[H];
#pragma unroll
      for (int tt = 0; tt < H; ++tt) {
        xp[tt] = make_float4(0.f, 0.f, 0.f, 0.f);
        xq[tt] = xp[tt];
      }
      if (row_live) {
#pragma unroll
        for (int tt = 0; tt < H; ++tt) {
          const int u = u0 + H * half + tt;
          const int64_t off = (int64_t)m * K + 32 * (u < U ? u : U - 1) + 8 * hi4;
          const float4* src = reinterpret_cast<const float4*>(a.x + off);
          xp[tt] = src[0];  // units past K (clamped address) are masked below
          xq[tt] = src[1];
          if constexpr (mode_gates_input(MODE)) {
            const float4* src2 = reinterpret_cast<const float4*>(a.x2 + off);
            xp[tt] = gate4<MODE>(xp[tt], src2[0]);
            xq[tt] = gate4<MODE>(xq[tt], src2[1]);
          }
        }
      }
      if (first_pass) {
        // The table: the first chunks are in flight, the rest (long rows
        // only) load here; then every wave's table writes complete before
        // any wave reads (LDS counter, then a barrier with no memory
        // fence).  The barrier also makes every wave issue its activation
        // loads before any wave issues weight loads: the memory pipeline
        // serves a CU's loads in issue order, so the small activation reads
        // must not queue behind the tiles.
        // The thread index made opaque here, so that the table's per-element
        // addresses are computed where they are used rather than hoisted
        // and held across the activation loads.
        int tid = (int)threadIdx.x;
        asm volatile("" : "+v"(tid));
#pragma unroll
        for (int b = 0; b < NB; ++b) table_put(tid + b * (int)blockDim.x, tsv[b], tzv[b]);
        for (int c = tid + NB * (int)blockDim.x; c < nchunk; c += (int)blockDim.x) {
          const u32x4 sv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)c * 16u, 0, kLoadNonTemporal));
          const u32x4 zv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, (uint32_t)c * 16u, 0, kLoadNonTemporal));
          table_put(c, sv, zv);
        }
        if constexpr (NV == 2) {  // the up stream's table
          const auto rs1 = table_rsrc(sbase(1));
          const auto rz1 = table_rsrc(zbase(1));
          for (int c = tid; c < nchunk; c += (int)blockDim.x) {
            const u32x4 sv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs1, (uint32_t)c * 16u, 0, kLoadNonTemporal));
            const u32x4 zv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz1, (uint32_t)c * 16u, 0, kLoadNonTemporal));
            table_put(c, sv, zv, 1);
          }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_s_barrier();
      }

      // Tile vt of the round (stream vt / rn, column tile vt % rn); tiles
      // past the round read nothing (an empty buffer range), so every load
      // is unconditional.
      auto load = [&](int vt, SliceTile<SU>& r) {
        const bool live = vt < vn;
        const int v = NV == 2 && live && vt >= rn ? 1 : 0;
        const int ti = live ? vt - v * rn : 0;
        const int64_t col0 = cb + 16 * (int64_t)(r0 + ti);
        const int ncols = live ? (ce - col0 < 16 ? (int)(ce - col0) : 16) : 0;
        const auto rq = __builtin_amdgcn_make_buffer_rsrc((void*)(qbase(v) + col0 * (int64_t)U * 16), (short)0,
                                                          ncols * U * 16, kBufferWord3);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          r.c[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rq, ld_unit[j] * 16u, (uint32_t)u0 * 16u, kLoadNonTemporal));
      };
      // Codes to [col][unit][word].
      auto write_stage = [&](const SliceTile<SU>& r) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) *reinterpret_cast<u32x4*>(stage + st_off[j]) = r.c[j];
      };

      // All but the last ring slot load now; the last one after the A
      // operand is built, when the activations' registers are free.
      SliceTile<SU> ring[DEPTH];
#pragma unroll
      for (int d = 0; d + 1 < DEPTH; ++d) load(d, ring[d]);
      __builtin_amdgcn_sched_barrier(0);

      // The slice's A operand.  The row maximum is reduced over the row's 8
      // lanes; e is per (row, slice).  Lanes i < 8 keep hi of their units
      // and take hi of the other half from lane i + 8; lanes i >= 8 keep lo
      // and take lo from lane i - 8 (DPP row rotation by 8, written only to
      // the receiving half's banks).
      u32x4 A[SU];
      float f[4];
      {
        float mx = 0.0f;
#pragma unroll
        for (int tt = 0; tt < H; ++tt) {
          const bool ok = u0 + H * half + tt < U;
          float v = fmaxf(fmaxf(fabsf(xp[tt].x), fabsf(xp[tt].y)), fmaxf(fabsf(xp[tt].z), fabsf(xp[tt].w)));
          v = fmaxf(v, fmaxf(fmaxf(fabsf(xq[tt].x), fabsf(xq[tt].y)), fmaxf(fabsf(xq[tt].z), fabsf(xq[tt].w))));
          mx = fmaxf(mx, ok ? v : 0.0f);
        }
        auto r32 = __builtin_amdgcn_permlane32_swap(fbits(mx), fbits(mx), false, false);
        mx = fmaxf(bitsf(r32[0]), bitsf(r32[1]));
        auto r16 = __builtin_amdgcn_permlane16_swap(fbits(mx), fbits(mx), false, false);
        mx = fmaxf(bitsf(r16[0]), bitsf(r16[1]));
        mx = fmaxf(mx, dpp_move<0x128>(mx));
        const int e = row_exponent(mx);
        const float sc = pow2f(e);
        const float sc16 = pow2f(e - 4);
#pragma unroll
        for (int tt = 0; tt < H; ++tt) {
          const bool ok = u0 + H * half + tt < U;
          const float s0 = ok ? sc : 0.0f, s1 = ok ? sc16 : 0.0f;
          const float4 p = xp[tt], q = xq[tt];
          const float y[8] = {p.x * s0, q.x * s0, p.y * s1, q.y * s1, p.z * s0, q.z * s0, p.w * s1, q.w * s1};
          u32x4 h, l;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const auto hh = __builtin_amdgcn_cvt_pkrtz(y[2 * k], y[2 * k + 1]);
            const auto ll = __builtin_amdgcn_cvt_pkrtz(y[2 * k] - (float)hh[0], y[2 * k + 1] - (float)hh[1]);
            h[k] = __builtin_bit_cast(uint32_t, hh);
            l[k] = __builtin_bit_cast(uint32_t, ll);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            A[tt][k] = __builtin_amdgcn_update_dpp(h[k], l[k], 0x128, 0xF, 0xC, false);
            A[H + tt][k] = __builtin_amdgcn_update_dpp(l[k], h[k], 0x128, 0xF, 0x3, false);
          }
        }
        const int rbase = 4 * (hi4 & 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e_lo = __builtin_amdgcn_readlane(e, r);
          const int e_hi = __builtin_amdgcn_readlane(e, 4 + r);
          f[r] = pow2f(24 - (rbase ? e_hi : e_lo));
        }
      }
      load(DEPTH - 1, ring[DEPTH - 1]);
      __builtin_amdgcn_sched_barrier(0);
      const int rem0 = u0 - h0 * gsu;  // unit-in-group of the slice's first unit

      auto compute = [&](int vt) {
        const uint32_t* cs = stage + lo16 * CS + hi4;
        // The tile's stream and column tile; the lane's column in the round
        // (the round's last one past its end) and the slice's first group.
        const int vs = NV == 2 && vt >= rn ? 1 : 0;
        const int i = vt - vs * rn;
        const int colr = 16 * i + lo16 < ncr ? 16 * i + lo16 : ncr - 1;
        const uint32_t* ts = s_tab + vs * RT * 16 * GP + colr * GP + h0;
        const uint32_t* tz = z_tab + vs * RT * 16 * GP + colr * GP + h0;
        uint32_t wd[SU];
#pragma unroll
        for (int t = 0; t < SU; ++t) wd[t] = cs[4 * t];
        const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4_t acc = z4;
        // B of unit t: nibbles minus zero point (zh: the group's zero point
        // as an fp16 subnormal pair).
        auto unit_b = [&](int t, uint32_t zh) {
          const half2_t z0 = as_half2(zh), z1 = as_half2(zh << 4);
          const uint32_t w = wd[t], w8 = wd[t] >> 8;
          u32x4 bw;
          bw[0] = __builtin_bit_cast(uint32_t, as_half2(w & 0x000F000Fu) - z0);
          bw[1] = __builtin_bit_cast(uint32_t, as_half2(w & 0x00F000F0u) - z1);
          bw[2] = __builtin_bit_cast(uint32_t, as_half2(w8 & 0x000F000Fu) - z0);
          bw[3] = __builtin_bit_cast(uint32_t, as_half2(w8 & 0x00F000F0u) - z1);
          return __builtin_bit_cast(half8_t, bw);
        };
        if constexpr (GS != 0) {
          // Groups alternate between two accumulators; a group is scaled
          // into acc after the next group's products are issued, so the
          // matrix core never waits for the scaling.
          constexpr int NG = SU / GS;
          f32x4_t dd[2] = {z4, z4};
#pragma unroll
          for (int t = 0; t < SU; ++t) {
            const int hh = t / GS;
            dd[hh & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, A[t]), unit_b(t, tz[hh]),
                                                               t % GS == 0 ? z4 : dd[hh & 1], 0, 0, 0);
            if (t % GS == GS - 1 && hh > 0) {
              const float sv = bitsf(ts[hh - 1]);
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) acc[rr] = fmaf(sv, dd[(hh - 1) & 1][rr], acc[rr]);
            }
          }
          const float sv = bitsf(ts[NG - 1]);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc[rr] = fmaf(sv, dd[(NG - 1) & 1][rr], acc[rr]);
        } else {
          f32x4_t d = z4;
          int rem = rem0, h = 0;
#pragma unroll
          for (int t = 0; t < SU; ++t) {
            const int hh = h;
            const bool first = rem == 0 || t == 0;
            const bool last = rem == gsu - 1 || t == SU - 1;
            rem = rem + 1 == gsu ? 0 : rem + 1;
            h += rem == 0 ? 1 : 0;
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, A[t]), unit_b(t, tz[hh]),
                                                       first ? z4 : d, 0, 0, 0);
            if (last) {
              const float sv = bitsf(ts[hh]);
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) acc[rr] = fmaf(sv, d[rr], acc[rr]);
            }
          }
        }
        // Lanes 0..31 hold the hi rows, lanes 32..63 the lo rows.
        float v[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) v[rr] = add_swap32(acc[rr], acc[rr]) * f[rr];
        if (hi4 < 2) {
          float* pp = part + ((size_t)(vt * W + wave) * 8 + 4 * hi4) * 16 + lo16;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) pp[16 * rr] = first_pass ? v[rr] : pp[16 * rr] + v[rr];
        }
      };

      // Whole turns of the ring: stage writes and loads unconditional
      // (tiles past the round read nothing), one back edge, so each stage
      // write waits only for its own slot; only the compute is skipped past
      // the round's last tile.
      for (int i = 0; i < vn; i += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
          write_stage(ring[d]);
          load(i + d + DEPTH, ring[d]);
          __builtin_amdgcn_sched_barrier(0);
          if (i + d < vn) compute(i + d);
        }
      }
      // The refills past the round are still in flight; let them land before
      // the ring registers are reused.
      __builtin_amdgcn_s_waitcnt(0);
      first_pass = false;
    }
    __syncthreads();
    // Y for the round's tiles: the waves' partials added in wave order.
    const int nout = rn * M * 16;
    for (int o = threadIdx.x; o < nout; o += blockDim.x) {
      const int c = o & 15;
      const int tm = o >> 4;
      const int i = tm / M;
      const int mm = tm - i * M;
      const int64_t col = cb + 16 * (int64_t)(r0 + i) + c;
      if (col < ce) {
        const float* pp = part + ((size_t)(i * W) * 8 + mm) * 16 + c;
        float y = pp[0];
        for (int w = 1; w < W; ++w) y += pp[(size_t)w * 128];
        if constexpr (NV == 2) {  // y is g; u from the up stream's tile rn + i
          const float* pu = part + ((size_t)((rn + i) * W) * 8 + mm) * 16 + c;
          float u = pu[0];
          for (int w = 1; w < W; ++w) u += pu[(size_t)w * 128];
          y = silu_f32(y) * u;
        }
        yout[(int64_t)mm * N + col] = y;
      }
    }
    __syncthreads();
  }
}

template <typename Kern>
hipError_t raise_lds_once(Kern kern, std::atomic<bool>& done, const LaunchShape& s) {
  // Dynamic LDS beyond 64 KiB must be allowed per kernel; once, for the
  // device maximum, before the first large launch of this instantiation.
  if (s.lds_bytes <= 65536 || done.load(std::memory_order_acquire)) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)s.lds_max);
  if (e == hipSuccess) done.store(true, std::memory_order_release);
  return e;
}

template <typename Kern>
hipError_t launch_or_query(Kern kern, std::atomic<bool>& raised, const GemvArgs& a,
                           const LaunchShape& s, hipStream_t stream, int* occupancy) {
  hipError_t e = raise_lds_once(kern, raised, s);
  if (e != hipSuccess) return e;
  if (occupancy)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, kern, s.block_threads, s.lds_bytes);
  hipLaunchKernelGGL(kern, dim3(s.grid), dim3(s.block_threads), s.lds_bytes, stream, a);
  return hipGetLastError();
}

template <int MODE, int M, int NCOL>
hipError_t launch_reg(const GemvArgs& a, const LaunchShape& s, hipStream_t stream, int* occupancy) {
  static std::atomic<bool> raised1{false}, raised2{false};
  if (s.depth == 2)
    return launch_or_query(gemv_reg_kernel<M, NCOL, MODE, 2>, raised2, a, s, stream, occupancy);
  return launch_or_query(gemv_reg_kernel<M, NCOL, MODE, 1>, raised1, a, s, stream, occupancy);
}

template <int MODE, int M, int NCOL>
hipError_t launch_lds(const GemvArgs& a, const LaunchShape& s, hipStream_t stream, int* occupancy) {
  static std::atomic<bool> raised{false};
  return launch_or_query(gemv_lds_kernel<M, NCOL, MODE>, raised, a, s, stream, occupancy);
}

template <int MODE>
hipError_t dispatch_reg(const GemvArgs& a, const LaunchShape& s, hipStream_t st, int* occ) {
  if (a.M != 1) return hipErrorInvalidValue;  // the register kernel runs one lane
  if constexpr (mode_streams(MODE) == 2) {
    return s.ncol == 1 ? launch_reg<MODE, 1, 1>(a, s, st, occ) : launch_reg<MODE, 1, 2>(a, s, st, occ);
  } else {
    switch (s.ncol) {
      case 1: return launch_reg<MODE, 1, 1>(a, s, st, occ);
      case 2: return launch_reg<MODE, 1, 2>(a, s, st, occ);
      default: return launch_reg<MODE, 1, 4>(a, s, st, occ);
    }
  }
}

template <int M>
hipError_t dispatch_lds_m(const GemvArgs& a, const LaunchShape& s, hipStream_t st, int* occ) {
  return s.ncol == 1 ? launch_lds<kPlain, M, 1>(a, s, st, occ) : launch_lds<kPlain, M, 2>(a, s, st, occ);
}

template <int SU, int DEPTH, int MODE>
hipError_t dispatch_slice_su(const GemvArgs& a, const LaunchShape& s, hipStream_t st, int* occ) {
  static std::atomic<bool> raised1{false}, raised2{false}, raised4{false}, raised0{false};
  switch (slice_class(a.U / a.G)) {
    case 1: return launch_or_query(gemv_slice_kernel<SU, 1, DEPTH, MODE>, raised1, a, s, st, occ);
    case 2: return launch_or_query(gemv_slice_kernel<SU, 2, DEPTH, MODE>, raised2, a, s, st, occ);
    case 4: return launch_or_query(gemv_slice_kernel<SU, 4, DEPTH, MODE>, raised4, a, s, st, occ);
    default: return launch_or_query(gemv_slice_kernel<SU, 0, DEPTH, MODE>, raised0, a, s, st, occ);
  }
}

template <int MODE>
hipError_t dispatch_slice_mode(const GemvArgs& a, const LaunchShape& s, hipStream_t st, int* occ) {
  if (a.su == 24) return dispatch_slice_su<24, 2, MODE>(a, s, st, occ);
  if (a.su == 20) return dispatch_slice_su<20, 3, MODE>(a, s, st, occ);
  return dispatch_slice_su<16, 3, MODE>(a, s, st, occ);
}

hipError_t dispatch_slice(Mode mode, const GemvArgs& a, const LaunchShape& s, hipStream_t st, int* occ) {
  switch (mode) {
    case kPlain: return dispatch_slice_mode<kPlain>(a, s, st, occ);
    case kDual: return dispatch_slice_mode<kDual>(a, s, st, occ);
    case kSigIn: return dispatch_slice_mode<kSigIn>(a, s, st, occ);
    case kSwiIn: return dispatch_slice_mode<kSwiIn>(a, s, st, occ);
    case kGated: return dispatch_slice_mode<kGated>(a, s, st, occ);
    default: return hipErrorInvalidValue;  // no matrix-core form of this mode
  }
}

hipError_t dispatch(Mode mode, const GemvArgs& a, const LaunchShape& s, hipStream_t st, int* occ) {
  if (s.variant == kVariantSlice) return dispatch_slice(mode, a, s, st, occ);
  if (s.variant == kVariantReg) {
    switch (mode) {
      case kSplit4: return dispatch_reg<kSplit4>(a, s, st, occ);
      case kGated: return dispatch_reg<kGated>(a, s, st, occ);
      case kNorm: return dispatch_reg<kNorm>(a, s, st, occ);
      case kDual: return dispatch_reg<kDual>(a, s, st, occ);
      case kSigIn: return dispatch_reg<kSigIn>(a, s, st, occ);
      case kSwiIn: return dispatch_reg<kSwiIn>(a, s, st, occ);
      case kNormSwi: return dispatch_reg<kNormSwi>(a, s, st, occ);
      default: return dispatch_reg<kPlain>(a, s, st, occ);
    }
  }
  switch (mode) {
    case kSplit4: return launch_lds<kSplit4, 1, 1>(a, s, st, occ);
    case kGated: return launch_lds<kGated, 1, 1>(a, s, st, occ);
    case kNorm: return launch_lds<kNorm, 1, 1>(a, s, st, occ);
    case kDual: return launch_lds<kDual, 1, 1>(a, s, st, occ);
    case kSigIn: return launch_lds<kSigIn, 1, 1>(a, s, st, occ);
    case kSwiIn: return launch_lds<kSwiIn, 1, 1>(a, s, st, occ);
    case kNormSwi: return launch_lds<kNormSwi, 1, 1>(a, s, st, occ);
    default: break;
  }
  switch (a.M) {
    case 1: return dispatch_lds_m<1>(a, s, st, occ);
    case 2: return dispatch_lds_m<2>(a, s, st, occ);
    case 3: return dispatch_lds_m<3>(a, s, st, occ);
    case 4: return dispatch_lds_m<4>(a, s, st, occ);
    case 5: return dispatch_lds_m<5>(a, s, st, occ);
    case 6: return dispatch_lds_m<6>(a, s, st, occ);
    case 7: return dispatch_lds_m<7>(a, s, st, occ);
    default: return dispatch_lds_m<8>(a, s, st, occ);
  }
}

}  // namespace

int max_ncol(Mode mode, int M, int variant) {
  if (variant == kVariantReg) {
    if (mode_streams(mode) == 2) return 2;
    return M == 1 ? 4 : 2;
  }
  return mode == kPlain ? 2 : 1;
}

hipError_t gemv_occupancy(Mode mode, const GemvArgs& a, const LaunchShape& s, int* blocks_per_cu) {
  *blocks_per_cu = 0;
  return dispatch(mode, a, s, nullptr, blocks_per_cu);
}

hipError_t launch_gemv(Mode mode, const GemvArgs& a, const LaunchShape& s, hipStream_t stream) {
  return dispatch(mode, a, s, stream, nullptr);
}

hipError_t launch_embedding(const int32_t* ids, int64_t T, const uint32_t* q, const float* scales,
                            const float* zeros, int64_t N, int32_t K, int32_t gs, float* out,
                            hipStream_t stream) {
  const int64_t total = T * (K / 8);
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;  // grid-stride beyond this
  hipLaunchKernelGGL(embedding_gather_kernel, dim3((unsigned)grid), dim3(256), 0, stream, ids, T, q,
                     scales, zeros, N, K, gs, out);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* W, int64_t total_groups, int32_t gs, uint32_t* q,
                           float* scales, float* zeros, hipStream_t stream) {
  const int wpg = gs / 8;
  if (wpg <= 512) {
    // Wave kernel: tpg = next power of two >= words per group (<= 64 lanes),
    // WPT words per lane.
    int tpg = 1;
    while (tpg < wpg && tpg < 64) tpg <<= 1;
    const int wpt = (wpg + tpg - 1) / tpg;
    const int64_t groups_per_block = 4 * (64 / tpg);
    const int64_t grid = (total_groups + groups_per_block - 1) / groups_per_block;
    if (wpt == 1)
      hipLaunchKernelGGL(quantize_pack_wave_kernel<1>, dim3((unsigned)grid), dim3(256), 0, stream, W, total_groups, gs, tpg, q, scales, zeros);
    else if (wpt == 2)
      hipLaunchKernelGGL(quantize_pack_wave_kernel<2>, dim3((unsigned)grid), dim3(256), 0, stream, W, total_groups, gs, tpg, q, scales, zeros);
    else if (wpt <= 4)
      hipLaunchKernelGGL(quantize_pack_wave_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream, W, total_groups, gs, tpg, q, scales, zeros);
    else
      hipLaunchKernelGGL(quantize_pack_wave_kernel<8>, dim3((unsigned)grid), dim3(256), 0, stream, W, total_groups, gs, tpg, q, scales, zeros);
    return hipGetLastError();
  }
  const int tpg = wpg < 256 ? wpg : 256;
  const int gpb = 256 / tpg < 64 ? 256 / tpg : 64;
  const int64_t grid = (total_groups + gpb - 1) / gpb;
  hipLaunchKernelGGL(quantize_pack_kernel, dim3((unsigned)grid), dim3(256), 0, stream, W,
                     total_groups, gs, tpg, gpb, q, scales, zeros);
  return hipGetLastError();
}

}  // namespace int4gemv
