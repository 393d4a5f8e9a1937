// kernels.hip -- HIP kernels for gfx950 (CDNA4, wave64): the int4 group-quantized
// streaming matvec family and the quantize/pack kernel.
//
// Sources: [P4] gerbil 1.12.0 -> 1.13.0, page 12 (WGSL_QUAD_MATVEC_INT4,
// WGSL_NORM_MATVEC_INT4: layout, dequant (code - zero) * scale, routing, norm
// prologue); [P1] gerbil 1.11.4 -> 1.13.0, page 9 (SwiGLU fusion, batched INT4
// GEMM for decode lanes).  The WGSL kernels give 16 lanes per column with a
// shared-memory lane sum; the design here is CDNA-native instead.
//
// Shared by both matvec kernels:
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
// gemv_reg_kernel (one or two lanes, K <= 16384): K is cut into nch chunks
// of at most 64 units.  A block holds P rows of nch waves (about 8 waves);
// the block stages the activations once in LDS, then wave (p, c) keeps the
// inputs of chunk c in registers, streams the columns of row p NCOL at a
// time with the loads DEPTH steps ahead, and writes one partial per (column,
// chunk) to an LDS table.  After one barrier the block sums each column's
// partials in chunk order and runs the epilogue (routing, SiLU gate, norm
// scale, plain store).  Blocks are persistent: one per CU.
//
// gemv_lds_kernel (three to eight lanes, or longer K): the activation rows
// are staged in LDS, transposed so lane l reads unit l's inputs with
// conflict-free ds_read_b128; each wave walks whole columns chunk by chunk
// (the register kernel's nch chunks of cw units), reducing every chunk
// across the wave and summing the chunk totals in chunk order -- the
// register kernel's order, so every lane count gives the same bits.
//
// No MFMA: at one to eight lanes the work is a bandwidth-bound stream.
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

// Column epilogue shared by both kernels: `tot[st][m]` are the finished sums
// of column `col` (stream st: 0 = the weights / gate, 1 = up).
// `inv` is inv_rms for kNorm and unused otherwise.
template <int M, int MODE>
__device__ __forceinline__ void store_column(const GemvArgs& a, int64_t col,
                                             const float (&tot)[MODE == kGated ? 2 : 1][M],
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
  } else {
    // silu(g) = g / (1 + e^-g), evaluated as g e / (1 + e) with e = e^g for
    // negative g so that e^-g never overflows ([P1] SwiGLU: silu(gate) * up).
    const float g = tot[0][0];
    const float u = tot[1][0];
    const float e = expf(-fabsf(g));
    const float silu = g >= 0.0f ? g / (1.0f + e) : (g * e) / (1.0f + e);
    a.out[0][col] = silu * u;
  }
}

// ------------------------------------------------------------ register kernel


template <int M, int NCOL, int MODE, int DEPTH>
__global__ __launch_bounds__(512) void gemv_reg_kernel(GemvArgs a) {
  constexpr int NSTREAM = MODE == kGated ? 2 : 1;
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
  // the norm, x = (a_a + a_b) * w_norm and block 0 writes residual_out),
  // then each lane keeps its unit's 32 inputs in registers for the sweep.
  float4* xl = reinterpret_cast<float4*>(part + x_lds_offset(a.part_floats));
  const int n4 = a.K >> 2;
  if constexpr (MODE == kNorm) {
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
  if constexpr (MODE == kNorm) {
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
  constexpr int NSTREAM = MODE == kGated ? 2 : 1;
  constexpr int NSLOT = NCOL * NSTREAM;
  extern __shared__ float4 xl[];
  float inv = 1.0f;  // inv_rms (kNorm)

  if constexpr (MODE == kNorm) {
    float* scratch = reinterpret_cast<float*>(xl + (size_t)8 * a.U);
    inv = block_inv_rms(a, scratch);
    for (int i = threadIdx.x; i < (a.K >> 2); i += blockDim.x) {
      float4 r, v;
      norm_in4(a, i, r, v);
      xl[(i & 7) * a.U + (i >> 3)] = prescale4(v);
    }
    write_norm_outputs(a, inv);
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

// ------------------------------------------------------------ MFMA lane kernel

// Three to eight decode lanes on the matrix cores: v_mfma_f32_16x16x32_f16
// with D[m][col] = sum_k A[m][k] * B[k][col] over one 32-input unit, where
//  * B[k][col] = (code - zero) * 2^-24, the nibble masked into an fp16
//    subnormal and the zero point subtracted with v_pk_add_f16, both exact
//    (the matrix cores keep fp16 subnormal inputs);
//  * A[m][k] = x[m][k] * 2^e_m split into two fp16 parts hi + lo (hi the
//    rounded value, lo the rounded remainder), e_m a power of two that puts
//    the row's largest |x| just below 2^14; the two MFMAs accumulate the
//    exact products hi*B and lo*B in fp32.
// Lane l of a wave holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16]
// and D[4*(l/16) .. +3][l%16].  A 16-column tile is streamed with one 16-byte
// unit per lane: lane (col, g) loads unit 4s+g of column col, and a 4x4
// transpose across the lane groups (two permlane32 and two permlane16
// swaps) leaves word g of unit 4s+t in register t, so step t's MFMA covers
// exactly unit 4s+t, which lies in one group.  Each unit's D is scaled by
// its group's scale into the lane's four accumulators; at the end of a tile
// the rows m < M are multiplied by 2^(24 - e_m) and stored.  Rows of A are
// independent, so a lane's outputs never depend on the other lanes.

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaDepth = 5;  // quads of loads in flight ahead of the compute

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pick4(u32x4 v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Groups a quad of units can touch: 4 when a group is one unit (or of a
// size that is not 2 or a multiple of 4), 2 for two-unit groups, 1 when the
// group size is a multiple of 4 units.  Loading exactly these keeps every
// loaded register live, so the register allocator never reuses one that a
// load in flight will still write (which would force a full wait).
template <int GSU>
struct QuadGroups {
  static constexpr int n = GSU == 2 ? 2 : (GSU == 4 ? 1 : 4);
};

template <int NG>
struct GroupVals;
template <>
struct GroupVals<4> {
  u32x4 v;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  }
  __device__ __forceinline__ uint32_t get(int j) const { return pick4(v, j); }
};
template <>
struct GroupVals<2> {
  u32x2 v;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
  }
  __device__ __forceinline__ uint32_t get(int j) const { return j == 0 ? v.x : v.y; }
};
template <>
struct GroupVals<1> {
  uint32_t v;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    v = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  }
  __device__ __forceinline__ uint32_t get(int) const { return v; }
};

template <int GSU>
struct Quad {
  u32x4 q;                                   // one 16-byte unit of the lane's column
  GroupVals<QuadGroups<GSU>::n> s;           // scales from the quad's first group on
  GroupVals<QuadGroups<GSU>::n> z;           // zero points of the same groups
};

// Rows of 16 lanes x 4 registers, transposed: register t of lane group g
// ends up holding what register g of lane group t held.
__device__ __forceinline__ void transpose4x4(u32x4& w) {
  auto a = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
  auto b = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  w.x = c[0];
  w.y = c[1];
  w.z = d[0];
  w.w = d[1];
}


// 2^e as a float, e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return bitsf((uint32_t)(e + 127) << 23); }

// e_m for a row whose largest magnitude is amax: amax * 2^e < 2^14.
__device__ __forceinline__ int row_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int biased = (int)((fbits(amax) >> 23) & 0xFFu);
  const int E = biased == 0 ? -126 : biased - 126;  // amax < 2^E
  const int e = 14 - E;
  return e < -100 ? -100 : (e > 100 ? 100 : e);
}

// Largest value over the wave (butterfly with the same swaps and DPP row
// rotations as the sums).
__device__ __forceinline__ float wave_max(float v) {
  auto r32 = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
  v = fmaxf(bitsf(r32[0]), bitsf(r32[1]));
  auto r16 = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  v = fmaxf(bitsf(r16[0]), bitsf(r16[1]));
  v = fmaxf(v, dpp_move<0x128>(v));
  v = fmaxf(v, dpp_move<0x124>(v));
  v = fmaxf(v, dpp_move<0x122>(v));
  v = fmaxf(v, dpp_move<0x121>(v));
  return bitsf(__builtin_amdgcn_readfirstlane(fbits(v)));
}

// Group offset of unit t of a quad (t = 0..3) from the quad's first group.
// GSU is the group size in units when it is 1 or 2, 4 when it is a multiple
// of 4 (a quad then lies in one group), and 0 for any other size (the offset
// is computed from the unit-in-group counter uig, uniform over the wave).
template <int GSU>
__device__ __forceinline__ int quad_group_offset(int t, int uig, int gsu) {
  if constexpr (GSU == 1) return t;
  if constexpr (GSU == 2) return t >> 1;
  if constexpr (GSU == 4) return 0;
  int j = 0;
  j += (uig + t >= gsu) ? 1 : 0;
  j += (uig + t >= 2 * gsu) ? 1 : 0;
  j += (uig + t >= 3 * gsu) ? 1 : 0;
  return j;
}

// Slot of row m of entry ug in an A plane (16-byte slots, M per entry).
// For M = 4 and 8 the row is XOR-swizzled with bits of ug so that 16
// consecutive entries written for one row, and the M rows of one entry read
// by the MFMA lanes, both fall on distinct LDS banks; odd M needs no swizzle
// (its stride is already odd), M = 6 keeps a two-way conflict.
template <int M>
__device__ __forceinline__ int a_slot(int ug, int m) {
  if constexpr (M == 8) return ug * 8 + (m ^ ((ug >> 1) & 7));
  if constexpr (M == 4) return ug * 4 + (m ^ ((ug >> 2) & 3));
  return ug * M + m;
}

template <int MR, int GSU>
__global__ __launch_bounds__(512) void gemv_mfma_kernel(GemvArgs a) {
  extern __shared__ float4 lds4[];
  constexpr int M = MR;
  // Staging entries per thread: the LDS holds at most 160 KiB of planes,
  // i.e. at most 5120 / M entries of (unit, lane group) for M rows.
  constexpr int kEntries = (5120 / M + 511) / 512;
  const int K = a.K;
  const int U = a.U;
  const int G = a.G;
  const int gsu = U / G;        // units per group
  const int Up = (U + 3) & ~3;  // units padded to whole quads
  const int S = Up >> 2;        // quads per column
  const int lane = threadIdx.x & 63;
  const int wave = uniform_int(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;

  // 1. One pass over the activations: each thread loads the M rows of its
  // (unit, lane group) entries (8 inputs each) together, keeps them in
  // registers, and the block reduces every row's largest magnitude.
  // Entry ug = u*4 + g covers inputs 32u + 8g .. +7; units past K are zero.
  const int nug = Up * 4;
  float4 v0[kEntries][M], v1[kEntries][M];
#pragma unroll
  for (int e = 0; e < kEntries; ++e) {
    const int ug = threadIdx.x + e * blockDim.x;
    const int u = ug >> 2, g = ug & 3;
    const bool live = ug < nug && u < U;
    const int uc = live ? u : 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float4* src = reinterpret_cast<const float4*>(a.x + (int64_t)m * K + 32 * uc + 8 * g);
      v0[e][m] = src[0];
      v1[e][m] = src[1];
      if (!live) {
        v0[e][m] = make_float4(0.f, 0.f, 0.f, 0.f);
        v1[e][m] = v0[e][m];
      }
    }
  }
  float* red = reinterpret_cast<float*>(lds4);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float mx = 0.0f;
#pragma unroll
    for (int e = 0; e < kEntries; ++e) {
      const float4 p = v0[e][m], q = v1[e][m];
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(p.x), fabsf(p.y)), fmaxf(fabsf(p.z), fabsf(p.w))));
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(q.x), fabsf(q.y)), fmaxf(fabsf(q.z), fabsf(q.w))));
    }
    const float w = wave_max(mx);
    if (lane == 0) red[m * nwaves + wave] = w;
  }
  __syncthreads();
  float rowmax[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    rowmax[m] = red[m * nwaves];
    for (int w = 1; w < nwaves; ++w) rowmax[m] = fmaxf(rowmax[m], red[m * nwaves + w]);
  }
  float outf[4];  // 2^(24 - e_m) for this lane's output rows m = 4*(lane/16) + r
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    outf[r] = 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (4 * (lane >> 4) + r == m) outf[r] = pow2f(24 - row_exponent(rowmax[m]));
  }
  __syncthreads();

  // 2. Stage A from the registers: entry (u*4 + g)*M + m of the hi plane (lo
  // plane after it) holds the 8 fp16 values of row m for MFMA k-slots
  // 8g .. 8g+7 of unit u; slot 8g + 2v is input 32u + 8g + v and slot
  // 8g + 2v + 1 is input 32u + 8g + v + 4 (the order the nibble masks
  // produce).  y = x * 2^e_m is split into hi = fp16(y) and
  // lo = fp16(y - hi), both rounded toward zero two at a time
  // (v_cvt_pkrtz_f16_f32): y - hi is exact in fp32, so hi + lo carries y to
  // 2^-20 relative, or 2^-24 absolute below the fp16 normal range.
  const int plane = Up * 4 * M;
  half8_t* hi_plane = reinterpret_cast<half8_t*>(lds4);
  half8_t* lo_plane = hi_plane + plane;
#pragma unroll
  for (int e = 0; e < kEntries; ++e) {
    const int ug = threadIdx.x + e * blockDim.x;
    if (ug < nug) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float sc = pow2f(row_exponent(rowmax[m]));
        const float4 p = v0[e][m], q = v1[e][m];
        const float xv[8] = {p.x, q.x, p.y, q.y, p.z, q.z, p.w, q.w};
        u32x4 h, l;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float y0 = xv[2 * k] * sc, y1 = xv[2 * k + 1] * sc;
          const auto hh = __builtin_amdgcn_cvt_pkrtz(y0, y1);
          const auto ll = __builtin_amdgcn_cvt_pkrtz(y0 - (float)hh[0], y1 - (float)hh[1]);
          h[k] = __builtin_bit_cast(uint32_t, hh);
          l[k] = __builtin_bit_cast(uint32_t, ll);
        }
        hi_plane[a_slot<M>(ug, m)] = __builtin_bit_cast(half8_t, h);
        lo_plane[a_slot<M>(ug, m)] = __builtin_bit_cast(half8_t, l);
      }
    }
  }
  __syncthreads();

  // 3. Tiles of 16 columns: block b owns tiles [tb, te), wave w takes tiles
  // tb + w, tb + w + nwaves, ...
  const int64_t T = (a.N + 15) >> 4;
  const int64_t tb = uniform_i64((int64_t)blockIdx.x * T / gridDim.x);
  const int64_t te = uniform_i64(((int64_t)blockIdx.x + 1) * T / gridDim.x);
  const int64_t ntiles = te - tb > wave ? (te - tb - wave + nwaves - 1) / nwaves : 0;

  const int col_l = lane & 15;
  const int g = lane >> 4;
  const int m_a = col_l;  // A row of this lane
  const uint32_t a_mask = m_a < M ? 0xFFFFFFFFu : 0u;
  const int m_c = m_a < M ? m_a : M - 1;
  const char* hi_bytes = reinterpret_cast<const char*>(hi_plane);
  const char* lo_bytes = reinterpret_cast<const char*>(lo_plane);
  const uint32_t qcol = (uint32_t)U * 16u;
  const uint32_t gcol = (uint32_t)G * 4u;

  for (int64_t i = 0; i < ntiles; ++i) {
    const int64_t col0 = (tb + wave + i * nwaves) * 16;
    const int ncols = a.N - col0 < 16 ? (int)(a.N - col0) : 16;
    const uint32_t cl = (uint32_t)(col_l < ncols ? col_l : ncols - 1);
    const auto rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.q[0]) + col0 * qcol), (short)0, (int)(ncols * qcol), kBufferWord3);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.s[0]) + col0 * gcol), (short)0, (int)(ncols * gcol), kBufferWord3);
    const auto rz = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<const char*>(a.z[0]) + col0 * gcol), (short)0, (int)(ncols * gcol), kBufferWord3);
    const uint32_t vq = (cl * (uint32_t)U + (uint32_t)g) * 16u;
    const uint32_t vs = cl * (uint32_t)G * 4u;

    // Load cursor: quad ls and its first group lg (uniform).  Loads past the
    // column's last quad re-read it.
    int ls = 0, lg = 0, luig = 0;
    auto load = [&](Quad<GSU>& r) {
      r.q = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, vq, 64u * (uint32_t)ls,
                                                                            kLoadNonTemporal));
      r.s.load(rs, vs, 4u * (uint32_t)lg);
      r.z.load(rz, vs, 4u * (uint32_t)lg);
      // Advance one quad (none past the last), branch-free.
      const int adv = ls + 1 < S ? 1 : 0;
      const int t4 = luig + 4 * adv;
      const int inc = (t4 >= gsu ? 1 : 0) + (t4 >= 2 * gsu ? 1 : 0) + (t4 >= 3 * gsu ? 1 : 0) +
                      (t4 >= 4 * gsu ? 1 : 0);
      ls += adv;
      lg += inc;
      luig = t4 - inc * gsu;
    };
    // Compute cursor: quad cs, first group's unit-in-group counter cuig.
    int cs = 0, cuig = 0;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    auto compute = [&](Quad<GSU> r) {
      // The quad's A operands first: eight LDS reads in flight together.
      u32x4 ah[4], al[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t off = (uint32_t)a_slot<M>(4 * (4 * cs + t) + g, m_c) * 16u;
        ah[t] = *reinterpret_cast<const u32x4*>(hi_bytes + off) & a_mask;
        al[t] = *reinterpret_cast<const u32x4*>(lo_bytes + off) & a_mask;
      }
      transpose4x4(r.q);
      const uint32_t words[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
      const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
      f32x4_t d4 = z4;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = quad_group_offset<GSU>(t, cuig, gsu);
        const uint32_t zi = (uint32_t)bitsf(r.z.get(j));
        const half2_t zh = as_half2(zi | (zi << 16));
        u32x4 bw;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          bw[v] = __builtin_bit_cast(uint32_t, as_half2((words[t] >> (4 * v)) & 0x000F000Fu) - zh);
        const half8_t b = __builtin_bit_cast(half8_t, bw);
        // Units of one group accumulate in the matrix core; the group's
        // scale is applied once its last unit of the quad is in.
        const bool first = GSU == 0 || GSU == 1 || (GSU == 2 && (t & 1) == 0) || (GSU == 4 && t == 0);
        const bool last = GSU == 0 || GSU == 1 || (GSU == 2 && (t & 1) == 1) || (GSU == 4 && t == 3);
        d4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ah[t]), b, first ? z4 : d4, 0, 0, 0);
        d4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, al[t]), b, d4, 0, 0, 0);
        if (last) {
          const float sv = bitsf(r.s.get(j));
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc[rr] = fmaf(sv, d4[rr], acc[rr]);
        }
      }
      ++cs;
      const int t4 = cuig + 4;
      cuig = t4 - gsu * ((t4 >= gsu ? 1 : 0) + (t4 >= 2 * gsu ? 1 : 0) + (t4 >= 3 * gsu ? 1 : 0) +
                         (t4 >= 4 * gsu ? 1 : 0));
    };

    // Ring of kMfmaDepth + 1 quads; every load is unconditional.
    static_assert(kMfmaDepth == 5, "the ring below holds six quads");
    Quad<GSU> r0, r1, r2, r3, r4, r5;
    load(r0);
    load(r1);
    load(r2);
    load(r3);
    load(r4);
    while (true) {
      load(r5);
      __builtin_amdgcn_sched_barrier(0);
      compute(r0);
      if (cs >= S) break;
      load(r0);
      __builtin_amdgcn_sched_barrier(0);
      compute(r1);
      if (cs >= S) break;
      load(r1);
      __builtin_amdgcn_sched_barrier(0);
      compute(r2);
      if (cs >= S) break;
      load(r2);
      __builtin_amdgcn_sched_barrier(0);
      compute(r3);
      if (cs >= S) break;
      load(r3);
      __builtin_amdgcn_sched_barrier(0);
      compute(r4);
      if (cs >= S) break;
      load(r4);
      __builtin_amdgcn_sched_barrier(0);
      compute(r5);
      if (cs >= S) break;
    }

    if (col_l < ncols) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int m = 4 * g + rr;
        if (m < M) a.out[0][(int64_t)m * a.N + col0 + col_l] = acc[rr] * outf[rr];
      }
    }
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
  if constexpr (MODE == kGated) {
    return s.ncol == 1 ? launch_reg<MODE, 1, 1>(a, s, st, occ) : launch_reg<MODE, 1, 2>(a, s, st, occ);
  } else if constexpr (MODE == kPlain) {
    if (a.M == 2)
      return s.ncol == 1 ? launch_reg<MODE, 2, 1>(a, s, st, occ) : launch_reg<MODE, 2, 2>(a, s, st, occ);
    switch (s.ncol) {
      case 1: return launch_reg<MODE, 1, 1>(a, s, st, occ);
      case 2: return launch_reg<MODE, 1, 2>(a, s, st, occ);
      default: return launch_reg<MODE, 1, 4>(a, s, st, occ);
    }
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

template <int M>
hipError_t dispatch_mfma(const GemvArgs& a, const LaunchShape& s, hipStream_t st, int* occ) {
  static std::atomic<bool> raised1{false}, raised2{false}, raised4{false}, raised0{false};
  const int gsu = a.U / a.G;
  if (gsu == 1) return launch_or_query(gemv_mfma_kernel<M, 1>, raised1, a, s, st, occ);
  if (gsu == 2) return launch_or_query(gemv_mfma_kernel<M, 2>, raised2, a, s, st, occ);
  if (gsu % 4 == 0) return launch_or_query(gemv_mfma_kernel<M, 4>, raised4, a, s, st, occ);
  return launch_or_query(gemv_mfma_kernel<M, 0>, raised0, a, s, st, occ);
}

hipError_t dispatch(Mode mode, const GemvArgs& a, const LaunchShape& s, hipStream_t st, int* occ) {
  if (s.variant == kVariantMfma) {
    switch (a.M) {
      case 3: return dispatch_mfma<3>(a, s, st, occ);
      case 4: return dispatch_mfma<4>(a, s, st, occ);
      case 5: return dispatch_mfma<5>(a, s, st, occ);
      case 6: return dispatch_mfma<6>(a, s, st, occ);
      case 7: return dispatch_mfma<7>(a, s, st, occ);
      default: return dispatch_mfma<8>(a, s, st, occ);
    }
  }
  if (s.variant == kVariantReg) {
    switch (mode) {
      case kSplit4: return dispatch_reg<kSplit4>(a, s, st, occ);
      case kGated: return dispatch_reg<kGated>(a, s, st, occ);
      case kNorm: return dispatch_reg<kNorm>(a, s, st, occ);
      default: return dispatch_reg<kPlain>(a, s, st, occ);
    }
  }
  switch (mode) {
    case kSplit4: return launch_lds<kSplit4, 1, 1>(a, s, st, occ);
    case kGated: return launch_lds<kGated, 1, 1>(a, s, st, occ);
    case kNorm: return launch_lds<kNorm, 1, 1>(a, s, st, occ);
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
    if (mode == kGated) return 2;
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
