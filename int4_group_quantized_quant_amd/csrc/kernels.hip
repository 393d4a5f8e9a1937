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
//    power-of-two scalings.  The zero point, as an fp16 subnormal pair, is
//    subtracted from each pair of masked codes with one packed fp16
//    subtraction (exact), so each product is x * (code - zero) with one
//    rounding, as the definition (code - zero) * scale gives it.  Per 32
//    weights: 4 shifts, 16 AND, 16 packed subtractions, 32 mixed FMAs and
//    one multiply by the group's scale.
//  * Cross-lane sums are butterflies in the fixed order xor 32, xor 16 (lane
//    swaps across wave halves / row pairs), then xor 8, 4, 2, 1 (DPP row
//    rotations).  Several values are reduced at once by pairing them in the
//    swap steps; every value still sees exactly the single-value tree.
//
// gemv_reg_kernel (one lane, K <= 16384; every fused variant): K is cut into nch chunks
// of at most 64 units.  A block holds P rows of nch waves (about 8 waves);
// the block stages the activations once in LDS, then wave (p, c) keeps the
// inputs of chunk c in registers, streams the columns of row p NCOL at a
// time with the loads one step ahead, and writes one partial per (column,
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
// gemv_slice_kernel (two to eight lanes; slice.hip): the matrix cores, with
// K sliced over the waves of a block.
#include "device_common.h"

namespace int4gemv {
namespace {

// ------------------------------------------------------------ reductions

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

// The zero point of a group as the fp16 subnormal pair (zero * 2^-24,
// 16 * zero * 2^-24).  Zero points are integers in [0, 15], so the
// conversion is exact.
__device__ __forceinline__ uint32_t zero_pair(float zero) { return (uint32_t)zero * 0x00100001u; }

// The dequantized codes (code - zero) of the 32 inputs of one unit as 16
// fp16 pairs.  A nibble masked in place into an fp16 half is the exact
// subnormal code * 2^-24 (bits 0-3 of the half) or 16 * code * 2^-24 (bits
// 4-7).  Word i gives the pairs (c0, 16 c5), (16 c1, c4), (c2, 16 c7) and
// (16 c3, c6) of its inputs 8i..8i+7, so one zero pair (z, 16 z) and its
// half swap (taken for free by the packed subtraction) serve all four; one
// packed fp16 subtraction per pair is exact (integers times 2^-24 below
// 2^-14), as the definition (code - zero) * scale asks.  Even inputs come
// out scaled by 2^-24 and odd ones by 2^-20.
__device__ __forceinline__ void unit_codes(u32x4 w, uint32_t zh, half2_t (&d)[16]) {
  const half2_t za = as_half2(zh);
  const half2_t zb = __builtin_shufflevector(za, za, 1, 0);
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = words[i];
    const uint32_t hi = words[i] >> 8;
    d[4 * i + 0] = as_half2(lo & 0x00F0000Fu) - za;
    d[4 * i + 1] = as_half2(lo & 0x000F00F0u) - zb;
    d[4 * i + 2] = as_half2(hi & 0x00F0000Fu) - za;
    d[4 * i + 3] = as_half2(hi & 0x000F00F0u) - zb;
  }
}

// sum_k x[k] * (code_k - zero) over one unit (x pre-scaled), accumulated k
// ascending with one rounding per product: every product is of an fp32
// activation and an exact small integer, so the only errors are the 32
// roundings of the running sum.
__device__ __forceinline__ float unit_dot(const float (&x)[32], const half2_t (&d)[16]) {
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t = fmaf(x[8 * i + 0], (float)d[4 * i + 0].x, t);
    t = fmaf(x[8 * i + 1], (float)d[4 * i + 1].x, t);
    t = fmaf(x[8 * i + 2], (float)d[4 * i + 2].x, t);
    t = fmaf(x[8 * i + 3], (float)d[4 * i + 3].x, t);
    t = fmaf(x[8 * i + 4], (float)d[4 * i + 1].y, t);
    t = fmaf(x[8 * i + 5], (float)d[4 * i + 0].y, t);
    t = fmaf(x[8 * i + 6], (float)d[4 * i + 3].y, t);
    t = fmaf(x[8 * i + 7], (float)d[4 * i + 2].y, t);
  }
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
    // Wave-uniform by contract; stated so that the offset is a scalar operand
    // and never a per-lane loop over the distinct values.
    const uint32_t col = __builtin_amdgcn_readfirstlane(col0 < last ? col0 : last);
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
  for (int i = threadIdx.x; i < n4; i += a.block_threads) {
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
  const int nw = a.block_threads >> 6;
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
  for (int i = threadIdx.x; i < (a.K >> 2); i += a.block_threads) {
    float4 r, x;
    norm_in4(a, i, r, x);
    if (res) res[i] = r;
    if (nrm) nrm[i] = make_float4(x.x * inv, x.y * inv, x.z * inv, x.w * inv);
  }
}

template <int MODE>
__device__ __forceinline__ float4 gated_in4(const GemvArgs& a, int i) {
  return gate4<MODE>(reinterpret_cast<const float4*>(a.x)[i], reinterpret_cast<const float4*>(a.x2)[i]);
}

// Column epilogue shared by both kernels: `tot[st][m]` are the finished sums
// of column `col` (stream st: 0 = the weights / gate / first projection,
// 1 = up / second projection).  `inv` is inv_rms for the norm modes and
// unused otherwise.
template <int M, int MODE, bool kPublish = false>
__device__ __forceinline__ void store_column(const GemvArgs& a, int64_t col,
                                             const float (&tot)[mode_streams(MODE)][M],
                                             float inv) {
  static_assert(!kPublish || MODE == kGated, "only the gated pass publishes its outputs");
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
  } else if constexpr (kPublish) {
    // Stored at device scope: read back by other blocks of the same launch.
    __hip_atomic_store(a.out[0] + col, silu_f32(tot[0][0]) * tot[1][0], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  } else {
    a.out[0][col] = silu_f32(tot[0][0]) * tot[1][0];
  }
}

// ------------------------------------------------------------ register kernel


// The activations of a pass are ready when it starts (a kernel's own inputs).
struct InputsReady {
  __device__ void operator()() const {}
};

// One pass of the register kernel over its columns.  `part` is the block's
// LDS: [cols of the block][NSTREAM][M][nch] partials, 16 floats of per-wave
// sums, 8 column-group counters (one per chunk), then the staged
// activations (x_lds_offset).  The block may hold more waves than the pass's
// P rows of nch waves; the extra waves own no columns.
//
// Activations: the block loads its rows coalesced into registers, issues
// the first step of weight loads behind them, then writes the rows to LDS
// (for the norm, x = (a_a + a_b) * w_norm and block 0 writes residual_out;
// for a gated input, the gated vector); after one barrier each lane keeps
// its unit's 32 inputs in registers for the sweep.  `inputs_ready` is called
// by every thread before the activations are loaded: with InputsReady they
// are a kernel input; otherwise the first step of weight loads is issued
// before the call, so that they stream while it waits, and the activations
// (written by other blocks of the launch) are read at device scope.
//
// Columns: the block owns [blk_begin, blk_end), in groups of NCOL.  The P
// waves of chunk c share that chunk's column groups: wave p starts with
// group p and then claims the next free group from the chunk's LDS counter,
// two groups ahead, so the waves of a chunk finish together whatever order
// the SIMDs run them in.  A (column, chunk) partial does not depend on which
// wave computes it, so the results do not depend on the claiming order.
// kPublish stores the outputs at device scope.
template <int M, int NCOL, int MODE, bool kPublish, class Ready>
__device__ __forceinline__ void reg_pass(const GemvArgs& a, float* part, Ready inputs_ready) {
  constexpr int NSTREAM = mode_streams(MODE);
  constexpr int NSLOT = NCOL * NSTREAM;
  constexpr int V = M * NSLOT;
  constexpr int NZ = (V + 3) / 4;
  constexpr bool kWaits = !__is_same(Ready, InputsReady);
  static_assert(M == 1, "the register kernel runs one lane");

  const int bd = a.block_threads;  // threads per block, from the arguments
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_int(threadIdx.x >> 6);
  const int nch = a.nch;
  const int P = a.rows_per_block;
  const int p = wave / nch;
  const int c = wave - p * nch;
  const int64_t R = (int64_t)gridDim.x * P;
  const int64_t blk_begin = uniform_i64((int64_t)blockIdx.x * P * a.N / R);
  const int64_t blk_end = uniform_i64(((int64_t)blockIdx.x * P + P) * a.N / R);
  const int ncols = (int)(blk_end - blk_begin);
  const int ngroups = (ncols + NCOL - 1) / NCOL;
  const int u = c * a.cw + lane;
  const bool active = lane < a.cw && u < a.U;
  const uint32_t qoff = (uint32_t)(active ? u : 0) * 16u;
  const uint32_t soff = (uint32_t)(active ? unit_group(a, u) : 0) * 4u;
  float* scratch = part + a.part_floats;
  uint32_t* claims = reinterpret_cast<uint32_t*>(scratch + 16);
  float4* xl = reinterpret_cast<float4*>(part + x_lds_offset(a.part_floats));
  const int xs = x_plane_stride(a.U);  // float4s between staging planes
  const int n4 = a.K >> 2;

  // The block's weight streams (scalar buffer resources from its first
  // column, so every offset is 32-bit).  Every load is unconditional: a
  // group past the block's last column re-reads that column (its result is
  // never stored), and a block without columns has an empty range, whose
  // loads return 0 without touching memory.
  const StreamBufs bufs = make_stream_bufs<NSTREAM>(a, blk_begin, blk_end);
  const uint32_t last = ncols > 0 ? (uint32_t)(ncols - 1) : 0u;
  // One step of loads in flight ahead of the arithmetic: two or three
  // measured slower on every call shape (more requests outstanding per CU
  // only add contention for the memory pipeline).
  Step<NSLOT> s0, s1;
  const int g_first = p < P ? p : ngroups;  // waves past the P rows own nothing
  if (threadIdx.x < (unsigned)nch) claims[threadIdx.x] = (uint32_t)P;

  // Activation float4 i = threadIdx.x + j * bd of a row, for j < nper (at
  // most 8: the planner keeps K <= 16384 and blocks of at least 64 * nch
  // threads).
  const int nper = (n4 + bd - 1) / bd;
  auto row_rsrc = [&](const float* src) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, a.K * 4, kBufferWord3);
  };
  auto ld4 = [&](__amdgpu_buffer_rsrc_t r, int j) {
    return __builtin_bit_cast(
        float4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(threadIdx.x + j * bd) * 16u, 0, 0));
  };
  auto put_lds = [&](int j, float4 v) {
    const int i = (int)threadIdx.x + j * bd;
    if (i < n4) xl[(i & 7) * xs + (i >> 3)] = v;
  };
  constexpr int kStageMax = 8;
  if constexpr (kWaits) {
    load_units<NCOL, NSTREAM>(a, bufs, (uint32_t)(g_first * NCOL), last, qoff, soff, s0);
    inputs_ready();
    const auto rx = row_rsrc(a.x);
    for (int i = threadIdx.x; i < n4; i += bd)
      xl[(i & 7) * xs + (i >> 3)] = __builtin_bit_cast(
          float4, __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)i * 16u, 0, kLoadDeviceCoherent));
  } else if constexpr (mode_has_norm(MODE)) {
    const auto ra = row_rsrc(a.x), rb = row_rsrc(a.x2), rg = row_rsrc(a.w_norm);
    float4 va[kStageMax], vb[kStageMax], vg[kStageMax];
#pragma unroll
    for (int j = 0; j < kStageMax; ++j)
      if (j < nper) {
        va[j] = ld4(ra, j);
        vb[j] = ld4(rb, j);
        vg[j] = ld4(rg, j);
      }
    __builtin_amdgcn_sched_barrier(0);
    load_units<NCOL, NSTREAM>(a, bufs, (uint32_t)(g_first * NCOL), last, qoff, soff, s0);
    __builtin_amdgcn_sched_barrier(0);
    // Per-thread share of sum_k r_k^2 (its float4s in order), then the
    // wave's total in its slot.
    float ssq = 0.0f;
#pragma unroll
    for (int j = 0; j < kStageMax; ++j)
      if (j < nper) {
        const int i = (int)threadIdx.x + j * bd;
        if (i < n4) {
          const float4 r = make_float4(va[j].x + vb[j].x, va[j].y + vb[j].y, va[j].z + vb[j].z, va[j].w + vb[j].w);
          ssq = fmaf(r.x, r.x, ssq);
          ssq = fmaf(r.y, r.y, ssq);
          ssq = fmaf(r.z, r.z, ssq);
          ssq = fmaf(r.w, r.w, ssq);
          if (blockIdx.x == 0 && a.residual_out) reinterpret_cast<float4*>(a.residual_out)[i] = r;
          xl[(i & 7) * xs + (i >> 3)] =
              make_float4(r.x * vg[j].x, r.y * vg[j].y, r.z * vg[j].z, r.w * vg[j].w);
        }
      }
    const float wsum = wave_sum(ssq);
    if (lane == 0) scratch[wave] = wsum;
  } else if constexpr (mode_gates_input(MODE)) {
    const auto rp = row_rsrc(a.x), rr = row_rsrc(a.x2);
    float4 vp[kStageMax], vr[kStageMax];
#pragma unroll
    for (int j = 0; j < kStageMax; ++j)
      if (j < nper) {
        vp[j] = ld4(rp, j);
        vr[j] = ld4(rr, j);
      }
    __builtin_amdgcn_sched_barrier(0);
    load_units<NCOL, NSTREAM>(a, bufs, (uint32_t)(g_first * NCOL), last, qoff, soff, s0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kStageMax; ++j)
      if (j < nper) put_lds(j, gate4<MODE>(vp[j], vr[j]));
  } else {
    const auto rx = row_rsrc(a.x);
    float4 v[kStageMax];
#pragma unroll
    for (int j = 0; j < kStageMax; ++j)
      if (j < nper) v[j] = ld4(rx, j);
    __builtin_amdgcn_sched_barrier(0);
    load_units<NCOL, NSTREAM>(a, bufs, (uint32_t)(g_first * NCOL), last, qoff, soff, s0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kStageMax; ++j)
      if (j < nper) put_lds(j, v[j]);
  }
  __syncthreads();
  float x[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) put4(x, j, active ? xl[j * xs + u] : make_float4(0.f, 0.f, 0.f, 0.f));

  const bool writer = V >= 4 ? (lane & 15) == 0 : (V == 2 ? (lane & 31) == 0 : lane == 0);
  // Compute the group starting at block column n0 from the loaded step r.
  auto step = [&](int n0, const Step<NSLOT>& r) {
    float vals[V];
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) {
      half2_t d[16];
      unit_codes(r.q[sl], zero_pair(r.z[sl]), d);
      vals[sl] = r.s[sl] * unit_dot(x, d);
    }
    float z[NZ];
    wave_reduce<V>(vals, z);
    if (writer) {
      const int rrow = lane >> 4;
#pragma unroll
      for (int j = 0; j < NZ; ++j) {
        const int vi = reduced_index<V>(j, rrow);
        const int col = n0 + vi / NSTREAM;
        if (col < ncols) part[((col * NSTREAM + vi % NSTREAM) * M) * nch + c] = z[j];
      }
    }
  };
  // The next free group of this wave's chunk, claimed by lane 0 from the
  // chunk's LDS counter with one increment (ds_inc_rtn, which the compiler
  // keeps as a single-lane atomic).  It is read out (wave-uniform) only
  // where the next loads need it, one step later, so the atomic's latency
  // hides behind that step.
  auto claim = [&]() -> uint32_t {
    uint32_t g = 0;
    if (lane == 0) g = __builtin_amdgcn_atomic_inc32(claims + c, 0xFFFFFFFFu, __ATOMIC_RELAXED, "workgroup");
    return g;
  };
  // The empty asm takes the claimed value as an operand at this point, after
  // the step's stores, so the compiler cannot move the read-out (and its wait
  // for the atomic) up into the step.
  auto group = [](uint32_t claimed) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" : "+v"(claimed));
    return (int)__builtin_amdgcn_readfirstlane(claimed);
  };

  // Pipeline: s0 holds the loads of group g; the loads of the next group are
  // issued before g is computed, and the group after it is claimed
  // meanwhile.
  if (g_first < ngroups) {
    int g = g_first;
    uint32_t next = claim();
    while (true) {
      const int g1 = group(next);
      load_units<NCOL, NSTREAM>(a, bufs, (uint32_t)(g1 * NCOL), last, qoff, soff, s1);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the arithmetic
      next = claim();
      step(g * NCOL, s0);
      if (g1 >= ngroups) break;
      g = g1;
      const int g2 = group(next);
      load_units<NCOL, NSTREAM>(a, bufs, (uint32_t)(g2 * NCOL), last, qoff, soff, s0);
      __builtin_amdgcn_sched_barrier(0);
      next = claim();
      step(g * NCOL, s1);
      if (g2 >= ngroups) break;
      g = g2;
    }
  }
  __syncthreads();

  // inv_rms = 1 / sqrt(sum_k r_k^2 / K + eps) ([P4] WGSL_NORM_MATVEC_INT4),
  // from the wave totals in wave order: the same value in every block.
  // Block 0 writes norm_out = x * inv_rms from the staged x.
  float inv = 1.0f;
  if constexpr (mode_has_norm(MODE)) {
    float ss = scratch[0];
    for (int w = 1; w < (bd >> 6); ++w) ss += scratch[w];
    inv = 1.0f / sqrtf(ss / (float)a.K + a.eps);
    if (blockIdx.x == 0 && a.norm_out) {
      for (int i = threadIdx.x; i < n4; i += bd) {
        const float4 v = xl[(i & 7) * xs + (i >> 3)];
        reinterpret_cast<float4*>(a.norm_out)[i] = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
      }
    }
  }

  // Each column's chunk partials, summed in chunk order.
  for (int j = threadIdx.x; j < ncols; j += bd) {
    float tot[NSTREAM][M];
#pragma unroll
    for (int st = 0; st < NSTREAM; ++st) {
      const float* pp = part + (j * NSTREAM + st) * M * nch;
      float sum = pp[0];
      for (int cc = 1; cc < nch; ++cc) sum += pp[cc];
      tot[st][0] = sum;
    }
    store_column<M, MODE, kPublish>(a, blk_begin + j, tot, inv);
  }
}

template <int M, int NCOL, int MODE>
__global__ __launch_bounds__(512) void gemv_reg_kernel(GemvArgs a) {
  extern __shared__ float part[];
  reg_pass<M, NCOL, MODE, false>(a, part, InputsReady{});
}

// ------------------------------------------------------------ fused MLP

// Polls before a block stops waiting for the others (about a second): a
// grid whose blocks are not all resident at once must not hang the device.
constexpr uint32_t kGridWaitPolls = 1u << 20;

// The fused MLP's workspace, 32-bit words: [0] the call count (epoch),
// [1] the timeout flag, [kMlpFlags + b] the epoch block b last published.
constexpr int kMlpFlags = 32;
static_assert(kMlpWorkspaceBytes / 4 - kMlpFlags == kMlpMaxBlocks, "one flag per block");

// Waits until every block of the grid has published this call's epoch in
// its flag.  The flags and the activations behind them were stored at
// device scope, and the activations stores completed before each flag was
// written; the waiting pass reads them at device scope, so no cache
// maintenance is needed.  Wave 0 polls all flags at once; on a timeout it
// records the failure in word 1 and goes on.
struct GridWait {
  uint32_t* ws;
  uint32_t epoch;
  __device__ void operator()() const {
    if (threadIdx.x < 64) {
      const uint32_t* flags = ws + kMlpFlags;
      const int nb = (int)gridDim.x;
      for (uint32_t polls = 0;; ++polls) {
        bool done = true;
        for (int b0 = 4 * (int)threadIdx.x; b0 < nb; b0 += 256) {
          // Four loads in flight at once (indices past the grid re-read the
          // last flag).
          uint32_t f[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            f[j] = __hip_atomic_load(flags + (b0 + j < nb ? b0 + j : nb - 1), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
          for (int j = 0; j < 4; ++j) done &= f[j] == epoch;
        }
        if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
        if (polls == kGridWaitPolls) {
          if (threadIdx.x == 0) __hip_atomic_store(ws + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
  }
};

// h = silu(x Wg^T) * (x Wu^T), then y = h Wd^T, in one persistent grid:
// every block runs its columns of the gated pass, stores them at device
// scope, waits for those stores to complete and publishes the call's epoch
// in its flag; its first step of down-projection weights is loaded while it
// waits for every flag, and the down pass then stages the whole of h.
// Block 0 advances the stored epoch once it has seen every flag (by then
// every block has read it), unless a wait has timed out.  No
// read-modify-write: all blocks' atomics on one word would be serialized at
// the memory.  Once the timeout flag is set (by this call's or an earlier
// call's wait), a call only writes NaN to h and y, and leaves the
// workspace as it is.
template <int NCOL1, int NCOL2>
__global__ __launch_bounds__(512) void mlp_reg_kernel(GemvArgs gate_up, GemvArgs down, uint32_t* ws) {
  extern __shared__ float part[];
  __shared__ uint32_t stuck;
  // Wave 0 publishes and polls; it alone needs the epoch.  The timeout word
  // is loaded with it at the start but examined only after the gated pass,
  // so the pass does not wait for the load.
  uint32_t epoch = 0, stuck_word = 0;
  if (threadIdx.x < 64) {
    epoch = __hip_atomic_load(ws, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    stuck_word = __hip_atomic_load(ws + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  reg_pass<1, NCOL1, kGated, true>(gate_up, part, InputsReady{});
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores of h have completed
  if (threadIdx.x == 0) stuck = stuck_word;
  __syncthreads();
  if (stuck != 0u) {
    // A wait timed out in an earlier call: no waiting; this block's own
    // columns of h and of y (the two passes' static column ranges) become
    // NaN.
    const float nan = __builtin_nanf("");
    for (const GemvArgs* a : {&gate_up, &down}) {
      const int64_t R = (int64_t)gridDim.x * a->rows_per_block;
      const int64_t b0 = (int64_t)blockIdx.x * a->rows_per_block * a->N / R;
      const int64_t b1 = ((int64_t)blockIdx.x * a->rows_per_block + a->rows_per_block) * a->N / R;
      for (int64_t i = b0 + threadIdx.x; i < b1; i += blockDim.x) a->out[0][i] = nan;
    }
    return;
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(ws + kMlpFlags + blockIdx.x, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  reg_pass<1, NCOL2, kPlain, false>(down, part, GridWait{ws, epoch});
  if (blockIdx.x == 0 && threadIdx.x == 0 && __hip_atomic_load(ws + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u)
    __hip_atomic_store(ws, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ LDS kernel

// Activation row m is stored as float4 xl[m][j][u] = inputs 32u+4j .. 32u+4j+3,
// pre-scaled like the register kernel's activations (prescale4).
template <int M>
__device__ __forceinline__ void stage_x(const float* __restrict__ X, int K, int U, int bd, float4* xl) {
  const int n4 = K >> 2;
  for (int m = 0; m < M; ++m) {
    const float4* src = reinterpret_cast<const float4*>(X + (size_t)m * K);
    for (int i = threadIdx.x; i < n4; i += bd)
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
    for (int i = threadIdx.x; i < (a.K >> 2); i += a.block_threads) {
      float4 r, v;
      norm_in4(a, i, r, v);
      xl[(i & 7) * a.U + (i >> 3)] = prescale4(v);
    }
    write_norm_outputs(a, inv);
  } else if constexpr (mode_gates_input(MODE)) {
    for (int i = threadIdx.x; i < (a.K >> 2); i += a.block_threads)
      xl[(i & 7) * a.U + (i >> 3)] = prescale4(gated_in4<MODE>(a, i));
  } else {
    stage_x<M>(a.x, a.K, a.U, a.block_threads, xl);
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform_int(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * (a.block_threads >> 6) + wave;
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
    for (int sl = 0; sl < NSLOT; ++sl) unit_codes(r.q[sl], zero_pair(r.z[sl]), d[sl]);
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
#pragma unroll
      for (int sl = 0; sl < NSLOT; ++sl) vals[m * NSLOT + sl] = r.s[sl] * unit_dot(x, d[sl]);
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

// Threads per block of the embedding gather and the quantizers, a constant
// in the kernels as well: blockDim.x would cost a load of the dispatch
// packet before the first index is known.
constexpr int kSmallBlock = 256;

// out[t][k] = (code - zero) * scale of row ids[t] of a table stored like the
// weight columns ([P1] EmbeddingInt4 and the per-layer-embedding row gather).
// One lane per 32-bit code word: a 4-byte load, eight values, two 16-byte
// stores, so a wave reads 256 contiguous bytes and writes 2 KiB.  The value
// is rounded once, as the definition states.  Ids outside [0, N) write zeros.
__global__ __launch_bounds__(kSmallBlock) void embedding_gather_kernel(const int32_t* __restrict__ ids, int64_t T,
                                                               const uint32_t* __restrict__ q,
                                                               const float* __restrict__ scales,
                                                               const float* __restrict__ zeros, int64_t N,
                                                               int32_t K, int32_t gs, float* __restrict__ out) {
  const int64_t wpr = K >> 3;  // code words per row
  const int64_t total = T * wpr;
  const int64_t stride = (int64_t)gridDim.x * kSmallBlock;
  for (int64_t i = (int64_t)blockIdx.x * kSmallBlock + threadIdx.x; i < total; i += stride) {
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
// Each wave handles R consecutive batches of 64 / TPG groups; the next
// batch's loads are issued before the current batch is quantized, so a wave
// keeps two batches of inputs in flight.
template <int WPT, int R>
__global__ __launch_bounds__(kSmallBlock) void quantize_pack_wave_kernel(const float* __restrict__ W,
                                                                 int64_t total_groups, int gs, int tpg,
                                                                 uint32_t* __restrict__ q,
                                                                 float* __restrict__ scales,
                                                                 float* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int gpw = 64 / tpg;  // groups per wave and batch
  const int64_t wave_id = (int64_t)blockIdx.x * (kSmallBlock >> 6) + (threadIdx.x >> 6);
  const int64_t grp0 = wave_id * gpw * R + lane / tpg;
  const int part = lane & (tpg - 1);
  const int wpg = gs >> 3;

  // The batch's inputs: words part + j * tpg of the lane's group (a dead
  // group reads group 0 and is never stored).
  auto load = [&](int64_t grp, float (&v)[WPT][8]) {
    const float* wg = W + (grp < total_groups ? grp : 0) * gs;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int wi = part + j * tpg;
      const int wc = wi < wpg ? wi : 0;
      const float4 a0 = reinterpret_cast<const float4*>(wg)[2 * wc];
      const float4 a1 = reinterpret_cast<const float4*>(wg)[2 * wc + 1];
      v[j][0] = a0.x; v[j][1] = a0.y; v[j][2] = a0.z; v[j][3] = a0.w;
      v[j][4] = a1.x; v[j][5] = a1.y; v[j][6] = a1.z; v[j][7] = a1.w;
    }
  };
  auto quantize = [&](int64_t grp, const float (&v)[WPT][8]) {
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      if (part + j * tpg < wpg) {
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
  };

  float va[WPT][8], vb[WPT][8];
  load(grp0, va);
#pragma unroll
  for (int r = 0; r < R; r += 2) {
    const int64_t ga = grp0 + (int64_t)r * gpw, gb = ga + gpw;
    if (r + 1 < R) load(gb, vb);
    if (ga >= total_groups) return;  // later batches of this lane's group are dead too
    quantize(ga, va);
    if (r + 1 >= R) break;
    if (r + 2 < R) load(gb + gpw, va);
    if (gb >= total_groups) return;
    quantize(gb, vb);
  }
}

__global__ __launch_bounds__(kSmallBlock) void quantize_pack_kernel(const float* __restrict__ W,
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

template <int MODE, int M, int NCOL>
hipError_t launch_reg(const GemvArgs& a, const LaunchShape& s, hipStream_t stream, int* occupancy) {
  static std::atomic<bool> raised{false};
  if (s.depth != 1) return hipErrorInvalidValue;  // one step ahead is the only form built
  // The staging holds at most 8 float4s of a row per thread.
  if ((a.K / 4 + s.block_threads - 1) / s.block_threads > 8) return hipErrorInvalidValue;
  return launch_or_query(gemv_reg_kernel<M, NCOL, MODE>, raised, a, s, stream, occupancy);
}

template <int NCOL1, int NCOL2>
hipError_t launch_mlp_t(const GemvArgs& gate_up, const GemvArgs& down, const LaunchShape& s, uint32_t* ws,
                        hipStream_t stream, int* occupancy) {
  static std::atomic<bool> raised{false};
  const auto kern = mlp_reg_kernel<NCOL1, NCOL2>;
  hipError_t e = raise_lds_once(kern, raised, s);
  if (e != hipSuccess) return e;
  if (occupancy)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(occupancy, kern, s.block_threads, s.lds_bytes);
  GemvArgs g = gate_up, d = down;
  g.block_threads = d.block_threads = s.block_threads;
  hipLaunchKernelGGL(kern, dim3(s.grid), dim3(s.block_threads), s.lds_bytes, stream, g, d, ws);
  return hipGetLastError();
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
    // Measured per mode: two weight streams step one column at a time, the
    // routed split4 call two, the other one-lane calls four.
    if (mode_streams(mode) == 2) return 1;
    if (mode == kSplit4) return 2;
    return M == 1 ? 4 : 2;
  }
  return mode == kPlain ? 2 : 1;
}

hipError_t launch_mlp(const GemvArgs& gate_up, int ncol_gate_up, const GemvArgs& down, int ncol_down,
                      const LaunchShape& s, uint32_t* ws, hipStream_t stream, int* occupancy) {
  if (s.depth != 1) return hipErrorInvalidValue;
  const bool g2 = ncol_gate_up != 1;
  switch (ncol_down) {
    case 1: return g2 ? launch_mlp_t<2, 1>(gate_up, down, s, ws, stream, occupancy)
                      : launch_mlp_t<1, 1>(gate_up, down, s, ws, stream, occupancy);
    case 2: return g2 ? launch_mlp_t<2, 2>(gate_up, down, s, ws, stream, occupancy)
                      : launch_mlp_t<1, 2>(gate_up, down, s, ws, stream, occupancy);
    default: return g2 ? launch_mlp_t<2, 4>(gate_up, down, s, ws, stream, occupancy)
                       : launch_mlp_t<1, 4>(gate_up, down, s, ws, stream, occupancy);
  }
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
  int64_t grid = (total + kSmallBlock - 1) / kSmallBlock;
  if (grid > 65536) grid = 65536;  // grid-stride beyond this
  hipLaunchKernelGGL(embedding_gather_kernel, dim3((unsigned)grid), dim3(kSmallBlock), 0, stream, ids, T, q,
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
    constexpr int R = 4;  // batches per wave
    const int64_t groups_per_block = 4 * (64 / tpg) * R;
    const int64_t grid = (total_groups + groups_per_block - 1) / groups_per_block;
    if (wpt == 1)
      hipLaunchKernelGGL((quantize_pack_wave_kernel<1, R>), dim3((unsigned)grid), dim3(kSmallBlock), 0, stream, W, total_groups, gs, tpg, q, scales, zeros);
    else if (wpt == 2)
      hipLaunchKernelGGL((quantize_pack_wave_kernel<2, R>), dim3((unsigned)grid), dim3(kSmallBlock), 0, stream, W, total_groups, gs, tpg, q, scales, zeros);
    else if (wpt <= 4)
      hipLaunchKernelGGL((quantize_pack_wave_kernel<4, R>), dim3((unsigned)grid), dim3(kSmallBlock), 0, stream, W, total_groups, gs, tpg, q, scales, zeros);
    else
      hipLaunchKernelGGL((quantize_pack_wave_kernel<8, R>), dim3((unsigned)grid), dim3(kSmallBlock), 0, stream, W, total_groups, gs, tpg, q, scales, zeros);
    return hipGetLastError();
  }
  const int tpg = wpg < 256 ? wpg : 256;
  const int gpb = 256 / tpg < 64 ? 256 / tpg : 64;
  const int64_t grid = (total_groups + gpb - 1) / gpb;
  hipLaunchKernelGGL(quantize_pack_kernel, dim3((unsigned)grid), dim3(kSmallBlock), 0, stream, W,
                     total_groups, gs, tpg, gpb, q, scales, zeros);
  return hipGetLastError();
}

}  // namespace int4gemv
