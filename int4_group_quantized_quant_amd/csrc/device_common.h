// device_common.h -- device helpers shared by the matvec kernels
// (kernels.hip) and the matrix-core lanes kernel (slice.hip): vector types,
// bit casts, wave-uniform moves, lane permutes, the elementwise gates, the
// activation exponent of the split-fp16 operands, buffer-resource constants
// and the launch helpers.  Internal; not part of the public ABI.
#pragma once

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

constexpr int kBufferWord3 = 0x00020000;  // raw buffer, 32-bit dwords (gfx9 family)
constexpr int kLoadNonTemporal = 2;       // cache policy: streamed, no reuse expected
constexpr int kLoadDeviceCoherent = 16;   // cache policy: device scope, coherent across the L2 caches

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
  GemvArgs b = a;
  b.block_threads = s.block_threads;
  hipLaunchKernelGGL(kern, dim3(s.grid), dim3(s.block_threads), s.lds_bytes, stream, b);
  return hipGetLastError();
}

}  // namespace
}  // namespace int4gemv
