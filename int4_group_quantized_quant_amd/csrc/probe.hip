// probe.hip -- a plain streaming read of one device buffer, the measured
// ceiling that the matvec kernels' effective bandwidth is set against: no
// arithmetic beyond an XOR of every 32-bit word read, so its rate is what one
// launch can pull from HBM at a given size.  Not part of the method.
//
// Each block (persistent grid, `waves` waves per block) reads one contiguous
// slice of the buffer; each lane loads 16-byte units with buffer loads
// marked for streaming, UNROLL of them in flight, and XORs every word into
// its checksum.  The block's checksum goes to sink[block].
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "int4gemv.h"

namespace int4gemv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit dwords
constexpr int kNonTemporal = 2;

template <int UNROLL>
__global__ __launch_bounds__(1024) void stream_read_kernel(const unsigned char* buf, uint64_t units,
                                                           uint32_t* sink, int block_threads) {
  const uint64_t b = blockIdx.x, nb = gridDim.x;
  const uint64_t u0 = b * units / nb, u1 = (b + 1) * units / nb;
  const uint64_t n = u1 - u0;  // < 2^27 units (2 GiB) per block
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(buf + u0 * 16), (short)0,
                                                      (int)(n * 16 < 0x7FFFFFFFull ? n * 16 : 0x7FFFFFFFull),
                                                      kBufWord3);
  uint32_t acc = 0;
  const uint32_t step = (uint32_t)block_threads * UNROLL;
  for (uint32_t i = threadIdx.x; i < (uint32_t)n; i += step) {
    u32x4 v[UNROLL];
    // Units past the slice read 0 from the buffer resource's range check.
#pragma unroll
    for (int j = 0; j < UNROLL; ++j)
      v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rsrc, (i + (uint32_t)j * block_threads) * 16u, 0, kNonTemporal));
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // Block XOR: wave shuffles, then one word per wave in LDS.
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  __shared__ uint32_t part[16];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < block_threads / 64; ++w) t ^= part[w];
    sink[b] = t;
  }
}

}  // namespace
}  // namespace int4gemv

using namespace int4gemv;

extern "C" int int4_probe_stream_read(const void* buf, size_t bytes, int32_t blocks, int32_t waves,
                                      int32_t unroll, uint32_t* sink, void* stream) {
  if (!buf || !sink) return INT4_ERR_NULL;
  if (bytes % 16 != 0 || (uintptr_t)buf % 16 != 0 || (uintptr_t)sink % 4 != 0) return INT4_ERR_ALIGN;
  if (blocks < 1 || waves < 1 || waves > 16 ||
      (bytes / 16 + (uint64_t)blocks - 1) / (uint64_t)blocks >= ((uint64_t)1 << 27))
    return INT4_ERR_SHAPE;
  if (unroll != 1 && unroll != 2 && unroll != 4) return INT4_ERR_ARG;
  const int threads = 64 * waves;
  const uint64_t units = bytes / 16;
  hipStream_t st = (hipStream_t)stream;
  const auto* p = static_cast<const unsigned char*>(buf);
  if (unroll == 1)
    hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(threads), 0, st, p, units, sink, threads);
  else if (unroll == 2)
    hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(threads), 0, st, p, units, sink, threads);
  else
    hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(threads), 0, st, p, units, sink, threads);
  return hipGetLastError() == hipSuccess ? INT4_OK : INT4_ERR_HIP;
}
