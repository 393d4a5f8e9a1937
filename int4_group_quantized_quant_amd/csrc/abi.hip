// abi.hip -- the extern "C" entry points declared in include/int4gemv.h:
// argument validation (pure host logic, done before any HIP call), launch
// geometry, and dispatch to the kernels in kernels.hip.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <array>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "int4gemv.h"
#include "internal.h"

// One copy per device of the allocation-free GEMM's workspace
// (int4_gemm_noalloc), held from the code object's load until the process
// ends.
static __device__ __align__(256) unsigned char scratch[INT4_GEMM_NOALLOC_SCRATCH_BYTES];

namespace int4gemv {
namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = std::string(int4_status_str(status)) + ": " + buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return INT4_OK;
}

// ------------------------------------------------------------------ checks

struct Span {
  const void* p;
  uint64_t bytes;
  const char* name;
};

bool overlaps(const Span& a, const Span& b) {
  if (a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Outputs must not overlap any input or each other.
int check_alias(const Span* ins, int n_in, const Span* outs, int n_out) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(outs[i], ins[j]))
        return fail(INT4_ERR_ALIAS, "output %s overlaps input %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(outs[i], outs[j]))
        return fail(INT4_ERR_ALIAS, "output %s overlaps output %s", outs[i].name, outs[j].name);
  }
  return INT4_OK;
}

int check_align(const void* p, unsigned align, const char* name) {
  if (p != nullptr && ((uintptr_t)p % align) != 0)
    return fail(INT4_ERR_ALIGN, "%s must be %u-byte aligned", name, align);
  return INT4_OK;
}

#define RETURN_IF(expr)          \
  do {                           \
    int _st = (expr);            \
    if (_st != INT4_OK) return _st; \
  } while (0)

// K, group size: the kernels read 32 codes (16 bytes) at a time and a group
// must hold whole 16-byte units ([P4] WGSL_QUAD_MATVEC_INT4 reads vec4u units
// and indexes groups per unit).
int check_kgs(int64_t K, int32_t gs) {
  if (gs < 32 || gs % 32 != 0)
    return fail(INT4_ERR_SHAPE, "group_size must be a positive multiple of 32 (got %d)", (int)gs);
  if (K < gs || K % gs != 0)
    return fail(INT4_ERR_SHAPE, "K must be a positive multiple of group_size (K=%lld, gs=%d)",
                (long long)K, (int)gs);
  if (K > (int64_t)1 << 30)
    return fail(INT4_ERR_SHAPE, "K=%lld is larger than supported", (long long)K);
  return INT4_OK;
}

// ------------------------------------------------------------------ device

struct DeviceInfo {
  int cus = 0;
  size_t lds_block = 0;
  size_t lds_cu = 0;
  bool valid = false;
};

std::mutex g_dev_mu;
std::array<DeviceInfo, 64> g_dev;

int device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= (int)g_dev.size()) return fail(INT4_ERR_HIP, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.valid) {
    int cus = 0, lds_block = 0, lds_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e == hipSuccess)
      e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e != hipSuccess) return fail(INT4_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    d.cus = cus > 0 ? cus : 1;
    d.lds_block = (size_t)lds_block;
    d.lds_cu = lds_cu > 0 ? (size_t)lds_cu : (size_t)lds_block;
    d.valid = true;
  }
  *out = d;
  return INT4_OK;
}

// Blocks per CU for one launch shape, cached: the occupancy query is host
// work that would otherwise run on every call.
int cached_occupancy(Mode mode, const GemvArgs& a, const LaunchShape& s, int* bpc) {
  struct Key {
    int dev, mode, variant, M, ncol, depth, threads;
    size_t lds;
    bool operator<(const Key& o) const {
      return std::tie(dev, mode, variant, M, ncol, depth, threads, lds) <
             std::tie(o.dev, o.mode, o.variant, o.M, o.ncol, o.depth, o.threads, o.lds);
    }
  };
  static std::mutex mu;
  static std::map<Key, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  const Key key{dev, (int)mode, s.variant, a.M, s.ncol, s.depth, s.block_threads, s.lds_bytes};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      *bpc = it->second;
      return INT4_OK;
    }
  }
  int v = 0;
  e = gemv_occupancy(mode, a, s, &v);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
  if (v < 1)
    return fail(INT4_ERR_SHAPE, "kernel does not fit on a CU (%d threads, %zu bytes of LDS)",
                s.block_threads, s.lds_bytes);
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = v;
  *bpc = v;
  return INT4_OK;
}

// Launch geometry.  Both kernels run persistent grids: as many blocks as are
// resident on the device at once, so no block waits for a second round.
//
// Register kernel (M = 1, K <= 16384): nch = ceil(K/2048) chunks of cw units,
// P = 8/nch rows of nch waves per block (about 8 waves: two per SIMD, which
// streams best), the columns split evenly over the blocks (the P waves of a
// chunk share the block's columns), one LDS partial per (column, stream,
// lane, chunk), the activations staged once per block.
//
// Matrix-core kernel (plain, M >= 2): blocks of W <= 8 waves, each wave one
// slice of 16, 20 or 24 units of K per pass, 8 / W blocks per CU, the
// block's tiles of 16 columns in rounds that fit the partial table in LDS.
//
// LDS kernel (larger K for one lane): 256-thread blocks, the activation row
// staged in LDS (K*4 bytes), columns split evenly over the waves.
int plan(Mode mode, GemvArgs& a, LaunchShape* s) {
  DeviceInfo dev;
  RETURN_IF(device_info(&dev));
  const int M = a.M;
  const int64_t N = a.N;
  const int nstream = mode_streams(mode);
  s->lds_max = dev.lds_block;
  const int rows = M;  // activation rows staged per block (M = 1 except plain lanes)
  if (M == 1 && a.nch <= 8) {
    const int nch = a.nch;
    const int P = nch >= 8 ? 1 : 8 / nch;
    auto table = [&](int64_t blocks) {
      return (int64_t)((N + blocks - 1) / blocks) * nstream * M * nch;
    };
    // Partial table, wave slots and the staged activations.
    auto lds_for = [&](int64_t blocks) -> size_t {
      const int64_t t = table(blocks);
      if (t > ((int64_t)1 << 28)) return (size_t)-1;
      return ((size_t)x_lds_offset((int)t) + (size_t)rows * 32 * (size_t)x_plane_stride(a.U)) * sizeof(float);
    };
    if (lds_for(dev.cus) <= dev.lds_block) {
      a.rows_per_block = P;
      s->variant = kVariantReg;
      s->depth = 1;
      s->block_threads = 64 * P * nch;
      int ncol = max_ncol(mode, M, kVariantReg);
      while (ncol > 1 && N / ((int64_t)dev.cus * P) < ncol) ncol /= 2;
      s->ncol = ncol;
      s->lds_bytes = lds_for(dev.cus);
      int bpc = 1;
      RETURN_IF(cached_occupancy(mode, a, *s, &bpc));
      // One block of about 8 waves per CU; more resident waves per CU only
      // add contention for the memory pipeline.
      const int waves_per_block = P * nch;
      if (bpc > 1 && waves_per_block * bpc > 8) bpc = waves_per_block >= 8 ? 1 : 8 / waves_per_block;
      int64_t B = (int64_t)dev.cus * bpc;
      const int64_t max_blocks = (N + P - 1) / P;  // at least one column per row
      if (B > max_blocks) B = max_blocks;
      if (B < 1) B = 1;
      while (s->ncol > 1 && N / (B * P) < s->ncol) s->ncol /= 2;
      if (lds_for(B) <= dev.lds_block) {
        a.part_floats = (int32_t)table(B);
        s->lds_bytes = lds_for(B);
        s->grid = (int)B;
        a.total_waves = B * P * nch;
        return INT4_OK;
      }
    }
    // Too little LDS for the partial table and the activations: the LDS
    // kernel needs only the activations.
  }
  if ((mode == kPlain || mode == kDual || mode == kGated || mode_gates_input(mode)) && M >= 2) {
    // Matrix-core lanes: slices of SU = 16, 20 or 24 units, at most 8 waves
    // (two per SIMD) per block, P passes of the waves over the slices; one
    // block's columns in rounds of RT tiles whose partials fit the LDS.
    const int U = a.U;
    int su = 16;
    int mix24 = 0;
    if (U > kSliceMaxWaves * 16) {
      const int P = (U + kSliceMaxWaves * 24 - 1) / (kSliceMaxWaves * 24);
      const int per_wave = ((U + P - 1) / P + kSliceMaxWaves - 1) / kSliceMaxWaves;
      su = per_wave <= 16 ? 16 : (per_wave <= 20 ? 20 : 24);
      if (P == 1 && su == 20) {
        // One pass of 20-unit slices would split a cache line of every
        // column between two waves; slices of 24 and 16 units (3 and 2
        // lines) cover U instead, every wave holding one:
        // 24 n + 16 (8 - n) >= U, and the last wave starts at 112 + 8 n < U.
        mix24 = (U - kSliceMaxWaves * 16 + 7) / 8;
        su = 24;
      }
    }
    const int cls = slice_class(U / a.G);
    const int nsl = mix24 > 0 ? kSliceMaxWaves : (U + su - 1) / su;
    const int W = nsl < kSliceMaxWaves ? nsl : kSliceMaxWaves;
    const int bpc = kSliceMaxWaves / W;
    const int64_t tiles = (N + 15) / 16;
    // Blocks per weight stream (the dual mode runs one grid half per stream).
    const int nstreams = mode == kDual ? 2 : 1;
    int64_t B = (int64_t)dev.cus * bpc / nstreams;
    if (B > tiles) B = tiles;
    if (B < 1) B = 1;
    int64_t tiles_per_block = ((N + B - 1) / B + 15) / 16;
    const size_t budget = dev.lds_cu / (size_t)bpc < dev.lds_block ? dev.lds_cu / (size_t)bpc : dev.lds_block;
    const int nv = mode == kGated ? 2 : 1;  // both streams of a tile in one block
    const size_t fixed = slice_lds_bytes(su, cls, a.G, W, 0, nv);
    const size_t per_tile = slice_lds_bytes(su, cls, a.G, W, 1, nv) - fixed;
    if (fixed + per_tile > budget)
      return fail(INT4_ERR_SHAPE, "matrix-core lanes need %zu bytes of LDS per block; %zu available",
                  fixed + per_tile, budget);
    int64_t rt = (int64_t)((budget - fixed) / per_tile);
    if (rt < tiles_per_block) {
      // A block runs its tiles in one round: more blocks, of at most 16 * rt
      // columns each, which then take turns on the CUs.
      B = (N + 16 * rt - 1) / (16 * rt);
      tiles_per_block = ((N + B - 1) / B + 15) / 16;
    }
    if (rt > tiles_per_block) rt = tiles_per_block;
    a.rt = (int32_t)rt;
    a.su = su;
    a.mix24 = mix24;
    s->variant = kVariantSlice;
    s->ncol = 16;
    s->depth = 1;
    s->block_threads = 64 * W;
    s->lds_bytes = slice_lds_bytes(su, cls, a.G, W, (int)rt, nv);
    a.g_recip = a.G == 1 ? 0u : (uint32_t)((((uint64_t)1 << 32) + (uint64_t)a.G - 1) / (uint64_t)a.G);
    s->grid = (int)(B * nstreams);
    a.total_waves = B * nstreams * W;
    return INT4_OK;
  }
  const size_t lds = (size_t)rows * (size_t)a.K * sizeof(float) + (mode_has_norm(mode) ? 64 : 0);
  if (lds > dev.lds_block)
    return fail(INT4_ERR_SHAPE, "activations need %zu bytes of LDS per block; the device allows %zu",
                lds, dev.lds_block);
  s->variant = kVariantLds;
  s->block_threads = 256;
  s->lds_bytes = lds;
  int ncol = max_ncol(mode, M, kVariantLds);
  const int64_t target_waves = (int64_t)dev.cus * 16;
  while (ncol > 1 && (N + ncol - 1) / ncol < target_waves) ncol /= 2;
  s->ncol = ncol;
  int bpc = 1;
  RETURN_IF(cached_occupancy(mode, a, *s, &bpc));
  const int64_t groups = (N + ncol - 1) / ncol;
  int64_t waves = (int64_t)dev.cus * bpc * 4;
  if (waves > groups) waves = groups;
  if (waves < 1) waves = 1;
  s->grid = (int)((waves + 3) / 4);
  a.total_waves = (int64_t)s->grid * 4;
  return INT4_OK;
}

// Resident blocks per CU of the fused MLP kernel for one shape, cached like
// cached_occupancy.
int mlp_occupancy(const GemvArgs& gu, int ncol1, const GemvArgs& dn, int ncol2, const LaunchShape& s,
                  int* bpc) {
  struct Key {
    int dev, ncol1, ncol2, threads;
    size_t lds;
    bool operator<(const Key& o) const {
      return std::tie(dev, ncol1, ncol2, threads, lds) < std::tie(o.dev, o.ncol1, o.ncol2, o.threads, o.lds);
    }
  };
  static std::mutex mu;
  static std::map<Key, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  const Key key{dev, ncol1, ncol2, s.block_threads, s.lds_bytes};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      *bpc = it->second;
      return INT4_OK;
    }
  }
  int v = 0;
  e = launch_mlp(gu, ncol1, dn, ncol2, s, nullptr, nullptr, &v);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = v;
  *bpc = v;
  return INT4_OK;
}

uint64_t group_magic(int32_t gs) {
  const uint64_t d = (uint64_t)(gs / 32);
  return (((uint64_t)1 << 40) + d - 1) / d;
}

void fill_common(GemvArgs& a, int64_t N, int64_t K, int32_t gs) {
  a.N = N;
  a.K = (int32_t)K;
  a.U = (int32_t)(K / 32);
  a.G = (int32_t)(K / gs);
  a.nch = (a.U + 63) / 64;
  a.cw = (a.U + a.nch - 1) / a.nch;
  a.g_magic = group_magic(gs);
}

// ------------------------------------------------------------ prefill GEMM

// Checks shared by both GEMM entry points (everything but the workspace);
// fills the workspace layout.
int gemm_validate(const float* X, int64_t T, const uint32_t* q, const float* scales, const float* zeros,
                  int64_t N, int64_t K, int32_t group_size, float* Y, GemmLayout* L) {
  if (N < 0 || T < 0) return fail(INT4_ERR_SHAPE, "N and T must be >= 0 (N=%lld, T=%lld)", (long long)N,
                                  (long long)T);
  RETURN_IF(check_kgs(K, group_size));
  if (N == 0 || T == 0) return INT4_OK;
  if ((uint64_t)N * (uint64_t)K / 2 >= ((uint64_t)1 << 31))
    return fail(INT4_ERR_SHAPE, "N*K/2 = %llu bytes of codes exceed 2^31", (unsigned long long)N * K / 2);
  *L = gemm_layout(T, N, K, group_size);
  if ((uint64_t)L->Tp * (uint64_t)L->Kp * 4 >= ((uint64_t)1 << 40) || L->Tp / 128 * (L->Np / 128) >= ((int64_t)1 << 30))
    return fail(INT4_ERR_SHAPE, "T=%lld is larger than supported", (long long)T);
  if (!X || !q || !scales || !zeros || !Y) return fail(INT4_ERR_NULL, "X, q, scales, zeros and Y are required");
  RETURN_IF(check_align(X, 16, "X"));
  RETURN_IF(check_align(q, 16, "q"));
  RETURN_IF(check_align(scales, 4, "scales"));
  RETURN_IF(check_align(zeros, 4, "zeros"));
  RETURN_IF(check_align(Y, 4, "Y"));
  return INT4_OK;
}

// The prep and GEMM launches over a validated problem and a workspace of at
// least L.bytes (256-byte aligned).
int gemm_launch(const float* X, int64_t T, const uint32_t* q, const float* scales, const float* zeros,
                int64_t N, int64_t K, int32_t group_size, float* Y, const GemmLayout& L, char* ws,
                void* stream) {
  GemmArgs a{};
  a.X = X;
  a.s = scales;
  a.z = zeros;
  a.q = q;
  a.Y = Y;
  a.xs = reinterpret_cast<uint32_t*>(ws + L.xs_off);
  a.fac = reinterpret_cast<float*>(ws + L.fac_off);
  a.st = reinterpret_cast<float*>(ws + L.st_off);
  a.zt = reinterpret_cast<uint32_t*>(ws + L.zt_off);
  a.T = T;
  a.N = N;
  a.Tp = L.Tp;
  a.Np = L.Np;
  a.Gp = L.Gp;
  a.RB = L.Tp / 128;
  // 128 x 256 tiles halve the activation bytes each CU loads per product
  // (the activations are re-read once per column tile); they need enough
  // row blocks to keep the CUs busy, so short prompts use 128 x 128.
  a.BN = gemm_block_cols(L.Tp, group_size);
  a.CB = (N + a.BN - 1) / a.BN;
  a.qbytes = (int64_t)(N * K / 2);
  a.K = (int32_t)K;
  a.Kp = (int32_t)L.Kp;
  a.gs = group_size;
  a.G = (int32_t)(K / group_size);
  // Split K in two when the 128 x 128 tiles alone would leave CUs idle.
  DeviceInfo dev;
  RETURN_IF(device_info(&dev));
  a.S = (a.RB * a.CB < dev.cus && L.Kp / 64 >= 2) ? 2 : 1;
  hipError_t e = launch_gemm(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

// Scratch of int4_gemm_noalloc.  `scratch` names the host-side stand-in of
// the device array; its device address on each device comes from
// hipGetSymbolAddress, once per device (with that device current), and only
// that address is ever handed to a kernel.
constexpr size_t kGemmScratchBytes = INT4_GEMM_NOALLOC_SCRATCH_BYTES;
std::mutex g_scratch_mu;
std::array<char*, 64> g_scratch_ptr{};

int gemm_scratch(char** out);

int run(Mode mode, GemvArgs& a, void* stream) {
  LaunchShape s{};
  RETURN_IF(plan(mode, a, &s));
  hipError_t e = launch_gemv(mode, a, s, (hipStream_t)stream);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}


int gemm_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= (int)g_scratch_ptr.size()) return fail(INT4_ERR_HIP, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(INT4_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return INT4_OK;
}
}  // namespace
}  // namespace int4gemv

using namespace int4gemv;

extern "C" {

const char* int4_status_str(int status) {
  switch (status) {
    case INT4_OK: return "INT4_OK";
    case INT4_ERR_NULL: return "INT4_ERR_NULL";
    case INT4_ERR_SHAPE: return "INT4_ERR_SHAPE";
    case INT4_ERR_ALIGN: return "INT4_ERR_ALIGN";
    case INT4_ERR_ALIAS: return "INT4_ERR_ALIAS";
    case INT4_ERR_ARG: return "INT4_ERR_ARG";
    case INT4_ERR_HIP: return "INT4_ERR_HIP";
    default: return "INT4_ERR_UNKNOWN";
  }
}

const char* int4_last_error(void) { return g_last_error.c_str(); }

int int4_quantize_pack(const float* W, int64_t N, int64_t K, int32_t group_size, uint32_t* q,
                       float* scales, float* zeros, void* stream) {
  if (N < 0) return fail(INT4_ERR_SHAPE, "N must be >= 0 (got %lld)", (long long)N);
  RETURN_IF(check_kgs(K, group_size));
  if (N == 0) return ok();
  if (!W || !q || !scales || !zeros) return fail(INT4_ERR_NULL, "W, q, scales and zeros are required");
  RETURN_IF(check_align(W, 16, "W"));
  RETURN_IF(check_align(q, 4, "q"));
  RETURN_IF(check_align(scales, 4, "scales"));
  RETURN_IF(check_align(zeros, 4, "zeros"));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{W, (uint64_t)N * K * 4, "W"}};
  const Span outs[] = {{q, (uint64_t)N * K / 2, "q"}, {scales, G * 4, "scales"}, {zeros, G * 4, "zeros"}};
  RETURN_IF(check_alias(ins, 1, outs, 3));
  hipError_t e = launch_quantize(W, (int64_t)G, group_size, q, scales, zeros, (hipStream_t)stream);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int int4_matvec(const float* X, int32_t M, const uint32_t* q, const float* scales, const float* zeros,
                int64_t N, int64_t K, int32_t group_size, float* Y, void* stream) {
  if (N < 0) return fail(INT4_ERR_SHAPE, "N must be >= 0 (got %lld)", (long long)N);
  if (M < 0 || M > 8) return fail(INT4_ERR_SHAPE, "M must be in [0, 8] (got %d)", (int)M);
  RETURN_IF(check_kgs(K, group_size));
  if (N == 0 || M == 0) return ok();
  if (!X || !q || !scales || !zeros || !Y)
    return fail(INT4_ERR_NULL, "X, q, scales, zeros and Y are required");
  RETURN_IF(check_align(X, 16, "X"));
  RETURN_IF(check_align(q, 16, "q"));
  RETURN_IF(check_align(scales, 4, "scales"));
  RETURN_IF(check_align(zeros, 4, "zeros"));
  RETURN_IF(check_align(Y, 4, "Y"));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{X, (uint64_t)M * K * 4, "X"}, {q, (uint64_t)N * K / 2, "q"},
                      {scales, G * 4, "scales"}, {zeros, G * 4, "zeros"}};
  const Span outs[] = {{Y, (uint64_t)M * N * 4, "Y"}};
  RETURN_IF(check_alias(ins, 4, outs, 1));
  GemvArgs a{};
  fill_common(a, N, K, group_size);
  a.x = X;
  a.M = M;
  a.q[0] = reinterpret_cast<const uint4*>(q);
  a.s[0] = scales;
  a.z[0] = zeros;
  a.out[0] = Y;
  return run(kPlain, a, stream);
}

int int4_matvec_split4(const float* x, const uint32_t* q, const float* scales, const float* zeros,
                       int64_t N, int64_t K, int32_t group_size, int64_t n0, int64_t n1, int64_t n2,
                       float* out0, float* out1, float* out2, float* out3, void* stream) {
  if (N < 0) return fail(INT4_ERR_SHAPE, "N must be >= 0 (got %lld)", (long long)N);
  RETURN_IF(check_kgs(K, group_size));
  if (!(0 <= n0 && n0 <= n1 && n1 <= n2 && n2 <= N))
    return fail(INT4_ERR_ARG, "split points must satisfy 0 <= n0 <= n1 <= n2 <= N (%lld %lld %lld, N=%lld)",
                (long long)n0, (long long)n1, (long long)n2, (long long)N);
  if (N == 0) return ok();
  const int64_t len[4] = {n0, n1 - n0, n2 - n1, N - n2};
  float* outs_p[4] = {out0, out1, out2, out3};
  if (!x || !q || !scales || !zeros) return fail(INT4_ERR_NULL, "x, q, scales and zeros are required");
  for (int j = 0; j < 4; ++j)
    if (len[j] > 0 && !outs_p[j])
      return fail(INT4_ERR_NULL, "out%d is NULL but its range holds %lld columns", j, (long long)len[j]);
  RETURN_IF(check_align(x, 16, "x"));
  RETURN_IF(check_align(q, 16, "q"));
  RETURN_IF(check_align(scales, 4, "scales"));
  RETURN_IF(check_align(zeros, 4, "zeros"));
  static const char* names[4] = {"out0", "out1", "out2", "out3"};
  for (int j = 0; j < 4; ++j) RETURN_IF(check_align(outs_p[j], 4, names[j]));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{x, (uint64_t)K * 4, "x"}, {q, (uint64_t)N * K / 2, "q"},
                      {scales, G * 4, "scales"}, {zeros, G * 4, "zeros"}};
  const Span outs[] = {{out0, (uint64_t)len[0] * 4, "out0"}, {out1, (uint64_t)len[1] * 4, "out1"},
                       {out2, (uint64_t)len[2] * 4, "out2"}, {out3, (uint64_t)len[3] * 4, "out3"}};
  RETURN_IF(check_alias(ins, 4, outs, 4));
  GemvArgs a{};
  fill_common(a, N, K, group_size);
  a.x = x;
  a.M = 1;
  a.q[0] = reinterpret_cast<const uint4*>(q);
  a.s[0] = scales;
  a.z[0] = zeros;
  for (int j = 0; j < 4; ++j) a.out[j] = outs_p[j];
  a.n0 = n0;
  a.n1 = n1;
  a.n2 = n2;
  return run(kSplit4, a, stream);
}

int int4_matvec_gated(const float* x, const uint32_t* q_gate, const float* s_gate, const float* z_gate,
                      const uint32_t* q_up, const float* s_up, const float* z_up, int64_t N, int64_t K,
                      int32_t group_size, float* h, void* stream) {
  if (N < 0) return fail(INT4_ERR_SHAPE, "N must be >= 0 (got %lld)", (long long)N);
  RETURN_IF(check_kgs(K, group_size));
  if (N == 0) return ok();
  if (!x || !q_gate || !s_gate || !z_gate || !q_up || !s_up || !z_up || !h)
    return fail(INT4_ERR_NULL, "x, both weight triplets and h are required");
  RETURN_IF(check_align(x, 16, "x"));
  RETURN_IF(check_align(q_gate, 16, "q_gate"));
  RETURN_IF(check_align(q_up, 16, "q_up"));
  RETURN_IF(check_align(s_gate, 4, "s_gate"));
  RETURN_IF(check_align(z_gate, 4, "z_gate"));
  RETURN_IF(check_align(s_up, 4, "s_up"));
  RETURN_IF(check_align(z_up, 4, "z_up"));
  RETURN_IF(check_align(h, 4, "h"));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{x, (uint64_t)K * 4, "x"},
                      {q_gate, (uint64_t)N * K / 2, "q_gate"}, {s_gate, G * 4, "s_gate"},
                      {z_gate, G * 4, "z_gate"},
                      {q_up, (uint64_t)N * K / 2, "q_up"}, {s_up, G * 4, "s_up"}, {z_up, G * 4, "z_up"}};
  const Span outs[] = {{h, (uint64_t)N * 4, "h"}};
  RETURN_IF(check_alias(ins, 7, outs, 1));
  GemvArgs a{};
  fill_common(a, N, K, group_size);
  a.x = x;
  a.M = 1;
  a.q[0] = reinterpret_cast<const uint4*>(q_gate);
  a.s[0] = s_gate;
  a.z[0] = z_gate;
  a.q[1] = reinterpret_cast<const uint4*>(q_up);
  a.s[1] = s_up;
  a.z[1] = z_up;
  a.out[0] = h;
  return run(kGated, a, stream);
}

size_t int4_mlp_workspace_bytes(void) { return kMlpWorkspaceBytes; }

int int4_mlp_timed_out(const void* workspace, int32_t* timed_out, void* stream) {
  if (!workspace || !timed_out) return fail(INT4_ERR_NULL, "workspace and timed_out are required");
  RETURN_IF(check_align(workspace, 16, "workspace"));
  uint32_t word = 0;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(&word, static_cast<const uint32_t*>(workspace) + 1, sizeof(word),
                                hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "reading the workspace: %s", hipGetErrorString(e));
  *timed_out = word != 0u;
  return ok();
}

int int4_mlp(const float* x, const uint32_t* q_gate, const float* s_gate, const float* z_gate,
             const uint32_t* q_up, const float* s_up, const float* z_up, const uint32_t* q_down,
             const float* s_down, const float* z_down, int64_t D, int64_t F, int32_t group_size, float* h,
             float* y, void* workspace, size_t workspace_bytes, void* stream) {
  RETURN_IF(check_kgs(D, group_size));
  RETURN_IF(check_kgs(F, group_size));
  if (!x || !q_gate || !s_gate || !z_gate || !q_up || !s_up || !z_up || !q_down || !s_down || !z_down || !h || !y)
    return fail(INT4_ERR_NULL, "x, the three weight triplets, h and y are required");
  if (!workspace) return fail(INT4_ERR_NULL, "workspace is required (int4_mlp_workspace_bytes, zeroed)");
  if (workspace_bytes < int4_mlp_workspace_bytes())
    return fail(INT4_ERR_SHAPE, "workspace holds %zu bytes; the call needs %zu", workspace_bytes,
                int4_mlp_workspace_bytes());
  RETURN_IF(check_align(x, 16, "x"));
  RETURN_IF(check_align(q_gate, 16, "q_gate"));
  RETURN_IF(check_align(q_up, 16, "q_up"));
  RETURN_IF(check_align(q_down, 16, "q_down"));
  RETURN_IF(check_align(s_gate, 4, "s_gate"));
  RETURN_IF(check_align(z_gate, 4, "z_gate"));
  RETURN_IF(check_align(s_up, 4, "s_up"));
  RETURN_IF(check_align(z_up, 4, "z_up"));
  RETURN_IF(check_align(s_down, 4, "s_down"));
  RETURN_IF(check_align(z_down, 4, "z_down"));
  RETURN_IF(check_align(h, 16, "h"));
  RETURN_IF(check_align(y, 4, "y"));
  RETURN_IF(check_align(workspace, 16, "workspace"));
  const uint64_t Gf = (uint64_t)F * (uint64_t)(D / group_size);  // gate/up groups
  const uint64_t Gd = (uint64_t)D * (uint64_t)(F / group_size);  // down groups
  const uint64_t qb = (uint64_t)F * (uint64_t)D / 2;               // bytes of codes per matrix
  const Span ins[] = {{x, (uint64_t)D * 4, "x"},
                      {q_gate, qb, "q_gate"}, {s_gate, Gf * 4, "s_gate"}, {z_gate, Gf * 4, "z_gate"},
                      {q_up, qb, "q_up"}, {s_up, Gf * 4, "s_up"}, {z_up, Gf * 4, "z_up"},
                      {q_down, qb, "q_down"}, {s_down, Gd * 4, "s_down"}, {z_down, Gd * 4, "z_down"}};
  const Span outs[] = {{h, (uint64_t)F * 4, "h"}, {y, (uint64_t)D * 4, "y"},
                       {workspace, int4_mlp_workspace_bytes(), "workspace"}};
  RETURN_IF(check_alias(ins, 10, outs, 3));

  GemvArgs gu{};
  fill_common(gu, F, D, group_size);
  gu.x = x;
  gu.M = 1;
  gu.q[0] = reinterpret_cast<const uint4*>(q_gate);
  gu.s[0] = s_gate;
  gu.z[0] = z_gate;
  gu.q[1] = reinterpret_cast<const uint4*>(q_up);
  gu.s[1] = s_up;
  gu.z[1] = z_up;
  gu.out[0] = h;
  GemvArgs dn{};
  fill_common(dn, D, F, group_size);
  dn.x = h;
  dn.M = 1;
  dn.q[0] = reinterpret_cast<const uint4*>(q_down);
  dn.s[0] = s_down;
  dn.z[0] = z_down;
  dn.out[0] = y;
  LaunchShape s1{}, s2{};
  RETURN_IF(plan(kGated, gu, &s1));
  RETURN_IF(plan(kPlain, dn, &s2));
  hipStream_t st = (hipStream_t)stream;
  // One launch when both passes run the register kernel on the same grid
  // and that grid is resident at once; the passes then keep the shapes of
  // the standalone calls, so their results are the same bits.
  if (s1.variant == kVariantReg && s2.variant == kVariantReg && s1.grid == s2.grid && s1.grid <= kMlpMaxBlocks) {
    LaunchShape s = s1;
    s.block_threads = s1.block_threads > s2.block_threads ? s1.block_threads : s2.block_threads;
    s.lds_bytes = s1.lds_bytes > s2.lds_bytes ? s1.lds_bytes : s2.lds_bytes;
    DeviceInfo dev;
    RETURN_IF(device_info(&dev));
    int bpc = 0;
    RETURN_IF(mlp_occupancy(gu, s1.ncol, dn, s2.ncol, s, &bpc));
    if ((int64_t)bpc * dev.cus >= s.grid) {
      hipError_t e = launch_mlp(gu, s1.ncol, dn, s2.ncol, s, static_cast<uint32_t*>(workspace), st, nullptr);
      if (e != hipSuccess) return fail(INT4_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
      return ok();
    }
  }
  hipError_t e = launch_gemv(kGated, gu, s1, st);
  if (e == hipSuccess) e = launch_gemv(kPlain, dn, s2, st);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int int4_matvec_gated_lanes(const float* X, int32_t M, const uint32_t* q_gate, const float* s_gate,
                            const float* z_gate, const uint32_t* q_up, const float* s_up,
                            const float* z_up, int64_t N, int64_t K, int32_t group_size, float* H,
                            void* stream) {
  if (N < 0) return fail(INT4_ERR_SHAPE, "N must be >= 0 (got %lld)", (long long)N);
  if (M < 0 || M > 8) return fail(INT4_ERR_SHAPE, "M must be in [0, 8] (got %d)", (int)M);
  RETURN_IF(check_kgs(K, group_size));
  if (N == 0 || M == 0) return ok();
  if (!X || !q_gate || !s_gate || !z_gate || !q_up || !s_up || !z_up || !H)
    return fail(INT4_ERR_NULL, "X, both weight triplets and H are required");
  RETURN_IF(check_align(X, 16, "X"));
  RETURN_IF(check_align(q_gate, 16, "q_gate"));
  RETURN_IF(check_align(q_up, 16, "q_up"));
  RETURN_IF(check_align(s_gate, 4, "s_gate"));
  RETURN_IF(check_align(z_gate, 4, "z_gate"));
  RETURN_IF(check_align(s_up, 4, "s_up"));
  RETURN_IF(check_align(z_up, 4, "z_up"));
  RETURN_IF(check_align(H, 4, "H"));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{X, (uint64_t)M * K * 4, "X"},
                      {q_gate, (uint64_t)N * K / 2, "q_gate"}, {s_gate, G * 4, "s_gate"},
                      {z_gate, G * 4, "z_gate"},
                      {q_up, (uint64_t)N * K / 2, "q_up"}, {s_up, G * 4, "s_up"}, {z_up, G * 4, "z_up"}};
  const Span outs[] = {{H, (uint64_t)M * N * 4, "H"}};
  RETURN_IF(check_alias(ins, 7, outs, 1));
  GemvArgs a{};
  fill_common(a, N, K, group_size);
  a.x = X;
  a.M = M;
  a.q[0] = reinterpret_cast<const uint4*>(q_gate);
  a.s[0] = s_gate;
  a.z[0] = z_gate;
  a.q[1] = reinterpret_cast<const uint4*>(q_up);
  a.s[1] = s_up;
  a.z[1] = z_up;
  a.out[0] = H;
  return run(kGated, a, stream);
}

int int4_matvec_norm(const float* a_a, const float* a_b, const float* w_norm, float eps,
                     const uint32_t* q, const float* scales, const float* zeros, int64_t N, int64_t K,
                     int32_t group_size, float* y, float* residual_out, float* norm_out, void* stream) {
  if (N < 0) return fail(INT4_ERR_SHAPE, "N must be >= 0 (got %lld)", (long long)N);
  RETURN_IF(check_kgs(K, group_size));
  if (!(isfinite(eps) && eps >= 0.0f)) return fail(INT4_ERR_ARG, "eps must be finite and >= 0");
  if (N == 0 && !residual_out && !norm_out) return ok();
  if (!a_a || !a_b || !w_norm) return fail(INT4_ERR_NULL, "a_a, a_b and w_norm are required");
  if (N > 0 && (!q || !scales || !zeros || !y))
    return fail(INT4_ERR_NULL, "q, scales, zeros and y are required when N > 0");
  RETURN_IF(check_align(a_a, 16, "a_a"));
  RETURN_IF(check_align(a_b, 16, "a_b"));
  RETURN_IF(check_align(w_norm, 16, "w_norm"));
  RETURN_IF(check_align(q, 16, "q"));
  RETURN_IF(check_align(scales, 4, "scales"));
  RETURN_IF(check_align(zeros, 4, "zeros"));
  RETURN_IF(check_align(y, 4, "y"));
  RETURN_IF(check_align(residual_out, 16, "residual_out"));
  RETURN_IF(check_align(norm_out, 16, "norm_out"));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{a_a, (uint64_t)K * 4, "a_a"}, {a_b, (uint64_t)K * 4, "a_b"},
                      {w_norm, (uint64_t)K * 4, "w_norm"}, {q, (uint64_t)N * K / 2, "q"},
                      {scales, G * 4, "scales"}, {zeros, G * 4, "zeros"}};
  const Span outs[] = {{y, (uint64_t)N * 4, "y"},
                       {residual_out, residual_out ? (uint64_t)K * 4 : 0, "residual_out"},
                       {norm_out, norm_out ? (uint64_t)K * 4 : 0, "norm_out"}};
  RETURN_IF(check_alias(ins, 6, outs, 3));
  GemvArgs a{};
  fill_common(a, N, K, group_size);
  a.x = a_a;
  a.x2 = a_b;
  a.w_norm = w_norm;
  a.eps = eps;
  a.M = 1;
  a.q[0] = reinterpret_cast<const uint4*>(q);
  a.s[0] = scales;
  a.z[0] = zeros;
  a.out[0] = y;
  a.residual_out = residual_out;
  a.norm_out = norm_out;
  return run(kNorm, a, stream);
}

int int4_matvec_dual(const float* X, int32_t M, const uint32_t* q0, const float* s0, const float* z0,
                     const uint32_t* q1, const float* s1, const float* z1, int64_t N, int64_t K,
                     int32_t group_size, float* y0, float* y1, void* stream) {
  if (N < 0) return fail(INT4_ERR_SHAPE, "N must be >= 0 (got %lld)", (long long)N);
  if (M < 0 || M > 8) return fail(INT4_ERR_SHAPE, "M must be in [0, 8] (got %d)", (int)M);
  RETURN_IF(check_kgs(K, group_size));
  if (N == 0 || M == 0) return ok();
  if (!X || !q0 || !s0 || !z0 || !q1 || !s1 || !z1 || !y0 || !y1)
    return fail(INT4_ERR_NULL, "X, both weight triplets, y0 and y1 are required");
  RETURN_IF(check_align(X, 16, "X"));
  RETURN_IF(check_align(q0, 16, "q0"));
  RETURN_IF(check_align(q1, 16, "q1"));
  RETURN_IF(check_align(s0, 4, "s0"));
  RETURN_IF(check_align(z0, 4, "z0"));
  RETURN_IF(check_align(s1, 4, "s1"));
  RETURN_IF(check_align(z1, 4, "z1"));
  RETURN_IF(check_align(y0, 4, "y0"));
  RETURN_IF(check_align(y1, 4, "y1"));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{X, (uint64_t)M * K * 4, "X"},
                      {q0, (uint64_t)N * K / 2, "q0"}, {s0, G * 4, "s0"}, {z0, G * 4, "z0"},
                      {q1, (uint64_t)N * K / 2, "q1"}, {s1, G * 4, "s1"}, {z1, G * 4, "z1"}};
  const Span outs[] = {{y0, (uint64_t)M * N * 4, "y0"}, {y1, (uint64_t)M * N * 4, "y1"}};
  RETURN_IF(check_alias(ins, 7, outs, 2));
  GemvArgs a{};
  fill_common(a, N, K, group_size);
  a.x = X;
  a.M = M;
  a.q[0] = reinterpret_cast<const uint4*>(q0);
  a.s[0] = s0;
  a.z[0] = z0;
  a.q[1] = reinterpret_cast<const uint4*>(q1);
  a.s[1] = s1;
  a.z[1] = z1;
  a.out[0] = y0;
  a.out[1] = y1;
  return run(kDual, a, stream);
}

// Shared by the two input-gated entry points: p and r are the two input
// row sets [M][K] (a and gate, or gate and up).
static int input_gated(Mode mode, const float* p, const float* r, int32_t M, const char* pn,
                       const char* rn, const uint32_t* q, const float* scales, const float* zeros,
                       int64_t N, int64_t K, int32_t group_size, float* y, void* stream) {
  if (N < 0) return fail(INT4_ERR_SHAPE, "N must be >= 0 (got %lld)", (long long)N);
  if (M < 0 || M > 8) return fail(INT4_ERR_SHAPE, "M must be in [0, 8] (got %d)", (int)M);
  RETURN_IF(check_kgs(K, group_size));
  if (N == 0 || M == 0) return ok();
  if (!p || !r || !q || !scales || !zeros || !y)
    return fail(INT4_ERR_NULL, "%s, %s, q, scales, zeros and y are required", pn, rn);
  RETURN_IF(check_align(p, 16, pn));
  RETURN_IF(check_align(r, 16, rn));
  RETURN_IF(check_align(q, 16, "q"));
  RETURN_IF(check_align(scales, 4, "scales"));
  RETURN_IF(check_align(zeros, 4, "zeros"));
  RETURN_IF(check_align(y, 4, "y"));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{p, (uint64_t)M * K * 4, pn}, {r, (uint64_t)M * K * 4, rn},
                      {q, (uint64_t)N * K / 2, "q"}, {scales, G * 4, "scales"}, {zeros, G * 4, "zeros"}};
  const Span outs[] = {{y, (uint64_t)M * N * 4, "y"}};
  RETURN_IF(check_alias(ins, 5, outs, 1));
  GemvArgs a{};
  fill_common(a, N, K, group_size);
  a.x = p;
  a.x2 = r;
  a.M = M;
  a.q[0] = reinterpret_cast<const uint4*>(q);
  a.s[0] = scales;
  a.z[0] = zeros;
  a.out[0] = y;
  return run(mode, a, stream);
}

int int4_matvec_sigmoid_gated(const float* a_in, const float* gate, int32_t M, const uint32_t* q,
                              const float* scales, const float* zeros, int64_t N, int64_t K,
                              int32_t group_size, float* y, void* stream) {
  return input_gated(kSigIn, a_in, gate, M, "a", "gate", q, scales, zeros, N, K, group_size, y, stream);
}

int int4_matvec_swiglu_gated(const float* gate, const float* up, int32_t M, const uint32_t* q,
                             const float* scales, const float* zeros, int64_t N, int64_t K,
                             int32_t group_size, float* y, void* stream) {
  return input_gated(kSwiIn, gate, up, M, "gate", "up", q, scales, zeros, N, K, group_size, y, stream);
}

int int4_matvec_norm_swiglu(const float* a_a, const float* a_b, const float* w_norm, float eps,
                            const uint32_t* q_gate, const float* s_gate, const float* z_gate,
                            const uint32_t* q_up, const float* s_up, const float* z_up, int64_t N,
                            int64_t K, int32_t group_size, float* h, float* residual_out,
                            void* stream) {
  if (N < 0) return fail(INT4_ERR_SHAPE, "N must be >= 0 (got %lld)", (long long)N);
  RETURN_IF(check_kgs(K, group_size));
  if (!(isfinite(eps) && eps >= 0.0f)) return fail(INT4_ERR_ARG, "eps must be finite and >= 0");
  if (N == 0 && !residual_out) return ok();
  if (!a_a || !a_b || !w_norm) return fail(INT4_ERR_NULL, "a_a, a_b and w_norm are required");
  if (N > 0 && (!q_gate || !s_gate || !z_gate || !q_up || !s_up || !z_up || !h))
    return fail(INT4_ERR_NULL, "both weight triplets and h are required when N > 0");
  RETURN_IF(check_align(a_a, 16, "a_a"));
  RETURN_IF(check_align(a_b, 16, "a_b"));
  RETURN_IF(check_align(w_norm, 16, "w_norm"));
  RETURN_IF(check_align(q_gate, 16, "q_gate"));
  RETURN_IF(check_align(q_up, 16, "q_up"));
  RETURN_IF(check_align(s_gate, 4, "s_gate"));
  RETURN_IF(check_align(z_gate, 4, "z_gate"));
  RETURN_IF(check_align(s_up, 4, "s_up"));
  RETURN_IF(check_align(z_up, 4, "z_up"));
  RETURN_IF(check_align(h, 4, "h"));
  RETURN_IF(check_align(residual_out, 16, "residual_out"));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{a_a, (uint64_t)K * 4, "a_a"}, {a_b, (uint64_t)K * 4, "a_b"},
                      {w_norm, (uint64_t)K * 4, "w_norm"},
                      {q_gate, (uint64_t)N * K / 2, "q_gate"}, {s_gate, G * 4, "s_gate"},
                      {z_gate, G * 4, "z_gate"},
                      {q_up, (uint64_t)N * K / 2, "q_up"}, {s_up, G * 4, "s_up"}, {z_up, G * 4, "z_up"}};
  const Span outs[] = {{h, (uint64_t)N * 4, "h"},
                       {residual_out, residual_out ? (uint64_t)K * 4 : 0, "residual_out"}};
  RETURN_IF(check_alias(ins, 9, outs, 2));
  GemvArgs a{};
  fill_common(a, N, K, group_size);
  a.x = a_a;
  a.x2 = a_b;
  a.w_norm = w_norm;
  a.eps = eps;
  a.M = 1;
  a.q[0] = reinterpret_cast<const uint4*>(q_gate);
  a.s[0] = s_gate;
  a.z[0] = z_gate;
  a.q[1] = reinterpret_cast<const uint4*>(q_up);
  a.s[1] = s_up;
  a.z[1] = z_up;
  a.out[0] = h;
  a.residual_out = residual_out;
  a.norm_out = nullptr;
  return run(kNormSwi, a, stream);
}

int int4_embedding_gather(const int32_t* ids, int64_t T, const uint32_t* q, const float* scales,
                          const float* zeros, int64_t N, int64_t K, int32_t group_size, float* out,
                          void* stream) {
  if (N < 0 || T < 0) return fail(INT4_ERR_SHAPE, "N and T must be >= 0 (N=%lld, T=%lld)", (long long)N,
                                  (long long)T);
  RETURN_IF(check_kgs(K, group_size));
  if (T == 0) return ok();
  if (!ids || !out) return fail(INT4_ERR_NULL, "ids and out are required");
  if (N > 0 && (!q || !scales || !zeros)) return fail(INT4_ERR_NULL, "q, scales and zeros are required when N > 0");
  RETURN_IF(check_align(ids, 4, "ids"));
  RETURN_IF(check_align(q, 4, "q"));
  RETURN_IF(check_align(scales, 4, "scales"));
  RETURN_IF(check_align(zeros, 4, "zeros"));
  RETURN_IF(check_align(out, 16, "out"));
  if ((uint64_t)T * (uint64_t)K > ((uint64_t)1 << 40))
    return fail(INT4_ERR_SHAPE, "T*K=%llu is larger than supported", (unsigned long long)T * K);
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{ids, (uint64_t)T * 4, "ids"}, {q, (uint64_t)N * K / 2, "q"},
                      {scales, G * 4, "scales"}, {zeros, G * 4, "zeros"}};
  const Span outs[] = {{out, (uint64_t)T * K * 4, "out"}};
  RETURN_IF(check_alias(ins, 4, outs, 1));
  hipError_t e = launch_embedding(ids, T, q, scales, zeros, N, (int32_t)K, group_size, out,
                                  (hipStream_t)stream);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

// The device-side address of a table in page-locked host memory (hipHostMalloc,
// mapped into the device's address space); anything else (pageable or device
// memory) is refused, because a kernel reading pageable memory faults.
static int host_table_ptr(const void* p, const char* name, const void** dev) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the next call
    return fail(INT4_ERR_ARG, "%s is not page-locked host memory (allocate it with hipHostMalloc)", name);
  }
  if (at.type != hipMemoryTypeHost || !at.devicePointer || !at.hostPointer)
    return fail(INT4_ERR_ARG, "%s is not page-locked host memory mapped for the device", name);
  *dev = static_cast<const char*>(at.devicePointer) +
         (static_cast<const char*>(p) - static_cast<const char*>(at.hostPointer));
  return INT4_OK;
}

int int4_embedding_gather_host(const int32_t* ids, int64_t T, const uint32_t* q, const float* scales,
                               const float* zeros, int64_t N, int64_t K, int32_t group_size, float* out,
                               void* stream) {
  if (N < 0 || T < 0) return fail(INT4_ERR_SHAPE, "N and T must be >= 0 (N=%lld, T=%lld)", (long long)N,
                                  (long long)T);
  RETURN_IF(check_kgs(K, group_size));
  if (T == 0) return ok();
  if (!ids || !out) return fail(INT4_ERR_NULL, "ids and out are required");
  if (N > 0 && (!q || !scales || !zeros)) return fail(INT4_ERR_NULL, "q, scales and zeros are required when N > 0");
  RETURN_IF(check_align(ids, 4, "ids"));
  RETURN_IF(check_align(q, 4, "q"));
  RETURN_IF(check_align(scales, 4, "scales"));
  RETURN_IF(check_align(zeros, 4, "zeros"));
  RETURN_IF(check_align(out, 16, "out"));
  if ((uint64_t)T * (uint64_t)K > ((uint64_t)1 << 40))
    return fail(INT4_ERR_SHAPE, "T*K=%llu is larger than supported", (unsigned long long)T * K);
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{ids, (uint64_t)T * 4, "ids"}, {q, (uint64_t)N * K / 2, "q"},
                      {scales, G * 4, "scales"}, {zeros, G * 4, "zeros"}};
  const Span outs[] = {{out, (uint64_t)T * K * 4, "out"}};
  RETURN_IF(check_alias(ins, 4, outs, 1));
  const void *dq = nullptr, *ds = nullptr, *dz = nullptr;
  if (N > 0) {
    RETURN_IF(host_table_ptr(q, "q", &dq));
    RETURN_IF(host_table_ptr(scales, "scales", &ds));
    RETURN_IF(host_table_ptr(zeros, "zeros", &dz));
  }
  hipError_t e = launch_embedding(ids, T, static_cast<const uint32_t*>(dq), static_cast<const float*>(ds),
                                  static_cast<const float*>(dz), N, (int32_t)K, group_size, out,
                                  (hipStream_t)stream);
  if (e != hipSuccess) return fail(INT4_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

size_t int4_gemm_workspace_bytes(int64_t T, int64_t N, int64_t K, int32_t group_size) {
  if (T <= 0 || N <= 0 || K <= 0 || group_size <= 0) return 0;
  return gemm_layout(T, N, K, group_size).bytes;
}

int int4_gemm(const float* X, int64_t T, const uint32_t* q, const float* scales, const float* zeros,
              int64_t N, int64_t K, int32_t group_size, float* Y, void* workspace,
              size_t workspace_bytes, void* stream) {
  GemmLayout L;
  RETURN_IF(gemm_validate(X, T, q, scales, zeros, N, K, group_size, Y, &L));
  if (N == 0 || T == 0) return ok();
  if (!workspace) return fail(INT4_ERR_NULL, "workspace is required (int4_gemm_workspace_bytes)");
  if (workspace_bytes < L.bytes)
    return fail(INT4_ERR_SHAPE, "workspace holds %zu bytes; this call needs %zu", workspace_bytes, L.bytes);
  RETURN_IF(check_align(workspace, 256, "workspace"));
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{X, (uint64_t)T * K * 4, "X"}, {q, (uint64_t)N * K / 2, "q"},
                      {scales, G * 4, "scales"}, {zeros, G * 4, "zeros"}};
  const Span outs[] = {{Y, (uint64_t)T * N * 4, "Y"}, {workspace, L.bytes, "workspace"}};
  RETURN_IF(check_alias(ins, 4, outs, 2));
  return gemm_launch(X, T, q, scales, zeros, N, K, group_size, Y, L, static_cast<char*>(workspace), stream);
}

int int4_gemm_noalloc(const float* X, int64_t T, const uint32_t* q, const float* scales,
                      const float* zeros, int64_t N, int64_t K, int32_t group_size, float* Y,
                      void* stream) {
  GemmLayout L;
  RETURN_IF(gemm_validate(X, T, q, scales, zeros, N, K, group_size, Y, &L));
  if (N == 0 || T == 0) return ok();
  if (L.bytes > kGemmScratchBytes)
    return fail(INT4_ERR_SHAPE,
                "T=%lld, N=%lld, K=%lld need %zu bytes of scratch; the allocation-free GEMM holds %zu "
                "(use int4_gemm with a workspace)",
                (long long)T, (long long)N, (long long)K, L.bytes, kGemmScratchBytes);
  const uint64_t G = (uint64_t)N * (uint64_t)(K / group_size);
  const Span ins[] = {{X, (uint64_t)T * K * 4, "X"}, {q, (uint64_t)N * K / 2, "q"},
                      {scales, G * 4, "scales"}, {zeros, G * 4, "zeros"}};
  const Span outs[] = {{Y, (uint64_t)T * N * 4, "Y"}};
  RETURN_IF(check_alias(ins, 4, outs, 1));
  char* ws = nullptr;
  RETURN_IF(gemm_scratch(&ws));
  return gemm_launch(X, T, q, scales, zeros, N, K, group_size, Y, L, ws, stream);
}

}  // extern "C"
