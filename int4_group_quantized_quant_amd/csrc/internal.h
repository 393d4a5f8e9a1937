// internal.h -- launch interface between the C ABI layer (abi.hip) and the
// kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace int4gemv {

// Epilogue / prologue variant of the streaming matvec kernel.
enum Mode : int {
  kPlain = 0,    // Y[m][n] for M lanes
  kSplit4 = 1,   // one lane, columns routed into four buffers
  kGated = 2,    // one lane, two weight streams, h = silu(g) * u
  kNorm = 3,     // one lane, residual-add + RMSNorm prologue
  kDual = 4,     // one lane, two weight streams, y0 = g and y1 = u
  kSigIn = 5,    // one lane, input x = a * sigmoid(gate)
  kSwiIn = 6,    // one lane, input x = silu(gate) * up
  kNormSwi = 7,  // one lane, RMSNorm prologue, two streams, h = silu(g) * u
};

// Weight streams a mode reads (gate/up or the two projections of a pair).
__host__ __device__ constexpr int mode_streams(int mode) {
  return mode == kGated || mode == kDual || mode == kNormSwi ? 2 : 1;
}
// Modes whose input is the residual-add + RMSNorm of (a_a, a_b, w_norm).
__host__ __device__ constexpr bool mode_has_norm(int mode) { return mode == kNorm || mode == kNormSwi; }
// Modes whose input is an elementwise gate of two vectors (x, x2).
__host__ __device__ constexpr bool mode_gates_input(int mode) { return mode == kSigIn || mode == kSwiIn; }

// Everything a matvec launch needs; passed by value as the kernel argument.
struct GemvArgs {
  const float* x;       // X [M][K]; norm modes: a_a [K]; kSigIn: a [K]; kSwiIn: gate [K]
  const float* x2;      // norm modes: a_b [K]; kSigIn: gate [K]; kSwiIn: up [K]
  const float* w_norm;  // norm modes: RMSNorm gain [K]
  float eps;            // norm modes
  const uint4* q[2];    // packed codes per weight stream, 16-byte units [N][K/32]
  const float* s[2];    // scales per stream [N][K/gs]
  const float* z[2];    // zero points per stream [N][K/gs]
  float* out[4];        // kPlain: out[0] = Y [M][N]; kSplit4: four routed buffers;
                        // kGated, kNormSwi: out[0] = h; kDual: out[0] = y0, out[1] = y1;
                        // kNorm, kSigIn, kSwiIn: out[0] = y
  float* residual_out;  // norm modes, nullable
  float* norm_out;      // kNorm, nullable (null for kNormSwi)
  int64_t N;            // output columns
  int64_t n0, n1, n2;   // kSplit4 split points
  int64_t total_waves;  // waves in the grid; wave w owns columns [w*N/W, (w+1)*N/W)
  uint64_t g_magic;     // ceil(2^40 / (gs/32)): unit u lies in group (u*g_magic) >> 40
  int32_t K;            // inputs per column
  int32_t U;            // 16-byte units per column = K/32
  int32_t G;            // groups per column = K/gs
  int32_t nch;          // chunks per column = ceil(U/64)
  int32_t cw;           // units per chunk = ceil(U/nch) (register kernel)
  int32_t rows_per_block;  // P: rows of nch waves per block (register kernel)
  int32_t part_floats;  // floats of the per-block partial table (register kernel)
  int32_t M;            // lanes (kPlain)
  int32_t rt;           // tiles of 16 columns per round (matrix-core kernel)
  int32_t su;           // units per K slice (matrix-core kernel; 24 when mixed)
  int32_t mix24;        // matrix-core kernel: > 0 runs one slice per wave, this many
                        // waves of 24 units and the rest of 16 (whole cache lines)
  uint32_t g_recip;     // ceil(2^32 / G), 0 when G = 1 (matrix-core kernel's table copy)
  int32_t block_threads;  // threads per block as launched, set by the launcher: the
                          // kernels read it from their arguments, since blockDim.x
                          // costs a vector load of the dispatch packet at entry
};

// Float offset of the staged activations in the register kernel's LDS: after
// the partial table, one float per wave (at most 16 waves) and one column
// group counter per chunk (at most 8), rounded up to a float4.
__host__ __device__ inline int x_lds_offset(int part_floats) { return (part_floats + 24 + 3) & ~3; }
// The register kernel stages activation float4 i at plane i % 8, position
// i / 8 (so that lane u later reads its 32 inputs as 8 contiguous-across-
// lanes float4s).  Planes are x_plane_stride(U) float4s apart, U rounded up
// to 9 mod 16: the 8 planes a group of consecutive staging writes touches
// then start in distinct 16-byte bank groups (with 32 or 64 four-byte
// banks), where a stride of U (a multiple of 16 for U = 128, 160 or 448)
// would put them all in one.  The LDS after x_lds_offset holds
// 32 * x_plane_stride(U) floats.
__host__ __device__ inline int x_plane_stride(int U) { return U + ((9 - U) & 15); }

enum Variant : int {
  kVariantLds = 0,   // activations staged in LDS, one wave per column group
  kVariantReg = 1,   // activations in registers, one wave per (row, K chunk)
  kVariantSlice = 2, // two to eight lanes on the matrix cores, K sliced over the waves
};

// Matrix-core lanes kernel.  K is cut into slices of SU units (SU = 16, 20
// or 24); each wave holds one slice's activations in registers and streams
// the block's tiles of 16 columns over it.  Its LDS holds, per wave, a stage
// of one tile's codes (16 columns of 4*SU + 4 dwords) and, per block, for a
// round of RT tiles: the partial sums (8 rows x 16 columns per (tile, wave))
// and a table of the round's scales and zero points (16*RT columns of GP
// dwords each, for both).
constexpr int kSliceMaxWaves = 8;  // two waves per SIMD

// Group-size class of gsu = gs/32 units per group: 1, 2 or 4 (slices start
// on group boundaries and the group structure is fixed at compile time), or
// 0 for any other size (worked out per unit at run time; gsu >= 3).
__host__ __device__ constexpr int slice_class(int gsu) { return gsu == 1 || gsu == 2 || gsu == 4 ? gsu : 0; }

// Groups a slice of su units can touch: su / gsu for the fixed classes,
// ceil((su - 1) / 3) + 1 otherwise.
__host__ __device__ constexpr int slice_groups(int su, int cls) { return cls ? su / cls : (su + 1) / 3 + 1; }
// Dwords per column of the code stage: padded so that the 16 columns start on
// distinct pairs of banks.
__host__ __device__ constexpr int slice_code_stride(int su) { return 4 * su + 4; }
__host__ __device__ constexpr int slice_stage_words(int su) { return 16 * slice_code_stride(su); }
// Dwords per column of the scale / zero-point table: the G groups, then
// zeros for the groups a slice past K can name, rounded up to an odd count
// so that the 16 columns of a tile fall on distinct banks.
__host__ __device__ constexpr int slice_table_stride(int G, int su, int cls) {
  return (G + slice_groups(su, cls)) | 1;
}
// nv: weight streams per column tile (2 for the gated lanes), each with its
// own partials and tables.
inline size_t slice_lds_bytes(int su, int cls, int G, int waves, int rt, int nv = 1) {
  return ((size_t)waves * slice_stage_words(su) + (size_t)nv * rt * waves * 128 +
          (size_t)nv * 2 * rt * 16 * slice_table_stride(G, su, cls)) * sizeof(float);
}

struct LaunchShape {
  int variant;        // Variant
  int ncol;           // columns per wave step (1, 2 or 4)
  int depth;          // register kernel: steps of loads in flight ahead of compute (1)
  int block_threads;  // threads per block (multiple of 64)
  int grid;           // blocks
  size_t lds_bytes;   // dynamic LDS per block
  size_t lds_max;     // device limit of dynamic LDS per block
};

// Launches the matvec kernel for `mode` / `a.M` / `shape`; returns the launch
// status (hipGetLastError after the launch).
hipError_t launch_gemv(Mode mode, const GemvArgs& a, const LaunchShape& shape, hipStream_t stream);

// Resident blocks per CU of the kernel `launch_gemv` would run for this shape.
hipError_t gemv_occupancy(Mode mode, const GemvArgs& a, const LaunchShape& shape, int* blocks_per_cu);

// The fused MLP (gated pass, grid-wide wait, down pass) in one launch of
// the register kernel's passes: `gate_up` and `down` are planned as the
// standalone kGated and kPlain register-kernel calls with the same grid;
// `shape` holds that grid and the larger block and LDS of the two.
// `ws` is the caller's workspace (kMlpWorkspaceBytes, zeroed before its
// first use): a call counter, a timeout flag and one flag per block, for
// grids of at most kMlpMaxBlocks.  With `occupancy` set only queries the
// resident blocks per CU.
constexpr size_t kMlpWorkspaceBytes = 8192;
constexpr int kMlpMaxBlocks = (int)(kMlpWorkspaceBytes / 4) - 32;
hipError_t launch_mlp(const GemvArgs& gate_up, int ncol_gate_up, const GemvArgs& down, int ncol_down,
                      const LaunchShape& shape, uint32_t* ws, hipStream_t stream, int* occupancy);

// The matrix-core lanes kernel (slice.hip) for modes kPlain, kDual, kGated,
// kSigIn and kSwiIn; launches, or with `occupancy` set only queries.
hipError_t dispatch_slice(Mode mode, const GemvArgs& a, const LaunchShape& s, hipStream_t stream,
                          int* occupancy);

// Largest `ncol` instantiated for (mode, M, variant).
int max_ncol(Mode mode, int M, int variant);

// ------------------------------------------------------------ prefill GEMM

// Everything the prefill GEMM's two launches need.  The workspace (owned by
// the caller) holds, in this order, each region 256-byte aligned:
//   xs   [Tp][Kp] split activations: per 8-input block, 4 dwords of fp16 hi
//        then 4 dwords of fp16 lo (slot order 0, 4, 1, 5, 2, 6, 3, 7)
//   fac  [Tp] 2^(24 - e_t) per token row (0 for the pad rows)
//   st   [Gp][Np] scales, transposed; zt [Gp][Np] zero points as fp16
//        subnormal pairs (zero | zero << 16), transposed; 0 outside the matrix
// with Tp = T rounded up to 128, Np = N rounded up to 256, Kp = K rounded
// up to 64, Gp = ceil(Kp / gs).
struct GemmArgs {
  const float* X;     // [T][K]
  const float* s;     // [N][G]
  const float* z;     // [N][G]
  const uint32_t* q;  // [N][K/8]
  float* Y;           // [T][N]
  uint32_t* xs;
  float* fac;
  float* st;
  uint32_t* zt;
  int64_t T, N, Tp, Np, Gp, RB, CB;
  int64_t qbytes;  // N * K / 2
  int32_t K, Kp, gs, G;
  int32_t S;   // K parts per tile (1 or 2)
  int32_t BN;  // columns per block tile (128 or 256)
};

struct GemmLayout {
  int64_t Tp, Np, Kp, Gp;
  size_t xs_off, fac_off, st_off, zt_off, bytes;
};

inline size_t gemm_align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline GemmLayout gemm_layout(int64_t T, int64_t N, int64_t K, int32_t gs) {
  GemmLayout L;
  L.Tp = (T + 127) / 128 * 128;
  L.Np = (N + 255) / 256 * 256;
  L.Kp = (K + 63) / 64 * 64;
  L.Gp = (L.Kp + gs - 1) / gs;
  L.xs_off = 0;
  L.fac_off = gemm_align256(L.xs_off + (size_t)L.Tp * (size_t)L.Kp * 4);
  L.st_off = gemm_align256(L.fac_off + (size_t)L.Tp * 4);
  L.zt_off = gemm_align256(L.st_off + (size_t)L.Gp * (size_t)L.Np * 4);
  L.bytes = gemm_align256(L.zt_off + (size_t)L.Gp * (size_t)L.Np * 4);
  return L;
}

// Columns per block tile: 256 (half the activation bytes per product) when
// there are enough row blocks to fill the CUs and the group size is 64 or
// 128, else 128.
int gemm_block_cols(int64_t Tp, int32_t gs);

// Dynamic LDS of the GEMM kernel (two stages) for block tiles 128 x bn.
size_t gemm_lds_bytes(int bn);

// The prep launch (split activations, transposed scale / zero tables) and
// the GEMM launch, in stream order.
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream);

// Int4 embedding row gather: out [T][K] from rows ids[t] of the table.
hipError_t launch_embedding(const int32_t* ids, int64_t T, const uint32_t* q, const float* scales,
                            const float* zeros, int64_t N, int32_t K, int32_t gs, float* out,
                            hipStream_t stream);

// Quantize + pack launch: groups [0, total_groups), each gs consecutive floats.
hipError_t launch_quantize(const float* W, int64_t total_groups, int32_t gs, uint32_t* q,
                           float* scales, float* zeros, hipStream_t stream);

}  // namespace int4gemv
