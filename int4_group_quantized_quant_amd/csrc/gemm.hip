// gemm.hip -- int4 group-quantized GEMM for prefill on the matrix cores:
// Y[t][n] = sum_k X[t][k] * w[n][k] for T tokens at once ([P1] the prefill
// path runs a tiled matmul for any M, decode the K-parallel matvec).  Unlike
// the decode matvec this is a dense contraction with T-fold reuse of every
// weight, so it is bound by the matrix cores, not by HBM.
//
// Operands of v_mfma_f32_16x16x32_f16 (lane l holds A[l%16][8(l/16)..+7],
// B[8(l/16)..+7][l%16], D[4(l/16)..+3][l%16]):
//  * B = (code - zero) as exact fp16 subnormals: the even nibbles of a code
//    word masked in place (code * 2^-24), the odd ones four bits up
//    (code * 2^-20), minus the zero point shifted the same way.  A word's
//    eight slots hold inputs 0, 4, 1, 5, 2, 6, 3, 7 of its 8-input block.
//  * A = the activations split into hi = fp16(y) and lo = fp16(y - hi) (both
//    rounded toward zero; y - hi is exact in fp32), y = x * 2^e_t with the odd
//    inputs also times 2^-4, in the slot order above; e_t per token puts the
//    row's largest |x| just below 2^14.  hi + lo carries y to 2^-21 relative.
//    A prep kernel writes this split once per call into the caller's
//    workspace, so the GEMM's inner loop holds no conversions.
//  * Two MFMAs per fragment pair (hi, lo) into one accumulator; the group's
//    scale multiplies that accumulator into the total once per group, and
//    the total is finally multiplied by 2^(24 - e_t).
//
// Tiling: a block of 8 waves (two per SIMD) computes a 128 x 128 tile of Y;
// wave (wr, wc) owns rows 32 wr .. +31 and columns 64 wc .. +63 as 2 x 4
// MFMA tiles.  K is streamed in stages of 64 inputs (activations, code
// words, and the stage's scales and zero points) through two LDS slots; the
// global loads run two stages ahead in two register sets.  When the tiles
// alone would not fill the CUs, K is split in two and both halves are added
// into Y (zeroed by the prep launch): a + b is order-independent, so the
// result stays deterministic.  Blocks are mapped so that each XCD works
// through consecutive work items of one row block: the row block's
// activations stay in that XCD's L2 while its columns stream past.
#include "device_common.h"

namespace int4gemv {
namespace {

constexpr int kTile = 128;      // rows of a block tile
constexpr int kStageK = 64;     // inputs per LDS stage
// LDS stage layout: planes of 128 rows (or BN columns) x 16 bytes.  A
// 16-byte LDS access of a wave runs in 16-lane cycles over the 64 banks (16
// quads of 16 bytes); by the bank-conflict counter on this chip, lanes 0-7
// share a cycle with lanes 24-31 and lanes 8-15 with lanes 16-23 (likewise
// in the upper half), and a cycle whose 16 lanes hit 16 distinct quads costs
// no extra cycle.  A fragment read has each quarter-wave read 16 consecutive
// rows of its own plane, and a stage write has 8 lanes write 8 planes of one
// row (activations) or 2-4 planes of a few columns (B).  Two devices keep
// both kinds on distinct quads:
//  * some planes start 128 bytes (8 quads) past a 256-byte boundary: the lo
//    activation plane of each 8-input block, and the B planes of the
//    stage's second 32-input step;
//  * within an aligned run of 16 rows (columns) the slots are permuted by an
//    XOR with a constant below 8 that depends only on the quarter-wave that
//    reads the plane (a_slot, b_slot), so each lane's read address is one
//    per-lane base plus compile-time offsets.
// Activation block b (planes 2b = hi, 2b + 1 = lo) takes kAPair dwords: hi
// at 0, lo at kALo (2176 bytes, 128 past a 256-byte boundary).
constexpr int kAPair = 2 * kTile * 4 + 64;
constexpr int kALo = kTile * 4 + 32;
constexpr int kABlocks = 8;     // 8-input blocks of a stage (planes 2b = hi, 2b + 1 = lo)
constexpr int kBPlanes = 8;     // B fragment of code word w of the stage: plane w
constexpr int kAWords = kABlocks * kAPair;
constexpr int kThreads = 512;   // 8 waves, 2 per SIMD

// Dword offset of row r of activation plane (block b, half hl) in a stage.
__device__ __forceinline__ int a_slot(int b, int hl, int r) {
  return b * kAPair + hl * kALo + (r ^ (2 * (b & 3))) * 4;
}

// hi and lo of two binary32 values as fp16 pairs, both rounded toward zero.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(a, b));
  const half2_t l = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(a - (float)h[0], b - (float)h[1]));
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

// ------------------------------------------------------------ prep

// Blocks [0, Tp): the split activations of token row blockIdx.x (zeros for
// the pad rows and the pad inputs).  Blocks [Tp, Tp + tiles): one 32 x 32
// tile of the transposed scale table st[g][n] and zero-point table zt[g][n]
// (zt holds zero | zero << 16, the fp16 subnormal pair), zeros outside
// [0, G) x [0, N).
__global__ __launch_bounds__(256) void gemm_prep_kernel(GemmArgs a) {
  __shared__ float red[4];
  __shared__ uint32_t ts[32][33];
  __shared__ uint32_t tz[32][33];
  const int tid = threadIdx.x;
  if ((int64_t)blockIdx.x < a.Tp) {
    const int64_t m = blockIdx.x;
    const bool real = m < a.T;
    const float* x = a.X + m * (int64_t)a.K;
    const int nblk = a.Kp / 8;       // 8-input blocks of the row
    const int nreal = a.K / 8;       // blocks inside K
    u32x4* dst = reinterpret_cast<u32x4*>(a.xs + m * (int64_t)nblk * 8);
    // Rows of up to 512 blocks (K <= 4096) stay in registers between the
    // maximum and the split: thread t holds blocks t and t + 256.
    const bool in_regs = nblk <= 512;
    float4 v[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int b = tid + 256 * h;
      const bool ok = in_regs && real && b < nreal;
      v[2 * h] = ok ? reinterpret_cast<const float4*>(x)[2 * b] : make_float4(0.f, 0.f, 0.f, 0.f);
      v[2 * h + 1] = ok ? reinterpret_cast<const float4*>(x)[2 * b + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float amax = 0.0f;
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    } else if (real) {
      for (int i = tid; i < (a.K >> 2); i += 256) {
        const float4 w = reinterpret_cast<const float4*>(x)[i];
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w))));
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int e = row_exponent(amax);
    if (tid == 0) a.fac[m] = real ? pow2f(24 - e) : 0.0f;
    if (real && a.S > 1)  // the GEMM adds its K parts into Y
      for (int64_t n = tid; n < a.N; n += 256) a.Y[m * a.N + n] = 0.0f;
    const float fe = pow2f(e), fo = pow2f(e - 4);
    // slots 0..7 = inputs 0, 4, 1, 5, 2, 6, 3, 7; odd inputs times 2^-4
    auto split_block = [&](int b, float4 p, float4 r) {
      uint32_t h[4], l[4];
      split2(p.x * fe, r.x * fe, h[0], l[0]);
      split2(p.y * fo, r.y * fo, h[1], l[1]);
      split2(p.z * fe, r.z * fe, h[2], l[2]);
      split2(p.w * fo, r.w * fo, h[3], l[3]);
      dst[2 * b] = u32x4{h[0], h[1], h[2], h[3]};
      dst[2 * b + 1] = u32x4{l[0], l[1], l[2], l[3]};
    };
    if (in_regs) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = tid + 256 * h;
        if (b < nblk) split_block(b, v[2 * h], v[2 * h + 1]);  // zeros past K and in pad rows
      }
    } else {
      for (int b = tid; b < nblk; b += 256) {
        const bool ok = real && b < nreal;
        const float4 p = ok ? reinterpret_cast<const float4*>(x)[2 * b] : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 r = ok ? reinterpret_cast<const float4*>(x)[2 * b + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
        split_block(b, p, r);
      }
    }
    return;
  }
  // Transposed scale / zero-point tile.
  const int64_t t = (int64_t)blockIdx.x - a.Tp;
  const int64_t ntn = a.Np / 32;
  const int64_t gt = t / ntn, nt = t - gt * ntn;
  const int64_t g0 = gt * 32, nb0 = nt * 32;
  const int c = tid & 31, r0 = tid >> 5;
#pragma unroll
  for (int r = r0; r < 32; r += 8) {
    const int64_t n = nb0 + r, g = g0 + c;
    uint32_t sv = 0u, zv = 0u;
    if (n < a.N && g < a.G) {
      sv = fbits(a.s[n * a.G + g]);
      zv = (uint32_t)a.z[n * a.G + g] * 0x00010001u;
    }
    ts[r][c] = sv;
    tz[r][c] = zv;
  }
  __syncthreads();
#pragma unroll
  for (int r = r0; r < 32; r += 8) {
    const int64_t g = g0 + r, n = nb0 + c;
    if (g < a.Gp) {
      a.st[g * a.Np + n] = bitsf(ts[c][r]);
      a.zt[g * a.Np + n] = tz[c][r];
    }
  }
}

// ------------------------------------------------------------ GEMM

// Block tile 128 x BN (BN = 128 or 256): WC = BN / 64 waves across the
// columns, 8 / WC across the rows, each wave 64 columns x (128 / (8 / WC))
// rows as RW x 4 MFMA tiles.
template <int BN>
struct TileShape {
  static constexpr int WC = BN / 64;
  static constexpr int WR = 8 / WC;
  static constexpr int RW = 128 / WR / 16;         // 16-row MFMA tiles per wave
  static constexpr int BPlane = BN * 4;            // dwords per B-fragment plane
  static constexpr int BWords = kBPlanes * BPlane + 32;
  // Dword offset of column c of B plane p (planes 4-7 shifted 128 bytes).
  static __device__ __forceinline__ int b_slot(int p, int c) {
    return p * BPlane + 32 * (p >> 2) + (c ^ (4 * ((p >> 1) & 1))) * 4;
  }
  static constexpr int SCWords = 2 * BN;           // scales, 2 steps x BN columns
  static constexpr int StageWords = kAWords + BWords + SCWords;
  static constexpr int WPT = BN / 64;              // code words per thread per stage (2 or 4)
};

template <int BN>
struct Prefetch {
  u32x4 a[4];                   // activation pieces c = tid + 512 i
  uint32_t w[TileShape<BN>::WPT];  // code words of one column, one step
  uint32_t zh;                  // that column's zero-point pair for the step
  uint32_t sc;                  // one scale of the stage
};

// GSTEPS = group size / 32 when it is 1, 2 or 4 (group ends known at
// compile time), 0 for any other group size.
template <int GSTEPS, int BN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_int4_kernel(GemmArgs a) {
  using TS = TileShape<BN>;
  constexpr int RW = TS::RW;
  extern __shared__ uint32_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int wr = wave % TS::WR, wc = wave / TS::WR;  // rows 16 RW wr .., columns 64 wc ..
  const int l16 = lane & 15, q4 = lane >> 4;

  // XCD-aware order: XCD x (= block id mod 8) takes a contiguous run of
  // work items; items are row block major, then column block, then K part.
  const int64_t nb = a.RB * a.CB * a.S;
  const int64_t b = blockIdx.x;
  const int64_t x8 = b & 7, i8 = b >> 3, q8 = nb >> 3, r8 = nb & 7;
  const int64_t item = x8 * q8 + (x8 < r8 ? x8 : r8) + i8;
  const int64_t rb = item / (a.CB * a.S);
  const int64_t rem = item - rb * a.CB * a.S;
  const int64_t cb = rem / a.S;
  const int part = (int)(rem - cb * a.S);
  const int64_t m0 = rb * kTile, n0 = cb * BN;
  const int nst_all = a.Kp / kStageK;
  // Sums are closed once per stage when a group is one stage (GSTEPS 2);
  // otherwise once per group.
  constexpr bool kStageFlush = GSTEPS == 2;
  // K parts cover whole groups when a group's sums span two stages.
  int per = (nst_all + a.S - 1) / a.S;
  if (GSTEPS == 4 && !kStageFlush) per = (per + 1) & ~1;
  const int st_begin = part * per;
  const int st_end = st_begin + per < nst_all ? st_begin + per : nst_all;
  if (st_begin >= st_end) return;  // an empty K part adds nothing (Y starts at 0)
  const int nsteps = a.Kp / 32;
  const int last_step = 2 * st_end - 1;
  const int gsteps = a.gs / 32;

  // Stage loads (all unconditional, so every wait is exact).  Activations:
  // 128 rows x 256 bytes, thread t takes the 16-byte pieces t + 512 i.
  // Codes: the stage's 8 words of each column are split into WPT-word runs,
  // one per thread, through a buffer resource (columns past N and words past
  // the matrix read 0), with that column's zero point for the run's step.
  // Scales: thread t takes column t % BN of step t / BN (BN = 128: threads
  // t < 256 store).
  const int64_t xrow = a.Kp;  // dwords per token row
  const uint32_t* xsb = a.xs + m0 * xrow;
  constexpr int RUNS = 8 / TS::WPT;  // runs per column (4 or 2)
  const int wcol = tid / RUNS, wrun = tid % RUNS;
  const int wstep = wrun * TS::WPT / 4;
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.q, (short)0, (int)a.qbytes, kBufferWord3);
  const uint32_t qcol_off = (uint32_t)(n0 + wcol) * (uint32_t)(a.K / 2) + (uint32_t)(wrun * TS::WPT * 4);
  const int scstep = (tid / BN) & 1, sccol = tid % BN;
  // Per-lane parts of the LDS offsets; every access adds only compile-time
  // (or wave-uniform) terms to them.  The XOR constants are below 8 and the
  // added row / column terms are multiples of 16, so the terms commute with
  // the XOR; the plane terms stay the same across the planes an access
  // spans (b_slot's shift and XOR depend on p >> 2 and (p >> 1) & 1 only).
  //  * activation store of piece tid & 15 of row tid >> 4 (+ 32 rows per i);
  const int a_st = a_slot((tid & 15) >> 1, tid & 1, tid >> 4);
  //  * B stores of words h and h + 1 (h even) of the lane's run;
  const int b_st0 = TS::b_slot(wrun * TS::WPT, wcol);
  const int b_st2 = TS::b_slot(wrun * TS::WPT + (TS::WPT > 2 ? 2 : 0), wcol);
  //  * fragment reads of block 4 ks + q4: rows 16 RW wr + 16 i + l16 and
  //    columns 64 wc + 16 j + l16.
  const int a_rd = a_slot(q4, 0, 16 * RW * wr + l16);
  const int b_rd = TS::b_slot(q4, 64 * wc + l16);
  auto group_of = [&](int kk) -> int64_t {
    if constexpr (GSTEPS == 1) return kk;
    else if constexpr (GSTEPS == 2) return kk >> 1;
    else if constexpr (GSTEPS == 4) return kk >> 2;
    else return kk / gsteps;
  };

  auto load_stage = [&](int st, Prefetch<BN>& p) {
    const int64_t kw = (int64_t)st * (kStageK / 8) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      const int row = c >> 4, piece = c & 15;
      p.a[i] = *reinterpret_cast<const u32x4*>(xsb + row * xrow + kw + piece * 4);
    }
    const uint32_t off = qcol_off + (uint32_t)(st * (kStageK / 2));
    if constexpr (TS::WPT == 2) {
      const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(qr, off, 0, 0));
      p.w[0] = v[0];
      p.w[1] = v[1];
    } else {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, off, 0, 0));
#pragma unroll
      for (int h = 0; h < 4; ++h) p.w[h] = v[h];
    }
    p.zh = a.zt[group_of(2 * st + wstep) * a.Np + n0 + wcol];
    p.sc = __builtin_bit_cast(uint32_t, a.st[group_of(2 * st + scstep) * a.Np + n0 + sccol]);
  };
  // LDS stage: activation planes (piece p of a row's 256 bytes is plane p),
  // B fragment planes (fragment of step ks, lane group q: plane 4 ks + q),
  // scales [2 steps][BN columns].
  auto store_stage = [&](int slot, const Prefetch<BN>& p) {
    uint32_t* sa = lds + slot * TS::StageWords;
    uint32_t* sb = sa + kAWords;
    uint32_t* ss = sb + TS::BWords;
#pragma unroll
    for (int i = 0; i < 4; ++i)  // piece c & 15 of row c >> 4, c = tid + 512 i
      *reinterpret_cast<u32x4*>(sa + a_st + i * (kThreads / 16) * 4) = p.a[i];
    const half2_t z0 = as_half2(p.zh), z1 = as_half2(p.zh << 4);
#pragma unroll
    for (int h = 0; h < TS::WPT; ++h) {
      const uint32_t w = p.w[h], w8 = w >> 8;
      u32x4 bw;
      bw[0] = __builtin_bit_cast(uint32_t, as_half2(w & 0x000F000Fu) - z0);
      bw[1] = __builtin_bit_cast(uint32_t, as_half2(w & 0x00F000F0u) - z1);
      bw[2] = __builtin_bit_cast(uint32_t, as_half2(w8 & 0x000F000Fu) - z0);
      bw[3] = __builtin_bit_cast(uint32_t, as_half2(w8 & 0x00F000F0u) - z1);
      *reinterpret_cast<u32x4*>(sb + (h < 2 ? b_st0 : b_st2) + (h & 1) * TS::BPlane) = bw;
    }
    if (tid < TS::SCWords) ss[tid] = p.sc;
  };

  const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc[RW][4], tmp[RW][4];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = z4;
      tmp[i][j] = z4;
    }

  // One 32-input step: FIRST = the step opens a group (the products start
  // from 0), LAST = it closes one (its scale multiplies the sums into acc).
  auto step = [&](const uint32_t* sa, const uint32_t* sb, const uint32_t* ss, int ks, bool first,
                  bool last) {
    u32x4 bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const u32x4*>(sb + b_rd + ks * (4 * TS::BPlane + 32) + 64 * j);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const u32x4 ah = *reinterpret_cast<const u32x4*>(sa + a_rd + 4 * ks * kAPair + 64 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        tmp[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ah),
                                                           __builtin_bit_cast(half8_t, bf[j]),
                                                           first ? z4 : tmp[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const u32x4 al = *reinterpret_cast<const u32x4*>(sa + a_rd + 4 * ks * kAPair + kALo + 64 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        tmp[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, al),
                                                           __builtin_bit_cast(half8_t, bf[j]),
                                                           tmp[i][j], 0, 0, 0);
    }
    if (last) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = bitsf(ss[ks * BN + 64 * wc + 16 * j + l16]);
#pragma unroll
        for (int i = 0; i < RW; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc, tmp[i][j][r], acc[i][j][r]);
      }
    }
  };
  // A stage is two steps.  For GSTEPS 1 and 2 the group ends are fixed per
  // step; GSTEPS 4 spans a stage pair (PHASE: the stage's place in it, the
  // parity of its index in the part); the general case tests the step index,
  // and every case closes the sums at the part's last step.  With GSTEPS 4,
  // K is a multiple of 128 and a part an even number of stages, so a part
  // ends on phase 1.  Inlined: as a call it spills.
  auto compute = [&](int slot, int st, int phase) __attribute__((always_inline)) {
    const uint32_t* sa = lds + slot * TS::StageWords;
    const uint32_t* sb = sa + kAWords;
    const uint32_t* ss = sb + TS::BWords;
    const int kk = 2 * st;
    if constexpr (GSTEPS == 1) {
      step(sa, sb, ss, 0, true, true);
      step(sa, sb, ss, 1, true, true);
    } else if constexpr (kStageFlush) {
      step(sa, sb, ss, 0, true, false);
      step(sa, sb, ss, 1, false, true);
    } else if constexpr (GSTEPS == 4) {
      if (phase == 0) {
        step(sa, sb, ss, 0, true, false);
        step(sa, sb, ss, 1, false, false);
      } else {
        step(sa, sb, ss, 0, false, false);
        step(sa, sb, ss, 1, false, true);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k = kk + ks;
        const bool first = k % gsteps == 0 || k == 2 * st_begin;
        const bool last = (k + 1) % gsteps == 0 || k + 1 == nsteps || k == last_step;
        if (first && last) step(sa, sb, ss, ks, true, true);
        else if (first) step(sa, sb, ss, ks, true, false);
        else if (last) step(sa, sb, ss, ks, false, true);
        else step(sa, sb, ss, ks, false, false);
      }
    }
  };

  // Two register prefetch sets: the loads of stage st + 2 are issued while
  // stage st is computed, and stage st + 1 (loaded one iteration earlier)
  // is written to the other LDS slot after it.  Past the part's last stage
  // the loads re-read it, so the count in flight is fixed.  Both tile widths
  // hold the two sets: closing the sums once per group (not per stage)
  // leaves the wide tile the registers for them (252 VGPRs, no scratch).
  auto clamp = [&](int x) { return x < st_end ? x : st_end - 1; };
  Prefetch<BN> p0, p1;
  load_stage(st_begin, p0);
  load_stage(clamp(st_begin + 1), p1);
  store_stage(0, p0);
  __syncthreads();
  int st = st_begin;
  while (true) {
    load_stage(clamp(st + 2), p0);
    compute(0, st, 0);
    store_stage(1, p1);
    __syncthreads();
    if (++st >= st_end) break;
    load_stage(clamp(st + 2), p1);
    compute(1, st, 1);
    store_stage(0, p0);
    __syncthreads();
    if (++st >= st_end) break;
  }

  // Y = total * 2^(24 - e_t); with K split in two, the two halves are added
  // into Y (zeroed by the prep launch), an order-independent sum.
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + 16 * RW * wr + 16 * i + 4 * q4 + r;
      if (row >= a.T) continue;
      const float f = a.fac[row];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + 64 * wc + 16 * j + l16;
        if (col >= a.N) continue;
        if (a.S == 1) a.Y[row * a.N + col] = acc[i][j][r] * f;
        else unsafeAtomicAdd(a.Y + row * a.N + col, acc[i][j][r] * f);
      }
    }
}

// Dynamic LDS beyond 64 KiB must be allowed once per kernel.
template <int GSTEPS, int BN>
hipError_t launch_gemm_kernel(dim3 grid, hipStream_t stream, const GemmArgs& a) {
  static std::atomic<bool> raised{false};  // one per instantiation
  const size_t lds = gemm_lds_bytes(BN);
  if (!raised.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_int4_kernel<GSTEPS, BN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    raised.store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL((gemm_int4_kernel<GSTEPS, BN>), grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_128(dim3 grid, hipStream_t stream, const GemmArgs& a) {
  switch (a.gs) {
    case 32: return launch_gemm_kernel<1, 128>(grid, stream, a);
    case 64: return launch_gemm_kernel<2, 128>(grid, stream, a);
    case 128: return launch_gemm_kernel<4, 128>(grid, stream, a);
    default: return launch_gemm_kernel<0, 128>(grid, stream, a);
  }
}

// The wide tile is built for group sizes 64 and 128 only (gemm_block_cols).
hipError_t launch_gemm_256(dim3 grid, hipStream_t stream, const GemmArgs& a) {
  switch (a.gs) {
    case 64: return launch_gemm_kernel<2, 256>(grid, stream, a);
    case 128: return launch_gemm_kernel<4, 256>(grid, stream, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_block_cols(int64_t Tp, int32_t gs) { return Tp >= 1024 && (gs == 64 || gs == 128) ? 256 : 128; }

size_t gemm_lds_bytes(int bn) {
  return (size_t)2 * (bn == 256 ? TileShape<256>::StageWords : TileShape<128>::StageWords) * sizeof(uint32_t);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  const int64_t prep_blocks = a.Tp + (a.Np / 32) * ((a.Gp + 31) / 32);
  hipLaunchKernelGGL(gemm_prep_kernel, dim3((unsigned)prep_blocks), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(a.RB * a.CB * a.S));
  return a.BN == 256 ? launch_gemm_256(grid, stream, a) : launch_gemm_128(grid, stream, a);
}

}  // namespace int4gemv
