// slice.hip -- the matrix-core kernel for two to eight decode lanes
// (gemv_slice_kernel) and its dispatch.  Sources: [P1] gerbil 1.11.4 ->
// 1.13.0, page 9 (batched INT4 GEMM of the lockstep batch decode and its
// fusion passes); [P4] gerbil 1.12.0 -> 1.13.0, page 12 (the int4 triplet,
// dequant (code - zero) * scale).
#include "device_common.h"

namespace int4gemv {
namespace {

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
// and written to the block's partial table.  After its tiles (at most RT, a
// round), the block adds the waves' partials in wave order and stores Y.
// Every row's arithmetic reads only that row's activations, so a lane's
// outputs never depend on the other lanes.


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
// One wave's share of the kernel: slices of SU units starting at units
// u_first, u_first + u_step, ... below U, over the block's round of tiles.
// SUS is the largest slice size of the launch: it sets the per-wave LDS
// stage and the table stride, which all waves of a block share.  Every wave
// reaches the same barriers, whatever its SU.
template <int SU, int SUS, int GS, int DEPTH, int MODE>
__device__ __forceinline__ void slice_wave(const GemvArgs& a, float4* lds4, int u_first, int u_step) {
  constexpr int NJ = SU / 4;  // load instructions per tile
  constexpr int CS = slice_code_stride(SU);
  constexpr int kStage = slice_stage_words(SUS);
  constexpr int H = SU / 2;  // units each half of a row's lanes converts
  constexpr int NB = 5;      // table chunks per thread loaded ahead of the activations
  static_assert(DEPTH == 2 || DEPTH == 3, "the ring below holds two or three tiles");
  constexpr int NV = MODE == kGated ? 2 : 1;  // weight streams per column tile
  const int M = a.M;
  const int K = a.K;
  const int U = a.U;
  const int G = a.G;
  const int GP = slice_table_stride(G, SUS, GS);
  const int gsu = U / G;
  const int64_t N = a.N;
  const int lane = threadIdx.x & 63;
  const int hi4 = lane >> 4;   // matrix layout: k group / D row group
  const int lo16 = lane & 15;  // matrix layout: column
  const int wave = uniform_int(threadIdx.x >> 6);
  const int W = a.block_threads >> 6;
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

  // One round of tiles per block: the planner gives a block at most RT
  // tiles, with more blocks than the device holds at once where the columns
  // need more (a loop over rounds here costs every launch time, through the
  // code generated around it, even when it runs once).  The clamp only keeps
  // the tables inside the LDS should a launch break that rule.
  {
    const int r0 = 0;
    const int rn = ntile < RT ? ntile : RT;

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
      const uint32_t off = (uint32_t)(threadIdx.x + b * a.block_threads) * 16u;
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
    for (int u0 = u_first; u0 < U; u0 += u_step) {
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
        for (int b = 0; b < NB; ++b) table_put(tid + b * a.block_threads, tsv[b], tzv[b]);
        for (int c = tid + NB * a.block_threads; c < nchunk; c += a.block_threads) {
          const u32x4 sv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)c * 16u, 0, kLoadNonTemporal));
          const u32x4 zv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, (uint32_t)c * 16u, 0, kLoadNonTemporal));
          table_put(c, sv, zv);
        }
        if constexpr (NV == 2) {  // the up stream's table
          const auto rs1 = table_rsrc(sbase(1));
          const auto rz1 = table_rsrc(zbase(1));
          for (int c = tid; c < nchunk; c += a.block_threads) {
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
    for (int o = threadIdx.x; o < nout; o += a.block_threads) {
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
  }
}

template <int SU, int GS, int DEPTH, int MODE>
__global__ __launch_bounds__(64 * kSliceMaxWaves) void gemv_slice_kernel(GemvArgs a) {
  extern __shared__ float4 lds4[];
  const int wave = uniform_int(threadIdx.x >> 6);
  const int W = a.block_threads >> 6;
  slice_wave<SU, SU, GS, DEPTH, MODE>(a, lds4, SU * wave, SU * W);
}

// One slice per wave of two sizes, whole cache lines each: waves
// [0, a.mix24) take 24 units (384 bytes of a column), the others 16 units
// (256 bytes), so no two waves split a line of a column.  Waves w and
// w + 4 share a SIMD, so with four of each every SIMD holds 40 units.  Both
// sizes keep two tiles in flight (three for the 16-unit waves measured
// slower here).
template <int GS, int MODE>
__global__ __launch_bounds__(64 * kSliceMaxWaves) void gemv_slice_mixed_kernel(GemvArgs a) {
  extern __shared__ float4 lds4[];
  const int wave = uniform_int(threadIdx.x >> 6);
  const int na = a.mix24;
  constexpr int kOnce = 1 << 30;  // one slice per wave
  if (wave < na) slice_wave<24, 24, GS, 2, MODE>(a, lds4, 24 * wave, kOnce);
  else slice_wave<16, 24, GS, 2, MODE>(a, lds4, 24 * na + 16 * (wave - na), kOnce);
}

template <int MODE>
hipError_t dispatch_slice_mixed(const GemvArgs& a, const LaunchShape& s, hipStream_t st, int* occ) {
  static std::atomic<bool> raised1{false}, raised2{false}, raised4{false}, raised0{false};
  switch (slice_class(a.U / a.G)) {
    case 1: return launch_or_query(gemv_slice_mixed_kernel<1, MODE>, raised1, a, s, st, occ);
    case 2: return launch_or_query(gemv_slice_mixed_kernel<2, MODE>, raised2, a, s, st, occ);
    case 4: return launch_or_query(gemv_slice_mixed_kernel<4, MODE>, raised4, a, s, st, occ);
    default: return launch_or_query(gemv_slice_mixed_kernel<0, MODE>, raised0, a, s, st, occ);
  }
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
  if (a.mix24 > 0) return dispatch_slice_mixed<MODE>(a, s, st, occ);
  if (a.su == 24) return dispatch_slice_su<24, 2, MODE>(a, s, st, occ);
  // Two tiles of loads in flight at every slice size: three measured 7-11%
  // slower at 16 and 20 units.
  if (a.su == 20) return dispatch_slice_su<20, 2, MODE>(a, s, st, occ);
  return dispatch_slice_su<16, 2, MODE>(a, s, st, occ);
}

}  // namespace

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

}  // namespace int4gemv
