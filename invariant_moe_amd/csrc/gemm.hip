// Grouped expert GEMM kernels: the bf16 / MXFP4 MFMA tiles of gemm_core.hpp
// launched one tile per workgroup from a tile table, an fp32 VALU kernel, the
// FP4 x FP8 (W4A8) kernel, and the host planner that picks the tile shapes.
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace moe {

// bf16 / MXFP4 MFMA kernel: one tile per workgroup, from the tile table.
template <int BM, int BN, int WM, int WN, int P, bool GATED, bool FP4>
__global__ __launch_bounds__(64 * WM * WN, 2) void k_grouped_gemm_bf16(GemmArgs args) {
  __shared__ __align__(16) unsigned char smem[gemm_smem_bytes<BM, BN, GATED, FP4>()];
  TileInfo ti;
  if (!read_tile(args, blockIdx.x, BM, ti)) return;
  gemm_tile_bf16<BM, BN, WM, WN, P, GATED, FP4>(args.seg[ti.seg], ti, args.glu, smem);
}

// ---------------------------------------------------------------------------
// fp32 kernel (VALU): each output element is one fmaf chain over K in
// increasing order from +0, whatever the tile.  Tile 16 rows x 16 features.
// ---------------------------------------------------------------------------
template <bool GATED>
__global__ __launch_bounds__(256) void k_grouped_gemm_f32(GemmArgs args) {
  constexpr int BM = 16, BN = 16, KC = 32;
  constexpr int NMAT = GATED ? 2 : 1;
  __shared__ float As[BM][KC + 1];
  __shared__ float Bs[NMAT][BN][KC + 1];
  TileInfo ti;
  if (!read_tile(args, blockIdx.x, BM, ti)) return;
  const GemmSeg& s = args.seg[ti.seg];
  const int K = s.K, N = s.N;
  const int tid = threadIdx.x;
  const int r = tid / 16, n = tid % 16;
  float acc[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) acc[m] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += KC) {
    __syncthreads();
    for (int i = tid; i < BM * KC; i += 256) {
      const int rr = min(i / KC, ti.rows - 1), kk = i % KC;
      const int64_t row = ti.row0 + rr;
      const int64_t src = s.a_index ? (int64_t)s.a_index[row] : row;
      As[i / KC][kk] = (k0 + kk < K) ? static_cast<const float*>(s.A)[src * K + k0 + kk] : 0.0f;
    }
    for (int i = tid; i < NMAT * BN * KC; i += 256) {
      const int m = i / (BN * KC), nn = min(ti.n0 + (i / KC) % BN, N - 1), kk = i % KC;
      const float* W = static_cast<const float*>(m ? s.W1 : s.W0);
      Bs[m][(i / KC) % BN][kk] = (k0 + kk < K) ? W[((int64_t)ti.g * N + nn) * K + k0 + kk] : 0.0f;
    }
    __syncthreads();
    const int kc = min(KC, K - k0);
    for (int kk = 0; kk < kc; ++kk)
#pragma unroll
      for (int m = 0; m < NMAT; ++m) acc[m] = __builtin_fmaf(As[r][kk], Bs[m][n][kk], acc[m]);
  }
  if (r < ti.rows && ti.n0 + n < N) {
    const float v = GATED ? glu_act<LibMath>(acc[0], acc[NMAT - 1], args.glu) : acc[0];
    static_cast<float*>(s.out)[(ti.row0 + r) * (int64_t)N + ti.n0 + n] = v;
  }
}

// ---------------------------------------------------------------------------
// FP4 x FP8 kernel (W4A8; the DeepSeek-V4 walkthrough, section 6.2, runs FP4
// expert weights in an FP8 GEMM): MXFP4 weights as operand A and MXFP8 token
// rows (E4M3 + E8M0 per 32, quant.hip) as operand B of gfx950's
// v_mfma_scale_f32_16x16x128_f8f6f4, which applies both E8M0 block scales
// itself.  K steps by 128 in increasing order from a zero accumulator, one
// instruction per (16 features, 16 tokens, 128 of K): one chain per output
// element whatever the tile, so T changes no bit.
// Operand layout (measured on MI355X with one-hot operands):
//   A (E2M1, 4 VGPRs): lane 16g + i holds weight row i, K 32g .. 32g+31,
//       element e in nibble e (low nibble first);
//   B (E4M3, 8 VGPRs): lane 16g + j holds token row j, K 16g .. 16g+15 in
//       bytes 0..15 and K 64+16g .. 64+16g+15 in bytes 16..31;
//   scales: lane 16b + i (A) or 16b + j (B) passes the E8M0 byte of K block b
//       (K 32b .. 32b+31) of its row in bits 0..7;
//   result: lane l, element v is feature 4(l/16) + v, token l % 16, as for
//       the bf16 MFMA above.
// LDS: token rows of a stage are 128 bytes, weight rows 64 bytes paired into
// 128-byte lines; 16-byte chunks XOR-swizzled by line as in lds_off.
// Weight loads are plain: non-temporal ones (nt_load16) measured 23 % slower
// here with 8 rows per expert.
// ---------------------------------------------------------------------------
constexpr int KQ = 128;  // K per stage

__device__ __forceinline__ int lds_line_off(int line, int chunk) {
  return line * 128 + ((chunk ^ (line & 7)) << 4);
}

template <int BM, int BN, int WM, int WN, bool GATED, int MINW>
__global__ __launch_bounds__(64 * WM * WN, MINW) void k_grouped_gemm_w4a8(GemmArgs args) {
  constexpr int NT = 64 * WM * WN;
  constexpr int NMAT = GATED ? 2 : 1;
  constexpr int TBW = BM / 16 / WM;
  constexpr int NBW = BN / 16 / WN;
  static_assert(TBW >= 1 && NBW >= 1, "tile too small for the wave grid");
  constexpr int XCH = BM * 8;         // 16-byte chunks of a token stage
  constexpr int WCH = NMAT * BN * 4;  // 16-byte chunks of a weight stage
  constexpr int XPT = (XCH + NT - 1) / NT;
  constexpr int WPT = (WCH + NT - 1) / NT;
  __shared__ __align__(16) uint8_t sx[2][BM * 128];
  __shared__ __align__(16) uint8_t sw[2][NMAT * BN * 64];
  __shared__ uint32_t ssx[2][BM];
  __shared__ uint32_t ssw[2][NMAT * BN];

  TileInfo ti;
  if (!read_tile(args, blockIdx.x, BM, ti)) return;
  const GemmSeg& s = args.seg[ti.seg];
  const int K = s.K, N = s.N, nst = K / KQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // In 128-row tiles a wave whose rows all lie past the tile's valid rows
  // issues no MFMA (it still loads and stages its share of each stage): an
  // expert's last row tile is often less than half full.  Measured on the
  // hash-routed MXFP4 layer (D=7168, E=256, k=8, I=2048) at T=8192, 256 rows
  // per expert: gate/up 3.78 -> 3.40 ms.  At 64 rows per expert (T=2048)
  // these tiles measured the same as 64 x 128 on 2 x 2 waves.
  const bool active = BM < 128 || wm * TBW * 16 < ti.rows;  // uniform per wave
  const uint8_t* X = static_cast<const uint8_t*>(s.A);

  // sources: token chunk c = (row, 16-byte chunk), weight chunk c = (mat, row, chunk)
  const uint8_t* xsrc[XPT];
  const uint8_t* wsrc[WPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = min(tid + i * NT, XCH - 1);
    const int r = min(c / 8, ti.rows - 1);
    int64_t row = ti.row0 + r;
    if (s.a_index) row = s.a_index[row];
    xsrc[i] = X + row * K + (c % 8) * 16;
  }
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int c = min(tid + i * NT, WCH - 1);
    const int mat = c / (BN * 4), n = (c / 4) % BN;
    const int nn = min(ti.n0 + n, N - 1);
    const uint8_t* base = static_cast<const uint8_t*>(mat ? s.W1 : s.W0);
    wsrc[i] = base + ((int64_t)ti.g * N + nn) * (K / 2) + (c % 4) * 16;
  }
  // scale words (the 4 E8M0 bytes of one row's stage): word w < BM is token
  // row w, word BM + c weight row c; thread t takes words t + i * NT (words
  // past the end read token row 0's word and are not stored)
  constexpr int SW = BM + NMAT * BN;
  constexpr int SPT = (SW + NT - 1) / NT;
  const uint8_t* scsrc[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int w = tid + i * NT;
    if (w >= BM && w < SW) {
      const int c = w - BM, mat = c / BN, nn = min(ti.n0 + c % BN, N - 1);
      scsrc[i] = (mat ? s.S1 : s.S0) + ((int64_t)ti.g * N + nn) * (K / 32);
    } else {
      int64_t row = ti.row0 + (w < BM ? min(w, ti.rows - 1) : 0);
      if (s.a_index) row = s.a_index[row];
      scsrc[i] = s.AS + row * (K / 32);
    }
  }

  f32x4_t acc[NMAT][NBW][TBW];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int tb = 0; tb < TBW; ++tb) acc[m][nb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native: plain loads and stores
  u32x4 xr[XPT], wr[WPT];
  // Scale words of four consecutive stages (stage kt's word in slot kt % 4),
  // loaded together every fourth stage: a row's scales span K / 32 bytes,
  // and reading one 4-byte word of a line per stage let the line leave L2
  // between stages (measured on the hash-routed MXFP4 layer, D=7168, E=256,
  // k=8, I=2048, at T=2048: gate/up HBM reads 5.91 -> 5.41 GB, 1.34 ->
  // 1.27 ms).  Loading the weight codes of two stages together (the two
  // 64-byte halves of a row's line) read 5.13 GB but took 1.38 ms, and
  // 6.13 GB and 1.62 ms with non-temporal loads.
  uint32_t sc[SPT][4];
  auto sload = [&](int kt) {  // kt % 4 == 0; words past the last stage are not loaded
#pragma unroll
    for (int i = 0; i < SPT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (kt + j < nst) sc[i][j] = *reinterpret_cast<const uint32_t*>(scsrc[i] + (kt + j) * 4);
  };
  // stage loads into registers, then into LDS (the arrays are passed, not
  // captured, so that they stay in registers)
  auto gload = [&](u32x4 (&xq)[XPT], u32x4 (&wq)[WPT], int kt) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) xq[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + kt * KQ);
#pragma unroll
    for (int i = 0; i < WPT; ++i) wq[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + kt * (KQ / 2));
  };
  auto lstore = [&](const u32x4 (&xq)[XPT], const u32x4 (&wq)[WPT], int slot, int buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * NT;
      if (c < XCH)
        *reinterpret_cast<u32x4*>(&sx[buf][lds_line_off(c / 8, c % 8)]) = xq[i];
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + i * NT;
      if (c < WCH) {
        const int wrow = c / 4;  // mat * BN + n
        *reinterpret_cast<u32x4*>(&sw[buf][lds_line_off(wrow >> 1, ((wrow & 1) << 2) | (c % 4))]) =
            wq[i];
      }
    }
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int w = tid + i * NT;
      if (w < BM)
        ssx[buf][w] = sc[i][slot];
      else if (w < SW)
        ssw[buf][w - BM] = sc[i][slot];
    }
  };
  const int g4 = lane >> 4, r16 = lane & 15;
  auto compute = [&](int buf) {
    typedef int v8i __attribute__((ext_vector_type(8)));
    v8i bfr[TBW];
    int bsc[TBW];
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      const int trow = (wm * TBW + tb) * 16 + r16;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&sx[buf][lds_line_off(trow, g4)]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&sx[buf][lds_line_off(trow, 4 + g4)]);
      bfr[tb] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      bsc[tb] = (int)((ssx[buf][trow] >> (8 * g4)) & 0xffu);
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int wrow = m * BN + (wn * NBW + nb) * 16 + r16;
        const u32x4 q =
            *reinterpret_cast<const u32x4*>(&sw[buf][lds_line_off(wrow >> 1, ((wrow & 1) << 2) | g4)]);
        const v8i afr = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        const int asc = (int)((ssw[buf][wrow] >> (8 * g4)) & 0xffu);
#pragma unroll
        for (int tb = 0; tb < TBW; ++tb)
          acc[m][nb][tb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              afr, bfr[tb], acc[m][nb][tb], 4, 0, 0, asc, 0, bsc[tb]);
      }
  };

  sload(0);
  gload(xr, wr, 0);
  lstore(xr, wr, 0, 0);
  __syncthreads();
  // four stages per iteration, so that the scale slot of each is static
  for (int k4 = 0; k4 < nst; k4 += 4) {
    static_for<0, 4>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      const int kt = k4 + q;
      if (kt < nst) {  // uniform
        const bool more = kt + 1 < nst;
        if (more) {
          if (q == 3) sload(kt + 1);  // the next four stages' scale words
          gload(xr, wr, kt + 1);
        }
        if (active) compute(kt & 1);
        if (more) lstore(xr, wr, (q + 1) & 3, (kt + 1) & 1);
        __syncthreads();
      }
    });
  }

  // epilogue (as the bf16 kernel): features n = base + 4*(lane/16) + v of token
  // row base + lane%16 -> one 8-byte store of 4 bf16
  uint16_t* out = static_cast<uint16_t*>(s.out);
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      const int r = (wm * TBW + tb) * 16 + r16;
      const int n = ti.n0 + (wn * NBW + nb) * 16 + 4 * g4;
      if (r < ti.rows && n < N) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = GATED ? glu_act<FastMath>(acc[0][nb][tb][i], acc[NMAT - 1][nb][tb][i], args.glu)
                       : acc[0][nb][tb][i];
        uint2 pk = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        *reinterpret_cast<uint2*>(out + (ti.row0 + r) * (int64_t)N + n) = pk;
      }
    }
}

// ---------------------------------------------------------------------------
// Host planning and launch.  The grid of a launch is an upper bound of its
// tile count known without a device sync; surplus workgroups read an empty
// descriptor and exit.
// ---------------------------------------------------------------------------
static int64_t seg_tile_bound(const SegShape& s, int BM, int BN) {
  const int64_t nt = (s.N + BN - 1) / BN;
  if (!s.grouped) return ((s.M + BM - 1) / BM) * nt;
  // sum_g ceil(M_g/BM) <= ceil(R/BM) + (number of non-empty groups)
  const int64_t nonempty = s.M < s.G ? s.M : s.G;
  return ((s.M + BM - 1) / BM + nonempty) * nt;
}

struct LaunchEvents {
  hipEvent_t start, stop;
};

template <int BM, int BN, int WM, int WN, int P, bool GATED, bool FP4>
static hipError_t launch_one(const GemmArgs& a, int64_t grid, hipStream_t st, LaunchEvents ev) {
  hipExtLaunchKernelGGL((k_grouped_gemm_bf16<BM, BN, WM, WN, P, GATED, FP4>),
                        dim3((unsigned)grid), dim3(64 * WM * WN), 0, st, ev.start, ev.stop, 0, a);
  return hipGetLastError();
}

// Tile configurations (BM token rows, BN features, WM x WN waves, P stages in
// flight).  Every configuration computes identical bits (same MFMA chain per
// output element); they differ in occupancy, workgroup count and reuse.
enum TileCfg {
  TILE_16x16_1x1_P4 = 0,  // decode gate/up: one wave per workgroup, ~4.5 per CU
  TILE_16x64_1x4_P4,
  TILE_32x64_1x4_P4,
  TILE_64x32_4x1_P2,      // tens of rows per expert
  TILE_64x64_4x1_P2,
  TILE_128x128_2x4_P2,    // gate/up above 96 rows per expert (MXFP4: above 16), 8 waves
  TILE_128x256_2x4_P2,    // down, the same brackets, 8 waves
  TILE_COUNT,
  TILE_F32 = 100,         // fp32 VALU kernel, 16 x 16 tiles
  TILE_W4A8 = 200,        // FP4 x FP8 kernel, 64 x 64 tiles on 2 x 2 waves
  TILE_W4A8_N128 = 201,   // FP4 x FP8 kernel, 64 x 128 tiles on 2 x 2 waves
  TILE_W4A8_128 = 202     // FP4 x FP8 kernel, 128 x 128 tiles on 2 x 4 waves
};

struct TileShape {
  int BM, BN;
};

static TileShape tile_shape(int cfg) {
  switch (cfg) {
    case TILE_16x16_1x1_P4: return {16, 16};
    case TILE_16x64_1x4_P4: return {16, 64};
    case TILE_32x64_1x4_P4: return {32, 64};
    case TILE_64x32_4x1_P2: return {64, 32};
    case TILE_64x64_4x1_P2: return {64, 64};
    case TILE_128x128_2x4_P2: return {128, 128};
    case TILE_128x256_2x4_P2: return {128, 256};
    case TILE_W4A8: return {64, 64};
    case TILE_W4A8_N128: return {64, 128};
    case TILE_W4A8_128: return {128, 128};
    default: return {16, 16};  // TILE_F32
  }
}

// The (configuration, branch, weight format) combinations the planner can
// select: every configuration for either format, since a launch of one
// format carries the configuration chosen for the other when shared and
// routed experts come in different formats.
template <bool FP4>
static hipError_t launch_tile_cfg(int cfg, const GemmArgs& a, bool gated, int64_t grid,
                                  hipStream_t st, LaunchEvents ev) {
  if (gated) {
    switch (cfg) {
      case TILE_16x16_1x1_P4: return launch_one<16, 16, 1, 1, 4, true, FP4>(a, grid, st, ev);
      case TILE_32x64_1x4_P4: return launch_one<32, 64, 1, 4, 4, true, FP4>(a, grid, st, ev);
      case TILE_64x32_4x1_P2: return launch_one<64, 32, 4, 1, 2, true, FP4>(a, grid, st, ev);
      case TILE_128x128_2x4_P2: return launch_one<128, 128, 2, 4, 2, true, FP4>(a, grid, st, ev);
      default: break;
    }
  } else {
    switch (cfg) {
      case TILE_16x64_1x4_P4: return launch_one<16, 64, 1, 4, 4, false, FP4>(a, grid, st, ev);
      case TILE_32x64_1x4_P4: return launch_one<32, 64, 1, 4, 4, false, FP4>(a, grid, st, ev);
      case TILE_64x64_4x1_P2: return launch_one<64, 64, 4, 1, 2, false, FP4>(a, grid, st, ev);
      case TILE_128x256_2x4_P2: return launch_one<128, 256, 2, 4, 2, false, FP4>(a, grid, st, ev);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

// Host-side choice from the average rows per group (no device sync), from
// measured sweeps on MI355X (all choices give identical bits).
static int pick_tile_cfg(bool gated, int64_t rows_per_group_hint, bool fp4) {
  // At most two rows per expert (decode): the gate/up launch in single-wave
  // workgroups spreads the weight stream evenly over the CUs (measured 3-4 %
  // faster than two-wave 16 x 32 tiles from T=1 to T=4).  Down tiles of
  // 16 x 16 and 16 x 32 measured the same as 16 x 64 at T=1; single-wave tiles
  // that load both MFMA operands straight into registers (16-byte pieces of
  // 16 rows per instruction, no LDS) streamed 30 % slower.
  if (rows_per_group_hint <= 2) return gated ? TILE_16x16_1x1_P4 : TILE_16x64_1x4_P4;
  if (rows_per_group_hint <= 16) return TILE_32x64_1x4_P4;
  // MXFP4 weights: 128-row tiles on 8 waves, those of the empty row block
  // loading and staging for the others.  Measured at 64 rows per expert (the
  // hash-routed MXFP4 layer, T=2048, D=7168, E=256, k=8, I=2048; gate/up,
  // down): 1.97 and 1.00 ms; 128 x 64 gate/up and
  // 128 x 128 down on 2 x 2 waves 1.99 and 1.05 ms; 64 x 128 on 1 x 4 waves
  // (each wave decodes and reads all 64 token rows) 2.69 ms; 64 x 64 on 2 x 2
  // waves, where no wave idles, 2.45 ms.
  if (fp4 && rows_per_group_hint <= 96) return gated ? TILE_128x128_2x4_P2 : TILE_128x256_2x4_P2;
  if (rows_per_group_hint <= 96) return gated ? TILE_64x32_4x1_P2 : TILE_64x64_4x1_P2;
  // many rows per expert: gate/up 128 x 128 and down 128 x 256 tiles, both
  // on 8 waves, two per SIMD (the down GEMM of the DeepSeek-V3-shaped layer,
  // T=4096, D=7168, E=256, k=8, I=2048: 1.84 ms, against
  // 1.94 ms for 128 x 128 on 4 waves and 2.23 ms for 128 x 128 on 8; 5.33
  // against 5.64 ms at T=16384).
  // Stages brought into LDS by direct loads (global_load_lds_dwordx4, no
  // staging registers, a 3- or 4-stage LDS ring) measured no faster on
  // that layer: gate/up 3.35 ms on the 128 x 128 tile with 3 stages, down
  // 2.16 ms on 8 waves with 4; 64-row tiles with a 4-stage ring of mostly
  // weights, 4.22 and 2.20 ms; register-path 64 x 64 (gate/up) and 64 x 128
  // (down) tiles on 2 x 2 waves, three workgroups per CU, 4.48 and 2.27 ms.
  return gated ? TILE_128x128_2x4_P2 : TILE_128x256_2x4_P2;
}

GemmPlan plan_grouped_gemm(const SegShape* segs, int nseg, bool gated, int act,
                           int64_t rows_per_group_hint) {
  GemmPlan p{};
  p.valid = true;
  p.gated = gated;
  p.act = act;
  p.nseg = nseg;
  for (int i = 0; i < nseg; ++i) p.seg[i] = segs[i];
  const int cfg = act == MOE_F32 ? (int)TILE_F32
                                  : pick_tile_cfg(gated, rows_per_group_hint, segs[0].wfmt != 0);
  // Segments with the same weight format share one launch; a mixed pair
  // (MXFP4 routed experts + bf16 shared expert) takes one launch per format.
  const bool split = nseg == 2 && segs[0].wfmt != segs[1].wfmt;
  const int nl = split ? 2 : 1;
  for (int l = 0; l < nl; ++l) {
    PlanLaunch& L = p.l[p.n];
    L.seg_mask = split ? (1 << l) : (nseg == 2 ? 3 : 1);
    L.cfg = cfg;  // every tile configuration is compiled for both weight formats
    const TileShape ls = tile_shape(L.cfg);
    L.BM = ls.BM;
    L.BN = ls.BN;
    int64_t tiles = 0;
    for (int i = 0; i < nseg; ++i)
      if (L.seg_mask & (1 << i)) tiles += seg_tile_bound(segs[i], ls.BM, ls.BN);
    L.grid = (tiles + 7) / 8 * 8;
    if (L.grid > 0x7ffffff8) p.valid = false;  // one launch holds < 2^31 workgroups
    if (L.grid > 0) ++p.n;
  }
  return p;
}

GemmPlan plan_w4a8_gemm(const SegShape& seg, bool gated, int64_t rows_per_group_hint) {
  GemmPlan p{};
  p.valid = true;
  p.gated = gated;
  p.act = MOE_BF16;
  p.nseg = 1;
  p.seg[0] = seg;
  PlanLaunch& L = p.l[0];
  L.seg_mask = 1;
  // Measured at D=7168, I=2048: 64 x 64 is the fastest at 8 rows per expert
  // (most workgroups for the weight stream), 64 x 128 at 64 rows (half the
  // token re-reads, -12 %), 128 x 128 at 256 rows.  A 64 x 256 tile on 2 x 4
  // waves at 64 rows lost 8 % to 64 x 128 (fewer workgroups per weight byte).
  L.cfg = rows_per_group_hint > 96   ? TILE_W4A8_128
          : rows_per_group_hint > 16 ? TILE_W4A8_N128
                                     : TILE_W4A8;
  const TileShape ts = tile_shape(L.cfg);
  L.BM = ts.BM;
  L.BN = ts.BN;
  L.grid = (seg_tile_bound(seg, ts.BM, ts.BN) + 7) / 8 * 8;
  if (L.grid > 0x7ffffff8) p.valid = false;
  if (L.grid > 0) p.n = 1;
  return p;
}

int64_t plan_table_entries(const GemmPlan& p) {
  int64_t n = 0;
  for (int i = 0; i < p.n; ++i) n += p.l[i].grid;
  return n;
}

bool plan_tile_jobs(const GemmPlan& p, int4* tables, TileJobs& jobs) {
  for (int i = 0; i < p.n; ++i) {
    const PlanLaunch& L = p.l[i];
    bool grouped = false;
    for (int sg = 0; sg < p.nseg; ++sg)
      if ((L.seg_mask & (1 << sg)) && p.seg[sg].grouped) grouped = true;
    if (jobs.n == MOE_MAX_TILE_JOBS) return false;
    if (grouped) {  // grouped segments of one call share their m-tile counts
      if (jobs.BM > 0 && jobs.BM != L.BM) return false;
      jobs.BM = L.BM;
    }
    TileJob& J = jobs.job[jobs.n++];
    J = TileJob{};
    J.table = tables;
    J.grid = L.grid;
    J.BM = L.BM;
    J.BN = L.BN;
    for (int sg = 0; sg < p.nseg; ++sg) {
      if (!(L.seg_mask & (1 << sg))) continue;
      J.grouped[J.nseg] = p.seg[sg].grouped ? 1 : 0;
      J.M[J.nseg] = p.seg[sg].M;
      J.N[J.nseg] = p.seg[sg].N;
      ++J.nseg;
    }
    tables += L.grid;
  }
  return true;
}

hipError_t launch_grouped_gemm(const GemmPlan& p, const GemmArgs& a, int4* tables,
                               hipStream_t st, hipEvent_t ev_start, hipEvent_t ev_stop) {
  for (int i = 0; i < p.n; ++i) {
    const PlanLaunch& L = p.l[i];
    GemmArgs one{};
    for (int sg = 0; sg < a.nseg; ++sg)
      if (L.seg_mask & (1 << sg)) one.seg[one.nseg++] = a.seg[sg];
    one.tiles = tables;
    one.glu = a.glu;
    const LaunchEvents ev{i == 0 ? ev_start : nullptr, i == p.n - 1 ? ev_stop : nullptr};
    hipError_t e;
    if (L.cfg == TILE_W4A8 || L.cfg == TILE_W4A8_N128 || L.cfg == TILE_W4A8_128) {
      const dim3 g((unsigned)L.grid);
      if (L.cfg == TILE_W4A8 && p.gated)
        hipExtLaunchKernelGGL((k_grouped_gemm_w4a8<64, 64, 2, 2, true, 2>), g, dim3(256), 0, st,
                              ev.start, ev.stop, 0, one);
      else if (L.cfg == TILE_W4A8)
        hipExtLaunchKernelGGL((k_grouped_gemm_w4a8<64, 64, 2, 2, false, 2>), g, dim3(256), 0, st,
                              ev.start, ev.stop, 0, one);
      else if (L.cfg == TILE_W4A8_N128 && p.gated)
        hipExtLaunchKernelGGL((k_grouped_gemm_w4a8<64, 128, 2, 2, true, 2>), g, dim3(256), 0, st,
                              ev.start, ev.stop, 0, one);
      else if (L.cfg == TILE_W4A8_N128)
        hipExtLaunchKernelGGL((k_grouped_gemm_w4a8<64, 128, 2, 2, false, 2>), g, dim3(256), 0, st,
                              ev.start, ev.stop, 0, one);
      else if (p.gated)
        hipExtLaunchKernelGGL((k_grouped_gemm_w4a8<128, 128, 2, 4, true, 1>), g, dim3(512), 0, st,
                              ev.start, ev.stop, 0, one);
      else
        hipExtLaunchKernelGGL((k_grouped_gemm_w4a8<128, 128, 2, 4, false, 1>), g, dim3(512), 0, st,
                              ev.start, ev.stop, 0, one);
      e = hipGetLastError();
    } else if (L.cfg == TILE_F32) {
      if (p.gated)
        hipExtLaunchKernelGGL(k_grouped_gemm_f32<true>, dim3((unsigned)L.grid), dim3(256), 0, st,
                              ev.start, ev.stop, 0, one);
      else
        hipExtLaunchKernelGGL(k_grouped_gemm_f32<false>, dim3((unsigned)L.grid), dim3(256), 0, st,
                              ev.start, ev.stop, 0, one);
      e = hipGetLastError();
    } else {
      e = one.seg[0].wfmt ? launch_tile_cfg<true>(L.cfg, one, p.gated, L.grid, st, ev)
                          : launch_tile_cfg<false>(L.cfg, one, p.gated, L.grid, st, ev);
    }
    if (e != hipSuccess) return e;
    tables += L.grid;
  }
  return hipSuccess;
}

// Standalone table builder (caller-supplied offsets): one workgroup.
__global__ __launch_bounds__(1024) void k_tile_tables(const int32_t* __restrict__ offsets, int E,
                                                      TileJobs jobs) {
  __shared__ int soff[MOE_MAX_EXPERTS + 1];
  __shared__ int mpre[MOE_MAX_EXPERTS + 1];
  __shared__ int unused[MOE_MAX_EXPERTS + 1];
  __shared__ int wsum[2 * (1024 / 64)];
  __shared__ int omap[kTileOwnerMax];
  for (int e = threadIdx.x; e <= E; e += 1024) soff[e] = offsets[e];
  __syncthreads();
  // m-tile counts of the grouped segment (the same rows in every job)
  int64_t M = 0;
  for (int j = 0; j < jobs.n; ++j)
    for (int sg = 0; sg < jobs.job[j].nseg; ++sg)
      if (jobs.job[j].grouped[sg]) M = jobs.job[j].M[sg];
  for (int e = threadIdx.x; e < E; e += 1024) {
    mpre[e] = jobs.BM > 0 ? (tile_group_rows(soff, e, M) + jobs.BM - 1) / jobs.BM : 0;
    unused[e] = 0;
  }
  __syncthreads();
  tile_scan2<1024>(mpre, unused, E, wsum);
  const bool map = build_tile_owner<1024>(mpre, E, omap);
  build_tile_tables<1024>(jobs, soff, mpre, map ? omap : nullptr, E, 0, 1);
}

hipError_t launch_tile_tables(const int32_t* offsets, int E, const TileJobs& jobs, hipStream_t s) {
  if (jobs.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_tile_tables, dim3(1), dim3(1024), 0, s, offsets, E, jobs);
  return hipGetLastError();
}

}  // namespace moe
