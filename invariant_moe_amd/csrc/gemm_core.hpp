// Grouped expert GEMM tiles with the SwiGLU epilogue, as device functions of
// the calling workgroup (used by the grouped-GEMM kernels and by the
// single-launch layer kernel).
//
// Expert FFN: g = W_gate a, u = W_up a, h = SiLU(g) * u, o = W_down h
// (SwiGLU, "6 基建与训练稳定性优化" section 6.5; gate and up branches, forum
// article feedbbs.com/linuxdo/72580, GLU section).  Every GEMM sees its whole
// K in one workgroup (no split sums: the LongCat parity article,
// "美团把训练和推理的概率做到逐位相同"), so each output element is one fixed
// chain of MFMA steps over K.
//
// Batch invariance.  All bf16 tiles here use ONE instruction,
// v_mfma_f32_16x16x32_bf16, with the weight tile as operand A (16 output
// features) and the token tile as operand B (16 rows), K stepped by 32 in
// increasing order into an accumulator that starts at 0.  An output element
// depends only on its own weight row and token row and on this fixed chain,
// never on the other rows of its tile, the tile shape, the number of rows of
// its expert, or T.  The tile variants differ only in how many blocks a
// workgroup holds, so they give identical bits.
//
// MXFP4 weights (E2M1 codes + one E8M0 scale per 32 along K; FP4 expert
// weights, same DeepSeek-V4 page section 6.2) are decoded exactly to bf16 in
// LDS and then go through the same bf16 MFMA chain, so the result equals the
// bf16 tile on the decoded weights bit for bit.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Calls f(integral_constant<int, I>) for I = B..E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int KT = 64;         // K per LDS stage (two MFMA k-steps)

// 16-byte weight load marked non-temporal (streamed past the caches' normal
// replacement).  Used by the small-row tiles, where one m-tile covers all of
// an expert's rows and so reads its weight panel exactly once: measured on
// MI355X, decode steps 9-10 % faster (gate/up weights at 6.0 instead of
// 5.4 TB/s); in 128-row prefill tiles, where several m-tiles of an expert
// re-read the panel from L2, it is 6 % slower, so those keep plain loads.
// MXFP4 tiles keep them too: a stage reads only 32 bytes of a weight row, and
// non-temporal loads then fetch each piece of a 128-byte line from HBM on its
// own (measured 45 % slower at 64 rows per expert; the same for the FP4 x FP8
// kernel, whose stages read 64 bytes of a row).
__device__ __forceinline__ uint4 nt_load16(const uint8_t* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// An LDS row holds one stage of one token or weight row: 64 bf16 = 128 B, no
// padding.  Its eight 16-byte chunks are stored XOR-swizzled (chunk j of row r
// at position j ^ (r & 7)), so that both the row-major staging writes and the
// 16-row MFMA fragment reads spread over distinct banks.  (Measured on
// MI355X: fragment reads over 144-byte padded rows run at 76 % of the
// contiguous rate, over swizzled 128-byte rows at the full rate.)
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * KT + ((chunk ^ (row & 7)) << 3);
}

// ---------------------------------------------------------------------------
// Work list: one tile descriptor per workgroup, written on the device from the
// group offsets before the launch (tile order and XCD placement: tiles.hpp).
// A descriptor that does not fit its segment is treated as "no tile", so no
// access leaves the row, weight or output ranges whatever the table holds.
// ---------------------------------------------------------------------------
struct TileInfo {
  int seg, g;
  int64_t row0;  // first output row of the tile
  int rows;      // valid rows in the tile
  int n0;        // first output feature
};

__device__ __forceinline__ bool read_tile(const GemmArgs& a, int64_t tile, int BM, TileInfo& ti) {
  const int4 d = a.tiles[tile];
  const int seg = d.z >> 16, g = d.z & 0xffff;
  if (d.y <= 0 || d.y > BM || d.x < 0 || seg >= a.nseg) return false;
  const GemmSeg& s = a.seg[seg];
  if (g >= s.G || (int64_t)d.x + d.y > s.M || d.w < 0 || d.w >= s.N) return false;
  ti.seg = seg;
  ti.g = g;
  ti.row0 = d.x;
  ti.rows = d.y;
  ti.n0 = d.w;
  return true;
}

// The gated activation a(g, u) of the gate branch g and the up branch u, in
// fp32 (M: the math of the kernel, FastMath or LibMath below):
//  GLU_SWIGLU  SiLU(g) * u;
//  GLU_CLAMP   the clamped SwiGLU of the DeepSeek-V4 infrastructure
//              walkthrough, section 6.5: g capped from above at 10, u clamped
//              to [-10, 10], then SiLU(g) * u;
//  GLU_SITU    SiTU-GLU (forum article on MoE variants, section "SiTU-GLU"):
//              the soft cap b tanh(x / b) on each branch, b = 4 on the gate and
//              25 on the up branch, times the sigmoid of the uncapped gate.
// The comparisons keep a NaN branch value NaN.  Per element and uniform over
// the launch, so the activation never depends on the batch.
template <typename M>
__device__ __forceinline__ float glu_act(float g, float u, int glu) {
  if (glu == GLU_SITU)
    return M::softcap(g, 4.0f, 0.25f) * M::recip(1.0f + M::exp(-g)) *
           M::softcap(u, 25.0f, 0.04f);
  if (glu == GLU_CLAMP) {
    g = g > 10.0f ? 10.0f : g;
    u = u > 10.0f ? 10.0f : (u < -10.0f ? -10.0f : u);
  }
  return g / (1.0f + M::exp(-g)) * u;
}

// bf16 outputs (8 significant bits): hardware exp and reciprocal, and tanh
// from one exponential, tanh|x| = (1 - e) / (1 + e) with e = exp(-2|x|), or,
// below |x| = 1/16 where 1 - e cancels, the odd Taylor terms
// x - x^3/3 + 2x^5/15 (truncation under 4e-9 relative there).
struct FastMath {
  static __device__ float exp(float a) { return __expf(a); }
  static __device__ float recip(float a) { return __builtin_amdgcn_rcpf(a); }
  static __device__ float tanh(float x) {
    const float ax = fabsf(x), x2 = x * x;
    const float e = __expf(-2.0f * ax);
    const float big = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
    const float small = ax * (1.0f + x2 * (-1.0f / 3.0f + x2 * (2.0f / 15.0f)));
    return copysignf(ax < 0.0625f ? small : big, x);
  }
  static __device__ float softcap(float x, float b, float inv_b) { return b * tanh(x * inv_b); }
};

// fp32 outputs: the device library's functions and IEEE division.
struct LibMath {
  static __device__ float exp(float a) { return expf(a); }
  static __device__ float recip(float a) { return 1.0f / a; }
  static __device__ float softcap(float x, float b, float) { return b * tanhf(x / b); }
};

// ---------------------------------------------------------------------------
// bf16 / MXFP4 MFMA kernel.  BM token rows x BN output features per tile
// (x2 matrices when GATED: gate rows then up rows in LDS).  Waves form a
// WM x WN grid; each wave holds TBW token blocks x NBW feature blocks of 16.
// ---------------------------------------------------------------------------
// One LDS stage: the token rows (bf16), then the weight rows: bf16, or for
// MXFP4 the raw E2M1 codes (two 16-byte chunks of 32 codes per row, chunk-major)
// and their E8M0 scale bytes, decoded to bf16 only when a wave reads its
// fragment (a quarter of the LDS writes and reads of decoded weights).  A
// row-major code layout with an XOR swizzle of the two chunks and one scale
// word per row (no bank conflicts on the fragment reads) measured 12 % slower
// on the 128-row gate/up tiles: its extra address and scale-pairing work
// pushed the 128 x 64 gated tile over 256 VGPRs.
template <int BM, int BN, bool GATED, bool FP4 = false>
constexpr int gemm_stage_bytes() {
  return FP4 ? (BM * KT * 2 + (GATED ? 2 : 1) * BN * 34 + 15) / 16 * 16
             : (BM + (GATED ? 2 : 1) * BN) * KT * 2;
}

template <int BM, int BN, bool GATED, bool FP4 = false>
constexpr int gemm_smem_bytes() {
  return 2 * gemm_stage_bytes<BM, BN, GATED, FP4>();  // two stages
}

// Exact decode of eight E2M1 codes (one 32-bit word, element 2i in the low
// nibble of byte i) with one E8M0 scale byte into eight bf16, by gfx950's
// scaled conversion (two codes times an fp32 scale to two bf16 per
// instruction).  The scale 2^(s-127) is built exactly in fp32 (subnormal for
// s = 0; s = 255 is the E8M0 NaN and gives NaN weights).  Every product
// code * 2^(s-127) has at most two significant bits, so it is exact in bf16
// (subnormals included) unless it overflows; checked on MI355X against the
// bit-level decode for all 256 x 256 (scale, code byte) pairs.
__device__ __forceinline__ bf16x8_t decode_mxfp4_8(uint32_t q, uint32_t sbyte) {
  const float scale = sbyte ? __uint_as_float(sbyte << 23) : __uint_as_float(0x00400000u);
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// One tile (BM rows x BN features of segment s) by the 64 * WM * WN threads of
// the calling workgroup; smem: gemm_smem_bytes<BM, BN, GATED>() bytes of LDS.
// The workgroup may run further tiles afterwards once every thread has
// returned (the caller synchronises before the next tile's LDS writes).
// CO: coherent output stores (Out<CO>), for tiles whose outputs other
// workgroups of the same launch read.
template <int BM, int BN, int WM, int WN, int P, bool GATED, bool FP4, bool CO = false>
__device__ __forceinline__ void gemm_tile_bf16(const GemmSeg& s, const TileInfo& ti, int glu,
                                               unsigned char* smem) {
  constexpr int NT = 64 * WM * WN;
  constexpr int NMAT = GATED ? 2 : 1;
  constexpr int TBW = BM / 16 / WM;
  constexpr int NBW = BN / 16 / WN;
  static_assert(TBW >= 1 && NBW >= 1, "tile too small for the wave grid");
  constexpr int XCH = BM * (KT / 8);          // 16-byte chunks of the token tile
  constexpr int WCH = NMAT * BN * (KT / 8);   // 16-byte chunks of the weight tile (bf16)
  constexpr int QCH = NMAT * BN * 2;          // 16-byte chunks of an MXFP4 weight tile
  constexpr int XPT = (XCH + NT - 1) / NT;
  constexpr int WPT = (WCH + NT - 1) / NT;
  constexpr int QPT = (QCH + NT - 1) / NT;
  constexpr int WQ = FP4 ? QPT : WPT;
  constexpr int NR = NMAT * BN;                // weight rows of the tile
  constexpr int SB = gemm_stage_bytes<BM, BN, GATED, FP4>();  // bytes of one LDS stage
  constexpr bool kStreamW = BM <= 32;          // weights read once per launch: nt_load16
  // stage buf: token rows Xs [BM][KT] bf16, swizzled; weight rows Ws [NR][KT]
  // bf16, swizzled, or (MXFP4) codes Wq [2][NR][16 B] and scales Wsc [2][NR]
  auto stage_x = [&](int buf) { return reinterpret_cast<uint16_t*>(smem + buf * SB); };
  auto stage_w = [&](int buf) { return smem + buf * SB + BM * KT * 2; };
  const int K = s.K, N = s.N;
  constexpr bool fp4 = FP4;  // weight format of this instantiation (the launcher splits segments)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Wave w takes row block wm = w / WN and feature block wn = w % WN.  In
  // 128-row tiles a wave whose rows all lie past the tile's valid rows does no
  // MFMA work (only its share of the loads and LDS writes); waves are dealt to
  // the four SIMDs round-robin, so with WN a multiple of 4 the waves of one
  // SIMD hold different row blocks and a half-empty tile frees half of every
  // SIMD.  (Measured: 9-10 % off the MXFP4 expert GEMMs at 64 rows per
  // expert; in 64-row tiles the skip costs more than it saves.)  Row blocks
  // do not change any element's chain.
  const int wm = wave / WN, wn = wave % WN;
  const bool active = BM < 128 || wm * TBW * 16 < ti.rows;  // uniform per wave

  // Token rows of this thread's chunks (rows clamped into the tile).  With a
  // row index the indices are loaded here, before the weight prefetch below,
  // so that waiting for them does not wait for the weights.
  int64_t xrow[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = tid + i * NT;
    const int r = min(min(c / (KT / 8), BM - 1), ti.rows - 1);
    xrow[i] = ti.row0 + r;
  }
  if (s.a_index) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) xrow[i] = s.a_index[xrow[i]];
  }
  const uint16_t* xsrc[XPT];
  // weight tile sources
  const uint8_t* wsrc[WQ];
  const uint8_t* ssrc[QPT];
  if constexpr (!fp4) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = min(tid + i * NT, WCH - 1);
      const int mat = c / (BN * (KT / 8));
      const int n = (c / (KT / 8)) % BN;
      const int nn = min(ti.n0 + n, N - 1);
      const uint16_t* base = static_cast<const uint16_t*>(mat ? s.W1 : s.W0);
      wsrc[i] = reinterpret_cast<const uint8_t*>(base + ((int64_t)ti.g * N + nn) * K +
                                                 (c % (KT / 8)) * 8);
    }
  } else {
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int c = min(tid + i * NT, QCH - 1);
      const int mat = c / (BN * 2);
      const int n = (c / 2) % BN;
      const int nn = min(ti.n0 + n, N - 1);
      const int half = c % 2;
      const uint8_t* base = static_cast<const uint8_t*>(mat ? s.W1 : s.W0);
      const uint8_t* sb = mat ? s.S1 : s.S0;
      const int64_t row = (int64_t)ti.g * N + nn;
      wsrc[i] = base + row * (K / 2) + half * 16;
      ssrc[i] = sb + row * (K / 32) + half;
    }
  }

  f32x4_t acc[NMAT][NBW][TBW];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int tb = 0; tb < TBW; ++tb) acc[m][nb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // P register stages in flight; LDS holds two stages.
  uint4 xr[P][XPT];
  uint4 wr[P][WQ];
  uint32_t sr[P][QPT];

  // Branch-free stage load (every lane always issues the same loads, from
  // clamped in-range addresses; out-of-tile parts are zeroed afterwards), so
  // the compiler can wait for exactly one stage while P-1 stay in flight.
  // Stage load.  In the pipelined loop (half == false) every lane issues the
  // same unconditional loads (lanes without a chunk read a clamped in-range
  // address and skip the LDS store), so the compiler can wait for exactly one
  // stage while the others stay in flight.  half == true loads the first 32
  // k of the last stage when K % 64 == 32 and zeroes the rest.
  auto gload_x = [&](uint4 (&xq)[XPT], int kt, bool half) {
    const int k0 = kt * KT;
    const bool none = half && (K % KT) == 0;  // trailing step over zeros
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * NT;
      if (half && (none || (c % (KT / 8)) >= 4))
        xq[i] = make_uint4(0, 0, 0, 0);
      else
        xq[i] = *reinterpret_cast<const uint4*>(xsrc[i] + k0);
    }
  };
  auto gload_w = [&](uint4 (&wq)[WQ], uint32_t (&sq)[QPT], int kt, bool half) {
    const int k0 = kt * KT;
    const bool none = half && (K % KT) == 0;
    if constexpr (!fp4) {
#pragma unroll
      for (int i = 0; i < WPT; ++i) {
        const int c = tid + i * NT;
        if (half && (none || (c % (KT / 8)) >= 4))
          wq[i] = make_uint4(0, 0, 0, 0);
        else
          wq[i] = kStreamW ? nt_load16(wsrc[i] + (int64_t)k0 * 2)
                           : *reinterpret_cast<const uint4*>(wsrc[i] + (int64_t)k0 * 2);
      }
    } else {
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        const int c = tid + i * NT;
        if (half && (none || (c % 2) == 1)) {
          wq[i] = make_uint4(0, 0, 0, 0);
          sq[i] = 127u;
        } else {
          wq[i] = kStreamW ? nt_load16(wsrc[i] + k0 / 2)
                           : *reinterpret_cast<const uint4*>(wsrc[i] + k0 / 2);
          sq[i] = ssrc[i][k0 / 32];
        }
      }
    }
  };
  auto gload = [&](uint4 (&xq)[XPT], uint4 (&wq)[WQ], uint32_t (&sq)[QPT], int kt, bool half) {
    gload_x(xq, kt, half);
    gload_w(wq, sq, kt, half);
  };
  auto lstore = [&](const uint4 (&xq)[XPT], const uint4 (&wq)[WQ], const uint32_t (&sq)[QPT],
                    int buf) {
    uint16_t* Xs = stage_x(buf);
    uint16_t* Ws = reinterpret_cast<uint16_t*>(stage_w(buf));
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * NT;
      if (XCH % NT == 0 || c < XCH)
        *reinterpret_cast<uint4*>(&Xs[lds_off(c / (KT / 8), c % (KT / 8))]) = xq[i];
    }
    if constexpr (!fp4) {
#pragma unroll
      for (int i = 0; i < WPT; ++i) {
        const int c = tid + i * NT;
        if (WCH % NT == 0 || c < WCH)
          *reinterpret_cast<uint4*>(&Ws[lds_off(c / (KT / 8), c % (KT / 8))]) = wq[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        const int c = tid + i * NT;
        if (QCH % NT == 0 || c < QCH) {
          uint8_t* Wq = stage_w(buf);
          const int row = c / 2, ks = c % 2;  // the 32 codes of k-step ks of row `row`
          *reinterpret_cast<uint4*>(Wq + (ks * NR + row) * 16) = wq[i];
          Wq[2 * NR * 16 + ks * NR + row] = (uint8_t)sq[i];
        }
      }
    }
  };
  // The fixed per-element chain: for each 32-wide k-step in increasing order,
  // acc = mfma(weights, tokens, acc).  One k-step's operands are read from
  // LDS into a fragment set, so that the reads of the next k-step are in
  // flight while the MFMAs of this one run.
  struct Frag {
    bf16x8_t a[NMAT][NBW];
    bf16x8_t b[TBW];
  };
  auto read_frag = [&](Frag& f, int buf, int ks) {
    const uint16_t* Xs = stage_x(buf);
    // Rows n and r below are 16-row block bases plus lane & 15, so row & 7 is
    // lane & 7 and the swizzled chunk is the same for every block.
    const int sw = ((ks * 4 + (lane >> 4)) ^ (lane & 7)) << 3;
    if constexpr (!fp4) {
      const uint16_t* Ws = reinterpret_cast<const uint16_t*>(stage_w(buf));
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const int n = m * BN + (wn * NBW + nb) * 16 + (lane & 15);
          f.a[m][nb] = *reinterpret_cast<const bf16x8_t*>(&Ws[n * KT + sw]);
        }
    } else {
      // lane: 8 codes of row n at k 8 * (lane / 16) of the k-step (one word of
      // the row's chunk; the 16 rows x 4 words of a fragment hit 64 banks)
      const uint8_t* Wq = stage_w(buf);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const int n = m * BN + (wn * NBW + nb) * 16 + (lane & 15);
          const uint32_t q =
              *reinterpret_cast<const uint32_t*>(Wq + (ks * NR + n) * 16 + 4 * (lane >> 4));
          f.a[m][nb] = decode_mxfp4_8(q, Wq[2 * NR * 16 + ks * NR + n]);
        }
    }
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      const int r = (wm * TBW + tb) * 16 + (lane & 15);
      f.b[tb] = *reinterpret_cast<const bf16x8_t*>(&Xs[r * KT + sw]);
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int tb = 0; tb < TBW; ++tb)
          acc[m][nb][tb] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[m][nb], f.b[tb], acc[m][nb][tb], 0, 0, 0);
  };

  // Full 64-wide stages 0..nkf-1.  Stage s lives in register slot s % P until
  // it is written to LDS buffer s & 1.  Step k (slot q = k % P):
  //   issue the loads of stage k+P (clamped to the last stage) into slot q,
  //   which stage k left at step k-1;
  //   read the second k-step of stage k (fragment set fb);
  //   MFMAs of the first k-step of stage k (fa), with the LDS writes of stage
  //   k+1 (from its slot into buffer (k+1)&1, whose last readers, stage k-1,
  //   finished before the previous barrier) spread between them;
  //   barrier: stage k+1 is in LDS, buffer k&1 is no longer read;
  //   MFMAs of the second k-step of stage k (fb), with the reads of the first
  //   k-step of stage k+1 into fa spread between them (on the last step these
  //   read a buffer nobody uses and fa is overwritten afterwards).
  // The scheduling groups fix that interleaving; they move instructions, never
  // the order of the MFMAs on one accumulator.  Full groups of P steps run
  // branch-free; the remaining nkf % P steps follow with uniform guards.
  // Instruction counts of one step for the scheduling groups (masks of
  // sched_group_barrier: MFMA, LDS read, LDS write).
  constexpr int kMfmas = NMAT * NBW * TBW;                    // per k-step
  constexpr int kFragReads = (FP4 ? 2 : 1) * NMAT * NBW + TBW;  // per fragment set
  constexpr int kLdsWrites = XPT + (FP4 ? 2 * QPT : WPT);       // per stage
  constexpr int kMfmaPerWrite = kMfmas / kLdsWrites > 0 ? kMfmas / kLdsWrites : 1;
  constexpr int kMfmaPerRead = kMfmas / kFragReads > 0 ? kMfmas / kFragReads : 1;
  constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;
  const int nkf = K / KT;
  Frag fa, fb;
  auto step = [&](auto qc, int k) {
    constexpr int q = decltype(qc)::value;
    gload(xr[q], wr[q], sr[q], min(k + P, nkf - 1), false);
    read_frag(fb, k & 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(fa);
    lstore(xr[(q + 1) % P], wr[(q + 1) % P], sr[(q + 1) % P], (k + 1) & 1);
    static_for<0, kLdsWrites>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMfmaPerWrite, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
    });
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMfmas, 0);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    read_frag(fa, (k + 1) & 1, 0);
    mma(fb);
    static_for<0, kFragReads>([&](auto) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMfmaPerRead, 1);
    });
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kMfmas, 1);
    __builtin_amdgcn_sched_barrier(0);
  };
  if (nkf > 0) {
#pragma unroll
    for (int q = 0; q < P; ++q) gload_w(wr[q], sr[q], min(q, nkf - 1), false);
  }
  // The weight stream does not depend on the token rows: it is in flight
  // before the row indices are consumed.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = tid + i * NT;
    xsrc[i] = static_cast<const uint16_t*>(s.A) + xrow[i] * K + (c % (KT / 8)) * 8;
  }
  if (nkf > 0) {
#pragma unroll
    for (int q = 0; q < P; ++q) gload_x(xr[q], min(q, nkf - 1), false);
    lstore(xr[0], wr[0], sr[0], 0);
    __syncthreads();
    const int nfull = nkf / P * P;
    if (active) {
      read_frag(fa, 0, 0);
      for (int kt = 0; kt < nfull; kt += P) static_for<0, P>([&](auto qc) { step(qc, kt + qc); });
      static_for<0, P>([&](auto qc) {
        if (nfull + qc < nkf) step(qc, nfull + qc);
      });
    } else {
      // Same loads, LDS writes and barriers as step(), without fragments.
      auto idle_step = [&](auto qc, int k) {
        constexpr int q = decltype(qc)::value;
        gload(xr[q], wr[q], sr[q], min(k + P, nkf - 1), false);
        lstore(xr[(q + 1) % P], wr[(q + 1) % P], sr[(q + 1) % P], (k + 1) & 1);
        __syncthreads();
      };
      for (int kt = 0; kt < nfull; kt += P)
        static_for<0, P>([&](auto qc) { idle_step(qc, kt + qc); });
      static_for<0, P>([&](auto qc) {
        if (nfull + qc < nkf) idle_step(qc, nfull + qc);
      });
    }
  }
  // Trailing k-step: the last 32 of K when K % 64 == 32, and a step over zero
  // operands otherwise.  Running it unconditionally keeps one chain for every
  // tile variant (a zero step leaves every nonzero accumulator unchanged).
  // Buffer nkf&1 was last read for stage nkf-2, before the last barrier.
  gload(xr[0], wr[0], sr[0], nkf, true);
  lstore(xr[0], wr[0], sr[0], nkf & 1);
  __syncthreads();
  if (active) {
    read_frag(fa, nkf & 1, 0);
    mma(fa);
  }

  // epilogue: lane holds features n = base + 4*(lane/16) + i (i = 0..3) of
  // token row base + lane%16 -> one 8-byte store of 4 bf16.
  uint16_t* out = static_cast<uint16_t*>(s.out);
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      const int r = (wm * TBW + tb) * 16 + (lane & 15);
      const int n = ti.n0 + (wn * NBW + nb) * 16 + 4 * (lane >> 4);
      if (r < ti.rows && n < N) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[i] = GATED ? glu_act<FastMath>(acc[0][nb][tb][i], acc[NMAT - 1][nb][tb][i], glu)
                       : acc[0][nb][tb][i];
        uint2 pk = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        Out<CO>::put2(reinterpret_cast<uint2*>(out + (ti.row0 + r) * (int64_t)N + n), pk);
      }
    }
}

}  // namespace moe
