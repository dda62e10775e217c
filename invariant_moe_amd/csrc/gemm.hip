// Grouped expert GEMMs with the SwiGLU epilogue.
//
// Expert FFN: g = W_gate a, u = W_up a, h = SiLU(g) * u, o = W_down h
// (SwiGLU, "6 基建与训练稳定性优化" section 6.5; gate and up branches, forum
// article feedbbs.com/linuxdo/72580, GLU section).  Every GEMM sees its whole
// K in one workgroup (no split sums: the LongCat parity article,
// "美团把训练和推理的概率做到逐位相同"), so each output element is one fixed
// chain of MFMA steps over K.
//
// Batch invariance.  All bf16 kernels here use ONE instruction,
// v_mfma_f32_16x16x32_bf16, with the weight tile as operand A (16 output
// features) and the token tile as operand B (16 rows), K stepped by 32 in
// increasing order into an accumulator that starts at 0.  An output element
// depends only on its own weight row and token row and on this fixed chain,
// never on the other rows of its tile, the tile shape, the number of rows of
// its expert, or T.  The tile variants below differ only in how many blocks a
// workgroup holds, so they give identical bits.
//
// MXFP4 weights (E2M1 codes + one E8M0 scale per 32 along K; FP4 expert
// weights, same DeepSeek-V4 page section 6.2) are decoded exactly to bf16 in
// LDS and then go through the same bf16 MFMA chain, so the result equals the
// bf16 kernel on the decoded weights bit for bit.
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

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

__device__ __forceinline__ bool read_tile(const GemmArgs& a, int BM, TileInfo& ti) {
  const int4 d = a.tiles[blockIdx.x];
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

// Exact decode of 32 E2M1 codes (16 bytes, element 2i in the low nibble of
// byte i) with one E8M0 scale byte into 32 bf16 values, by gfx950's scaled
// conversion (two codes times an fp32 scale to two bf16 per instruction).  The
// scale 2^(s-127) is built exactly in fp32 (subnormal for s = 0; s = 255 is
// the E8M0 NaN and gives NaN weights).  Every product code * 2^(s-127) has at
// most two significant bits, so it is exact in bf16 (subnormals included)
// unless it overflows; checked on MI355X against the bit-level decode for all
// 256 x 256 (scale, code byte) pairs.
__device__ __forceinline__ void decode_mxfp4_32(const uint4 q, uint32_t sbyte, uint32_t (&o)[16]) {
  const float scale = sbyte ? __uint_as_float(sbyte << 23) : __uint_as_float(0x00400000u);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i * 4 + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 0));
    o[i * 4 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 1));
    o[i * 4 + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 2));
    o[i * 4 + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 3));
  }
}

// ---------------------------------------------------------------------------
// bf16 / MXFP4 MFMA kernel.  BM token rows x BN output features per tile
// (x2 matrices when GATED: gate rows then up rows in LDS).  Waves form a
// WM x WN grid; each wave holds TBW token blocks x NBW feature blocks of 16.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int P, bool GATED, bool FP4>
__global__ __launch_bounds__(64 * WM * WN, 2) void k_grouped_gemm_bf16(GemmArgs args) {
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
  constexpr int BUF = (BM + NMAT * BN) * KT;  // bf16 elements of one LDS stage
  constexpr bool kStreamW = BM <= 32;          // weights read once per launch: nt_load16
  __shared__ __align__(16) unsigned char smem[2 * BUF * 2];

  TileInfo ti;
  if (!read_tile(args, BM, ti)) return;
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);  // [2][BM + NMAT*BN][KT], swizzled
  const GemmSeg& s = args.seg[ti.seg];
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
    uint16_t* Xs = lds + buf * BUF;
    uint16_t* Ws = Xs + BM * KT;
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
          uint32_t o[16];
          decode_mxfp4_32(wq[i], sq[i], o);
          const int row = c / 2, ch = (c % 2) * 4;  // 32 k values = chunks ch..ch+3
#pragma unroll
          for (int j = 0; j < 4; ++j)
            *reinterpret_cast<uint4*>(&Ws[lds_off(row, ch + j)]) =
                make_uint4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
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
    const uint16_t* Xs = lds + buf * BUF;
    const uint16_t* Ws = Xs + BM * KT;
    // Rows n and r below are 16-row block bases plus lane & 15, so row & 7 is
    // lane & 7 and the swizzled chunk is the same for every block.
    const int sw = ((ks * 4 + (lane >> 4)) ^ (lane & 7)) << 3;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int n = m * BN + (wn * NBW + nb) * 16 + (lane & 15);
        f.a[m][nb] = *reinterpret_cast<const bf16x8_t*>(&Ws[n * KT + sw]);
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
  constexpr int kFragReads = NMAT * NBW + TBW;                // per fragment set
  constexpr int kLdsWrites = XPT + (FP4 ? 4 * QPT : WPT);     // per stage
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
          v[i] = GATED ? glu_act<FastMath>(acc[0][nb][tb][i], acc[NMAT - 1][nb][tb][i], args.glu)
                       : acc[0][nb][tb][i];
        uint2 pk = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        *reinterpret_cast<uint2*>(out + (ti.row0 + r) * (int64_t)N + n) = pk;
      }
    }
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
  if (!read_tile(args, BM, ti)) return;
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
  if (!read_tile(args, BM, ti)) return;
  const GemmSeg& s = args.seg[ti.seg];
  const int K = s.K, N = s.N, nst = K / KQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
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
  uint32_t sc[SPT];
  // stage loads into registers, then into LDS (the arrays are passed, not
  // captured, so that they stay in registers)
  auto gload = [&](u32x4 (&xq)[XPT], u32x4 (&wq)[WPT], uint32_t (&scq)[SPT], int kt) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) xq[i] = *reinterpret_cast<const u32x4*>(xsrc[i] + kt * KQ);
#pragma unroll
    for (int i = 0; i < WPT; ++i) wq[i] = *reinterpret_cast<const u32x4*>(wsrc[i] + kt * (KQ / 2));
#pragma unroll
    for (int i = 0; i < SPT; ++i) scq[i] = *reinterpret_cast<const uint32_t*>(scsrc[i] + kt * 4);
  };
  auto lstore = [&](const u32x4 (&xq)[XPT], const u32x4 (&wq)[WPT], const uint32_t (&scq)[SPT],
                    int buf) {
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
        ssx[buf][w] = scq[i];
      else if (w < SW)
        ssw[buf][w - BM] = scq[i];
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

  gload(xr, wr, sc, 0);
  lstore(xr, wr, sc, 0);
  __syncthreads();
  for (int kt = 0; kt < nst; ++kt) {
    const bool more = kt + 1 < nst;  // uniform
    if (more) gload(xr, wr, sc, kt + 1);
    compute(kt & 1);
    if (more) lstore(xr, wr, sc, (kt + 1) & 1);
    __syncthreads();
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
  TILE_128x64_2x2_P2,     // MXFP4 weights with tens of rows per expert
  TILE_128x128_2x2_P2,    // prefill
  TILE_128x128_2x4_P2,    // prefill gate/up: 8 waves, two per SIMD
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
    case TILE_128x64_2x2_P2: return {128, 64};
    case TILE_128x128_2x2_P2: return {128, 128};
    case TILE_128x128_2x4_P2: return {128, 128};
    case TILE_W4A8: return {64, 64};
    case TILE_W4A8_N128: return {64, 128};
    case TILE_W4A8_128: return {128, 128};
    default: return {16, 16};  // TILE_F32
  }
}

// The (configuration, branch, weight format) combinations the planner can
// select: every configuration for either format, since a launch of one
// format may carry the configuration chosen for the other (shared and routed
// experts in different formats), except the 128 x 64 gate/up tile, which only
// MXFP4 launches get (a bf16 launch takes its twin of the same row tile).
template <bool FP4>
static hipError_t launch_tile_cfg(int cfg, const GemmArgs& a, bool gated, int64_t grid,
                                  hipStream_t st, LaunchEvents ev) {
  if (gated) {
    switch (cfg) {
      case TILE_16x16_1x1_P4: return launch_one<16, 16, 1, 1, 4, true, FP4>(a, grid, st, ev);
      case TILE_32x64_1x4_P4: return launch_one<32, 64, 1, 4, 4, true, FP4>(a, grid, st, ev);
      case TILE_64x32_4x1_P2: return launch_one<64, 32, 4, 1, 2, true, FP4>(a, grid, st, ev);
      case TILE_128x64_2x2_P2:
        if constexpr (FP4) return launch_one<128, 64, 2, 2, 2, true, true>(a, grid, st, ev);
        break;
      case TILE_128x128_2x4_P2: return launch_one<128, 128, 2, 4, 2, true, FP4>(a, grid, st, ev);
      default: break;
    }
  } else {
    switch (cfg) {
      case TILE_16x64_1x4_P4: return launch_one<16, 64, 1, 4, 4, false, FP4>(a, grid, st, ev);
      case TILE_32x64_1x4_P4: return launch_one<32, 64, 1, 4, 4, false, FP4>(a, grid, st, ev);
      case TILE_64x64_4x1_P2: return launch_one<64, 64, 4, 1, 2, false, FP4>(a, grid, st, ev);
      case TILE_128x128_2x2_P2: return launch_one<128, 128, 2, 2, 2, false, FP4>(a, grid, st, ev);
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
  // faster than two-wave 16 x 32 tiles from T=1 to T=4).
  if (rows_per_group_hint <= 2) return gated ? TILE_16x16_1x1_P4 : TILE_16x64_1x4_P4;
  if (rows_per_group_hint <= 16) return TILE_32x64_1x4_P4;
  // MXFP4 weights: the decode in the LDS staging favours 128-row tiles
  // (each decoded weight serves more token rows)
  if (fp4 && rows_per_group_hint <= 96) return gated ? TILE_128x64_2x2_P2 : TILE_128x128_2x2_P2;
  if (rows_per_group_hint <= 96) return gated ? TILE_64x32_4x1_P2 : TILE_64x64_4x1_P2;
  // many rows per expert: 128 x 128 tiles (gate/up on 8 waves, two per SIMD)
  return gated ? TILE_128x128_2x4_P2 : TILE_128x128_2x2_P2;
}

// Configuration of one launch whose weights are bf16 (fp4 == false) or MXFP4
// within a layer planned as cfg: a bf16 launch next to MXFP4 routed experts
// (the shared expert) takes the bf16 configuration with the same row tile.
static int launch_cfg_for_format(int cfg, bool gated, bool fp4) {
  if (!fp4 && gated && cfg == TILE_128x64_2x2_P2) return TILE_128x128_2x4_P2;
  return cfg;
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
    L.cfg = cfg == TILE_F32 ? cfg
                            : launch_cfg_for_format(cfg, gated, segs[split ? l : 0].wfmt != 0);
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
  // token re-reads, -12 %), 128 x 128 at 256 rows.
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
    if (jobs.n == MOE_MAX_TILE_JOBS || (jobs.n > 0 && jobs.BM != L.BM)) return false;
    jobs.BM = L.BM;
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
    mpre[e] = (tile_group_rows(soff, e, M) + jobs.BM - 1) / jobs.BM;
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
