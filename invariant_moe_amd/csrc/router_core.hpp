// Router logits in the fixed fp32 order of the routing contract, as device
// functions of the calling 256-thread workgroup (used by the router kernels
// and by the single-launch layer kernel).
//
// Learned routing is scores = W h followed by top-k ("6 基建与训练稳定性优化",
// section 6.3; the "V4" article, section 2.2, describes the router as a small
// linear layer giving E logits).
//
// One tile = TT tokens x (4 * EW) experts; wave w owns experts
// [e0 + w*EW, e0 + (w+1)*EW).  Lane j owns partial sum j of every
// (token, expert) pair: it accumulates elements d = 8j + 512 i + c (c = 0..7),
// i increasing, with fmaf — the fixed order of the routing contract.  The 64
// partials of a pair are then summed by one lane in the fixed pairwise tree
// (partial[j] += partial[j + m], m = 32..1) after a transpose through LDS.
// The result of a pair does not depend on TT, EW, T or the grid.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <typename ACT>
struct ActIO;
template <>
struct ActIO<uint16_t> {  // bf16 bits
  __device__ static void load8(const uint16_t* p, float (&v)[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
    v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  }
};
template <>
struct ActIO<float> {
  __device__ static void load8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// x and w chunks of one 512-wide step, loaded straight into registers
// (small T): lane j reads elements 8j .. 8j+7 of the step.
template <typename ACT>
struct Chunk8;
template <>
struct Chunk8<uint16_t> {  // 8 bf16
  uint4 q;
  __device__ void load(const uint16_t* p) { q = *reinterpret_cast<const uint4*>(p); }
  __device__ void zero() { q = make_uint4(0, 0, 0, 0); }
  __device__ void store(uint16_t* p) const { *reinterpret_cast<uint4*>(p) = q; }
  __device__ void unpack(float (&v)[8]) const {
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
    v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  }
};
template <>
struct Chunk8<float> {  // 8 fp32
  float4 a, b;
  __device__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ void zero() { a = make_float4(0.f, 0.f, 0.f, 0.f); b = a; }
  __device__ void store(float* p) const {
    reinterpret_cast<float4*>(p)[0] = a;
    reinterpret_cast<float4*>(p)[1] = b;
  }
  __device__ void unpack(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// Fixed-tree reduction of the 64 partials of each (token, expert) pair of a
// wave, 32 pairs per round: partial[j] += partial[j + m], m = 32..1, by one
// lane per pair after a transpose through LDS.  Element (pair q, partial j)
// sits at q*64 + (j ^ q) so that both the write (fixed q, lanes j) and the
// read (lanes q, fixed j) hit distinct banks.  myred: this wave's 32*64 floats.
template <int TT, int EW, bool CO = false>
__device__ __forceinline__ void logits_tree_store(const float (&acc)[TT][EW], float* myred,
                                                  int64_t t0, int ew0, int64_t T, int E,
                                                  float* __restrict__ logits) {
  constexpr int NP = TT * EW;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int base = 0; base < NP; base += 32) {
    __syncthreads();
#pragma unroll
    for (int q = base; q < NP && q < base + 32; ++q)
      myred[(q - base) * 64 + (lane ^ (q - base))] = acc[q / EW][q % EW];
    __syncthreads();
    const int q = base + lane;
    if (lane < 32 && q < NP) {
      float p[64];
#pragma unroll
      for (int j = 0; j < 64; ++j) p[j] = myred[lane * 64 + (j ^ lane)];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
        for (int j = 0; j < m; ++j) p[j] = p[j] + p[j + m];
      const int64_t t = t0 + q / EW;
      const int e = ew0 + q % EW;
      if (t < T && e < E) Out<CO>::put(&logits[t * E + e], p[0]);
    }
  }
}

// Words that a later stage of the call counts into are cleared by the
// logit blocks: block b of nb clears words b*256 + tid, stepping by nb*256.
template <bool CO = false>
__device__ __forceinline__ void clear_words(unsigned long long* __restrict__ zero_words,
                                            int64_t n_zero, int64_t b, int64_t nb) {
  if (zero_words)
    for (int64_t i = b * 256 + threadIdx.x; i < n_zero; i += nb * 256)
      Out<CO>::put(&zero_words[i], 0ull);
}

template <typename ACT, int TT>
constexpr int router_logits_smem_bytes() {
  return 2 * TT * 512 * (int)sizeof(ACT) > 4 * 32 * 64 * 4 ? 2 * TT * 512 * (int)sizeof(ACT)
                                                              : 4 * 32 * 64 * 4;
}

// Logits of token tile bx (TT tokens) x expert tile by (4 * EW experts) by a
// workgroup of 256 threads; smem: router_logits_smem_bytes<ACT, TT>() bytes.
template <typename ACT, int TT, int EW, bool CO = false>
__device__ __forceinline__ void router_logits_tile(const ACT* __restrict__ x,
                                                   const ACT* __restrict__ w, int64_t T, int D,
                                                   int E, float* __restrict__ logits, int64_t bx,
                                                   int by, unsigned char* smem) {
  constexpr int XS_ELEMS = TT * 512;               // one step of x, TT tokens
  constexpr int XCH = TT * 64;                     // 8-element chunks of a step
  constexpr int XPT = (XCH + 255) / 256;
  ACT* xs = reinterpret_cast<ACT*>(smem);          // [2][TT][512]
  float* red = reinterpret_cast<float*>(smem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = bx * TT;
  const int ew0 = by * 4 * EW + wave * EW;
  const int NI = (D + 511) / 512;

  float acc[TT][EW];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int e = 0; e < EW; ++e) acc[t][e] = 0.0f;

  // Ring of depth two: the x chunks (to LDS) and w chunks (registers) of step
  // i + 1 are loaded before step i is summed.  Out-of-range tokens, experts
  // and the tail of D are read at clamped addresses and their x chunks
  // stored as zero (never summed into a stored logit, or zero terms skipped).
  Chunk8<ACT> xq[XPT], wq[2][EW];
  auto load = [&](int slot, int i) {
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int c = min((int)threadIdx.x + u * 256, XCH - 1);
      const int tt = c >> 6, j = c & 63;
      const int64_t t = min(t0 + tt, T - 1);
      const int d = min(i * 512 + 8 * j, D - 8);
      xq[u].load(x + t * (int64_t)D + d);
    }
    const int d = min(i * 512 + 8 * lane, D - 8);
#pragma unroll
    for (int e = 0; e < EW; ++e) wq[slot][e].load(w + (int64_t)min(ew0 + e, E - 1) * D + d);
  };
  auto stash = [&](int buf, int i) {
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const int c = (int)threadIdx.x + u * 256;
      if (c < XCH) {
        const int tt = c >> 6, j = c & 63;
        Chunk8<ACT> v = xq[u];
        if (!(t0 + tt < T && i * 512 + 8 * j < D)) v.zero();
        v.store(xs + buf * XS_ELEMS + tt * 512 + 8 * j);
      }
    }
  };
  auto step = [&](auto slot_c, int i) {
    constexpr int cur = decltype(slot_c)::value;
    if (i + 1 < NI) load(cur ^ 1, i + 1);  // uniform
    const int d = i * 512 + 8 * lane;
    if (d < D) {
      float wv[EW][8];
#pragma unroll
      for (int e = 0; e < EW; ++e) {
        if (ew0 + e < E) {
          wq[cur][e].unpack(wv[e]);
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) wv[e][c] = 0.0f;
        }
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        float xv[8];
        ActIO<ACT>::load8(xs + cur * XS_ELEMS + t * 512 + 8 * lane, xv);
#pragma unroll
        for (int e = 0; e < EW; ++e)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[t][e] = __builtin_fmaf(xv[c], wv[e][c], acc[t][e]);
      }
    }
    if (i + 1 < NI) stash(cur ^ 1, i + 1);
    __syncthreads();
  };
  load(0, 0);
  stash(0, 0);
  __syncthreads();
  for (int i = 0; i < NI; i += 2) {  // ring slots fixed at compile time
    step(std::integral_constant<int, 0>{}, i);
    if (i + 1 < NI) step(std::integral_constant<int, 1>{}, i + 1);
  }

  logits_tree_store<TT, EW, CO>(acc, red + wave * 32 * 64, t0, ew0, T, E, logits);
}

// Router logits for small T: the same pairs, partials and order as above, but
// every lane reads its x and w chunks from global memory into a register ring
// P steps deep (loads of step i+P are issued before step i is summed), with
// no LDS staging and no barrier in the loop.  Out-of-range rows, experts and
// the tail of D are read at clamped addresses and never summed.
constexpr int kRouterSmallSmemBytes = 4 * 32 * 64 * 4;

template <typename ACT, int TT, int EW, int P, bool CO = false>
__device__ __forceinline__ void router_logits_small_tile(const ACT* __restrict__ x,
                                                         const ACT* __restrict__ w, int64_t T,
                                                         int D, int E, float* __restrict__ logits,
                                                         int64_t bx, int by,
                                                         unsigned char* smem) {
  float* red = reinterpret_cast<float*>(smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = bx * TT;
  const int ew0 = by * 4 * EW + wave * EW;
  const int NI = (D + 511) / 512;
  const ACT* xrow[TT];
  const ACT* wrow[EW];
#pragma unroll
  for (int t = 0; t < TT; ++t) xrow[t] = x + (t0 + t < T ? t0 + t : T - 1) * (int64_t)D;
#pragma unroll
  for (int e = 0; e < EW; ++e) wrow[e] = w + (int64_t)(ew0 + e < E ? ew0 + e : E - 1) * D;

  float acc[TT][EW];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int e = 0; e < EW; ++e) acc[t][e] = 0.0f;

  Chunk8<ACT> xr[P][TT], wr[P][EW];
  auto load = [&](int q, int i) {
    const int d = min(i * 512 + 8 * lane, D - 8);
#pragma unroll
    for (int t = 0; t < TT; ++t) xr[q][t].load(xrow[t] + d);
#pragma unroll
    for (int e = 0; e < EW; ++e) wr[q][e].load(wrow[e] + d);
  };
#pragma unroll
  for (int q = 0; q < P; ++q) load(q, min(q, NI - 1));
  for (int i0 = 0; i0 < NI; i0 += P) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const int i = i0 + q;
      if (i < NI) {  // uniform
        if (i * 512 + 8 * lane < D) {
          float wv[EW][8];
#pragma unroll
          for (int e = 0; e < EW; ++e) wr[q][e].unpack(wv[e]);
#pragma unroll
          for (int t = 0; t < TT; ++t) {
            float xv[8];
            xr[q][t].unpack(xv);
#pragma unroll
            for (int e = 0; e < EW; ++e)
#pragma unroll
              for (int c = 0; c < 8; ++c) acc[t][e] = __builtin_fmaf(xv[c], wv[e][c], acc[t][e]);
          }
        }
        load(q, min(i + P, NI - 1));
      }
    }
  }
  logits_tree_store<TT, EW, CO>(acc, red + wave * 32 * 64, t0, ew0, T, E, logits);
}

// ---------------------------------------------------------------------------
// Hash routing: one thread per token of a 64-token block.  Slot j takes
// fmix32(tid + j * 0x9E3779B9) mod E, stepping forward (mod E) past experts
// this token already took; every weight is 1/k.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {  // MurmurHash3 finaliser
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

struct HashLds {
  unsigned long long smask[MOE_MAX_EXPERTS];
  int chosen[64][MOE_MAX_TOPK];
};

// 64-token block tb by a workgroup of NT threads (the first 64 take a token
// each); with MASK, the block's mask words mask[e][tb] are written whole.
template <int NT, bool MASK, bool CO = false>
__device__ __forceinline__ void hash_route_block(const int32_t* __restrict__ token_ids,
                                                 int64_t T, int E, int k,
                                                 int32_t* __restrict__ topk_idx,
                                                 float* __restrict__ topk_w,
                                                 uint64_t* __restrict__ mask, int64_t W,
                                                 int64_t tb, HashLds& L) {
  const int tt = threadIdx.x;
  if (MASK) {
    for (int e = tt; e < E; e += NT) L.smask[e] = 0ull;
    __syncthreads();
  }
  const int64_t t = tb * 64 + tt;
  if (tt < 64 && t < T) {
    const uint32_t tid = (uint32_t)token_ids[t];
    const float wk = 1.0f / (float)k;
    for (int j = 0; j < k; ++j) {
      uint32_t c = fmix32(tid + (uint32_t)j * 0x9E3779B9u) % (uint32_t)E;
      for (;;) {
        bool dup = false;
        for (int q = 0; q < j; ++q) dup |= (L.chosen[tt][q] == (int)c);
        if (!dup) break;
        c = (c + 1u) % (uint32_t)E;
      }
      L.chosen[tt][j] = (int)c;
      Out<CO>::put(&topk_idx[t * k + j], (int32_t)c);
      Out<CO>::put(&topk_w[t * k + j], wk);
      if (MASK) atomicOr(&L.smask[c], 1ull << tt);
    }
  }
  if (MASK) {
    __syncthreads();
    for (int e = tt; e < E; e += NT)
      Out<CO>::put(reinterpret_cast<unsigned long long*>(&mask[(int64_t)e * W + tb]), L.smask[e]);
  }
}

}  // namespace moe
