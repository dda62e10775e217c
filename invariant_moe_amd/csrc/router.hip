// Routing kernels: router logits in a fixed fp32 order (VALU), sigmoid/softmax
// keys with the library's own exp, wave-level top-k, and hash routing.
//
// Learned routing is scores = W h followed by top-k ("6 基建与训练稳定性优化",
// section 6.3; the "V4" article, section 2.2, describes the router as a small
// linear layer giving E logits).  Hash routing maps hash(token id) mod E to an
// expert (same DeepSeek-V4 page, section 6.3).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Routing exp (fp32): Cody–Waite argument reduction x = n ln2 + r with
// n = rint(x log2e) and ln2 split into fp32(ln2) + fp32(ln2 - fp32(ln2)),
// then the degree-7 Taylor polynomial sum_{j<=7} r^j / j! with fp32-rounded
// coefficients by Horner's rule with fused multiply-adds, then p * 2^n (two
// exact power-of-two scalings outside [2^-126, 2^127]).  Written from the
// mathematics; the routing keys depend on every bit of it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float pow2i(int m) {  // 2^m for -126 <= m <= 127
  return __uint_as_float((uint32_t)(m + 127) << 23);
}

__device__ float routing_exp(float x) {
  if (x != x) return x;
  if (x > 89.0f) return __builtin_inff();
  if (x < -104.0f) return 0.0f;
  const float n = __builtin_rintf(x * 0x1.715476p+0f);
  float r = __builtin_fmaf(-n, 0x1.62e430p-1f, x);
  r = __builtin_fmaf(-n, -0x1.05c610p-29f, r);
  float p = 0x1.a01a02p-13f;               // 1/7!
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  const int ni = (int)n;
  if (ni > 127) return (p * pow2i(ni - 64)) * pow2i(64);
  if (ni < -126) return (p * pow2i(ni + 64)) * pow2i(-64);
  return p * pow2i(ni);
}

__device__ __forceinline__ float routing_sigmoid(float l) {
  return 1.0f / (1.0f + routing_exp(-l));
}

// ---------------------------------------------------------------------------
// Router logits.  One workgroup = TT tokens x (4 * EW) experts; wave w owns
// experts [e0 + w*EW, e0 + (w+1)*EW).  Lane j owns partial sum j of every
// (token, expert) pair: it accumulates elements d = 8j + 512 i + c (c = 0..7),
// i increasing, with fmaf — the fixed order of the routing contract.  The 64
// partials of a pair are then summed by one lane in the fixed pairwise tree
// (partial[j] += partial[j + m], m = 32..1) after a transpose through LDS.
// The result of a pair does not depend on TT, EW, T or the grid.
// ---------------------------------------------------------------------------
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

template <typename ACT, int TT, int EW>
__global__ __launch_bounds__(256) void k_router_logits(const ACT* __restrict__ x,
                                                       const ACT* __restrict__ w, int64_t T,
                                                       int D, int E, float* __restrict__ logits,
                                                       unsigned long long* __restrict__ zero_words,
                                                       int64_t n_zero) {
  // clear the (expert, token-block) words the top-k kernel ORs into
  if (zero_words) {
    const int64_t nb = (int64_t)gridDim.x * gridDim.y;
    const int64_t b = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (int64_t i = b * 256 + threadIdx.x; i < n_zero; i += nb * 256) zero_words[i] = 0ull;
  }
  constexpr int NP = TT * EW;  // pairs per wave
  constexpr int XS_BYTES = TT * 512 * (int)sizeof(ACT);
  constexpr int RED_BYTES = 4 * 32 * 64 * 4;
  constexpr int SMEM = XS_BYTES > RED_BYTES ? XS_BYTES : RED_BYTES;
  __shared__ __align__(16) unsigned char smem[SMEM];
  ACT* xs = reinterpret_cast<ACT*>(smem);
  float* red = reinterpret_cast<float*>(smem);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int ew0 = blockIdx.y * 4 * EW + wave * EW;

  float acc[TT][EW];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int e = 0; e < EW; ++e) acc[t][e] = 0.0f;

  for (int i0 = 0; i0 < D; i0 += 512) {
    __syncthreads();
    for (int c = threadIdx.x; c < TT * 64; c += 256) {
      const int tt = c >> 6, j = c & 63;
      const int d = i0 + 8 * j;
      ACT* dst = xs + tt * 512 + 8 * j;
      if (t0 + tt < T && d < D) {
        const ACT* src = x + (t0 + tt) * (int64_t)D + d;
        if (sizeof(ACT) == 2) {
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
          reinterpret_cast<uint4*>(dst)[0] = reinterpret_cast<const uint4*>(src)[0];
          reinterpret_cast<uint4*>(dst)[1] = reinterpret_cast<const uint4*>(src)[1];
        }
      } else {
        if (sizeof(ACT) == 2) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(0, 0, 0, 0);
        } else {
          reinterpret_cast<uint4*>(dst)[0] = make_uint4(0, 0, 0, 0);
          reinterpret_cast<uint4*>(dst)[1] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    __syncthreads();
    const int d = i0 + 8 * lane;
    if (d < D) {
      float wv[EW][8];
#pragma unroll
      for (int e = 0; e < EW; ++e) {
        if (ew0 + e < E) {
          ActIO<ACT>::load8(w + (int64_t)(ew0 + e) * D + d, wv[e]);
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) wv[e][c] = 0.0f;
        }
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        float xv[8];
        ActIO<ACT>::load8(xs + t * 512 + 8 * lane, xv);
#pragma unroll
        for (int e = 0; e < EW; ++e)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[t][e] = __builtin_fmaf(xv[c], wv[e][c], acc[t][e]);
      }
    }
  }

  // Fixed-tree reduction of the 64 partials of each pair, 32 pairs per round.
  // Element (pair q, partial j) sits at q*64 + (j ^ q) so that both the
  // write (fixed q, lanes j) and the read (lanes q, fixed j) hit distinct banks.
  float* myred = red + wave * 32 * 64;
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
      if (t < T && e < E) logits[t * E + e] = p[0];
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k, one wave per token, C = ceil(E/64) expert slots per lane.  Selection
// key order: larger key first, then lower expert id; keys are compared as
// floats (+0 == -0).  A NaN key is treated as -inf so the selection stays a
// total order (inputs are required to be finite; this only keeps the kernel
// memory-safe).  k rounds of a 64-lane butterfly arg-max; lane r keeps the
// rank-r winner.  The weights' normaliser sums the selected terms in ascending
// expert id.  With a mask, each selected (token, expert) sets bit t%64 of
// word mask[e][t/64] (integer OR: order-free; the words were zeroed by the
// logits kernel).
// ---------------------------------------------------------------------------
struct Cand {
  float key;
  int id;  // -1 = none
};

__device__ __forceinline__ bool cand_better(const Cand& a, const Cand& b) {
  if (a.id < 0) return false;
  if (b.id < 0) return true;
  return a.key > b.key || (a.key == b.key && a.id < b.id);
}

template <int C>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits,
                                              const float* __restrict__ bias, int64_t T, int E,
                                              int k, int mode, int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w,
                                              unsigned long long* __restrict__ mask, int64_t W) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave; no workgroup barriers below
  float key[C], val[C];
  uint32_t taken = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = lane + 64 * c;
    key[c] = 0.0f;
    val[c] = 0.0f;
    if (e < E) {
      const float l = logits[t * E + e];
      const float sc = (mode == MOE_ROUTE_SIGMOID) ? routing_sigmoid(l) : l;
      float kk = bias ? sc + bias[e] : sc;
      if (kk != kk) kk = -__builtin_inff();
      key[c] = kk;
      val[c] = sc;
    } else {
      taken |= 1u << c;
    }
  }
  int my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
    Cand best{0.0f, -1};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      Cand cc{key[c], ((taken >> c) & 1u) ? -1 : lane + 64 * c};
      if (cand_better(cc, best)) best = cc;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      Cand o{__shfl_xor(best.key, m), __shfl_xor(best.id, m)};
      if (cand_better(o, best)) best = o;
    }
    const int win = best.id < 0 ? 0 : best.id;  // k <= E: always a winner
    const int owner = win & 63;
    float ov = 0.0f;
    if (lane == owner) {
      taken |= 1u << (win >> 6);
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (c == (win >> 6)) ov = val[c];
    }
    ov = __shfl(ov, owner);
    if (lane == r) {
      my_id = win;
      my_val = ov;
    }
  }
  const float top = __shfl(my_val, 0);
  const bool act = lane < k;
  const float z = !act ? 0.0f
                       : (mode == MOE_ROUTE_SOFTMAX ? routing_exp(my_val - top) : my_val);
  int pos = 0;  // rank of this slot by ascending expert id
  for (int q = 0; q < k; ++q) pos += (__shfl(my_id, q) < my_id) ? 1 : 0;
  float Z = 0.0f;
  for (int i = 0; i < k; ++i) {
    const unsigned long long b = __ballot(act && pos == i);
    const int src = b ? __builtin_ctzll(b) : 0;
    Z = Z + __shfl(z, src);
  }
  if (act) {
    topk_idx[t * k + lane] = my_id;
    topk_w[t * k + lane] = z / Z;
    if (mask) atomicOr(&mask[(int64_t)my_id * W + (t >> 6)], 1ull << (t & 63));
  }
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

template <bool MASK>
__global__ __launch_bounds__(64) void k_hash_route(const int32_t* __restrict__ token_ids,
                                                   int64_t T, int E, int k,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w,
                                                   uint64_t* __restrict__ mask, int64_t W) {
  __shared__ unsigned long long smask[MOE_MAX_EXPERTS];
  __shared__ int chosen[64][MOE_MAX_TOPK];
  const int tt = threadIdx.x;
  const int64_t tb = blockIdx.x;
  if (MASK) {
    for (int e = tt; e < E; e += 64) smask[e] = 0ull;
    __syncthreads();
  }
  const int64_t t = tb * 64 + tt;
  if (t < T) {
    const uint32_t tid = (uint32_t)token_ids[t];
    const float wk = 1.0f / (float)k;
    for (int j = 0; j < k; ++j) {
      uint32_t c = fmix32(tid + (uint32_t)j * 0x9E3779B9u) % (uint32_t)E;
      for (;;) {
        bool dup = false;
        for (int q = 0; q < j; ++q) dup |= (chosen[tt][q] == (int)c);
        if (!dup) break;
        c = (c + 1u) % (uint32_t)E;
      }
      chosen[tt][j] = (int)c;
      topk_idx[t * k + j] = (int32_t)c;
      topk_w[t * k + j] = wk;
      if (MASK) atomicOr(&smask[c], 1ull << tt);
    }
  }
  if (MASK) {
    __syncthreads();
    for (int e = tt; e < E; e += 64) mask[(int64_t)e * W + tb] = smask[e];
  }
}

// Elementwise routing scores (sigmoid or exp), exposed for callers.
__global__ __launch_bounds__(256) void k_routing_scores(const float* __restrict__ in, int64_t n,
                                                        int mode, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * 256)
    out[i] = (mode == MOE_ROUTE_SIGMOID) ? routing_sigmoid(in[i]) : routing_exp(in[i]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int TT, int EW>
static void launch_logits_cfg(const void* x, int act, const void* w, int64_t T, int D, int E,
                              float* logits, unsigned long long* zw, int64_t nz, hipStream_t s) {
  dim3 grid((unsigned)((T + TT - 1) / TT), (unsigned)((E + 4 * EW - 1) / (4 * EW)));
  if (act == MOE_BF16)
    hipLaunchKernelGGL((k_router_logits<uint16_t, TT, EW>), grid, dim3(256), 0, s,
                       (const uint16_t*)x, (const uint16_t*)w, T, D, E, logits, zw, nz);
  else
    hipLaunchKernelGGL((k_router_logits<float, TT, EW>), grid, dim3(256), 0, s, (const float*)x,
                       (const float*)w, T, D, E, logits, zw, nz);
}

hipError_t launch_router_logits(const void* x, int act, const void* w, int64_t T, int D, int E,
                                float* logits, uint64_t* zero_mask, hipStream_t s) {
  if (T == 0) return hipSuccess;
  unsigned long long* zw = reinterpret_cast<unsigned long long*>(zero_mask);
  const int64_t nz = zero_mask ? (int64_t)E * ((T + 63) / 64) : 0;
  // Tile choice only changes how many (token, expert) pairs a workgroup holds
  // (enough workgroups to stream the router weights); every pair's logit is
  // the same fixed chain.
  if (((T + 15) / 16) * ((E + 31) / 32) >= 512)
    launch_logits_cfg<16, 8>(x, act, w, T, D, E, logits, zw, nz, s);
  else if (T >= 8)
    launch_logits_cfg<4, 2>(x, act, w, T, D, E, logits, zw, nz, s);
  else
    launch_logits_cfg<1, 1>(x, act, w, T, D, E, logits, zw, nz, s);
  return hipGetLastError();
}

template <int C>
static void launch_topk_cfg(const float* logits, const float* bias, int64_t T, int E, int k,
                            int mode, int32_t* idx, float* w, uint64_t* mask, hipStream_t s) {
  const int64_t W = (T + 63) / 64;
  hipLaunchKernelGGL(k_topk<C>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits, bias, T,
                     E, k, mode, idx, w, reinterpret_cast<unsigned long long*>(mask), W);
}

hipError_t launch_topk(const float* logits, const float* bias, int64_t T, int E, int k, int mode,
                       int32_t* idx, float* w, uint64_t* mask, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int c = (E + 63) / 64;
  if (c <= 1) launch_topk_cfg<1>(logits, bias, T, E, k, mode, idx, w, mask, s);
  else if (c <= 2) launch_topk_cfg<2>(logits, bias, T, E, k, mode, idx, w, mask, s);
  else if (c <= 4) launch_topk_cfg<4>(logits, bias, T, E, k, mode, idx, w, mask, s);
  else if (c <= 8) launch_topk_cfg<8>(logits, bias, T, E, k, mode, idx, w, mask, s);
  else launch_topk_cfg<16>(logits, bias, T, E, k, mode, idx, w, mask, s);
  return hipGetLastError();
}

hipError_t launch_hash_route(const int32_t* token_ids, int64_t T, int E, int k, int32_t* idx,
                             float* w, uint64_t* mask, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t W = (T + 63) / 64;
  if (mask)
    hipLaunchKernelGGL(k_hash_route<true>, dim3((unsigned)W), dim3(64), 0, s, token_ids, T, E,
                       k, idx, w, mask, W);
  else
    hipLaunchKernelGGL(k_hash_route<false>, dim3((unsigned)W), dim3(64), 0, s, token_ids, T, E,
                       k, idx, w, (uint64_t*)nullptr, W);
  return hipGetLastError();
}

hipError_t launch_routing_scores(const float* in, int64_t n, int mode, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 262144) blocks = 262144;
  hipLaunchKernelGGL(k_routing_scores, dim3((unsigned)blocks), dim3(256), 0, s, in, n, mode, out);
  return hipGetLastError();
}

}  // namespace moe
