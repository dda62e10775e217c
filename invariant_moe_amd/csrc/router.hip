// Routing kernels: router logits in a fixed fp32 order (VALU), sigmoid/softmax
// keys with the library's own exp, wave-level top-k, and hash routing.
//
// Learned routing is scores = W h followed by top-k ("6 基建与训练稳定性优化",
// section 6.3; the "V4" article, section 2.2, describes the router as a small
// linear layer giving E logits).  Hash routing maps hash(token id) mod E to an
// expert (same DeepSeek-V4 page, section 6.3).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "router_core.hpp"
#include "routing.hpp"

namespace moe {

// Router logits: one workgroup per tile of router_core.hpp (the fixed order
// of the routing contract, whatever the tile).
template <typename ACT, int TT, int EW>
__global__ __launch_bounds__(256) void k_router_logits(const ACT* __restrict__ x,
                                                       const ACT* __restrict__ w, int64_t T,
                                                       int D, int E, float* __restrict__ logits,
                                                       unsigned long long* __restrict__ zero_words,
                                                       int64_t n_zero) {
  __shared__ __align__(16) unsigned char smem[router_logits_smem_bytes<ACT, TT>()];
  clear_words(zero_words, n_zero, (int64_t)blockIdx.y * gridDim.x + blockIdx.x,
              (int64_t)gridDim.x * gridDim.y);
  router_logits_tile<ACT, TT, EW>(x, w, T, D, E, logits, blockIdx.x, blockIdx.y, smem);
}

// Router logits for small T: the same pairs, partials and order, with x and w
// chunks going straight to registers in a ring P steps deep (no LDS staging,
// no barrier in the loop).
template <typename ACT, int TT, int EW, int P>
__global__ __launch_bounds__(256) void k_router_logits_small(
    const ACT* __restrict__ x, const ACT* __restrict__ w, int64_t T, int D, int E,
    float* __restrict__ logits, unsigned long long* __restrict__ zero_words, int64_t n_zero) {
  __shared__ __align__(16) unsigned char smem[kRouterSmallSmemBytes];
  clear_words(zero_words, n_zero, (int64_t)blockIdx.y * gridDim.x + blockIdx.x,
              (int64_t)gridDim.x * gridDim.y);
  router_logits_small_tile<ACT, TT, EW, P>(x, w, T, D, E, logits, blockIdx.x, blockIdx.y, smem);
}

// ---------------------------------------------------------------------------
// Top-k, one wave per token (topk_token in routing.hpp: a token's selection
// is a long dependent chain, so tokens run side by side).  With a mask, each
// selected (token, expert) sets bit t%64 of word mask[e][t/64] (integer OR:
// order-free; the words were zeroed by the router-logits kernel).
// ---------------------------------------------------------------------------
template <int C>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits,
                                              const float* __restrict__ bias, int64_t T, int E,
                                              int k, int mode, int32_t* __restrict__ topk_idx,
                                              float* __restrict__ topk_w,
                                              unsigned long long* __restrict__ mask, int64_t W) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave; no workgroup barriers below
  int my_id;
  if (topk_token<C>(logits + t * E, bias, E, k, mode, topk_idx + t * k, topk_w + t * k, my_id) &&
      mask)
    atomicOr(&mask[(int64_t)my_id * W + (t >> 6)], 1ull << (t & 63));
}

// ---------------------------------------------------------------------------
// Hash routing (router_core.hpp): one 64-thread workgroup per 64-token block.
// ---------------------------------------------------------------------------
template <bool MASK>
__global__ __launch_bounds__(64) void k_hash_route(const int32_t* __restrict__ token_ids,
                                                   int64_t T, int E, int k,
                                                   int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w,
                                                   uint64_t* __restrict__ mask, int64_t W) {
  __shared__ HashLds L;
  hash_route_block<64, MASK>(token_ids, T, E, k, topk_idx, topk_w, mask, W, blockIdx.x, L);
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

template <int TT, int EW, int P>
static void launch_logits_small(const void* x, int act, const void* w, int64_t T, int D, int E,
                                float* logits, unsigned long long* zw, int64_t nz,
                                hipStream_t s) {
  dim3 grid((unsigned)((T + TT - 1) / TT), (unsigned)((E + 4 * EW - 1) / (4 * EW)));
  if (act == MOE_BF16)
    hipLaunchKernelGGL((k_router_logits_small<uint16_t, TT, EW, P>), grid, dim3(256), 0, s,
                       (const uint16_t*)x, (const uint16_t*)w, T, D, E, logits, zw, nz);
  else
    hipLaunchKernelGGL((k_router_logits_small<float, TT, EW, P>), grid, dim3(256), 0, s,
                       (const float*)x, (const float*)w, T, D, E, logits, zw, nz);
}

hipError_t launch_router_logits(const void* x, int act, const void* w, int64_t T, int D, int E,
                                float* logits, uint64_t* zero, int64_t n_zero, hipStream_t s) {
  if (T == 0) return hipSuccess;
  unsigned long long* zw = reinterpret_cast<unsigned long long*>(zero);
  const int64_t nz = zero ? n_zero : 0;
  // Tile choice only changes how many (token, expert) pairs a workgroup holds
  // and how x reaches the lanes; every pair's logit is the same fixed chain.
  // Small T (decode): register ring, latency bound.  Larger T: x staged
  // through LDS once per workgroup (measured faster from a few hundred tokens).
  if (((T + 15) / 16) * ((E + 15) / 16) >= 1024)
    launch_logits_cfg<16, 4>(x, act, w, T, D, E, logits, zw, nz, s);
  else if (T > 128)
    launch_logits_cfg<4, 2>(x, act, w, T, D, E, logits, zw, nz, s);
  else if (T >= 16)
    launch_logits_small<4, 2, 4>(x, act, w, T, D, E, logits, zw, nz, s);
  else if (T >= 8)  // measured at T=8: 16.5 us vs 21.3 us for the 4 x 2 tile
    launch_logits_small<2, 1, 16>(x, act, w, T, D, E, logits, zw, nz, s);
  else  // 16 stages of 512 in flight: a whole 7168-wide row per lane at once
    launch_logits_small<1, 1, 16>(x, act, w, T, D, E, logits, zw, nz, s);
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
