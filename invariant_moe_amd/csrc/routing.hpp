// Routing math shared by the routing kernels: the library's fp32 exp and
// sigmoid, and the per-token top-k selection.
//
// Learned routing is scores = W h followed by top-k ("6 基建与训练稳定性优化",
// section 6.3; the "V4" article, section 2.2, describes the router as a small
// linear layer giving E logits).
#pragma once

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

__device__ __forceinline__ float routing_exp(float x) {
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
// Top-k of one token by one wave, C = ceil(E/64) expert slots per lane
// (expert e = lane + 64 c).  Selection order: larger key first, then lower
// expert id; keys compare as floats (+0 == -0).  A NaN key is treated as -inf
// so the selection stays a total order (inputs are required to be finite;
// this only keeps the kernel memory-safe).  Round r picks the best key not
// yet taken: keys are mapped to order-preserving uint32 codes, the wave
// maximum comes from four DPP steps within each row of 16 lanes and a scalar
// maximum over the four rows, and the winner is the lowest expert id holding
// that code (ballots in ascending id order).  Lane r keeps the rank-r winner.
// The weights' normaliser sums the selected terms in ascending expert id.
// Writes idx[0..k) and w[0..k) of the token; lanes r < k return their expert
// in my_id and true.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t key_code(float kk) {
  if (kk == 0.0f) kk = 0.0f;  // -0 -> +0
  const uint32_t u = __float_as_uint(kk);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // > 0 for every non-NaN key
}

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Maximum over the 64 lanes, returned uniform (scalar).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax32(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = umax32(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = umax32(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  v = umax32(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return umax32(umax32(r0, r1), umax32(r2, r3));
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Raw loads of one token's logits (lane + 64 c) and of the bias, kept apart
// from the selection so that a caller can issue the next token's loads early.
template <int C>
__device__ __forceinline__ void topk_load(const float* __restrict__ row, int E, float (&raw)[C]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = lane + 64 * c;
    raw[c] = e < E ? row[e] : 0.0f;
  }
}

template <int C, bool CO = false>
__device__ __forceinline__ bool topk_select(const float (&raw)[C], const float (&bias_v)[C],
                                            bool has_bias, int E, int k, int mode,
                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                            int& my_id_out) {
  const int lane = threadIdx.x & 63;
  uint32_t code[C];  // 0 = no expert / already taken
  float val[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = lane + 64 * c;
    code[c] = 0u;
    val[c] = 0.0f;
    if (e < E) {
      const float l = raw[c];
      const float sc = (mode == MOE_ROUTE_SIGMOID) ? routing_sigmoid(l) : l;
      float kk = has_bias ? sc + bias_v[c] : sc;
      if (kk != kk) kk = -__builtin_inff();
      code[c] = key_code(kk);
      val[c] = sc;
    }
  }
  int my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint32_t best = code[0];
#pragma unroll
    for (int c = 1; c < C; ++c) best = umax32(best, code[c]);
    const uint32_t m = wave_max_u32(best);
    int win = 0;  // k <= E: some expert holds the maximum
#pragma unroll
    for (int c = C - 1; c >= 0; --c) {  // the lowest slot with a hit wins
      const unsigned long long hit = __ballot(code[c] == m);
      if (hit) win = 64 * c + __builtin_ctzll(hit);
    }
    const int owner = win & 63, wc = win >> 6;
    float ov = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (c == wc) {
        ov = val[c];
        if (lane == owner) code[c] = 0u;
      }
    ov = readlane_f32(ov, owner);
    if (lane == r) {
      my_id = win;
      my_val = ov;
    }
  }
  // Softmax shift: the largest selected logit (an exact maximum, so the same
  // bits whatever the order).  With a bias the rank-0 expert need not hold it,
  // and exp(l - l_rank0) could overflow.
  float top = readlane_f32(my_val, 0);
  for (int q = 1; q < k; ++q) top = fmaxf(top, readlane_f32(my_val, q));
  const bool act = lane < k;
  const float z = !act ? 0.0f
                       : (mode == MOE_ROUTE_SOFTMAX ? routing_exp(my_val - top) : my_val);
  int pos = 0;  // rank of this slot by ascending expert id
  for (int q = 0; q < k; ++q) pos += (__builtin_amdgcn_readlane(my_id, q) < my_id) ? 1 : 0;
  float Z = 0.0f;
  for (int i = 0; i < k; ++i) {
    const unsigned long long b = __ballot(act && pos == i);
    const int src = b ? __builtin_ctzll(b) : 0;
    Z = Z + readlane_f32(z, src);
  }
  if (act) {
    Out<CO>::put(&idx[lane], my_id);
    Out<CO>::put(&w[lane], z / Z);
  }
  my_id_out = my_id;
  return act;
}

template <int C>
__device__ __forceinline__ void topk_load_bias(const float* __restrict__ bias, int E,
                                               float (&bias_v)[C]) {
  if (bias) {
    topk_load<C>(bias, E, bias_v);
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) bias_v[c] = 0.0f;
  }
}

template <int C, bool CO = false>
__device__ __forceinline__ bool topk_token(const float* __restrict__ logit_row,
                                           const float* __restrict__ bias, int E, int k,
                                           int mode, int32_t* __restrict__ idx,
                                           float* __restrict__ w, int& my_id_out) {
  float raw[C], bias_v[C];
  topk_load<C>(logit_row, E, raw);
  topk_load_bias<C>(bias, E, bias_v);
  return topk_select<C, CO>(raw, bias_v, bias != nullptr, E, k, mode, idx, w, my_id_out);
}

}  // namespace moe
