// The MoE finalize (weighted combine) as device functions: per token, the k
// expert outputs are summed in fp32 in ascending expert id with fused
// multiply-adds, the shared expert's output is added after the routed sum, and
// the result is rounded once (the Fireworks parity post,
// "MoE 模型中的訓練與推論一致性：數值漂移發生之處", trap 3 and the Qwen3.5-MoE
// case study).  Used by the combine kernels and the single-launch layer kernel.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <typename ACT>
struct Row8;
template <>
struct Row8<uint16_t> {
  using Raw = uint4;
  __device__ static Raw load_raw(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void unpack(const Raw& q, float (&v)[8]) {
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
    v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  }
  __device__ static void load(const uint16_t* p, float (&v)[8]) { unpack(load_raw(p), v); }
  __device__ static void store(uint16_t* p, const float (&v)[8]) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
};
template <>
struct Row8<float> {
  struct Raw {
    float4 a, b;
  };
  __device__ static Raw load_raw(const float* p) {
    return Raw{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
  }
  __device__ static void unpack(const Raw& q, float (&v)[8]) {
    v[0] = q.a.x; v[1] = q.a.y; v[2] = q.a.z; v[3] = q.a.w;
    v[4] = q.b.x; v[5] = q.b.y; v[6] = q.b.z; v[7] = q.b.w;
  }
  __device__ static void load(const float* p, float (&v)[8]) { unpack(load_raw(p), v); }
  __device__ static void store(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// Slot setup of token t by the threads lt = 0..63 of one wave (lt == lane):
// the first k lanes load their slot, and each slot's position in ascending
// expert id (ties by slot: a permutation even for repeated ids) comes from the
// other lanes' ids through shuffles.  Loads at clamped in-range indices for
// every lane, so all three go out together (T >= 1 here).  The caller
// synchronises before reading s_row / s_w.
__device__ __forceinline__ void combine_slots(const int32_t* __restrict__ topk_idx,
                                              const float* __restrict__ topk_w,
                                              const int32_t* __restrict__ pair_row, int64_t t,
                                              int64_t T, int k, int lt, int64_t* s_row,
                                              float* s_w) {
  const bool slot = t < T && lt < k;
  const int64_t pidx = (t < T ? t : T - 1) * k + (lt < k ? lt : k - 1);
  const int e_ld = topk_idx[pidx];
  const int64_t row_ld = pair_row[pidx];
  const float w_ld = topk_w[pidx];
  const int e = slot ? e_ld : 0;
  int pos = 0;
  for (int q = 0; q < k; ++q) {
    const int eq = __shfl(e, q);  // lane q of this token's threads
    pos += (eq < e || (eq == e && q < lt)) ? 1 : 0;
  }
  if (slot) {
    const int64_t R = T * k;
    const int64_t row = row_ld < 0 ? 0 : (row_ld >= R ? R - 1 : row_ld);  // memory safety
    s_row[pos] = row;
    s_w[pos] = w_ld;
  }
}

// The routed sum of one 8-feature chunk at feature d: acc = fmaf(w, o, acc)
// over the token's slots in ascending expert id, from acc = +0.  Up to eight
// expert rows in flight (rows past k are loaded from the last slot and not
// used).
template <typename ACT>
__device__ __forceinline__ void combine_chunk(const ACT* __restrict__ eo, const int64_t* s_row,
                                              const float* s_w, int k, int D, int d,
                                              float (&acc)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  for (int q0 = 0; q0 < k; q0 += 8) {
    typename Row8<ACT>::Raw raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      raw[u] = Row8<ACT>::load_raw(eo + s_row[min(q0 + u, k - 1)] * D + d);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u < k) {
        float v[8];
        Row8<ACT>::unpack(raw[u], v);
        const float wq = s_w[q0 + u];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __builtin_fmaf(wq, v[c], acc[c]);
      }
  }
}

// One combine tile by a workgroup of 256 threads: TPT threads per token (a
// power of two covering D/8, at most 256), 256/TPT tokens per tile (token tile
// bx); each thread owns 8 consecutive features per pass.  Wide rows are split
// over gy feature tiles (this is feature tile by, one pass per thread).
struct CombineLds {
  int64_t s_rows[256 / 64][MOE_MAX_TOPK];
  float s_ws[256 / 64][MOE_MAX_TOPK];
};

template <typename ACT>
__device__ __forceinline__ void combine_tile(const ACT* __restrict__ eo,
                                             const int32_t* __restrict__ topk_idx,
                                             const float* __restrict__ topk_w,
                                             const int32_t* __restrict__ pair_row,
                                             const ACT* __restrict__ shared, int64_t T, int k,
                                             int D, int TPT, ACT* __restrict__ y, int64_t bx,
                                             int by, int gy, CombineLds& L) {
  const int sub = threadIdx.x / TPT, lt = threadIdx.x % TPT;
  const int64_t t = bx * (256 / TPT) + sub;
  int64_t* s_row = L.s_rows[sub];
  float* s_w = L.s_ws[sub];
  const int d0 = (by * TPT + lt) * 8;
  const int64_t dstep = (int64_t)gy * TPT * 8;
  // The shared expert's row for this thread's first pass does not depend on
  // the routing: its load goes out first.
  // Unconditional, at a clamped in-range address (the expert output, which has
  // at least T*D elements, stands in when there is no shared expert), so that
  // no branch waits for it.
  const ACT* sbase = shared ? shared : eo;
  const typename Row8<ACT>::Raw sv0 =
      Row8<ACT>::load_raw(sbase + (t < T ? t : T - 1) * D + (d0 < D ? d0 : D - 8));
  // Slot setup by the first k lanes of the token (one wave, TPT >= 64 > k).
  if (lt < 64) combine_slots(topk_idx, topk_w, pair_row, t, T, k, lt, s_row, s_w);
  __syncthreads();
  if (t < T) {
    for (int d = d0; d < D; d += dstep) {
      float acc[8];
      combine_chunk(eo, s_row, s_w, k, D, d, acc);
      if (shared) {
        float sv[8];
        if (d == d0)
          Row8<ACT>::unpack(sv0, sv);
        else
          Row8<ACT>::load(shared + t * D + d, sv);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = acc[c] + sv[c];
      }
      Row8<ACT>::store(y + t * D + d, acc);
    }
  }
}

}  // namespace moe
