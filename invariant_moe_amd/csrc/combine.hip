// Weighted combine ("MoE finalize"): per token, the k expert outputs are
// summed in fp32 in ascending expert id with fused multiply-adds, the shared
// expert's output is added after the routed sum, and the result is rounded
// once.  Keeping all k contributions in fp32 and casting once, and adding the
// shared expert after the finalize, follow the Fireworks parity post
// ("MoE 模型中的訓練與推論一致性：數值漂移發生之處", trap 3 and the Qwen3.5-MoE
// case study).  The order is fixed per token, so the bits do not depend on T.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <typename ACT>
struct Row8;
template <>
struct Row8<uint16_t> {
  __device__ static void load(const uint16_t* p, float (&v)[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
    v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  }
  __device__ static void store(uint16_t* p, const float (&v)[8]) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                              pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  }
};
template <>
struct Row8<float> {
  __device__ static void load(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ static void store(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// TPT threads per token (a power of two covering D/8, at most 256), 256/TPT
// tokens per workgroup; each thread owns 8 consecutive features per pass.
// Wide rows are split over gridDim.y workgroups (one pass per thread).
template <typename ACT>
__global__ __launch_bounds__(256) void k_combine(const ACT* __restrict__ eo,
                                                 const int32_t* __restrict__ topk_idx,
                                                 const float* __restrict__ topk_w,
                                                 const int32_t* __restrict__ pair_row,
                                                 const ACT* __restrict__ shared, int64_t T, int k,
                                                 int D, int TPT, ACT* __restrict__ y) {
  __shared__ int64_t s_rows[256 / 64][MOE_MAX_TOPK];
  __shared__ float s_ws[256 / 64][MOE_MAX_TOPK];
  const int sub = threadIdx.x / TPT, lt = threadIdx.x % TPT;
  const int64_t t = (int64_t)blockIdx.x * (256 / TPT) + sub;
  int64_t* s_row = s_rows[sub];
  float* s_w = s_ws[sub];
  if (t < T && lt < k) {
    // position of this slot in ascending expert id
    const int j = lt;
    const int e = topk_idx[t * k + j];
    int pos = 0;  // rank by (expert id, slot): a permutation even for repeated ids
    for (int q = 0; q < k; ++q) {
      const int eq = topk_idx[t * k + q];
      pos += (eq < e || (eq == e && q < j)) ? 1 : 0;
    }
    const int64_t R = T * k;
    int64_t row = pair_row[t * k + j];
    row = row < 0 ? 0 : (row >= R ? R - 1 : row);  // memory safety outside the contract
    s_row[pos] = row;
    s_w[pos] = topk_w[t * k + j];
  }
  __syncthreads();
  if (t >= T) return;
  for (int d = (blockIdx.y * TPT + lt) * 8; d < D; d += gridDim.y * TPT * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < k; ++q) {
      float v[8];
      Row8<ACT>::load(eo + s_row[q] * D + d, v);
      const float wq = s_w[q];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_fmaf(wq, v[c], acc[c]);
    }
    if (shared) {
      float sv[8];
      Row8<ACT>::load(shared + t * D + d, sv);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = acc[c] + sv[c];
    }
    Row8<ACT>::store(y + t * D + d, acc);
  }
}

hipError_t launch_combine(const void* eo, const int32_t* topk_idx, const float* topk_w,
                          const int32_t* pair_row, const void* shared, int64_t T, int k, int D,
                          int act, void* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int tpt = 64;  // >= k (k <= 32) so the slot setup fits in one token's threads
  while (tpt < 256 && tpt * 8 < D) tpt *= 2;
  const dim3 grid((unsigned)((T + (256 / tpt) - 1) / (256 / tpt)),
                   (unsigned)((D / 8 + tpt - 1) / tpt));
  if (act == MOE_BF16)
    hipLaunchKernelGGL(k_combine<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)eo, topk_idx,
                       topk_w, pair_row, (const uint16_t*)shared, T, k, D, tpt, (uint16_t*)y);
  else
    hipLaunchKernelGGL(k_combine<float>, grid, dim3(256), 0, s, (const float*)eo, topk_idx,
                       topk_w, pair_row, (const float*)shared, T, k, D, tpt, (float*)y);
  return hipGetLastError();
}

}  // namespace moe
