// Weighted combine ("MoE finalize"): per token, the k expert outputs are
// summed in fp32 in ascending expert id with fused multiply-adds, the shared
// expert's output is added after the routed sum, and the result is rounded
// once.  Keeping all k contributions in fp32 and casting once, and adding the
// shared expert after the finalize, follow the Fireworks parity post
// ("MoE 模型中的訓練與推論一致性：數值漂移發生之處", trap 3 and the Qwen3.5-MoE
// case study).  The order is fixed per token, so the bits do not depend on T.
#include "combine_core.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// The combine: one tile of combine_core.hpp per workgroup.
template <typename ACT>
__global__ __launch_bounds__(256) void k_combine(const ACT* __restrict__ eo,
                                                 const int32_t* __restrict__ topk_idx,
                                                 const float* __restrict__ topk_w,
                                                 const int32_t* __restrict__ pair_row,
                                                 const ACT* __restrict__ shared, int64_t T, int k,
                                                 int D, int TPT, ACT* __restrict__ y) {
  __shared__ CombineLds L;
  combine_tile<ACT>(eo, topk_idx, topk_w, pair_row, shared, T, k, D, TPT, y, blockIdx.x,
                    blockIdx.y, gridDim.y, L);
}

// ---------------------------------------------------------------------------
// Residual add + RMSNorm of the next block's input: the end of the unfused
// MoE tail in the Fireworks parity post (trap 3: finalize, += shared expert,
// then rmsnorm(out + residual)), RMSNorm as the forum article on MoE variants
// defines it (section "RMSNorm before up-projection"):
//   h = round(y + residual) (the new residual), normed = round(g * (h * inv)),
//   inv = 1 / sqrt(ss / D + eps), ss = sum of h^2.
// The post's point is that the norm's reduction tree changes with the thread
// layout of whichever kernel runs it; here ss has one order, fixed by D alone:
// kNormPartials partials, partial p summing h[d]^2 (fmaf, from +0) over the
// 8-feature chunks c = d / 8 with c % kNormPartials == p in increasing d, then
// the halving tree p += p + m for m = kNormPartials / 2, ..., 1.  TPT threads
// per token (a power of two, 64..kNormPartials) all compute that order:
// thread l owns partials l + TPT q, runs the tree steps m >= TPT in its
// registers and the rest across threads.  So the standalone norm and the norm
// fused into the combine (FUSED: y is the combine, rounded as the combine's
// output is) give the same bits, at every T and every TPT.
// ---------------------------------------------------------------------------
constexpr int kNormPartials = 1024;

template <typename ACT>
struct TailArgs {
  const ACT* eo;  // FUSED: expert outputs, slots and the shared expert's output
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* pair_row;
  const ACT* shared;
  const ACT* x;  // otherwise: the rows to normalise
  const ACT* residual;
  const ACT* gamma;
  float eps;
  int64_t T;
  int k, D;
  ACT* residual_out;
  ACT* normed;
};

template <typename ACT>
__device__ __forceinline__ float round_act(float v);
template <>
__device__ __forceinline__ float round_act<uint16_t>(float v) {
  return bf16_lo(f32_to_bf16_rne(v));
}
template <>
__device__ __forceinline__ float round_act<float>(float v) {
  return v;
}

template <typename ACT, bool FUSED, int TPT>
__global__ __launch_bounds__(TPT > 256 ? TPT : 256) void k_residual_rmsnorm(TailArgs<ACT> a) {
  constexpr int NT = TPT > 256 ? TPT : 256;
  constexpr int TPW = NT / TPT;             // tokens per workgroup
  constexpr int Q = kNormPartials / TPT;    // partials per thread = passes per round
  static_assert(TPT >= 64 && Q >= 1 && (TPT & (TPT - 1)) == 0, "TPT: power of two, 64..1024");
  __shared__ int64_t s_rows[TPW][MOE_MAX_TOPK];
  __shared__ float s_ws[TPW][MOE_MAX_TOPK];
  __shared__ float s_part[NT];
  __shared__ float s_total[TPW];
  using R8 = Row8<ACT>;
  const int sub = threadIdx.x / TPT, lt = threadIdx.x % TPT;
  const int64_t t = (int64_t)blockIdx.x * TPW + sub;
  const bool live = t < a.T;
  const int D = a.D;
  const int64_t row = (live ? t : a.T - 1) * D;
  // First-pass loads that do not depend on the routing go out first, at a
  // clamped in-range feature of a clamped token.
  const int dc = min(lt * 8, D - 8);
  const typename R8::Raw r0 = R8::load_raw(a.residual + row + dc);
  const ACT* ybase = FUSED ? (a.shared ? a.shared : a.eo) : a.x;
  const typename R8::Raw y0 = R8::load_raw(ybase + row + dc);
  if (FUSED) {
    if (lt < 64) combine_slots(a.topk_idx, a.topk_w, a.pair_row, t, a.T, a.k, lt, s_rows[sub],
                               s_ws[sub]);
    __syncthreads();
  }
  float part[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) part[q] = 0.f;
  float hreg[Q][8];  // the first Q passes (D <= 8 * kNormPartials) stay in registers
  // h for the chunk at feature d (pass j): the row value (combine or x) plus
  // the residual, rounded; stored as the new residual and summed into its
  // partial.
  auto pass = [&](int j, int d, float (&h)[8], float& pq) {
    float y[8], r[8];
    if (FUSED) {
      float acc[8];
      combine_chunk(a.eo, s_rows[sub], s_ws[sub], a.k, D, d, acc);
      if (a.shared) {
        float sv[8];
        if (j == 0)
          R8::unpack(y0, sv);
        else
          R8::load(a.shared + row + d, sv);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = acc[c] + sv[c];
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = round_act<ACT>(acc[c]);
    } else if (j == 0) {
      R8::unpack(y0, y);
    } else {
      R8::load(a.x + row + d, y);
    }
    if (j == 0)
      R8::unpack(r0, r);
    else
      R8::load(a.residual + row + d, r);
#pragma unroll
    for (int c = 0; c < 8; ++c) h[c] = round_act<ACT>(y[c] + r[c]);
    R8::store(a.residual_out + row + d, h);
#pragma unroll
    for (int c = 0; c < 8; ++c) pq = __builtin_fmaf(h[c], h[c], pq);
  };
  if (live) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int d = (lt + q * TPT) * 8;
      if (d < D) pass(q, d, hreg[q], part[q]);
    }
    for (int j0 = Q; (lt + j0 * TPT) * 8 < D; j0 += Q) {  // wider rows: partial q again
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int d = (lt + (j0 + q) * TPT) * 8;
        float h[8];
        if (d < D) pass(j0 + q, d, h, part[q]);
      }
    }
  }
  // the tree: steps m >= TPT within the thread, then across the token's threads
#pragma unroll
  for (int m = Q / 2; m >= 1; m /= 2)
#pragma unroll
    for (int q = 0; q < m; ++q) part[q] = part[q] + part[q + m];
  float v = part[0];
  if (TPT > 64) {
    s_part[threadIdx.x] = v;
    __syncthreads();
#pragma unroll
    for (int m = TPT / 2; m >= 64; m /= 2) {
      if (lt < m) s_part[threadIdx.x] = s_part[threadIdx.x] + s_part[threadIdx.x + m];
      __syncthreads();
    }
    v = s_part[threadIdx.x];
  }
  if (lt < 64) {
#pragma unroll
    for (int m = 32; m >= 1; m /= 2) v = v + __shfl_down(v, m);  // lane p += lane p + m
    if (lt == 0) s_total[sub] = v;
  }
  __syncthreads();
  if (!live) return;
  const float inv = 1.0f / sqrtf(s_total[sub] / (float)D + a.eps);
  auto out = [&](int d, const float (&h)[8]) {
    float g[8], o[8];
    R8::load(a.gamma + d, g);
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = g[c] * (h[c] * inv);
    R8::store(a.normed + row + d, o);
  };
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int d = (lt + q * TPT) * 8;
    if (d < D) out(d, hreg[q]);
  }
  for (int j = Q; (lt + j * TPT) * 8 < D; ++j) {  // wider rows: h from this thread's own stores
    const int d = (lt + j * TPT) * 8;
    float h[8];
    R8::load(a.residual_out + row + d, h);
    out(d, h);
  }
}

// Threads per token: one pass over the row, at least 256.  (Measured on the
// 7168-wide rows: 1024 threads per token is the fastest at T = 1, 64, 4096
// and 16384 alike; 256 threads with 3.5 passes is 8 % slower at T = 4096.)
static int tail_tpt(int D) {
  int tpt = 256;
  while (tpt < kNormPartials && tpt < D / 8) tpt *= 2;
  return tpt;
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

template <typename ACT, bool FUSED, int TPT>
static hipError_t launch_tail_tpt(const TailArgs<ACT>& a, hipStream_t s) {
  constexpr int NT = TPT > 256 ? TPT : 256;
  const int64_t grid = (a.T + NT / TPT - 1) / (NT / TPT);
  hipLaunchKernelGGL((k_residual_rmsnorm<ACT, FUSED, TPT>), dim3((unsigned)grid), dim3(NT), 0, s,
                     a);
  return hipGetLastError();
}

template <typename ACT, bool FUSED>
static hipError_t launch_tail(const TailArgs<ACT>& a, hipStream_t s) {
  switch (tail_tpt(a.D)) {
    case 256: return launch_tail_tpt<ACT, FUSED, 256>(a, s);
    case 512: return launch_tail_tpt<ACT, FUSED, 512>(a, s);
    default: return launch_tail_tpt<ACT, FUSED, 1024>(a, s);
  }
}

hipError_t launch_residual_rmsnorm(const void* x, const void* residual, const void* gamma,
                                   float eps, int64_t T, int D, int act, void* residual_out,
                                   void* normed, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (act == MOE_BF16) {
    TailArgs<uint16_t> a{};
    a.x = (const uint16_t*)x;
    a.residual = (const uint16_t*)residual;
    a.gamma = (const uint16_t*)gamma;
    a.eps = eps;
    a.T = T;
    a.D = D;
    a.residual_out = (uint16_t*)residual_out;
    a.normed = (uint16_t*)normed;
    return launch_tail<uint16_t, false>(a, s);
  }
  TailArgs<float> a{};
  a.x = (const float*)x;
  a.residual = (const float*)residual;
  a.gamma = (const float*)gamma;
  a.eps = eps;
  a.T = T;
  a.D = D;
  a.residual_out = (float*)residual_out;
  a.normed = (float*)normed;
  return launch_tail<float, false>(a, s);
}

hipError_t launch_combine_rmsnorm(const void* eo, const int32_t* topk_idx, const float* topk_w,
                                  const int32_t* pair_row, const void* shared,
                                  const void* residual, const void* gamma, float eps, int64_t T,
                                  int k, int D, int act, void* residual_out, void* normed,
                                  hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (act == MOE_BF16) {
    TailArgs<uint16_t> a{};
    a.eo = (const uint16_t*)eo;
    a.shared = (const uint16_t*)shared;
    a.residual = (const uint16_t*)residual;
    a.gamma = (const uint16_t*)gamma;
    a.residual_out = (uint16_t*)residual_out;
    a.normed = (uint16_t*)normed;
    a.topk_idx = topk_idx;
    a.topk_w = topk_w;
    a.pair_row = pair_row;
    a.eps = eps;
    a.T = T;
    a.k = k;
    a.D = D;
    return launch_tail<uint16_t, true>(a, s);
  }
  TailArgs<float> a{};
  a.eo = (const float*)eo;
  a.shared = (const float*)shared;
  a.residual = (const float*)residual;
  a.gamma = (const float*)gamma;
  a.residual_out = (float*)residual_out;
  a.normed = (float*)normed;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.pair_row = pair_row;
  a.eps = eps;
  a.T = T;
  a.k = k;
  a.D = D;
  return launch_tail<float, true>(a, s);
}

}  // namespace moe
