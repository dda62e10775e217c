// Dispatch: the stable counting sort of the (token, slot) pairs by expert
// (dispatch -> compute -> combine, "6 基建与训练稳定性优化" section 6.1; no
// capacity and no dropping, since dropping makes a token's output depend on
// the rest of the batch — forum article feedbbs.com/linuxdo/72580, section on
// why MoE outputs are not deterministic).
//
// Representation: for each expert e and each 64-token block b, a 64-bit word
// mask[e][b] whose bit t%64 says token t selected e.  Integer popcounts then
// give every pair its row directly:
//   row(t, e) = offsets[e] + (tokens of earlier blocks that chose e)
//               + popcount(mask[e][t/64] & bits below t%64)
// so rows of an expert are in ascending token order, as the counting sort.
#include "common.hpp"
#include "kernels.hpp"
#include "permute_core.hpp"

namespace moe {

// mask words from topk_idx: one workgroup per 64-token block.
__global__ __launch_bounds__(256) void k_mask_from_idx(const int32_t* __restrict__ topk_idx,
                                                       int64_t T, int k, int E,
                                                       uint64_t* __restrict__ mask, int64_t W) {
  __shared__ unsigned long long smask[MOE_MAX_EXPERTS];
  const int64_t tb = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) smask[e] = 0ull;
  __syncthreads();
  for (int p = threadIdx.x; p < 64 * k; p += 256) {
    const int tt = p / k;
    const int64_t t = tb * 64 + tt;
    if (t < T) {
      const int e = topk_idx[t * k + (p % k)];
      if (e >= 0 && e < E) atomicOr(&smask[e], 1ull << tt);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) mask[(int64_t)e * W + tb] = smask[e];
}

__global__ __launch_bounds__(1024) void k_permute(const int32_t* __restrict__ topk_idx,
                                                  int64_t T, int k, int E,
                                                  const uint64_t* __restrict__ mask, int64_t W,
                                                  int32_t* __restrict__ wprefix,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ row_token,
                                                  int32_t* __restrict__ pair_row,
                                                  TileJobs jobs) {
  __shared__ PermuteLds<1024> L;
  permute_core<1024>(topk_idx, T, k, E, mask, W, wprefix, counts, offsets, row_token, pair_row,
                     jobs, L, blockIdx.x, gridDim.x);
}


// x_perm[r] = x[row_token[r]], 16-byte chunks.
__global__ __launch_bounds__(256) void k_gather_rows(const uint8_t* __restrict__ x,
                                                     const int32_t* __restrict__ row_token,
                                                     int64_t T, int64_t R, int64_t row_bytes,
                                                     uint8_t* __restrict__ out) {
  const int64_t chunks = row_bytes / 16;
  const int64_t total = R * chunks;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / chunks, c = i % chunks;
    int64_t src = row_token[r];
    src = src < 0 ? 0 : (src >= T ? T - 1 : src);  // repeated ids per token leave rows unset
    reinterpret_cast<uint4*>(out + r * row_bytes)[c] =
        reinterpret_cast<const uint4*>(x + src * row_bytes)[c];
  }
}

hipError_t launch_mask_from_idx(const int32_t* topk_idx, int64_t T, int k, int E, uint64_t* mask,
                                hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t W = (T + 63) / 64;
  hipLaunchKernelGGL(k_mask_from_idx, dim3((unsigned)W), dim3(256), 0, s, topk_idx, T, k, E,
                     mask, W);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* topk_idx, int64_t T, int k, int E, const uint64_t* mask,
                          int32_t* wprefix, int32_t* counts, int32_t* offsets, int32_t* row_token,
                          int32_t* pair_row, const TileJobs* jobs, hipStream_t s) {
  const int64_t W = (T + 63) / 64;
  TileJobs none{};
  // Workgroups: enough that each scatters at most 4 pairs and writes at most
  // two table entries per thread (each repeats the cheap counting and scans).
  int64_t entries = 0;
  if (jobs)
    for (int j = 0; j < jobs->n; ++j) entries += jobs->job[j].grid;
  int64_t nwg = (T * k + 4095) / 4096;
  if ((entries + 2047) / 2048 > nwg) nwg = (entries + 2047) / 2048;
  nwg = nwg < 1 ? 1 : (nwg > 32 ? 32 : nwg);
  hipLaunchKernelGGL(k_permute, dim3((unsigned)nwg), dim3(1024), 0, s, topk_idx, T, k, E, mask, W,
                     wprefix, counts, offsets, row_token, pair_row, jobs ? *jobs : none);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* row_token, int64_t T, int64_t R,
                              int64_t row_bytes, void* out, hipStream_t s) {
  if (R == 0) return hipSuccess;
  int64_t total = R * (row_bytes / 16);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t*)x,
                     row_token, T, R, row_bytes, (uint8_t*)out);
  return hipGetLastError();
}

}  // namespace moe
