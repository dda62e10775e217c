// The permutation proper (counting sort of the (token, slot) pairs by expert,
// see permute.hip) and the GEMM tile tables, as a device function of the
// workgroups of one launch.
#pragma once

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace moe {

template <int NT>
struct PermuteLds {
  int soff[MOE_MAX_EXPERTS + 1];
  int mpre[MOE_MAX_EXPERTS + 1];
  int wsum[2 * (NT / 64)];
  int omap[kTileOwnerMax];
};

// counts, offsets, per-(expert, block) prefixes, the tile tables of the
// grouped GEMMs that follow, then the scatter.  Run by nwg workgroups of NT
// threads: each computes the counts and prefixes itself (all get the same
// values), then writes its share of the tables and of the scatter.
template <int NT>
__device__ void permute_core(const int32_t* __restrict__ topk_idx, int64_t T, int k, int E,
                             const uint64_t* __restrict__ mask, int64_t W,
                             int32_t* __restrict__ wprefix, int32_t* __restrict__ counts,
                             int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
                             int32_t* __restrict__ pair_row, const TileJobs& jobs,
                             PermuteLds<NT>& L, int wg, int nwg) {
  const int BM = jobs.n > 0 ? jobs.BM : 1;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += NT) {
    int c = 0;
    const uint64_t* me = mask + (int64_t)e * W;
    int32_t* pe = wprefix + (int64_t)e * W;
    for (int b0 = 0; b0 < (int)W; b0 += 8) {  // eight mask words in flight
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = b0 + u < W ? me[b0 + u] : 0ull;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < W) pe[b0 + u] = c;  // the same value from every workgroup
        c += __popcll(v[u]);
      }
    }
    if (wg == 0) counts[e] = c;
    L.soff[e] = c;
    L.mpre[e] = (c + BM - 1) / BM;
  }
  __syncthreads();
  tile_scan2<NT>(L.soff, L.mpre, E, L.wsum);
  if (wg == 0)
    for (int e = tid; e <= E; e += NT) offsets[e] = L.soff[e];
  if (jobs.n > 0) {
    const bool map = build_tile_owner<NT>(L.mpre, E, L.omap);
    build_tile_tables<NT>(jobs, L.soff, L.mpre, map ? L.omap : nullptr, E, wg, nwg);
  }
  // wprefix written above by this workgroup is visible after the barriers.
  // Four pairs per thread per round, their loads issued together; indices
  // fit in 32 bits (T * k < 2^31).
  const unsigned R = (unsigned)(T * k), uk = (unsigned)k;
  for (unsigned p0 = (unsigned)wg * 4 * NT + tid; p0 < R; p0 += (unsigned)nwg * 4 * NT) {
    int e[4];
    uint64_t word[4];
    int32_t pre_b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned p = p0 + u * NT;
      e[u] = p < R ? topk_idx[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned p = p0 + u * NT;
      const bool valid = p < R && e[u] >= 0 && e[u] < E;
      const int64_t at = valid ? (int64_t)e[u] * W + ((p / uk) >> 6) : 0;
      word[u] = valid ? mask[at] : 0ull;
      pre_b[u] = valid ? wprefix[at] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned p = p0 + u * NT;
      if (p >= R) continue;
      if (e[u] < 0 || e[u] >= E) {  // outside the contract; keep memory safe
        pair_row[p] = -1;
        continue;
      }
      const unsigned t = p / uk;
      const uint64_t below = word[u] & ((1ull << (t & 63)) - 1ull);
      const int32_t r = L.soff[e[u]] + pre_b[u] + __popcll(below);
      row_token[r] = (int32_t)t;
      pair_row[p] = r;
    }
  }
}

}  // namespace moe
