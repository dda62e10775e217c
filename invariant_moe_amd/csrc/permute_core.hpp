// The permutation proper (counting sort of the (token, slot) pairs by expert,
// see permute.hip) and the GEMM tile tables, as a device function of the
// workgroups of one launch.
#pragma once

#include "common.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace moe {

// Mask words (and their prefixes) are kept in LDS when the mask has at most
// this many words (E * ceil(T / 64)); otherwise prefixes go through wprefix.
constexpr int kPermLdsWords = 4096;

// LDSW: mask words that may be kept in LDS (0: never); OMAP: entries of the
// row-tile owner map (more row tiles fall back to a binary search).
template <int NT, int LDSW = kPermLdsWords, int OMAP = kTileOwnerMax>
struct PermuteLds {
  int soff[MOE_MAX_EXPERTS + 1];
  int mpre[MOE_MAX_EXPERTS + 1];
  int wsum[2 * (NT / 64)];
  int omap[OMAP];
  unsigned long long wmask[LDSW > 0 ? LDSW : 1];
  int wpre[LDSW > 0 ? LDSW : 1];
};

// counts, offsets, per-(expert, word) prefixes, the tile tables of the
// grouped GEMMs that follow, then the scatter.  Run by nwg workgroups of NT
// threads: each computes the counts and prefixes itself (all get the same
// values), then writes its share of the tables and of the scatter.
template <int NT, int LDSW, int OMAP, bool CO = false>
__device__ void permute_core(const int32_t* __restrict__ topk_idx, int64_t T, int k, int E,
                             const uint64_t* __restrict__ mask, int64_t W,
                             int32_t* __restrict__ wprefix, int32_t* __restrict__ counts,
                             int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
                             int32_t* __restrict__ pair_row, const TileJobs& jobs,
                             PermuteLds<NT, LDSW, OMAP>& L, int wg, int nwg) {
  const int BM = jobs.BM > 0 ? jobs.BM : 1;  // no grouped job: the m-tile counts go unused
  const int tid = threadIdx.x;
  const int Wi = (int)W;
  // LDS path for small masks of several words per expert (measured: 0.5 us
  // faster at 512 tokens x 64 experts, slower with a single word, and the
  // one-thread-per-expert walk is faster for masks past the LDS limit).
  const bool in_lds = LDSW > 0 && W >= 2 && (int64_t)E * W <= LDSW && E <= NT;

  // The scatter's first four pairs per thread do not depend on anything
  // below: their expert ids are loaded first.  Indices fit in 32 bits
  // (T * k < 2^31).
  const unsigned R = (unsigned)(T * k), uk = (unsigned)k;
  const unsigned pstart = (unsigned)wg * 4 * NT + tid, pstep = (unsigned)nwg * 4 * NT;
  int efirst[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const unsigned p = pstart + u * NT;
    efirst[u] = p < R ? topk_idx[p] : -1;
  }

  // Per-(expert, word) exclusive prefixes of the mask popcounts.
  if (in_lds) {
    // tpe consecutive threads share an expert, each taking a run of S words
    // (all its loads in flight), then scan their run totals with shuffles;
    // words and prefixes stay in LDS.
    int tpe = 1;
    while (tpe < 64 && 2 * tpe * E <= NT) tpe *= 2;
    const int e1 = tid / tpe, s1 = tid % tpe;
    const int S = (Wi + tpe - 1) / tpe;
    const int b0 = min(s1 * S, Wi), b1 = min(b0 + S, Wi);
    int run = 0;
    if (e1 < E) {
      const uint64_t* me = mask + (int64_t)e1 * W;
      for (int b = b0; b < b1; b += 8) {
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = b + u < b1 ? me[b + u] : 0ull;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (b + u < b1) L.wmask[e1 * Wi + b + u] = v[u];
          run += __popcll(v[u]);
        }
      }
    }
    int incl = run;  // every thread takes part in the shuffles (tpe is uniform)
    for (int m = 1; m < tpe; m <<= 1) {
      const int o = __shfl_up(incl, m, tpe);
      if (s1 >= m) incl += o;
    }
    if (e1 < E) {
      int pre = incl - run;
      for (int b = b0; b < b1; ++b) {
        L.wpre[e1 * Wi + b] = pre;
        pre += __popcll(L.wmask[e1 * Wi + b]);
      }
      if (s1 == tpe - 1) {
        if (wg == 0) Out<CO>::put(&counts[e1], incl);
        L.soff[e1] = incl;
        L.mpre[e1] = (incl + BM - 1) / BM;
      }
    }
  } else {
    // One thread per expert walks its words, eight loads in flight, writing
    // the prefixes to wprefix (the same values from every workgroup).
    for (int e = tid; e < E; e += NT) {
      int c = 0;
      const uint64_t* me = mask + (int64_t)e * W;
      int32_t* pe = wprefix + (int64_t)e * W;
      for (int b0 = 0; b0 < Wi; b0 += 8) {
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = b0 + u < Wi ? me[b0 + u] : 0ull;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (b0 + u < Wi) pe[b0 + u] = c;
          c += __popcll(v[u]);
        }
      }
      if (wg == 0) Out<CO>::put(&counts[e], c);
      L.soff[e] = c;
      L.mpre[e] = (c + BM - 1) / BM;
    }
  }
  __syncthreads();
  tile_scan2<NT>(L.soff, L.mpre, E, L.wsum);
  if (wg == 0)
    for (int e = tid; e <= E; e += NT) Out<CO>::put(&offsets[e], L.soff[e]);
  if (jobs.n > 0) {
    const bool map = build_tile_owner<NT, OMAP>(L.mpre, E, L.omap);
    build_tile_tables<NT, CO>(jobs, L.soff, L.mpre, map ? L.omap : nullptr, E, wg, nwg);
  }
  // The LDS words and prefixes, or the wprefix entries this workgroup wrote,
  // are visible after the barriers above.  Four pairs per thread per round.
  for (unsigned p0 = pstart; p0 < R; p0 += pstep) {
    int e[4];
    uint64_t word[4];
    int32_t pre_b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned p = p0 + u * NT;
      e[u] = p0 == pstart ? efirst[u] : (p < R ? topk_idx[p] : -1);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned p = p0 + u * NT;
      const bool valid = p < R && e[u] >= 0 && e[u] < E;
      const int64_t at = valid ? (int64_t)e[u] * W + ((p / uk) >> 6) : 0;
      if (in_lds) {
        word[u] = valid ? L.wmask[at] : 0ull;
        pre_b[u] = valid ? L.wpre[at] : 0;
      } else {
        word[u] = valid ? mask[at] : 0ull;
        pre_b[u] = valid ? wprefix[at] : 0;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned p = p0 + u * NT;
      if (p >= R) continue;
      if (e[u] < 0 || e[u] >= E) {  // outside the contract; keep memory safe
        Out<CO>::put(&pair_row[p], -1);
        continue;
      }
      const unsigned t = p / uk;
      const uint64_t below = word[u] & ((1ull << (t & 63)) - 1ull);
      const int32_t r = L.soff[e[u]] + pre_b[u] + __popcll(below);
      Out<CO>::put(&row_token[r], (int32_t)t);
      Out<CO>::put(&pair_row[p], r);
    }
  }
}

}  // namespace moe
