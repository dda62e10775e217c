// Tile tables of the grouped GEMMs, written on the device from the group
// offsets, so that a GEMM workgroup finds its tile with one 16-byte load.
//
// Tiles of a launch are numbered segment by segment, group-major, then by
// feature tile, then by row tile (row tiles of one feature tile are
// neighbours, so they share a weight panel in L2).  Tile l is given to the
// workgroup b whose XCD-major position is l: the hardware deals workgroups to
// the 8 XCDs round-robin, so b = (l mod chunk) * 8 + l / chunk with
// chunk = ceil(total / 8) puts tiles l of one chunk on one XCD.  Every other
// entry of the table gets a descriptor with zero rows.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Rows of group e from exclusive offsets; offsets outside [0, M] or
// decreasing give an empty group (same rule as the GEMM kernels).
__device__ __forceinline__ int tile_group_rows(const int* soff, int e, int64_t M) {
  const int a = soff[e], b = soff[e + 1];
  return (a < 0 || (int64_t)b > M || b < a) ? 0 : b - a;
}

// Exclusive scans of a[0..n) and b[0..n) in place, sharing the barriers; the
// totals go to a[n] and b[n].  Thread i takes the run of c = ceil(n / NT)
// consecutive entries from i*c (one entry when n <= NT); lanes scan the run
// sums within their wave, then the first wave scans the NT/64 wave sums.
// wsum: 2 * (NT/64) ints.
template <int NT>
__device__ void tile_scan2(int* a, int* b, int n, int* wsum) {
  static_assert(NT / 64 <= 64, "one wave scans the wave sums");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = (n + NT - 1) / NT;
  const int i0 = min(tid * c, n), i1 = min(i0 + c, n);
  int xa = 0, xb = 0;
  for (int i = i0; i < i1; ++i) {
    xa += a[i];
    xb += b[i];
  }
  int ia = xa, ib = xb;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int oa = __shfl_up(ia, m), ob = __shfl_up(ib, m);
    if (lane >= m) {
      ia += oa;
      ib += ob;
    }
  }
  if (lane == 63) {
    wsum[wave] = ia;
    wsum[NW + wave] = ib;
  }
  __syncthreads();
  if (wave == 0) {
    const int sa = lane < NW ? wsum[lane] : 0, sb = lane < NW ? wsum[NW + lane] : 0;
    int wa = sa, wb = sb;
#pragma unroll
    for (int m = 1; m < NW; m <<= 1) {
      const int oa = __shfl_up(wa, m), ob = __shfl_up(wb, m);
      if (lane >= m) {
        wa += oa;
        wb += ob;
      }
    }
    if (lane < NW) {
      wsum[lane] = wa - sa;
      wsum[NW + lane] = wb - sb;
    }
    if (lane == NW - 1) {
      a[n] = wa;
      b[n] = wb;
    }
  }
  __syncthreads();
  int pa = wsum[wave] + ia - xa, pb = wsum[NW + wave] + ib - xb;
  for (int i = i0; i < i1; ++i) {
    const int va = a[i], vb = b[i];
    a[i] = pa;
    b[i] = pb;
    pa += va;
    pb += vb;
  }
  __syncthreads();
}

// Owner map: omap[m] = group of the m-th row tile of the grouped segment
// (row tiles numbered group by group), when they fit.
constexpr int kTileOwnerMax = 8192;

// Builds omap from the exclusive m-tile prefix mpre[E+1] (call after the
// scan, by all threads; ends with a barrier).  Returns false (map unused)
// when there are more than OMAP row tiles.
template <int NT, int OMAP = kTileOwnerMax>
__device__ bool build_tile_owner(const int* mpre, int E, int* omap) {
  const bool fits = mpre[E] <= OMAP;
  if (fits)
    for (int e = threadIdx.x; e < E; e += NT)
      for (int m = mpre[e]; m < mpre[e + 1]; ++m) omap[m] = e;
  __syncthreads();
  return fits;
}

// Workgroup wg of nwg (NT threads each) writes entries wg*NT + tid, stepping
// by nwg*NT, of every job's table, in table order (coalesced stores).  soff: exclusive group offsets
// [E+1]; mpre: exclusive prefix [E+1] of ceil(rows_e / jobs.BM); omap: owner
// map or nullptr.  Tiles of a grouped segment are numbered group-major, then
// by feature tile, then by row tile, so tile li lies in the group whose row
// tile range holds floor(li / nt).  Grouped segments are tiled by jobs.BM
// (every job that has one shares it: the host planner guarantees it);
// ungrouped ones by their job's BM.  All counts fit in int32 (the planner
// rejects launches of 2^31 or more workgroups).
template <int NT, bool CO = false>
__device__ void build_tile_tables(const TileJobs& jobs, const int* soff, const int* mpre,
                                  const int* omap, int E, int wg, int nwg) {
  const int BM = jobs.BM;
#pragma unroll 1
  for (int j = 0; j < jobs.n; ++j) {  // uniform: job fields come from scalar loads
    const TileJob& J = jobs.job[j];
    const int grid = (int)J.grid, BN = J.BN, nseg = J.nseg, DBM = J.BM;
    int tot[2] = {0, 0}, nt[2] = {1, 1}, Ms[2] = {0, 0}, grouped[2] = {0, 0};
    for (int sg = 0; sg < nseg; ++sg) {
      nt[sg] = (J.N[sg] + BN - 1) / BN;
      grouped[sg] = J.grouped[sg];
      Ms[sg] = (int)J.M[sg];
      tot[sg] = grouped[sg] ? mpre[E] * nt[sg] : (Ms[sg] + DBM - 1) / DBM * nt[sg];
    }
    const int total = tot[0] + tot[1];
    const unsigned chunk = (unsigned)(total + 7) / 8u;
    for (int b = wg * NT + threadIdx.x; b < grid; b += nwg * NT) {
      int4 d = make_int4(0, 0, 0, 0);
      const unsigned q = (unsigned)b / 8u;
      const unsigned l = ((unsigned)b % 8u) * chunk + q;
      if (q < chunk && l < (unsigned)total) {
        const int sg = l < (unsigned)tot[0] ? 0 : 1;
        const int li = (int)l - (sg ? tot[0] : 0);
        const unsigned ntg = (unsigned)nt[sg];
        if (grouped[sg]) {
          const int key = (int)((unsigned)li / ntg);
          int e;
          if (omap) {
            e = omap[key];
          } else {  // last group whose row-tile prefix is <= key
            int lo = 0, hi = E - 1;
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (mpre[mid] <= key) lo = mid; else hi = mid - 1;
            }
            e = lo;
          }
          const int rows = tile_group_rows(soff, e, Ms[sg]);
          const unsigned mt = (unsigned)(mpre[e + 1] - mpre[e]);
          const unsigned i = (unsigned)li - (unsigned)mpre[e] * ntg;
          const unsigned ntile = i / mt, mtile = i - ntile * mt;
          d = make_int4(soff[e] + (int)mtile * BM, min(BM, rows - (int)mtile * BM),
                        (sg << 16) | e, (int)ntile * BN);
        } else {
          const unsigned mt = (unsigned)(Ms[sg] + DBM - 1) / (unsigned)DBM;
          const unsigned ntile = (unsigned)li / mt, mtile = (unsigned)li - ntile * mt;
          d = make_int4((int)mtile * DBM, min(DBM, Ms[sg] - (int)mtile * DBM), sg << 16,
                        (int)ntile * BN);
        }
      }
      Out<CO>::put4(&J.table[b], d);
    }
  }
}

}  // namespace moe
