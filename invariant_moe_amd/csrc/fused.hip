// Single-launch layer forward: routing, permutation, the gate/up and down
// expert GEMMs (routed and shared) and the combine in one persistent kernel.
//
// The DeepSeek-V4 infrastructure walkthrough ("6 基建与训练稳定性优化",
// section 6.1) fuses dispatch, expert compute and combine into one kernel
// whose experts are processed in waves, so that later steps start while
// earlier ones finish.  Here the layer's steps become tasks of one ordered
// queue that every workgroup of the launch draws from:
//   [router logits][shared gate/up][top-k][permute][routed gate/up]
//   [shared down][routed down][combine]
// A task waits only for whole phases earlier in the queue (per-phase done
// counters).  Tasks are handed out in queue order, so every task a workgroup
// waits for was taken earlier by a workgroup that is already running: no wait
// can depend on a workgroup that has not started, whatever the grid or the
// residency.  Each wait is bounded (spin limit); a wait that gives up sets a
// sticky error word in the queue header and the kernel still exits.
//
// Every task runs the device functions of the separate kernels (the same
// fixed chains: router order, top-k, counting sort, one MFMA chain per GEMM
// output, fixed-order combine), so the outputs are bit-identical to the
// unfused path; only the tile shapes may differ, and they do not change bits.
#include <hip/hip_runtime.h>

#include "combine_core.hpp"
#include "common.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"
#include "permute_core.hpp"
#include "router_core.hpp"
#include "routing.hpp"

namespace moe {

// Tile shapes of the fused configurations (256-thread workgroups).
template <int CFG>
struct FusedTiles;
// The decode shapes use wide feature tiles.  The kernel runs one workgroup
// per CU, and a timeline of its tasks (per-task timestamps, T = 1..64) showed
// each workgroup's weight stream bound by the latency of its K-stage loop, not
// by the loads in flight (more stages in flight changed nothing): a 16 x 64
// down tile streamed about 11 GB/s per workgroup.  Wider tiles move more bytes
// per loop step.  (Tasks of four one-wave 16 x 16 tiles, each wave with its
// own K-stage loop and LDS quarter as in the separate decode kernels, measured
// slower: 0.229 against 0.177 ms at T=1, 4.44 against 3.15 ms at T=64.)
template <>
struct FusedTiles<0> {  // <= 2 rows per expert (decode)
  static constexpr int BM = 16, GBN = 128, GWM = 1, GWN = 4, GP = 4;
  static constexpr int DBN = 256, DWM = 1, DWN = 4, DP = 4;
};
template <>
struct FusedTiles<1> {  // <= 16 rows per expert
  static constexpr int BM = 32, GBN = 128, GWM = 1, GWN = 4, GP = 4;
  static constexpr int DBN = 128, DWM = 1, DWN = 4, DP = 4;
};
// Above 16 rows per expert: 128-row tiles.  Per-task costs (drawing the task,
// waiting for its phase, the pipeline's fill) dominate small layers, so the
// fewer, larger tasks win even where most rows are padding: at 48 rows per
// expert (T=512, D=1024, E=64, k=6) 0.177 ms per step against 0.240 ms with
// 64 x 32 gate/up and 64 x 64 down tiles on four waves.
template <>
struct FusedTiles<2> {  // more than 16 rows per expert
  static constexpr int BM = 128, GBN = 64, GWM = 2, GWN = 2, GP = 2;
  static constexpr int DBN = 128, DWM = 2, DWN = 2, DP = 2;
};

constexpr int kFusedOwnerMap = 2048;
using FusedPermLds = PermuteLds<256, 0, kFusedOwnerMap>;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int CFG>
constexpr int fused_smem_bytes() {
  using TL = FusedTiles<CFG>;
  return cmax(cmax(cmax(gemm_smem_bytes<TL::BM, TL::GBN, true>(),
                        gemm_smem_bytes<TL::BM, TL::DBN, false>()),
                   cmax(router_logits_smem_bytes<uint16_t, 16>(), kRouterSmallSmemBytes)),
              cmax(cmax((int)sizeof(FusedPermLds), (int)sizeof(HashLds)),
                   (int)sizeof(CombineLds)));
}

// Spin limit of a wait: on the order of ten seconds of polling (each round is
// an acquire load plus a short sleep), far past any phase of a layer.  Once
// one wait has given up, every later wait returns at once.
constexpr unsigned kFusedSpinLimit = 1u << 23;

// Polls use relaxed agent-scope loads (coherent, no cache invalidation); the
// one acquire fence after the wait makes the producers' stores visible.  (An
// acquire load per poll would invalidate the XCD's L2 on every round, under
// the feet of every other workgroup of that XCD.)
__device__ __forceinline__ unsigned load_relaxed(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 waits until every task of phase p has finished.
__device__ __forceinline__ void wait_phase(const FusedArgs& a, int p) {
  const unsigned need = a.start[p + 1] - a.start[p];
  unsigned n = 0;
  while (load_relaxed(&a.hdr->done[p]) < need) {
    if (++n > kFusedSpinLimit) {
      __hip_atomic_fetch_or(&a.hdr->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (__hip_atomic_load(&a.hdr->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
    __builtin_amdgcn_s_sleep(8);
  }
}

// Dependencies of a task of phase ph (earlier phases only).  Thread 0 waits,
// then takes one agent-scope acquire (it invalidates the CU's and the XCD's
// caches that the workgroup's waves share) before the barrier releases them.
__device__ __forceinline__ void fused_wait(const FusedArgs& a, int ph) {
  if (ph == FP_ROUTE || ph == FP_SGU) return;  // inputs only
  if (threadIdx.x == 0) {
    switch (ph) {
      case FP_TOPK: wait_phase(a, FP_ROUTE); break;
      case FP_PERM: wait_phase(a, FP_ROUTE); wait_phase(a, FP_TOPK); break;
      case FP_GU: wait_phase(a, FP_PERM); break;
      case FP_SDN: wait_phase(a, FP_SGU); break;
      case FP_DN: wait_phase(a, FP_PERM); break;  // rows: per row tile, below
      default: wait_phase(a, FP_DN); wait_phase(a, FP_SDN); break;  // FP_COMB
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// A finished task.  Every result a later task reads was written with a
// coherent store (Out<true>); each thread waits until its stores have
// completed (vmcnt 0), then one thread counts the task for its phase.  No L2
// write-back fence is needed, which is what makes per-task signalling cheap
// on this GPU (an agent-scope release fence measured 9-35 us per task).
__device__ __forceinline__ void fused_done(const FusedArgs& a, int ph) {
  if (ph == FP_COMB) {  // nothing waits for the combine
    __syncthreads();
    return;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores are done
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(&a.hdr->done[ph], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A descriptor of a routed tile table (one segment), read with coherent
// loads (the table was written by the permutation task of this launch).
__device__ __forceinline__ bool fused_read_tile(const int4* tab, int64_t tile, const GemmSeg& s,
                                                int BM, TileInfo& ti) {
  const unsigned long long* q = reinterpret_cast<const unsigned long long*>(tab + tile);
  const unsigned long long lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long hi =
      __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int4 d = make_int4((int)(unsigned)lo, (int)(unsigned)(lo >> 32), (int)(unsigned)hi,
                           (int)(unsigned)(hi >> 32));
  const int seg = d.z >> 16, g = d.z & 0xffff;
  if (d.y <= 0 || d.y > BM || d.x < 0 || seg != 0) return false;
  if (g >= s.G || (int64_t)d.x + d.y > s.M || d.w < 0 || d.w >= s.N) return false;
  ti.seg = 0;
  ti.g = g;
  ti.row0 = d.x;
  ti.rows = d.y;
  ti.n0 = d.w;
  return true;
}

// Tile j of the shared expert (one group of T rows): row tiles inner.
__device__ __forceinline__ TileInfo fused_shared_tile(unsigned j, int mt, int BM, int BN,
                                                      int64_t T) {
  TileInfo ti;
  const int nt = (int)(j / (unsigned)mt), m = (int)(j % (unsigned)mt);
  ti.seg = 0;
  ti.g = 0;
  ti.row0 = (int64_t)m * BM;
  ti.rows = (int)min((int64_t)BM, T - ti.row0);
  ti.n0 = nt * BN;
  return ti;
}

// Task bodies.  All are inlined into the kernel, which runs one workgroup of
// four waves per CU: the union of the bodies' registers fits one wave per
// SIMD without spilling (two waves per SIMD do not).
template <int C>
__device__ __forceinline__ void fused_topk_task(const FusedArgs& a, unsigned j) {
  const int64_t t = (int64_t)j * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;  // whole wave
  int my_id;
  if (topk_token<C, true>(a.logits + t * a.E, a.bias, a.E, a.k, a.mode, a.idx + t * a.k,
                          a.tw + t * a.k, my_id))
    atomicOr(reinterpret_cast<unsigned long long*>(&a.mask[(int64_t)my_id * a.W + (t >> 6)]),
             1ull << (t & 63));
}

__device__ __forceinline__ void fused_topk(const FusedArgs& a, unsigned j) {
  switch (a.topk_c) {
    case 1: fused_topk_task<1>(a, j); break;
    case 2: fused_topk_task<2>(a, j); break;
    case 4: fused_topk_task<4>(a, j); break;
    case 8: fused_topk_task<8>(a, j); break;
    default: fused_topk_task<16>(a, j); break;
  }
}

__device__ __forceinline__ void fused_route(const FusedArgs& a, unsigned j, unsigned char* smem) {
  if (a.route_var == 3) {
    hash_route_block<256, true, true>(a.token_ids, a.T, a.E, a.k, a.idx, a.tw, a.mask, a.W, j,
                                *reinterpret_cast<HashLds*>(smem));
    return;
  }
  clear_words<true>(reinterpret_cast<unsigned long long*>(a.mask), a.n_zero, j,
              a.start[FP_ROUTE + 1] - a.start[FP_ROUTE]);
  const int64_t bx = j / (unsigned)a.route_gy;
  const int by = (int)(j % (unsigned)a.route_gy);
  if (a.route_var == 0)
    router_logits_small_tile<uint16_t, 1, 1, 16, true>(a.x, a.w_router, a.T, a.D, a.E, a.logits, bx,
                                                 by, smem);
  else if (a.route_var == 1)
    router_logits_small_tile<uint16_t, 4, 2, 4, true>(a.x, a.w_router, a.T, a.D, a.E, a.logits, bx,
                                                by, smem);
  else
    router_logits_tile<uint16_t, 16, 4, true>(a.x, a.w_router, a.T, a.D, a.E, a.logits, bx, by, smem);
}

__device__ __forceinline__ void fused_perm(const FusedArgs& a, unsigned j, unsigned char* smem) {
  const int64_t R = a.T * a.k;
  for (int64_t i = (int64_t)j * 256 + threadIdx.x; i < R; i += (int64_t)a.n_perm * 256)
    Out<true>::put(&a.row_done[i], 0u);
  permute_core<256, 0, kFusedOwnerMap, true>(a.idx, a.T, a.k, a.E, a.mask, a.W, a.wprefix, a.counts,
                                       a.offsets, a.row_token, a.pair_row, a.jobs,
                                       *reinterpret_cast<FusedPermLds*>(smem), (int)j, a.n_perm);
}

__device__ __forceinline__ void fused_comb(const FusedArgs& a, unsigned j, unsigned char* smem) {
  combine_tile<uint16_t>(a.o, a.idx, a.tw, a.pair_row, a.s, a.T, a.k, a.D, a.comb_tpt, a.y,
                         j / (unsigned)a.comb_gy, (int)(j % (unsigned)a.comb_gy), a.comb_gy,
                         *reinterpret_cast<CombineLds*>(smem));
}

// A GEMM tile task.  SEL: 0 shared gate/up, 1 routed gate/up, 2 shared down,
// 3 routed down.
template <int CFG, bool FP4, int SEL>
__device__ __forceinline__ void fused_gemm(const FusedArgs& a, unsigned j, unsigned char* smem) {
  using TL = FusedTiles<CFG>;
  constexpr bool gated = SEL < 2, routed = SEL & 1;
  constexpr int BN = gated ? TL::GBN : TL::DBN;
  const GemmSeg& s = SEL == 0 ? a.gu_s : SEL == 1 ? a.gu_r : SEL == 2 ? a.dn_s : a.dn_r;
  TileInfo ti;
  if (routed) {
    if (!fused_read_tile(gated ? a.tab_gu : a.tab_dn, j, s, TL::BM, ti)) return;
  } else {
    ti = fused_shared_tile(j, a.sh_mt, TL::BM, BN, a.T);
  }
  if constexpr (SEL == 3) {  // routed down: wait for the gate/up tiles of these rows
    if (threadIdx.x == 0) {
      unsigned n = 0;
      while (load_relaxed(&a.row_done[ti.row0]) < (unsigned)a.gu_ntiles) {
        if (++n > kFusedSpinLimit) {
          __hip_atomic_fetch_or(&a.hdr->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        if (__hip_atomic_load(&a.hdr->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
        __builtin_amdgcn_s_sleep(4);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
  }
  if constexpr (gated)
    gemm_tile_bf16<TL::BM, TL::GBN, TL::GWM, TL::GWN, TL::GP, true, FP4 && routed, true>(
        s, ti, a.glu, smem);
  else
    gemm_tile_bf16<TL::BM, TL::DBN, TL::DWM, TL::DWN, TL::DP, false, FP4 && routed, true>(
        s, ti, 0, smem);
  if constexpr (SEL == 1) {  // routed gate/up: count this feature tile for its rows
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's h stores are done
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(&a.row_done[ti.row0], 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int CFG, bool FP4, int PH>
__device__ __forceinline__ void fused_run(const FusedArgs& a, unsigned j, unsigned char* smem) {
  if constexpr (PH == FP_ROUTE) fused_route(a, j, smem);
  else if constexpr (PH == FP_TOPK) fused_topk(a, j);
  else if constexpr (PH == FP_PERM) fused_perm(a, j, smem);
  else if constexpr (PH == FP_COMB) fused_comb(a, j, smem);
  else if constexpr (PH == FP_SGU) fused_gemm<CFG, FP4, 0>(a, j, smem);
  else if constexpr (PH == FP_GU) fused_gemm<CFG, FP4, 1>(a, j, smem);
  else if constexpr (PH == FP_SDN) fused_gemm<CFG, FP4, 2>(a, j, smem);
  else fused_gemm<CFG, FP4, 3>(a, j, smem);
}

// Next task for the workgroup (one atomic by thread 0, broadcast through LDS;
// the caller's last barrier has freed the slot).
__device__ __forceinline__ unsigned fused_grab(const FusedArgs& a, unsigned* slot) {
  if (threadIdx.x == 0)
    *slot = __hip_atomic_fetch_add(&a.hdr->next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*slot);  // the same value in every lane
}

// The tasks a workgroup takes only increase, so it walks the phases in queue
// order: each phase is its own loop, over the tasks of that phase it draws.
template <int CFG, bool FP4>
__global__ __launch_bounds__(256, 1) void k_layer_fused(FusedArgs a) {
  __shared__ __align__(16) unsigned char smem[fused_smem_bytes<CFG>()];
  __shared__ unsigned s_task;
  unsigned task = fused_grab(a, &s_task);
  static_for<0, FP_COUNT>([&](auto pc) {
    constexpr int ph = decltype(pc)::value;
    while (task < a.start[ph + 1]) {  // uniform; task >= a.start[ph] here
      // The next task is drawn before this one runs (its fetch overlaps the
      // work).  Still deadlock-free: a drawn task that has not started
      // belongs to a workgroup running an earlier task.
      unsigned nxt = 0;
      if (threadIdx.x == 0)
        nxt = __hip_atomic_fetch_add(&a.hdr->next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      fused_wait(a, ph);
      fused_run<CFG, FP4, ph>(a, task - a.start[ph], smem);
      fused_done(a, ph);  // ends with a barrier: s_task and LDS are free again
      if (threadIdx.x == 0) s_task = nxt;
      __syncthreads();
      task = __builtin_amdgcn_readfirstlane(s_task);
    }
  });
  // Leave the queue; the last workgroup to leave resets it for the next call
  // (every other one has made its last access to the header: its final task
  // fetch returned before it counted itself out).  The kernel's end makes the
  // reset visible to the next launch.
  if (threadIdx.x == 0) {
    const unsigned n =
        __hip_atomic_fetch_add(&a.hdr->exited, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n == gridDim.x - 1) {
      for (int p = 0; p < FP_COUNT; ++p)
        __hip_atomic_store(&a.hdr->done[p], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.hdr->next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.hdr->exited, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int fused_cfg(int64_t hint, bool) {
  if (hint <= 2) return 0;
  if (hint <= 16) return 1;
  return 2;
}

void fused_tiles(int cfg, int* BM, int* BN_gu, int* BN_dn) {
  switch (cfg) {
    case 0: *BM = FusedTiles<0>::BM; *BN_gu = FusedTiles<0>::GBN; *BN_dn = FusedTiles<0>::DBN; break;
    case 1: *BM = FusedTiles<1>::BM; *BN_gu = FusedTiles<1>::GBN; *BN_dn = FusedTiles<1>::DBN; break;
    default: *BM = FusedTiles<2>::BM; *BN_gu = FusedTiles<2>::GBN; *BN_dn = FusedTiles<2>::DBN; break;
  }
}

template <int CFG, bool FP4>
static int64_t resident_blocks() {
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_layer_fused<CFG, FP4>, 256, 0) !=
      hipSuccess)
    return 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return (int64_t)per_cu * cus;
}

int64_t fused_grid(int cfg, bool fp4, int64_t ntasks) {
  int64_t r = 0;
  switch (cfg * 2 + (fp4 ? 1 : 0)) {
    case 0: r = resident_blocks<0, false>(); break;
    case 1: r = resident_blocks<0, true>(); break;
    case 2: r = resident_blocks<1, false>(); break;
    case 3: r = resident_blocks<1, true>(); break;
    case 4: r = resident_blocks<2, false>(); break;
    default: r = resident_blocks<2, true>(); break;
  }
  return r < ntasks ? r : ntasks;
}

hipError_t launch_layer_fused(const FusedArgs& a, int cfg, bool fp4, int64_t grid,
                              hipStream_t s) {
  const dim3 g((unsigned)grid), b(256);
  switch (cfg * 2 + (fp4 ? 1 : 0)) {
    case 0: hipLaunchKernelGGL((k_layer_fused<0, false>), g, b, 0, s, a); break;
    case 1: hipLaunchKernelGGL((k_layer_fused<0, true>), g, b, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_layer_fused<1, false>), g, b, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_layer_fused<1, true>), g, b, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_layer_fused<2, false>), g, b, 0, s, a); break;
    default: hipLaunchKernelGGL((k_layer_fused<2, true>), g, b, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace moe
