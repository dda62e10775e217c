// Internal launch interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Sets the thread-local message that moe_last_error() returns (printf
// format) and returns status.
int set_error(int status, const char* fmt, ...);

// One segment of a grouped GEMM: G groups of rows that share the reduction
// input layout; group g uses weights [g] of W0/W1 (and scales S0/S1).
struct GemmSeg {
  const void* A;           // reduction input rows [*, K] (bf16 bits or fp32)
  const int32_t* a_index;  // output row r reads A[a_index[r]] (nullptr: A[r])
  const int32_t* offsets;  // [G+1] device row offsets (nullptr: one group of M rows)
  int64_t M;               // total rows of the segment (= offsets[G] when offsets != nullptr)
  int G;
  int K, N;
  const void* W0;          // [G, N, K] gate (gated) or down; MXFP4: codes [G, N, K/2]
  const void* W1;          // [G, N, K] up (gated only)
  const uint8_t* S0;       // MXFP4 scales [G, N, K/32]
  const uint8_t* S1;
  int wfmt;                // 0 bf16/fp32 (as act), 1 MXFP4
  void* out;               // [rows, N]
  const uint8_t* AS;       // FP4 x FP8 launches: A is E4M3 codes [*, K], AS E8M0 [*, K/32]
};

// Tile descriptor, one per workgroup of a GEMM launch (int4):
//   x = first output row, y = valid rows (0: the workgroup has no tile),
//   z = (segment << 16) | group, w = first output feature.
struct GemmArgs {
  GemmSeg seg[2];
  int nseg;
  const int4* tiles;  // [grid] descriptors, indexed by blockIdx.x
  int glu;            // gated activation of a gated GEMM (GluMode)
};

// Gated activation of the gate/up GEMM's epilogue.
enum GluMode { GLU_SWIGLU = 0, GLU_CLAMP = 1, GLU_SITU = 2 };

// Shape of a segment as the host planner sees it.
struct SegShape {
  bool grouped;  // rows grouped by device offsets (E groups); else one group of M rows
  int64_t M;
  int G, K, N;
  int wfmt;
};

// One launch of a planned grouped GEMM.
struct PlanLaunch {
  int seg_mask;  // which segments of the GEMM this launch covers
  int cfg;       // kernel configuration (tile shape)
  int BM, BN;
  int64_t grid;  // workgroups = tile-table entries
};

struct GemmPlan {
  PlanLaunch l[2];
  int n;
  bool valid;  // false: a launch would exceed the grid limit
  bool gated;
  int act;
  SegShape seg[2];
  int nseg;
};

// Tile-table job: the device writes the descriptors of one launch.
struct TileJob {
  int4* table;
  int64_t grid;
  int BM, BN;
  int nseg;
  int grouped[2];  // 1: E groups from the device offsets; 0: one group of M rows
  int64_t M[2];
  int N[2];
};

constexpr int MOE_MAX_TILE_JOBS = 4;
struct TileJobs {
  TileJob job[MOE_MAX_TILE_JOBS];
  int n;
  int BM;  // row tile of the grouped segments, shared by every job that has
           // one; a job of ungrouped segments only tiles by its own BM (0: no
           // grouped job)
};

// zero / n_zero (optional): 64-bit words cleared for a later kernel of the call.
hipError_t launch_router_logits(const void* x, int act, const void* w, int64_t T, int D, int E,
                                float* logits, uint64_t* zero, int64_t n_zero, hipStream_t s);
// mask (optional): bit t%64 of word [e][t/64] is ORed in for each selected
// (token t, expert e); the words must be zero at launch.
hipError_t launch_topk(const float* logits, const float* bias, int64_t T, int E, int k, int mode,
                       int32_t* idx, float* w, uint64_t* mask, hipStream_t s);
hipError_t launch_hash_route(const int32_t* token_ids, int64_t T, int E, int k, int32_t* idx,
                             float* w, uint64_t* mask, hipStream_t s);
hipError_t launch_routing_scores(const float* in, int64_t n, int mode, float* out, hipStream_t s);
hipError_t launch_mask_from_idx(const int32_t* topk_idx, int64_t T, int k, int E, uint64_t* mask,
                                hipStream_t s);
// jobs (optional): tile tables written from the new offsets in the same launch.
hipError_t launch_permute(const int32_t* topk_idx, int64_t T, int k, int E, const uint64_t* mask,
                          int32_t* wprefix, int32_t* counts, int32_t* offsets, int32_t* row_token,
                          int32_t* pair_row, const TileJobs* jobs, hipStream_t s);
hipError_t launch_gather_rows(const void* x, const int32_t* row_token, int64_t T, int64_t R,
                              int64_t row_bytes, void* out, hipStream_t s);
// Tile tables from caller-supplied offsets [E+1] (one small launch).
hipError_t launch_tile_tables(const int32_t* offsets, int E, const TileJobs& jobs, hipStream_t s);

// MXFP8 activation quantisation (E4M3 + E8M0 per 32 along K) of R bf16 rows
// of K (K % 32 == 0); row r reads x[row_index[r]] (row_index NULL: x[r]).
hipError_t launch_mx_e4m3_quantize(const void* x, const int32_t* row_index, int64_t R, int K,
                                   uint8_t* codes, uint8_t* scales, hipStream_t s);
// Plan of an FP4 x FP8 grouped GEMM (one segment of MXFP4 weights, K % 128 == 0);
// 128-row tiles above 96 rows per group, else 64-row tiles (128 or 64 features).
GemmPlan plan_w4a8_gemm(const SegShape& seg, bool gated, int64_t rows_per_group_hint);

// Host planning of a grouped GEMM (tile shape, launches, table sizes).
GemmPlan plan_grouped_gemm(const SegShape* segs, int nseg, bool gated, int act,
                           int64_t rows_per_group_hint);
int64_t plan_table_entries(const GemmPlan& p);
// Appends the table jobs of p (tables carved from `tables`, plan_table_entries(p) entries).
// Returns false when p's row tile differs from the jobs already appended.
bool plan_tile_jobs(const GemmPlan& p, int4* tables, TileJobs& jobs);
// Launches the planned GEMM; a.tiles is ignored (each launch uses its own table).
// ev_start / ev_stop (optional) are recorded at the start of the first and the
// end of the last kernel of the plan.
hipError_t launch_grouped_gemm(const GemmPlan& p, const GemmArgs& a, int4* tables, hipStream_t s,
                               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// ---------------------------------------------------------------------------
// Single-launch layer forward (fused.hip).  One kernel runs every step of the
// layer as tasks of one ordered queue; a task waits only for tasks of earlier
// phases (counted per phase), so no wait can block on a workgroup that has not
// started.
// ---------------------------------------------------------------------------
enum FusedPhase {
  FP_ROUTE = 0,  // router logits (+ clearing the mask words) or hash routing
  FP_SGU,        // shared expert gate/up tiles (need only x)
  FP_TOPK,       // top-k + weights, 4 tokens per task
  FP_PERM,       // permutation + routed tile tables
  FP_GU,         // routed gate/up tiles (table)
  FP_SDN,        // shared expert down tiles
  FP_DN,         // routed down tiles (table)
  FP_COMB,       // combine tiles
  FP_COUNT
};

// Queue state at the start of the workspace: zero before the first call, and
// left zero by every call that completes (the last workgroup to leave resets
// it).  err is sticky: a wait that gave up (spin limit) sets it, and the
// outputs of that call are undefined.
struct FusedHdr {
  unsigned next;    // next task to hand out
  unsigned exited;  // workgroups that have left the queue
  unsigned err;
  unsigned pad;
  unsigned done[FP_COUNT];  // finished tasks per phase
};
constexpr size_t kFusedHdrBytes = 256;

struct FusedArgs {
  FusedHdr* hdr;
  unsigned start[FP_COUNT + 1];  // task ranges of the phases, in queue order
  // routing
  const uint16_t* x;
  const int32_t* token_ids;
  const uint16_t* w_router;
  const float* bias;
  int64_t T;
  int D, E, k, mode;
  int route_var;  // 0: small-T logit tiles 1x1x16, 1: 4x2x4, 2: LDS tiles 16x4, 3: hash
  int route_gy;   // expert tiles of the logit tiling
  int topk_c;     // keys per lane of the top-k (1, 2, 4, 8, 16)
  float* logits;
  int32_t* idx;
  float* tw;
  uint64_t* mask;
  int64_t W;       // mask words per expert
  int64_t n_zero;  // mask words the logit tasks clear
  // permutation
  int32_t* wprefix;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* pair_row;
  TileJobs jobs;  // routed gate/up and down tile tables
  int n_perm;
  // expert GEMMs
  GemmSeg gu_r, gu_s, dn_r, dn_s;
  const int4* tab_gu;
  const int4* tab_dn;
  // Finished gate/up tiles per routed row tile, indexed by the tile's first
  // row (row tiles of different experts never share a first row): a down
  // tile starts once all gu_ntiles feature tiles of its rows are done.
  // Cleared by the permutation tasks.  [R]
  unsigned* row_done;
  int gu_ntiles;
  int sh_mt;  // row tiles of the shared expert
  int glu;
  // combine
  const uint16_t* o;
  const uint16_t* s;  // shared expert rows or nullptr
  int comb_tpt, comb_gy;
  uint16_t* y;
};

// Tile configuration of the fused kernel by rows per expert (bit-identical
// choices): 0 <= 2, 1 <= 16, 2 above (either weight format).
int fused_cfg(int64_t rows_per_group_hint, bool fp4);
// Row tile and feature tiles of a fused configuration.
void fused_tiles(int cfg, int* BM, int* BN_gu, int* BN_dn);
// Workgroups that one launch may use: resident capacity of the kernel (at
// most ntasks).  Returns 0 on a HIP error.
int64_t fused_grid(int cfg, bool fp4, int64_t ntasks);
hipError_t launch_layer_fused(const FusedArgs& a, int cfg, bool fp4, int64_t grid,
                              hipStream_t s);

hipError_t launch_combine(const void* expert_out, const int32_t* topk_idx, const float* topk_w,
                          const int32_t* pair_row, const void* shared_out, int64_t T, int k,
                          int D, int act, void* y, hipStream_t s);
// Residual add + RMSNorm (one workgroup per token); the second form computes
// its input rows as launch_combine does, without writing them.
hipError_t launch_residual_rmsnorm(const void* x, const void* residual, const void* gamma,
                                   float eps, int64_t T, int D, int act, void* residual_out,
                                   void* normed, hipStream_t s);
hipError_t launch_combine_rmsnorm(const void* expert_out, const int32_t* topk_idx,
                                  const float* topk_w, const int32_t* pair_row,
                                  const void* shared_out, const void* residual, const void* gamma,
                                  float eps, int64_t T, int k, int D, int act, void* residual_out,
                                  void* normed, hipStream_t s);

}  // namespace moe
