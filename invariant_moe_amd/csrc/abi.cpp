// C ABI: argument validation, workspace carving and kernel launches on the
// caller's stream.  Declarations and the contract of every entry point are in
// include/moe.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/moe.h"
#include "kernels.hpp"

#ifndef MOE_BUILD_ID
#define MOE_BUILD_ID "unversioned"
#endif

namespace {

thread_local char g_err[512] = "";
thread_local void* const* g_stage_events = nullptr;
thread_local int g_n_stage_events = 0;

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

// The gated activation that a call's flags select (MOE_FLAG_GLU_*).
int glu_from_flags(uint32_t flags, int* glu) {
  constexpr uint32_t known = MOE_FLAG_GLU_CLAMP | MOE_FLAG_GLU_SITU;
  if (flags & ~known) return fail(MOE_ERR_UNSUPPORTED, "flags 0x%x: unknown bits", flags);
  if (flags == known)
    return fail(MOE_ERR_UNSUPPORTED, "flags 0x%x: at most one gated activation", flags);
  *glu = (flags & MOE_FLAG_GLU_CLAMP) ? moe::GLU_CLAMP
         : (flags & MOE_FLAG_GLU_SITU) ? moe::GLU_SITU
                                       : moe::GLU_SWIGLU;
  return MOE_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t act_size(moe_dtype a) { return a == MOE_F32 ? 4 : 2; }

// Workspace carving.  Each region starts on a 256-byte boundary.
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

// The two grouped GEMMs of the expert FFN (gate/up, then down) as the host
// planner sees them: routed experts grouped by the device offsets, plus the
// shared expert as one group of T rows.  (Measured on MI355X: the shared
// expert in launches of its own on a second stream, concurrent with routing
// and permutation, was slower at prefill, 5.87 against 5.83 ms per layer at
// T=4096, and at decode, 156 against 153 us at T=1: it slowed the small
// kernels it overlapped and added a cross-queue wait.)
struct FfnPlans {
  moe::GemmPlan up, dn;
};

FfnPlans ffn_plans(int64_t R, int64_t T, int D, int E, int I, int Is, moe_dtype act,
                   int routed_wfmt, int shared_wfmt) {
  const int64_t hint = R / E;
  moe::SegShape su[2] = {{true, R, E, D, I, routed_wfmt}, {false, T, 1, D, Is, shared_wfmt}};
  moe::SegShape sd[2] = {{true, R, E, I, D, routed_wfmt}, {false, T, 1, Is, D, shared_wfmt}};
  const int nseg = Is > 0 ? 2 : 1;
  FfnPlans p;
  p.up = moe::plan_grouped_gemm(su, nseg, true, act, hint);
  p.dn = moe::plan_grouped_gemm(sd, nseg, false, act, hint);
  return p;
}

// Tile-table entries reserved for the two GEMMs: the largest over the weight
// formats of the routed and shared experts (the formats change the launches
// and tile shapes), so the workspace size does not depend on them.
int64_t ffn_table_entries(int64_t R, int64_t T, int D, int E, int I, int Is, moe_dtype act) {
  int64_t n = 0;
  for (int rf = 0; rf < 2; ++rf)
    for (int sf = 0; sf < 2; ++sf) {
      const FfnPlans p = ffn_plans(R, T, D, E, I, Is, act, rf, sf);
      const int64_t m = moe::plan_table_entries(p.up) + moe::plan_table_entries(p.dn);
      n = m > n ? m : n;
    }
  return n;
}

int64_t layer_table_entries(int64_t T, int D, int E, int k, int I, int Is, moe_dtype act) {
  return ffn_table_entries(T * k, T, D, E, I, Is, act);
}

// Plans of the layer's FFN when the routed experts run FP4 x FP8: the routed
// GEMMs on the W4A8 kernel, the bf16 shared expert on the bf16 kernel with
// the tiles the planner picks for its T rows (its tables are dense, so they
// need not share the routed row tile); one permutation launch writes all four
// tile tables.
struct W4a8Plans {
  moe::GemmPlan up_r, up_s, dn_r, dn_s;
  bool shared;
};

W4a8Plans w4a8_plans(int64_t R, int64_t T, int D, int E, int I, int Is) {
  W4a8Plans p{};
  const int64_t hint = R / E;
  p.up_r = moe::plan_w4a8_gemm({true, R, E, D, I, 2}, true, hint);
  p.dn_r = moe::plan_w4a8_gemm({true, R, E, I, D, 2}, false, hint);
  p.shared = Is > 0;
  if (p.shared) {
    const moe::SegShape su{false, T, 1, D, Is, 0}, sd{false, T, 1, Is, D, 0};
    p.up_s = moe::plan_grouped_gemm(&su, 1, true, MOE_BF16, T);
    p.dn_s = moe::plan_grouped_gemm(&sd, 1, false, MOE_BF16, T);
  }
  return p;
}

int64_t w4a8_layer_entries(const W4a8Plans& p) {
  int64_t n = moe::plan_table_entries(p.up_r) + moe::plan_table_entries(p.dn_r);
  if (p.shared) n += moe::plan_table_entries(p.up_s) + moe::plan_table_entries(p.dn_s);
  return n;
}

struct LayerLayout {
  size_t logits, idx, w, mask, wprefix, counts, offsets, row_token, pair_row, h, hs, o, s, tiles,
      xq, xsc, hq, hsc, total;
  int64_t tile_entries;
};

// w4a8: also the MXFP8 copies of x and h (FP4 x FP8 routed experts).
LayerLayout layer_layout(int64_t T, int D, int E, int k, int I, int Is, moe_dtype act,
                         bool w4a8 = false) {
  const int64_t R = T * k, W = (T + 63) / 64;
  const size_t es = act_size(act);
  Carver c;
  LayerLayout L;
  L.logits = c.take((size_t)T * E * 4);
  L.idx = c.take((size_t)R * 4);
  L.w = c.take((size_t)R * 4);
  L.mask = c.take((size_t)E * W * 8);
  L.wprefix = c.take((size_t)E * W * 4);
  L.counts = c.take((size_t)E * 4);
  L.offsets = c.take((size_t)(E + 1) * 4);
  L.row_token = c.take((size_t)R * 4);
  L.pair_row = c.take((size_t)R * 4);
  L.h = c.take((size_t)R * I * es);
  L.hs = c.take((size_t)T * (Is > 0 ? Is : 0) * es);
  L.o = c.take((size_t)R * D * es);
  L.s = c.take((size_t)T * (Is > 0 ? D : 0) * es);
  L.tile_entries = layer_table_entries(T, D, E, k, I, Is, act);
  L.xq = L.xsc = L.hq = L.hsc = 0;
  if (w4a8) {
    const int64_t n = w4a8_layer_entries(w4a8_plans(R, T, D, E, I, Is));
    if (n > L.tile_entries) L.tile_entries = n;
  }
  L.tiles = c.take((size_t)L.tile_entries * sizeof(int4));
  if (w4a8) {
    L.xq = c.take((size_t)T * D);
    L.xsc = c.take((size_t)T * (D / 32));
    L.hq = c.take((size_t)R * I);
    L.hsc = c.take((size_t)R * (I / 32));
  }
  L.total = c.off;
  return L;
}

// The FP4 x FP8 layout is reserved for MXFP4 routed weights whenever the
// shapes allow it, so a caller sizing for MXFP4 weights may set the flag.
bool w4a8_shapes(int D, int I, moe_dtype act) {
  return act == MOE_BF16 && D % 128 == 0 && I % 128 == 0;
}

// One FP4 x FP8 GEMM segment: A = E4M3 codes, AS = their scales.
moe::GemmSeg w4a8_seg(const uint8_t* A, const uint8_t* AS, const int32_t* a_index,
                      const int32_t* offsets, int64_t M, int G, int K, int N,
                      const moe_expert_weights* w, bool gated, void* out) {
  moe::GemmSeg g{};
  g.A = A;
  g.AS = AS;
  g.a_index = a_index;
  g.offsets = offsets;
  g.M = M;
  g.G = G;
  g.K = K;
  g.N = N;
  g.W0 = gated ? w->gate : w->down;
  g.W1 = gated ? w->up : nullptr;
  g.S0 = gated ? w->gate_scale : w->down_scale;
  g.S1 = gated ? w->up_scale : nullptr;
  g.wfmt = 2;
  g.out = out;
  return g;
}

int check_dims(int64_t T, int D, int E, int k) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T=%lld must be >= 0", (long long)T);
  if (E < 1 || E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_SHAPE, "E=%d must be in [1, %d]", E, MOE_MAX_EXPERTS);
  if (k < 1 || k > E || k > MOE_MAX_TOPK)
    return fail(MOE_ERR_SHAPE, "k=%d must be in [1, min(E=%d, %d)]", k, E, MOE_MAX_TOPK);
  if (D < 32 || D % 32) return fail(MOE_ERR_SHAPE, "D=%d must be a positive multiple of 32", D);
  if (T * (int64_t)k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "T*k must be < 2^31");
  return MOE_OK;
}

int check_weights(const moe_expert_weights* w, moe_dtype act, const char* which) {
  if (!w) return fail(MOE_ERR_NULL, "%s weights are NULL", which);
  if (!w->gate || !w->up || !w->down) return fail(MOE_ERR_NULL, "%s weight pointer is NULL", which);
  if (!aligned(w->gate, 16) || !aligned(w->up, 16) || !aligned(w->down, 16))
    return fail(MOE_ERR_ALIGN, "%s weights must be 16-byte aligned", which);
  if (w->dtype == MOE_MXFP4) {
    if (act != MOE_BF16) return fail(MOE_ERR_DTYPE, "MXFP4 %s weights need bf16 activations", which);
    if (!w->gate_scale || !w->up_scale || !w->down_scale)
      return fail(MOE_ERR_NULL, "MXFP4 %s weights need scale pointers", which);
  } else {
    if (w->dtype != act)
      return fail(MOE_ERR_DTYPE, "%s weight dtype %d does not match activation dtype %d", which,
                  (int)w->dtype, (int)act);
    if (w->gate_scale || w->up_scale || w->down_scale)
      return fail(MOE_ERR_DTYPE, "%s scale pointers must be NULL unless dtype is MXFP4", which);
  }
  return MOE_OK;
}

int check_act(moe_dtype act) {
  if (act != MOE_F32 && act != MOE_BF16)
    return fail(MOE_ERR_DTYPE, "activation dtype must be MOE_F32 or MOE_BF16");
  return MOE_OK;
}

hipEvent_t kernel_event(int i) {
  return (g_stage_events && i < g_n_stage_events) ? static_cast<hipEvent_t>(g_stage_events[i])
                                                  : nullptr;
}

void record_stage(int i, hipStream_t s) {
  if (g_stage_events && i < g_n_stage_events && g_stage_events[i])
    (void)hipEventRecord(static_cast<hipEvent_t>(g_stage_events[i]), s);
}

moe::GemmSeg make_seg(const void* A, const int32_t* a_index, const int32_t* offsets, int64_t M,
                      int G, int K, int N, const moe_expert_weights* w, bool gated, void* out) {
  moe::GemmSeg s{};
  s.A = A;
  s.a_index = a_index;
  s.offsets = offsets;
  s.M = M;
  s.G = G;
  s.K = K;
  s.N = N;
  s.W0 = gated ? w->gate : w->down;
  s.W1 = gated ? w->up : nullptr;
  s.S0 = gated ? w->gate_scale : w->down_scale;
  s.S1 = gated ? w->up_scale : nullptr;
  s.wfmt = w->dtype == MOE_MXFP4 ? 1 : 0;
  s.out = out;
  return s;
}

}  // namespace

namespace moe {
int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}
}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_build_id(void) { return MOE_BUILD_ID; }

const char* moe_last_error(void) { return g_err; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "unknown status";
  }
}

int moe_set_stage_events(void* const* events, int n_events) {
  if (n_events < 0) return fail(MOE_ERR_SHAPE, "n_events must be >= 0");
  g_stage_events = n_events > 0 ? events : nullptr;
  g_n_stage_events = events ? n_events : 0;
  return ok();
}

size_t moe_router_workspace_bytes(int64_t T, int E, moe_route mode) {
  if (mode == MOE_ROUTE_HASH || T <= 0 || E <= 0) return 0;
  return align_up((size_t)T * (size_t)E * 4);
}

int moe_router_topk(const void* x, moe_dtype act, const void* w_router, const float* bias,
                    const int32_t* token_ids, int64_t T, int D, int E, int k, moe_route mode,
                    int32_t* topk_idx, float* topk_w, void* workspace, size_t workspace_bytes,
                    void* stream) {
  int rc;
  if ((rc = check_dims(T, D, E, k))) return rc;
  if (mode != MOE_ROUTE_SOFTMAX && mode != MOE_ROUTE_SIGMOID && mode != MOE_ROUTE_HASH)
    return fail(MOE_ERR_SHAPE, "unknown routing mode %d", (int)mode);
  if (!topk_idx || !topk_w) return fail(MOE_ERR_NULL, "topk_idx / topk_w are NULL");
  if (!aligned(topk_idx, 4) || !aligned(topk_w, 4)) return fail(MOE_ERR_ALIGN, "outputs misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == MOE_ROUTE_HASH) {
    if (!token_ids) return fail(MOE_ERR_NULL, "hash routing needs token_ids");
    if (T == 0) return ok();
    return hip_status(moe::launch_hash_route(token_ids, T, E, k, topk_idx, topk_w, nullptr, s),
                      "hash routing");
  }
  if ((rc = check_act(act))) return rc;
  if (!x || !w_router) return fail(MOE_ERR_NULL, "x / w_router are NULL");
  if (!aligned(x, 16) || !aligned(w_router, 16)) return fail(MOE_ERR_ALIGN, "x / w_router must be 16-byte aligned");
  if (bias && !aligned(bias, 4)) return fail(MOE_ERR_ALIGN, "bias misaligned");
  const size_t need = moe_router_workspace_bytes(T, E, mode);
  if (need && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "router workspace needs %zu bytes", need);
  if (workspace && !aligned(workspace, 16)) return fail(MOE_ERR_ALIGN, "workspace misaligned");
  if (T == 0) return ok();
  float* logits = static_cast<float*>(workspace);
  hipError_t e = moe::launch_router_logits(x, act, w_router, T, D, E, logits, nullptr, 0, s);
  if (e == hipSuccess)
    e = moe::launch_topk(logits, bias, T, E, k, mode, topk_idx, topk_w, nullptr, s);
  return hip_status(e, "router");
}

int moe_routing_scores(const float* logits, int64_t n, moe_route mode, float* out, void* stream) {
  if (n < 0) return fail(MOE_ERR_SHAPE, "n must be >= 0");
  if (mode != MOE_ROUTE_SOFTMAX && mode != MOE_ROUTE_SIGMOID)
    return fail(MOE_ERR_SHAPE, "routing scores exist for softmax and sigmoid modes only");
  if (n > 0 && (!logits || !out)) return fail(MOE_ERR_NULL, "NULL argument");
  if (n > 0 && (!aligned(logits, 4) || !aligned(out, 4))) return fail(MOE_ERR_ALIGN, "misaligned");
  return hip_status(moe::launch_routing_scores(logits, n, mode, out, static_cast<hipStream_t>(stream)),
                    "routing scores");
}

size_t moe_permute_workspace_bytes(int64_t T, int E) {
  if (T < 0 || E <= 0) return 0;
  const int64_t W = (T + 63) / 64;
  Carver c;
  c.take((size_t)E * W * 8);
  c.take((size_t)E * W * 4);
  return c.off;
}

int moe_permute(const int32_t* topk_idx, int64_t T, int k, int E, int32_t* expert_counts,
                int32_t* expert_offsets, int32_t* row_token, int32_t* pair_row, const void* x,
                moe_dtype act, int D, void* x_perm, void* workspace, size_t workspace_bytes,
                void* stream) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T must be >= 0");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_SHAPE, "E=%d out of range", E);
  if (k < 1 || k > E || k > MOE_MAX_TOPK) return fail(MOE_ERR_SHAPE, "k=%d out of range", k);
  if (T * (int64_t)k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "T*k must be < 2^31");
  if (!expert_counts || !expert_offsets || !row_token || !pair_row)
    return fail(MOE_ERR_NULL, "permutation outputs are NULL");
  if (T > 0 && !topk_idx) return fail(MOE_ERR_NULL, "topk_idx is NULL");
  if (x) {
    int rc;
    if ((rc = check_act(act))) return rc;
    if (D < 32 || D % 32) return fail(MOE_ERR_SHAPE, "D=%d must be a positive multiple of 32", D);
    if (!x_perm) return fail(MOE_ERR_NULL, "x_perm is NULL while x is given");
    if (!aligned(x, 16) || !aligned(x_perm, 16)) return fail(MOE_ERR_ALIGN, "x / x_perm misaligned");
  }
  const size_t need = moe_permute_workspace_bytes(T, E);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "permute workspace needs %zu bytes", need);
  if (!aligned(workspace, 16)) return fail(MOE_ERR_ALIGN, "workspace misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t W = (T + 63) / 64;
  uint64_t* mask = static_cast<uint64_t*>(workspace);
  int32_t* wprefix = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align_up((size_t)E * W * 8));
  hipError_t e = moe::launch_mask_from_idx(topk_idx, T, k, E, mask, s);
  if (e == hipSuccess)
    e = moe::launch_permute(topk_idx, T, k, E, mask, wprefix, expert_counts, expert_offsets,
                            row_token, pair_row, nullptr, s);
  if (e == hipSuccess && x)
    e = moe::launch_gather_rows(x, row_token, T, T * k, (int64_t)D * act_size(act), x_perm, s);
  return hip_status(e, "permute");
}

// h rows, then the tile tables of the two GEMMs.
size_t moe_grouped_swiglu_workspace_bytes(int64_t R, int E, int D, int I, moe_dtype act) {
  if (R <= 0 || E <= 0 || D <= 0 || I <= 0) return 0;
  const moe_dtype a = act == MOE_F32 ? MOE_F32 : MOE_BF16;
  Carver c;
  c.take((size_t)R * I * act_size(a));
  c.take((size_t)ffn_table_entries(R, 0, D, E, I, 0, a) * sizeof(int4));
  return c.off;
}

int moe_grouped_swiglu(const void* x_rows, const int32_t* row_index, const int32_t* expert_offsets,
                       int64_t R, int E, int D, int I, const moe_expert_weights* w, moe_dtype act,
                       uint32_t flags, void* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc;
  if ((rc = check_act(act))) return rc;
  int glu;
  if ((rc = glu_from_flags(flags, &glu))) return rc;
  if (R < 0 || R >= ((int64_t)1 << 31)) return fail(MOE_ERR_SHAPE, "R out of range");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_SHAPE, "E=%d out of range", E);
  if (D < 32 || D % 32 || I < 32 || I % 32)
    return fail(MOE_ERR_SHAPE, "D=%d and I=%d must be positive multiples of 32", D, I);
  if ((rc = check_weights(w, act, "expert"))) return rc;
  if (!expert_offsets || !out || (R > 0 && !x_rows)) return fail(MOE_ERR_NULL, "NULL argument");
  if ((x_rows && !aligned(x_rows, 16)) || !aligned(out, 16)) return fail(MOE_ERR_ALIGN, "x_rows / out misaligned");
  const size_t need = moe_grouped_swiglu_workspace_bytes(R, E, D, I, act);
  if (need && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "grouped_swiglu workspace needs %zu bytes", need);
  if (workspace && !aligned(workspace, 16)) return fail(MOE_ERR_ALIGN, "workspace misaligned");
  if (R == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FfnPlans p = ffn_plans(R, 0, D, E, I, 0, act, w->dtype == MOE_MXFP4 ? 1 : 0, 0);
  if (!p.up.valid || !p.dn.valid) return fail(MOE_ERR_SHAPE, "problem too large for one launch");
  if (moe::plan_table_entries(p.up) + moe::plan_table_entries(p.dn) >
      ffn_table_entries(R, 0, D, E, I, 0, act))
    return fail(MOE_ERR_WORKSPACE, "tile tables exceed their workspace region");
  Carver c;
  c.take((size_t)R * I * act_size(act));
  int4* tiles_up = reinterpret_cast<int4*>(static_cast<char*>(workspace) + c.off);
  int4* tiles_dn = tiles_up + moe::plan_table_entries(p.up);
  moe::TileJobs jobs{};
  if (!moe::plan_tile_jobs(p.up, tiles_up, jobs) || !moe::plan_tile_jobs(p.dn, tiles_dn, jobs))
    return fail(MOE_ERR_UNSUPPORTED, "gate/up and down GEMM plans use different row tiles");
  hipError_t e = moe::launch_tile_tables(expert_offsets, E, jobs, s);
  moe::GemmArgs up{};
  up.nseg = 1;
  up.seg[0] = make_seg(x_rows, row_index, expert_offsets, R, E, D, I, w, true, workspace);
  up.glu = glu;
  if (e == hipSuccess) e = moe::launch_grouped_gemm(p.up, up, tiles_up, s);
  if (e == hipSuccess) {
    moe::GemmArgs dn{};
    dn.nseg = 1;
    dn.seg[0] = make_seg(workspace, nullptr, expert_offsets, R, E, I, D, w, false, out);
    e = moe::launch_grouped_gemm(p.dn, dn, tiles_dn, s);
  }
  return hip_status(e, "grouped_swiglu");
}

int moe_mx_e4m3_quantize(const void* x, const int32_t* row_index, int64_t R, int K,
                         uint8_t* codes, uint8_t* scales, void* stream) {
  if (R < 0 || R >= ((int64_t)1 << 31)) return fail(MOE_ERR_SHAPE, "R out of range");
  if (K < 32 || K % 32) return fail(MOE_ERR_SHAPE, "K=%d must be a positive multiple of 32", K);
  if (R > 0 && (!x || !codes || !scales)) return fail(MOE_ERR_NULL, "NULL argument");
  if (R > 0 && (!aligned(x, 16) || !aligned(codes, 8)))
    return fail(MOE_ERR_ALIGN, "x must be 16-byte and codes 8-byte aligned");
  return hip_status(moe::launch_mx_e4m3_quantize(x, row_index, R, K, codes, scales,
                                                 static_cast<hipStream_t>(stream)),
                    "mx_e4m3_quantize");
}

// x codes + scales, h (bf16), h codes + scales, then the two GEMMs' tile tables.
static int64_t w4a8_table_entries(int64_t R, int E, int D, int I) {
  moe::SegShape up{true, R, E, D, I, 2}, dn{true, R, E, I, D, 2};
  int64_t n = 0;
  for (int64_t hint : {(int64_t)0, (int64_t)64, (int64_t)1 << 30})  // every tile shape
    n = std::max(n, moe::plan_table_entries(moe::plan_w4a8_gemm(up, true, hint)) +
                        moe::plan_table_entries(moe::plan_w4a8_gemm(dn, false, hint)));
  return n;
}

size_t moe_grouped_swiglu_w4a8_workspace_bytes(int64_t R, int E, int D, int I) {
  if (R <= 0 || E <= 0 || D <= 0 || I <= 0) return 0;
  Carver c;
  c.take((size_t)R * D);
  c.take((size_t)R * (D / 32));
  c.take((size_t)R * I * 2);
  c.take((size_t)R * I);
  c.take((size_t)R * (I / 32));
  c.take((size_t)w4a8_table_entries(R, E, D, I) * sizeof(int4));
  return c.off;
}

int moe_grouped_swiglu_w4a8(const void* x_rows, const int32_t* row_index,
                            const int32_t* expert_offsets, int64_t R, int E, int D, int I,
                            const moe_expert_weights* w, uint32_t flags, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  int rc, glu;
  if ((rc = glu_from_flags(flags, &glu))) return rc;
  if (R < 0 || R >= ((int64_t)1 << 31)) return fail(MOE_ERR_SHAPE, "R out of range");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_SHAPE, "E=%d out of range", E);
  if (D < 128 || D % 128 || I < 128 || I % 128)
    return fail(MOE_ERR_SHAPE, "D=%d and I=%d must be positive multiples of 128", D, I);
  if (!w) return fail(MOE_ERR_NULL, "weights are NULL");
  if (w->dtype != MOE_MXFP4) return fail(MOE_ERR_DTYPE, "FP4 x FP8 needs MXFP4 weights");
  if ((rc = check_weights(w, MOE_BF16, "expert"))) return rc;
  if (!expert_offsets || !out || (R > 0 && !x_rows)) return fail(MOE_ERR_NULL, "NULL argument");
  if ((x_rows && !aligned(x_rows, 16)) || !aligned(out, 16))
    return fail(MOE_ERR_ALIGN, "x_rows / out misaligned");
  const size_t need = moe_grouped_swiglu_w4a8_workspace_bytes(R, E, D, I);
  if (need && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "grouped_swiglu_w4a8 workspace needs %zu bytes", need);
  if (workspace && !aligned(workspace, 256)) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (R == 0) return ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  moe::SegShape su{true, R, E, D, I, 2}, sd{true, R, E, I, D, 2};
  const moe::GemmPlan pu = moe::plan_w4a8_gemm(su, true, R / E),
                      pd = moe::plan_w4a8_gemm(sd, false, R / E);
  if (!pu.valid || !pd.valid) return fail(MOE_ERR_SHAPE, "problem too large for one launch");
  char* ws = static_cast<char*>(workspace);
  Carver c;
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws + c.take((size_t)R * D));
  uint8_t* xs = reinterpret_cast<uint8_t*>(ws + c.take((size_t)R * (D / 32)));
  void* h = ws + c.take((size_t)R * I * 2);
  uint8_t* hq = reinterpret_cast<uint8_t*>(ws + c.take((size_t)R * I));
  uint8_t* hs = reinterpret_cast<uint8_t*>(ws + c.take((size_t)R * (I / 32)));
  int4* tiles_up = reinterpret_cast<int4*>(ws + c.off);
  int4* tiles_dn = tiles_up + moe::plan_table_entries(pu);
  moe::TileJobs jobs{};
  if (!moe::plan_tile_jobs(pu, tiles_up, jobs) || !moe::plan_tile_jobs(pd, tiles_dn, jobs))
    return fail(MOE_ERR_UNSUPPORTED, "gate/up and down GEMM plans use different row tiles");
  hipError_t e = moe::launch_tile_tables(expert_offsets, E, jobs, s);
  if (e == hipSuccess) e = moe::launch_mx_e4m3_quantize(x_rows, row_index, R, D, xq, xs, s);
  moe::GemmArgs up{};
  up.nseg = 1;
  up.glu = glu;
  up.seg[0] = w4a8_seg(xq, xs, nullptr, expert_offsets, R, E, D, I, w, true, h);
  if (e == hipSuccess) e = moe::launch_grouped_gemm(pu, up, tiles_up, s);
  if (e == hipSuccess) e = moe::launch_mx_e4m3_quantize(h, nullptr, R, I, hq, hs, s);
  moe::GemmArgs dn{};
  dn.nseg = 1;
  dn.seg[0] = w4a8_seg(hq, hs, nullptr, expert_offsets, R, E, I, D, w, false, out);
  if (e == hipSuccess) e = moe::launch_grouped_gemm(pd, dn, tiles_dn, s);
  return hip_status(e, "grouped_swiglu_w4a8");
}

int moe_combine(const void* expert_out, const int32_t* topk_idx, const float* topk_w,
                const int32_t* pair_row, const void* shared_out, int64_t T, int k, int D,
                moe_dtype act, void* y, void* stream) {
  int rc;
  if ((rc = check_act(act))) return rc;
  if (T < 0) return fail(MOE_ERR_SHAPE, "T must be >= 0");
  if (k < 1 || k > MOE_MAX_TOPK) return fail(MOE_ERR_SHAPE, "k=%d out of range", k);
  if (D < 32 || D % 32) return fail(MOE_ERR_SHAPE, "D=%d must be a positive multiple of 32", D);
  if (T > 0 && (!expert_out || !topk_idx || !topk_w || !pair_row || !y))
    return fail(MOE_ERR_NULL, "NULL argument");
  if (T > 0 && (!aligned(expert_out, 16) || !aligned(y, 16) ||
                (shared_out && !aligned(shared_out, 16))))
    return fail(MOE_ERR_ALIGN, "expert_out / shared_out / y must be 16-byte aligned");
  return hip_status(moe::launch_combine(expert_out, topk_idx, topk_w, pair_row, shared_out, T, k,
                                        D, act, y, static_cast<hipStream_t>(stream)),
                    "combine");
}

static int check_norm(int64_t T, int D, float eps, const void* x, const void* residual,
                      const void* gamma, const void* residual_out, const void* normed) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T must be >= 0");
  if (D < 32 || D % 32) return fail(MOE_ERR_SHAPE, "D=%d must be a positive multiple of 32", D);
  if (!(eps >= 0.0f) || !std::isfinite(eps))
    return fail(MOE_ERR_UNSUPPORTED, "eps must be finite and >= 0");
  if (T > 0 && (!x || !residual || !gamma || !residual_out || !normed))
    return fail(MOE_ERR_NULL, "NULL argument");
  if (T > 0 && (!aligned(x, 16) || !aligned(residual, 16) || !aligned(gamma, 16) ||
                !aligned(residual_out, 16) || !aligned(normed, 16)))
    return fail(MOE_ERR_ALIGN, "rows and gamma must be 16-byte aligned");
  return MOE_OK;
}

int moe_residual_rmsnorm(const void* x, const void* residual, const void* gamma, float eps,
                         int64_t T, int D, moe_dtype act, void* residual_out, void* normed,
                         void* stream) {
  int rc;
  if ((rc = check_act(act))) return rc;
  if ((rc = check_norm(T, D, eps, x, residual, gamma, residual_out, normed))) return rc;
  return hip_status(moe::launch_residual_rmsnorm(x, residual, gamma, eps, T, D, act, residual_out,
                                                 normed, static_cast<hipStream_t>(stream)),
                    "residual_rmsnorm");
}

int moe_combine_rmsnorm(const void* expert_out, const int32_t* topk_idx, const float* topk_w,
                        const int32_t* pair_row, const void* shared_out, const void* residual,
                        const void* gamma, float eps, int64_t T, int k, int D, moe_dtype act,
                        void* residual_out, void* normed, void* stream) {
  int rc;
  if ((rc = check_act(act))) return rc;
  if (k < 1 || k > MOE_MAX_TOPK) return fail(MOE_ERR_SHAPE, "k=%d out of range", k);
  if ((rc = check_norm(T, D, eps, expert_out, residual, gamma, residual_out, normed))) return rc;
  if (T > 0 && (!topk_idx || !topk_w || !pair_row)) return fail(MOE_ERR_NULL, "NULL argument");
  if (T > 0 && shared_out && !aligned(shared_out, 16))
    return fail(MOE_ERR_ALIGN, "shared_out must be 16-byte aligned");
  return hip_status(moe::launch_combine_rmsnorm(expert_out, topk_idx, topk_w, pair_row, shared_out,
                                                residual, gamma, eps, T, k, D, act, residual_out,
                                                normed, static_cast<hipStream_t>(stream)),
                    "combine_rmsnorm");
}

size_t moe_layer_workspace_bytes(int64_t T, int D, int E, int k, int I, int I_shared,
                                 moe_dtype act, moe_dtype w) {
  if (T < 0 || D <= 0 || E <= 0 || k <= 0 || I <= 0) return 0;
  return layer_layout(T, D, E, k, I, I_shared, act, w == MOE_MXFP4 && w4a8_shapes(D, I, act))
      .total;
}

int moe_layer_forward(const void* x, const int32_t* token_ids, const void* w_router,
                      const float* bias, const moe_expert_weights* routed,
                      const moe_expert_weights* shared, int64_t T, int D, int E, int k, int I,
                      int I_shared, moe_route mode, moe_dtype act, uint32_t flags, void* y,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_act(act))) return rc;
  if ((rc = check_dims(T, D, E, k))) return rc;
  int glu;
  const bool w4a8 = (flags & MOE_FLAG_W4A8) != 0;
  if ((rc = glu_from_flags(flags & ~MOE_FLAG_W4A8, &glu))) return rc;
  if (I < 32 || I % 32) return fail(MOE_ERR_SHAPE, "I=%d must be a positive multiple of 32", I);
  if (mode != MOE_ROUTE_SOFTMAX && mode != MOE_ROUTE_SIGMOID && mode != MOE_ROUTE_HASH)
    return fail(MOE_ERR_SHAPE, "unknown routing mode %d", (int)mode);
  if ((rc = check_weights(routed, act, "routed"))) return rc;
  const int Is = shared ? I_shared : 0;
  if (shared) {
    if ((rc = check_weights(shared, act, "shared"))) return rc;
    if (Is < 32 || Is % 32)
      return fail(MOE_ERR_SHAPE, "I_shared=%d must be a positive multiple of 32", I_shared);
  }
  if (T > 0 && (!x || !y)) return fail(MOE_ERR_NULL, "x / y are NULL");
  if (T > 0 && (!aligned(x, 16) || !aligned(y, 16))) return fail(MOE_ERR_ALIGN, "x / y must be 16-byte aligned");
  if (mode == MOE_ROUTE_HASH) {
    if (!token_ids) return fail(MOE_ERR_NULL, "hash routing needs token_ids");
  } else {
    if (!w_router) return fail(MOE_ERR_NULL, "w_router is NULL");
    if (!aligned(w_router, 16)) return fail(MOE_ERR_ALIGN, "w_router must be 16-byte aligned");
    if (bias && !aligned(bias, 4)) return fail(MOE_ERR_ALIGN, "bias misaligned");
  }
  if (w4a8) {
    if (!routed || routed->dtype != MOE_MXFP4)
      return fail(MOE_ERR_DTYPE, "MOE_FLAG_W4A8 needs MXFP4 routed weights");
    if (!w4a8_shapes(D, I, act))
      return fail(MOE_ERR_SHAPE, "MOE_FLAG_W4A8 needs bf16 activations and D, I multiples of 128");
    if (shared && shared->dtype != MOE_BF16)
      return fail(MOE_ERR_UNSUPPORTED, "MOE_FLAG_W4A8 runs a bf16 shared expert only");
  }
  const LayerLayout L = layer_layout(T, D, E, k, I, Is, act, w4a8);
  if (!workspace || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "layer workspace needs %zu bytes", L.total);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (T == 0) return ok();

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
  float* tw = reinterpret_cast<float*>(ws + L.w);
  uint64_t* mask = reinterpret_cast<uint64_t*>(ws + L.mask);
  int32_t* wprefix = reinterpret_cast<int32_t*>(ws + L.wprefix);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* row_token = reinterpret_cast<int32_t*>(ws + L.row_token);
  int32_t* pair_row = reinterpret_cast<int32_t*>(ws + L.pair_row);
  void* h = ws + L.h;
  void* hs = ws + L.hs;
  void* o = ws + L.o;
  void* sh = ws + L.s;
  const int64_t R = T * k;

  // Tile plans; the permutation launch writes their tables.
  int4* tiles = reinterpret_cast<int4*>(ws + L.tiles);
  moe::TileJobs jobs{};
  FfnPlans p{};
  W4a8Plans q{};
  int4 *tiles_up = tiles, *tiles_dn = nullptr, *tiles_up_s = nullptr, *tiles_dn_s = nullptr;
  if (!w4a8) {
    p = ffn_plans(R, T, D, E, I, Is, act, routed->dtype == MOE_MXFP4 ? 1 : 0,
                  shared && shared->dtype == MOE_MXFP4 ? 1 : 0);
    if (!p.up.valid || !p.dn.valid) return fail(MOE_ERR_SHAPE, "problem too large for one launch");
    if (moe::plan_table_entries(p.up) + moe::plan_table_entries(p.dn) > L.tile_entries)
      return fail(MOE_ERR_WORKSPACE, "tile tables exceed their workspace region");
    tiles_dn = tiles_up + moe::plan_table_entries(p.up);
    if (!moe::plan_tile_jobs(p.up, tiles_up, jobs) || !moe::plan_tile_jobs(p.dn, tiles_dn, jobs))
      return fail(MOE_ERR_UNSUPPORTED, "gate/up and down GEMM plans use different row tiles");
  } else {
    q = w4a8_plans(R, T, D, E, I, Is);
    if (!q.up_r.valid || !q.dn_r.valid || (shared && (!q.up_s.valid || !q.dn_s.valid)))
      return fail(MOE_ERR_SHAPE, "problem too large for one launch");
    if (w4a8_layer_entries(q) > L.tile_entries)
      return fail(MOE_ERR_WORKSPACE, "tile tables exceed their workspace region");
    tiles_up_s = tiles_up + moe::plan_table_entries(q.up_r);
    tiles_dn = tiles_up_s + (shared ? moe::plan_table_entries(q.up_s) : 0);
    tiles_dn_s = tiles_dn + moe::plan_table_entries(q.dn_r);
    if (!moe::plan_tile_jobs(q.up_r, tiles_up, jobs) ||
        (shared && !moe::plan_tile_jobs(q.up_s, tiles_up_s, jobs)) ||
        !moe::plan_tile_jobs(q.dn_r, tiles_dn, jobs) ||
        (shared && !moe::plan_tile_jobs(q.dn_s, tiles_dn_s, jobs)))
      return fail(MOE_ERR_UNSUPPORTED, "the FFN plans use different row tiles");
  }

  record_stage(0, s);
  hipError_t e;
  if (mode == MOE_ROUTE_HASH) {
    e = moe::launch_hash_route(token_ids, T, E, k, idx, tw, mask, s);
  } else {
    e = moe::launch_router_logits(x, act, w_router, T, D, E, logits, mask, E * ((T + 63) / 64), s);
    if (e == hipSuccess) e = moe::launch_topk(logits, bias, T, E, k, mode, idx, tw, mask, s);
  }
  if (e != hipSuccess) return hip_status(e, "routing");
  record_stage(1, s);
  e = moe::launch_permute(idx, T, k, E, mask, wprefix, counts, offsets, row_token, pair_row, &jobs,
                          s);
  if (e != hipSuccess) return hip_status(e, "permute");
  record_stage(2, s);

  if (!w4a8) {
    moe::GemmArgs up{};
    up.seg[0] = make_seg(x, row_token, offsets, R, E, D, I, routed, true, h);
    up.nseg = 1;
    up.glu = glu;
    if (shared) {
      up.seg[1] = make_seg(x, nullptr, nullptr, T, 1, D, Is, shared, true, hs);
      up.nseg = 2;
    }
    e = moe::launch_grouped_gemm(p.up, up, tiles_up, s, kernel_event(MOE_STAGE_EVENTS),
                                 kernel_event(MOE_STAGE_EVENTS + 1));
  } else {
    // x quantised once per token; the routed GEMM gathers codes and scales
    // through row_token
    uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.xq);
    uint8_t* xsc = reinterpret_cast<uint8_t*>(ws + L.xsc);
    e = moe::launch_mx_e4m3_quantize(x, nullptr, T, D, xq, xsc, s);
    moe::GemmArgs up{};
    up.seg[0] = w4a8_seg(xq, xsc, row_token, offsets, R, E, D, I, routed, true, h);
    up.nseg = 1;
    up.glu = glu;
    if (e == hipSuccess)
      e = moe::launch_grouped_gemm(q.up_r, up, tiles_up, s, kernel_event(MOE_STAGE_EVENTS),
                                   shared ? nullptr : kernel_event(MOE_STAGE_EVENTS + 1));
    if (e == hipSuccess && shared) {
      moe::GemmArgs us{};
      us.seg[0] = make_seg(x, nullptr, nullptr, T, 1, D, Is, shared, true, hs);
      us.nseg = 1;
      us.glu = glu;
      e = moe::launch_grouped_gemm(q.up_s, us, tiles_up_s, s, nullptr,
                                   kernel_event(MOE_STAGE_EVENTS + 1));
    }
  }
  if (e != hipSuccess) return hip_status(e, "gate/up GEMM");
  record_stage(3, s);

  if (!w4a8) {
    moe::GemmArgs dn{};
    dn.seg[0] = make_seg(h, nullptr, offsets, R, E, I, D, routed, false, o);
    dn.nseg = 1;
    if (shared) {
      dn.seg[1] = make_seg(hs, nullptr, nullptr, T, 1, Is, D, shared, false, sh);
      dn.nseg = 2;
    }
    e = moe::launch_grouped_gemm(p.dn, dn, tiles_dn, s, kernel_event(MOE_STAGE_EVENTS + 2),
                                 kernel_event(MOE_STAGE_EVENTS + 3));
  } else {
    uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.hq);
    uint8_t* hsc = reinterpret_cast<uint8_t*>(ws + L.hsc);
    e = moe::launch_mx_e4m3_quantize(h, nullptr, R, I, hq, hsc, s);
    moe::GemmArgs dn{};
    dn.seg[0] = w4a8_seg(hq, hsc, nullptr, offsets, R, E, I, D, routed, false, o);
    dn.nseg = 1;
    if (e == hipSuccess)
      e = moe::launch_grouped_gemm(q.dn_r, dn, tiles_dn, s, kernel_event(MOE_STAGE_EVENTS + 2),
                                   shared ? nullptr : kernel_event(MOE_STAGE_EVENTS + 3));
    if (e == hipSuccess && shared) {
      moe::GemmArgs ds{};
      ds.seg[0] = make_seg(hs, nullptr, nullptr, T, 1, Is, D, shared, false, sh);
      ds.nseg = 1;
      e = moe::launch_grouped_gemm(q.dn_s, ds, tiles_dn_s, s, nullptr,
                                   kernel_event(MOE_STAGE_EVENTS + 3));
    }
  }
  if (e != hipSuccess) return hip_status(e, "down GEMM");
  record_stage(4, s);

  e = moe::launch_combine(o, idx, tw, pair_row, shared ? sh : nullptr, T, k, D, act, y, s);
  if (e != hipSuccess) return hip_status(e, "combine");
  record_stage(5, s);
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Single-launch layer forward
// ---------------------------------------------------------------------------
static int64_t round8(int64_t v) { return (v + 7) / 8 * 8; }

// Table entries of a routed GEMM with row tile BM and feature tile BN (the
// bound the unfused planner uses: every non-empty group may add one partial
// row tile).
static int64_t routed_tile_bound(int64_t R, int E, int N, int BM, int BN) {
  const int64_t nonempty = R < E ? R : E;
  return round8(((R + BM - 1) / BM + nonempty) * ((N + BN - 1) / BN));
}

struct FusedLayout {
  LayerLayout L;   // offsets relative to `layer`
  size_t layer, tab_gu, tab_dn, row_done, total;
  int64_t n_gu, n_dn;
};

// Queue header, the layer's workspace, then the two routed tile tables (sized
// for either routed weight format).
static FusedLayout fused_layout(int64_t T, int D, int E, int k, int I, int Is) {
  FusedLayout f{};
  const int64_t R = T * k;
  Carver c;
  c.take(moe::kFusedHdrBytes);
  f.L = layer_layout(T, D, E, k, I, Is, MOE_BF16);
  f.layer = c.take(f.L.total);
  for (int fp4 = 0; fp4 < 2; ++fp4) {
    int BM, BNg, BNd;
    moe::fused_tiles(moe::fused_cfg(R / E, fp4 != 0), &BM, &BNg, &BNd);
    f.n_gu = std::max(f.n_gu, routed_tile_bound(R, E, I, BM, BNg));
    f.n_dn = std::max(f.n_dn, routed_tile_bound(R, E, D, BM, BNd));
  }
  f.tab_gu = c.take((size_t)f.n_gu * sizeof(int4));
  f.tab_dn = c.take((size_t)f.n_dn * sizeof(int4));
  f.row_done = c.take((size_t)R * 4);
  f.total = c.off;
  return f;
}

extern "C" {

size_t moe_layer_fused_workspace_bytes(int64_t T, int D, int E, int k, int I, int I_shared) {
  if (T < 0 || D <= 0 || E <= 0 || k <= 0 || I <= 0) return 0;
  return fused_layout(T, D, E, k, I, I_shared > 0 ? I_shared : 0).total;
}

int moe_layer_forward_fused(const void* x, const int32_t* token_ids, const void* w_router,
                            const float* bias, const moe_expert_weights* routed,
                            const moe_expert_weights* shared, int64_t T, int D, int E, int k,
                            int I, int I_shared, moe_route mode, moe_dtype act, uint32_t flags,
                            void* y, void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  if (act != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the single-launch forward runs bf16 activations only");
  if ((rc = check_dims(T, D, E, k))) return rc;
  int glu;
  if (flags & MOE_FLAG_W4A8)
    return fail(MOE_ERR_UNSUPPORTED, "the single-launch forward does not run MOE_FLAG_W4A8");
  if ((rc = glu_from_flags(flags, &glu))) return rc;
  if (I < 32 || I % 32) return fail(MOE_ERR_SHAPE, "I=%d must be a positive multiple of 32", I);
  if (mode != MOE_ROUTE_SOFTMAX && mode != MOE_ROUTE_SIGMOID && mode != MOE_ROUTE_HASH)
    return fail(MOE_ERR_SHAPE, "unknown routing mode %d", (int)mode);
  if ((rc = check_weights(routed, act, "routed"))) return rc;
  const int Is = shared ? I_shared : 0;
  if (shared) {
    if ((rc = check_weights(shared, act, "shared"))) return rc;
    if (shared->dtype != MOE_BF16)
      return fail(MOE_ERR_UNSUPPORTED, "the single-launch forward runs a bf16 shared expert");
    if (Is < 32 || Is % 32)
      return fail(MOE_ERR_SHAPE, "I_shared=%d must be a positive multiple of 32", I_shared);
  }
  if (T > 0 && (!x || !y)) return fail(MOE_ERR_NULL, "x / y are NULL");
  if (T > 0 && (!aligned(x, 16) || !aligned(y, 16)))
    return fail(MOE_ERR_ALIGN, "x / y must be 16-byte aligned");
  if (mode == MOE_ROUTE_HASH) {
    if (!token_ids) return fail(MOE_ERR_NULL, "hash routing needs token_ids");
  } else {
    if (!w_router) return fail(MOE_ERR_NULL, "w_router is NULL");
    if (!aligned(w_router, 16)) return fail(MOE_ERR_ALIGN, "w_router must be 16-byte aligned");
    if (bias && !aligned(bias, 4)) return fail(MOE_ERR_ALIGN, "bias misaligned");
  }
  const FusedLayout F = fused_layout(T, D, E, k, I, Is);
  if (!workspace || workspace_bytes < F.total)
    return fail(MOE_ERR_WORKSPACE, "fused layer workspace needs %zu bytes", F.total);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (T == 0) return ok();

  const bool fp4 = routed->dtype == MOE_MXFP4;
  const int64_t R = T * k, W = (T + 63) / 64;
  const int cfg = moe::fused_cfg(R / E, fp4);
  int BM, BNg, BNd;
  moe::fused_tiles(cfg, &BM, &BNg, &BNd);
  char* ws = static_cast<char*>(workspace);
  char* lw = ws + F.layer;
  const LayerLayout& L = F.L;

  moe::FusedArgs a{};
  a.hdr = reinterpret_cast<moe::FusedHdr*>(ws);
  a.x = static_cast<const uint16_t*>(x);
  a.token_ids = token_ids;
  a.w_router = static_cast<const uint16_t*>(w_router);
  a.bias = bias;
  a.T = T;
  a.D = D;
  a.E = E;
  a.k = k;
  a.mode = (int)mode;
  a.logits = reinterpret_cast<float*>(lw + L.logits);
  a.idx = reinterpret_cast<int32_t*>(lw + L.idx);
  a.tw = reinterpret_cast<float*>(lw + L.w);
  a.mask = reinterpret_cast<uint64_t*>(lw + L.mask);
  a.W = W;
  a.wprefix = reinterpret_cast<int32_t*>(lw + L.wprefix);
  a.counts = reinterpret_cast<int32_t*>(lw + L.counts);
  a.offsets = reinterpret_cast<int32_t*>(lw + L.offsets);
  a.row_token = reinterpret_cast<int32_t*>(lw + L.row_token);
  a.pair_row = reinterpret_cast<int32_t*>(lw + L.pair_row);
  void* h = lw + L.h;
  void* hs = lw + L.hs;
  void* o = lw + L.o;
  void* sh = lw + L.s;
  int4* tab_gu = reinterpret_cast<int4*>(ws + F.tab_gu);
  int4* tab_dn = reinterpret_cast<int4*>(ws + F.tab_dn);
  a.tab_gu = tab_gu;
  a.tab_dn = tab_dn;
  a.row_done = reinterpret_cast<unsigned*>(ws + F.row_done);
  a.gu_ntiles = (I + BNg - 1) / BNg;
  a.glu = glu;

  int64_t n[moe::FP_COUNT] = {};
  // routing: logit tiles as the router kernels choose them by T, or hash blocks
  if (mode == MOE_ROUTE_HASH) {
    a.route_var = 3;
    n[moe::FP_ROUTE] = W;
  } else {
    int TT, EXP;  // tokens and experts per logit tile
    if (T < 16) { a.route_var = 0; TT = 1; EXP = 4; }
    else if (T <= 128) { a.route_var = 1; TT = 4; EXP = 8; }
    else { a.route_var = 2; TT = 16; EXP = 16; }
    a.route_gy = (E + EXP - 1) / EXP;
    n[moe::FP_ROUTE] = (T + TT - 1) / TT * a.route_gy;
    a.n_zero = (int64_t)E * W;
    n[moe::FP_TOPK] = (T + 3) / 4;
    int c = 1;
    while (c * 64 < E) c *= 2;
    a.topk_c = c;
  }
  // permutation and the routed tile tables
  moe::TileJobs jobs{};
  jobs.n = 2;
  jobs.BM = BM;
  const int64_t n_gu = routed_tile_bound(R, E, I, BM, BNg), n_dn = routed_tile_bound(R, E, D, BM, BNd);
  if (n_gu > F.n_gu || n_dn > F.n_dn)
    return fail(MOE_ERR_WORKSPACE, "tile tables exceed their workspace region");
  jobs.job[0] = moe::TileJob{tab_gu, n_gu, BM, BNg, 1, {1, 0}, {R, 0}, {I, 0}};
  jobs.job[1] = moe::TileJob{tab_dn, n_dn, BM, BNd, 1, {1, 0}, {R, 0}, {D, 0}};
  a.jobs = jobs;
  int64_t nperm = std::max((R + 1023) / 1024, (n_gu + n_dn + 511) / 512);
  a.n_perm = (int)std::min<int64_t>(std::max<int64_t>(nperm, 1), 64);
  n[moe::FP_PERM] = a.n_perm;
  n[moe::FP_GU] = n_gu;
  n[moe::FP_DN] = n_dn;
  // expert GEMM segments (routed rows gathered through row_token)
  a.gu_r = make_seg(x, a.row_token, a.offsets, R, E, D, I, routed, true, h);
  a.dn_r = make_seg(h, nullptr, a.offsets, R, E, I, D, routed, false, o);
  if (shared) {
    a.gu_s = make_seg(x, nullptr, nullptr, T, 1, D, Is, shared, true, hs);
    a.dn_s = make_seg(hs, nullptr, nullptr, T, 1, Is, D, shared, false, sh);
    a.sh_mt = (int)((T + BM - 1) / BM);
    n[moe::FP_SGU] = (int64_t)a.sh_mt * ((Is + BNg - 1) / BNg);
    n[moe::FP_SDN] = (int64_t)a.sh_mt * ((D + BNd - 1) / BNd);
  }
  // combine
  int tpt = 64;
  while (tpt < 256 && tpt * 8 < D) tpt *= 2;
  a.comb_tpt = tpt;
  a.comb_gy = (D / 8 + tpt - 1) / tpt;
  n[moe::FP_COMB] = (T + (256 / tpt) - 1) / (256 / tpt) * a.comb_gy;
  a.o = static_cast<const uint16_t*>(o);
  a.s = shared ? static_cast<const uint16_t*>(sh) : nullptr;
  a.y = static_cast<uint16_t*>(y);

  int64_t total = 0;
  for (int p = 0; p < moe::FP_COUNT; ++p) {
    a.start[p] = (unsigned)total;
    total += n[p];
  }
  if (total >= ((int64_t)1 << 31)) return fail(MOE_ERR_SHAPE, "too many tasks for one launch");
  a.start[moe::FP_COUNT] = (unsigned)total;
  const int64_t grid = moe::fused_grid(cfg, fp4, total);
  if (grid <= 0) return hip_status(hipGetLastError(), "fused occupancy query");
  return hip_status(moe::launch_layer_fused(a, cfg, fp4, grid, static_cast<hipStream_t>(stream)),
                    "fused layer");
}

}  // extern "C"
