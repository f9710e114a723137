// C ABI entry points: validation, planning, and the launch sequence.
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"
#include "muon.h"
#include "plan.h"

namespace {

using namespace muon;

struct State {
  hipStream_t stream = nullptr;
  void *ws = nullptr;
  size_t ws_bytes = 0;
  int32_t iters = 5;
  float coeffs[3] = {3.4445f, -4.7750f, 2.0315f};
  float eps = 1e-7f;
  uint32_t mode = MUON_NS_FULL | MUON_PACK_COST | MUON_AA_PLAIN;
  std::string err;
};

thread_local State g_state;

// Optional per-launch event pairs (muon_set_phase_timing).
struct Timing {
  bool on = false;
  std::vector<hipEvent_t> pool;  // 2 events per record, reused
  std::vector<int> kinds;        // kernel kind of record i
  ~Timing() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};
thread_local Timing g_timing;

enum TimedKind { kTPrep = 0, kTNorm, kTGram, kTAA, kTBX, kTFinish, kTAdamW, kTReduce, kTKinds };

// Runs `launch` (returning hipError_t) bracketed by events when timing is on.
template <class F>
hipError_t timed(int kind, hipStream_t st, F &&launch) {
  if (!g_timing.on) return launch();
  const size_t i = g_timing.kinds.size();
  while (g_timing.pool.size() < 2 * (i + 1)) {
    hipEvent_t e;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) return r;
    g_timing.pool.push_back(e);
  }
  hipError_t r = hipEventRecord(g_timing.pool[2 * i], st);
  if (r != hipSuccess) return r;
  r = launch();
  if (r != hipSuccess) return r;
  r = hipEventRecord(g_timing.pool[2 * i + 1], st);
  if (r != hipSuccess) return r;
  g_timing.kinds.push_back(kind);
  return hipSuccess;
}

muon_status fail(const Error &e) {
  g_state.err = e.msg;
  return e.status;
}
muon_status fail(muon_status s, const std::string &msg) {
  g_state.err = msg;
  return s;
}
muon_status ok() {
  g_state.err.clear();
  return MUON_OK;
}

// The A*A kernel forms B = c (A A + (b / c) A), so c must be nonzero and
// b / c finite.
bool coeffs_ok(const float *c) {
  return std::isfinite(c[0]) && std::isfinite(c[1]) && std::isfinite(c[2]) && c[2] != 0.f &&
         std::isfinite(c[1] / c[2]);
}
constexpr const char *kCoeffMsg = "coefficients must be finite, with c != 0 and b / c finite";

struct Sources {
  const muon_mat *data = nullptr;  // muon_ns_batched
  const muon_mat *W = nullptr, *G = nullptr, *M = nullptr;  // muon_step
};

// Workgroups of a persistent launch: one per compute unit of the current
// device, rounded down to a multiple of the 8 XCDs (0 if unknown).
int persistent_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return (cus / 8) * 8;
}

// Persistent launch of `grid` workgroups over a's tiles (phase: whose K
// loop), if there are more tiles than workgroups: the XCDs' tile ranges
// balanced by estimated time (xcd_ranges).
void set_persistent(GemmArgs &a, int phase, int grid) {
  a.persistent = (grid > 0 && a.total_tiles > grid) ? grid : 0;
  if (!a.persistent) return;
  int64_t tiles[kSegsMax], ksteps[kSegsMax];
  for (int s = 0; s < a.nseg; ++s) {
    const GemmSeg &g = a.seg[s];
    tiles[s] = int64_t(g.tiles_per_view) * g.count;
    const int64_t k = phase == kGram ? g.np : phase == kAA ? (a.aa_plain ? g.mp : 3 * g.mp) : g.mp;
    ksteps[s] = k / 32;
  }
  xcd_ranges(tiles, ksteps, a.nseg, a.xcd_begin);
}

muon_status hip_fail(hipError_t e, const char *what) {
  return fail(MUON_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Launch sequence for every group of views that fits the workspace.
muon_status execute(const Plan &plan, const Sources &src, bool step, float lr, float beta, int nesterov,
                    const float coeffs[3], float eps, void *workspace) {
  hipStream_t st = g_state.stream;
  char *ws = static_cast<char *>(workspace);
  const bool bf16 = plan.bf16;
  const int iters = plan.iters;
  const int fin = iters & 1;
  const int slots = bf16 ? persistent_slots() : 0;

  for (const Chunk &ch : plan.chunks) {
    // per-view workspace blocks, in plan order
    std::vector<char *> blocks;
    blocks.reserve(ch.count);
    for (const Segment &sg : ch.segs)
      for (int32_t k = 0; k < sg.count; ++k) blocks.push_back(ws + sg.base + size_t(k) * sg.stride);

    // grouped-launch segment descriptors
    GemmArgs ga{};
    ga.nseg = int32_t(ch.segs.size());
    ga.a = coeffs[0];
    ga.b = coeffs[1];
    ga.c = coeffs[2];
    ga.r = coeffs[1] / coeffs[2];
    ga.eps = eps;
    ga.aa_plain = ((plan.mode & MUON_AA_SPLIT) || iters > kPlainMaxIters) ? 0 : 1;
    ga.group = plan.distributed ? plan.shards : 1;
    // halves of A written (by the Gram, or in distributed mode by the sum)
    ga.gram_halves = ga.aa_plain ? 1 : 2;
    ga.tri_out = (plan.distributed && bf16) ? 1 : 0;
    ga.remap = 1;
    int32_t view_begin = 0;
    for (size_t s = 0; s < ch.segs.size(); ++s) {
      const Segment &sg = ch.segs[s];
      const Layout L = view_layout(sg.mp, sg.np, bf16, plan.distributed);
      GemmSeg &g = ga.seg[s];
      g.base = ws + sg.base;
      g.stride = int64_t(sg.stride);
      for (int p = 0; p < 2; ++p) g.off_xa[p] = int64_t(L.xa[p]);
      for (int p = 0; p < 2; ++p) g.off_xt[p] = int64_t(L.xt[p]);
      g.off_ahi = int64_t(L.ahi);
      g.off_alo = int64_t(L.alo);
      g.off_b = int64_t(L.b);
      g.off_bdiag = int64_t(L.bdiag);
      g.off_part = int64_t(L.partials);
      g.off_scale = int64_t(L.scale);
      g.off_tri = int64_t(L.tri);
      g.mp = int32_t(sg.mp);
      g.np = int32_t(sg.np);
      g.count = sg.count;
      g.tn = int32_t(sg.np / (bf16 ? kGemmTile : kPadF32));
      g.nparts = int32_t(L.nparts);
      g.view_begin = view_begin;
      view_begin += sg.count;
    }
    auto set_tiles = [&](bool syrk) {
      int64_t t = 0;
      for (size_t s = 0; s < ch.segs.size(); ++s) {
        const int64_t per = syrk ? ch.segs[s].tiles_syrk : ch.segs[s].tiles_gemm;
        ga.seg[s].tiles_per_view = int32_t(per);
        ga.seg[s].tile_begin = int32_t(t);
        t += per * ch.segs[s].count;
      }
      ga.total_tiles = int32_t(t);
    };

    // element-wise launches, up to kPrepViewsMax views each
    auto elem_pass = [&](bool prep) -> muon_status {
      ElemArgs ea{};
      ea.kind = prep ? (step ? kPrepStep : kPrepNs) : (step ? kFinishStep : kFinishNs);
      ea.beta = beta;
      ea.lr = lr;
      ea.nesterov = nesterov;
      ea.final_scale = iters == 0 ? 1 : 0;
      int32_t tiles = 0;
      auto flush = [&]() -> muon_status {
        ea.total_tiles = tiles;
        hipError_t e = timed(prep ? kTPrep : kTFinish, st, [&] { return launch_elem(ea, bf16, st); });
        if (e != hipSuccess) return hip_fail(e, prep ? "prep launch" : "finish launch");
        ea.nv = 0;
        tiles = 0;
        return MUON_OK;
      };
      for (int32_t k = 0; k < ch.count; ++k) {
        const View &v = plan.views[ch.first + k];
        const Layout L = view_layout(v.mp, v.np, bf16);
        const size_t es = bf16 ? 2 : 4;
        ElemView &e = ea.v[ea.nv];
        e = ElemView{};
        const muon_mat &mm = step ? src.M[v.mat] : src.data[v.mat];
        e.m = static_cast<char *>(mm.data) + size_t(v.col_off) * es;
        e.ld_m = mm.ld;
        if (step) {
          e.g = static_cast<const char *>(src.G[v.mat].data) + size_t(v.col_off) * es;
          e.ld_g = src.G[v.mat].ld;
          e.w = static_cast<char *>(src.W[v.mat].data) + size_t(v.col_off) * es;
          e.ld_w = src.W[v.mat].ld;
        }
        auto rows16 = [&](const void *ptr, int64_t ld) {
          return (reinterpret_cast<uintptr_t>(ptr) % 16 == 0 && (size_t(ld) * es) % 16 == 0) ? 1 : 0;
        };
        e.vec = (step ? rows16(e.g, e.ld_g) : 0) | (rows16(e.m, e.ld_m) << 1) | (step ? rows16(e.w, e.ld_w) << 2 : 0);
        e.blk = blocks[k];
        const int buf = prep ? 0 : fin;
        e.off_x = int64_t(L.xa[buf]);
        // X0^T too when a bf16 B X will read it
        e.off_xt = (prep && bf16 && iters > 0) ? int64_t(L.xt[0]) : -1;
        e.pitch_xt = int32_t(v.mp);
        e.off_part = int64_t(L.partials);
        e.off_scale = int64_t(L.scale);
        e.rows = int32_t(v.rows);
        e.cols = int32_t(v.cols);
        e.pitch_x = int32_t(v.np);
        e.tall = v.tall ? 1 : 0;
        int64_t tr, tcn;
        if (prep) {  // whole padded extent, so the padding is written as zeros
          tr = (v.tall ? v.np : v.mp) / kElemTile;
          tcn = (v.tall ? v.mp : v.np) / kElemTile;
        } else {
          tr = (v.rows + kElemTile - 1) / kElemTile;
          tcn = (v.cols + kElemTile - 1) / kElemTile;
        }
        e.tiles_c = int32_t(tcn);
        e.tile_begin = tiles;
        tiles += int32_t(tr * tcn);
        ea.nv++;
        if (ea.nv == kPrepViewsMax) {
          muon_status s = flush();
          if (s != MUON_OK) return s;
        }
      }
      if (ea.nv) return flush();
      return MUON_OK;
    };

    muon_status s = elem_pass(true);
    if (s != MUON_OK) return s;
    hipError_t e = timed(kTNorm, st, [&] { return launch_norm_finalize(ga, ch.count, st); });
    if (e != hipSuccess) return hip_fail(e, "norm launch");
    for (int it = 0; it < iters; ++it) {
      ga.src = it & 1;
      ga.first = it == 0 ? 1 : 0;
      set_tiles(true);
      // Gram: persistent workgroups, one per CU, each looping over tiles of
      // its XCD's range (measured -0.8% against one workgroup per tile)
      set_persistent(ga, kGram, slots);
      e = timed(kTGram, st, [&] { return launch_gemm(ga, kGram, bf16, st); });
      ga.persistent = 0;
      if (e != hipSuccess) return hip_fail(e, "gram launch");
      if (plan.distributed) {
        // the all-reduce of the partial Grams, simulated on this GPU
        auto per_matrix = [&](int64_t tile) {  // tile: edge of the tiles summed
          int64_t t = 0;
          for (size_t s = 0; s < ch.segs.size(); ++s) {
            const int64_t tt = ch.segs[s].mp / tile;
            ga.seg[s].tiles_per_view = int32_t(tt * (tt + 1) / 2 * (bf16 ? 4 : 1));
            ga.seg[s].tile_begin = int32_t(t);
            t += ga.seg[s].tiles_per_view * (ch.segs[s].count / ga.group);
          }
        };
        if (bf16) {
          // the Gram wrote tile-packed float32 partials: one workgroup per
          // quarter of an upper 256 x 256 tile of each matrix
          per_matrix(kGemmTile);
          e = timed(kTReduce, st, [&] { return launch_tile_sum(ga, st); });
          if (e != hipSuccess) return hip_fail(e, "tile sum launch");
        } else {
          // one workgroup per row of each view (pack), then per 64 x 64
          // upper tile of each matrix (sum)
          int64_t t = 0;
          for (size_t s = 0; s < ch.segs.size(); ++s) {
            ga.seg[s].tiles_per_view = int32_t(ch.segs[s].mp);
            ga.seg[s].tile_begin = int32_t(t);
            t += ch.segs[s].mp * ch.segs[s].count;
          }
          e = timed(kTReduce, st, [&] { return launch_tri_pack(ga, st); });
          if (e != hipSuccess) return hip_fail(e, "triangle pack launch");
          per_matrix(64);
          e = timed(kTReduce, st, [&] { return launch_tri_reduce(ga, st); });
          if (e != hipSuccess) return hip_fail(e, "triangle reduce launch");
        }
        set_tiles(true);
      }
      // A*A (short K loop as well): persistent workgroups (measured -1.5%)
      set_persistent(ga, kAA, slots);
      e = timed(kTAA, st, [&] { return launch_gemm(ga, kAA, bf16, st); });
      ga.persistent = 0;
      if (e != hipSuccess) return hip_fail(e, "A*A launch");
      set_tiles(false);
      // B X (short K loop): persistent workgroups, so that a tile's epilogue
      // stores overlap the next tile's first operand loads. The last one
      // writes the caller's matrices (data <- O or W <- W - lr O).
      set_persistent(ga, kBX, slots);
      ga.last = it == iters - 1 ? 1 : 0;
      ga.lr = lr;
      e = timed(kTBX, st, [&] { return launch_gemm(ga, kBX, bf16, st); });
      ga.persistent = 0;
      ga.last = 0;
      if (e != hipSuccess) return hip_fail(e, "B*X launch");
    }
    if (iters == 0) {  // nothing to fuse with: write back the normalized source
      s = elem_pass(false);
      if (s != MUON_OK) return s;
    }
  }
  return ok();
}

bool check_iters(int32_t iters, Error *err) {
  if (iters < 0 || iters > kMaxIters) return err->set(MUON_ERR_INVALID_ARG, "iters out of range [0, 64]");
  return true;
}

bool need_workspace(Error *err) {
  if (!g_state.ws) return err->set(MUON_ERR_WORKSPACE, "no workspace set (muon_set_workspace)");
  return true;
}

// Phase timing off for the duration of a call that may create no events.
struct TimingOff {
  bool was;
  TimingOff() : was(g_timing.on) { g_timing.on = false; }
  ~TimingOff() { g_timing.on = was; }
};

// muon_step on the given workspace (the thread's, or with noalloc the
// library's device scratch, whose address is looked up only after every
// host-side check has passed).
muon_status step_impl(const muon_mat *params, const muon_mat *grads, const muon_mat *moms, int32_t n_mats,
                      float lr, float beta, int32_t nesterov, bool noalloc) {
  Error err;
  const uint32_t mode = g_state.mode;
  if (!validate_descs(params, n_mats, mode, "params", &err) || !validate_descs(grads, n_mats, mode, "grads", &err) ||
      !validate_descs(moms, n_mats, mode, "moms", &err))
    return fail(err);
  if (n_mats > 0 && !validate_step_triplets(params, grads, moms, n_mats, &err)) return fail(err);
  if (!std::isfinite(lr) || !std::isfinite(beta)) return fail(MUON_ERR_INVALID_ARG, "lr and beta must be finite");
  if (nesterov != 0 && nesterov != 1) return fail(MUON_ERR_INVALID_ARG, "nesterov must be 0 or 1");
  if (n_mats == 0) return ok();
  const muon_mat *arrays[3] = {params, grads, moms};
  const bool writable[3] = {true, false, true};
  if (!check_alias(arrays, writable, 3, n_mats, &err)) return fail(err);
  const char *names[3] = {"params", "grads", "moms"};
  Plan plan;
  void *ws = g_state.ws;
  size_t ws_bytes = g_state.ws_bytes;
  if (noalloc) {
    ws_bytes = kNoAllocScratchBytes;
    if (!build_plan(params, n_mats, g_state.iters, mode, ws_bytes, &plan, &err))
      return fail(err.status, err.msg + " (muon_step_noalloc: the device scratch holds " +
                                  std::to_string(kNoAllocScratchBytes >> 20) + " MiB)");
    hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "scratch symbol address");
    if (!check_workspace_alias(arrays, names, 3, n_mats, ws, ws_bytes, &err)) return fail(err);
  } else if (!need_workspace(&err) || !check_workspace_alias(arrays, names, 3, n_mats, ws, ws_bytes, &err) ||
             !build_plan(params, n_mats, g_state.iters, mode, ws_bytes, &plan, &err)) {
    return fail(err);
  }
  Sources src;
  src.W = params;
  src.G = grads;
  src.M = moms;
  if (noalloc) {
    TimingOff off;
    return execute(plan, src, true, lr, beta, nesterov, g_state.coeffs, g_state.eps, ws);
  }
  return execute(plan, src, true, lr, beta, nesterov, g_state.coeffs, g_state.eps, ws);
}

}  // namespace

extern "C" {

muon_status muon_ns_batched(const muon_mat *descs, int32_t n_mats, int32_t iters, const float coeffs[3],
                            uint32_t mode) {
  Error err;
  static const float kDefault[3] = {3.4445f, -4.7750f, 2.0315f};
  const float *cf = coeffs ? coeffs : kDefault;
  if (!validate_mode(mode, &err) || !check_iters(iters, &err)) return fail(err);
  if (!coeffs_ok(cf)) return fail(MUON_ERR_INVALID_ARG, kCoeffMsg);
  if (!validate_descs(descs, n_mats, mode, "descs", &err)) return fail(err);
  if (n_mats == 0) return ok();
  const muon_mat *arrays[1] = {descs};
  const bool writable[1] = {true};
  if (!check_alias(arrays, writable, 1, n_mats, &err)) return fail(err);
  const char *names[1] = {"descs"};
  Plan plan;
  if (!need_workspace(&err) ||
      !check_workspace_alias(arrays, names, 1, n_mats, g_state.ws, g_state.ws_bytes, &err) ||
      !build_plan(descs, n_mats, iters, mode, g_state.ws_bytes, &plan, &err))
    return fail(err);
  Sources src;
  src.data = descs;
  return execute(plan, src, false, 0.f, 0.f, 0, cf, g_state.eps, g_state.ws);
}

muon_status muon_step(const muon_mat *params, const muon_mat *grads, const muon_mat *moms, int32_t n_mats,
                      float lr, float beta, int32_t nesterov) {
  return step_impl(params, grads, moms, n_mats, lr, beta, nesterov, false);
}

muon_status muon_step_noalloc(const muon_mat *params, const muon_mat *grads, const muon_mat *moms, int32_t n_mats,
                              float lr, float beta, int32_t nesterov) {
  return step_impl(params, grads, moms, n_mats, lr, beta, nesterov, true);
}

muon_status muon_set_stream(void *hip_stream) {
  g_state.stream = static_cast<hipStream_t>(hip_stream);
  return ok();
}

muon_status muon_workspace_size(const muon_mat *descs, int32_t n_mats, uint32_t mode, size_t *bytes) {
  Error err;
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  if (!validate_mode(mode, &err) || !validate_descs(descs, n_mats, mode, "descs", &err)) return fail(err);
  Plan plan;
  if (!build_plan(descs, n_mats, 1, mode, 0, &plan, &err)) return fail(err);
  *bytes = plan.full_bytes;
  return ok();
}

muon_status muon_workspace_min_size(const muon_mat *descs, int32_t n_mats, uint32_t mode, size_t *bytes) {
  Error err;
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  if (!validate_mode(mode, &err) || !validate_descs(descs, n_mats, mode, "descs", &err)) return fail(err);
  Plan plan;
  if (!build_plan(descs, n_mats, 1, mode, 0, &plan, &err)) return fail(err);
  *bytes = plan.min_bytes;
  return ok();
}

muon_status muon_set_workspace(void *device_ptr, size_t bytes) {
  if ((device_ptr == nullptr) != (bytes == 0))
    return fail(MUON_ERR_INVALID_ARG, "workspace pointer and size must both be set or both be empty");
  if (reinterpret_cast<uintptr_t>(device_ptr) % 256) return fail(MUON_ERR_ALIGN, "workspace not 256-byte aligned");
  g_state.ws = device_ptr;
  g_state.ws_bytes = bytes;
  return ok();
}

muon_status muon_set_step_options(int32_t iters, const float coeffs[3], float eps, uint32_t mode) {
  Error err;
  if (!check_iters(iters, &err) || !validate_mode(mode, &err)) return fail(err);
  if (!std::isfinite(eps) || eps < 0.f) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (coeffs && !coeffs_ok(coeffs)) return fail(MUON_ERR_INVALID_ARG, kCoeffMsg);
  g_state.iters = iters;
  if (coeffs) std::memcpy(g_state.coeffs, coeffs, sizeof g_state.coeffs);
  g_state.eps = eps;
  g_state.mode = mode;
  return ok();
}

const char *muon_last_error(void) { return g_state.err.c_str(); }

muon_status muon_set_phase_timing(int32_t enable) {
  g_timing.on = enable != 0;
  return ok();
}

muon_status muon_phase_times(double ms[8], int64_t launches[8]) {
  double acc[kTKinds] = {};
  int64_t cnt[kTKinds] = {};
  for (size_t i = 0; i < g_timing.kinds.size(); ++i) {
    hipError_t r = hipEventSynchronize(g_timing.pool[2 * i + 1]);
    float t = 0.f;
    if (r == hipSuccess) r = hipEventElapsedTime(&t, g_timing.pool[2 * i], g_timing.pool[2 * i + 1]);
    if (r != hipSuccess) {
      g_timing.kinds.clear();
      return hip_fail(r, "phase timing");
    }
    acc[g_timing.kinds[i]] += double(t);
    cnt[g_timing.kinds[i]] += 1;
  }
  g_timing.kinds.clear();
  for (int k = 0; k < kTKinds; ++k) {
    if (ms) ms[k] = acc[k];
    if (launches) launches[k] = cnt[k];
  }
  return ok();
}

muon_status muon_plan_info(const muon_mat *descs, int32_t n_mats, int32_t iters, uint32_t mode,
                           size_t workspace_bytes, char *buf, size_t len, size_t *needed) {
  Error err;
  if (!validate_mode(mode, &err) || !check_iters(iters, &err) ||
      !validate_descs(descs, n_mats, mode, "descs", &err))
    return fail(err);
  Plan plan;
  if (!build_plan(descs, n_mats, iters, mode, workspace_bytes, &plan, &err)) return fail(err);
  const std::string js = plan_json(plan);
  if (needed) *needed = js.size() + 1;
  if (buf && len) {
    const size_t n = js.size() < len - 1 ? js.size() : len - 1;
    std::memcpy(buf, js.data(), n);
    buf[n] = 0;
  }
  return ok();
}

muon_status muon_place(const double *costs, int32_t n_mats, int32_t ranks, uint32_t policy,
                       int32_t *owner, double *load, double *imbalance) {
  if (n_mats < 0 || n_mats > kMaxMats) return fail(MUON_ERR_INVALID_ARG, "n_mats out of range");
  if (ranks < 1 || ranks > 65536) return fail(MUON_ERR_INVALID_ARG, "ranks out of range [1, 65536]");
  if (policy != MUON_PLACE_RR && policy != MUON_PLACE_LPT) return fail(MUON_ERR_INVALID_ARG, "unknown policy");
  if (n_mats > 0 && (!costs || !owner)) return fail(MUON_ERR_INVALID_ARG, "costs and owner must not be NULL");
  for (int32_t i = 0; i < n_mats; ++i)
    if (!std::isfinite(costs[i]) || costs[i] < 0)
      return fail(MUON_ERR_INVALID_ARG, "costs must be finite and >= 0 (index " + std::to_string(i) + ")");
  std::vector<double> ld(static_cast<size_t>(ranks));
  std::vector<int32_t> own(static_cast<size_t>(n_mats));
  place(costs, n_mats, ranks, policy, own.data(), ld.data());
  for (int32_t i = 0; i < n_mats; ++i) owner[i] = own[size_t(i)];
  if (load)
    for (int32_t r = 0; r < ranks; ++r) load[r] = ld[size_t(r)];
  if (imbalance) {
    double mx = 0, sum = 0;
    for (double v : ld) {
      mx = v > mx ? v : mx;
      sum += v;
    }
    *imbalance = sum > 0 ? mx / (sum / ranks) : 1.0;
  }
  return ok();
}

muon_status muon_adamw_step(const muon_mat *params, const muon_mat *grads, const muon_mat *exp_avg,
                            const muon_mat *exp_avg_sq, int32_t n_mats, float lr, float beta1, float beta2,
                            float eps, float weight_decay, int32_t step) {
  Error err;
  if (n_mats < 0 || n_mats > kMaxMats) return fail(MUON_ERR_INVALID_ARG, "n_mats out of range");
  if (n_mats > 0 && (!params || !grads || !exp_avg || !exp_avg_sq))
    return fail(MUON_ERR_INVALID_ARG, "descriptor arrays must not be NULL");
  if (!std::isfinite(lr) || !std::isfinite(weight_decay))
    return fail(MUON_ERR_INVALID_ARG, "lr and weight_decay must be finite");
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
    return fail(MUON_ERR_INVALID_ARG, "beta1 and beta2 must lie in [0, 1)");
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (step < 1) return fail(MUON_ERR_INVALID_ARG, "step must be >= 1");
  if (n_mats == 0) return ok();
  const int32_t pdt = params[0].dtype;
  if (pdt != MUON_F32 && pdt != MUON_BF16) return fail(MUON_ERR_DTYPE, "params: unknown dtype");
  const size_t pes = dtype_size(pdt);
  for (int32_t i = 0; i < n_mats; ++i) {
    const muon_mat *ds[4] = {&params[i], &grads[i], &exp_avg[i], &exp_avg_sq[i]};
    const char *names[4] = {"params", "grads", "exp_avg", "exp_avg_sq"};
    for (int k = 0; k < 4; ++k) {
      const muon_mat &d = *ds[k];
      const std::string at = std::string(names[k]) + "[" + std::to_string(i) + "]";
      const int32_t want = k < 2 ? pdt : int32_t(MUON_F32);
      if (d.dtype != want)
        return fail(MUON_ERR_DTYPE, at + ": params and grads share one dtype; exp_avg and exp_avg_sq are float32");
      if (!d.data) return fail(MUON_ERR_INVALID_ARG, at + ": NULL data");
      if (d.rows <= 0 || d.cols <= 0 || d.ld < d.cols)
        return fail(MUON_ERR_SHAPE, at + ": rows, cols must be > 0 and ld >= cols");
      if (d.rows != params[i].rows || d.cols != params[i].cols)
        return fail(MUON_ERR_SHAPE, at + ": shape differs from params[" + std::to_string(i) + "]");
      if (reinterpret_cast<uintptr_t>(d.data) % dtype_size(d.dtype))
        return fail(MUON_ERR_ALIGN, at + ": data not aligned to its element size");
    }
    if (params[i].rows * ((params[i].cols + 7) / 8) > (int64_t(1) << 30))
      return fail(MUON_ERR_SHAPE, "params[" + std::to_string(i) + "]: more than 2^33 elements");
  }
  const muon_mat *arrays[4] = {params, exp_avg, exp_avg_sq, grads};
  const bool writable[4] = {true, true, true, false};
  if (!check_alias(arrays, writable, 4, n_mats, &err)) return fail(err);

  const double bc1 = 1.0 - std::pow(double(beta1), double(step));
  const double bc2 = 1.0 - std::pow(double(beta2), double(step));
  AdamArgs a{};
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  a.decay = float(1.0 - double(lr) * double(weight_decay));
  a.step_size = float(double(lr) / bc1);
  a.inv_sqrt_bc2 = float(1.0 / std::sqrt(bc2));
  hipStream_t st = g_state.stream;
  auto flush = [&]() -> muon_status {
    hipError_t e = timed(kTAdamW, st, [&] { return launch_adamw(a, pdt == MUON_BF16, st); });
    a.nv = 0;
    a.total_chunks = 0;
    return e == hipSuccess ? MUON_OK : hip_fail(e, "adamw launch");
  };
  auto rows16 = [](const void *p, int64_t ld, size_t es) {
    return reinterpret_cast<uintptr_t>(p) % 16 == 0 && (size_t(ld) * es) % 16 == 0;
  };
  for (int32_t i = 0; i < n_mats; ++i) {
    const int64_t cpr = (params[i].cols + 7) / 8;
    const int64_t chunks = params[i].rows * cpr;
    if (a.nv == kAdamViewsMax || int64_t(a.total_chunks) + chunks > (int64_t(1) << 31) - 256) {
      muon_status s = flush();
      if (s != MUON_OK) return s;
    }
    AdamView &v = a.v[a.nv];
    v = AdamView{};
    v.w = params[i].data;
    v.g = grads[i].data;
    v.m = static_cast<float *>(exp_avg[i].data);
    v.v = static_cast<float *>(exp_avg_sq[i].data);
    v.ld_w = params[i].ld;
    v.ld_g = grads[i].ld;
    v.ld_m = exp_avg[i].ld;
    v.ld_v = exp_avg_sq[i].ld;
    v.rows = int32_t(params[i].rows);
    v.cols = int32_t(params[i].cols);
    v.chunks_per_row = int32_t(cpr);
    v.chunk_begin = a.total_chunks;
    v.vec = (params[i].cols % 8 == 0 && rows16(v.w, v.ld_w, pes) && rows16(v.g, v.ld_g, pes) &&
             rows16(v.m, v.ld_m, 4) && rows16(v.v, v.ld_v, 4)) ? 1 : 0;
    a.total_chunks += int32_t(chunks);
    a.nv++;
  }
  if (a.nv) return flush();
  return ok();
}

}  // extern "C"
