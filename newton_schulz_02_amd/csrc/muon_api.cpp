// C ABI of libmuon: argument validation, planning, descriptor upload and the launch
// sequence of one owner-side Muon step (DMuon summary §2.1: the owner computes each
// update once; §2.2: Gram Newton-Schulz with the symmetric path and shape batching).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/muon.h"
#include "../../include/muon_test_hooks.h"
#include "muon_internal.h"
#include "planner.h"
#include "shampoo_plan.h"
#include "split_protocol.h"

using namespace muon;

// Set by the build to the hash of the kernel sources (build.py: kernel_hash).
#ifndef MUON_KERNEL_HASH
#define MUON_KERNEL_HASH "unversioned"
#endif

namespace {

thread_local std::string t_last_error;

int fail(int status, const std::string& msg) {
  t_last_error = msg;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  t_last_error = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
  return MUON_EHIP;
}

std::mutex g_mu;

// Pinned host staging for descriptor uploads: a ring of slots per device, each guarded by
// an event so a slot is rewritten only after its previous copy has left host memory.
struct Slot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool used = false;
};
struct DeviceState {
  bool checked = false;
  bool supported = false;
  int units = kMaxUnits;  // compute units (the tail split plans for them)
  Slot ring[4];
  int next = 0;
};
std::map<int, DeviceState> g_dev;

// Profiling records.
struct Rec {
  std::string name;
  int device;
  hipEvent_t a, b;
  double flops, bytes;
};
bool g_prof = false;
std::vector<Rec> g_recs;

// Kernel configuration per launch signature (filled by muon_tune or muon_tune_import), and
// a forced configuration for every launch (-1: none).
std::map<std::string, int> g_tune;
int g_force_cfg = -1;
// Test hook: run every 256 x 256 launch with 64-bit operand pointers (the path of operands of
// 2 GB and more).
bool g_flat_loads = false;
// Polls of a tail-split last piece's bounded wait (kSplitSpins; a test hook lowers it).
int g_split_spins = kSplitSpins;

// Caller holds g_mu.
int choose_cfg(const std::string& sig) {
  if (g_force_cfg >= 0) return g_force_cfg;
  auto it = g_tune.find(sig);
  return it == g_tune.end() ? -1 : it->second;  // -1: the planner's default for the launch
}
std::map<int, std::vector<hipEvent_t>> g_event_pool;

int current_device(int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return MUON_OK;
}

// Caller holds g_mu.
int check_device(int dev) {
  DeviceState& st = g_dev[dev];
  if (!st.checked) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    st.supported = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    st.units = std::max(1, std::min(int(prop.multiProcessorCount), kMaxUnits));
    st.checked = true;
    if (!st.supported)
      t_last_error = std::string("device architecture ") + prop.gcnArchName + " is not gfx950";
  }
  return st.supported ? MUON_OK : fail(MUON_EUNSUPPORTED, t_last_error);
}

// Caller holds g_mu.
int upload(int dev, const void* src, size_t bytes, void* dst, hipStream_t s) {
  DeviceState& st = g_dev[dev];
  Slot& sl = st.ring[st.next];
  st.next = (st.next + 1) % 4;
  hipError_t e;
  if (!sl.ev) {
    e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  }
  if (sl.used) {
    e = hipEventSynchronize(sl.ev);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (staging)");
  }
  if (sl.cap < bytes) {
    if (sl.host) hipHostFree(sl.host);
    sl.host = nullptr;
    sl.cap = 0;
    size_t cap = 4096;
    while (cap < bytes) cap *= 2;
    e = hipHostMalloc(&sl.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc (staging)");
    sl.cap = cap;
  }
  std::memcpy(sl.host, src, bytes);
  e = hipMemcpyAsync(dst, sl.host, bytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (descriptors)");
  e = hipEventRecord(sl.ev, s);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord (staging)");
  sl.used = true;
  return MUON_OK;
}

// Caller holds g_mu.
hipEvent_t take_event(int dev) {
  auto& pool = g_event_pool[dev];
  if (!pool.empty()) {
    hipEvent_t e = pool.back();
    pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // Timing only: the events are read after the stream has been synchronized, so they need
  // no system-scope fence, whose cache writeback would also slow the launch that follows.
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Run one launch, bracketed by timing events when profiling.  Caller holds g_mu.
template <typename F>
int timed(int dev, hipStream_t s, const char* name, double flops, double bytes, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  if (g_prof) {
    a = take_event(dev);
    b = take_event(dev);
    if (!a || !b) return fail(MUON_EHIP, "hipEventCreate (profiling)");
    const hipError_t e = hipEventRecord(a, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord (profiling)");
  }
  const int e = launch();
  if (e != hipSuccess) return hip_fail(hipError_t(e), name);
  if (g_prof) {
    const hipError_t eb = hipEventRecord(b, s);
    if (eb != hipSuccess) return hip_fail(eb, "hipEventRecord (profiling)");
    g_recs.push_back({name, dev, a, b, flops, bytes});
  }
  return MUON_OK;
}

// Enqueue one launch of the plan on stream s.  Caller holds g_mu.
int run_launch(int dev, hipStream_t s, const Plan& plan, const PlanLaunch& L, int cfg, char* ws,
               const muon_hparams* hp, int count) {
  const MatDesc* ddesc = reinterpret_cast<const MatDesc*>(ws + plan.desc_off);
  float* scale = reinterpret_cast<float*>(ws + plan.scale_off);
  float* partials = reinterpret_cast<float*>(ws + plan.partial_off);
  int32_t* split_cnt = reinterpret_cast<int32_t*>(ws + plan.split_cnt_off);
  int32_t* status = reinterpret_cast<int32_t*>(ws);
  if (L.kind == kLaunchMomentum) {
    MomArgs a;
    a.desc = ddesc;
    a.partials = partials;
    const bool first = &L == &plan.launches.front();
    a.status = first ? status : nullptr;
    a.split_cnt = first ? split_cnt : nullptr;
    a.split_cnt_n = first ? plan.split_cnt_n : 0;
    a.first = L.first;
    a.last = L.last;
    a.tile_begin = int32_t(plan.mats[L.first].mom_prefix);
    a.total_tiles = int32_t(L.tiles);
    a.beta = hp->beta;
    return timed(dev, s, L.dtype == kBF16 ? "momentum_bf16" : "momentum_f32", 0.0, L.bytes,
                 [&] { return muon_launch_momentum(a, L.dtype, s); });
  }
  if (L.kind == kLaunchNorm) {
    NormArgs a;
    a.desc = ddesc;
    a.partials = partials;
    a.scale = scale;
    a.count = count;
    a.eps = hp->eps;
    a.split_cnt = split_cnt;
    a.split_cnt_n = plan.split_cnt_n;
    return timed(dev, s, "norm", 0.0, 0.0, [&] { return muon_launch_norm(a, s); });
  }
  GemmArgs a;
  std::memset(&a, 0, sizeof a);
  a.desc = ddesc;
  a.scale = scale;
  a.pa = L.own_coef ? L.pa : hp->ns_a;
  a.pb = L.own_coef ? L.pb : hp->ns_b;
  a.pc = L.own_coef ? L.pc : hp->ns_c;
  const int shape = cfg_shape(cfg);
  const std::vector<GroupArg>& groups = L.groups_cfg[shape];
  a.ngroups = int32_t(groups.size());
  a.total_tiles = int32_t(L.tiles_cfg[shape]);
  for (size_t g = 0; g < groups.size(); ++g) a.g[g] = groups[g];
  const SplitPlan& sp = L.split_cfg[shape];
  const bool split = cfg_split(cfg) && sp.mode != kSplitNone;
  a.dp_tiles = split ? sp.dp_tiles : a.total_tiles;
  a.split_mode = split ? sp.mode : int(kSplitNone);
  a.split_c = sp.c;
  a.split_n = sp.n;
  a.tail_tiles = split ? sp.tail : 0;
  a.tail_wgs = split ? sp.tail_wgs : 0;
  a.split_cnt = split_cnt;
  a.split_slots = reinterpret_cast<float*>(ws + plan.split_slot_off);
  a.status = status;
  a.split_spins = g_split_spins;
  a.grid = a.dp_tiles + a.tail_wgs;
  a.buf32 = (L.buf_ok && !g_flat_loads) ? 1 : 0;
  if (split && (sp.tail > plan.split_cnt_n / 2 || sp.slots > plan.split_slots))
    return fail(MUON_EINVAL, "internal: tail split exceeds its workspace");
  const bool bf = L.dtype == kBF16;
  if (cfg_deep(cfg))
    return timed(dev, s, bf ? "gemm_deep_bf16" : "gemm_deep_f32", L.flops, 0.0,
                 [&] { return muon_launch_gemm_deep(a, L.dtype, s); });
  if (shape == kCfgWide)
    return timed(dev, s, bf ? "gemm_wide_bf16" : "gemm_wide_f32", L.flops, 0.0,
                 [&] { return muon_launch_gemm_wide(a, L.dtype, s); });
  if (shape == kShapeSmall)
    return timed(dev, s, bf ? "gemm_small_bf16" : "gemm_small_f32", L.flops, 0.0,
                 [&] { return muon_launch_gemm_small(a, L.dtype, s); });
  return timed(dev, s, bf ? "gemm_bf16" : "gemm_f32", L.flops, 0.0,
               [&] { return muon_launch_gemm(a, L.dtype, s); });
}

// Validate, plan (with the tuned kernel choices) and upload the descriptors.  Caller holds
// g_mu.
int prepare(const muon_matrix* mats, int32_t count, const muon_hparams* hp, void* workspace,
            size_t workspace_bytes, hipStream_t s, Plan* plan, int* dev) {
  std::string err;
  const CfgChooser chooser = [](const std::string& sig) { return choose_cfg(sig); };
  int rc = build_plan(mats, count, hp, plan, &err, &chooser);
  if (rc != MUON_OK) return fail(rc, err);
  if (count == 0) return MUON_OK;
  if (!workspace) return fail(MUON_EINVAL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(MUON_EINVAL, "workspace is not 256-byte aligned");
  if (workspace_bytes < plan->ws_bytes) {
    char buf[128];
    snprintf(buf, sizeof buf, "workspace has %zu bytes, needs %zu", workspace_bytes, plan->ws_bytes);
    return fail(MUON_ENOSPC, buf);
  }
  char* ws = static_cast<char*>(workspace);
  std::vector<MatDesc> descs;
  fill_descs(*plan, mats, hp, ws, &descs);
  if ((rc = current_device(dev)) != MUON_OK) return rc;
  if ((rc = check_device(*dev)) != MUON_OK) return rc;
  if (g_dev[*dev].units != plan->units) plan_splits(plan, g_dev[*dev].units);
  return upload(*dev, descs.data(), descs.size() * sizeof(MatDesc), ws + plan->desc_off, s);
}

}  // namespace

extern "C" {

const char* muon_version(void) { return "muon-gfx950 0.1.0"; }

const char* muon_strerror(int status) {
  switch (status) {
    case MUON_OK: return "success";
    case MUON_EINVAL: return "invalid argument";
    case MUON_ENOSPC: return "workspace too small";
    case MUON_EALIAS: return "overlapping buffers";
    case MUON_EHIP: return "HIP runtime error";
    case MUON_EUNSUPPORTED: return "unsupported device or request";
    case MUON_ESTALE: return "tuning table of other kernels";
    default: return "unknown status";
  }
}

const char* muon_last_error(void) { return t_last_error.c_str(); }

int muon_workspace_size(const muon_matrix* mats, int32_t count, const muon_hparams* hp,
                        size_t* bytes) {
  try {
    if (!bytes) return fail(MUON_EINVAL, "bytes is NULL");
    Plan plan;
    std::string err;
    const int rc = build_plan(mats, count, hp, &plan, &err);
    if (rc != MUON_OK) return fail(rc, err);
    *bytes = count > 0 ? plan.ws_bytes : 0;
    return MUON_OK;
  } catch (const std::exception& e) {
    return fail(MUON_EINVAL, e.what());
  }
}

int muon_step_cost(const muon_matrix* mats, int32_t count, const muon_hparams* hp, double* flops,
                   double* bytes) {
  try {
    Plan plan;
    std::string err;
    const int rc = build_plan(mats, count, hp, &plan, &err);
    if (rc != MUON_OK) return fail(rc, err);
    if (flops) *flops = plan.flops;
    if (bytes) *bytes = plan.bytes;
    return MUON_OK;
  } catch (const std::exception& e) {
    return fail(MUON_EINVAL, e.what());
  }
}

int muon_plan_describe(const muon_matrix* mats, int32_t count, const muon_hparams* hp, char* buf,
                       size_t len) {
  try {
    if (!buf || len == 0) return fail(MUON_EINVAL, "buf is NULL or empty");
    Plan plan;
    std::string err;
    std::lock_guard<std::mutex> lock(g_mu);
    const CfgChooser chooser = [](const std::string& sig) { return choose_cfg(sig); };
    const int rc = build_plan(mats, count, hp, &plan, &err, &chooser);
    if (rc != MUON_OK) return fail(rc, err);
    const std::string s = describe_plan(plan);
    const size_t n = std::min(len - 1, s.size());
    std::memcpy(buf, s.data(), n);
    buf[n] = '\0';
    if (s.size() >= len) return fail(MUON_ENOSPC, "description truncated");
    return MUON_OK;
  } catch (const std::exception& e) {
    return fail(MUON_EINVAL, e.what());
  }
}

int muon_step(const muon_matrix* mats, int32_t count, const muon_hparams* hp, void* workspace,
              size_t workspace_bytes, void* hip_stream) {
  try {
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    std::lock_guard<std::mutex> lock(g_mu);
    Plan plan;
    int dev = 0;
    int rc = prepare(mats, count, hp, workspace, workspace_bytes, s, &plan, &dev);
    if (rc != MUON_OK || count == 0) return rc;
    char* ws = static_cast<char*>(workspace);
    for (const PlanLaunch& L : plan.launches) {
      rc = run_launch(dev, s, plan, L, L.cfg, ws, hp, count);
      if (rc != MUON_OK) return rc;
    }
    return MUON_OK;
  } catch (const std::exception& e) {
    return fail(MUON_EHIP, std::string("exception: ") + e.what());
  }
}

namespace {
// Bytes of the tuning copies of a list: its params and momenta, each 256-byte aligned.
size_t tune_scratch_bytes(const muon_matrix* mats, int32_t count) {
  size_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    const size_t bytes = size_t(mats[i].rows) * size_t(mats[i].cols) * (mats[i].dtype == MUON_BF16 ? 2 : 4);
    total += 2 * ((bytes + 255) / 256 * 256);
  }
  return total;
}
}  // namespace

int muon_step_noalloc(const muon_matrix* mats, int32_t count, const muon_hparams* hp, void* hip_stream) {
  try {
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    std::lock_guard<std::mutex> lock(g_mu);
    Plan plan;
    std::string err;
    const CfgChooser chooser = [](const std::string& sig) { return choose_cfg(sig); };
    int rc = build_plan(mats, count, hp, &plan, &err, &chooser);
    if (rc != MUON_OK) return fail(rc, err);
    if (count == 0) return MUON_OK;
    int dev = 0;
    if ((rc = current_device(&dev)) != MUON_OK) return rc;
    if ((rc = check_device(dev)) != MUON_OK) return rc;
    if (g_dev[dev].units != plan.units) plan_splits(&plan, g_dev[dev].units);
    if (plan.ws_bytes > kNoAllocBytes)
      return fail(MUON_ENOSPC, "muon_step_noalloc: the list needs " + std::to_string(plan.ws_bytes) +
                                   " bytes of scratch, more than the " + std::to_string(kNoAllocBytes) +
                                   " it has; use muon_step with a workspace");
    void* scratch = nullptr;
    const int e = muon_noalloc_scratch(dev, &scratch);
    if (e != hipSuccess) return hip_fail(hipError_t(e), "hipGetSymbolAddress (no-allocation scratch)");
    char* ws = static_cast<char*>(scratch);
    std::vector<MatDesc> descs;
    fill_descs(plan, mats, hp, ws, &descs);
    const int eu = muon_put_words(ws + plan.desc_off, descs.data(), descs.size() * sizeof(MatDesc), s);
    if (eu != hipSuccess) return hip_fail(hipError_t(eu), "descriptor upload (kernel arguments)");
    const bool prof = g_prof;
    g_prof = false;  // no profiling events on this path
    for (const PlanLaunch& L : plan.launches) {
      rc = run_launch(dev, s, plan, L, L.cfg, ws, hp, count);
      if (rc != MUON_OK) break;
    }
    g_prof = prof;
    return rc;
  } catch (const std::exception& ex) {
    return fail(MUON_EHIP, std::string("exception: ") + ex.what());
  }
}

int muon_tune_scratch_size(const muon_matrix* mats, int32_t count, const muon_hparams* hp, size_t* bytes) {
  try {
    if (!bytes) return fail(MUON_EINVAL, "bytes is NULL");
    Plan check;
    std::string err;
    const int rc = build_plan(mats, count, hp, &check, &err);
    if (rc != MUON_OK) return fail(rc, err);
    *bytes = count == 0 ? 0 : tune_scratch_bytes(mats, count);
    return MUON_OK;
  } catch (const std::exception& e) {
    return fail(MUON_EHIP, std::string("exception: ") + e.what());
  }
}

int muon_tune(const muon_matrix* mats, int32_t count, const muon_hparams* hp, void* workspace,
              size_t workspace_bytes, void* scratch, size_t scratch_bytes, void* hip_stream, int32_t reps) {
  try {
    if (reps < 1 || reps > 64) return fail(MUON_EINVAL, "reps must be in [1, 64]");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    std::lock_guard<std::mutex> lock(g_mu);
    {  // validate the caller's list as muon_step would (host only)
      Plan check;
      std::string err;
      const int rc = build_plan(mats, count, hp, &check, &err);
      if (rc != MUON_OK) return fail(rc, err);
      if (count == 0) return MUON_OK;
    }
    // The trial launches re-run in-place phases (momentum, the weight update), so the step
    // runs on copies of the params and momenta in the caller's scratch; the caller's
    // matrices are unchanged.
    const size_t total = tune_scratch_bytes(mats, count);
    if (!scratch) return fail(MUON_EINVAL, "scratch is NULL");
    if (scratch_bytes < total)
      return fail(MUON_ENOSPC, "tuning scratch too small: " + std::to_string(scratch_bytes) + " < " +
                                   std::to_string(total) + " bytes");
    if (reinterpret_cast<uintptr_t>(scratch) % 256 != 0) return fail(MUON_EINVAL, "scratch is not 256-byte aligned");
    char* copy = static_cast<char*>(scratch);
    std::vector<muon_matrix> shadow(mats, mats + count);
    hipError_t e = hipSuccess;
    size_t off = 0;
    for (int32_t i = 0; i < count && e == hipSuccess; ++i) {
      const size_t bytes = size_t(mats[i].rows) * size_t(mats[i].cols) * (mats[i].dtype == MUON_BF16 ? 2 : 4);
      const size_t step = (bytes + 255) / 256 * 256;
      shadow[size_t(i)].param = copy + off;
      shadow[size_t(i)].momentum = copy + off + step;
      off += 2 * step;
      e = hipMemcpyAsync(shadow[size_t(i)].param, mats[i].param, bytes, hipMemcpyDeviceToDevice, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(shadow[size_t(i)].momentum, mats[i].momentum, bytes, hipMemcpyDeviceToDevice, s);
    }
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (tuning copies)");

    const int saved_force = g_force_cfg;
    g_force_cfg = kCfgSquare;  // the plan's own groups are the square ones; trials use all
    Plan plan;
    int dev = 0;
    int rc = prepare(shadow.data(), count, hp, workspace, workspace_bytes, s, &plan, &dev);
    g_force_cfg = saved_force;
    if (rc != MUON_OK) {
      hipStreamSynchronize(s);
      return rc;
    }
    char* ws = static_cast<char*>(workspace);
    const bool prof = g_prof;
    g_prof = false;  // the trial launches are not part of a profile
    // Two events per trial: rounds x configurations trials per launch.
    std::vector<hipEvent_t> ev(size_t(2 * reps * kNumCfg), nullptr);
    for (size_t i = 0; i < ev.size() && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
    // Every launch runs once in order, so that each sees the operands of a real step.  Then
    // each MFMA launch is timed in `reps` rounds; a round runs it once under every kernel
    // configuration that applies to it (the 256 x 384 tiles when its operands fit their
    // offsets, the tail split when it has a tail to cut), so clock drift affects all of
    // them alike.  The configuration with the smallest median wins, and a non-default one
    // only when it is at least kTuneMargin faster than the default: near-ties keep the
    // default, so repeated tunings agree.  The kernels' run time does not depend on the
    // values, so the trials' repeated in-place writes do not bias later timings.
    constexpr float kTuneMargin = 0.01f;
    for (const PlanLaunch& L : plan.launches) {
      if (e != hipSuccess || rc != MUON_OK) break;
      rc = run_launch(dev, s, plan, L, kCfgSquare, ws, hp, count);
      if (rc != MUON_OK || L.kind != kLaunchGemm) continue;
      bool valid[kNumCfg];
      for (int cfg = 0; cfg < kNumCfg; ++cfg)
        valid[cfg] = (cfg_shape(cfg) != kCfgWide || L.wide_ok) &&
                     (!cfg_split(cfg) || L.split_cfg[cfg_shape(cfg)].mode != kSplitNone);
      for (int r = 0; r < reps && rc == MUON_OK && e == hipSuccess; ++r)
        for (int cfg = 0; cfg < kNumCfg && rc == MUON_OK && e == hipSuccess; ++cfg) {
          if (!valid[cfg]) continue;
          hipEvent_t* pair = &ev[size_t(2 * (r * kNumCfg + cfg))];
          e = hipEventRecord(pair[0], s);
          if (e == hipSuccess) rc = run_launch(dev, s, plan, L, cfg, ws, hp, count);
          if (e == hipSuccess && rc == MUON_OK) e = hipEventRecord(pair[1], s);
        }
      if (e == hipSuccess && rc == MUON_OK) e = hipStreamSynchronize(s);
      float med[kNumCfg] = {};
      for (int cfg = 0; cfg < kNumCfg && e == hipSuccess; ++cfg) {
        if (!valid[cfg]) continue;
        std::vector<float> t(size_t(reps), 0.0f);
        for (int r = 0; r < reps && e == hipSuccess; ++r)
          e = hipEventElapsedTime(&t[size_t(r)], ev[size_t(2 * (r * kNumCfg + cfg))],
                                  ev[size_t(2 * (r * kNumCfg + cfg)) + 1]);
        std::sort(t.begin(), t.end());
        med[cfg] = reps % 2 ? t[size_t(reps / 2)] : 0.5f * (t[size_t(reps / 2) - 1] + t[size_t(reps / 2)]);
      }
      if (e == hipSuccess && rc == MUON_OK) {
        const int base = default_cfg(L.tiles_cfg[kCfgSquare]);  // what an untuned step runs
        int best = base;
        for (int cfg = 0; cfg < kNumCfg; ++cfg)
          if (valid[cfg] && med[cfg] < med[best]) best = cfg;
        g_tune[L.signature] = med[best] < (1.0f - kTuneMargin) * med[base] ? best : base;
      }
    }
    g_prof = prof;
    const hipError_t es = hipStreamSynchronize(s);  // the caller may reuse the scratch on return
    for (hipEvent_t x : ev)
      if (x) hipEventDestroy(x);
    if (rc != MUON_OK) return rc;
    if (e != hipSuccess) return hip_fail(e, "muon_tune timing");
    if (es != hipSuccess) return hip_fail(es, "hipStreamSynchronize (tuning)");
    return MUON_OK;
  } catch (const std::exception& ex) {
    return fail(MUON_EHIP, std::string("exception: ") + ex.what());
  }
}

int shampoo_workspace_size(const shampoo_matrix* mats, int32_t count, const shampoo_hparams* hp,
                           size_t* bytes) {
  try {
    if (!bytes) return fail(MUON_EINVAL, "bytes is NULL");
    ShampooPlan sp;
    std::string err;
    const int rc = build_shampoo_plan(mats, count, hp, &sp, &err);
    if (rc != MUON_OK) return fail(rc, err);
    *bytes = count > 0 ? sp.plan.ws_bytes : 0;
    return MUON_OK;
  } catch (const std::exception& e) {
    return fail(MUON_EINVAL, e.what());
  }
}

int shampoo_plan_describe(const shampoo_matrix* mats, int32_t count, const shampoo_hparams* hp,
                          char* buf, size_t len) {
  try {
    if (!buf || len == 0) return fail(MUON_EINVAL, "buf is NULL or empty");
    ShampooPlan sp;
    std::string err;
    std::lock_guard<std::mutex> lock(g_mu);
    const int rc = build_shampoo_plan(mats, count, hp, &sp, &err);
    if (rc != MUON_OK) return fail(rc, err);
    shampoo_plan_splits(&sp, kMaxUnits, g_force_cfg);
    const std::string s = describe_shampoo_plan(sp);
    const size_t n = std::min(len - 1, s.size());
    std::memcpy(buf, s.data(), n);
    buf[n] = '\0';
    if (s.size() >= len) return fail(MUON_ENOSPC, "description truncated");
    return MUON_OK;
  } catch (const std::exception& e) {
    return fail(MUON_EINVAL, e.what());
  }
}

int shampoo_step(const shampoo_matrix* mats, int32_t count, const shampoo_hparams* hp,
                 void* workspace, size_t workspace_bytes, void* hip_stream) {
  try {
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    std::lock_guard<std::mutex> lock(g_mu);
    ShampooPlan sp;
    std::string err;
    int rc = build_shampoo_plan(mats, count, hp, &sp, &err);
    if (rc != MUON_OK) return fail(rc, err);
    if (count == 0) return MUON_OK;
    if (!workspace) return fail(MUON_EINVAL, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(MUON_EINVAL, "workspace is not 256-byte aligned");
    if (workspace_bytes < sp.plan.ws_bytes) {
      char buf[128];
      snprintf(buf, sizeof buf, "workspace has %zu bytes, needs %zu", workspace_bytes, sp.plan.ws_bytes);
      return fail(MUON_ENOSPC, buf);
    }
    char* ws = static_cast<char*>(workspace);
    std::vector<MatDesc> descs;
    fill_shampoo_descs(sp, mats, hp, ws, &descs);
    int dev = 0;
    if ((rc = current_device(&dev)) != MUON_OK) return rc;
    if ((rc = check_device(dev)) != MUON_OK) return rc;
    shampoo_plan_splits(&sp, g_dev[dev].units, g_force_cfg);
    rc = upload(dev, descs.data(), descs.size() * sizeof(MatDesc), ws + sp.plan.desc_off, s);
    if (rc != MUON_OK) return rc;
    // The launches read only eps (the norm) and beta (unused: no momentum buffer) from here.
    muon_hparams h;
    std::memset(&h, 0, sizeof h);
    h.lr = hp->lr;
    h.eps = hp->eps;
    const int entries = int(descs.size());
    for (const PlanLaunch& L : sp.plan.launches) {
      if (L.kind == kLaunchCopyIn || L.kind == kLaunchCopyOut) {
        const bool in = L.kind == kLaunchCopyIn;
        double bytes = 0.0;
        for (int e = L.first; e < L.last; ++e) {
          const double m = double(sp.plan.mats[size_t(e)].m);
          bytes += 8.0 * m * m;
        }
        rc = timed(dev, s, "copy_stat", 0.0, bytes, [&]() -> int {
          for (int e = L.first; e < L.last; ++e) {
            const PlanMat& p = sp.plan.mats[size_t(e)];
            const int j = e - count;
            const shampoo_matrix& x = mats[sp.stat_mat[size_t(j)]];
            char* state = static_cast<char*>(sp.stat_right[size_t(j)] ? x.stat_right : x.stat_left);
            char* slot = ws + p.off[sp.stat_slot];
            const size_t row = size_t(p.m) * 4, pitch = size_t(p.mp) * 4;
            const hipError_t e2 = in ? hipMemcpy2DAsync(slot, pitch, state, row, row, size_t(p.m),
                                                        hipMemcpyDeviceToDevice, s)
                                     : hipMemcpy2DAsync(state, row, slot, pitch, row, size_t(p.m),
                                                        hipMemcpyDeviceToDevice, s);
            if (e2 != hipSuccess) return int(e2);
          }
          return int(hipSuccess);
        });
      } else {
        rc = run_launch(dev, s, sp.plan, L, L.cfg, ws, &h, entries);
      }
      if (rc != MUON_OK) return rc;
    }
    return MUON_OK;
  } catch (const std::exception& e) {
    return fail(MUON_EHIP, std::string("exception: ") + e.what());
  }
}

int muon_workspace_check(void* workspace, size_t workspace_bytes, void* hip_stream) {
  try {
    if (!workspace) {  // the current device's muon_step_noalloc scratch
      std::lock_guard<std::mutex> lock(g_mu);
      int dev = 0;
      const int rc = current_device(&dev);
      if (rc != MUON_OK) return rc;
      const int e = muon_noalloc_scratch(dev, &workspace);
      if (e != hipSuccess) return hip_fail(hipError_t(e), "hipGetSymbolAddress (no-allocation scratch)");
      workspace_bytes = kNoAllocBytes;
    }
    if (workspace_bytes < size_t(kStatusBytes)) return fail(MUON_EINVAL, "workspace smaller than its status word");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    int32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, workspace, sizeof word, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading the workspace status word");
    if (word == 0) return MUON_OK;
    const int32_t zero = 0;
    e = hipMemcpy(workspace, &zero, sizeof zero, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "clearing the workspace status word");
    if (word == kStatusSplitTimeout)
      return fail(MUON_EHIP, "a tail-split wait timed out in the last step on this workspace; "
                             "the tile it was completing was stored as NaN");
    return fail(MUON_EHIP, "workspace status word " + std::to_string(word));
  } catch (const std::exception& e) {
    return fail(MUON_EHIP, std::string("exception: ") + e.what());
  }
}

int muon_debug_split_spins(int32_t spins) {
  if (spins < -2) return fail(MUON_EINVAL, "muon_debug_split_spins: spins must be >= -2");
  std::lock_guard<std::mutex> lock(g_mu);
  g_split_spins = spins == -1 ? kSplitSpins : spins;
  return MUON_OK;
}

namespace {
struct HostSplitOps {
  int32_t fetch_add(int32_t* p, int32_t v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
  int32_t load(int32_t* p) { return __atomic_load_n(p, __ATOMIC_SEQ_CST); }
  void store(int32_t* p, int32_t v) { __atomic_store_n(p, v, __ATOMIC_SEQ_CST); }
  void pause() { std::this_thread::yield(); }
};
}  // namespace

int muon_debug_split_protocol(int32_t pieces, int32_t mode, int32_t spin_limit, int32_t* out) {
  if (!out || pieces < 2 || pieces > kMaxPieces || mode < 0 || mode > 2 || spin_limit < -1)
    return fail(MUON_EINVAL, "muon_debug_split_protocol: bad arguments");
  int32_t cnt[2] = {0, 0}, status = 0, lasts = 0, ok = -1, seen = 0;
  int32_t slot[kMaxPieces] = {};
  HostSplitOps ops;
  // A piece of the tile: arrive; the others write their slot and publish; the last collects
  // and then checks that every other slot is written.
  auto piece = [&](int p, bool publish) {
    if (split_arrive(ops, cnt, pieces)) {
      __atomic_fetch_add(&lasts, 1, __ATOMIC_SEQ_CST);
      const bool good = split_collect(ops, cnt, pieces, spin_limit, &status);
      __atomic_store_n(&ok, good ? 1 : 0, __ATOMIC_SEQ_CST);
      if (good) {
        int n = 0;
        for (int q = 0; q < pieces; ++q) n += (q == p) || __atomic_load_n(&slot[q], __ATOMIC_SEQ_CST) == q + 1;
        __atomic_store_n(&seen, n, __ATOMIC_SEQ_CST);
      }
    } else if (publish) {
      __atomic_store_n(&slot[p], p + 1, __ATOMIC_SEQ_CST);
      split_publish(ops, cnt);
    }
  };
  if (mode == 0) {  // every piece on its own host thread
    std::vector<std::thread> th;
    for (int p = 0; p < pieces; ++p) th.emplace_back(piece, p, true);
    for (std::thread& t : th) t.join();
  } else {          // in piece order; mode 1: piece 0 arrives but does not publish in time
    for (int p = 0; p < pieces; ++p) piece(p, !(mode == 1 && p == 0));
  }
  out[0] = lasts;
  out[1] = ok;
  out[2] = cnt[0];
  out[3] = cnt[1];
  out[4] = status;
  out[5] = seen;
  out[6] = -1;
  out[7] = -1;
  if (mode == 1) {
    // The stalled piece publishes late; then a later launch's pieces of the same tile
    // arrive on the uncleared counters: none of them takes the last-piece role.
    __atomic_store_n(&slot[0], 1, __ATOMIC_SEQ_CST);
    split_publish(ops, cnt);
    int32_t later = 0;
    for (int p = 0; p < pieces; ++p) later += split_arrive(ops, cnt, pieces) ? 1 : 0;
    out[6] = cnt[1];
    out[7] = later;
  }
  return MUON_OK;
}

int muon_debug_split(int tiles, int units, int ksteps, int* plan, int* items, int max_items) {
  if (!plan || tiles < 0 || units < 1 || ksteps < 0 || max_items < 0)
    return fail(MUON_EINVAL, "muon_debug_split: bad arguments");
  const SplitPlan sp = plan_split(tiles, units, ksteps, kSplitUnit);
  const int out[6] = {sp.mode, sp.mode == kSplitEqual ? sp.c : sp.n, sp.dp_tiles, sp.tail,
                      sp.tail_wgs, sp.slots};
  std::memcpy(plan, out, sizeof out);
  for (int j = 0; items && j < sp.tail_wgs && j < max_items; ++j) {
    int t, piece, pieces, k0 = 0, k1 = 0;
    if (!split_item(sp.mode, sp.tail, sp.tail_wgs, sp.c, j, t, piece, pieces)) {
      const int none[5] = {-1, -1, -1, -1, -1};
      std::memcpy(items + 5 * j, none, sizeof none);
      continue;
    }
    split_range(sp.mode, sp.n, ksteps, kSplitUnit, piece, pieces, k0, k1);
    const int it[5] = {t, piece, pieces, k0, k1};
    std::memcpy(items + 5 * j, it, sizeof it);
  }
  return sp.tail_wgs;
}

int muon_debug_flat_loads(int32_t on) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_flat_loads = on != 0;
  return MUON_OK;
}

int muon_tune_force(int32_t cfg) {
  if (cfg < -1 || cfg >= kNumCfg) return fail(MUON_EINVAL, "cfg must be -1 or 0 .. 5");
  std::lock_guard<std::mutex> lock(g_mu);
  g_force_cfg = cfg;
  return MUON_OK;
}

void muon_tune_clear(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_tune.clear();
}

const char* muon_kernel_hash(void) { return MUON_KERNEL_HASH; }

int muon_tune_export(char* buf, size_t len, size_t* needed) {
  std::lock_guard<std::mutex> lock(g_mu);
  std::string out = std::string("# muon-tune ") + MUON_KERNEL_HASH + "\n";
  for (const auto& kv : g_tune) out += kv.first + " " + std::to_string(kv.second) + "\n";
  if (needed) *needed = out.size() + 1;
  if (!buf) return MUON_OK;
  if (len < out.size() + 1) return fail(MUON_ENOSPC, "buffer too small for the tuning table");
  std::memcpy(buf, out.c_str(), out.size() + 1);
  return MUON_OK;
}

int muon_tune_import(const char* text) {
  if (!text) return fail(MUON_EINVAL, "text is NULL");
  std::map<std::string, int> add;
  const char* p = text;
  while (*p) {
    const char* eol = std::strchr(p, '\n');
    const std::string line(p, eol ? size_t(eol - p) : std::strlen(p));
    p = eol ? eol + 1 : p + line.size();
    if (line.empty()) continue;
    if (line[0] == '#') {
      // "# muon-tune <hash>": the kernels the table was measured on
      static const std::string kTag = "# muon-tune ";
      if (line.compare(0, kTag.size(), kTag) == 0 && line.substr(kTag.size()) != MUON_KERNEL_HASH)
        return fail(MUON_ESTALE, "tuning table measured on kernels " + line.substr(kTag.size()) +
                                     ", this library's are " + MUON_KERNEL_HASH);
      continue;
    }
    const size_t sp = line.rfind(' ');
    if (sp == std::string::npos || sp == 0 || sp + 1 >= line.size())
      return fail(MUON_EINVAL, "tuning line without 'signature cfg': " + line);
    const std::string sig = line.substr(0, sp), val = line.substr(sp + 1);
    if (sig.find(' ') != std::string::npos || val.size() != 1 || val[0] < '0' ||
        val[0] >= char('0' + kNumCfg))
      return fail(MUON_EINVAL, "bad tuning line: " + line);
    add[sig] = val[0] - '0';
  }
  std::lock_guard<std::mutex> lock(g_mu);
  for (const auto& kv : add) g_tune[kv.first] = kv.second;
  return MUON_OK;
}

int adamw_step(float* p, const float* g, float* m, float* v, int64_t n, const adamw_hparams* hp,
               void* hip_stream) {
  try {
    if (!hp) return fail(MUON_EINVAL, "hparams is NULL");
    if (n < 0) return fail(MUON_EINVAL, "n is negative");
    const float fs[] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
    for (float f : fs)
      if (!std::isfinite(f)) return fail(MUON_EINVAL, "non-finite hyperparameter");
    if (hp->step < 1) return fail(MUON_EINVAL, "step must be >= 1");
    if (hp->beta1 < 0.0f || hp->beta1 >= 1.0f || hp->beta2 < 0.0f || hp->beta2 >= 1.0f)
      return fail(MUON_EINVAL, "beta1/beta2 outside [0, 1)");
    if (n == 0) return MUON_OK;
    if (!p || !g || !m || !v) return fail(MUON_EINVAL, "NULL pointer");
    const uintptr_t ptrs[4] = {(uintptr_t)p, (uintptr_t)g, (uintptr_t)m, (uintptr_t)v};
    for (uintptr_t x : ptrs)
      if (x % 4) return fail(MUON_EINVAL, "pointer not 4-byte aligned");
    const uintptr_t bytes = uintptr_t(n) * 4;
    for (int i = 0; i < 4; ++i)
      for (int j = i + 1; j < 4; ++j)
        if (ptrs[i] < ptrs[j] + bytes && ptrs[j] < ptrs[i] + bytes)
          return fail(MUON_EALIAS, "AdamW buffers overlap");
    AdamArgs a;
    a.p = p;
    a.g = g;
    a.m = m;
    a.v = v;
    a.n = n;
    a.lr = hp->lr;
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.eps = hp->eps;
    a.wd = hp->weight_decay;
    a.bc1 = float(1.0 - std::pow(double(hp->beta1), double(hp->step)));
    a.bc2 = float(1.0 - std::pow(double(hp->beta2), double(hp->step)));
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0, rc;
    if ((rc = current_device(&dev)) != MUON_OK) return rc;
    if ((rc = check_device(dev)) != MUON_OK) return rc;
    return timed(dev, s, "adamw", 0.0, 28.0 * double(n), [&] { return muon_launch_adamw(a, s); });
  } catch (const std::exception& e) {
    return fail(MUON_EHIP, std::string("exception: ") + e.what());
  }
}

int muon_profile_begin(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_prof = true;
  return MUON_OK;
}

int muon_profile_end(muon_kernel_stat* out, int32_t max, int32_t* count) {
  try {
    std::lock_guard<std::mutex> lock(g_mu);
    g_prof = false;
    std::vector<muon_kernel_stat> stats;
    int rc = MUON_OK;
    for (Rec& r : g_recs) {
      float ms = 0.0f;
      hipError_t e = hipEventSynchronize(r.b);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
      if (e != hipSuccess && rc == MUON_OK) rc = hip_fail(e, "hipEventElapsedTime");
      muon_kernel_stat* st = nullptr;
      for (auto& x : stats)
        if (r.name == x.name) st = &x;
      if (!st) {
        muon_kernel_stat z;
        std::memset(&z, 0, sizeof z);
        std::snprintf(z.name, sizeof z.name, "%s", r.name.c_str());
        stats.push_back(z);
        st = &stats.back();
      }
      st->launches += 1;
      st->ms += double(ms);
      st->flops += r.flops;
      st->bytes += r.bytes;
      g_event_pool[r.device].push_back(r.a);
      g_event_pool[r.device].push_back(r.b);
    }
    g_recs.clear();
    const int32_t n = int32_t(stats.size());
    if (count) *count = n;
    if (out)
      for (int32_t i = 0; i < n && i < max; ++i) out[i] = stats[size_t(i)];
    return rc;
  } catch (const std::exception& e) {
    return fail(MUON_EHIP, std::string("exception: ") + e.what());
  }
}

void muon_shutdown(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  for (auto& kv : g_dev) {
    for (Slot& sl : kv.second.ring) {
      if (sl.used && sl.ev) hipEventSynchronize(sl.ev);
      if (sl.host) hipHostFree(sl.host);
      if (sl.ev) hipEventDestroy(sl.ev);
      sl = Slot();
    }
  }
  for (auto& kv : g_event_pool)
    for (hipEvent_t e : kv.second) hipEventDestroy(e);
  g_event_pool.clear();
  g_dev.clear();
}

}  // extern "C"
