// api.cpp -- the C ABI (include/muon.h): plan lifecycle and the launch sequence.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/muon.h"
#include "kernels.h"
#include "planner.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MUON_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr uint32_t kPlanMagic = 0x4d554f4eu;  // "MUON"

struct TimedLaunch {
  int cls;
  hipEvent_t start, stop;
};

}  // namespace

struct muon_plan {
  uint32_t magic = kPlanMagic;
  muon::Plan p;
  int device = 0;
  char* ws = nullptr;
  std::vector<muon::PtrEntry> ptrs;  // last table uploaded (n_params entries, sized at creation)
  bool ptrs_valid = false;
  muon::PtrEntry* pinned = nullptr;  // staging for the upload
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
  // End of the last enqueued step: muon_plan_status and muon_plan_destroy
  // wait on it, and a step on another stream is ordered after it.
  hipEvent_t step_done = nullptr;
  hipStream_t step_stream = nullptr;
  bool step_recorded = false;
  muon::SkinnyBucket skinny_b0{};  // first skinny bucket (launch arguments); the table is in the workspace
  // graph of the streamed launches, keyed by ns_steps and stream
  hipGraphExec_t gexec = nullptr;
  int graph_ns = -1;
  hipStream_t graph_stream = nullptr;
  // timing
  std::vector<TimedLaunch> timed;
  std::vector<hipEvent_t> event_pool;
  double acc_ms[muon::kNumClasses] = {};
  int64_t acc_cnt[muon::kNumClasses] = {};
  uint32_t* err_word = nullptr;  // the device error word (in the workspace, or the caller's)
};

namespace {

bool plan_ok(muon_plan_t plan) { return plan != nullptr && plan->magic == kPlanMagic; }

template <typename T>
T* at(muon_plan_t plan, uint64_t off) {
  return reinterpret_cast<T*>(plan->ws + off);
}

hipEvent_t take_event(muon_plan_t plan) {
  if (!plan->event_pool.empty()) {
    hipEvent_t e = plan->event_pool.back();
    plan->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// A table the kernels read from the workspace: its offset and bytes.
struct Upload {
  uint64_t off;
  std::vector<char> bytes;
};

template <typename T>
void add_upload(std::vector<Upload>* ups, uint64_t off, const std::vector<T>& v) {
  Upload u{off, std::vector<char>(sizeof(T) * v.size())};
  std::memcpy(u.bytes.data(), v.data(), u.bytes.size());
  ups->push_back(std::move(u));
}

// The device tables of a plan whose workspace starts at plan->ws: every
// bucket's slice table, the skinny and large bucket arrays (which hold
// workspace addresses) and the large-tile tables.  Also sets
// plan->skinny_b0.  Returns false if the host is out of memory.
bool device_tables(muon_plan_t plan, std::vector<Upload>* ups) try {
  const muon::Plan& p = plan->p;
  for (const auto& bp : p.buckets) {
    std::vector<muon::DevMat> table;
    for (int si : bp.slices) {
      const muon::Slice& s = p.slices[si];
      muon::DevMat d;
      d.param = s.param;
      d.transposed = s.transposed;
      d.pdtype = s.pdtype;
      d.gdtype = s.gdtype;
      d.slice_off = s.slice_off;
      table.push_back(d);
    }
    add_upload(ups, bp.off_mats, table);
  }
  if (!p.skinny.empty()) {
    std::vector<muon::SkinnyBucket> sbs;
    int item0 = 0, slice0 = 0;
    for (int b : p.skinny) {
      const muon::BucketPlan& bp = p.buckets[b];
      muon::SkinnyBucket sb{};
      sb.mats = at<muon::DevMat>(plan, bp.off_mats);
      sb.gram_parts = at<double>(plan, bp.off_gram);
      sb.qs = at<float>(plan, bp.off_qs);
      sb.m = (int32_t)bp.m;
      sb.n = (int32_t)bp.n;
      sb.n_chunks = bp.n_chunks;
      sb.count = (int32_t)bp.slices.size();
      sb.item0 = item0;
      sb.slice0 = slice0;
      item0 += sb.count * sb.n_chunks;
      slice0 += sb.count;
      sbs.push_back(sb);
    }
    plan->skinny_b0 = sbs[0];
    add_upload(ups, p.off_skinny_params, sbs);
  }
  // The grouped streamed buckets: workgroup ranges counted in each phase's
  // output tiles (tile[ph] x tile[ph]).
  auto group_params = [&](const std::vector<int>& group, const int tile[3]) {
    std::vector<muon::SmallBucket> sbs;
    int64_t t0[3] = {0, 0, 0};
    for (int b : group) {
      const muon::BucketPlan& bp = p.buckets[b];
      muon::SmallBucket sb{};
      sb.mats = at<muon::DevMat>(plan, bp.off_mats);
      for (int i = 0; i < 2; ++i) {
        sb.x[i] = plan->ws + bp.off_x[i];
        sb.xt[i] = plan->ws + bp.off_xt[i];
      }
      sb.a32 = at<float>(plan, bp.off_a32);
      sb.phi = plan->ws + bp.off_phi;
      sb.plo = bp.p_hilo ? at<uint16_t>(plan, bp.off_plo) : nullptr;
      sb.scale = at<float>(plan, bp.off_scale);
      sb.m = bp.m;
      sb.n = bp.n;
      sb.mp = bp.mp;
      sb.np = bp.np;
      sb.count = (int32_t)bp.slices.size();
      for (int ph = 0; ph < 3; ++ph) {
        const int64_t ti = bp.mp / tile[ph], tj = (ph == 2 ? bp.np : bp.mp) / tile[ph];
        sb.t0[ph] = (int32_t)t0[ph];
        t0[ph] += ti * tj * sb.count;
      }
      sbs.push_back(sb);
    }
    return sbs;
  };
  if (!p.small.empty()) {
    const int tile[3] = {muon::kSmallTile, muon::kSmallTile, muon::kSmallTile};
    add_upload(ups, p.off_small_params, group_params(p.small, tile));
  }
  if (!p.mid.empty()) add_upload(ups, p.off_mid_params, group_params(p.mid, p.mid_bt));
  if (!p.big.empty()) {
    std::vector<muon::BigBucket> bbs;
    for (int b : p.big) {
      const muon::BucketPlan& bp = p.buckets[b];
      muon::BigBucket bb{};
      for (int i = 0; i < 2; ++i) {
        bb.x[i] = plan->ws + bp.off_x[i];
        bb.xt[i] = plan->ws + bp.off_xt[i];
      }
      bb.a32 = at<float>(plan, bp.off_a32);
      bb.e16 = at<uint16_t>(plan, bp.off_a16);
      bb.dg = at<float>(plan, bp.off_dg);
      bb.r16 = at<uint16_t>(plan, bp.off_phi);
      bb.scale = at<float>(plan, bp.off_scale);
      bb.mats = at<muon::DevMat>(plan, bp.off_mats);
      bb.m = bp.m;
      bb.n = bp.n;
      bb.mp = bp.mp;
      bb.np = bp.np;
      bb.vec = (bp.m % 4 == 0) && (bp.n % 4 == 0);
      bbs.push_back(bb);
    }
    add_upload(ups, p.off_big_params, bbs);
    for (int ph = 0; ph < 3; ++ph) add_upload(ups, p.off_big_tab[ph], p.big_tab[ph]);
  }
  return true;
} catch (const std::bad_alloc&) {
  return false;
}

// Run one launch, bracketed by events when timing is on.
template <class F>
hipError_t timed(muon_plan_t plan, int cls, hipStream_t s, bool timing, F&& launch) {
  if (!timing) return launch();
  hipEvent_t a = take_event(plan), b = take_event(plan);
  if (!a || !b) return hipErrorOutOfMemory;
  hipEventRecord(a, s);
  hipError_t e = launch();
  hipEventRecord(b, s);
  plan->timed.push_back({cls, a, b});
  return e;
}

// All skinny buckets: one launch per stage, each walking the bucket table.
hipError_t enqueue_skinny(muon_plan_t plan, hipStream_t s, bool timing, const muon::DevScalars* first) {
  const muon::Plan& p = plan->p;
  muon::SkinnyLaunch L{};
  L.b0 = plan->skinny_b0;
  L.buckets = at<muon::SkinnyBucket>(plan, p.off_skinny_params);
  L.n_buckets = (int)p.skinny.size();
  L.ptrs = at<muon::PtrEntry>(plan, p.off_ptrs);
  L.sc = at<muon::DevScalars>(plan, p.off_scalars);
  if (first) {
    L.sv = *first;
    L.sc_out = at<muon::DevScalars>(plan, p.off_scalars);
  }
  L.err = plan->err_word;
  L.items = p.skinny_items;
  L.slices = p.skinny_slices;
  L.m_max = p.skinny_m_max;
  L.bf16 = p.mode == MUON_MODE_BF16_MFMA;
  L.nesterov = p.nesterov;
  hipError_t e;
  if ((e = timed(plan, muon::kClsSkinnyGram, s, timing, [&] { return muon::launch_skinny_gram(L, s); })) != hipSuccess)
    return e;
  L.sc_out = nullptr;  // the scalar block is filled from here on
  if ((e = timed(plan, muon::kClsSkinnyPoly, s, timing, [&] { return muon::launch_skinny_poly(L, s); })) != hipSuccess)
    return e;
  return timed(plan, muon::kClsSkinnyApply, s, timing, [&] { return muon::launch_skinny_apply(L, s); });
}

// Newton-Schulz rounds of a group of streamed buckets (the small ones, or
// the others that do not take the large tiles): one launch per product
// phase and round over all of them.
hipError_t enqueue_group_rounds(muon_plan_t plan, bool small, int ns, hipStream_t s, bool timing) {
  const muon::Plan& p = plan->p;
  muon::SmallArgs g{};
  g.buckets = at<muon::SmallBucket>(plan, small ? p.off_small_params : p.off_mid_params);
  g.nb = (int)(small ? p.small.size() : p.mid.size());
  g.sc = at<muon::DevScalars>(plan, p.off_scalars);
  g.ptrs = at<muon::PtrEntry>(plan, p.off_ptrs);
  const bool f32 = p.mode == MUON_MODE_FP32;
  auto launch = [&](int ph, bool final_round) {
    return small ? muon::launch_small(ph, final_round, f32, g, p.small_wgs[ph], s)
                 : muon::launch_mid(ph, final_round, f32, g, p.mid_wgs[ph], p.mid_bt[ph], s);
  };
  hipError_t e;
  for (int it = 0; it < ns; ++it) {
    g.src = it & 1;
    g.first = it == 0;
    if ((e = timed(plan, muon::kClsGram, s, timing, [&] { return launch(0, false); })) != hipSuccess) return e;
    if ((e = timed(plan, muon::kClsPoly, s, timing, [&] { return launch(1, false); })) != hipSuccess) return e;
    if ((e = timed(plan, muon::kClsApply, s, timing, [&] { return launch(2, it == ns - 1); })) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

// Newton-Schulz rounds of all large bf16 buckets: one launch per product
// phase and round, each walking its tile table across the buckets.
hipError_t enqueue_big_rounds(muon_plan_t plan, int ns, hipStream_t s, bool timing) {
  const muon::Plan& p = plan->p;
  muon::BigArgs g{};
  g.buckets = at<muon::BigBucket>(plan, p.off_big_params);
  g.sc = at<muon::DevScalars>(plan, p.off_scalars);
  g.ptrs = at<muon::PtrEntry>(plan, p.off_ptrs);
  hipError_t e;
  for (int it = 0; it < ns; ++it) {
    g.src = it & 1;
    g.first = it == 0;
    g.tiles = at<muon::BigTile>(plan, p.off_big_tab[0]);
    g.t8 = (int)p.big_tab[0].size();
    if ((e = timed(plan, muon::kClsGram, s, timing, [&] { return muon::launch_big(muon::kBigGram, g, s); })) != hipSuccess)
      return e;
    g.tiles = at<muon::BigTile>(plan, p.off_big_tab[1]);
    g.t8 = (int)p.big_tab[1].size();
    if ((e = timed(plan, muon::kClsPoly, s, timing, [&] { return muon::launch_big(muon::kBigPoly, g, s); })) != hipSuccess)
      return e;
    g.tiles = at<muon::BigTile>(plan, p.off_big_tab[2]);
    g.t8 = (int)p.big_tab[2].size();
    const muon::BigKind k = it == ns - 1 ? muon::kBigFinal : muon::kBigApply;
    if ((e = timed(plan, muon::kClsApply, s, timing, [&] { return muon::launch_big(k, g, s); })) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

hipError_t enqueue_stream(muon_plan_t plan, const muon::BucketPlan& bp, int ns, hipStream_t s,
                          bool timing, const muon::DevScalars* first) {
  const muon::Plan& p = plan->p;
  const int cnt = (int)bp.slices.size();
  const muon::DevMat* mats = at<muon::DevMat>(plan, bp.off_mats);
  const muon::PtrEntry* ptrs = at<muon::PtrEntry>(plan, p.off_ptrs);
  const muon::DevScalars* sc = at<muon::DevScalars>(plan, p.off_scalars);
  float* scale = at<float>(plan, bp.off_scale);
  hipError_t e;

  muon::MomentumLaunch mo{};
  mo.mats = mats;
  mo.ptrs = ptrs;
  mo.sc = sc;
  if (first) {
    mo.sv = *first;
    mo.sc_out = const_cast<muon::DevScalars*>(sc);
  }
  mo.x = plan->ws + bp.off_x[0];
  mo.xt = plan->ws + bp.off_xt[0];
  mo.sq = at<float>(plan, bp.off_sq);
  mo.m = bp.m;
  mo.n = bp.n;
  mo.mp = bp.mp;
  mo.np = bp.np;
  mo.count = cnt;
  mo.km_tiles = bp.km_tiles;
  mo.x_bytes = bp.x_bytes;
  if ((e = timed(plan, muon::kClsMomentum, s, timing, [&] { return muon::launch_momentum(mo, s); })) != hipSuccess)
    return e;
  muon::NormLaunch no{at<float>(plan, bp.off_sq), scale, sc, plan->err_word, cnt, bp.km_tiles};
  if ((e = timed(plan, muon::kClsNorm, s, timing, [&] { return muon::launch_norm(no, s); })) != hipSuccess)
    return e;
  if (ns == 0) {
    muon::Update0Launch u{mats, ptrs, sc, scale, bp.m, bp.n, cnt};
    return timed(plan, muon::kClsUpdate, s, timing, [&] { return muon::launch_update0(u, s); });
  }
  return hipSuccess;  // the rounds run grouped over the buckets (small, other, large)
}

// Every bucket's launches, in plan order.  The number of Newton-Schulz
// rounds is read by the skinny kernels from the scalar block and fixes the
// streamed launch sequence.
// `first`: the step's scalars, to be written by the first kernel (eager
// steps), or null when a prologue kernel has already written them.
hipError_t enqueue_buckets(muon_plan_t plan, int ns, hipStream_t s, bool timing,
                           const muon::DevScalars* first) {
  if (!plan->p.skinny.empty()) {
    hipError_t e = enqueue_skinny(plan, s, timing, first);
    if (e != hipSuccess) return e;
    first = nullptr;
  }
  for (const muon::BucketPlan& bp : plan->p.buckets) {
    if (bp.path == MUON_PATH_SKINNY) continue;
    hipError_t e = enqueue_stream(plan, bp, ns, s, timing, first);
    if (e != hipSuccess) return e;
    first = nullptr;
  }
  if (!plan->p.small.empty() && ns > 0) {
    hipError_t e = enqueue_group_rounds(plan, true, ns, s, timing);
    if (e != hipSuccess) return e;
  }
  if (!plan->p.mid.empty() && ns > 0) {
    hipError_t e = enqueue_group_rounds(plan, false, ns, s, timing);
    if (e != hipSuccess) return e;
  }
  if (!plan->p.big.empty() && ns > 0) return enqueue_big_rounds(plan, ns, s, timing);
  return hipSuccess;
}

// Checks of muon_step's arguments that need no device: pointers (non-null,
// 16-byte aligned), ns_steps range, finite scalars.
int check_step_args(const muon::Plan& p, void* const* params, const void* const* grads, void* const* momentum,
                    float lr, float beta, int32_t ns_steps, float a, float b, float c) {
  if (!params || !grads || !momentum) return fail(MUON_ERR_INVALID_ARGUMENT, "null pointer array");
  for (int i = 0; i < p.n_params; ++i) {
    const void* ptr3[3] = {params[i], grads[i], momentum[i]};
    const char* names[3] = {"params", "grads", "momentum"};
    for (int k = 0; k < 3; ++k) {
      if (ptr3[k] == nullptr) return fail(MUON_ERR_INVALID_ARGUMENT, "%s[%d] is null", names[k], i);
      if ((reinterpret_cast<uintptr_t>(ptr3[k]) & 15) != 0)
        return fail(MUON_ERR_INVALID_ARGUMENT, "%s[%d] is not 16-byte aligned", names[k], i);
    }
  }
  if (ns_steps < 0 || ns_steps > p.max_ns_steps)
    return fail(MUON_ERR_INVALID_ARGUMENT, "ns_steps %d outside [0, %d]", ns_steps, p.max_ns_steps);
  const float sc5[5] = {lr, beta, a, b, c};
  const char* sn[5] = {"lr", "beta", "a", "b", "c"};
  for (int k = 0; k < 5; ++k)
    if (!std::isfinite(sc5[k])) return fail(MUON_ERR_INVALID_ARGUMENT, "%s is not finite", sn[k]);
  return MUON_OK;
}

muon::DevScalars step_scalars(const muon::Plan& p, float lr, float beta, int32_t ns_steps, float a, float b,
                              float c) {
  muon::DevScalars v;
  v.lr = lr;
  v.beta = beta;
  v.a = a;
  v.b = b;
  v.c = c;
  v.eps = p.eps;
  v.decay = lr * p.weight_decay;
  v.ns_steps = ns_steps;
  v.nesterov = p.nesterov;
  v.scale_mode = p.update_scale;
  return v;
}

// Mark the end of the step just enqueued on s.
int record_step(muon_plan_t plan, hipStream_t s) {
  const hipError_t e = hipEventRecord(plan->step_done, s);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  plan->step_stream = s;
  plan->step_recorded = true;
  return MUON_OK;
}

// Wait for the plan's last step (not for other work on the device).
hipError_t wait_plan(muon_plan_t plan) {
  return plan->step_recorded ? hipEventSynchronize(plan->step_done) : hipSuccess;
}

void drop_graph(muon_plan_t plan) {
  if (plan->gexec) hipGraphExecDestroy(plan->gexec);
  plan->gexec = nullptr;
  plan->graph_ns = -1;
  plan->graph_stream = nullptr;
}

}  // namespace

extern "C" {

void muon_default_opts(muon_plan_opts_t* opts) {
  if (opts) muon::default_opts(opts);
}

const char* muon_last_error(void) { return g_last_error.c_str(); }

int muon_plan_describe(const muon_param_desc_t* descs, int32_t n_params, const muon_plan_opts_t* opts,
                       muon_plan_info_t* info) {
  if (info == nullptr) return fail(MUON_ERR_INVALID_ARGUMENT, "info is null");
  const int n_cu = (opts && opts->n_cu > 0) ? opts->n_cu : 256;
  muon::Plan p;
  std::string err;
  const int rc = muon::make_plan(descs, n_params, opts, n_cu, &p, &err);
  if (rc != MUON_OK) return fail(rc, "%s", err.c_str());
  muon::fill_info(p, info);
  g_last_error.clear();
  return MUON_OK;
}

int muon_plan_create(const muon_param_desc_t* descs, int32_t n_params, const muon_plan_opts_t* opts,
                     muon_plan_t* out_plan) {
  if (out_plan == nullptr) return fail(MUON_ERR_INVALID_ARGUMENT, "out_plan is null");
  *out_plan = nullptr;
  // Validate the request before touching the device.
  {
    muon::Plan probe;
    std::string err;
    const int rc = muon::make_plan(descs, n_params, opts, 256, &probe, &err);
    if (rc != MUON_OK && rc != MUON_ERR_OOM) return fail(rc, "%s", err.c_str());
  }
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  if (opts && opts->n_cu > 0 && opts->n_cu < n_cu) n_cu = opts->n_cu;

  muon_plan* plan = new (std::nothrow) muon_plan;
  if (!plan) return fail(MUON_ERR_OOM, "host allocation failed");
  plan->device = dev;
  std::string err;
  int rc = muon::make_plan(descs, n_params, opts, n_cu, &plan->p, &err);
  if (rc != MUON_OK) {
    delete plan;
    return fail(rc, "%s", err.c_str());
  }
  const muon::Plan& p = plan->p;
  e = hipMalloc(&plan->ws, p.ws_total);
  if (e != hipSuccess) {
    hipGetLastError();
    delete plan;
    return fail(MUON_ERR_OOM, "workspace of %llu bytes: %s", (unsigned long long)p.ws_total,
                hipGetErrorString(e));
  }
  plan->err_word = at<uint32_t>(plan, p.off_err);
  // Zero once: padding of the streamed workspace must stay exactly zero.
  e = hipMemset(plan->ws, 0, p.ws_total);
  std::vector<Upload> ups;
  if (e == hipSuccess && !device_tables(plan, &ups)) e = hipErrorOutOfMemory;
  for (const Upload& u : ups) {
    if (e != hipSuccess) break;
    e = hipMemcpy(plan->ws + u.off, u.bytes.data(), u.bytes.size(), hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&plan->pinned),
                                         sizeof(muon::PtrEntry) * p.n_params, hipHostMallocDefault);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&plan->upload_done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&plan->step_done, hipEventDisableTiming);
  if (e == hipSuccess) {
    try {
      plan->ptrs.resize(p.n_params);
    } catch (const std::bad_alloc&) {
      e = hipErrorOutOfMemory;
    }
  }
  if (e != hipSuccess) {
    muon_plan_destroy(plan);
    return hip_fail(e, "plan setup");
  }
  *out_plan = plan;
  g_last_error.clear();
  return MUON_OK;
}

int muon_plan_query(muon_plan_t plan, muon_plan_info_t* info) {
  if (!plan_ok(plan)) return fail(MUON_ERR_INVALID_ARGUMENT, "invalid plan handle");
  if (!info) return fail(MUON_ERR_INVALID_ARGUMENT, "info is null");
  muon::fill_info(plan->p, info);
  return MUON_OK;
}

int muon_step(muon_plan_t plan, void* const* params, const void* const* grads, void* const* momentum,
              float lr, float beta, int32_t ns_steps, float a, float b, float c, void* stream) {
  if (!plan_ok(plan)) return fail(MUON_ERR_INVALID_ARGUMENT, "invalid plan handle");
  const muon::Plan& p = plan->p;
  const int bad = check_step_args(p, params, grads, momentum, lr, beta, ns_steps, a, b, c);
  if (bad != MUON_OK) return bad;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(MUON_ERR_DEVICE_MISMATCH, "plan lives on device %d, current device is %d", plan->device, dev);
  hipStream_t s = static_cast<hipStream_t>(stream);

  // A step enqueued on another stream than the previous one waits for it:
  // both use the plan's workspace.
  if (plan->step_recorded && s != plan->step_stream) {
    e = hipStreamWaitEvent(s, plan->step_done, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }

  // Pointer table: upload only when it changed (compared in place, so a step
  // allocates no host memory).
  bool same = plan->ptrs_valid;
  for (int i = 0; same && i < p.n_params; ++i) {
    const muon::PtrEntry& o = plan->ptrs[i];
    same = o.w == params[i] && o.g == grads[i] && o.m == momentum[i];
  }
  if (!same) {
    if (plan->upload_pending) {
      e = hipEventSynchronize(plan->upload_done);  // the staging buffer is still being read
      if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    }
    for (int i = 0; i < p.n_params; ++i) {
      muon::PtrEntry& o = plan->ptrs[i];
      o.w = params[i];
      o.g = grads[i];
      o.m = static_cast<float*>(momentum[i]);
      plan->pinned[i] = o;
    }
    e = hipMemcpyAsync(plan->ws + p.off_ptrs, plan->pinned, sizeof(muon::PtrEntry) * p.n_params,
                       hipMemcpyHostToDevice, s);
    if (e != hipSuccess) {
      plan->ptrs_valid = false;
      return hip_fail(e, "pointer table upload");
    }
    e = hipEventRecord(plan->upload_done, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    plan->upload_pending = true;
    plan->ptrs_valid = true;
  }

  const muon::DevScalars v = step_scalars(p, lr, beta, ns_steps, a, b, c);
  const bool timing = p.timing != 0;
  const bool graph = p.use_graph && !timing && s != nullptr;
  if (!graph) {
    // Eager: the first kernel writes the scalar block itself.
    e = enqueue_buckets(plan, ns_steps, s, timing, &v);
    if (e != hipSuccess) return hip_fail(e, "launch");
    return record_step(plan, s);
  }
  // Graph replay: kernel arguments are frozen in the graph, so a prologue
  // outside it writes this step's scalars first.
  e = muon::launch_prologue(at<muon::DevScalars>(plan, p.off_scalars), v, s);
  if (e != hipSuccess) return hip_fail(e, "prologue launch");
  if (plan->gexec == nullptr || plan->graph_ns != ns_steps || plan->graph_stream != s) {
    drop_graph(plan);
    e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
    hipError_t le = enqueue_buckets(plan, ns_steps, s, false, nullptr);
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(s, &g);
    if (le != hipSuccess) {
      if (g) hipGraphDestroy(g);
      return hip_fail(le, "launch during capture");
    }
    if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
    e = hipGraphInstantiate(&plan->gexec, g, nullptr, nullptr, 0);
    hipGraphDestroy(g);
    if (e != hipSuccess) {
      plan->gexec = nullptr;
      return hip_fail(e, "hipGraphInstantiate");
    }
    plan->graph_ns = ns_steps;
    plan->graph_stream = s;
  }
  e = hipGraphLaunch(plan->gexec, s);
  if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  return record_step(plan, s);
}

int muon_step_noalloc(const muon_param_desc_t* descs, int32_t n_params, const muon_plan_opts_t* opts,
                      void* const* params, const void* const* grads, void* const* momentum, float lr,
                      float beta, int32_t ns_steps, float a, float b, float c, uint32_t* device_error,
                      void* stream) {
  if (opts && (opts->use_graph || opts->timing))
    return fail(MUON_ERR_INVALID_ARGUMENT, "muon_step_noalloc takes neither use_graph nor timing");
  // The plan lives on this stack frame; its workspace is the fixed scratch.
  muon_plan plan;
  std::string err;
  int rc;
  try {
    rc = muon::make_plan(descs, n_params, opts, 256, &plan.p, &err);
  } catch (const std::bad_alloc&) {
    return fail(MUON_ERR_OOM, "host memory for the plan");
  }
  if (rc != MUON_OK) return fail(rc, "%s", err.c_str());
  const muon::Plan& p = plan.p;
  if (p.ws_total > muon::kScratchBytes)
    return fail(MUON_ERR_UNSUPPORTED,
                "muon_step_noalloc: these parameters need %llu bytes of scratch, the fixed array holds %llu "
                "(use a plan)",
                (unsigned long long)p.ws_total, (unsigned long long)muon::kScratchBytes);
  if ((reinterpret_cast<uintptr_t>(device_error) & 3) != 0)
    return fail(MUON_ERR_INVALID_ARGUMENT, "device_error is not 4-byte aligned");
  const int bad = check_step_args(p, params, grads, momentum, lr, beta, ns_steps, a, b, c);
  if (bad != MUON_OK) return bad;

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  e = muon::scratch_address(dev, &plan.ws);
  if (e != hipSuccess) return hip_fail(e, "address of the fixed scratch");
  plan.device = dev;
  plan.err_word = device_error ? device_error : at<uint32_t>(&plan, p.off_err);
  hipStream_t s = static_cast<hipStream_t>(stream);

  // The tables this step's kernels read, built on the host with the
  // scratch's addresses; the pointer table last.
  std::vector<Upload> ups;
  if (!device_tables(&plan, &ups)) return fail(MUON_ERR_OOM, "host memory for the tables");
  try {
    std::vector<muon::PtrEntry> ptrs(p.n_params);
    for (int i = 0; i < p.n_params; ++i) {
      ptrs[i].w = params[i];
      ptrs[i].g = grads[i];
      ptrs[i].m = static_cast<float*>(momentum[i]);
    }
    add_upload(&ups, p.off_ptrs, ptrs);
  } catch (const std::bad_alloc&) {
    return fail(MUON_ERR_OOM, "host memory for the tables");
  }
  // The scratch keeps whatever the last call on this device left: clear the
  // part this step uses (the streamed path relies on zero padding, the
  // error word starts at zero), then write the tables.  The copies read
  // pageable host memory, which the runtime consumes before returning.
  e = muon::launch_fill_zero(plan.ws, p.ws_total, s);
  if (e != hipSuccess) return hip_fail(e, "clearing the scratch");
  for (const Upload& u : ups) {
    e = hipMemcpyAsync(plan.ws + u.off, u.bytes.data(), u.bytes.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "table upload");
  }
  const muon::DevScalars v = step_scalars(p, lr, beta, ns_steps, a, b, c);
  e = enqueue_buckets(&plan, ns_steps, s, false, &v);
  if (e != hipSuccess) return hip_fail(e, "launch");
  g_last_error.clear();
  return MUON_OK;
}

int muon_plan_status(muon_plan_t plan, uint32_t* device_error) {
  if (!plan_ok(plan)) return fail(MUON_ERR_INVALID_ARGUMENT, "invalid plan handle");
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess && cur != plan->device) e = hipSetDevice(plan->device);
  if (e == hipSuccess) e = wait_plan(plan);
  if (e != hipSuccess) return hip_fail(e, "waiting for the plan's last step");
  // Blocking copies: the word is read after the step, and cleared before
  // this call returns.
  uint32_t word = 0;
  const uint32_t zero = 0;
  e = hipMemcpy(&word, plan->ws + plan->p.off_err, sizeof word, hipMemcpyDeviceToHost);
  if (e == hipSuccess && word != 0)
    e = hipMemcpy(plan->ws + plan->p.off_err, &zero, sizeof zero, hipMemcpyHostToDevice);
  if (cur >= 0 && cur != plan->device) hipSetDevice(cur);
  if (e != hipSuccess) return hip_fail(e, "reading the device error word");
  if (device_error) *device_error = word;
  if (word != 0) return fail(MUON_ERR_DEVICE, "device error word 0x%x (bit 0: non-finite momentum norm)", word);
  return MUON_OK;
}

int muon_plan_timings(muon_plan_t plan, double* out_ms, int64_t* out_count, int32_t n_out) {
  if (!plan_ok(plan)) return fail(MUON_ERR_INVALID_ARGUMENT, "invalid plan handle");
  for (TimedLaunch& t : plan->timed) {
    hipError_t e = hipEventSynchronize(t.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    hipEventElapsedTime(&ms, t.start, t.stop);
    plan->acc_ms[t.cls] += ms;
    plan->acc_cnt[t.cls] += 1;
    plan->event_pool.push_back(t.start);
    plan->event_pool.push_back(t.stop);
  }
  plan->timed.clear();
  for (int i = 0; i < n_out && i < muon::kNumClasses; ++i) {
    if (out_ms) out_ms[i] = plan->acc_ms[i];
    if (out_count) out_count[i] = plan->acc_cnt[i];
    plan->acc_ms[i] = 0.0;
    plan->acc_cnt[i] = 0;
  }
  return muon::kNumClasses;
}

int muon_plan_destroy(muon_plan_t plan) {
  if (plan == nullptr) return MUON_OK;
  if (!plan_ok(plan)) return fail(MUON_ERR_INVALID_ARGUMENT, "invalid plan handle");
  int cur = -1;
  hipGetDevice(&cur);
  if (cur != plan->device) hipSetDevice(plan->device);
  wait_plan(plan);  // the plan's last step (its timing events and uploads precede it)
  if (plan->upload_pending) hipEventSynchronize(plan->upload_done);
  drop_graph(plan);
  for (TimedLaunch& t : plan->timed) {
    hipEventDestroy(t.start);
    hipEventDestroy(t.stop);
  }
  for (hipEvent_t ev : plan->event_pool) hipEventDestroy(ev);
  if (plan->upload_done) hipEventDestroy(plan->upload_done);
  if (plan->step_done) hipEventDestroy(plan->step_done);
  if (plan->pinned) hipHostFree(plan->pinned);
  if (plan->ws) hipFree(plan->ws);
  if (cur >= 0 && cur != plan->device) hipSetDevice(cur);
  plan->magic = 0;
  delete plan;
  return MUON_OK;
}

}  // extern "C"
