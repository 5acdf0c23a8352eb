// The C ABI of liblq (declared in include/lq.h): argument validation,
// workspace carving and dispatch to the HIP launchers. Every check runs on the
// host before anything is enqueued, so a rejected call launches nothing.
#include "lq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cmath>
#include <mutex>
#include <vector>

#include "lq_internal.h"

namespace lq {
LaunchEvents& launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}
}  // namespace lq

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = INT32_MAX;          // N, K, B each
constexpr int64_t kMaxBatch = 1 << 20;
constexpr int64_t kMaxElems = int64_t(1) << 40;  // B*K, B*L, N*L

lq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return LQ_OK;
  g_last_hip_error = (int)e;
  return LQ_ERR_HIP;
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool valid_dtype(lq_dtype t) { return t == LQ_F32 || t == LQ_BF16; }
size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

bool mul_ok(int64_t a, int64_t b, int64_t lim) { return a == 0 || b <= lim / a; }

// Checks shared by every entry point that takes (N, K, d, D); writes L.
lq_status check_layer_dims(int64_t N, int64_t K, int32_t d, int32_t D, int64_t* L) {
  if (N < 0 || K < 1 || d < 1 || D < d) return LQ_ERR_INVALID_ARG;
  if (D > LQ_MAX_D || N > kMaxDim || K > kMaxDim) return LQ_ERR_UNSUPPORTED;
  const int64_t Kb = (K + d - 1) / d;
  *L = Kb * D;
  // (L <= LQ_MAX_L keeps every byte offset within a panel, 2 L, in 32 bits)
  if (N % lq::kPanelRows != 0 || *L % 8 != 0 || *L > LQ_MAX_L) return LQ_ERR_UNSUPPORTED;
  if (!mul_ok(N, *L, kMaxElems * 64)) return LQ_ERR_UNSUPPORTED;
  return LQ_OK;
}

lq_status check_sign_dims(int64_t B, int64_t N, int64_t L) {
  if (B < 0 || N < 0 || L < 1) return LQ_ERR_INVALID_ARG;
  if (B > kMaxBatch || N > kMaxDim || L > LQ_MAX_L) return LQ_ERR_UNSUPPORTED;
  if (N % lq::kPanelRows != 0 || L % 8 != 0) return LQ_ERR_UNSUPPORTED;
  if (!mul_ok(B, L, kMaxElems) || !mul_ok(B, N, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  return LQ_OK;
}

// Event ring of lq_profile_events.
struct ProfileRing {
  std::mutex mu;
  std::vector<hipEvent_t> starts, stops;
  size_t next = 0;
};
ProfileRing& profile_ring() {
  static ProfileRing ring;
  return ring;
}

// Launch `fn` (which enqueues one sign-product kernel) with the ring's next
// event pair pending: the kernel's dispatch records them at its start and end.
template <typename Fn>
hipError_t profiled(hipStream_t stream, Fn fn) {
  (void)stream;
  ProfileRing& ring = profile_ring();
  std::unique_lock<std::mutex> lock(ring.mu);
  if (ring.starts.empty()) {
    lock.unlock();
    return fn();
  }
  const size_t i = ring.next;
  ring.next = (ring.next + 1) % ring.starts.size();
  lq::LaunchEvents& ev = lq::launch_events();
  ev.start = ring.starts[i];
  ev.stop = ring.stops[i];
  const hipError_t e = fn();
  ev = lq::LaunchEvents{};
  return e;
}


static_assert(lq::kControlBytes == LQ_WS_CONTROL_BYTES, "control area size");
static_assert(lq::kFusedErrorWord == LQ_WS_ERROR_WORD, "error word");
static_assert(lq::kMultiMax == LQ_MULTI_MAX, "layers per grouped call");

// Compute units of the current device (0 when there is none), cached.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const bool cached = dev >= 0 && dev < 64;
  if (cached) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (cached) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool valid_algo(lq_algo algo, bool linear) {
  return algo >= LQ_ALGO_AUTO && algo <= (linear ? LQ_ALGO_FUSED_SPLIT : LQ_ALGO_MFMA_LARGE);
}

// Everything one sign product (or one whole lq_linear) needs: algorithm,
// geometry, plans and the byte offsets of its pieces in the workspace.
struct Exec {
  lq_algo algo;
  lq::PackedGeom g;
  lq::ValuPlan vp;
  lq::Fp6Plan fp;
  lq::OperandShape os;
  lq::FusedPlan fu;
  lq::SelfPlan sp;
  lq::SplitPlan spl;
  int tickets;
  size_t off_tickets, off_aop, off_partial, off_zf32, off_xt, off_zp, off_tslots, total;
  int d, D;
  lq_dtype ztype;
};

// Plans a sign product of z (ztype) or, when `linear`, the whole operator
// for activations of type ztype with K input features.
// Every workspace that is used at all starts with the control area of the
// one-launch decode (only that kernel writes it), so one workspace can serve
// calls of every algorithm in turn.
lq_status plan_exec(int64_t B, int64_t N, int64_t L, int64_t K, int d, int D, lq_dtype ztype,
                    lq_algo algo, bool linear, Exec* e) {
  e->g = lq::make_geom(N, L);
  e->algo = algo;
  e->d = d;
  e->D = D;
  e->ztype = ztype;
  if (algo == LQ_ALGO_AUTO) {
    if (B > 16) {
      // W space where it applies: D / d times fewer MACs on the same bf16
      // operands (bf16 x: the lifted product would round z to bf16 too).
      e->algo = linear && ztype == LQ_BF16 && lq::wspace_supported(d, D) ? LQ_ALGO_WSPACE
                                                                          : LQ_ALGO_MFMA_LARGE;
    } else if (ztype == LQ_F32) {
      e->algo = LQ_ALGO_VALU;
    } else {
      // The one-launch decode is correct but, as measured so far, slower
      // than the preparation launch plus the product launch: its chain of
      // dependent memory round trips (load x, publish, poll, copy the
      // operand) outweighs the launch it saves. It is chosen explicitly.
      e->algo = LQ_ALGO_MFMA_SMALL;
    }
  }
  e->tickets = 0;
  e->off_tickets = e->off_aop = e->off_partial = 0;
  e->off_zf32 = e->off_xt = e->off_zp = e->off_tslots = 0;
  const size_t ctl = align_up(lq::kControlBytes);
  size_t at = ctl;
  auto take = [&](size_t bytes) { const size_t o = at; at += align_up(bytes); return o; };
  switch (e->algo) {
    case LQ_ALGO_VALU:
      if (B > 16 && linear) return LQ_ERR_UNSUPPORTED;
      e->vp = lq::plan_valu(B, e->g);
      e->tickets = e->vp.ksplit > 1 ? e->vp.groups : 0;
      e->off_tickets = take((size_t)e->tickets * 4);
      e->off_partial = take(e->vp.partial_bytes);
      if (linear) e->off_zf32 = take((size_t)B * L * sizeof(float));
      break;
    case LQ_ALGO_MFMA_SMALL:
      if (B > 16) return LQ_ERR_UNSUPPORTED;
      e->os = lq::operand_shape(B, ztype == LQ_BF16);
      e->fp = lq::plan_fp6(B, e->g, e->os, device_cus());
      e->off_aop = take(lq::operand_bytes(L, e->os));
      break;
    case LQ_ALGO_FUSED:
      if (!linear) return LQ_ERR_INVALID_ARG;
      if (B > 16) return LQ_ERR_UNSUPPORTED;
      e->os = lq::operand_shape(B, ztype == LQ_BF16);
      e->fu = lq::plan_fused(B, e->g, e->os, device_cus());
      if (!e->fu.ok) return LQ_ERR_UNSUPPORTED;
      e->off_aop = take(lq::operand_bytes(L, e->os));
      break;
    case LQ_ALGO_FUSED_LOCAL:
      if (!linear) return LQ_ERR_INVALID_ARG;
      e->os = lq::operand_shape(B, ztype == LQ_BF16);
      e->sp = lq::plan_self(B, K, d, D, e->g, e->os);
      if (!e->sp.ok) return LQ_ERR_UNSUPPORTED;
      break;
    case LQ_ALGO_FUSED_SPLIT:
      if (!linear) return LQ_ERR_INVALID_ARG;
      e->os = lq::operand_shape(B, ztype == LQ_BF16);
      e->spl = lq::plan_split(B, K, d, D, e->g, e->os, device_cus());
      if (!e->spl.ok) return LQ_ERR_UNSUPPORTED;
      e->off_partial = take(e->spl.partial_bytes);
      break;
    case LQ_ALGO_MFMA_LARGE:
      if (linear) e->off_xt = take((size_t)B * K * sizeof(float));
      {
        const lq::ZpGeom zg = lq::zp_geom(B, e->g, ztype == LQ_BF16);
        e->off_zp = take(zg.bytes);
        e->off_tslots = take(zg.tail_bytes);
        e->off_partial = take(lq::plan_large(B, e->g, ztype == LQ_BF16).partial_bytes);
      }
      break;
    case LQ_ALGO_WSPACE:
      if (!linear) return LQ_ERR_INVALID_ARG;
      if (ztype != LQ_BF16 || !lq::wspace_supported(d, D)) return LQ_ERR_UNSUPPORTED;
      {
        const lq::XpGeom xg = lq::xp_geom(B, e->g, d, D);
        e->off_zp = take(xg.bytes);
        e->off_tslots = take(xg.tail_bytes);
      }
      break;
    default:
      return LQ_ERR_INVALID_ARG;
  }
  e->total = at == ctl ? 0 : at;
  return LQ_OK;
}

// Sign product of a prepared input. `zin` is z (sign_gemm) or the raw
// activations x (linear, whitened and lifted by the preparation launch).
lq_status run_exec(const Exec& e, const uint8_t* packed, const void* zin, lq_dtype ztype,
                   int64_t B, int64_t N, int64_t L, const float* row_scale, void* y,
                   lq_dtype ytype, void* ws, hipStream_t st, const lq_layer* layer) {
  (void)N;   // carried by e.g
  char* base = static_cast<char*>(ws);
  const bool zb = ztype == LQ_BF16, yb = ytype == LQ_BF16;
  unsigned* tickets = reinterpret_cast<unsigned*>(base + e.off_tickets);
  float* partial = reinterpret_cast<float*>(base + e.off_partial);
  lq_status s = LQ_OK;
  switch (e.algo) {
    case LQ_ALGO_VALU: {
      const void* z = zin;
      bool z_bf16 = zb;
      if (layer) {
        float* zf = reinterpret_cast<float*>(base + e.off_zf32);
        s = hip_status(lq::launch_prep(zin, zb ? 1 : 0, B, layer->K, layer->d, layer->D, layer->hb,
                                       layer->c, layer->M, L, zf, nullptr, tickets, e.tickets, st));
        z = zf;
        z_bf16 = false;
      } else if (e.tickets > 0) {
        s = hip_status(lq::launch_zero_u32(tickets, e.tickets, st));
      }
      if (s != LQ_OK) return s;
      return hip_status(profiled(st, [&] {
        return lq::launch_sign_valu(packed, e.g, z, z_bf16, B, row_scale, y, yb, e.vp, partial,
                                    tickets, st);
      }));
    }
    case LQ_ALGO_MFMA_SMALL: {
      lq::OperandPlan op;
      op.s = e.os;
      op.aop = reinterpret_cast<uint8_t*>(base + e.off_aop);
      if (layer)
        s = hip_status(lq::launch_prep(zin, zb ? 1 : 0, B, layer->K, layer->d, layer->D, layer->hb,
                                       layer->c, layer->M, L, nullptr, &op, tickets, e.tickets, st));
      else
        s = hip_status(lq::launch_prep(zin, zb ? 3 : 2, B, 1, 1, 1, 1, nullptr, nullptr, L, nullptr,
                                       &op, tickets, e.tickets, st));
      if (s != LQ_OK) return s;
      return hip_status(profiled(st, [&] {
        return lq::launch_sign_fp6(packed, e.g, op, B, row_scale, y, yb, e.fp, st);
      }));
    }
    case LQ_ALGO_FUSED: {
      lq::OperandPlan op;
      op.s = e.os;
      op.aop = reinterpret_cast<uint8_t*>(base + e.off_aop);
      unsigned* ctl = reinterpret_cast<unsigned*>(base);
      return hip_status(profiled(st, [&] {
        return lq::launch_decode_fused(packed, e.g, zin, zb, B, layer->K, layer->d, layer->D,
                                       layer->hb, layer->c, layer->M, op, ctl, row_scale, y, yb,
                                       e.fu, st);
      }));
    }
    case LQ_ALGO_FUSED_LOCAL:
      return hip_status(profiled(st, [&] {
        return lq::launch_decode_self(packed, e.g, zin, zb, layer->K, layer->d, layer->D,
                                      layer->hb, layer->c, layer->M, e.os, row_scale, y, yb, e.sp,
                                      st);
      }));
    case LQ_ALGO_FUSED_SPLIT: {
      unsigned* tickets = reinterpret_cast<unsigned*>(base + lq::kFusedControlBytes);
      return hip_status(profiled(st, [&] {
        return lq::launch_decode_split(packed, e.g, zin, zb, layer->K, layer->d, layer->D,
                                       layer->hb, layer->c, layer->M, e.os, row_scale, y, yb,
                                       e.spl, partial, tickets, st);
      }));
    }
    case LQ_ALGO_MFMA_LARGE: {
      void* zp = base + e.off_zp;
      if (layer) {
        float* xt = reinterpret_cast<float*>(base + e.off_xt);
        s = hip_status(lq::launch_hadamard_scale(zin, zb, B, layer->K, layer->hb, layer->c, xt, st));
        if (s != LQ_OK) return s;
        s = hip_status(lq::launch_zp(xt, zb ? 3 : 2, B, L, layer->K, layer->d, layer->D, layer->M,
                                     e.g, zp, st));
      } else {
        s = hip_status(lq::launch_zp(zin, zb ? 1 : 0, B, L, 0, 1, 1, nullptr, e.g, zp, st));
      }
      if (s != LQ_OK) return s;
      return hip_status(profiled(st, [&] {
        return lq::launch_sign_mfma_large(packed, e.g, zp, base + e.off_tslots, zb, B, row_scale, y,
                                          yb, reinterpret_cast<float*>(base + e.off_partial), st);
      }));
    }
    case LQ_ALGO_WSPACE: {
      void* xp = base + e.off_zp;
      s = hip_status(lq::launch_xpw(zin, zb, B, layer->K, layer->hb, layer->c, e.d, e.D, e.g, xp, st));
      if (s != LQ_OK) return s;
      return hip_status(profiled(st, [&] {
        return lq::launch_wspace(packed, e.g, xp, base + e.off_tslots, B, layer->M, e.d, e.D,
                                 row_scale, y, yb, st);
      }));
    }
    default:
      return LQ_ERR_INVALID_ARG;
  }
}

// The launch shape of a planned call's sign-product kernel.
void fill_plan_info(const Exec& e, int64_t B, lq_plan_info* info) {
  const int64_t panels = e.g.panels;
  const int64_t B16 = (B + 15) / 16;
  lq_plan_info p{};
  p.algo = e.algo;
  p.ksplit = 1;
  p.batch_rows = (int32_t)B;
  switch (e.algo) {
    case LQ_ALGO_VALU:
      p.waves = lq::kValuWaves;
      p.panels = lq::kValuWaves;
      p.batch_rows = e.vp.bt;
      p.ksplit = e.vp.ksplit;
      p.workgroups = (int32_t)(((panels + 3) / 4) * e.vp.ksplit * ((B + e.vp.bt - 1) / e.vp.bt));
      break;
    case LQ_ALGO_MFMA_SMALL:
      p.waves = e.fp.chunked ? e.fp.w + lq::kChunkLoaders : e.fp.w;
      p.panels = e.fp.p;
      p.workgroups = e.fp.groups;
      break;
    case LQ_ALGO_FUSED:
      p.waves = lq::kOneLaunchWaves;
      p.panels = e.fu.p;
      p.workgroups = e.fu.groups;
      break;
    case LQ_ALGO_FUSED_LOCAL:
      p.waves = lq::kOneLaunchWaves;
      p.panels = e.sp.pw;
      p.workgroups = e.sp.groups;
      break;
    case LQ_ALGO_FUSED_SPLIT:
      p.waves = lq::kOneLaunchWaves;
      p.panels = lq::kSplitPanels;
      p.ksplit = e.spl.kgroups;
      p.workgroups = e.spl.kgroups * e.spl.pgroups;
      break;
    case LQ_ALGO_MFMA_LARGE: {
      const lq::LargePlan lp = lq::plan_large(B, e.g, e.ztype == LQ_BF16);
      p.waves = lq::kLargeWaves;
      p.panels = lq::kLargeWaves * lp.ppw;
      p.batch_rows = 16 * lp.jb;
      p.ksplit = lp.ksplit;
      p.workgroups = (int32_t)(((panels + p.panels - 1) / p.panels) * ((B16 + lp.jb - 1) / lp.jb) *
                               lp.ksplit);
      break;
    }
    case LQ_ALGO_WSPACE: {
      const int jb = lq::plan_wspace_jb(B, e.g, e.d);
      p.waves = lq::kLargeWaves;
      p.panels = lq::kLargeWaves * lq::kWsPanelsPerWave;
      p.batch_rows = 16 * jb;
      p.workgroups = (int32_t)(((panels + p.panels - 1) / p.panels) * ((B16 + jb - 1) / jb));
      break;
    }
    default:
      break;
  }
  *info = p;
}

lq_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return LQ_OK;
  if (ws == nullptr || ws_bytes < need) return LQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return LQ_ERR_INVALID_ARG;
  return LQ_OK;
}

lq_status check_layer(const lq_layer* layer, int64_t* L) {
  if (layer == nullptr || layer->reserved != 0) return LQ_ERR_INVALID_ARG;
  lq_status s = check_layer_dims(layer->N, layer->K, layer->d, layer->D, L);
  if (s != LQ_OK) return s;
  if (layer->hb < 1 || !is_pow2(layer->hb)) return LQ_ERR_INVALID_ARG;
  if (layer->hb > LQ_MAX_HB) return LQ_ERR_UNSUPPORTED;
  if (layer->K % layer->hb != 0) return LQ_ERR_INVALID_ARG;
  return LQ_OK;
}

// lq_linear_multi's plan: every layer checked and planned as lq_linear would;
// grouped (one preparation and one product launch) when every layer runs the
// small-batch matrix-core path with plans that can share one launch.
struct MultiPlan {
  int n;                    // layers with work (N > 0)
  int idx[LQ_MULTI_MAX];    // their indices
  Exec e[LQ_MULTI_MAX];
  int64_t L[LQ_MULTI_MAX];
  bool grouped;
  size_t off_aop[LQ_MULTI_MAX];
  size_t total;
};

lq_status plan_multi(const lq_layer* layers, int32_t n, int64_t B, lq_dtype xtype, MultiPlan* mp) {
  if (layers == nullptr || n < 1 || n > LQ_MULTI_MAX || !valid_dtype(xtype) || B < 0)
    return LQ_ERR_INVALID_ARG;
  mp->n = 0;
  mp->grouped = true;
  mp->total = 0;
  for (int i = 0; i < n; ++i) {
    int64_t L = 0;
    lq_status s = check_layer(&layers[i], &L);
    if (s != LQ_OK) return s;
    if (layers[i].K != layers[0].K) return LQ_ERR_INVALID_ARG;
    s = check_sign_dims(B, layers[i].N, L);
    if (s != LQ_OK) return s;
    if (!mul_ok(B, layers[i].K, kMaxElems)) return LQ_ERR_UNSUPPORTED;
    if (B == 0 || layers[i].N == 0) continue;
    const int j = mp->n++;
    mp->idx[j] = i;
    mp->L[j] = L;
    s = plan_exec(B, layers[i].N, L, layers[i].K, layers[i].d, layers[i].D, xtype, LQ_ALGO_AUTO,
                  true, &mp->e[j]);
    if (s != LQ_OK) return s;
    mp->total = std::max(mp->total, mp->e[j].total);
    if (mp->e[j].algo != LQ_ALGO_MFMA_SMALL || !lq::fp6_plans_match(mp->e[j].fp, mp->e[0].fp))
      mp->grouped = false;
  }
  if (mp->n < 2) mp->grouped = false;
  if (mp->grouped) {
    // one plan for all the layers' panels together (same kernel and panels
    // per workgroup), each layer's share under it
    lq::PackedGeom gs[LQ_MULTI_MAX];
    for (int j = 0; j < mp->n; ++j) gs[j] = mp->e[j].g;
    const lq::Fp6Plan group = lq::plan_fp6_group(B, gs, mp->n, mp->e[0].os, device_cus());
    for (int j = 0; j < mp->n; ++j) mp->e[j].fp = lq::plan_fp6_layer(group, mp->e[j].g, mp->e[j].os);
  }
  if (mp->grouped) {
    size_t at = align_up(lq::kControlBytes);
    for (int j = 0; j < mp->n; ++j) {
      mp->off_aop[j] = at;
      at += align_up(lq::operand_bytes(mp->L[j], mp->e[j].os));
    }
    mp->total = at;
  }
  return LQ_OK;
}

// Scratch of lq_linear_noalloc: a file-scope device array (one copy per GPU)
// whose device address is looked up once per device and kept. In host code
// `scratch` names only a host-side stand-in: kernels get the looked-up address.
static __device__ __align__(256) uint8_t scratch[LQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The current device's address of `scratch` (looked up on its first use on
// that device, with the device current).
lq_status noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return LQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess || p == nullptr) return hip_status(r != hipSuccess ? r : hipErrorInvalidSymbol);
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return LQ_OK;
}

}  // namespace

extern "C" {

int lq_version(void) { return 100; }

const char* lq_status_string(lq_status status) {
  switch (status) {
    case LQ_OK: return "LQ_OK";
    case LQ_ERR_INVALID_ARG: return "LQ_ERR_INVALID_ARG: invalid argument";
    case LQ_ERR_UNSUPPORTED: return "LQ_ERR_UNSUPPORTED: outside the library's limits";
    case LQ_ERR_WORKSPACE: return "LQ_ERR_WORKSPACE: workspace missing or too small";
    case LQ_ERR_HIP: return "LQ_ERR_HIP: HIP runtime error";
    case LQ_ERR_DEVICE: return "LQ_ERR_DEVICE: a kernel reported a failure; the call's output is wrong";
    default: return "unknown lq_status";
  }
}

int lq_last_hip_error(void) { return g_last_hip_error; }

lq_status lq_packed_size(int64_t N, int64_t K, int32_t d, int32_t D, size_t* bytes) {
  if (bytes == nullptr) return LQ_ERR_INVALID_ARG;
  int64_t L = 0;
  lq_status s = check_layer_dims(N, K, d, D, &L);
  if (s != LQ_OK) return s;
  *bytes = (size_t)(N * L / 8);
  return LQ_OK;
}

lq_status lq_pack_signs(const int8_t* signs, int64_t N, int64_t K, int32_t d, int32_t D,
                        uint8_t* packed, void* stream) {
  int64_t L = 0;
  lq_status s = check_layer_dims(N, K, d, D, &L);
  if (s != LQ_OK) return s;
  if (N == 0) return LQ_OK;
  if (!aligned16(signs) || !aligned16(packed)) return LQ_ERR_INVALID_ARG;
  return hip_status(lq::launch_pack(signs, N, L, packed, (hipStream_t)stream));
}

lq_status lq_unpack_signs(const uint8_t* packed, int64_t N, int64_t K, int32_t d, int32_t D,
                          int8_t* signs, void* stream) {
  int64_t L = 0;
  lq_status s = check_layer_dims(N, K, d, D, &L);
  if (s != LQ_OK) return s;
  if (N == 0) return LQ_OK;
  if (!aligned16(signs) || !aligned16(packed)) return LQ_ERR_INVALID_ARG;
  return hip_status(lq::launch_unpack(packed, N, L, signs, (hipStream_t)stream));
}

lq_status lq_hadamard_scale(const void* x, lq_dtype xtype, int64_t B, int64_t K, int32_t hb,
                            const float* c, float* xt, void* stream) {
  if (B < 0 || K < 1 || !valid_dtype(xtype)) return LQ_ERR_INVALID_ARG;
  if (hb < 1 || !is_pow2(hb)) return LQ_ERR_INVALID_ARG;
  if (hb > LQ_MAX_HB) return LQ_ERR_UNSUPPORTED;
  if (K % hb != 0) return LQ_ERR_INVALID_ARG;
  if (B > kMaxBatch || K > kMaxDim || !mul_ok(B, K, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  if (B == 0) return LQ_OK;
  if (!aligned16(x) || !aligned16(c) || !aligned16(xt)) return LQ_ERR_INVALID_ARG;
  return hip_status(lq::launch_hadamard_scale(x, xtype == LQ_BF16, B, K, hb, c, xt, (hipStream_t)stream));
}

lq_status lq_lift_activations(const float* xt, int64_t B, int64_t K, int32_t d, int32_t D,
                              const float* M, void* z, lq_dtype ztype, void* stream) {
  if (B < 0 || K < 1 || d < 1 || D < d || !valid_dtype(ztype)) return LQ_ERR_INVALID_ARG;
  if (D > LQ_MAX_D || B > kMaxBatch || K > kMaxDim) return LQ_ERR_UNSUPPORTED;
  const int64_t L = ((K + d - 1) / d) * D;
  if (!mul_ok(B, L, kMaxElems) || !mul_ok(B, K, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  if (B == 0) return LQ_OK;
  if (!aligned16(xt) || !aligned16(M) || !aligned16(z)) return LQ_ERR_INVALID_ARG;
  return hip_status(lq::launch_lift(xt, B, K, d, D, M, z, ztype == LQ_BF16, (hipStream_t)stream));
}

lq_status lq_sign_gemm_workspace_size(int64_t B, int64_t N, int64_t L, lq_dtype ztype,
                                      lq_algo algo, size_t* bytes) {
  if (bytes == nullptr || !valid_dtype(ztype)) return LQ_ERR_INVALID_ARG;
  if (!valid_algo(algo, false)) return LQ_ERR_INVALID_ARG;
  lq_status s = check_sign_dims(B, N, L);
  if (s != LQ_OK) return s;
  if (B == 0 || N == 0) { *bytes = 0; return LQ_OK; }
  Exec e;
  s = plan_exec(B, N, L, 0, 1, 1, ztype, algo, false, &e);
  if (s != LQ_OK) return s;
  *bytes = e.total;
  return LQ_OK;
}

lq_status lq_sign_gemm_ex(const uint8_t* packed, const void* z, lq_dtype ztype, int64_t B,
                          int64_t N, int64_t L, const float* row_scale, void* y, lq_dtype ytype,
                          lq_algo algo, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(ztype) || !valid_dtype(ytype)) return LQ_ERR_INVALID_ARG;
  if (!valid_algo(algo, false)) return LQ_ERR_INVALID_ARG;
  lq_status s = check_sign_dims(B, N, L);
  if (s != LQ_OK) return s;
  if (B == 0 || N == 0) return LQ_OK;
  Exec e;
  s = plan_exec(B, N, L, 0, 1, 1, ztype, algo, false, &e);
  if (s != LQ_OK) return s;
  if (!aligned16(packed) || !aligned16(z) || !aligned16(row_scale) || !aligned16(y))
    return LQ_ERR_INVALID_ARG;
  s = check_ws(ws, ws_bytes, e.total);
  if (s != LQ_OK) return s;
  return run_exec(e, packed, z, ztype, B, N, L, row_scale, y, ytype, ws, (hipStream_t)stream, nullptr);
}

lq_status lq_sign_gemm(const uint8_t* packed, const void* z, lq_dtype ztype, int64_t B, int64_t N,
                       int64_t L, const float* row_scale, void* y, lq_dtype ytype, void* ws,
                       size_t ws_bytes, void* stream) {
  return lq_sign_gemm_ex(packed, z, ztype, B, N, L, row_scale, y, ytype, LQ_ALGO_AUTO, ws,
                         ws_bytes, stream);
}

lq_status lq_linear_workspace_size_ex(const lq_layer* layer, int64_t B, lq_dtype xtype,
                                      lq_algo algo, size_t* bytes) {
  if (bytes == nullptr || !valid_dtype(xtype) || B < 0) return LQ_ERR_INVALID_ARG;
  if (!valid_algo(algo, true)) return LQ_ERR_INVALID_ARG;
  int64_t L = 0;
  lq_status s = check_layer(layer, &L);
  if (s != LQ_OK) return s;
  s = check_sign_dims(B, layer->N, L);
  if (s != LQ_OK) return s;
  if (!mul_ok(B, layer->K, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  if (B == 0 || layer->N == 0) { *bytes = 0; return LQ_OK; }
  Exec e;
  s = plan_exec(B, layer->N, L, layer->K, layer->d, layer->D, xtype, algo, true, &e);
  if (s != LQ_OK) return s;
  *bytes = e.total;
  return LQ_OK;
}

lq_status lq_linear_algo(const lq_layer* layer, int64_t B, lq_dtype xtype, lq_algo algo,
                         lq_algo* resolved) {
  if (resolved == nullptr || !valid_dtype(xtype) || B < 1) return LQ_ERR_INVALID_ARG;
  if (!valid_algo(algo, true)) return LQ_ERR_INVALID_ARG;
  int64_t L = 0;
  lq_status s = check_layer(layer, &L);
  if (s != LQ_OK) return s;
  s = check_sign_dims(B, layer->N, L);
  if (s != LQ_OK) return s;
  if (!mul_ok(B, layer->K, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  Exec e;
  s = plan_exec(B, layer->N, L, layer->K, layer->d, layer->D, xtype, algo, true, &e);
  if (s != LQ_OK) return s;
  *resolved = e.algo;
  return LQ_OK;
}

lq_status lq_linear_plan(const lq_layer* layer, int64_t B, lq_dtype xtype, lq_algo algo,
                         lq_plan_info* info) {
  if (info == nullptr || !valid_dtype(xtype) || B < 1) return LQ_ERR_INVALID_ARG;
  if (!valid_algo(algo, true)) return LQ_ERR_INVALID_ARG;
  int64_t L = 0;
  lq_status s = check_layer(layer, &L);
  if (s != LQ_OK) return s;
  s = check_sign_dims(B, layer->N, L);
  if (s != LQ_OK) return s;
  if (!mul_ok(B, layer->K, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  Exec e;
  s = plan_exec(B, layer->N, L, layer->K, layer->d, layer->D, xtype, algo, true, &e);
  if (s != LQ_OK) return s;
  fill_plan_info(e, B, info);
  return LQ_OK;
}

lq_status lq_sign_gemm_plan(int64_t B, int64_t N, int64_t L, lq_dtype ztype, lq_algo algo,
                            lq_plan_info* info) {
  if (info == nullptr || !valid_dtype(ztype) || B < 1) return LQ_ERR_INVALID_ARG;
  if (!valid_algo(algo, false)) return LQ_ERR_INVALID_ARG;
  lq_status s = check_sign_dims(B, N, L);
  if (s != LQ_OK) return s;
  Exec e;
  s = plan_exec(B, N, L, 0, 1, 1, ztype, algo, false, &e);
  if (s != LQ_OK) return s;
  fill_plan_info(e, B, info);
  return LQ_OK;
}

lq_status lq_linear_workspace_size(const lq_layer* layer, int64_t B, lq_dtype xtype,
                                   size_t* bytes) {
  return lq_linear_workspace_size_ex(layer, B, xtype, LQ_ALGO_AUTO, bytes);
}

lq_status lq_linear_ex(const lq_layer* layer, const void* x, lq_dtype xtype, int64_t B, void* y,
                       lq_dtype ytype, lq_algo algo, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(xtype) || !valid_dtype(ytype) || B < 0) return LQ_ERR_INVALID_ARG;
  if (!valid_algo(algo, true)) return LQ_ERR_INVALID_ARG;
  int64_t L = 0;
  lq_status s = check_layer(layer, &L);
  if (s != LQ_OK) return s;
  s = check_sign_dims(B, layer->N, L);
  if (s != LQ_OK) return s;
  if (!mul_ok(B, layer->K, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  if (B == 0 || layer->N == 0) return LQ_OK;
  if (!aligned16(x) || !aligned16(y) || !aligned16(layer->packed) || !aligned16(layer->M) ||
      !aligned16(layer->c) || !aligned16(layer->row_scale))
    return LQ_ERR_INVALID_ARG;
  Exec e;
  s = plan_exec(B, layer->N, L, layer->K, layer->d, layer->D, xtype, algo, true, &e);
  if (s != LQ_OK) return s;
  s = check_ws(ws, ws_bytes, e.total);
  if (s != LQ_OK) return s;
  return run_exec(e, layer->packed, x, xtype, B, layer->N, L, layer->row_scale, y, ytype, ws,
                  (hipStream_t)stream, layer);
}

lq_status lq_linear(const lq_layer* layer, const void* x, lq_dtype xtype, int64_t B, void* y,
                    lq_dtype ytype, void* ws, size_t ws_bytes, void* stream) {
  return lq_linear_ex(layer, x, xtype, B, y, ytype, LQ_ALGO_AUTO, ws, ws_bytes, stream);
}

lq_status lq_linear_noalloc(const lq_layer* layer, const void* x, lq_dtype xtype, int64_t B,
                            void* y, lq_dtype ytype, void* stream) {
  if (!valid_dtype(xtype) || !valid_dtype(ytype) || B < 0) return LQ_ERR_INVALID_ARG;
  int64_t L = 0;
  lq_status s = check_layer(layer, &L);
  if (s != LQ_OK) return s;
  s = check_sign_dims(B, layer->N, L);
  if (s != LQ_OK) return s;
  if (!mul_ok(B, layer->K, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  if (B == 0 || layer->N == 0) return LQ_OK;
  if (!aligned16(x) || !aligned16(y) || !aligned16(layer->packed) || !aligned16(layer->M) ||
      !aligned16(layer->c) || !aligned16(layer->row_scale))
    return LQ_ERR_INVALID_ARG;
  Exec e;
  s = plan_exec(B, layer->N, L, layer->K, layer->d, layer->D, xtype, LQ_ALGO_AUTO, true, &e);
  if (s != LQ_OK) return s;
  if (e.total > (size_t)LQ_NOALLOC_SCRATCH_BYTES) return LQ_ERR_UNSUPPORTED;
  void* ws = nullptr;
  s = noalloc_scratch(&ws);
  if (s != LQ_OK) return s;
  return run_exec(e, layer->packed, x, xtype, B, layer->N, L, layer->row_scale, y, ytype, ws,
                  (hipStream_t)stream, layer);
}

lq_status lq_linear_multi_workspace_size(const lq_layer* layers, int32_t n, int64_t B,
                                         lq_dtype xtype, size_t* bytes) {
  if (bytes == nullptr) return LQ_ERR_INVALID_ARG;
  MultiPlan mp;
  const lq_status s = plan_multi(layers, n, B, xtype, &mp);
  if (s != LQ_OK) return s;
  *bytes = mp.total;
  return LQ_OK;
}

lq_status lq_linear_multi(const lq_layer* layers, int32_t n, const void* x, lq_dtype xtype,
                          int64_t B, void* const* ys, lq_dtype ytype, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!valid_dtype(ytype) || ys == nullptr) return LQ_ERR_INVALID_ARG;
  MultiPlan mp;
  lq_status s = plan_multi(layers, n, B, xtype, &mp);
  if (s != LQ_OK) return s;
  if (mp.n == 0) return LQ_OK;
  if (!aligned16(x)) return LQ_ERR_INVALID_ARG;
  for (int j = 0; j < mp.n; ++j) {
    const lq_layer& l = layers[mp.idx[j]];
    if (!aligned16(ys[mp.idx[j]]) || !aligned16(l.packed) || !aligned16(l.M) ||
        !aligned16(l.c) || !aligned16(l.row_scale))
      return LQ_ERR_INVALID_ARG;
  }
  s = check_ws(ws, ws_bytes, mp.total);
  if (s != LQ_OK) return s;
  const hipStream_t st = (hipStream_t)stream;
  if (!mp.grouped) {
    for (int j = 0; j < mp.n; ++j) {
      const lq_layer& l = layers[mp.idx[j]];
      s = run_exec(mp.e[j], l.packed, x, xtype, B, l.N, mp.L[j], l.row_scale, ys[mp.idx[j]],
                   ytype, ws, st, &l);
      if (s != LQ_OK) return s;
    }
    return LQ_OK;
  }
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  lq::PrepLayerDesc pd[LQ_MULTI_MAX];
  lq::SignLayerDesc sd[LQ_MULTI_MAX];
  for (int j = 0; j < mp.n; ++j) {
    const lq_layer& l = layers[mp.idx[j]];
    uint8_t* aop = base + mp.off_aop[j];
    pd[j] = lq::PrepLayerDesc{l.d, l.D, l.hb, mp.L[j], l.c, l.M, aop};
    sd[j] = lq::SignLayerDesc{l.packed, mp.e[j].g, aop, l.row_scale, ys[mp.idx[j]], mp.e[j].fp};
  }
  s = hip_status(lq::launch_prep_multi(x, xtype == LQ_BF16, B, layers[0].K, mp.n, pd, mp.e[0].os, st));
  if (s != LQ_OK) return s;
  return hip_status(profiled(st, [&] {
    return lq::launch_sign_fp6_multi(mp.n, sd, mp.e[0].os, B, ytype == LQ_BF16, st);
  }));
}

lq_status lq_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (ws_bytes == 0) return LQ_OK;
  if (!aligned16(ws)) return LQ_ERR_INVALID_ARG;
  const size_t n = std::min(ws_bytes, (size_t)LQ_WS_CONTROL_BYTES) / 4;
  if (n == 0) return LQ_OK;
  return hip_status(lq::launch_zero_u32(static_cast<unsigned*>(ws), (int)n, (hipStream_t)stream));
}

lq_status lq_workspace_status(const void* ws, size_t ws_bytes, void* stream) {
  if (ws_bytes < (size_t)LQ_WS_CONTROL_BYTES) return LQ_OK;
  if (!aligned16(ws)) return LQ_ERR_INVALID_ARG;
  const hipStream_t st = (hipStream_t)stream;
  uint32_t word = 0;
  const uint32_t* src = static_cast<const uint32_t*>(ws) + LQ_WS_ERROR_WORD;
  hipError_t e = hipMemcpyAsync(&word, src, sizeof(word), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_status(e);
  return word != 0 ? LQ_ERR_DEVICE : LQ_OK;
}

lq_status lq_debug_fused_timeout(int32_t enable) {
  lq::set_fused_forced_timeout(enable != 0);
  return LQ_OK;
}

static_assert(LQ_ENCODE_MAX_D == lq::kEncodeMaxD && LQ_ENCODE_MAX_SMALL_D == lq::kEncodeMaxSmallD,
              "encoder limits");

static lq_status check_encode_dims(int64_t n, int32_t d, int32_t D) {
  if (n < 0 || d < 1 || D < 1) return LQ_ERR_INVALID_ARG;
  if (d > D) return LQ_ERR_INVALID_ARG;
  if (d > LQ_ENCODE_MAX_SMALL_D || D > LQ_ENCODE_MAX_D) return LQ_ERR_UNSUPPORTED;
  if (!mul_ok(n, D, kMaxElems) || !mul_ok(n, d, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  return LQ_OK;
}

static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

lq_status lq_encode(const float* w, int64_t nblocks, int32_t d, int32_t D, const float* M,
                    int8_t* signs, float* dist2, void* stream) {
  lq_status s = check_encode_dims(nblocks, d, D);
  if (s != LQ_OK) return s;
  if (nblocks == 0) return LQ_OK;
  if (w == nullptr || M == nullptr || signs == nullptr) return LQ_ERR_INVALID_ARG;
  if (!aligned4(w) || !aligned4(M) || !aligned4(dist2)) return LQ_ERR_INVALID_ARG;
  return hip_status(lq::launch_encode(w, nblocks, d, D, M, signs, dist2, (hipStream_t)stream));
}

static_assert(LQ_ENCODE_PINV_MAX_D == lq::kEncodePinvMaxD &&
              LQ_ENCODE_PINV_MAX_FREE == lq::kEncodePinvMaxFree, "partial search limits");

static lq_status check_pinv_dims(int64_t n, int32_t d, int32_t D) {
  if (n < 0 || d < 1 || D < 1) return LQ_ERR_INVALID_ARG;
  if (d > D) return LQ_ERR_INVALID_ARG;
  if (d > LQ_ENCODE_MAX_SMALL_D || D > LQ_ENCODE_PINV_MAX_D || D - d > LQ_ENCODE_PINV_MAX_FREE)
    return LQ_ERR_UNSUPPORTED;
  if (!mul_ok(n, D, kMaxElems) || !mul_ok(n, d, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  return LQ_OK;
}

static size_t pinv_table_bytes(int32_t d, int32_t D) {
  return ((size_t)d * (size_t)D * sizeof(double) + 255) / 256 * 256;
}

lq_status lq_encode_pinv_workspace_size(int32_t d, int32_t D, size_t* bytes) {
  if (bytes == nullptr) return LQ_ERR_INVALID_ARG;
  const lq_status s = check_pinv_dims(0, d, D);
  if (s != LQ_OK) return s;
  *bytes = pinv_table_bytes(d, D);
  return LQ_OK;
}

// A = M_a^-1 by Gauss-Jordan elimination with partial pivoting (fp64), then
// B = A M_f; false when a pivot is at most 2^-40 of M_a's largest magnitude.
static bool pinv_tables(const std::vector<float>& M, int d, int D, std::vector<double>& AB) {
  const int W = 2 * d;
  std::vector<double> a((size_t)d * W, 0.0);
  double amax = 0.0;
  for (int i = 0; i < d; ++i) {
    for (int e = 0; e < d; ++e) {
      a[(size_t)i * W + e] = (double)M[(size_t)i * D + e];
      amax = std::max(amax, std::fabs((double)M[(size_t)i * D + e]));
    }
    a[(size_t)i * W + d + i] = 1.0;
  }
  const double tol = std::ldexp(amax, -40);
  if (!(amax > 0.0)) return false;
  for (int c = 0; c < d; ++c) {
    int p = c;
    for (int r = c + 1; r < d; ++r)
      if (std::fabs(a[(size_t)r * W + c]) > std::fabs(a[(size_t)p * W + c])) p = r;
    if (!(std::fabs(a[(size_t)p * W + c]) > tol)) return false;
    if (p != c)
      for (int k = 0; k < W; ++k) std::swap(a[(size_t)p * W + k], a[(size_t)c * W + k]);
    const double piv = a[(size_t)c * W + c];
    for (int k = 0; k < W; ++k) a[(size_t)c * W + k] /= piv;
    for (int r = 0; r < d; ++r) {
      if (r == c) continue;
      const double f = a[(size_t)r * W + c];
      if (f == 0.0) continue;
      for (int k = 0; k < W; ++k) a[(size_t)r * W + k] -= f * a[(size_t)c * W + k];
    }
  }
  const int F = D - d;
  AB.assign((size_t)d * D, 0.0);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) AB[(size_t)i * d + j] = a[(size_t)i * W + d + j];
  for (int i = 0; i < d; ++i)
    for (int k = 0; k < F; ++k) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j) acc += AB[(size_t)i * d + j] * (double)M[(size_t)j * D + d + k];
      AB[(size_t)d * d + (size_t)i * F + k] = acc;
    }
  return true;
}

lq_status lq_encode_pinv(const float* w, int64_t nblocks, int32_t d, int32_t D, const float* M,
                         int8_t* signs, float* dist2, void* ws, size_t ws_bytes, void* stream) {
  lq_status s = check_pinv_dims(nblocks, d, D);
  if (s != LQ_OK) return s;
  if (nblocks == 0) return LQ_OK;
  if (w == nullptr || M == nullptr || signs == nullptr) return LQ_ERR_INVALID_ARG;
  if (!aligned4(w) || !aligned4(M) || !aligned4(dist2)) return LQ_ERR_INVALID_ARG;
  if (ws == nullptr || ws_bytes < pinv_table_bytes(d, D)) return LQ_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return LQ_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  // M to the host (the stream's earlier work first), the tables back
  std::vector<float> hm((size_t)d * D);
  hipError_t e = hipMemcpyAsync(hm.data(), M, hm.size() * sizeof(float), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_status(e);
  std::vector<double> ab;
  if (!pinv_tables(hm, d, D, ab)) return LQ_ERR_INVALID_ARG;
  e = hipMemcpyAsync(ws, ab.data(), ab.size() * sizeof(double), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);   // the host copy of the tables goes away
  if (e != hipSuccess) return hip_status(e);
  return hip_status(lq::launch_encode_pinv(w, nblocks, d, D, M, static_cast<const double*>(ws),
                                           signs, dist2, st));
}

lq_status lq_train_m_step_workspace_size(int64_t n, int32_t d, int32_t D, size_t* bytes) {
  if (bytes == nullptr) return LQ_ERR_INVALID_ARG;
  lq_status s = check_encode_dims(n, d, D);
  if (s != LQ_OK) return s;
  *bytes = n == 0 ? 0 : lq::train_workspace_bytes(n, d, D);
  return LQ_OK;
}

lq_status lq_train_m_step(float* M, const float* w, int64_t n, int32_t d, int32_t D, float lr,
                          float* loss, void* ws, size_t ws_bytes, void* stream) {
  lq_status s = check_encode_dims(n, d, D);
  if (s != LQ_OK) return s;
  if (n == 0) return LQ_OK;
  if (w == nullptr || M == nullptr) return LQ_ERR_INVALID_ARG;
  if (!aligned4(w) || !aligned4(M) || !aligned4(loss)) return LQ_ERR_INVALID_ARG;
  s = check_ws(ws, ws_bytes, lq::train_workspace_bytes(n, d, D));
  if (s != LQ_OK) return s;
  return hip_status(lq::launch_train_step(M, w, n, d, D, lr, loss, ws, (hipStream_t)stream));
}

lq_status lq_profile_events(void* const* starts, void* const* stops, int32_t count) {
  if (count < 0 || (count > 0 && (starts == nullptr || stops == nullptr))) return LQ_ERR_INVALID_ARG;
  ProfileRing& ring = profile_ring();
  std::lock_guard<std::mutex> lock(ring.mu);
  ring.starts.clear();
  ring.stops.clear();
  ring.next = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (starts[i] == nullptr || stops[i] == nullptr) {
      ring.starts.clear();
      ring.stops.clear();
      return LQ_ERR_INVALID_ARG;
    }
    ring.starts.push_back(static_cast<hipEvent_t>(starts[i]));
    ring.stops.push_back(static_cast<hipEvent_t>(stops[i]));
  }
  return LQ_OK;
}

}  // extern "C"
