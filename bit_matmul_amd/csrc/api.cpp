// The C ABI of liblq (declared in include/lq.h): argument validation,
// workspace carving and dispatch to the HIP launchers. Every check runs on the
// host before anything is enqueued, so a rejected call launches nothing.
#include "lq.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "lq_internal.h"

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
size_t dtype_size(lq_dtype t) { return t == LQ_F32 ? 4 : 2; }
size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

bool mul_ok(int64_t a, int64_t b, int64_t lim) { return a == 0 || b <= lim / a; }

// Checks shared by every entry point that takes (N, K, d, D); writes L.
lq_status check_layer_dims(int64_t N, int64_t K, int32_t d, int32_t D, int64_t* L) {
  if (N < 0 || K < 1 || d < 1 || D < d) return LQ_ERR_INVALID_ARG;
  if (D > LQ_MAX_D || N > kMaxDim || K > kMaxDim) return LQ_ERR_UNSUPPORTED;
  const int64_t Kb = (K + d - 1) / d;
  *L = Kb * D;
  if (N % lq::kPanelRows != 0 || *L % 8 != 0) return LQ_ERR_UNSUPPORTED;
  if (!mul_ok(N, *L, kMaxElems * 64)) return LQ_ERR_UNSUPPORTED;
  return LQ_OK;
}

lq_status check_sign_dims(int64_t B, int64_t N, int64_t L) {
  if (B < 0 || N < 0 || L < 1) return LQ_ERR_INVALID_ARG;
  if (B > kMaxBatch || N > kMaxDim || L > kMaxDim * LQ_MAX_D) return LQ_ERR_UNSUPPORTED;
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

// Launch `fn` (which enqueues one kernel) between the ring's next event pair.
template <typename Fn>
hipError_t profiled(hipStream_t stream, Fn fn) {
  ProfileRing& ring = profile_ring();
  std::unique_lock<std::mutex> lock(ring.mu);
  if (ring.starts.empty()) {
    lock.unlock();
    return fn();
  }
  const size_t i = ring.next;
  ring.next = (ring.next + 1) % ring.starts.size();
  hipError_t e = hipEventRecord(ring.starts[i], stream);
  if (e != hipSuccess) return e;
  e = fn();
  if (e != hipSuccess) return e;
  return hipEventRecord(ring.stops[i], stream);
}

lq_algo resolve_algo(lq_algo algo, lq_dtype ztype, int64_t B) {
  if (algo != LQ_ALGO_AUTO) return algo;
  if (B > 16) return LQ_ALGO_MFMA_LARGE;
  return ztype == LQ_F32 ? LQ_ALGO_VALU : LQ_ALGO_MFMA_SMALL;
}

// Workspace of the sign product; also validates the algorithm choice.
lq_status sign_ws(int64_t B, int64_t N, int64_t L, lq_dtype ztype, lq_algo algo, size_t* bytes) {
  const lq::PackedGeom g = lq::make_geom(N, L);
  switch (resolve_algo(algo, ztype, B)) {
    case LQ_ALGO_VALU: *bytes = lq::plan_valu(B, g).ws_bytes; return LQ_OK;
    case LQ_ALGO_MFMA_SMALL:
      if (B > 16) return LQ_ERR_UNSUPPORTED;
      *bytes = lq::plan_mfma_small(B, g, ztype == LQ_BF16).ws_bytes;
      return LQ_OK;
    case LQ_ALGO_MFMA_LARGE: *bytes = 0; return LQ_OK;
    default: return LQ_ERR_INVALID_ARG;
  }
}

lq_status run_sign(const uint8_t* packed, const void* z, lq_dtype ztype, int64_t B, int64_t N,
                   int64_t L, const float* row_scale, void* y, lq_dtype ytype, lq_algo algo,
                   void* ws, hipStream_t stream) {
  const lq::PackedGeom g = lq::make_geom(N, L);
  const bool zb = ztype == LQ_BF16, yb = ytype == LQ_BF16;
  switch (resolve_algo(algo, ztype, B)) {
    case LQ_ALGO_VALU: {
      const lq::SplitPlan plan = lq::plan_valu(B, g);
      float* partial = static_cast<float*>(ws);
      float* colsum = partial + (size_t)plan.ksplit * B * N;
      lq_status s = hip_status(profiled(stream, [&] {
        return lq::launch_sign_valu(packed, g, z, zb, B, plan, partial, colsum, stream);
      }));
      if (s != LQ_OK) return s;
      return hip_status(lq::launch_split_epilogue(partial, colsum, plan.ksplit, B, N, row_scale, y, yb, stream));
    }
    case LQ_ALGO_MFMA_SMALL: {
      const lq::SplitPlan plan = lq::plan_mfma_small(B, g, zb);
      float* partial = static_cast<float*>(ws);
      lq_status s = hip_status(profiled(stream, [&] {
        return lq::launch_sign_mfma_small(packed, g, z, zb, B, plan, partial, stream);
      }));
      if (s != LQ_OK) return s;
      return hip_status(lq::launch_split_epilogue(partial, nullptr, plan.ksplit, B, N, row_scale, y, yb, stream));
    }
    case LQ_ALGO_MFMA_LARGE:
      return hip_status(profiled(stream, [&] {
        return lq::launch_sign_mfma_large(packed, g, z, zb, B, row_scale, y, yb, stream);
      }));
    default:
      return LQ_ERR_INVALID_ARG;
  }
}

lq_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return LQ_OK;
  if (ws == nullptr || ws_bytes < need) return LQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return LQ_ERR_INVALID_ARG;
  return LQ_OK;
}

lq_status linear_ws(const lq_layer* layer, int64_t B, lq_dtype xtype, int64_t L, size_t* total,
                    size_t* off_z, size_t* off_sign) {
  const lq_dtype zt = xtype;   // lifted values keep the activation dtype
  size_t sbytes = 0;
  lq_status s = sign_ws(B, layer->N, L, zt, LQ_ALGO_AUTO, &sbytes);
  if (s != LQ_OK) return s;
  const size_t xt_bytes = align_up((size_t)B * layer->K * sizeof(float));
  const size_t z_bytes = align_up((size_t)B * L * dtype_size(zt));
  *off_z = xt_bytes;
  *off_sign = xt_bytes + z_bytes;
  *total = xt_bytes + z_bytes + align_up(sbytes);
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
  lq_status s = check_sign_dims(B, N, L);
  if (s != LQ_OK) return s;
  if (B == 0 || N == 0) { *bytes = 0; return LQ_OK; }
  return sign_ws(B, N, L, ztype, algo, bytes);
}

lq_status lq_sign_gemm_ex(const uint8_t* packed, const void* z, lq_dtype ztype, int64_t B,
                          int64_t N, int64_t L, const float* row_scale, void* y, lq_dtype ytype,
                          lq_algo algo, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(ztype) || !valid_dtype(ytype)) return LQ_ERR_INVALID_ARG;
  if (algo < LQ_ALGO_AUTO || algo > LQ_ALGO_MFMA_LARGE) return LQ_ERR_INVALID_ARG;
  lq_status s = check_sign_dims(B, N, L);
  if (s != LQ_OK) return s;
  if (B == 0 || N == 0) return LQ_OK;
  size_t need = 0;
  s = sign_ws(B, N, L, ztype, algo, &need);
  if (s != LQ_OK) return s;
  if (!aligned16(packed) || !aligned16(z) || !aligned16(row_scale) || !aligned16(y))
    return LQ_ERR_INVALID_ARG;
  s = check_ws(ws, ws_bytes, need);
  if (s != LQ_OK) return s;
  return run_sign(packed, z, ztype, B, N, L, row_scale, y, ytype, algo, ws, (hipStream_t)stream);
}

lq_status lq_sign_gemm(const uint8_t* packed, const void* z, lq_dtype ztype, int64_t B, int64_t N,
                       int64_t L, const float* row_scale, void* y, lq_dtype ytype, void* ws,
                       size_t ws_bytes, void* stream) {
  return lq_sign_gemm_ex(packed, z, ztype, B, N, L, row_scale, y, ytype, LQ_ALGO_AUTO, ws,
                         ws_bytes, stream);
}

lq_status lq_linear_workspace_size(const lq_layer* layer, int64_t B, lq_dtype xtype,
                                   size_t* bytes) {
  if (bytes == nullptr || !valid_dtype(xtype) || B < 0) return LQ_ERR_INVALID_ARG;
  int64_t L = 0;
  lq_status s = check_layer(layer, &L);
  if (s != LQ_OK) return s;
  s = check_sign_dims(B, layer->N, L);
  if (s != LQ_OK) return s;
  if (B == 0 || layer->N == 0) { *bytes = 0; return LQ_OK; }
  size_t oz = 0, os = 0;
  return linear_ws(layer, B, xtype, L, bytes, &oz, &os);
}

lq_status lq_linear(const lq_layer* layer, const void* x, lq_dtype xtype, int64_t B, void* y,
                    lq_dtype ytype, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_dtype(xtype) || !valid_dtype(ytype) || B < 0) return LQ_ERR_INVALID_ARG;
  int64_t L = 0;
  lq_status s = check_layer(layer, &L);
  if (s != LQ_OK) return s;
  s = check_sign_dims(B, layer->N, L);
  if (s != LQ_OK) return s;
  if (B > kMaxBatch || !mul_ok(B, layer->K, kMaxElems)) return LQ_ERR_UNSUPPORTED;
  if (B == 0 || layer->N == 0) return LQ_OK;
  if (!aligned16(x) || !aligned16(y) || !aligned16(layer->packed) || !aligned16(layer->M) ||
      !aligned16(layer->c) || !aligned16(layer->row_scale))
    return LQ_ERR_INVALID_ARG;
  size_t need = 0, off_z = 0, off_sign = 0;
  s = linear_ws(layer, B, xtype, L, &need, &off_z, &off_sign);
  if (s != LQ_OK) return s;
  s = check_ws(ws, ws_bytes, need);
  if (s != LQ_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  char* base = static_cast<char*>(ws);
  float* xt = reinterpret_cast<float*>(base);
  void* z = base + off_z;
  void* sws = base + off_sign;
  const lq_dtype zt = xtype;
  s = hip_status(lq::launch_hadamard_scale(x, xtype == LQ_BF16, B, layer->K, layer->hb, layer->c, xt, st));
  if (s != LQ_OK) return s;
  s = hip_status(lq::launch_lift(xt, B, layer->K, layer->d, layer->D, layer->M, z, zt == LQ_BF16, st));
  if (s != LQ_OK) return s;
  return run_sign(layer->packed, z, zt, B, layer->N, L, layer->row_scale, y, ytype, LQ_ALGO_AUTO,
                  sws, st);
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
