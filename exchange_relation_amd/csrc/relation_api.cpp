// librelation C ABI: argument validation and dispatch to the gfx950 kernels.
// Every check runs on the host before anything is enqueued; on any error
// nothing is written (see include/relation.h).
#include "relation.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.hpp"

namespace {

constexpr long long kMaxElems = (1LL << 40);  // generous; guards size_t maths

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

relation_status check_params(float scale, float tau_s, float lambda) {
  if (!isfinite(scale) || !isfinite(lambda) || !isfinite(tau_s) || !(tau_s > 0.f))
    return REL_ERR_PARAM;
  return REL_OK;
}

relation_status check_dtype_dim(relation_dtype dt, int D) {
  if (dt == REL_F32) return (D == 32 || D == 64) ? REL_OK : REL_ERR_UNSUPPORTED;
  if (dt == REL_BF16) return (D == 64) ? REL_OK : REL_ERR_UNSUPPORTED;
  return REL_ERR_UNSUPPORTED;
}

relation_status check_shape(int B, int H, int T, int D) {
  if (B < 1 || H < 1 || T < 1 || D < 1) return REL_ERR_SHAPE;
  const long long n = static_cast<long long>(B) * H * T;
  if (n * D > kMaxElems) return REL_ERR_SHAPE;
  // one workgroup per 32..128 rows: keep the 1-D grid within 2^31 - 1
  if (static_cast<long long>(B) * H * ((T + 31) / 32) > 0x7fffffffLL) return REL_ERR_SHAPE;
  return REL_OK;
}

relation_status from_hip(hipError_t e) { return e == hipSuccess ? REL_OK : REL_ERR_HIP; }

}  // namespace

extern "C" {

int relation_version(void) { return 100; }

const char* relation_status_string(relation_status s) {
  switch (s) {
    case REL_OK: return "ok";
    case REL_ERR_NULL: return "a required pointer is NULL";
    case REL_ERR_SHAPE: return "invalid shape (B, H, T must be >= 1 and sizes in range)";
    case REL_ERR_UNSUPPORTED: return "unsupported dtype or head dimension";
    case REL_ERR_PARAM: return "invalid scalar (scale, lambda finite; tau_s > 0)";
    case REL_ERR_CAPACITY: return "cache capacity exceeded (need 0 <= n_hist < capacity)";
    case REL_ERR_ALIGN: return "pointer not aligned (16 B tensors, 256 B workspace)";
    case REL_ERR_WORKSPACE: return "workspace missing or too small";
    case REL_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

relation_status relation_fwd(relation_dtype dtype, int B, int H, int T, int D, const void* q,
                             const void* k, const void* v, void* y, float* lse, float* gate,
                             float scale, float tau_s, float lambda, void* stream) {
  if (!q || !k || !v || !y) return REL_ERR_NULL;
  relation_status st = check_dtype_dim(dtype, D);
  if (st != REL_OK) return st;
  if ((st = check_shape(B, H, T, D)) != REL_OK) return st;
  if ((st = check_params(scale, tau_s, lambda)) != REL_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) ||
      (lse && !aligned4(lse)) || (gate && !aligned4(gate)))
    return REL_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == REL_F32)
    return from_hip(rel::launch_fwd_f32(B, H, T, D, static_cast<const float*>(q),
                                        static_cast<const float*>(k),
                                        static_cast<const float*>(v), static_cast<float*>(y), lse,
                                        gate, scale, tau_s, lambda, s));
  return from_hip(rel::launch_fwd_bf16(B, H, T, D, static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k),
                                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(y),
                                       lse, gate, scale, tau_s, lambda, s));
}

size_t relation_bwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D) {
  if (check_dtype_dim(dtype, D) != REL_OK || check_shape(B, H, T, D) != REL_OK) return 0;
  return rel::bwd_workspace_bytes(dtype == REL_BF16 ? 1 : 0, B, H, T, D);
}

relation_status relation_bwd(relation_dtype dtype, int B, int H, int T, int D, const void* q,
                             const void* k, const void* v, const void* y, const void* dy,
                             const float* lse, void* dq, void* dk, void* dv, float* dlambda,
                             void* workspace, size_t workspace_bytes, float scale, float tau_s,
                             float lambda, void* stream) {
  if (!q || !k || !v || !y || !dy || !lse || !dq || !dk || !dv) return REL_ERR_NULL;
  relation_status st = check_dtype_dim(dtype, D);
  if (st != REL_OK) return st;
  if ((st = check_shape(B, H, T, D)) != REL_OK) return st;
  if ((st = check_params(scale, tau_s, lambda)) != REL_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) || !aligned16(dy) ||
      !aligned4(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (dlambda && !aligned4(dlambda)))
    return REL_ERR_ALIGN;
  const size_t need = rel::bwd_workspace_bytes(dtype == REL_BF16 ? 1 : 0, B, H, T, D);
  if (!workspace || workspace_bytes < need) return REL_ERR_WORKSPACE;
  if (!aligned256(workspace)) return REL_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == REL_F32)
    return from_hip(rel::launch_bwd_f32(
        B, H, T, D, static_cast<const float*>(q), static_cast<const float*>(k),
        static_cast<const float*>(v), static_cast<const float*>(y), static_cast<const float*>(dy),
        lse, static_cast<float*>(dq), static_cast<float*>(dk), static_cast<float*>(dv), dlambda,
        workspace, scale, tau_s, lambda, s));
  return from_hip(rel::launch_bwd_bf16(
      B, H, T, D, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(y),
      static_cast<const uint16_t*>(dy), lse, static_cast<uint16_t*>(dq),
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), dlambda, workspace, scale, tau_s,
      lambda, s));
}

size_t relation_decode_workspace_bytes(relation_dtype dtype, int B, int H, int D, int capacity) {
  if (check_dtype_dim(dtype, D) != REL_OK || B < 1 || H < 1 || capacity < 1) return 0;
  return rel::decode_workspace_bytes(dtype == REL_BF16 ? 1 : 0, B, H, D, capacity);
}

relation_status relation_cache_decode(relation_dtype dtype, int B, int H, int D, const void* q,
                                      const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, int capacity, int n_hist, void* y,
                                      float* gate, void* workspace, size_t workspace_bytes,
                                      float scale, float tau_s, float lambda, void* stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !y) return REL_ERR_NULL;
  relation_status st = check_dtype_dim(dtype, D);
  if (st != REL_OK) return st;
  if (B < 1 || H < 1 || capacity < 1) return REL_ERR_SHAPE;
  if (static_cast<long long>(B) * H * capacity * D > kMaxElems) return REL_ERR_SHAPE;
  if ((st = check_params(scale, tau_s, lambda)) != REL_OK) return st;
  if (n_hist < 0 || n_hist >= capacity) return REL_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(y) || (gate && !aligned4(gate)))
    return REL_ERR_ALIGN;
  const size_t need = rel::decode_workspace_bytes(dtype == REL_BF16 ? 1 : 0, B, H, D, capacity);
  if (!workspace || workspace_bytes < need) return REL_ERR_WORKSPACE;
  if (!aligned256(workspace)) return REL_ERR_ALIGN;
  return from_hip(rel::launch_decode(dtype == REL_BF16 ? 1 : 0, B, H, D, q, k_new, v_new,
                                     k_cache, v_cache, capacity, n_hist, nullptr, y, gate,
                                     workspace, scale, tau_s, lambda,
                                     static_cast<hipStream_t>(stream)));
}

relation_status relation_cache_decode_ragged(relation_dtype dtype, int B, int H, int D,
                                             const void* q, const void* k_new, const void* v_new,
                                             void* k_cache, void* v_cache, int capacity,
                                             const int* n_hist, int max_n_hist, void* y,
                                             float* gate, void* workspace, size_t workspace_bytes,
                                             float scale, float tau_s, float lambda,
                                             void* stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !y || !n_hist) return REL_ERR_NULL;
  relation_status st = check_dtype_dim(dtype, D);
  if (st != REL_OK) return st;
  if (B < 1 || H < 1 || capacity < 1) return REL_ERR_SHAPE;
  if (static_cast<long long>(B) * H * capacity * D > kMaxElems) return REL_ERR_SHAPE;
  if ((st = check_params(scale, tau_s, lambda)) != REL_OK) return st;
  if (max_n_hist < 0 || max_n_hist >= capacity) return REL_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(y) || (gate && !aligned4(gate)) || !aligned4(n_hist))
    return REL_ERR_ALIGN;
  const size_t need = rel::decode_workspace_bytes(dtype == REL_BF16 ? 1 : 0, B, H, D, capacity);
  if (!workspace || workspace_bytes < need) return REL_ERR_WORKSPACE;
  if (!aligned256(workspace)) return REL_ERR_ALIGN;
  return from_hip(rel::launch_decode(dtype == REL_BF16 ? 1 : 0, B, H, D, q, k_new, v_new,
                                     k_cache, v_cache, capacity, max_n_hist, n_hist, y, gate,
                                     workspace, scale, tau_s, lambda,
                                     static_cast<hipStream_t>(stream)));
}

}  // extern "C"
