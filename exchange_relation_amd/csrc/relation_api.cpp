// librelation C ABI: argument validation and dispatch to the gfx950 kernels.
// Every check runs on the host before anything is enqueued; on any error
// nothing is written (see include/relation.h).
#include "relation.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bwd_common.hpp"
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

// Head dimensions built: fp32 (accurate VALU paths) D in {32, 64}; bf16
// forward, decode and prefill D in {48, 64, 80} (the paper's 10M / 30M /
// 100M head widths), bf16 backward D in {48, 64, 80}.
relation_status check_dtype_dim(relation_dtype dt, int D) {
  if (dt == REL_F32) return (D == 32 || D == 64) ? REL_OK : REL_ERR_UNSUPPORTED;
  if (dt == REL_BF16) return (D == 48 || D == 64 || D == 80) ? REL_OK : REL_ERR_UNSUPPORTED;
  return REL_ERR_UNSUPPORTED;
}
relation_status check_dtype_dim_bwd(relation_dtype dt, int D) {
  if (dt == REL_F32) return (D == 32 || D == 64) ? REL_OK : REL_ERR_UNSUPPORTED;
  if (dt == REL_BF16) return (D == 48 || D == 64 || D == 80) ? REL_OK : REL_ERR_UNSUPPORTED;
  return REL_ERR_UNSUPPORTED;
}

// The kernels index inside one head (rows x D, or capacity x D) with 32-bit
// offsets from the head's base.
constexpr long long kMaxHeadElems = 0x7fffffffLL;

relation_status check_shape(int B, int H, int T, int D) {
  if (B < 1 || H < 1 || T < 1 || D < 1) return REL_ERR_SHAPE;
  const long long n = static_cast<long long>(B) * H * T;
  if (n * D > kMaxElems) return REL_ERR_SHAPE;
  if (static_cast<long long>(T) * D > kMaxHeadElems) return REL_ERR_SHAPE;
  // one workgroup per 32..128 rows: keep the 1-D grid within 2^31 - 1
  if (static_cast<long long>(B) * H * ((T + 31) / 32) > 0x7fffffffLL) return REL_ERR_SHAPE;
  return REL_OK;
}

relation_status from_hip(hipError_t e) { return e == hipSuccess ? REL_OK : REL_ERR_HIP; }

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of the Multi-Head Relation entry points: the rotated / mixed
// q, k, v (the bf16 forward rotates its queries in registers and needs only
// k and v), then for the backward the plain backward's workspace, fp32 dk
// and dv (bf16 only) and the dtheta partials.
struct MhrLayout {
  size_t q, k, v, bwd, dk32, dv32, part, total;
};
MhrLayout mhr_layout(bool backward, relation_dtype dt, int B, int H, int T, int D) {
  MhrLayout L{};
  const size_t n = static_cast<size_t>(B) * H * T * D;
  const size_t esz = dt == REL_BF16 ? 2 : 4;
  size_t off = 0;
  if (backward || dt == REL_F32 || D != 64) {  // the bf16 kernel rotates queries itself at D = 64
    L.q = off; off += round256(n * esz);
  }
  L.k = off; off += round256(n * esz);
  L.v = off; off += round256(n * esz);
  if (backward) {
    L.bwd = off; off += round256(rel::bwd_workspace_bytes(dt == REL_BF16 ? 1 : 0, B, H, T, D));
    if (dt == REL_BF16) {
      L.dk32 = off; off += round256(n * 4);
      L.dv32 = off; off += round256(n * 4);
    }
    L.part = off; off += round256(rel::mhr_part_floats(B, H, T, D) * 4);
  }
  L.total = off;
  return L;
}

// Checks shared by the Multi-Head Relation entry points (tables and angles).
relation_status check_mhr(int H, const float* rope_cos, const float* rope_sin, const float* theta,
                          int pairing) {
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return REL_ERR_NULL;
  if (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) return REL_ERR_ALIGN;
  if (theta) {
    if (H % 2) return REL_ERR_SHAPE;
    if (pairing != 0 && pairing != 1) return REL_ERR_PARAM;
    if (!aligned4(theta)) return REL_ERR_ALIGN;
  }
  return REL_OK;
}

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
    case REL_ERR_SCRATCH: return "call needs more than the library's static scratch (8 MiB)";
  }
  return "unknown status";
}

size_t relation_fwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D) {
  if (dtype != REL_BF16 || check_dtype_dim(dtype, D) != REL_OK || check_shape(B, H, T, D) != REL_OK)
    return 0;
  return rel::fwd_bf16_workspace_bytes(B, H, T, D);
}

relation_status relation_fwd(relation_dtype dtype, int B, int H, int T, int D, const void* q,
                             const void* k, const void* v, void* y, float* lse, float* gate,
                             void* workspace, size_t workspace_bytes, float scale, float tau_s,
                             float lambda, const float* lambda_dev, void* stream) {
  if (!q || !k || !v || !y) return REL_ERR_NULL;
  relation_status st = check_dtype_dim(dtype, D);
  if (st != REL_OK) return st;
  if ((st = check_shape(B, H, T, D)) != REL_OK) return st;
  if ((st = check_params(scale, tau_s, lambda)) != REL_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) ||
      (lse && !aligned4(lse)) || (gate && !aligned4(gate)) ||
      (lambda_dev && !aligned4(lambda_dev)))
    return REL_ERR_ALIGN;
  const rel::Lam lam(lambda, lambda_dev);
  if (workspace) {
    if (workspace_bytes < relation_fwd_workspace_bytes(dtype, B, H, T, D))
      return REL_ERR_WORKSPACE;
    if (!aligned256(workspace)) return REL_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == REL_F32)
    return from_hip(rel::launch_fwd_f32(B, H, T, D, static_cast<const float*>(q),
                                        static_cast<const float*>(k),
                                        static_cast<const float*>(v), static_cast<float*>(y), lse,
                                        gate, scale, tau_s, lam, s));
  return from_hip(rel::launch_fwd_bf16(B, H, T, D, static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k),
                                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(y),
                                       lse, gate, scale, tau_s, lam, s, nullptr, nullptr,
                                       static_cast<float*>(workspace),
                                       workspace ? workspace_bytes : 0));
}

size_t relation_bwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D) {
  if (check_dtype_dim_bwd(dtype, D) != REL_OK || check_shape(B, H, T, D) != REL_OK) return 0;
  return rel::bwd_workspace_bytes(dtype == REL_BF16 ? 1 : 0, B, H, T, D);
}

static relation_status bwd_impl(relation_dtype dtype, int B, int H, int T, int D, const void* q,
                                const void* k, const void* v, const void* y, const void* dy,
                                const float* lse, void* dq, void* dk, void* dv, float* dlambda,
                                void* workspace, size_t workspace_bytes, float scale, float tau_s,
                                float lambda, const float* lambda_dev, void* stream,
                                hipEvent_t ev0, hipEvent_t ev1) {
  if (!q || !k || !v || !y || !dy || !lse || !dq || !dk || !dv) return REL_ERR_NULL;
  relation_status st = check_dtype_dim_bwd(dtype, D);
  if (st != REL_OK) return st;
  if ((st = check_shape(B, H, T, D)) != REL_OK) return st;
  if ((st = check_params(scale, tau_s, lambda)) != REL_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) || !aligned16(dy) ||
      !aligned4(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (dlambda && !aligned4(dlambda)) || (lambda_dev && !aligned4(lambda_dev)))
    return REL_ERR_ALIGN;
  const rel::Lam lam(lambda, lambda_dev);
  const size_t need = rel::bwd_workspace_bytes(dtype == REL_BF16 ? 1 : 0, B, H, T, D);
  if (!workspace || workspace_bytes < need) return REL_ERR_WORKSPACE;
  if (!aligned256(workspace)) return REL_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == REL_F32)
    return from_hip(rel::launch_bwd_f32(
        B, H, T, D, static_cast<const float*>(q), static_cast<const float*>(k),
        static_cast<const float*>(v), static_cast<const float*>(y), static_cast<const float*>(dy),
        lse, static_cast<float*>(dq), static_cast<float*>(dk), static_cast<float*>(dv), dlambda,
        workspace, scale, tau_s, lam, s, ev0, ev1));
  return from_hip(rel::launch_bwd_bf16(
      B, H, T, D, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(y),
      static_cast<const uint16_t*>(dy), lse, static_cast<uint16_t*>(dq),
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), dlambda, workspace, scale, tau_s,
      lam, s, nullptr, nullptr, nullptr, nullptr, ev0, ev1));
}

relation_status relation_bwd(relation_dtype dtype, int B, int H, int T, int D, const void* q,
                             const void* k, const void* v, const void* y, const void* dy,
                             const float* lse, void* dq, void* dk, void* dv, float* dlambda,
                             void* workspace, size_t workspace_bytes, float scale, float tau_s,
                             float lambda, const float* lambda_dev, void* stream) {
  return bwd_impl(dtype, B, H, T, D, q, k, v, y, dy, lse, dq, dk, dv, dlambda, workspace,
                  workspace_bytes, scale, tau_s, lambda, lambda_dev, stream, nullptr, nullptr);
}

relation_status relation_bwd_events(relation_dtype dtype, int B, int H, int T, int D,
                                    const void* q, const void* k, const void* v, const void* y,
                                    const void* dy, const float* lse, void* dq, void* dk,
                                    void* dv, float* dlambda, void* workspace,
                                    size_t workspace_bytes, float scale, float tau_s,
                                    float lambda, const float* lambda_dev, void* stream,
                                    void* ev_main_begin, void* ev_main_end) {
  return bwd_impl(dtype, B, H, T, D, q, k, v, y, dy, lse, dq, dk, dv, dlambda, workspace,
                  workspace_bytes, scale, tau_s, lambda, lambda_dev, stream,
                  static_cast<hipEvent_t>(ev_main_begin), static_cast<hipEvent_t>(ev_main_end));
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
  if (static_cast<long long>(B) * H * capacity * D > kMaxElems ||
      static_cast<long long>(capacity) * D > kMaxHeadElems)
    return REL_ERR_SHAPE;
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

relation_status relation_cache_decode_noalloc(relation_dtype dtype, int B, int H, int D,
                                              const void* q, const void* k_new,
                                              const void* v_new, void* k_cache, void* v_cache,
                                              int capacity, int n_hist, void* y, float* gate,
                                              float scale, float tau_s, float lambda,
                                              void* stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !y) return REL_ERR_NULL;
  relation_status st = check_dtype_dim(dtype, D);
  if (st != REL_OK) return st;
  if (B < 1 || H < 1 || capacity < 1) return REL_ERR_SHAPE;
  if (static_cast<long long>(B) * H * capacity * D > kMaxElems ||
      static_cast<long long>(capacity) * D > kMaxHeadElems)
    return REL_ERR_SHAPE;
  if ((st = check_params(scale, tau_s, lambda)) != REL_OK) return st;
  if (n_hist < 0 || n_hist >= capacity) return REL_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(y) || (gate && !aligned4(gate)))
    return REL_ERR_ALIGN;
  if (rel::decode_uniform_need_bytes(B, H, D, n_hist) > rel::decode_scratch_bytes())
    return REL_ERR_SCRATCH;
  return from_hip(rel::launch_decode_noalloc(dtype == REL_BF16 ? 1 : 0, B, H, D, q, k_new, v_new,
                                             k_cache, v_cache, capacity, n_hist, y, gate, scale,
                                             tau_s, lambda, static_cast<hipStream_t>(stream)));
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
  if (static_cast<long long>(B) * H * capacity * D > kMaxElems ||
      static_cast<long long>(capacity) * D > kMaxHeadElems)
    return REL_ERR_SHAPE;
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

size_t relation_prefill_workspace_bytes(relation_dtype dtype, int B, int H, int D, int m,
                                        int n_hist, int per_sequence) {
  if (dtype != REL_BF16 || check_dtype_dim(dtype, D) != REL_OK) return 0;
  if (B < 1 || H < 1 || m < 1 || n_hist < 0) return 0;
  if (static_cast<long long>(B) * H * ((m + 31) / 32) > 0x7fffffffLL) return 0;
  return rel::prefill_workspace_bytes(B, H, D, m, n_hist, per_sequence != 0);
}

relation_status relation_cache_prefill(relation_dtype dtype, int B, int H, int D, int m,
                                       const void* q, const void* k_new, const void* v_new,
                                       void* k_cache, void* v_cache, int capacity,
                                       const int* n_hist_dev, int n_hist, void* y, float* lse,
                                       float* gate, void* workspace, size_t workspace_bytes,
                                       float scale, float tau_s, float lambda, void* stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !y) return REL_ERR_NULL;
  if (dtype != REL_BF16 || check_dtype_dim(dtype, D) != REL_OK) return REL_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || m < 1 || capacity < 1) return REL_ERR_SHAPE;
  if (static_cast<long long>(B) * H * capacity * D > kMaxElems ||
      static_cast<long long>(capacity) * D > kMaxHeadElems)
    return REL_ERR_SHAPE;
  if (static_cast<long long>(B) * H * ((m + 31) / 32) > 0x7fffffffLL) return REL_ERR_SHAPE;
  relation_status st = check_params(scale, tau_s, lambda);
  if (st != REL_OK) return st;
  if (n_hist < 0 || static_cast<long long>(n_hist) + m > capacity) return REL_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(y) || (lse && !aligned4(lse)) ||
      (gate && !aligned4(gate)) || (n_hist_dev && !aligned4(n_hist_dev)))
    return REL_ERR_ALIGN;
  if (workspace) {
    if (workspace_bytes <
        relation_prefill_workspace_bytes(dtype, B, H, D, m, n_hist, n_hist_dev != nullptr))
      return REL_ERR_WORKSPACE;
    if (!aligned256(workspace)) return REL_ERR_ALIGN;
  }
  return from_hip(rel::launch_prefill_bf16(
      B, H, D, m, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_new),
      static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(k_cache),
      static_cast<uint16_t*>(v_cache), capacity, n_hist_dev, n_hist, static_cast<uint16_t*>(y),
      lse, gate, scale, tau_s, lambda, static_cast<hipStream_t>(stream),
      static_cast<float*>(workspace), workspace ? workspace_bytes : 0));
}

size_t relation_mhr_fwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D) {
  if (check_dtype_dim(dtype, D) != REL_OK || check_shape(B, H, T, D) != REL_OK) return 0;
  return mhr_layout(false, dtype, B, H, T, D).total;
}

relation_status relation_mhr_fwd(relation_dtype dtype, int B, int H, int T, int D, const void* p1,
                                 const void* p2, const void* I, const float* rope_cos,
                                 const float* rope_sin, const float* theta, int pairing, void* y,
                                 float* lse, float* gate, void* workspace, size_t workspace_bytes,
                                 float scale, float tau_s, float lambda, const float* lambda_dev,
                                 void* stream) {
  if (!p1 || !p2 || !I || !y) return REL_ERR_NULL;
  relation_status st = check_dtype_dim(dtype, D);
  if (st != REL_OK) return st;
  if ((st = check_shape(B, H, T, D)) != REL_OK) return st;
  if ((st = check_params(scale, tau_s, lambda)) != REL_OK) return st;
  if ((st = check_mhr(H, rope_cos, rope_sin, theta, pairing)) != REL_OK) return st;
  if (!aligned16(p1) || !aligned16(p2) || !aligned16(I) || !aligned16(y) ||
      (lse && !aligned4(lse)) || (gate && !aligned4(gate)) ||
      (lambda_dev && !aligned4(lambda_dev)))
    return REL_ERR_ALIGN;
  const rel::Lam lam(lambda, lambda_dev);
  const MhrLayout L = mhr_layout(false, dtype, B, H, T, D);
  if (!workspace || workspace_bytes < L.total) return REL_ERR_WORKSPACE;
  if (!aligned256(workspace)) return REL_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  const bool bf = dtype == REL_BF16;
  // rotated keys / mixed values once, in a pre-pass; the bf16 kernel rotates
  // its own query rows in registers
  void* q = (rope_cos && (!bf || D != 64)) ? w + L.q : nullptr;
  void* k = rope_cos ? w + L.k : nullptr;
  void* v = theta ? w + L.v : nullptr;
  if ((q || k || v) && rel::launch_mhr_prepare(bf ? 1 : 0, B, H, T, D, p1, p2, I, q, k, v,
                                               rope_cos, rope_sin, theta, pairing,
                                               s) != hipSuccess)
    return REL_ERR_HIP;
  const void* qe = q ? q : p1;
  const void* ke = k ? k : p2;
  const void* ve = v ? v : I;
  if (bf)
    return from_hip(rel::launch_fwd_bf16(
        B, H, T, D, static_cast<const uint16_t*>(qe), static_cast<const uint16_t*>(ke),
        static_cast<const uint16_t*>(ve), static_cast<uint16_t*>(y), lse, gate, scale, tau_s,
        lam, s, q ? nullptr : rope_cos, q ? nullptr : rope_sin));
  return from_hip(rel::launch_fwd_f32(B, H, T, D, static_cast<const float*>(qe),
                                      static_cast<const float*>(ke), static_cast<const float*>(ve),
                                      static_cast<float*>(y), lse, gate, scale, tau_s, lam, s));
}

size_t relation_mhr_bwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D) {
  if (check_dtype_dim_bwd(dtype, D) != REL_OK || check_shape(B, H, T, D) != REL_OK) return 0;
  return mhr_layout(true, dtype, B, H, T, D).total;
}

relation_status relation_mhr_bwd(relation_dtype dtype, int B, int H, int T, int D, const void* p1,
                                 const void* p2, const void* I, const float* rope_cos,
                                 const float* rope_sin, const float* theta, int pairing,
                                 const void* y, const void* dy, const float* lse, void* dp1,
                                 void* dp2, void* dI, float* dlambda, float* dtheta,
                                 const void* fwd_workspace, void* workspace,
                                 size_t workspace_bytes, float scale, float tau_s, float lambda,
                                 const float* lambda_dev, void* stream) {
  if (!p1 || !p2 || !I || !y || !dy || !lse || !dp1 || !dp2 || !dI) return REL_ERR_NULL;
  relation_status st = check_dtype_dim_bwd(dtype, D);
  if (st != REL_OK) return st;
  if ((st = check_shape(B, H, T, D)) != REL_OK) return st;
  if ((st = check_params(scale, tau_s, lambda)) != REL_OK) return st;
  if ((st = check_mhr(H, rope_cos, rope_sin, theta, pairing)) != REL_OK) return st;
  if (!aligned16(p1) || !aligned16(p2) || !aligned16(I) || !aligned16(y) || !aligned16(dy) ||
      !aligned4(lse) || !aligned16(dp1) || !aligned16(dp2) || !aligned16(dI) ||
      (dlambda && !aligned4(dlambda)) || (dtheta && !aligned4(dtheta)) ||
      (lambda_dev && !aligned4(lambda_dev)))
    return REL_ERR_ALIGN;
  const rel::Lam lam(lambda, lambda_dev);
  const MhrLayout L = mhr_layout(true, dtype, B, H, T, D);
  if (!workspace || workspace_bytes < L.total) return REL_ERR_WORKSPACE;
  if (!aligned256(workspace) || (fwd_workspace && !aligned256(fwd_workspace))) return REL_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  // the maps' outputs: formed here, or read from the forward's workspace
  // (which holds k and v, and q too where the forward does not rotate its
  // queries in registers)
  const MhrLayout F = mhr_layout(false, dtype, B, H, T, D);
  const char* fw = static_cast<const char*>(fwd_workspace);
  const bool fwd_q = fw && (dtype == REL_F32 || D != 64);
  void* q = rope_cos ? (fwd_q ? const_cast<char*>(fw) + F.q : w + L.q) : nullptr;
  void* k = rope_cos ? (fw ? const_cast<char*>(fw) + F.k : w + L.k) : nullptr;
  void* v = theta ? (fw ? const_cast<char*>(fw) + F.v : w + L.v) : nullptr;
  float* part = reinterpret_cast<float*>(w + L.part);
  const float* th = theta;
  float* dth = theta ? dtheta : nullptr;
  const int dcode = dtype == REL_BF16 ? 1 : 0;
  void* q_out = fwd_q ? nullptr : q;
  void* k_out = fw ? nullptr : k;
  void* v_out = fw ? nullptr : v;
  if ((q_out || k_out || v_out) &&
      rel::launch_mhr_prepare(dcode, B, H, T, D, p1, p2, I, q_out, k_out, v_out, rope_cos,
                              rope_sin, th, pairing, s) != hipSuccess)
    return REL_ERR_HIP;
  if (!q) q = const_cast<void*>(p1);
  if (!k) k = const_cast<void*>(p2);
  if (!v) v = const_cast<void*>(I);
  if (dtype == REL_F32) {
    // the plain backward writes dq, dk, dv of the rotated / mixed tensors into
    // the outputs; the transposes then run in place
    if (rel::launch_bwd_f32(B, H, T, D, static_cast<const float*>(q),
                            static_cast<const float*>(k), static_cast<const float*>(v),
                            static_cast<const float*>(y), static_cast<const float*>(dy), lse,
                            static_cast<float*>(dp1), static_cast<float*>(dp2),
                            static_cast<float*>(dI), dlambda, w + L.bwd, scale, tau_s, lam,
                            s) != hipSuccess)
      return REL_ERR_HIP;
    return from_hip(rel::launch_mhr_post(0, B, H, T, D, static_cast<const float*>(dp1), 1.0f,
                                         static_cast<const float*>(dp2),
                                         static_cast<const float*>(dI), v, dp1, dp2, dI, dth,
                                         part, rope_cos, rope_sin, th, pairing, s));
  }
  // At D = 64 the backward applies RoPE^T to dK itself and writes dp2; dV
  // (Givens pairs span two heads) and dQ (an accumulator until the end) stay
  // fp32 for the transpose passes, which also reduce dL/dlambda.
  const bool fuse_dk = D == 64 && rope_cos != nullptr;
  float* dk32 = fuse_dk ? nullptr : reinterpret_cast<float*>(w + L.dk32);
  float* dv32 = reinterpret_cast<float*>(w + L.dv32);
  if (rel::launch_bwd_bf16(B, H, T, D, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                           static_cast<const uint16_t*>(y), static_cast<const uint16_t*>(dy), lse,
                           static_cast<uint16_t*>(dp1), static_cast<uint16_t*>(dp2),
                           static_cast<uint16_t*>(dI), dlambda, w + L.bwd, scale, tau_s, lam,
                           s, dk32, dv32, fuse_dk ? rope_cos : nullptr,
                           fuse_dk ? rope_sin : nullptr) != hipSuccess)
    return REL_ERR_HIP;
  const rel::BwdWorkspace bl = rel::bwd_workspace_layout(1, B, H, T, D);
  const float* dq_acc = reinterpret_cast<const float*>(w + L.bwd + bl.off_dq);
  const float* dl_part = reinterpret_cast<const float*>(w + L.bwd + bl.off_part);
  return from_hip(rel::launch_mhr_post(1, B, H, T, D, dq_acc, scale, dk32, dv32, v, dp1, dp2, dI,
                                       dth, part, rope_cos, rope_sin, th, pairing, s,
                                       dlambda ? dl_part : nullptr, bl.npart, dlambda));
}

relation_status relation_linear_fwd(relation_dtype dtype, int B, int H, int T, int D,
                                    const void* p1, const void* p2, const void* I,
                                    const float* g, const float* rope_cos, const float* rope_sin,
                                    const float* state_in, void* y, float* state_out,
                                    float* states, float scale, float tau_s, void* stream) {
  if (!p1 || !p2 || !I || !g || !y) return REL_ERR_NULL;
  if (!rope_cos != !rope_sin) return REL_ERR_NULL;
  if (dtype != REL_BF16 || D != 64) return REL_ERR_UNSUPPORTED;
  relation_status st = check_shape(B, H, T, D);
  if (st != REL_OK) return st;
  if ((st = check_params(scale, tau_s, 0.f)) != REL_OK) return st;
  if (!aligned16(p1) || !aligned16(p2) || !aligned16(I) || !aligned16(g) || !aligned16(y) ||
      (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) ||
      (state_in && !aligned4(state_in)) || (state_out && !aligned4(state_out)) ||
      (states && !aligned16(states)))
    return REL_ERR_ALIGN;
  return from_hip(rel::launch_linear_fwd(
      B, H, T, static_cast<const uint16_t*>(p1), static_cast<const uint16_t*>(p2),
      static_cast<const uint16_t*>(I), g, rope_cos, rope_sin, state_in, static_cast<uint16_t*>(y),
      state_out, states, scale, tau_s, static_cast<hipStream_t>(stream)));
}

size_t relation_linear_states_bytes(relation_dtype dtype, int B, int H, int T, int D) {
  if (dtype != REL_BF16 || D != 64 || check_shape(B, H, T, D) != REL_OK) return 0;
  return rel::linear_states_bytes(B, H, T);
}

size_t relation_linear_bwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D) {
  if (dtype != REL_BF16 || D != 64 || check_shape(B, H, T, D) != REL_OK) return 0;
  return rel::linear_bwd_workspace_bytes(B, H, T, false);
}

size_t relation_linear_bwd_reuse_workspace_bytes(relation_dtype dtype, int B, int H, int T,
                                                 int D) {
  if (dtype != REL_BF16 || D != 64 || check_shape(B, H, T, D) != REL_OK) return 0;
  return rel::linear_bwd_workspace_bytes(B, H, T, true);
}

relation_status relation_linear_bwd(relation_dtype dtype, int B, int H, int T, int D,
                                    const void* p1, const void* p2, const void* I,
                                    const float* g, const float* rope_cos, const float* rope_sin,
                                    const float* state_in, const void* dy,
                                    const float* dstate_out, void* dp1, void* dp2, void* dI,
                                    float* dg, float* dstate_in, const float* fwd_states,
                                    void* workspace, size_t workspace_bytes, float scale,
                                    float tau_s, void* stream) {
  if (!p1 || !p2 || !I || !g || !dy || !dp1 || !dp2 || !dI || !dg) return REL_ERR_NULL;
  if (!rope_cos != !rope_sin) return REL_ERR_NULL;
  if (dtype != REL_BF16 || D != 64) return REL_ERR_UNSUPPORTED;
  relation_status st = check_shape(B, H, T, D);
  if (st != REL_OK) return st;
  if ((st = check_params(scale, tau_s, 0.f)) != REL_OK) return st;
  if (!aligned16(p1) || !aligned16(p2) || !aligned16(I) || !aligned16(g) || !aligned16(dy) ||
      !aligned16(dp1) || !aligned16(dp2) || !aligned16(dI) || !aligned16(dg) ||
      (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) ||
      (state_in && !aligned4(state_in)) || (dstate_out && !aligned4(dstate_out)) ||
      (dstate_in && !aligned4(dstate_in)) || (fwd_states && !aligned16(fwd_states)))
    return REL_ERR_ALIGN;
  const size_t need = rel::linear_bwd_workspace_bytes(B, H, T, fwd_states != nullptr);
  if (!workspace || workspace_bytes < need) return REL_ERR_WORKSPACE;
  if (!aligned256(workspace)) return REL_ERR_ALIGN;
  return from_hip(rel::launch_linear_bwd(
      B, H, T, static_cast<const uint16_t*>(p1), static_cast<const uint16_t*>(p2),
      static_cast<const uint16_t*>(I), g, rope_cos, rope_sin, state_in,
      static_cast<const uint16_t*>(dy), dstate_out, static_cast<uint16_t*>(dp1),
      static_cast<uint16_t*>(dp2), static_cast<uint16_t*>(dI), dg, dstate_in, fwd_states,
      static_cast<float*>(workspace), scale, tau_s, static_cast<hipStream_t>(stream)));
}

relation_status relation_linear_step(relation_dtype dtype, int B, int H, int D, const void* p1,
                                     const void* p2, const void* I, const float* g,
                                     const float* rope_cos, const float* rope_sin, float* state,
                                     void* y, float scale, float tau_s, void* stream) {
  if (!p1 || !p2 || !I || !g || !state || !y) return REL_ERR_NULL;
  if (!rope_cos != !rope_sin) return REL_ERR_NULL;
  if (dtype != REL_BF16 || D != 64) return REL_ERR_UNSUPPORTED;
  relation_status st = check_shape(B, H, 1, D);
  if (st != REL_OK) return st;
  if ((st = check_params(scale, tau_s, 0.f)) != REL_OK) return st;
  if (!aligned4(p1) || !aligned4(p2) || !aligned4(I) || !aligned4(g) || !aligned4(y) ||
      !aligned4(state) || (rope_cos && (!aligned4(rope_cos) || !aligned4(rope_sin))))
    return REL_ERR_ALIGN;
  return from_hip(rel::launch_linear_step(
      B, H, static_cast<const uint16_t*>(p1), static_cast<const uint16_t*>(p2),
      static_cast<const uint16_t*>(I), g, rope_cos, rope_sin, state, static_cast<uint16_t*>(y),
      scale, tau_s, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
