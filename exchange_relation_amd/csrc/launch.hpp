// Internal host-side launchers, one per kernel family. Arguments are already
// validated by relation_api.cpp; every launcher only enqueues work on
// `stream` and returns the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rel {

// Forward, fp32 storage and arithmetic (VALU), D in {32, 64}.
hipError_t launch_fwd_f32(int B, int H, int T, int D, const float* q, const float* k,
                          const float* v, float* y, float* lse, float* gate, float scale,
                          float tau, float lam, hipStream_t stream);

// Forward, bf16 storage, bf16 MFMA contractions with fp32 accumulation, D = 64.
hipError_t launch_fwd_bf16(int B, int H, int T, int D, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, uint16_t* y, float* lse, float* gate, float scale,
                           float tau, float lam, hipStream_t stream);

// Backward. Workspace layout and size are owned by the launcher.
size_t bwd_workspace_bytes(int dtype, int B, int H, int T, int D);
hipError_t launch_bwd_f32(int B, int H, int T, int D, const float* q, const float* k,
                          const float* v, const float* y, const float* dy, const float* lse,
                          float* dq, float* dk, float* dv, float* dlambda, void* ws, float scale,
                          float tau, float lam, hipStream_t stream);
hipError_t launch_bwd_bf16(int B, int H, int T, int D, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* y, const uint16_t* dy,
                           const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                           float* dlambda, void* ws, float scale, float tau, float lam,
                           hipStream_t stream);

// Relation Cache decode (one step). dtype 0 = fp32, 1 = bf16. n_hist_dev
// NULL: every sequence has n_hist slots of history; otherwise sequence b has
// n_hist_dev[b] (device ints) and n_hist is their upper bound.
size_t decode_workspace_bytes(int dtype, int B, int H, int D, int capacity);
hipError_t launch_decode(int dtype, int B, int H, int D, const void* q, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache, int capacity,
                         int n_hist, const int* n_hist_dev, void* y, float* gate, void* ws,
                         float scale, float tau, float lam, hipStream_t stream);

}  // namespace rel
