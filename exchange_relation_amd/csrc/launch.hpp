// Internal host-side launchers, one per kernel family. Arguments are already
// validated by relation_api.cpp; every launcher only enqueues work on
// `stream` and returns the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rel {

// The count correction's lambda (Sec. 3.1): a value, or a device fp32 scalar
// read by the kernels at run time (p non-NULL; v is then unused), so that a
// learnable lambda kept on the device needs no host synchronisation.
struct Lam {
  float v;
  const float* p;
  __host__ __device__ Lam(float x = 0.f, const float* ptr = nullptr) : v(x), p(ptr) {}
  __device__ __forceinline__ float get() const { return p ? *p : v; }
};

// Forward, fp32 storage and arithmetic (VALU), D in {32, 64}.
hipError_t launch_fwd_f32(int B, int H, int T, int D, const float* q, const float* k,
                          const float* v, float* y, float* lse, float* gate, float scale,
                          float tau, Lam lam, hipStream_t stream);

// Forward, bf16 storage, bf16 MFMA contractions with fp32 accumulation,
// D in {48, 64, 80}. rope_cos / rope_sin ([T, D/2] fp32, or NULL; D = 64
// only): RoPE of q fused into the Q fragment load (Multi-Head Relation; k and v come in already rotated /
// mixed).
// bf16 forward. ws (optional, fwd_bf16_workspace_bytes) lets a grid too
// small to fill the chip split its long query blocks over keys.
size_t fwd_bf16_workspace_bytes(int B, int H, int T, int D);
hipError_t launch_fwd_bf16(int B, int H, int T, int D, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, uint16_t* y, float* lse, float* gate, float scale,
                           float tau, Lam lam, hipStream_t stream,
                           const float* rope_cos = nullptr, const float* rope_sin = nullptr,
                           float* ws = nullptr, size_t ws_bytes = 0);

// Backward. Workspace layout and size are owned by the launcher. ev0 / ev1
// (either may be null) are recorded on the stream right before and right
// after the main backward kernel(s), without the preprocess and the dq
// finalize, so that a caller can time that part alone.
size_t bwd_workspace_bytes(int dtype, int B, int H, int T, int D);
hipError_t launch_bwd_f32(int B, int H, int T, int D, const float* q, const float* k,
                          const float* v, const float* y, const float* dy, const float* lse,
                          float* dq, float* dk, float* dv, float* dlambda, void* ws, float scale,
                          float tau, Lam lam, hipStream_t stream, hipEvent_t ev0 = nullptr,
                          hipEvent_t ev1 = nullptr);
// bf16 D in {48, 64, 80} (48 runs in the 64-wide tiles with zero columns, 80
// in the wider layout of bwd80.hip).
// dk32 / dv32 non-NULL: dk (scaled) and dv go there in fp32, and dq is left
// unscaled in the workspace accumulator (bwd_workspace_layout(...).off_dq).
hipError_t launch_bwd_bf16(int B, int H, int T, int D, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* y, const uint16_t* dy,
                           const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                           float* dlambda, void* ws, float scale, float tau, Lam lam,
                           hipStream_t stream, float* dk32 = nullptr,
                           float* dv32 = nullptr, const float* rope_cos = nullptr,
                           const float* rope_sin = nullptr, hipEvent_t ev0 = nullptr,
                           hipEvent_t ev1 = nullptr);

// The D = 80 backward kernel (bwd80.hip), after the shared preprocess; dq
// accumulates into dq_acc (fp32, unscaled) as for the other widths.
hipError_t launch_bwd80_kernel(int B, int H, int T, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const uint16_t* dy, const float* lse,
                               const float* Dr, float* dq_acc, uint16_t* dk, uint16_t* dv,
                               float scale, float tau, Lam lam, hipStream_t stream, float* dk32,
                               float* dv32);

// Relation Cache prefill (bf16, D in {48, 64, 80}): appends m new tokens per (b, h) at
// slot n_b (n_hist_dev[b] on the device, or the uniform n_hist when NULL;
// with the device array n_hist is their upper bound) and computes their rows
// against cache rows 0 .. n_b + m - 1.
size_t prefill_workspace_bytes(int B, int H, int D, int m, int n_hist, bool per_sequence);
hipError_t launch_prefill_bf16(int B, int H, int D, int m, const uint16_t* q, const uint16_t* k_new,
                               const uint16_t* v_new, uint16_t* k_cache, uint16_t* v_cache,
                               int capacity, const int* n_hist_dev, int n_hist, uint16_t* y,
                               float* lse, float* gate, float scale, float tau, float lam,
                               hipStream_t stream, float* ws = nullptr, size_t ws_bytes = 0);

// Relation Cache decode (one step). dtype 0 = fp32, 1 = bf16. n_hist_dev
// NULL: every sequence has n_hist slots of history; otherwise sequence b has
// n_hist_dev[b] (device ints) and n_hist is their upper bound.
size_t decode_workspace_bytes(int dtype, int B, int H, int D, int capacity);
hipError_t launch_decode(int dtype, int B, int H, int D, const void* q, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache, int capacity,
                         int n_hist, const int* n_hist_dev, void* y, float* gate, void* ws,
                         float scale, float tau, float lam, hipStream_t stream);

// Workspace bytes the uniform step actually uses at history n_hist (0 when
// it needs none: n_hist = 0, or one workgroup per head).
size_t decode_uniform_need_bytes(int B, int H, int D, int n_hist);
// The same uniform decode step with its workspace in the library's static
// per-device array of decode_scratch_bytes() bytes (callers check
// decode_uniform_need_bytes against it first); allocates nothing.
size_t decode_scratch_bytes();
hipError_t launch_decode_noalloc(int dtype, int B, int H, int D, const void* q,
                                 const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, int capacity, int n_hist, void* y, float* gate,
                                 float scale, float tau, float lam, hipStream_t stream);

// Multi-Head Relation passes (mhr.hip): RoPE of p1 / p2 into q / k and the
// Givens mixing of vi into v (an output pointer NULL: not produced); and the
// transposes of both on fp32 gradients (dq scaled by dq_scale), rounded once
// into dp1, dp2, dI, with dtheta [H/2] reduced from `part` (mhr_part_floats
// floats). dtype 0 = fp32, 1 = bf16.
size_t mhr_part_floats(int B, int H, int T, int D);
hipError_t launch_mhr_prepare(int dtype, int B, int H, int T, int D, const void* p1,
                              const void* p2, const void* vi, void* q, void* k, void* v,
                              const float* rope_cos, const float* rope_sin, const float* theta,
                              int pairing, hipStream_t stream);
// dk NULL: dp2 is already written (the bf16 backward's fused RoPE^T).
// dl_part (npart values, or NULL): the backward's dL/dlambda partials, summed
// in a fixed order into *dlambda by the dq transpose pass.
hipError_t launch_mhr_post(int dtype, int B, int H, int T, int D, const float* dq, float dq_scale,
                           const float* dk, const float* dv, const void* vmix, void* dp1,
                           void* dp2, void* dI, float* dtheta, float* part,
                           const float* rope_cos, const float* rope_sin, const float* theta,
                           int pairing, hipStream_t stream, const float* dl_part = nullptr,
                           int dl_npart = 0, float* dlambda = nullptr);

// Linear Relation (linear.hip), bf16, D = 64. g = log retention (fp32, same
// shape as p1). rope tables [T, D/2] or NULL; state_in / state_out [B, H, D, D]
// fp32 or NULL; states (or NULL): the state before every chunk of
// linear_chunk_rows() tokens, then the final state, [B, H, nchunks + 1, D, D]
// fp32.
int linear_chunk_rows();
hipError_t launch_linear_fwd(int B, int H, int T, const uint16_t* p1, const uint16_t* p2,
                             const uint16_t* iv, const float* g, const float* rope_cos,
                             const float* rope_sin, const float* state_in, uint16_t* y,
                             float* state_out, float* states, float scale, float tau,
                             hipStream_t stream);
// The forward's state pass: the state before every chunk, then the final
// state, into states [B, H, nchunks + 1, D, D] fp32 (no outputs).
hipError_t launch_linear_fwd_states(int B, int H, int T, const uint16_t* p1, const uint16_t* p2,
                                    const uint16_t* iv, const float* g, const float* rope_cos,
                                    const float* rope_sin, const float* state_in, float* states,
                                    float scale, float tau, hipStream_t stream);
// Backward: gradients of relation_linear_fwd. ws: linear_bwd_workspace_bytes()
// (the states of the state pass, then the gradient of the state after every
// chunk; with fwd_states, only the state gradients); dstate_out, the gradient
// of the final state, or NULL; dstate_in (out) or NULL.
size_t linear_bwd_workspace_bytes(int B, int H, int T, bool with_fwd_states);
// Bytes of the per-chunk states ([B, H, nchunks + 1, D, D] fp32).
size_t linear_states_bytes(int B, int H, int T);
hipError_t launch_linear_bwd(int B, int H, int T, const uint16_t* p1, const uint16_t* p2,
                             const uint16_t* iv, const float* g, const float* rope_cos,
                             const float* rope_sin, const float* state_in, const uint16_t* dy,
                             const float* dstate_out, uint16_t* dp1, uint16_t* dp2, uint16_t* dI,
                             float* dg, float* dstate_in, const float* fwd_states, float* ws,
                             float scale, float tau, hipStream_t stream);
// One token per head; state [B, H, D, D] fp32 updated in place; rope tables
// are the [D/2] rows of the token's position, or NULL.
hipError_t launch_linear_step(int B, int H, const uint16_t* p1, const uint16_t* p2,
                              const uint16_t* iv, const float* g, const float* rope_cos,
                              const float* rope_sin, float* state, uint16_t* y, float scale,
                              float tau, hipStream_t stream);

}  // namespace rel
