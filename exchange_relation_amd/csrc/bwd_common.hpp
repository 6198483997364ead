// Backward workspace layout and the shared preprocess launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace rel {

struct BwdWorkspace {
  size_t off_dr;    // float [B*H*T]: Dr_i = dY_i . Y_i
  size_t off_part;  // float [npart]: per-block partials of dL/dlambda
  size_t off_dq;    // float [B*H*T*D]: fp32 dq accumulator (bf16 path only)
  size_t total;
  int npart;
};

BwdWorkspace bwd_workspace_layout(int dtype, int B, int H, int T, int D);

// Dr rows and the dL/dlambda partials; also reduces the partials into
// *dlambda when dlambda != NULL (else the caller reduces them). dtype 0 =
// fp32, 1 = bf16.
hipError_t launch_bwd_pre(int dtype, int T, int D, const void* q, const void* k,
                          const void* v, const void* y, const void* dy, const float* lse,
                          float* dlambda, const BwdWorkspace& w, char* ws, float scale, float tau,
                          hipStream_t stream);

}  // namespace rel
