// Internal launch interface between the C ABI (fa_api.cpp) and the HIP
// kernels (fa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

struct FaLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t BH;  // B * H
  int64_t Nq;
  int64_t Nk;
  int D;
  int causal;
  int dtype;  // fa_dtype
  double scale;  // softmax scale applied to q.k (validated: finite, > 0)
  void* stream;
};

// Enqueues the forward pass.  Arguments are already validated.  Returns 0 on
// success, otherwise the HIP error code of the launch.
int fa_launch_fwd(const FaLaunch& a);
