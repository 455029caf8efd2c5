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
  int64_t cus;  // compute units of the current device (sizes the dispatch choices)
  void* workspace;  // split-KV partials (fa_launch_fwd_splitkv only)
  // packed variable-length batches (fa_launch_fwd_varlen only): BH = B*H,
  // Nq = longest sequence's query count, offsets on the device
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int64_t H = 0;
  int64_t total_q = 0;
  int64_t total_k = 0;
};

// Enqueues the forward pass.  Arguments are already validated.  Returns 0 on
// success, otherwise the HIP error code of the first launch that failed (the
// launches' own status: an error the caller's earlier HIP work left pending
// is neither reported nor cleared).
int fa_launch_fwd(const FaLaunch& a);

// Split-KV forward (16-bit dtypes): nsplit key ranges of split_len keys
// (nsplit = ceil(Nk / split_len)) write fp32 partials to a.workspace
// (nsplit * BH * Nq * (D + 1) floats), then a merge kernel writes o and lse.
int fa_launch_fwd_splitkv(const FaLaunch& a, int nsplit, int split_len);

// Device address of the library's static split-KV scratch
// (FA_STATIC_SCRATCH_BYTES) on the current device, looked up once per device.
// Returns 0, or the HIP error of the lookup.
int fa_static_scratch(void** addr);

// Packed variable-length forward (16-bit dtypes): q, o [H, total_q, D];
// k, v [H, total_k, D]; lse [H, total_q]; per-sequence offsets cu_q, cu_k.
int fa_launch_fwd_varlen(const FaLaunch& a);

// The D = 256 launchers of the three forward entry points above (a unit of
// their own; sl2 = scale * log2(e)).
int fa_launch_fwd_d256(const FaLaunch& a, float sl2);
int fa_launch_fwd_splitkv_d256(const FaLaunch& a, float sl2, int nsplit, int split_len);
int fa_launch_fwd_varlen_d256(const FaLaunch& a, float sl2);

struct FaBwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;  // 2 * BH * Nq floats: lse * log2(e), then delta
  int64_t BH;
  int64_t Nq;
  int64_t Nk;
  int D;
  int causal;
  int dtype;  // fa_dtype
  double scale;
  void* stream;
  int64_t cus;  // compute units of the current device
  // Packed sequences (fa_bwd_varlen), NULL otherwise: q, o, dout, dq are
  // [H, total_q, D], k, v, dk, dv [H, total_k, D], lse and the workspace
  // [H, total_q]; BH = B*H, Nq / Nk the longest sequence's counts.
  const int* cu_q = nullptr;
  const int* cu_k = nullptr;
  int64_t H = 0;
  int64_t total_q = 0;
  int64_t total_k = 0;
};

// Enqueues the backward pass (three kernels).  Arguments are already
// validated.  Returns 0 on success, otherwise the HIP error code.
int fa_launch_bwd(const FaBwdLaunch& a);

// The D = 32 and D = 64 backward launcher (a unit of its own; sl2 = scale *
// log2(e)), called by fa_launch_bwd.
int fa_launch_bwd_small_d(const FaBwdLaunch& a, float sl2, float scale);

// The fp32 backward launcher (D in {32, 64, 128}; its own unit), called by
// fa_launch_bwd.
int fa_launch_bwd32(const FaBwdLaunch& a, float sl2, float scale);
