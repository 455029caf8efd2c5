// C ABI of the exact tiled attention forward pass: argument validation
// (before any HIP call) and dispatch to the gfx950 kernels.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

// Compute units of the current device, read on every call: the workgroup
// shapes and the automatic key-range count are chosen against it.  0 when
// the runtime cannot say (no device).
int64_t device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
  return n;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Half-open byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  if (na <= 0 || nb <= 0) return false;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int dtype, bool* empty) {
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || D < 0) return FA_ERR_SHAPE;
  if (D != 32 && D != 64 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
  // fp32 at D = 256 would spill registers (its Q fragment, O and staged K/V
  // exceed one wave's 512); that head dimension runs the 16-bit kernel only.
  if (D == 256 && dtype == FA_DTYPE_FP32) return FA_ERR_HEAD_DIM;
  int64_t BH, rows, qel, kel;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, Nq, &rows) || !mul_ok(rows, D, &qel)) return FA_ERR_SHAPE;
  *empty = (rows == 0);
  if (*empty) return FA_OK;
  if (Nk < 1) return FA_ERR_SHAPE;  // a query row with no key has no softmax
  if (!mul_ok(BH, Nk, &kel) || !mul_ok(kel, D, &kel)) return FA_ERR_SHAPE;
  // Kernel index arithmetic: per-head row counts and the grid are 32-bit;
  // element offsets are 64-bit.
  const int64_t nqt = (Nq + 127) / 128;
  if (Nq > INT32_MAX / 2 || Nk > INT32_MAX / 2 || BH > INT32_MAX) return FA_ERR_SHAPE;
  int64_t grid;
  if (!mul_ok(BH, nqt, &grid) || grid > INT32_MAX) return FA_ERR_SHAPE;
  const int64_t esz = (dtype == FA_DTYPE_FP32) ? 4 : 2;
  int64_t qbytes, kbytes, lbytes;
  if (!mul_ok(qel, esz, &qbytes) || !mul_ok(kel, esz, &kbytes) || !mul_ok(rows, 4, &lbytes))
    return FA_ERR_SHAPE;
  // The kernels address one head through 32-bit buffer offsets, which reach
  // up to 256 rows past the end (a partial last Q tile, padding K/V tiles).
  if ((Nq + 256) * D * esz > INT32_MAX || (Nk + 256) * D * esz > INT32_MAX) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) ||
      overlaps(o, qbytes, v, kbytes) || overlaps(lse, lbytes, q, qbytes) ||
      overlaps(lse, lbytes, k, kbytes) || overlaps(lse, lbytes, v, kbytes) ||
      overlaps(o, qbytes, lse, lbytes))
    return FA_ERR_ALIAS;
  return FA_OK;
}

// The softmax scale a call asked for: FA_DEFAULT_SCALE (0) selects
// 1/sqrt(D), the scale every page divides the scores by; any other value
// must be finite and positive, and the kernels work in the log2 domain with
// scale * log2(e) as one fp32 factor, which must be a normal float.  False
// for an invalid scale.
bool resolve_scale(double requested, int64_t D, double* scale) {
  if (requested == FA_DEFAULT_SCALE) {
    *scale = 1.0 / sqrt((double)(D > 0 ? D : 1));
    return true;
  }
  if (!(requested > 0.0) || !isfinite(requested)) return false;
  const float sl2 = (float)(requested * 1.4426950408889634074);
  if (!isnormal(sl2) || !isfinite(sl2)) return false;
  *scale = requested;
  return true;
}

int fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
        int64_t Nq, int64_t Nk, int64_t D, const double* scale, int causal, int dtype, void* stream) {
  bool empty = false;
  const int st = validate(q, k, v, o, lse, B, H, Nq, Nk, D, dtype, &empty);
  if (st != FA_OK) return st;
  double sc;
  if (!resolve_scale(scale ? *scale : FA_DEFAULT_SCALE, D, &sc)) return FA_ERR_SCALE;
  if (empty) return FA_OK;
  FaLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = B * H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.D = (int)D;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.scale = sc;
  a.stream = stream;
  a.workspace = nullptr;
  a.cus = device_cus();
  if (a.cus <= 0) return FA_ERR_HIP;
  return fa_launch_fwd(a) == 0 ? FA_OK : FA_ERR_HIP;
}

constexpr int64_t kMaxSplits = 1024;

// Key ranges of the split-KV forward.  Automatic count: the one that
// minimises (waves of workgroups over the device's `cus` CUs) x (keys per workgroup),
// the fewest ranges among equals (each range adds partials to merge), with
// at least 256 keys a range.  A workgroup takes a 256-row Q tile and, at
// D = 128, an LDS ring that leaves room for one workgroup per CU, so a
// second, partial wave of workgroups costs a whole range's time (measured on
// the decoding shapes: 16 ranges of 32 heads, 512 workgroups, ran 6% slower
// than 8 ranges, 256 workgroups).  Range length: ceil(Nk / splits) rounded
// up to whole 64-key tiles; `n` is the number of non-empty ranges it gives.
void split_plan(int64_t BH, int64_t Nq, int64_t Nk, int64_t splits, int64_t cus, int64_t* len, int64_t* n) {
  if (splits <= 0) {
    const int64_t wgs = BH * ((Nq + 255) / 256);
    int64_t most = Nk / 256;
    if (most > kMaxSplits) most = kMaxSplits;
    splits = 1;
    int64_t best = -1;
    for (int64_t s = 1; s <= most && wgs > 0; ++s) {
      const int64_t waves = (wgs * s + cus - 1) / cus;
      const int64_t cost = waves * ((Nk + s - 1) / s);
      if (best < 0 || cost < best) {
        best = cost;
        splits = s;
      }
    }
  }
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits < 1) splits = 1;
  int64_t l = (Nk + splits - 1) / splits;
  l = (l + 63) / 64 * 64;
  if (l < 64) l = 64;
  *len = l;
  *n = Nk > 0 ? (Nk + l - 1) / l : 1;
}

// The CU count the automatic key-range count is planned against: the current
// device's, or the MI355X's 256 when no device answers (so that the
// workspace size can still be asked for without a GPU).
int64_t plan_cus() {
  const int64_t c = device_cus();
  return c > 0 ? c : 256;
}

}  // namespace

extern "C" int64_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                                                 int64_t num_splits) {
  int64_t BH, rows, per;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || D < 1 || num_splits < 0 || num_splits > kMaxSplits) return -1;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, Nq, &rows) || !mul_ok(rows, D + 1, &per) || !mul_ok(per, 4, &per))
    return -1;
  int64_t len, n;
  split_plan(BH, Nq, Nk, num_splits, plan_cus(), &len, &n);
  if (n <= 1) return 0;  // one range: the plain forward, no workspace
  int64_t bytes;
  if (!mul_ok(per, n, &bytes)) return -1;
  return bytes;
}

namespace {

// fa_fwd_splitkv and fa_fwd_splitkv_static: the partials go to the caller's
// workspace, or (use_static) to the library's static scratch.
int splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
            int64_t workspace_bytes, bool use_static, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
            double softmax_scale, int64_t num_splits, int causal, int dtype, void* stream) {
  bool empty = false;
  const int st = validate(q, k, v, o, lse, B, H, Nq, Nk, D, dtype, &empty);
  if (st != FA_OK) return st;
  double sc;
  if (!resolve_scale(softmax_scale, D, &sc)) return FA_ERR_SCALE;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_SHAPE;
  if (empty) return FA_OK;
  const int64_t BH = B * H, rows = BH * Nq;
  const int64_t cus = device_cus();
  int64_t len, n;
  split_plan(BH, Nq, Nk, num_splits, cus > 0 ? cus : 256, &len, &n);
  FaLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = BH;
  a.Nq = Nq;
  a.Nk = Nk;
  a.D = (int)D;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.scale = sc;
  a.stream = stream;
  a.workspace = nullptr;
  a.cus = cus;
  if (n <= 1) return cus > 0 && fa_launch_fwd(a) == 0 ? FA_OK : FA_ERR_HIP;
  // fp32 partials of one (range, head) are addressed with 32-bit offsets
  if ((Nq + 256) * (D * 4) > INT32_MAX) return FA_ERR_SHAPE;
  int64_t grid;  // Q tiles of 256 rows (16-bit) or 128 (fp32)
  if (!mul_ok(BH * ((Nq + 127) / 128), n, &grid) || grid > INT32_MAX || rows * (D / 4) / 256 >= INT32_MAX)
    return FA_ERR_SHAPE;
  const int64_t need = fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, num_splits);
  if (need < 0) return FA_ERR_SHAPE;
  if (use_static) {
    if (need > FA_STATIC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    if (cus <= 0 || fa_static_scratch(&workspace) != 0) return FA_ERR_HIP;
    a.workspace = workspace;
    return fa_launch_fwd_splitkv(a, (int)n, (int)len) == 0 ? FA_OK : FA_ERR_HIP;
  }
  if (!workspace) return FA_ERR_NULL;
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 15u) return FA_ERR_ALIGN;
  const int64_t esz = dtype == FA_DTYPE_FP32 ? 4 : 2;
  const int64_t qbytes = rows * D * esz, kbytes = BH * Nk * D * esz, lbytes = rows * 4;
  if (overlaps(workspace, need, q, qbytes) || overlaps(workspace, need, k, kbytes) ||
      overlaps(workspace, need, v, kbytes) || overlaps(workspace, need, o, qbytes) ||
      overlaps(workspace, need, lse, lbytes))
    return FA_ERR_ALIAS;
  a.workspace = workspace;
  if (cus <= 0) return FA_ERR_HIP;
  return fa_launch_fwd_splitkv(a, (int)n, (int)len) == 0 ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                              void* workspace, int64_t workspace_bytes, int64_t B, int64_t H, int64_t Nq,
                              int64_t Nk, int64_t D, double softmax_scale, int64_t num_splits, int causal,
                              int dtype, void* stream) {
  return splitkv(q, k, v, o, lse, workspace, workspace_bytes, false, B, H, Nq, Nk, D, softmax_scale, num_splits,
                 causal, dtype, stream);
}

extern "C" int fa_fwd_splitkv_static(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                                     double softmax_scale, int64_t num_splits, int causal, int dtype,
                                     void* stream) {
  return splitkv(q, k, v, o, lse, nullptr, 0, true, B, H, Nq, Nk, D, softmax_scale, num_splits, causal, dtype,
                 stream);
}

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                      int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal, int dtype,
                      void* stream) {
  return fwd(q, k, v, o, lse, B, H, Nq, Nk, D, nullptr, causal, dtype, stream);
}

extern "C" int fa_fwd_scaled(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                             double softmax_scale, int causal, int dtype, void* stream) {
  return fwd(q, k, v, o, lse, B, H, Nq, Nk, D, &softmax_scale, causal, dtype, stream);
}

extern "C" int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t B, int64_t H,
                             int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t D,
                             double softmax_scale, int causal, int dtype, void* stream) {
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || D < 0) return FA_ERR_SHAPE;
  if (D != 32 && D != 64 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
  if (D == 256 && dtype == FA_DTYPE_FP32) return FA_ERR_HEAD_DIM;
  double sc;
  if (!resolve_scale(softmax_scale, D, &sc)) return FA_ERR_SCALE;
  int64_t BH, qel, kel;
  if (!mul_ok(B, H, &BH) || !mul_ok(H, total_q, &qel) || !mul_ok(qel, D, &qel) || !mul_ok(H, total_k, &kel) ||
      !mul_ok(kel, D, &kel))
    return FA_ERR_SHAPE;
  if (BH == 0 || total_q == 0 || max_seqlen_q == 0) return FA_OK;  // no query row to compute
  if (max_seqlen_q > total_q || total_q > INT32_MAX / 2 || total_k > INT32_MAX / 2 || BH > INT32_MAX)
    return FA_ERR_SHAPE;
  const int64_t esz = dtype == FA_DTYPE_FP32 ? 4 : 2;
  // one head's packed rows are addressed with 32-bit offsets
  if ((total_q + 256) * D * esz > INT32_MAX || (total_k + 256) * D * esz > INT32_MAX) return FA_ERR_SHAPE;
  int64_t grid;
  if (!mul_ok((BH + 7) / 8 * 8, (max_seqlen_q + 127) / 128, &grid) || grid > INT32_MAX) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  if ((((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) ||
      (((uintptr_t)lse | (uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3u))
    return FA_ERR_ALIGN;
  const int64_t qbytes = qel * esz, kbytes = kel * esz, lbytes = H * total_q * 4, cbytes = (B + 1) * 4;
  const void* ins[5] = {q, k, v, cu_seqlens_q, cu_seqlens_k};
  const int64_t in_bytes[5] = {qbytes, kbytes, kbytes, cbytes, cbytes};
  for (int j = 0; j < 5; ++j)
    if (overlaps(o, qbytes, ins[j], in_bytes[j]) || overlaps(lse, lbytes, ins[j], in_bytes[j])) return FA_ERR_ALIAS;
  if (overlaps(o, qbytes, lse, lbytes)) return FA_ERR_ALIAS;
  FaLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = BH;
  a.Nq = max_seqlen_q;
  a.Nk = 0;
  a.D = (int)D;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.scale = sc;
  a.stream = stream;
  a.cus = device_cus();
  if (a.cus <= 0) return FA_ERR_HIP;
  a.workspace = nullptr;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.H = H;
  a.total_q = total_q;
  a.total_k = total_k;
  return fa_launch_fwd_varlen(a) == 0 ? FA_OK : FA_ERR_HIP;
}

extern "C" int64_t fa_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq) {
  int64_t BH, rows, bytes;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, Nq, &rows) || !mul_ok(rows, 8, &bytes)) return -1;
  return bytes;
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, void* workspace,
                      int64_t workspace_bytes, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                      double softmax_scale, int causal, int dtype, void* stream) {
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || D < 0) return FA_ERR_SHAPE;
  if (D != 32 && D != 64 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
  if (D == 256 && dtype == FA_DTYPE_FP32) return FA_ERR_HEAD_DIM;
  double sc;
  if (!resolve_scale(softmax_scale, D, &sc)) return FA_ERR_SCALE;
  int64_t BH, qel, kel;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, Nq, &qel) || !mul_ok(qel, D, &qel) || !mul_ok(BH, Nk, &kel) ||
      !mul_ok(kel, D, &kel))
    return FA_ERR_SHAPE;
  if (BH == 0 || (Nq == 0 && Nk == 0)) return FA_OK;  // nothing to write
  if (Nk == 0) return FA_ERR_SHAPE;  // query rows with no key have no softmax
  // Nq == 0 < Nk is valid: dK = dV = 0.
  if (Nq > INT32_MAX / 2 || Nk > INT32_MAX / 2 || BH > INT32_MAX) return FA_ERR_SHAPE;
  const int64_t esz = dtype == FA_DTYPE_FP32 ? 4 : 2;
  if ((Nq + 256) * D * esz > INT32_MAX || (Nk + 256) * D * esz > INT32_MAX) return FA_ERR_SHAPE;
  int64_t gq, gk;
  // dQ workgroups take 256 query rows (128 at D = 256 and for fp32), dK/dV
  // ones 128 keys; the statistics kernel takes D/8 (fp32: D/4) lanes a row
  if (!mul_ok(BH, (Nq + 127) / 128, &gq) || gq > INT32_MAX || !mul_ok(BH, (Nk + 127) / 128, &gk) ||
      gk > INT32_MAX || BH * Nq * (D / 4) / 256 >= INT32_MAX)
    return FA_ERR_SHAPE;
  const int64_t ws_need = fa_bwd_workspace_size(B, H, Nq);
  if (ws_need < 0) return FA_ERR_SHAPE;
  // the query-side buffers have zero size when Nq == 0 and may then be NULL
  if (!k || !v || !dk || !dv) return FA_ERR_NULL;
  if (Nq > 0 && (!q || !o || !lse || !dout || !dq || !workspace)) return FA_ERR_NULL;
  if (workspace_bytes < ws_need) return FA_ERR_WORKSPACE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace) & 15u)
    return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
  const int64_t qbytes = qel * esz, kbytes = kel * esz, lbytes = BH * Nq * 4;
  const void* ins[6] = {q, k, v, o, lse, dout};
  const int64_t in_bytes[6] = {qbytes, kbytes, kbytes, qbytes, lbytes, qbytes};
  void* outs[4] = {dq, dk, dv, workspace};
  const int64_t out_bytes[4] = {qbytes, kbytes, kbytes, ws_need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return FA_ERR_ALIAS;
  }
  FaBwdLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.workspace = workspace;
  a.BH = BH;
  a.Nq = Nq;
  a.Nk = Nk;
  a.D = (int)D;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.scale = sc;
  a.stream = stream;
  a.cus = device_cus();
  if (a.cus <= 0) return FA_ERR_HIP;
  return fa_launch_bwd(a) == 0 ? FA_OK : FA_ERR_HIP;
}

extern "C" int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, void* workspace, int64_t workspace_bytes, int64_t B,
                             int64_t H, int64_t total_q, int64_t total_k, int64_t max_seqlen_q,
                             int64_t max_seqlen_k, int64_t D, double softmax_scale, int causal, int dtype,
                             void* stream) {
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (B < 0 || H < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || D < 0)
    return FA_ERR_SHAPE;
  if (D != 32 && D != 64 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
  if (D == 256 && dtype == FA_DTYPE_FP32) return FA_ERR_HEAD_DIM;
  double sc;
  if (!resolve_scale(softmax_scale, D, &sc)) return FA_ERR_SCALE;
  int64_t BH, qel, kel;
  if (!mul_ok(B, H, &BH) || !mul_ok(H, total_q, &qel) || !mul_ok(qel, D, &qel) || !mul_ok(H, total_k, &kel) ||
      !mul_ok(kel, D, &kel))
    return FA_ERR_SHAPE;
  if (BH == 0 || (total_q == 0 && total_k == 0)) return FA_OK;  // nothing to write
  if (max_seqlen_q > total_q || max_seqlen_k > total_k || total_q > INT32_MAX / 2 || total_k > INT32_MAX / 2 ||
      BH > INT32_MAX)
    return FA_ERR_SHAPE;
  const int64_t esz = dtype == FA_DTYPE_FP32 ? 4 : 2;
  // one sequence's rows are addressed with 32-bit offsets
  if ((total_q + 256) * D * esz > INT32_MAX || (total_k + 256) * D * esz > INT32_MAX) return FA_ERR_SHAPE;
  int64_t gq, gk;
  if (!mul_ok(BH, (max_seqlen_q + 127) / 128, &gq) || gq > INT32_MAX ||
      !mul_ok(BH, (max_seqlen_k + 127) / 128, &gk) || gk > INT32_MAX || qel / 4 / 256 >= INT32_MAX)
    return FA_ERR_SHAPE;
  const int64_t ws_need = fa_bwd_workspace_size(1, H, total_q);
  if (ws_need < 0) return FA_ERR_SHAPE;
  // the buffers of an empty side have zero size and may then be NULL
  if (!cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  if (total_k > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULL;
  if (total_q > 0 && (!q || !o || !lse || !dout || !dq || !workspace)) return FA_ERR_NULL;
  if (workspace_bytes < ws_need) return FA_ERR_WORKSPACE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace) & 15u)
    return FA_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) & 3u) return FA_ERR_ALIGN;
  const int64_t qbytes = qel * esz, kbytes = kel * esz, lbytes = H * total_q * 4, cbytes = (B + 1) * 4;
  const void* ins[8] = {q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k};
  const int64_t in_bytes[8] = {qbytes, kbytes, kbytes, qbytes, lbytes, qbytes, cbytes, cbytes};
  void* outs[4] = {dq, dk, dv, workspace};
  const int64_t out_bytes[4] = {qbytes, kbytes, kbytes, ws_need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return FA_ERR_ALIAS;
  }
  FaBwdLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.workspace = workspace;
  a.BH = BH;
  a.Nq = max_seqlen_q;
  a.Nk = max_seqlen_k;
  a.D = (int)D;
  a.causal = causal != 0;
  a.dtype = dtype;
  a.scale = sc;
  a.stream = stream;
  a.cus = device_cus();
  if (a.cus <= 0) return FA_ERR_HIP;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.H = H;
  a.total_q = total_q;
  a.total_k = total_k;
  return fa_launch_bwd(a) == 0 ? FA_OK : FA_ERR_HIP;
}

extern "C" const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: negative, empty-key or too large shape";
    case FA_ERR_HEAD_DIM: return "FA_ERR_HEAD_DIM: head dimension must be 32, 64, 128 or 256 (256: 16-bit types only)";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype code";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: q/k/v/o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output overlaps an input or the other output";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported a launch error";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: softmax_scale must be a finite number > 0";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace smaller than the *_workspace_size() call returns";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the split-KV partials of this call exceed the library's static scratch "
             "(FA_STATIC_SCRATCH_BYTES = 32 MiB); use fa_fwd_splitkv with a workspace or fewer ranges";
    default: return "unknown fa_status code";
  }
}
