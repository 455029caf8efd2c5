// Exact attention backward for gfx950, fp32 inputs, D in {32, 64, 128}.
//
// The same recomputation as the 16-bit backward ("Building a FlashAttention-2
// Forward Kernel in Pure NumPy", Extending It): the forward's LSE is kept,
// every probability is recomputed as P = exp(s - LSE), and with
// delta_i = sum_d dO[i,d] O[i,d]
//
//   dP = dO V^T,  dS = P * (dP - delta),  dV = P^T dO,
//   dQ = scale dS K,  dK = scale dS^T Q,
//
// here with P and dS kept in fp32 (no rounding between the products) and
// v_mfma_f32_32x32x2_f32, the operand layout of the fp32 forward kernel:
// tiles are staged through registers into a double-buffered LDS stage with
// rows padded to D+4 floats, and a lane holds half of a row fragment (the
// MFMA step c pairs column c of the low half-wave with column D/2 + c of
// the high one).  Three kernels, no atomics, deterministic:
//  * bwd32_prep: delta and LSE * log2(e) per query row (the workspace);
//  * bwd32_dq: 4 waves x 32 query rows; K/V tiles of 64 keys (32 at D = 128);
//    per tile S^T = K Q^T and dP^T = V dO^T with the wave's Q and dO rows in
//    registers, P and dS, then dQ^T += K^T dS^T;
//  * bwd32_dkdv: 4 waves x 32 keys; Q/dO tiles of 64 rows (32 at D = 128)
//    with their LSE and delta; per tile S = Q K^T and dP = dO V^T with the
//    wave's K and V rows in registers (keys along the MFMA N dimension), then
//    dV^T += dO^T P and dK^T += Q^T dS.
// The products are recomputed in both big kernels (seven tile products).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace {

constexpr float kLog2e32 = 1.4426950408889634074f;
constexpr int kThreads32 = 256;  // 4 waves

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// delta = sum_d dO[d] O[d] and lse2 = LSE log2(e) per query row; D/4 lanes
// per row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(256) void bwd32_prep(const float* __restrict__ O, const float* __restrict__ dO,
                                                  const float* __restrict__ lse, float* __restrict__ lse2,
                                                  float* __restrict__ delta, int64_t rows) {
  constexpr int LPR = D / 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / LPR;
  const int c = (int)(t % LPR);
  float acc = 0.f;
  if (row < rows) {
    const f32x4 a = *(const f32x4*)(O + row * D + 4 * c);
    const f32x4 b = *(const f32x4*)(dO + row * D + 4 * c);
    acc = a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) {
    delta[row] = acc;
    lse2[row] = lse[row] * kLog2e32;
  }
}

// Half row fragment of row `row` of a [rows, D] tensor: lane half hf holds
// columns [D/2 hf, D/2 hf + D/2); rows past `rows` read as zero.
template <int D>
__device__ __forceinline__ void load_half_row(f32x4 (&f)[D / 8], const float* base, int rows, int row, int hf) {
#pragma unroll
  for (int c = 0; c < D / 8; ++c)
    f[c] = row < rows ? *(const f32x4*)(base + (size_t)row * D + (D / 2) * hf + 4 * c) : f32x4{0, 0, 0, 0};
}

// 32x32 product over the head dimension: rows 32 n + l32 of the LDS tile
// `rows_lds` (A operand) against the lane's half row fragment (B operand).
template <int D, int STR>
__device__ __forceinline__ f32x16 rows_times_frag(const float* rows_lds, int n, int l32, int hf,
                                                  const f32x4 (&f)[D / 8]) {
  f32x16 acc = {};
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const f32x4 a = *(const f32x4*)(rows_lds + (32 * n + l32) * STR + (D / 2) * hf + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma32(a[e], f[c][e], acc);
  }
  return acc;
}

// acc[dt] += T^T X over the 32 rows of block n of the LDS tile `t_lds`, where
// the lane holds X for row 32 n + 8 (r/4) + 4 hf + r%4 in x[r] (the layout of
// an S-like accumulator); MFMA step r pairs those rows across the half-waves.
template <int D, int STR>
__device__ __forceinline__ void acc_transposed(f32x16 (&acc)[D / 32], const float* t_lds, int n, int l32, int hf,
                                               const f32x16& x) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3);
      acc[dt] = mfma32(t_lds[row * STR + 32 * dt + l32], x[r], acc[dt]);
    }
}

// Store the transposed accumulators of row `row` (lane l32 of the wave's 32:
// columns 32 dt + 8 g + 4 hf + e), multiplied by `mul`.
template <int D>
__device__ __forceinline__ void store_row32(const f32x16 (&acc)[D / 32], float mul, float* out, int hf) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(f32x4*)(out + 32 * dt + 8 * g + 4 * hf) = f32x4{acc[dt][4 * g] * mul, acc[dt][4 * g + 1] * mul,
                                                         acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul};
}

// KS mode of both kernels: the four waves hold partial sums of the same 32
// rows; add waves 1-3's into wave 0's through LDS word
// ((w NDT + dt) 16 + r) 64 + lane (`x` holds 4 D/32 16 64 floats).  Every
// wave must call it (it contains barriers); the result is in wave 0.
template <int D>
__device__ __forceinline__ void sum_over_waves(f32x16 (&acc)[D / 32], float* x, int wave, int lane) {
  constexpr int NDT = D / 32;
  __syncthreads();
  if (wave != 0) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[((wave * NDT + dt) * 16 + r) * 64 + lane] = acc[dt][r];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w2 = 1; w2 < 4; ++w2)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] += x[((w2 * NDT + dt) * 16 + r) * 64 + lane];
  }
}

// ---------------------------------------------------------------------------
// dQ: 4 waves x 32 query rows per workgroup.  KS (grids with at most one
// 128-row workgroup per CU): 32 query rows per workgroup, 128-key tiles, wave
// w takes keys [32w, 32w + 32) of each and the waves' partial dQ are summed.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN, bool KS = false>
__global__ __launch_bounds__(kThreads32, 1) void bwd32_dq(const float* __restrict__ Qg, const float* __restrict__ Kg,
                                                          const float* __restrict__ Vg, const float* __restrict__ dOg,
                                                          const float* __restrict__ lse2g,
                                                          const float* __restrict__ deltag, float* __restrict__ dQg,
                                                          int BH, int Nq, int Nk, int nqt, float sl2, float scale,
                                                          const int* __restrict__ cuq, const int* __restrict__ cuk,
                                                          int H, int tq, int tk) {
  static_assert(!(KS && VARLEN), "the key split runs on dense inputs only");
  constexpr int BR = KS ? 32 : 128, BC = KS ? 128 : D <= 64 ? 64 : 32, NSUB = KS ? 1 : BC / 32;
  constexpr int STR = D + 4, ST = BC * STR, NDT = D / 32;
  constexpr int NSTG = (KS && D == 128) ? 1 : 2;  // LDS stages (a 128-key D = 128 stage takes 135 KB)
  constexpr int CPT = BC * D / 4 / kThreads32;  // 16-byte chunks per thread per tensor
  static_assert(CPT >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) float smem[NSTG * 2 * ST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  int bh, qt;
  tile_of_block(nqt, BH, bh, qt);
  const int q0 = qt * BR;
  const HeadRows hr = head_rows<VARLEN>(bh, Nq, Nk, D, cuq, cuk, H, tq, tk);
  const int nq = hr.nq, nk = hr.nk;
  if (q0 >= nq) return;  // past this sequence's queries: the whole workgroup
  const float* K = Kg + hr.ko;
  const float* V = Vg + hr.ko;
  const int kend = CAUSAL ? min(nk, min(q0 + BR, nq)) : nk;
  const int nt = (kend + BC - 1) / BC;
  const int wq0 = KS ? q0 : q0 + 32 * wave;
  const int kw = KS ? 32 * wave : 0;  // this wave's first key within a tile
  const int myq = wq0 + l32;
  const int wkend = CAUSAL ? min(kend, wq0 + 32) : kend;

  f32x4 qf[D / 8], df[D / 8];
  load_half_row<D>(qf, Qg + hr.qo, nq, myq, hf);
  load_half_row<D>(df, dOg + hr.qo, nq, myq, hf);
  // rows past nq: zero Q, dO and statistics, so dS = 0 (and they are not stored)
  const float lse2 = myq < nq ? lse2g[hr.so + myq] : 0.f;
  const float delta = myq < nq ? deltag[hr.so + myq] : 0.f;

  f32x4 kr[CPT], vr[CPT];
  auto load_tile = [&](int j) {
    const int k0 = j * BC;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kThreads32 * i;
      const int key = c / (D / 4), col = (c % (D / 4)) * 4;
      const bool ok = k0 + key < nk;
      kr[i] = ok ? *(const f32x4*)(K + (size_t)(k0 + key) * D + col) : f32x4{0, 0, 0, 0};
      vr[i] = ok ? *(const f32x4*)(V + (size_t)(k0 + key) * D + col) : f32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int stage) {
    float* ks = smem + stage * 2 * ST;
    float* vs = ks + ST;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kThreads32 * i;
      const int key = c / (D / 4), col = (c % (D / 4)) * 4;
      *(f32x4*)(ks + key * STR + col) = kr[i];
      *(f32x4*)(vs + key * STR + col) = vr[i];
    }
  };

  f32x16 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};

  if (nt > 0) load_tile(0);
  for (int j = 0; j < nt; ++j) {
    // two stages: stage j&1 was last read in step j-2, which every wave
    // finished before step j-1's barrier; one stage: wait for every wave
    const int stage = NSTG == 2 ? (j & 1) : 0;
    if (NSTG == 1 && j > 0) __syncthreads();
    store_tile(stage);
    __syncthreads();
    if (j + 1 < nt) load_tile(j + 1);
    const int k0 = j * BC + kw;  // this wave's first key of the tile
    if (k0 >= wkend) continue;
    const float* ks = smem + stage * 2 * ST + kw * STR;
    const float* vs = ks + ST;
    constexpr int BCW = 32 * NSUB;  // keys of the tile this wave attends to
    const bool need_mask = k0 + BCW > nk || (CAUSAL && k0 + BCW - 1 > wq0);
#pragma unroll
    for (int n = 0; n < NSUB; ++n) {
      // lane: query myq, keys k0 + 32 n + 8 (r/4) + 4 hf + r%4
      const f32x16 s = rows_times_frag<D, STR>(ks, n, l32, hf, qf);
      const f32x16 dp = rows_times_frag<D, STR>(vs, n, l32, hf, df);
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -lse2));
        if (need_mask) {
          const int key = k0 + 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= nk || (CAUSAL && key > myq)) p = 0.f;
        }
        ds[r] = p * (dp[r] - delta);
      }
      acc_transposed<D, STR>(acc, ks, n, l32, hf, ds);  // dQ^T += K^T dS^T
    }
  }
  if constexpr (KS) {
    sum_over_waves<D>(acc, smem, wave, lane);
    if (wave != 0) return;
  }
  if (myq < nq) store_row32<D>(acc, scale, dQg + hr.qo + (size_t)myq * D, hf);
}

// ---------------------------------------------------------------------------
// dK / dV: 4 waves x 32 keys per workgroup.  KS (D <= 64): 32 keys per
// workgroup, 128-query tiles, wave w takes queries [32w, 32w + 32) of each
// and the waves' partial dK and dV are summed.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN, bool KS = false>
__global__ __launch_bounds__(kThreads32, 1) void bwd32_dkdv(const float* __restrict__ Qg, const float* __restrict__ Kg,
                                                            const float* __restrict__ Vg,
                                                            const float* __restrict__ dOg,
                                                            const float* __restrict__ lse2g,
                                                            const float* __restrict__ deltag, float* __restrict__ dKg,
                                                            float* __restrict__ dVg, int BH, int Nq, int Nk,
                                                            float sl2, float scale, const int* __restrict__ cuq,
                                                            const int* __restrict__ cuk, int H, int tq, int tk) {
  static_assert(!(KS && (VARLEN || D > 64)), "the query split runs on dense inputs up to D = 64");
  constexpr int BK = KS ? 32 : 128, BQ = KS ? 128 : D <= 64 ? 64 : 32, NSUB = KS ? 1 : BQ / 32;
  constexpr int STR = D + 4, ST = BQ * STR, NDT = D / 32;
  constexpr int SS = 2 * ST + 2 * BQ;  // floats per stage: Q tile, dO tile, lse2, delta
  constexpr int NSTG = (KS && D == 128) ? 1 : 2;  // LDS stages (a 128-row D = 128 stage takes 136 KB)
  constexpr int CPT = BQ * D / 4 / kThreads32;
  static_assert(CPT >= 1 && 2 * BQ <= kThreads32, "tile shape");
  static_assert(!KS || NSTG * SS >= 2 * 4 * NDT * 16 * 64, "room for the sums over waves");
  __shared__ __attribute__((aligned(16))) float smem[NSTG * SS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  // Key blocks in ascending order: under the causal mask the first keys are
  // seen by the most queries, so the heaviest workgroups start first.
  const int bh = blockIdx.x % BH, kt = blockIdx.x / BH;
  const int kb0 = kt * BK;
  const int wk0 = KS ? kb0 : kb0 + 32 * wave;
  const int qw = KS ? 32 * wave : 0;  // this wave's first query within a tile
  const int mykey = wk0 + l32;
  const HeadRows hr = head_rows<VARLEN>(bh, Nq, Nk, D, cuq, cuk, H, tq, tk);
  const int nq = hr.nq, nk = hr.nk;
  if (kb0 >= nk) return;  // past this sequence's keys: the whole workgroup
  const float* Q = Qg + hr.qo;
  const float* dO = dOg + hr.qo;
  const float* l2h = lse2g + hr.so;
  const float* dlh = deltag + hr.so;
  const int t0 = CAUSAL ? kb0 / BQ : 0;  // first query tile that sees a key of the block
  const int nt = max((nq + BQ - 1) / BQ - t0, 0);

  f32x4 kf[D / 8], vf[D / 8];
  load_half_row<D>(kf, Kg + hr.ko, nk, mykey, hf);
  load_half_row<D>(vf, Vg + hr.ko, nk, mykey, hf);

  // Query rows past nq are staged as zero Q, dO and statistics: their P is
  // exp2(0) = 1 but dO = 0 and dS = P (0 - 0) = 0, so they add nothing.
  f32x4 qr[CPT], dr[CPT];
  float sr = 0.f;
  auto load_tile = [&](int t) {
    const int qb = t * BQ;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kThreads32 * i;
      const int row = c / (D / 4), col = (c % (D / 4)) * 4;
      const bool ok = qb + row < nq;
      qr[i] = ok ? *(const f32x4*)(Q + (size_t)(qb + row) * D + col) : f32x4{0, 0, 0, 0};
      dr[i] = ok ? *(const f32x4*)(dO + (size_t)(qb + row) * D + col) : f32x4{0, 0, 0, 0};
    }
    if (tid < 2 * BQ) {
      const int row = tid % BQ;
      const float* src = tid < BQ ? l2h : dlh;
      sr = qb + row < nq ? src[qb + row] : 0.f;
    }
  };
  auto store_tile = [&](int stage) {
    float* qs = smem + stage * SS;
    float* ds = qs + ST;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kThreads32 * i;
      const int row = c / (D / 4), col = (c % (D / 4)) * 4;
      *(f32x4*)(qs + row * STR + col) = qr[i];
      *(f32x4*)(ds + row * STR + col) = dr[i];
    }
    if (tid < 2 * BQ) qs[2 * ST + tid] = sr;  // lse2 then delta
  };

  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dk[dt] = dv[dt] = f32x16{};

  if (nt > 0) load_tile(t0);
  for (int j = 0; j < nt; ++j) {
    const int stage = NSTG == 2 ? (j & 1) : 0;
    if (NSTG == 1 && j > 0) __syncthreads();  // every wave is done with the one stage
    store_tile(stage);
    __syncthreads();
    if (j + 1 < nt) load_tile(t0 + j + 1);
    const int q0 = (t0 + j) * BQ + qw;  // this wave's first query of the tile
    constexpr int BQW = 32 * NSUB;      // queries of the tile this wave takes
    if (CAUSAL && q0 + BQW - 1 < wk0) continue;  // every query of the wave's rows precedes its keys
    const float* qs = smem + stage * SS + qw * STR;
    const float* dos = qs + ST;
    const float* l2s = smem + stage * SS + 2 * ST + qw;
    const float* dls = l2s + BQ;
    const bool need_mask = CAUSAL && q0 < wk0 + 31;
#pragma unroll
    for (int n = 0; n < NSUB; ++n) {
      // lane: key mykey, queries q0 + 32 n + 8 (r/4) + 4 hf + r%4
      const f32x16 s = rows_times_frag<D, STR>(qs, n, l32, hf, kf);
      const f32x16 dp = rows_times_frag<D, STR>(dos, n, l32, hf, vf);
      f32x16 p, ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3);
        float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -l2s[row]));
        if (need_mask && q0 + row < mykey) pr = 0.f;
        p[r] = pr;
        ds[r] = pr * (dp[r] - dls[row]);
      }
      acc_transposed<D, STR>(dv, dos, n, l32, hf, p);  // dV^T += dO^T P
      acc_transposed<D, STR>(dk, qs, n, l32, hf, ds);  // dK^T += Q^T dS
    }
  }
  if constexpr (KS) {
    sum_over_waves<D>(dk, smem, wave, lane);
    sum_over_waves<D>(dv, smem + 4 * NDT * 16 * 64, wave, lane);
    if (wave != 0) return;
  }
  if (mykey < nk) {
    store_row32<D>(dk, scale, dKg + hr.ko + (size_t)mykey * D, hf);
    store_row32<D>(dv, 1.0f, dVg + hr.ko + (size_t)mykey * D, hf);
  }
}

template <int D, bool CAUSAL, bool VARLEN>
int launch_bwd32(const FaBwdLaunch& a, float sl2, float scale) {
  const hipStream_t st = (hipStream_t)a.stream;
  const int64_t rows = VARLEN ? a.H * a.total_q : a.BH * a.Nq;  // query rows (statistics)
  const int H = (int)a.H, tq = (int)a.total_q, tk = (int)a.total_k;
  float* lse2 = (float*)a.workspace;
  float* delta = lse2 + rows;
  int rc = 0;
  if (rows > 0) {
    const int64_t threads = rows * (D / 4);
    rc = launch_kernel(bwd32_prep<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), st, (const float*)a.o,
                       (const float*)a.dout, a.lse, lse2, delta, rows);
    if (rc != 0) return rc;
    // At most one 128-row workgroup per CU: the key-split form (four times
    // the waves), as in the fp32 forward.
    const int nqt = (int)((a.Nq + 127) / 128);
    const bool ks = !VARLEN && a.BH * nqt <= a.cus;
    if (nqt > 0 && ks) {
      if constexpr (!VARLEN)
        rc = launch_kernel(bwd32_dq<D, CAUSAL, false, true>, dim3((unsigned)(a.BH * ((a.Nq + 31) / 32))),
                           dim3(kThreads32), st, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                           (const float*)a.dout, (const float*)lse2, (const float*)delta, (float*)a.dq, (int)a.BH,
                           (int)a.Nq, (int)a.Nk, (int)((a.Nq + 31) / 32), sl2, scale, a.cu_q, a.cu_k, H, tq, tk);
    } else if (nqt > 0) {
      rc = launch_kernel(bwd32_dq<D, CAUSAL, VARLEN>, dim3((unsigned)(a.BH * nqt)), dim3(kThreads32), st,
                         (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dout,
                         (const float*)lse2, (const float*)delta, (float*)a.dq, (int)a.BH, (int)a.Nq, (int)a.Nk,
                         nqt, sl2, scale, a.cu_q, a.cu_k, H, tq, tk);
    }
    if (rc != 0) return rc;
  }
  const int nkt = (int)((a.Nk + 127) / 128);
  // (not at D = 128: staging 128 query rows of Q and dO next to the K, V
  // fragments and both gradients spills registers)
  const bool ks = !VARLEN && D <= 64 && a.BH * nkt <= a.cus;
  if (nkt > 0 && ks) {
    if constexpr (!VARLEN && D <= 64)
      rc = launch_kernel(bwd32_dkdv<D, CAUSAL, false, true>, dim3((unsigned)(a.BH * ((a.Nk + 31) / 32))),
                         dim3(kThreads32), st, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                         (const float*)a.dout, (const float*)lse2, (const float*)delta, (float*)a.dk, (float*)a.dv,
                         (int)a.BH, (int)a.Nq, (int)a.Nk, sl2, scale, a.cu_q, a.cu_k, H, tq, tk);
  } else if (nkt > 0) {
    rc = launch_kernel(bwd32_dkdv<D, CAUSAL, VARLEN>, dim3((unsigned)(a.BH * nkt)), dim3(kThreads32), st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dout,
                       (const float*)lse2, (const float*)delta, (float*)a.dk, (float*)a.dv, (int)a.BH, (int)a.Nq,
                       (int)a.Nk, sl2, scale, a.cu_q, a.cu_k, H, tq, tk);
  }
  return rc;
}

template <int D>
int dispatch_bwd32(const FaBwdLaunch& a, float sl2, float scale) {
  if (a.cu_q)
    return a.causal ? launch_bwd32<D, true, true>(a, sl2, scale) : launch_bwd32<D, false, true>(a, sl2, scale);
  return a.causal ? launch_bwd32<D, true, false>(a, sl2, scale) : launch_bwd32<D, false, false>(a, sl2, scale);
}

}  // namespace

int fa_launch_bwd32(const FaBwdLaunch& a, float sl2, float scale) {
  switch (a.D) {
    case 32: return dispatch_bwd32<32>(a, sl2, scale);
    case 64: return dispatch_bwd32<64>(a, sl2, scale);
    default: return dispatch_bwd32<128>(a, sl2, scale);
  }
}
