// Exact tiled attention backward pass for gfx950 (CDNA4, MI355X), 16-bit
// inputs (bf16 / fp16), D in {32, 64, 128, 256}.
//
// "Building a FlashAttention-2 Forward Kernel in Pure NumPy" (Extending It)
// describes the backward pass as recomputation: keep the forward's softmax
// statistics, recompute the score tiles and stream the gradients tile by
// tile.  Here the statistic is the forward's LSE (m + ln l in one number),
// so every probability is recomputed exactly as P = exp(s - LSE) with no
// running max.  With dO the gradient of O and delta_i = sum_d dO[i,d] O[i,d]
// (= rowsum(P * dP), which is what makes the softmax Jacobian cheap):
//
//   dP = dO V^T,  dS = P * (dP - delta),  dV = P^T dO,
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, no atomics, deterministic:
//  * bwd_prep: delta and LSE * log2(e) per query row, into the workspace;
//  * bwd_dq: one workgroup per (batch*head, 256 query rows), 8 waves of 32
//    rows (the forward's shape): K/V tiles stream through the same 4-stage
//    direct-to-LDS ring; per tile S^T = K Q^T, dP^T = V dO^T, then
//    dQ^T += K^T dS^T (K read transposed);
//  * bwd_dkdv: one workgroup per (batch*head, 128 keys), 4 waves of 32 keys
//    (one wave per SIMD: 32 keys of K and V fragments plus fp32 dK and dV
//    accumulators need more than 256 registers); Q/dO tiles of 64 query
//    rows plus their LSE and delta stream through a 4-stage ring; per tile
//    S = Q K^T, dP = dO V^T (the wave's keys along the MFMA N dimension, so
//    P and dS come out in the B-operand layout of the next products), then
//    dV^T += dO^T P and dK^T += Q^T dS (dO and Q read transposed).
// S and dP are recomputed in both kernels: seven tile products instead of
// the five a single kernel with atomic dQ updates would need.
// At D = 256 bwd_dq has 4 waves (one per SIMD), bwd_dkdv runs as two kernels
// (dV, then dK: one gradient's accumulators per wave), and both rings have 2
// stages (a stage of two 64-row tiles takes 64 KB).
//
// The library compiles this file twice.  Without FA_BWD_SMALL_D it defines
// fa_launch_bwd and the D = 128 kernels; with FA_BWD_SMALL_D only the D = 32
// and 64 launcher (fa_launch_bwd_small_d), compiled with the MFMA
// accumulators in VGPRs: in the AGPR form the compiler copied the dK/dV
// accumulators and every S / dP value between the two register files
// (about 960 copies in the D = 64 dK/dV kernel), while at D = 128 the VGPR
// form runs out of registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634074f;
constexpr int kWavesKV = 4;  // bwd_dkdv: waves per workgroup (32 keys each)

// bwd_dq: waves per workgroup (32 query rows each).  Up to D = 128, 8 (two
// per SIMD); at D = 256 the Q and dO fragments and the fp32 dQ of 32 rows take
// more than half of a SIMD's registers, so 4 (one per SIMD).
template <int D>
constexpr int dq_waves() {
  return D == 256 ? 4 : 8;
}
// Stages of both kernels' LDS rings: 4 up to D = 128 (three tiles in flight);
// at D = 256 a stage (64 rows of two tensors) takes 64 KB, so 2 (one tile in
// flight: each tile waits for itself, then the next one starts).
template <int D>
constexpr int bwd_stages() {
  return D == 256 ? 2 : 4;
}

template <int DT>
__device__ __forceinline__ float lo16(unsigned x) {
  if constexpr (DT == kBF16) return __builtin_bit_cast(float, x << 16);
  else return (float)__builtin_bit_cast(_Float16, (u16)(x & 0xFFFFu));
}
template <int DT>
__device__ __forceinline__ float hi16(unsigned x) {
  if constexpr (DT == kBF16) return __builtin_bit_cast(float, x & 0xFFFF0000u);
  else return (float)__builtin_bit_cast(_Float16, (u16)(x >> 16));
}

// ---------------------------------------------------------------------------
// Per query row: delta = sum_d dO[d] O[d] (fp32, from the stored 16-bit
// values) and lse2 = LSE log2(e).  D/8 lanes per row, 16 bytes each.
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void bwd_prep(const u16* __restrict__ O, const u16* __restrict__ dO,
                                                const float* __restrict__ lse, float* __restrict__ lse2,
                                                float* __restrict__ delta, int64_t rows) {
  constexpr int LPR = D / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / LPR;
  const int c = (int)(t % LPR);
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(O + row * D + 8 * c);
    const u32x4 b = *(const u32x4*)(dO + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += lo16<DT>(a[e]) * lo16<DT>(b[e]) + hi16<DT>(a[e]) * hi16<DT>(b[e]);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) {
    delta[row] = acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

// Store a 32-row block of fp32 results (transposed accumulators: lane l holds
// row l % 32, columns 32 dt + 8 g + 4 (l / 32) + 0..3) as 16-bit rows,
// multiplied by `mul`; rows past the buffer range are dropped.
template <int DT, int D>
__device__ __forceinline__ void store_rows16(const f32x16 (&acc)[D / 32], float mul, __amdgpu_buffer_rsrc_t r,
                                             int row_byte, int base_byte, int hf) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 v;
      v[0] = pack2<DT>(acc[dt][4 * g + 0] * mul, acc[dt][4 * g + 1] * mul);
      v[1] = pack2<DT>(acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul);
      __builtin_amdgcn_raw_buffer_store_b64(v, r, row_byte + (32 * dt + 8 * g + 4 * hf) * 2, base_byte, 0);
    }
}

// Fragment of 32 rows of a 16-bit [N, D] tensor in the B-operand layout of
// v_mfma_f32_32x32x16: lane l holds row `row0 + l % 32`, columns
// 16 kk + 8 (l / 32) .. +7; rows past `rows` read as zero.
template <int D>
__device__ __forceinline__ void load_frag(u32x4 (&f)[D / 16], const u16* base, int rows, int row0,
                                          const Wave16& w) {
  const auto r = make_rsrc(base, rows * D * 2);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    f[kk] = __builtin_amdgcn_raw_buffer_load_b128(r, w.l32 * D * 2 + (16 * kk + 8 * w.hf) * 2, row0 * D * 2, 0);
}

// ---------------------------------------------------------------------------
// dQ kernel.
// ---------------------------------------------------------------------------
template <int DT, int D, bool CAUSAL>
__device__ __forceinline__ void dq_tile(const u16* Kh, const u16* Vh, int kbytes, int j, int nt,
                                        const unsigned char* src, unsigned char* dst, const Wave16& w,
                                        const u32x4 (&qf)[D / 16], const u32x4 (&dof)[D / 16],
                                        f32x16 (&acc)[D / 32], float lse2, float delta, float sl2) {
  constexpr int BC = 64, TILEB = BC * D * 2, NKK = D / 16, NDT = D / 32, NW = dq_waves<D>(), ST = bwd_stages<D>();
  const int k0 = j * BC;
  const unsigned char* ks = src;
  const unsigned char* vs = src + TILEB;
  // 4 stages: tile j is complete since the previous barrier; wait for tile
  // j+1.  2 stages: wait for tile j itself.  Then refill the stage of tile j-1.
  wait_tile_and_barrier(ST == 4 && j + 2 < nt ? loads_per_tile<D, NW>(w.wave) : 0);
  if (j + ST - 1 < nt) issue_tile16<D, NW>(Kh, Vh, kbytes, j + ST - 1, dst, w);
  if (k0 >= w.wkend) return;
  const bool need_mask = k0 + BC - 1 > w.wklim;  // causal diagonal or past Nk
  const int lim = w.klim - (k0 + 4 * w.hf);
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s = mfma_32x32x16<DT>(ks_operand<D>(ks, w, n * NKK + kk), qf[kk], s);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) dp = mfma_32x32x16<DT>(ks_operand<D>(vs, w, n * NKK + kk), dof[kk], dp);
    // P = exp2(s sl2 - lse2) (masked keys: 0), dS = P (dP - delta).
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -lse2));
      if (need_mask && 32 * n + 8 * (r >> 2) + (r & 3) > lim) p = 0.f;
      ds[r] = p * (dp[r] - delta);
    }
    u32x4 dsf[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) dsf[hh][i] = pack2<DT>(ds[8 * hh + 2 * i], ds[8 * hh + 2 * i + 1]);
    // dQ^T += K^T dS^T over this block's 32 keys.
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        acc[dt] = mfma_32x32x16<DT>(vt_operand<D>(ks, w, 4 * dt + 2 * n + hh), dsf[hh], acc[dt]);
  }
}

// VARLEN: packed sequences (the rows of head_rows); a workgroup past its
// sequence's queries exits, a sequence without keys gets dQ = 0.
template <int DT, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(64 * dq_waves<D>(), 1) void bwd_dq(const u16* __restrict__ Qg, const u16* __restrict__ Kg,
                                                          const u16* __restrict__ Vg, const u16* __restrict__ dOg,
                                                          const float* __restrict__ lse2g,
                                                          const float* __restrict__ deltag, u16* __restrict__ dQg,
                                                          int BH, int Nq, int Nk, int nqt, float sl2, float scale,
                                                          const int* __restrict__ cuq, const int* __restrict__ cuk,
                                                          int H, int tq, int tk) {
  constexpr int BC = 64, ROWB = D * 2, TILEB = BC * ROWB, NW = dq_waves<D>(), BR = 32 * NW, ST = bwd_stages<D>();
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[ST == 4 ? 2 * TILEB : 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[ST == 4 ? 2 * TILEB : 1024];

  Wave16 w;
  const int tid = threadIdx.x;
  w.lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.hf = w.lane >> 5;
  w.l32 = w.lane & 31;
  int bh, qt;
  tile_of_block(nqt, BH, bh, qt);
  const int q0 = qt * BR;
  const HeadRows hr = head_rows<VARLEN>(bh, Nq, Nk, D, cuq, cuk, H, tq, tk);
  const int nq = hr.nq, nk = hr.nk;
  if (q0 >= nq) return;  // past this sequence's queries: the whole workgroup
  const u16* Kh = Kg + hr.ko;
  const u16* Vh = Vg + hr.ko;
  const int kbytes = nk * ROWB;
  const int kend = CAUSAL ? min(nk, min(q0 + BR, nq)) : nk;
  const int nt = (kend + BC - 1) / BC;
  w.wq0 = q0 + 32 * w.wave;
  const int myq = w.wq0 + w.l32;
  w.wkend = CAUSAL ? min(kend, w.wq0 + 32) : kend;
  w.klim = CAUSAL ? min(myq, nk - 1) : nk - 1;
  w.wklim = CAUSAL ? min(w.wq0, nk - 1) : nk - 1;
  init_operand_offsets<D>(w);

  u32x4 qf[D / 16], dof[D / 16];
  load_frag<D>(qf, Qg + hr.qo, nq, w.wq0, w);
  load_frag<D>(dof, dOg + hr.qo, nq, w.wq0, w);
  const auto rs = make_rsrc(lse2g + hr.so, nq * 4);
  const auto rd = make_rsrc(deltag + hr.so, nq * 4);
  const float lse2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, myq * 4, 0, 0));
  const float delta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, myq * 4, 0, 0));

  // (a sequence without keys has no tile: nothing may be left in flight)
  if (!VARLEN || nt > 0) issue_tile16<D, NW>(Kh, Vh, kbytes, 0, stage0, w);
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  if constexpr (ST == 4) {
    if (nt > 1) issue_tile16<D, NW>(Kh, Vh, kbytes, 1, stage1, w);
    if (nt > 2) issue_tile16<D, NW>(Kh, Vh, kbytes, 2, stage2, w);
    // Tile 0 complete before the first tile's reads.
    wait_tile_and_barrier(nt > 2 ? loads_per_tile<D, NW>(w.wave) : 0);
    for (int j = 0; j < nt; j += 4) {
      dq_tile<DT, D, CAUSAL>(Kh, Vh, kbytes, j, nt, stage0, stage3, w, qf, dof, acc, lse2, delta, sl2);
      if (j + 1 < nt)
        dq_tile<DT, D, CAUSAL>(Kh, Vh, kbytes, j + 1, nt, stage1, stage0, w, qf, dof, acc, lse2, delta, sl2);
      if (j + 2 < nt)
        dq_tile<DT, D, CAUSAL>(Kh, Vh, kbytes, j + 2, nt, stage2, stage1, w, qf, dof, acc, lse2, delta, sl2);
      if (j + 3 < nt)
        dq_tile<DT, D, CAUSAL>(Kh, Vh, kbytes, j + 3, nt, stage3, stage2, w, qf, dof, acc, lse2, delta, sl2);
    }
  } else {
    for (int j = 0; j < nt; j += 2) {
      dq_tile<DT, D, CAUSAL>(Kh, Vh, kbytes, j, nt, stage0, stage1, w, qf, dof, acc, lse2, delta, sl2);
      if (j + 1 < nt)
        dq_tile<DT, D, CAUSAL>(Kh, Vh, kbytes, j + 1, nt, stage1, stage0, w, qf, dof, acc, lse2, delta, sl2);
    }
  }
  const auto rq = make_rsrc(dQg + hr.qo, nq * ROWB);
  store_rows16<DT, D>(acc, scale, rq, (32 * w.wave + w.l32) * ROWB, q0 * ROWB, w.hf);
}

// ---------------------------------------------------------------------------
// dK / dV kernel.
// ---------------------------------------------------------------------------
// Stage layout: Q tile, dO tile (64 rows each, the swizzled tile layout),
// then lse2 (64 floats) and delta (64 floats) of the tile's rows.
template <int D>
constexpr int kv_stage_bytes() {
  return 2 * 64 * D * 2 + 1024;
}

// Wave 0 also loads the tile's lse2 and delta (two 256-byte loads, 4 bytes a
// lane), so its count per tile is two higher.
template <int D>
__device__ __forceinline__ int kv_loads_per_tile(int wave) {
  return loads_per_tile<D, kWavesKV>(wave) + (wave == 0 ? 2 : 0);
}

template <int D>
__device__ __forceinline__ void issue_kv_tile(const u16* Qh, const u16* dOh, int qbytes, const float* l2h,
                                              const float* dlh, int Nq, int t, unsigned char* dst,
                                              const Wave16& w) {
  constexpr int TILEB = 64 * D * 2;
  issue_tile16<D, kWavesKV>(Qh, dOh, qbytes, t, dst, w);
  if (w.wave == 0) {
    const auto rl = make_rsrc(l2h, Nq * 4);
    const auto rd = make_rsrc(dlh, Nq * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)(dst + 2 * TILEB), 4, w.lane * 4, t * 256, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)(dst + 2 * TILEB + 256), 4, w.lane * 4, t * 256, 0, 0);
  }
}

// GRADS: 3 = dK and dV, 1 = dK only, 2 = dV only (D = 256, where the fp32 dK
// and dV of 32 keys plus the K and V fragments do not fit one wave's
// registers, so one kernel runs per gradient).
template <int DT, int D, bool CAUSAL, int GRADS>
__device__ __forceinline__ void kv_tile(const u16* Qh, const u16* dOh, int qbytes, const float* l2h,
                                        const float* dlh, int Nq, int t0, int j, int nt, const unsigned char* src,
                                        unsigned char* dst, const Wave16& w, int wk0, const u32x4 (&kf)[D / 16],
                                        const u32x4 (&vf)[D / 16], f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
                                        float sl2) {
  constexpr int TILEB = 64 * D * 2, NKK = D / 16, NDT = D / 32, ST = bwd_stages<D>();
  const int t = t0 + j;
  const int q0 = 64 * t;
  const unsigned char* qs = src;
  const unsigned char* dos = src + TILEB;
  const unsigned char* st = src + 2 * TILEB;
  // As in dq_tile: 4 stages wait for tile j+1, 2 stages for tile j.
  wait_tile_and_barrier(ST == 4 && j + 2 < nt ? kv_loads_per_tile<D>(w.wave) : 0);
  if (j + ST - 1 < nt) issue_kv_tile<D>(Qh, dOh, qbytes, l2h, dlh, Nq, t + ST - 1, dst, w);
  if (CAUSAL && q0 + 63 < wk0) return;  // every query of the tile precedes the wave's keys
  static_assert(GRADS == 3 || D == 256, "one gradient per kernel only at D = 256");
  if constexpr (D == 128) {
    // Queries of the tile below `qlim` (relative to q0) precede this lane's key
    // and are masked (causal diagonal tiles only; elsewhere no query is).
    const int qlim = (CAUSAL && q0 < wk0 + 31) ? wk0 + w.l32 - q0 : 0;
    // One wave per SIMD, so the wave overlaps its own work, in an order fixed
    // by scheduling fences: block 1's S and dP MFMAs each carry one score of
    // block 0's softmax arithmetic, block 0's dV and dK MFMAs each carry one of
    // block 1's, and every LDS operand is read a few MFMAs ahead.
    constexpr int NS = 2 * NKK;  // S and dP MFMAs of a 32-query block (interleaved)
    constexpr int NG = 4 * NDT;  // dV and dK MFMAs of a block (interleaved)
    // Lane l holds key wk0 + l % 32 and queries q0 + 32n + 8g + 4hf + e (r = 4g + e).
    f32x16 s[2], dp[2];
    u32x4 pf[2][2], dsf[2][2];
    float pv[2][16], dsv[2][16];
    // operand i of the score MFMAs of block n: even i -> Q row operand for S,
    // odd i -> dO row operand for dP, both at head-dimension step i / 2
    auto score_operand = [&](int n, int i) -> u32x4 {
      return (i & 1) ? ks_operand<D>(dos, w, n * NKK + (i >> 1)) : ks_operand<D>(qs, w, n * NKK + (i >> 1));
    };
    auto score_mfma = [&](int n, int i, u32x4 a) {
      if (i & 1)
        dp[n] = mfma_32x32x16<DT>(a, vf[i >> 1], dp[n]);
      else
        s[n] = mfma_32x32x16<DT>(a, kf[i >> 1], s[n]);
    };
    // operand i of the gradient MFMAs of block n: even i -> dO^T for dV,
    // odd i -> Q^T for dK, at (dt, hh) = ((i / 2) / 2, (i / 2) % 2)
    auto grad_operand = [&](int n, int i) -> u32x4 {
      const int u = i >> 1, idx = 4 * (u >> 1) + 2 * n + (u & 1);
      return (i & 1) ? vt_operand<D>(qs, w, idx) : vt_operand<D>(dos, w, idx);
    };
    auto grad_mfma = [&](int n, int i, u32x4 a) {
      const int u = i >> 1;
      if (i & 1)
        dk[u >> 1] = mfma_32x32x16<DT>(a, dsf[n][u & 1], dk[u >> 1]);
      else
        dv[u >> 1] = mfma_32x32x16<DT>(a, pf[n][u & 1], dv[u >> 1]);
    };
    // softmax-gradient arithmetic of score r of block n (and the packing of a
    // finished pair)
    f32x4 l4[2][4], d4[2][4];
    auto score_math = [&](int n, int r) {
      const int g = r >> 2, e = r & 3, qo = 32 * n + 8 * g + 4 * w.hf;
      float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][r], sl2, -l4[n][g][e]));
      pr = qo + e < qlim ? 0.f : pr;
      pv[n][r] = pr;
      dsv[n][r] = pr * (dp[n][r] - d4[n][g][e]);
      if (r & 1) {
        const int hh = r >> 3, i = (r & 7) >> 1;
        pf[n][hh][i] = pack2<DT>(pv[n][r - 1], pv[n][r]);
        dsf[n][hh][i] = pack2<DT>(dsv[n][r - 1], dsv[n][r]);
      }
    };
    auto load_stats = [&](int n) {
  #pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qo = 32 * n + 8 * g + 4 * w.hf;
        l4[n][g] = *(const f32x4*)(st + qo * 4);
        d4[n][g] = *(const f32x4*)(st + 256 + qo * 4);
      }
    };
    constexpr int PRE = 8;  // operand read-ahead, in MFMAs
    u32x4 op[NS > NG ? NS : NG];
    s[0] = dp[0] = s[1] = dp[1] = f32x16{};
    // block 0: score MFMAs
  #pragma unroll
    for (int i = 0; i < PRE; ++i) op[i] = score_operand(0, i);
    load_stats(0);
  #pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + PRE < NS) op[i + PRE] = score_operand(0, i + PRE);
      score_mfma(0, i, op[i]);
    }
    // block 1: score MFMAs, each with one score of block 0's arithmetic
  #pragma unroll
    for (int i = 0; i < PRE; ++i) op[i] = score_operand(1, i);
    load_stats(1);
    __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + PRE < NS) op[i + PRE] = score_operand(1, i + PRE);
      score_mfma(1, i, op[i]);
  #pragma unroll
      for (int r = i * 16 / NS; r < (i + 1) * 16 / NS; ++r) score_math(0, r);
      __builtin_amdgcn_sched_barrier(0);
    }
    // block 0: gradient MFMAs, each with one score of block 1's arithmetic
  #pragma unroll
    for (int i = 0; i < PRE; ++i) op[i] = grad_operand(0, i);
    __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (i + PRE < NG) op[i + PRE] = grad_operand(0, i + PRE);
      grad_mfma(0, i, op[i]);
  #pragma unroll
      for (int r = i * 16 / NG; r < (i + 1) * 16 / NG; ++r) score_math(1, r);
      __builtin_amdgcn_sched_barrier(0);
    }
    // block 1: gradient MFMAs
  #pragma unroll
    for (int i = 0; i < PRE; ++i) op[i] = grad_operand(1, i);
  #pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (i + PRE < NG) op[i + PRE] = grad_operand(1, i + PRE);
      grad_mfma(1, i, op[i]);
    }
  } else {
    // D <= 64 and D = 256: the compiler's own schedule (below D = 128 it
    // measured faster than the fenced one).
    constexpr bool kDK = GRADS & 1, kDV = GRADS & 2;
    const bool need_mask = CAUSAL && q0 < wk0 + 31;
    const int mykey = wk0 + w.l32;
  #pragma unroll
    for (int n = 0; n < 2; ++n) {
      f32x16 s = {}, dp = {};
  #pragma unroll
      for (int kk = 0; kk < NKK; ++kk) s = mfma_32x32x16<DT>(ks_operand<D>(qs, w, n * NKK + kk), kf[kk], s);
      if constexpr (kDK) {
  #pragma unroll
        for (int kk = 0; kk < NKK; ++kk) dp = mfma_32x32x16<DT>(ks_operand<D>(dos, w, n * NKK + kk), vf[kk], dp);
      }
      // Lane l holds key mykey and queries q0 + 32n + 8g + 4hf + e (r = 4g + e).
      float p[16], ds[16];
  #pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qo = 32 * n + 8 * g + 4 * w.hf;
        const f32x4 l4 = *(const f32x4*)(st + qo * 4);
        const f32x4 d4 = *(const f32x4*)(st + 256 + qo * 4);
  #pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -l4[e]));
          if (need_mask && q0 + qo + e < mykey) pr = 0.f;
          p[r] = pr;
          ds[r] = kDK ? pr * (dp[r] - d4[e]) : 0.f;
        }
      }
      u32x4 pf[2], dsf[2];
  #pragma unroll
      for (int hh = 0; hh < 2; ++hh)
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[hh][i] = pack2<DT>(p[8 * hh + 2 * i], p[8 * hh + 2 * i + 1]);
          dsf[hh][i] = pack2<DT>(ds[8 * hh + 2 * i], ds[8 * hh + 2 * i + 1]);
        }
      // dV^T += dO^T P and dK^T += Q^T dS over this block's 32 queries.
  #pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
  #pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          if constexpr (kDV) dv[dt] = mfma_32x32x16<DT>(vt_operand<D>(dos, w, 4 * dt + 2 * n + hh), pf[hh], dv[dt]);
          if constexpr (kDK) dk[dt] = mfma_32x32x16<DT>(vt_operand<D>(qs, w, 4 * dt + 2 * n + hh), dsf[hh], dk[dt]);
        }
    }
  }
}

// VARLEN: packed sequences (the rows of head_rows); a workgroup past its
// sequence's keys exits, keys of a sequence without queries get zeros.
template <int DT, int D, bool CAUSAL, int GRADS, bool VARLEN>
__global__ __launch_bounds__(64 * kWavesKV, 1) void bwd_dkdv(const u16* __restrict__ Qg, const u16* __restrict__ Kg,
                                                             const u16* __restrict__ Vg, const u16* __restrict__ dOg,
                                                             const float* __restrict__ lse2g,
                                                             const float* __restrict__ deltag, u16* __restrict__ dKg,
                                                             u16* __restrict__ dVg, int BH, int Nq, int Nk,
                                                             float sl2, float scale, const int* __restrict__ cuq,
                                                             const int* __restrict__ cuk, int H, int tq, int tk) {
  constexpr int ROWB = D * 2, SB = kv_stage_bytes<D>(), BK = 32 * kWavesKV, ST = bwd_stages<D>();
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[ST == 4 ? SB : 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[ST == 4 ? SB : 1024];

  Wave16 w;
  const int tid = threadIdx.x;
  w.lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.hf = w.lane >> 5;
  w.l32 = w.lane & 31;
  // Key blocks in ascending order: under the causal mask the first keys are
  // seen by the most queries, so the heaviest workgroups start first.
  const int bid = blockIdx.x;
  const int bh = bid % BH, kt = bid / BH;
  const int kb0 = kt * BK;
  const int wk0 = kb0 + 32 * w.wave;
  const HeadRows hr = head_rows<VARLEN>(bh, Nq, Nk, D, cuq, cuk, H, tq, tk);
  const int nq = hr.nq, nk = hr.nk;
  if (kb0 >= nk) return;  // past this sequence's keys: the whole workgroup
  const u16* Qh = Qg + hr.qo;
  const u16* dOh = dOg + hr.qo;
  const float* l2h = lse2g + hr.so;
  const float* dlh = deltag + hr.so;
  const int qbytes = nq * ROWB;
  const int t0 = CAUSAL ? kb0 / 64 : 0;  // first query tile that sees a key of the block
  const int nt = max((nq + 63) / 64 - t0, 0);
  w.wq0 = w.wkend = w.wklim = w.klim = 0;  // forward-only fields
  init_operand_offsets<D>(w);

  u32x4 kf[D / 16], vf[D / 16];
  load_frag<D>(kf, Kg + hr.ko, nk, wk0, w);
  if constexpr (GRADS & 1) load_frag<D>(vf, Vg + hr.ko, nk, wk0, w);
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dk[dt] = dv[dt] = f32x16{};

  if (nt > 0) {
    issue_kv_tile<D>(Qh, dOh, qbytes, l2h, dlh, nq, t0, stage0, w);
    if constexpr (ST == 2) {
      for (int j = 0; j < nt; j += 2) {
        kv_tile<DT, D, CAUSAL, GRADS>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j, nt, stage0, stage1, w, wk0, kf, vf, dk, dv, sl2);
        if (j + 1 < nt)
          kv_tile<DT, D, CAUSAL, GRADS>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j + 1, nt, stage1, stage0, w, wk0, kf, vf, dk, dv,
                                 sl2);
      }
    } else {
      if (nt > 1) issue_kv_tile<D>(Qh, dOh, qbytes, l2h, dlh, nq, t0 + 1, stage1, w);
      if (nt > 2) issue_kv_tile<D>(Qh, dOh, qbytes, l2h, dlh, nq, t0 + 2, stage2, w);
      wait_tile_and_barrier(nt > 2 ? kv_loads_per_tile<D>(w.wave) : 0);
      for (int j = 0; j < nt; j += 4) {
        kv_tile<DT, D, CAUSAL, GRADS>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j, nt, stage0, stage3, w, wk0, kf, vf, dk, dv, sl2);
        if (j + 1 < nt)
          kv_tile<DT, D, CAUSAL, GRADS>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j + 1, nt, stage1, stage0, w, wk0, kf, vf, dk, dv,
                                 sl2);
        if (j + 2 < nt)
          kv_tile<DT, D, CAUSAL, GRADS>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j + 2, nt, stage2, stage1, w, wk0, kf, vf, dk, dv,
                                 sl2);
        if (j + 3 < nt)
          kv_tile<DT, D, CAUSAL, GRADS>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j + 3, nt, stage3, stage2, w, wk0, kf, vf, dk, dv,
                                 sl2);
      }
    }
  }
  const auto rk = make_rsrc(dKg + hr.ko, nk * ROWB);
  const auto rv = make_rsrc(dVg + hr.ko, nk * ROWB);
  if constexpr (GRADS & 1) store_rows16<DT, D>(dk, scale, rk, (32 * w.wave + w.l32) * ROWB, kb0 * ROWB, w.hf);
  if constexpr (GRADS & 2) store_rows16<DT, D>(dv, 1.0f, rv, (32 * w.wave + w.l32) * ROWB, kb0 * ROWB, w.hf);
}

// VARLEN: q, o, dout, dq [H, total_q, D]; k, v, dk, dv [H, total_k, D]; lse
// and the workspace [H, total_q]; a.Nq / a.Nk are the longest sequence's
// query / key counts and size the grids.
template <int DT, int D, bool CAUSAL, bool VARLEN>
int launch_bwd(const FaBwdLaunch& a, float sl2, float scale) {
  const hipStream_t st = (hipStream_t)a.stream;
  const int64_t rows = VARLEN ? a.H * a.total_q : a.BH * a.Nq;  // query rows (statistics)
  const int H = (int)a.H, tq = (int)a.total_q, tk = (int)a.total_k;
  float* lse2 = (float*)a.workspace;
  float* delta = lse2 + rows;
  if (rows > 0) {
    const int64_t threads = rows * (D / 8);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    hipLaunchKernelGGL((bwd_prep<DT, D>), grid, block, 0, st, (const u16*)a.o, (const u16*)a.dout, a.lse, lse2,
                       delta, rows);
    constexpr int NWQ = dq_waves<D>();
    const int nqt = (int)((a.Nq + 32 * NWQ - 1) / (32 * NWQ));
    if (nqt > 0)
      hipLaunchKernelGGL((bwd_dq<DT, D, CAUSAL, VARLEN>), dim3((unsigned)(a.BH * nqt)), dim3(64 * NWQ), 0, st,
                         (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (const u16*)a.dout, (const float*)lse2,
                         (const float*)delta, (u16*)a.dq, (int)a.BH, (int)a.Nq, (int)a.Nk, nqt, sl2, scale, a.cu_q,
                         a.cu_k, H, tq, tk);
  }
  const int nkt = (int)((a.Nk + 32 * kWavesKV - 1) / (32 * kWavesKV));
  if (nkt > 0) {
    const dim3 grid((unsigned)(a.BH * nkt)), block(64 * kWavesKV);
    auto run = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, block, 0, st, (const u16*)a.q, (const u16*)a.k, (const u16*)a.v,
                         (const u16*)a.dout, (const float*)lse2, (const float*)delta, (u16*)a.dk, (u16*)a.dv,
                         (int)a.BH, (int)a.Nq, (int)a.Nk, sl2, scale, a.cu_q, a.cu_k, H, tq, tk);
    };
    if constexpr (D == 256) {  // one kernel per gradient: dV, then dK
      run(bwd_dkdv<DT, D, CAUSAL, 2, VARLEN>);
      run(bwd_dkdv<DT, D, CAUSAL, 1, VARLEN>);
    } else {
      run(bwd_dkdv<DT, D, CAUSAL, 3, VARLEN>);
    }
  }
  return (int)hipGetLastError();
}

template <int DT, int D>
int dispatch_bwd(const FaBwdLaunch& a, float sl2, float scale) {
  if (a.cu_q)
    return a.causal ? launch_bwd<DT, D, true, true>(a, sl2, scale) : launch_bwd<DT, D, false, true>(a, sl2, scale);
  return a.causal ? launch_bwd<DT, D, true, false>(a, sl2, scale) : launch_bwd<DT, D, false, false>(a, sl2, scale);
}

}  // namespace

#ifdef FA_BWD_SMALL_D

int fa_launch_bwd_small_d(const FaBwdLaunch& a, float sl2, float scale) {
  if (a.dtype == kBF16)
    return a.D == 32 ? dispatch_bwd<kBF16, 32>(a, sl2, scale) : dispatch_bwd<kBF16, 64>(a, sl2, scale);
  return a.D == 32 ? dispatch_bwd<kFP16, 32>(a, sl2, scale) : dispatch_bwd<kFP16, 64>(a, sl2, scale);
}

#else

int fa_launch_bwd(const FaBwdLaunch& a) {
  const float sl2 = (float)(a.scale * 1.4426950408889634074);
  const float scale = (float)a.scale;
  (void)hipGetLastError();  // clear a stale error so that the check below is ours
  if (a.dtype != kBF16 && a.dtype != kFP16) return fa_launch_bwd32(a, sl2, scale);
  if (a.D < 128) return fa_launch_bwd_small_d(a, sl2, scale);
  if (a.D == 256)
    return a.dtype == kBF16 ? dispatch_bwd<kBF16, 256>(a, sl2, scale) : dispatch_bwd<kFP16, 256>(a, sl2, scale);
  return a.dtype == kBF16 ? dispatch_bwd<kBF16, 128>(a, sl2, scale) : dispatch_bwd<kFP16, 128>(a, sl2, scale);
}

#endif  // FA_BWD_SMALL_D
