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
//  * bwd_prep: delta and LSE * log2(e) per query row, into the workspace
//    (before bwd_dq_rs; bwd_dq computes its rows' values itself);
//  * bwd_dq: one workgroup per (batch*head, 256 query rows), 8 waves of 32
//    rows (the forward's shape): K/V tiles stream through the same 4-stage
//    direct-to-LDS ring; per tile S^T = K Q^T, dP^T = V dO^T, then
//    dQ^T += K^T dS^T (K read transposed);
//  * bwd_dkdv (D = 32, 64): one workgroup per (batch*head, 128 keys), 4
//    waves of 32 keys (one wave per SIMD); Q/dO tiles of 64 query
//    rows plus their LSE and delta stream through a 4-stage ring; per tile
//    S = Q K^T, dP = dO V^T (the wave's keys along the MFMA N dimension, so
//    P and dS come out in the B-operand layout of the next products), then
//    dV^T += dO^T P and dK^T += Q^T dS (dO and Q read transposed);
//  * bwd_dkdv2 (D = 128 and 256): the same products with 8 waves, two per
//    key group on one SIMD: one computes S, P and dV, the other dP, dS and
//    dK with the P its sibling passes through LDS, so that each holds one
//    fragment and one gradient and two waves fit each SIMD (bwd_dkdv, one
//    wave per key group, serves D = 32 and 64).
// S and dP are recomputed in both kernels: seven tile products instead of
// the five a single kernel with atomic dQ updates would need.
// At D = 256, and at D = 128 on grids of fewer 256-row workgroups than CUs,
// the dQ kernel is bwd_dq_rs (score and dQ waves sharing each SIMD, 32-key
// tiles, 128 rows a workgroup); at D = 256 bwd_dkdv2 streams 32-row Q/dO
// tiles.
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

// Waves per workgroup of bwd_dq (32 query rows each, two waves per SIMD) and
// stages of the LDS rings of bwd_dq and bwd_dkdv (three tiles in flight).
// D = 256 (and small grids at D = 128) run bwd_dq_rs instead.
constexpr int kWavesDQ = 8;
constexpr int kStagesBwd = 4;

// ---------------------------------------------------------------------------
// Direct-to-LDS loads the compiler does not track (the kernels at D <= 128).
// ---------------------------------------------------------------------------
// The compiler's tracking of direct-to-LDS writes took some reads of one
// ring stage for reads of the stage being loaded and waited for loads still
// in flight (a vmcnt wait in one tile of three, in several of these
// kernels).  dma_to_lds_u writes the same instruction as assembly, which its
// wait-count insertion does not see.  A kernel using it waits for its own
// loads explicitly (a vmcnt count and a barrier before a stage is read,
// which is what orders the reads after these writes; loads complete in
// order) and calls settle_loads on the registers of its other global loads.

// A resource with base and size moved to scalar registers, as the resource
// operand of the assembly load must be (both are wave-uniform, but the
// compiler cannot always prove it, e.g. for offsets read from the
// packed-sequence tables).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, int off, int total) {
  const unsigned long long b = (unsigned long long)((const unsigned char*)base + off);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const int n = __builtin_amdgcn_readfirstlane(total - off > 0 ? total - off : 0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((unsigned long long)hi << 32) | lo), 0, n, kBufFlags);
}

// One direct-to-LDS buffer load: BYTES (16 or 4) per lane from byte `voff`
// of `r` into LDS from `dst` on (lane i's bytes at dst + BYTES i; the LDS
// address goes through M0).  The leading s_nop covers the wait states a
// VALU write of an SGPR (the resource or the M0 value) needs before a
// vector memory instruction reads it; the one after the M0 write, those of
// the M0 write.
template <int BYTES>
__device__ __forceinline__ void dma_to_lds_u(__amdgpu_buffer_rsrc_t r, const unsigned char* dst, int voff) {
  static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword");
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(__SIZE_TYPE__)(lds_void*)dst);
  if constexpr (BYTES == 16)
    asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                 :: "v"(voff), "s"(m0), "s"(r));
  else
    asm volatile("s_nop 4\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, 0 offen lds"
                 :: "v"(voff), "s"(m0), "s"(r));
}

// issue_tile16 (the same pieces into the same layout) with these loads.
template <int D, int NW, int BC = 64>
__device__ __forceinline__ void issue_tile16_u(const u16* Kh, const u16* Vh, int kbytes, int t,
                                               unsigned char* dst, const Wave16& w) {
  static_assert(BC % 16 == 0 && BC * D * 2 % 1024 == 0, "whole 16-row groups and 1 KB pieces");
  constexpr int TILEB = BC * D * 2;
  constexpr int NG = TILEB / 1024;
  const auto rk = make_rsrc_uniform(Kh, t * TILEB, kbytes);
  const auto rv = make_rsrc_uniform(Vh, t * TILEB, kbytes);
#pragma unroll
  for (int I = 0; I < (NG + NW - 1) / NW; ++I) {
    const int G = w.wave + NW * I;
    if (G < NG) {
      const int go = dma_src_off<D>(G, w.lane);
      dma_to_lds_u<16>(rk, dst + G * 1024, go);
      dma_to_lds_u<16>(rv, dst + TILEB + G * 1024, go);
    }
  }
}

// Make the compiler wait here for the global loads that produced these
// registers (it waits for a load before the first instruction that reads
// its result; this empty assembly reads them all).  Called once, after the
// first tiles' loads: the compiler does not count those, so it would
// otherwise keep treating the fragment loads as possibly in flight and wait
// for them again inside the tile loop, where its count would also wait for
// the tile loads.
template <int N>
__device__ __forceinline__ void settle_loads(const u32x4 (&f)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(f[i]));
}
__device__ __forceinline__ void settle_loads(float a) { asm volatile("" ::"v"(a)); }

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
                                             int row_byte, int hf) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 v;
      v[0] = pack2<DT>(acc[dt][4 * g + 0] * mul, acc[dt][4 * g + 1] * mul);
      v[1] = pack2<DT>(acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul);
      __builtin_amdgcn_raw_buffer_store_b64(v, r, row_byte + (32 * dt + 8 * g + 4 * hf) * 2, 0, 0);
    }
}

// Fragment of 32 rows of a 16-bit [N, D] tensor in the B-operand layout of
// v_mfma_f32_32x32x16: lane l holds row `row0 + l % 32`, columns
// 16 kk + 8 (l / 32) .. +7; rows past `rows` read as zero.
template <int D>
__device__ __forceinline__ void load_frag(u32x4 (&f)[D / 16], const u16* base, int rows, int row0,
                                          const Wave16& w) {
  const auto r = make_rsrc_at(base, row0 * D * 2, rows * D * 2);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    f[kk] = __builtin_amdgcn_raw_buffer_load_b128(r, w.l32 * D * 2 + (16 * kk + 8 * w.hf) * 2, 0, 0);
}

// Query tile of a dQ workgroup: the forward's order (tile_of_block: the
// heaviest causal tiles first) for causal and packed grids; otherwise, when
// the grid divides by the 8 XCDs (block ids go to them in turn), each XCD
// takes a contiguous run of heads with all their query tiles, so that the
// workgroups streaming one head's K/V tiles at the same time share an L2.
template <bool ORDERED>
__device__ __forceinline__ void dq_block(int nqt, int BH, int& bh, int& qt) {
  const int n = BH * nqt, bid = blockIdx.x;
  if (!ORDERED && n % 8 == 0) {
    const int v = (bid & 7) * (n >> 3) + (bid >> 3);
    bh = v / nqt;
    qt = v % nqt;
  } else {
    tile_of_block(nqt, BH, bh, qt);
  }
}

// ---------------------------------------------------------------------------
// dQ kernel.
// ---------------------------------------------------------------------------
template <int DT, int D, bool CAUSAL>
__device__ __forceinline__ void dq_tile(const u16* Kh, const u16* Vh, int kbytes, int j, int nt,
                                        const unsigned char* src, unsigned char* dst, const Wave16& w,
                                        const u32x4 (&qf)[D / 16], const u32x4 (&dof)[D / 16],
                                        f32x16 (&acc)[D / 32], float lse2, float delta, float sl2) {
  constexpr int BC = 64, TILEB = BC * D * 2, NKK = D / 16, NDT = D / 32, NW = kWavesDQ, ST = kStagesBwd;
  const int k0 = j * BC;
  const unsigned char* ks = src;
  const unsigned char* vs = src + TILEB;
  // Tile j is complete since the previous barrier; wait for tile j+1, then
  // refill the stage of tile j-1.
  static_assert(D <= 128 && ST == 4, "D = 256 runs bwd_dq_rs");
  wait_tile_and_barrier(j + 2 < nt ? loads_per_tile<D, NW>(w.wave) : 0);
  if (j + ST - 1 < nt) issue_tile16_u<D, NW>(Kh, Vh, kbytes, j + ST - 1, dst, w);
  if (k0 >= w.wkend) return;
  const bool need_mask = k0 + BC - 1 > w.wklim;  // causal diagonal or past Nk
  const int lim = w.klim - (k0 + 4 * w.hf);
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    f32x16 s = {}, dp = {};
    if constexpr (D == 128) {
      // S and dP MFMAs interleaved, operands read PRE MFMAs ahead; then the
      // K^T operands of this block's dQ MFMAs, read now so that the softmax
      // hides their latency (6 ahead leaves exactly 256 VGPRs; 8 spills).
      constexpr int NS = 2 * NKK, PRE = 6;
      u32x4 op[NS];
#pragma unroll
      for (int i = 0; i < PRE; ++i)
        op[i] = (i & 1) ? ks_operand<D>(vs, w, n * NKK + (i >> 1)) : ks_operand<D>(ks, w, n * NKK + (i >> 1));
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + PRE < NS) {
          const int ip = i + PRE;
          op[ip] = (ip & 1) ? ks_operand<D>(vs, w, n * NKK + (ip >> 1)) : ks_operand<D>(ks, w, n * NKK + (ip >> 1));
        }
        if (i & 1)
          dp = mfma_32x32x16<DT>(op[i], dof[i >> 1], dp);
        else
          s = mfma_32x32x16<DT>(op[i], qf[i >> 1], s);
      }
    } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s = mfma_32x32x16<DT>(ks_operand<D>(ks, w, n * NKK + kk), qf[kk], s);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) dp = mfma_32x32x16<DT>(ks_operand<D>(vs, w, n * NKK + kk), dof[kk], dp);
    }
    u32x4 kt[2 * NDT];
    if constexpr (D == 128) {
#pragma unroll
      for (int i = 0; i < 2 * NDT; ++i) kt[i] = vt_operand<D>(ks, w, 4 * (i >> 1) + 2 * n + (i & 1));
    }
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
        acc[dt] = mfma_32x32x16<DT>(D == 128 ? kt[2 * dt + hh] : vt_operand<D>(ks, w, 4 * dt + 2 * n + hh), dsf[hh],
                                    acc[dt]);
  }
}

// VARLEN: packed sequences (the rows of head_rows); a workgroup past its
// sequence's queries exits, a sequence without keys gets dQ = 0.
// The kernel also computes its rows' statistics (what bwd_prep computes for
// the D = 256 and fp32 paths): delta = sum_d dO[d] O[d] in fp32 from the
// stored 16-bit values, from the dO fragment it holds and the same fragment
// of O, and lse2 = LSE log2(e); it uses them and stores them for the dK/dV
// kernel that follows on the stream.
template <int DT, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(64 * kWavesDQ, 1) void bwd_dq(const u16* __restrict__ Qg, const u16* __restrict__ Kg,
                                                          const u16* __restrict__ Vg, const u16* __restrict__ dOg,
                                                          const u16* __restrict__ Og, const float* __restrict__ lseg,
                                                          float* __restrict__ lse2g,
                                                          float* __restrict__ deltag, u16* __restrict__ dQg,
                                                          int BH, int Nq, int Nk, int nqt, float sl2, float scale,
                                                          const int* __restrict__ cuq, const int* __restrict__ cuk,
                                                          int H, int tq, int tk) {
  constexpr int BC = 64, ROWB = D * 2, TILEB = BC * ROWB, NW = kWavesDQ, BR = 32 * NW;
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[2 * TILEB];

  Wave16 w;
  const int tid = threadIdx.x;
  w.lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.hf = w.lane >> 5;
  w.l32 = w.lane & 31;
  int bh, qt;
  dq_block<CAUSAL || VARLEN>(nqt, BH, bh, qt);
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

  u32x4 qf[D / 16], dof[D / 16], of[D / 16];
  load_frag<D>(qf, Qg + hr.qo, nq, w.wq0, w);
  load_frag<D>(dof, dOg + hr.qo, nq, w.wq0, w);
  load_frag<D>(of, Og + hr.qo, nq, w.wq0, w);
  const float lse =
      __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(lseg + hr.so, nq * 4), myq * 4, 0, 0));

  // (a sequence without keys has no tile: nothing may be left in flight)
  if (!VARLEN || nt > 0) issue_tile16_u<D, NW>(Kh, Vh, kbytes, 0, stage0, w);
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  if (nt > 1) issue_tile16_u<D, NW>(Kh, Vh, kbytes, 1, stage1, w);
  // Waits for the fragments and LSE (and with them tiles 0 and 1).
  settle_loads(qf);
  settle_loads(dof);
  settle_loads(of);
  settle_loads(lse);
  // The rows' statistics.  Lane l holds columns 16 kk + 8 (l / 32) .. +7 of
  // row l % 32 (rows past Nq read as zero): a half-row sum, then the lane
  // pair's.  The stores may still be in flight at the barriers below: they
  // only lengthen the count-based waits, which stay exact for the tile loads
  // (loads complete in order, so an outstanding needed load would leave all
  // later loads outstanding too).
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dsum += lo16<DT>(of[kk][e]) * lo16<DT>(dof[kk][e]) + hi16<DT>(of[kk][e]) * hi16<DT>(dof[kk][e]);
  const float delta = pair_sum(dsum);
  const float lse2 = lse * kLog2e;
  if (w.hf == 0) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse2), make_rsrc(lse2g + hr.so, nq * 4),
                                          myq * 4, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, delta), make_rsrc(deltag + hr.so, nq * 4),
                                          myq * 4, 0, 0);
  }
  if (nt > 2) issue_tile16_u<D, NW>(Kh, Vh, kbytes, 2, stage2, w);
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
  const auto rq = make_rsrc_at(dQg + hr.qo, q0 * ROWB, nq * ROWB);
  store_rows16<DT, D>(acc, scale, rq, (32 * w.wave + w.l32) * ROWB, w.hf);
}

// ---------------------------------------------------------------------------
// Role-split dQ kernel: D = 256, and small grids at D = 128.
// ---------------------------------------------------------------------------
// One workgroup per (batch*head, 128 query rows), 8 waves.  Waves g and g + 4
// share a SIMD and the 32 rows of group g: wave g (the score wave) holds the
// rows' Q and dO fragments and, per 32-key tile, computes S^T = K Q^T,
// dP^T = V dO^T, P and dS = P (dP - delta), and leaves dS (rounded to 16
// bits) in LDS; wave g + 4 (the dQ wave) holds the rows' fp32 dQ and one
// tile later adds K^T dS^T, its K^T operands read from the same K tile.  One
// wave holding both fragments and dQ (64 + 64 + 128 registers at D = 256)
// would fill a SIMD alone; split, two waves share each SIMD.  At D = 128
// (124 registers, 80 KB of LDS) two workgroups share a CU, and the 128-row
// workgroups double the grid of bwd_dq's 256-row ones, which is what pays
// where that grid leaves CUs idle.  K and V
// tiles stream through two 4-stage rings (a K tile is read in its own
// period and in the next); in period p every wave meets the others once (K
// and V tile p are then complete), starts the loads of K and V tile p+2, and
// the score waves handle tile p while the dQ waves handle tile p-1.
template <int D_>
struct Dqrs {
  static constexpr int D = D_, BC = 32, ROWB = D * 2, TILEB = BC * ROWB, NKK = D / 16, NDT = D / 32;
  static constexpr int kPieces = TILEB / 1024 / 8;  // 1 KB pieces per wave, tensor and tile
  static constexpr int kLoads = 2 * kPieces;        // direct-to-LDS loads per wave and period
  static constexpr int XG = 2 * 64;                 // u32x4 of dS per group and buffer
  static_assert(kPieces >= 1 && TILEB % 8192 == 0, "whole 1 KB pieces for each of 8 waves");
};

// One 1 KB direct-to-LDS load: 16 bytes a lane from byte `go` of `r`.
__device__ __forceinline__ void dqrs_piece(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int go) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, go, 0, 0, 0);
}

// This wave's two 1 KB pieces of 32-row tile t of one [N, 256] tensor.
template <int D>
__device__ __forceinline__ void dqrs_issue(const u16* Xh, int kbytes, int t, unsigned char* dst, const Wave16& w) {
  const auto r = make_rsrc_at(Xh, t * Dqrs<D>::TILEB, kbytes);
#pragma unroll
  for (int I = 0; I < Dqrs<D>::kPieces; ++I) {
    const int G = w.wave + 8 * I;
    dqrs_piece(r, dst + G * 1024, dma_src_off<D>(G, w.lane));
  }
}

// Score wave, tile j (K stage ks, V stage vs): S and dP (MFMAs interleaved,
// operands read 4 ahead), P = exp2(s scale log2 e - LSE log2 e) (masked keys
// 0), dS = P (dP - delta), packed to 16 bits into xo.
template <int DT, int D>
__device__ __forceinline__ void dqrs_score(int j, const unsigned char* ks, const unsigned char* vs, u32x4* xo,
                                           const Wave16& w, const u32x4 (&qf)[Dqrs<D>::NKK],
                                           const u32x4 (&dof)[Dqrs<D>::NKK], float lse2, float delta, float sl2) {
  using S = Dqrs<D>;
  constexpr int BC = S::BC, NKK = S::NKK;
  const int k0 = j * BC;
  if (k0 >= w.wkend) return;
  constexpr int NS = 2 * NKK, PRE = 4;
  f32x16 s = {}, dp = {};
  u32x4 op[NS];
#pragma unroll
  for (int i = 0; i < PRE; ++i) op[i] = (i & 1) ? ks_operand<D>(vs, w, i >> 1) : ks_operand<D>(ks, w, i >> 1);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int ip = i + PRE;
    if (ip < NS) op[ip] = (ip & 1) ? ks_operand<D>(vs, w, ip >> 1) : ks_operand<D>(ks, w, ip >> 1);
    if (i & 1)
      dp = mfma_32x32x16<DT>(op[i], dof[i >> 1], dp);
    else
      s = mfma_32x32x16<DT>(op[i], qf[i >> 1], s);
  }
  const bool need_mask = k0 + BC - 1 > w.wklim;  // causal diagonal or past Nk
  const int lim = w.klim - (k0 + 4 * w.hf);
  float ds[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], sl2, -lse2));
    if (need_mask && 8 * (r >> 2) + (r & 3) > lim) p = 0.f;
    ds[r] = p * (dp[r] - delta);
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    u32x4 d;
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = pack2<DT>(ds[8 * hh + 2 * i], ds[8 * hh + 2 * i + 1]);
    xo[64 * hh + w.lane] = d;
  }
}

// dQ wave, tile jj (K stage ks): dQ^T += K^T dS^T with the dS from xi
// (16-key step major, so consecutive MFMAs use different accumulators).
template <int DT, int D>
__device__ __forceinline__ void dqrs_acc(int jj, const unsigned char* ks, const u32x4* xi, const Wave16& w,
                                         f32x16 (&acc)[Dqrs<D>::NDT]) {
  using S = Dqrs<D>;
  constexpr int BC = S::BC, NDT = S::NDT;
  if (jj * BC >= w.wkend) return;
  constexpr int NG = 2 * NDT, PRE = 4;
  u32x4 op[NG];
#pragma unroll
  for (int i = 0; i < PRE; ++i) op[i] = vt_operand<D, BC>(ks, w, (i % NDT) * 2 + i / NDT);
  const u32x4 d0 = xi[w.lane], d1 = xi[64 + w.lane];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int ip = i + PRE;
    if (ip < NG) op[ip] = vt_operand<D, BC>(ks, w, (ip % NDT) * 2 + ip / NDT);
    acc[i % NDT] = mfma_32x32x16<DT>(op[i], i < NDT ? d0 : d1, acc[i % NDT]);
  }
}

// Period p of one role (P4 = p mod 4: stages p mod 4, buffers p mod 2).
template <int DT, int D, bool SCORE, int P4>
__device__ __forceinline__ void dqrs_period(int p, int nt, const u16* Kh, const u16* Vh, int kbytes,
                                            unsigned char* const (&kr)[4], unsigned char* const (&vr)[4],
                                            u32x4* const (&xb)[2], const Wave16& w, const u32x4 (&qf)[Dqrs<D>::NKK],
                                            const u32x4 (&dof)[Dqrs<D>::NKK], f32x16 (&acc)[Dqrs<D>::NDT], float lse2,
                                            float delta, float sl2) {
  wait_tile_and_barrier(Dqrs<D>::kLoads);
  dqrs_issue<D>(Kh, kbytes, p + 2, kr[(P4 + 2) % 4], w);
  dqrs_issue<D>(Vh, kbytes, p + 2, vr[(P4 + 2) % 4], w);
  if constexpr (SCORE) {
    if (p < nt) dqrs_score<DT, D>(p, kr[P4], vr[P4], xb[P4 % 2], w, qf, dof, lse2, delta, sl2);
  } else {
    if (p >= 1) dqrs_acc<DT, D>(p - 1, kr[(P4 + 3) % 4], xb[(P4 + 1) % 2], w, acc);
  }
}

template <int DT, int D, bool SCORE>
__device__ __forceinline__ void dqrs_loop(int nt, const u16* Kh, const u16* Vh, int kbytes,
                                          unsigned char* const (&kr)[4], unsigned char* const (&vr)[4],
                                          u32x4* const (&xb)[2], const Wave16& w, const u32x4 (&qf)[Dqrs<D>::NKK],
                                          const u32x4 (&dof)[Dqrs<D>::NKK], f32x16 (&acc)[Dqrs<D>::NDT], float lse2,
                                          float delta, float sl2) {
  // K and V tiles 0 and 1; each period then starts both tensors' tile p+2.
  // Loads run past the last tile (reading zeros into stages nobody reads),
  // so that every period waits for the same count.
  dqrs_issue<D>(Kh, kbytes, 0, kr[0], w);
  dqrs_issue<D>(Vh, kbytes, 0, vr[0], w);
  dqrs_issue<D>(Kh, kbytes, 1, kr[1], w);
  dqrs_issue<D>(Vh, kbytes, 1, vr[1], w);
#define DQRS_PERIOD(P4) \
  dqrs_period<DT, D, SCORE, P4>(p + P4, nt, Kh, Vh, kbytes, kr, vr, xb, w, qf, dof, acc, lse2, delta, sl2)
  for (int p = 0; p <= nt; p += 4) {
    DQRS_PERIOD(0);
    if (p + 1 <= nt) DQRS_PERIOD(1);
    if (p + 2 <= nt) DQRS_PERIOD(2);
    if (p + 3 <= nt) DQRS_PERIOD(3);
  }
#undef DQRS_PERIOD
  // The loads past the last tile complete before the workgroup's LDS is
  // released.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); lgkmcnt, expcnt: no wait
}

template <int DT, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(512, 1) void bwd_dq_rs(const u16* __restrict__ Qg, const u16* __restrict__ Kg,
                                                    const u16* __restrict__ Vg, const u16* __restrict__ dOg,
                                                    const float* __restrict__ lse2g,
                                                    const float* __restrict__ deltag, u16* __restrict__ dQg,
                                                    int BH, int Nq, int Nk, int nqt, float sl2, float scale,
                                                    const int* __restrict__ cuq, const int* __restrict__ cuk,
                                                    int H, int tq, int tk) {
  using S = Dqrs<D>;
  constexpr int BC = S::BC, ROWB = S::ROWB, TILEB = S::TILEB, NKK = S::NKK, NDT = S::NDT, XG = S::XG;
  constexpr int BR = 128;
  // Ring stages of 16 KB aligned to their size: none straddles a 64 KB
  // boundary, and as the most aligned arrays they come first (0-128 KB).
  __shared__ __attribute__((aligned(S::TILEB))) unsigned char k0s[TILEB];
  __shared__ __attribute__((aligned(S::TILEB))) unsigned char k1s[TILEB];
  __shared__ __attribute__((aligned(S::TILEB))) unsigned char k2s[TILEB];
  __shared__ __attribute__((aligned(S::TILEB))) unsigned char k3s[TILEB];
  __shared__ __attribute__((aligned(S::TILEB))) unsigned char v0s[TILEB];
  __shared__ __attribute__((aligned(S::TILEB))) unsigned char v1s[TILEB];
  __shared__ __attribute__((aligned(S::TILEB))) unsigned char v2s[TILEB];
  __shared__ __attribute__((aligned(S::TILEB))) unsigned char v3s[TILEB];
  __shared__ u32x4 x0[4 * XG];
  __shared__ u32x4 x1[4 * XG];

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
  const int grp = w.wave & 3;
  const bool score = w.wave < 4;
  w.wq0 = q0 + 32 * grp;
  const int myq = w.wq0 + w.l32;
  w.wkend = CAUSAL ? min(kend, w.wq0 + 32) : kend;
  w.klim = CAUSAL ? min(myq, nk - 1) : nk - 1;
  w.wklim = CAUSAL ? min(w.wq0, nk - 1) : nk - 1;
  init_operand_offsets<D>(w);

  unsigned char* const kr[4] = {k0s, k1s, k2s, k3s};
  unsigned char* const vr[4] = {v0s, v1s, v2s, v3s};
  u32x4* const xb[2] = {x0 + XG * grp, x1 + XG * grp};
  u32x4 qf[NKK], dof[NKK];
  f32x16 acc[NDT];
  if (score) {
    load_frag<D>(qf, Qg + hr.qo, nq, w.wq0, w);
    load_frag<D>(dof, dOg + hr.qo, nq, w.wq0, w);
    const auto rs = make_rsrc(lse2g + hr.so, nq * 4);
    const auto rd = make_rsrc(deltag + hr.so, nq * 4);
    const float lse2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, myq * 4, 0, 0));
    const float delta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, myq * 4, 0, 0));
    dqrs_loop<DT, D, true>(nt, Kh, Vh, kbytes, kr, vr, xb, w, qf, dof, acc, lse2, delta, sl2);
  } else {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
    dqrs_loop<DT, D, false>(nt, Kh, Vh, kbytes, kr, vr, xb, w, qf, dof, acc, 0.f, 0.f, sl2);
    const auto rq = make_rsrc_at(dQg + hr.qo, q0 * ROWB, nq * ROWB);
    store_rows16<DT, D>(acc, scale, rq, (32 * grp + w.l32) * ROWB, w.hf);
  }
}

// Key block of a dK/dV workgroup.  Ordered (causal, packed sequences):
// ascending key blocks over all heads, so that under the causal mask the
// heaviest workgroups start first.  Otherwise, when the grid divides by
// the 8 XCDs (block ids go to them in turn), each XCD takes a contiguous
// run of heads with all their key blocks, so that the workgroups reading
// one head's Q/dO tiles at the same time share that XCD's L2.
template <bool ORDERED>
__device__ __forceinline__ void kv_block(int bid, int BH, int& bh, int& kt) {
  const int n = (int)gridDim.x, nkt = n / BH;
  if (!ORDERED && n % 8 == 0) {
    const int v = (bid & 7) * (n >> 3) + (bid >> 3);
    bh = v / nkt;
    kt = v % nkt;
  } else {
    bh = bid % BH;
    kt = bid / BH;
  }
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
  issue_tile16_u<D, kWavesKV>(Qh, dOh, qbytes, t, dst, w);
  if (w.wave == 0) {
    const auto rl = make_rsrc_uniform(l2h, t * 256, Nq * 4);
    const auto rd = make_rsrc_uniform(dlh, t * 256, Nq * 4);
    dma_to_lds_u<4>(rl, dst + 2 * TILEB, w.lane * 4);
    dma_to_lds_u<4>(rd, dst + 2 * TILEB + 256, w.lane * 4);
  }
}

template <int DT, int D, bool CAUSAL>
__device__ __forceinline__ void kv_tile(const u16* Qh, const u16* dOh, int qbytes, const float* l2h,
                                        const float* dlh, int Nq, int t0, int j, int nt, const unsigned char* src,
                                        unsigned char* dst, const Wave16& w, int wk0, const u32x4 (&kf)[D / 16],
                                        const u32x4 (&vf)[D / 16], f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
                                        float sl2) {
  constexpr int TILEB = 64 * D * 2, NKK = D / 16, NDT = D / 32;
  static_assert(D <= 64, "D = 128 and 256 run bwd_dkdv2");
  const int t = t0 + j;
  const int q0 = 64 * t;
  const unsigned char* qs = src;
  const unsigned char* dos = src + TILEB;
  const unsigned char* st = src + 2 * TILEB;
  // Tile j complete (tile j+1 may still be loading); then tile j+2 into
  // the stage of tile j-1, which every wave is done with.
  wait_tile_and_barrier(j + 1 < nt ? kv_loads_per_tile<D>(w.wave) : 0);
  if (j + 2 < nt) issue_kv_tile<D>(Qh, dOh, qbytes, l2h, dlh, Nq, t + 2, dst, w);
  if (CAUSAL && q0 + 63 < wk0) return;  // every query of the tile precedes the wave's keys
  const bool need_mask = CAUSAL && q0 < wk0 + 31;
  const int mykey = wk0 + w.l32;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    // (fences: one 32-row block at a time, which keeps the kernel within the
    // 168 registers of three waves per SIMD)
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s = mfma_32x32x16<DT>(ks_operand<D>(qs, w, n * NKK + kk), kf[kk], s);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) dp = mfma_32x32x16<DT>(ks_operand<D>(dos, w, n * NKK + kk), vf[kk], dp);
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
        ds[r] = pr * (dp[r] - d4[e]);
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
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        dv[dt] = mfma_32x32x16<DT>(vt_operand<D>(dos, w, 4 * dt + 2 * n + hh), pf[hh], dv[dt]);
        dk[dt] = mfma_32x32x16<DT>(vt_operand<D>(qs, w, 4 * dt + 2 * n + hh), dsf[hh], dk[dt]);
      }
  }
}

// VARLEN: packed sequences (the rows of head_rows); a workgroup past its
// sequence's keys exits, keys of a sequence without queries get zeros.
template <int DT, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(64 * kWavesKV, 3) void bwd_dkdv(const u16* __restrict__ Qg, const u16* __restrict__ Kg,
                                                             const u16* __restrict__ Vg, const u16* __restrict__ dOg,
                                                             const float* __restrict__ lse2g,
                                                             const float* __restrict__ deltag, u16* __restrict__ dKg,
                                                             u16* __restrict__ dVg, int BH, int Nq, int Nk,
                                                             float sl2, float scale, const int* __restrict__ cuq,
                                                             const int* __restrict__ cuk, int H, int tq, int tk) {
  constexpr int ROWB = D * 2, SB = kv_stage_bytes<D>(), BK = 32 * kWavesKV;
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[SB];

  Wave16 w;
  const int tid = threadIdx.x;
  w.lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.hf = w.lane >> 5;
  w.l32 = w.lane & 31;
  int bh, kt;
  kv_block<CAUSAL || VARLEN>(blockIdx.x, BH, bh, kt);
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
  load_frag<D>(vf, Vg + hr.ko, nk, wk0, w);
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dk[dt] = dv[dt] = f32x16{};

  if (nt > 0) {
    issue_kv_tile<D>(Qh, dOh, qbytes, l2h, dlh, nq, t0, stage0, w);
    if (nt > 1) issue_kv_tile<D>(Qh, dOh, qbytes, l2h, dlh, nq, t0 + 1, stage1, w);
    settle_loads(kf);  // waits for the fragments and tiles t0 and t0 + 1
    settle_loads(vf);
    for (int j = 0; j < nt; j += 3) {
      kv_tile<DT, D, CAUSAL>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j, nt, stage0, stage2, w, wk0, kf, vf, dk, dv, sl2);
      if (j + 1 < nt)
        kv_tile<DT, D, CAUSAL>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j + 1, nt, stage1, stage0, w, wk0, kf, vf, dk, dv,
                               sl2);
      if (j + 2 < nt)
        kv_tile<DT, D, CAUSAL>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j + 2, nt, stage2, stage1, w, wk0, kf, vf, dk, dv,
                               sl2);
    }
  }
  const auto rk = make_rsrc_at(dKg + hr.ko, kb0 * ROWB, nk * ROWB);
  const auto rv = make_rsrc_at(dVg + hr.ko, kb0 * ROWB, nk * ROWB);
  store_rows16<DT, D>(dk, scale, rk, (32 * w.wave + w.l32) * ROWB, w.hf);
  store_rows16<DT, D>(dv, 1.0f, rv, (32 * w.wave + w.l32) * ROWB, w.hf);
}

// ---------------------------------------------------------------------------
// dK / dV kernel at D = 128 and 256 with two waves per SIMD.
// ---------------------------------------------------------------------------
// One workgroup per (batch*head, 128 keys), 8 waves.  Waves g and g + 4 share
// a SIMD and key group g (32 keys) and split the work of each Q/dO tile
// between them: wave g (the P wave) computes S = Q K^T, P and
// dV^T += dO^T P; wave g + 4 (the dS wave) computes dP = dO V^T and, with
// the P its sibling leaves in LDS, dS = P (dP - delta) and dK^T += Q^T dS.
// Each wave then holds one fragment (K or V) and one fp32 gradient, which
// fits two waves per SIMD, and one wave's exponentials and softmax-gradient
// arithmetic run while its sibling's MFMAs do.  A tile takes two barriers:
// the first (tile complete) opens the score phase, the second (P written)
// the gradient phase; at D = 128 the dS wave's dK product of a tile runs in
// the next tile's score phase.  Q/dO tiles stream through a 3-stage ring; each key
// group's P travels in fp32, so dS is computed exactly as with one wave.
// At D = 256 the K or V fragment (64 registers) and the fp32 gradient (128)
// of 32 keys leave a wave few registers, so the tiles have 32 rows and the
// operands are read only 2 MFMAs ahead (with 4 ahead the causal kernel
// spilled inside its loop and ran 15% slower).
constexpr int kWavesKV2 = 8;
constexpr int kStagesKV2 = 3;
// Query rows per Q/dO tile: 64 at D = 128; 32 at D = 256, where a stage of
// 64 rows of two tensors (64 KB) leaves no room for three stages.
template <int D>
constexpr int kv2_rows() {
  return D == 256 ? 32 : 64;
}
// Bytes of one stage: the Q tile, the dO tile, then lse2 and delta (256
// bytes each, of which the tile's rows use the first 4 * rows).
template <int D>
constexpr int kv2_stage_bytes() {
  return 2 * kv2_rows<D>() * D * 2 + 1024;
}

// Every wave loads the tile's lse2 and delta rows (the same 512 bytes; the
// copies write identical values), so that all waves issue the same number of
// loads per tile and every wait count is a compile-time constant.
template <int D>
constexpr int kv2_loads_per_tile() {
  static_assert(kv2_rows<D>() * D * 2 / 1024 % kWavesKV2 == 0, "whole 1 KB pieces per wave");
  return 2 * (kv2_rows<D>() * D * 2 / 1024 / kWavesKV2) + 2;
}

template <int D>
__device__ __forceinline__ void issue_kv2_tile(const u16* Qh, const u16* dOh, int qbytes, const float* l2h,
                                               const float* dlh, int Nq, int t, unsigned char* dst, const Wave16& w) {
  constexpr int QR = kv2_rows<D>(), TILEB = QR * D * 2;
  // D = 256 keeps the compiler-tracked loads: with the untracked ones its
  // schedule of this 256-register kernel spilled.
  if constexpr (D != 256) {
    issue_tile16_u<D, kWavesKV2, QR>(Qh, dOh, qbytes, t, dst, w);
    dma_to_lds_u<4>(make_rsrc_uniform(l2h, t * QR * 4, Nq * 4), dst + 2 * TILEB, w.lane * 4);
    dma_to_lds_u<4>(make_rsrc_uniform(dlh, t * QR * 4, Nq * 4), dst + 2 * TILEB + 256, w.lane * 4);
  } else {
    issue_tile16<D, kWavesKV2, QR>(Qh, dOh, qbytes, t, dst, w);
    const auto rl = make_rsrc_at(l2h, t * QR * 4, Nq * 4);
    const auto rd = make_rsrc_at(dlh, t * QR * 4, Nq * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)(dst + 2 * TILEB), 4, w.lane * 4, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)(dst + 2 * TILEB + 256), 4, w.lane * 4, 0, 0, 0);
  }
}

// Meet the other waves once this wave's LDS writes have completed, leaving
// its direct-to-LDS loads in flight (s_waitcnt: vmcnt 63 and expcnt 7, i.e.
// no wait; lgkmcnt 0).
__device__ __forceinline__ void lds_write_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool FIRST, class T>
__device__ __forceinline__ T& pick(T& a, T& b) {
  if constexpr (FIRST) return a;
  else return b;
}

// Score MFMAs of the two-role kernel: x[n] = A(block n) frag^T over the tile
// `as` (Q or dO rows; one 32-row block n per 32 rows), operands read PRE
// MFMAs ahead.
template <int DT, int D>
__device__ __forceinline__ void kv2_scores(const unsigned char* as, const Wave16& w, const u32x4 (&frag)[D / 16],
                                           f32x16 (&x)[kv2_rows<D>() / 32]) {
  constexpr int NB = kv2_rows<D>() / 32, NKK = D / 16, NS = NB * NKK, PRE = D == 256 ? 2 : 8;
  u32x4 op[NS];
#pragma unroll
  for (int i = 0; i < PRE; ++i) op[i] = ks_operand<D>(as, w, i);
#pragma unroll
  for (int n = 0; n < NB; ++n) x[n] = f32x16{};
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i + PRE < NS) op[i + PRE] = ks_operand<D>(as, w, i + PRE);
    x[i / NKK] = mfma_32x32x16<DT>(op[i], frag[i % NKK], x[i / NKK]);
  }
}

// Gradient MFMAs of the two-role kernel: acc[dt] += A^T pk over the tile `gs`
// (dO rows for dV, Q rows for dK) read transposed; operand i is
// dt = i / KS and 16-row step g = i % KS (block g / 2, half g % 2), with KS
// the tile's 16-row steps.
template <int DT, int D>
__device__ __forceinline__ void kv2_grads(const unsigned char* gs, const Wave16& w,
                                          const u32x4 (&pk)[kv2_rows<D>() / 32][2], f32x16 (&acc)[D / 32]) {
  constexpr int QR = kv2_rows<D>(), KS = QR / 16, NG = KS * (D / 32), PRE = D == 256 ? 2 : 8;
  u32x4 op[NG];
#pragma unroll
  for (int i = 0; i < PRE; ++i) op[i] = vt_operand<D, QR>(gs, w, i);
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    if (i + PRE < NG) op[i + PRE] = vt_operand<D, QR>(gs, w, i + PRE);
    const int g = i % KS;  // 16-row step: block g / 2, half g % 2
    acc[i / KS] = mfma_32x32x16<DT>(op[i], pk[g >> 1][g & 1], acc[i / KS]);
  }
}

// Tile j of the two-role kernel.  `frag` is the wave's K (P wave) or V (dS
// wave) fragment, `acc` its dV^T or dK^T accumulator, `xp` the key group's
// P exchange area (32 floats per tile row: chunk c = 4n + g of lane l at
// xp[4 (64 c + l)], the values of rows 32n + 8g + 4hf + 0..3).
template <int DT, int D, bool CAUSAL, bool PW>
__device__ __forceinline__ void kv2_tile(const u16* Qh, const u16* dOh, int qbytes, const float* l2h,
                                         const float* dlh, int Nq, int t0, int j, int nt, const unsigned char* src,
                                         unsigned char* dst, float* xp, const Wave16& w, int wk0,
                                         const u32x4 (&frag)[D / 16], f32x16 (&acc)[D / 32], float sl2,
                                         u32x4 (&pk_loop)[kv2_rows<D>() / 32][2], bool& prev_live) {
  constexpr int QR = kv2_rows<D>(), NB = QR / 32, TILEB = QR * D * 2;
  const int t = t0 + j;
  const int q0 = QR * t;
  const unsigned char* qs = src;
  const unsigned char* dos = src + TILEB;
  const unsigned char* st = src + 2 * TILEB;
  // Tile j+1 is always in flight: the loads run two tiles past the last one
  // (rows past Nq, read as zeros and never used), so that every tile waits
  // for the same fixed count.
  // At D = 128 the dS wave adds Q^T dS one tile late, in the next tile's
  // score phase, beside its sibling's score MFMAs and exponentials (the
  // second phase then holds the dV MFMAs against the dS arithmetic), and
  // the tile j+2 loads wait for the second barrier, as they go into the
  // stage whose Q rows that late product reads.  At D = 256 this order
  // measured slower.
  constexpr bool kLate = D != 256;
  // P wave: P packed for dV; dS wave: dS packed for dK (kept across tiles
  // only where the dS wave's product runs late).
  u32x4 pk_tile[NB][2];
  u32x4 (&pk)[NB][2] = pick<kLate>(pk_loop, pk_tile);
  wait_tile_and_barrier(kv2_loads_per_tile<D>());
  if constexpr (!kLate) issue_kv2_tile<D>(Qh, dOh, qbytes, l2h, dlh, Nq, t + kStagesKV2 - 1, dst, w);
  // No query of the tile sees the group's keys (causal): nothing to do, but
  // both barriers are still met.
  const bool live = !(CAUSAL && q0 + QR - 1 < wk0);
  // dS wave: dK^T += Q^T dS of the previous tile (its Q rows in `dst`).
  if constexpr (kLate && !PW) {
    if (prev_live) kv2_grads<DT, D>(dst, w, pk, acc);
  }
  // Queries of the tile below `qlim` (relative to q0) precede this lane's key.
  const int qlim = (CAUSAL && q0 < wk0 + 31) ? wk0 + w.l32 - q0 : 0;
  // Lane l holds key wk0 + l % 32 and queries q0 + 32n + 8g + 4hf + e (r = 4g + e).
  f32x16 x[NB];
  if (live) {
    // Score phase: S = Q K^T (P wave) or dP = dO V^T (dS wave), every block.
    kv2_scores<DT, D>(PW ? qs : dos, w, frag, x);
    if constexpr (PW) {
      // P = exp2(s scale log2 e - LSE log2 e), 0 where masked; fp32 to the
      // sibling, rounded to 16 bits for dV.
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qo = 32 * n + 8 * g + 4 * w.hf;
          const f32x4 l4 = *(const f32x4*)(st + qo * 4);
          f32x4 p4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(x[n][4 * g + e], sl2, -l4[e]));
            p4[e] = qo + e < qlim ? 0.f : pr;
            x[n][4 * g + e] = p4[e];
          }
          *(f32x4*)(xp + 4 * (64 * (4 * n + g) + w.lane)) = p4;
        }
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[n][hh][i] = pack2<DT>(x[n][8 * hh + 2 * i], x[n][8 * hh + 2 * i + 1]);
    }
  }
  lds_write_barrier();
  if constexpr (kLate) issue_kv2_tile<D>(Qh, dOh, qbytes, l2h, dlh, Nq, t + kStagesKV2 - 1, dst, w);
  if (live) {
    if constexpr (!PW) {
      // dS = P (dP - delta), rounded to 16 bits.
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        float ds[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qo = 32 * n + 8 * g + 4 * w.hf;
          const f32x4 d4 = *(const f32x4*)(st + 256 + qo * 4);
          const f32x4 p4 = *(const f32x4*)(xp + 4 * (64 * (4 * n + g) + w.lane));
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[4 * g + e] = p4[e] * (x[n][4 * g + e] - d4[e]);
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[n][hh][i] = pack2<DT>(ds[8 * hh + 2 * i], ds[8 * hh + 2 * i + 1]);
      }
    }
    // Gradient phase: dV^T += dO^T P (P wave) or dK^T += Q^T dS (dS wave;
    // at D = 128 only after the last tile).
    if (PW || !kLate || j + 1 == nt) kv2_grads<DT, D>(PW ? dos : qs, w, pk, acc);
  }
  prev_live = live;
}

// The tile loop of one role over the 3-stage ring (stages passed as the
// distinct __shared__ arrays they are).
template <int DT, int D, bool CAUSAL, bool PW>
__device__ __forceinline__ void kv2_loop(const u16* Qh, const u16* dOh, int qbytes, const float* l2h,
                                         const float* dlh, int nq, int t0, int nt, unsigned char* s0,
                                         unsigned char* s1, unsigned char* s2, float* xp, const Wave16& w, int wk0,
                                         const u32x4 (&frag)[D / 16], f32x16 (&acc)[D / 32], float sl2) {
  issue_kv2_tile<D>(Qh, dOh, qbytes, l2h, dlh, nq, t0, s0, w);
  issue_kv2_tile<D>(Qh, dOh, qbytes, l2h, dlh, nq, t0 + 1, s1, w);
  // Waits for the fragment and tiles t0 and t0 + 1 (the compiler-tracked
  // loads at D = 256 need no such wait).
  if constexpr (D != 256) settle_loads(frag);
  u32x4 pk[kv2_rows<D>() / 32][2];  // the dS wave's dS of the previous tile (D = 128)
  bool prev_live = false;
  for (int j = 0; j < nt; j += 3) {
    kv2_tile<DT, D, CAUSAL, PW>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j, nt, s0, s2, xp, w, wk0, frag, acc, sl2, pk,
                                prev_live);
    if (j + 1 < nt)
      kv2_tile<DT, D, CAUSAL, PW>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j + 1, nt, s1, s0, xp, w, wk0, frag, acc, sl2,
                                  pk, prev_live);
    if (j + 2 < nt)
      kv2_tile<DT, D, CAUSAL, PW>(Qh, dOh, qbytes, l2h, dlh, nq, t0, j + 2, nt, s2, s1, xp, w, wk0, frag, acc, sl2,
                                  pk, prev_live);
  }
  // The loads past the last tile complete before the workgroup's LDS is
  // released.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); lgkmcnt, expcnt: no wait
}

template <int DT, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(64 * kWavesKV2, 1) void bwd_dkdv2(const u16* __restrict__ Qg, const u16* __restrict__ Kg,
                                                               const u16* __restrict__ Vg, const u16* __restrict__ dOg,
                                                               const float* __restrict__ lse2g,
                                                               const float* __restrict__ deltag, u16* __restrict__ dKg,
                                                               u16* __restrict__ dVg, int BH, int Nq, int Nk,
                                                               float sl2, float scale, const int* __restrict__ cuq,
                                                               const int* __restrict__ cuk, int H, int tq, int tk) {
  constexpr int ROWB = D * 2, SB = kv2_stage_bytes<D>(), BK = 128, QR = kv2_rows<D>();
  static_assert(kStagesKV2 == 3, "the loop below is unrolled for three stages");
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[SB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[SB];
  __shared__ __attribute__((aligned(1024))) float xbuf[4 * 32 * QR];

  Wave16 w;
  const int tid = threadIdx.x;
  w.lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.hf = w.lane >> 5;
  w.l32 = w.lane & 31;
  const int grp = w.wave & 3;
  const bool pwave = w.wave < 4;
  int bh, kt;
  kv_block<CAUSAL || VARLEN>(blockIdx.x, BH, bh, kt);
  const int kb0 = kt * BK;
  const int wk0 = kb0 + 32 * grp;
  const HeadRows hr = head_rows<VARLEN>(bh, Nq, Nk, D, cuq, cuk, H, tq, tk);
  const int nq = hr.nq, nk = hr.nk;
  if (kb0 >= nk) return;  // past this sequence's keys: the whole workgroup
  const u16* Qh = Qg + hr.qo;
  const u16* dOh = dOg + hr.qo;
  const float* l2h = lse2g + hr.so;
  const float* dlh = deltag + hr.so;
  const int qbytes = nq * ROWB;
  const int t0 = CAUSAL ? kb0 / QR : 0;  // first query tile that sees a key of the block
  const int nt = max((nq + QR - 1) / QR - t0, 0);
  w.wq0 = w.wkend = w.wklim = w.klim = 0;  // forward-only fields
  init_operand_offsets<D>(w);
  float* xp = xbuf + 32 * QR * grp;

  u32x4 frag[D / 16];
  load_frag<D>(frag, (pwave ? Kg : Vg) + hr.ko, nk, wk0, w);
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  // Each role runs its own copy of the loop (the same barriers in the same
  // order), so that its LDS reads name their arrays directly.
  if (nt > 0) {
    if (pwave)
      kv2_loop<DT, D, CAUSAL, true>(Qh, dOh, qbytes, l2h, dlh, nq, t0, nt, stage0, stage1, stage2, xp, w, wk0, frag,
                                    acc, sl2);
    else
      kv2_loop<DT, D, CAUSAL, false>(Qh, dOh, qbytes, l2h, dlh, nq, t0, nt, stage0, stage1, stage2, xp, w, wk0, frag,
                                     acc, sl2);
  }
  const int row = (32 * grp + w.l32) * ROWB;
  if (pwave) {
    const auto rv = make_rsrc_at(dVg + hr.ko, kb0 * ROWB, nk * ROWB);
    store_rows16<DT, D>(acc, 1.0f, rv, row, w.hf);
  } else {
    const auto rk = make_rsrc_at(dKg + hr.ko, kb0 * ROWB, nk * ROWB);
    store_rows16<DT, D>(acc, scale, rk, row, w.hf);
  }
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
    int rc = 0;
    // The role-split dQ kernel (128 query rows a workgroup) at D = 256, and
    // at D = 128 where the 256-row kernel would leave CUs without a
    // workgroup; it takes its row statistics from bwd_prep.
    bool rs = false;
    if constexpr (D >= 128)
      rs = D == 256 || a.BH * ((a.Nq + 32 * kWavesDQ - 1) / (32 * kWavesDQ)) < a.cus;
    if (rs) {
      if constexpr (D >= 128) {
        const int64_t threads = rows * (D / 8);
        const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
        rc = launch_kernel(bwd_prep<DT, D>, grid, block, st, (const u16*)a.o, (const u16*)a.dout, a.lse, lse2,
                           delta, rows);
        if (rc != 0) return rc;
        const int nqt = (int)((a.Nq + 127) / 128);
        if (nqt > 0)
          rc = launch_kernel(bwd_dq_rs<DT, D, CAUSAL, VARLEN>, dim3((unsigned)(a.BH * nqt)), dim3(512), st,
                             (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (const u16*)a.dout,
                             (const float*)lse2, (const float*)delta, (u16*)a.dq, (int)a.BH, (int)a.Nq, (int)a.Nk,
                             nqt, sl2, scale, a.cu_q, a.cu_k, H, tq, tk);
      }
    } else if constexpr (D <= 128) {
      constexpr int NWQ = kWavesDQ;
      const int nqt = (int)((a.Nq + 32 * NWQ - 1) / (32 * NWQ));
      if (nqt > 0)
        rc = launch_kernel(bwd_dq<DT, D, CAUSAL, VARLEN>, dim3((unsigned)(a.BH * nqt)), dim3(64 * NWQ), st,
                           (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (const u16*)a.dout, (const u16*)a.o,
                           (const float*)a.lse, lse2, delta, (u16*)a.dq, (int)a.BH, (int)a.Nq, (int)a.Nk, nqt, sl2,
                           scale, a.cu_q, a.cu_k, H, tq, tk);
    }
    if (rc != 0) return rc;
  }
  const int nkt = (int)((a.Nk + 32 * kWavesKV - 1) / (32 * kWavesKV));
  if (nkt > 0) {
    const dim3 grid((unsigned)(a.BH * nkt)), block(64 * kWavesKV);
    auto run = [&](auto kern) {
      return launch_kernel(kern, grid, block, st, (const u16*)a.q, (const u16*)a.k, (const u16*)a.v,
                           (const u16*)a.dout, (const float*)lse2, (const float*)delta, (u16*)a.dk, (u16*)a.dv,
                           (int)a.BH, (int)a.Nq, (int)a.Nk, sl2, scale, a.cu_q, a.cu_k, H, tq, tk);
    };
    if constexpr (D >= 128) {
      return launch_kernel(bwd_dkdv2<DT, D, CAUSAL, VARLEN>, grid, dim3(64 * kWavesKV2), st, (const u16*)a.q,
                           (const u16*)a.k, (const u16*)a.v, (const u16*)a.dout, (const float*)lse2,
                           (const float*)delta, (u16*)a.dk, (u16*)a.dv, (int)a.BH, (int)a.Nq, (int)a.Nk, sl2, scale,
                           a.cu_q, a.cu_k, H, tq, tk);
    } else {
      return run(bwd_dkdv<DT, D, CAUSAL, VARLEN>);
    }
  }
  return 0;
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
  if (a.dtype != kBF16 && a.dtype != kFP16) return fa_launch_bwd32(a, sl2, scale);
  if (a.D < 128) return fa_launch_bwd_small_d(a, sl2, scale);
  if (a.D == 256)
    return a.dtype == kBF16 ? dispatch_bwd<kBF16, 256>(a, sl2, scale) : dispatch_bwd<kFP16, 256>(a, sl2, scale);
  return a.dtype == kBF16 ? dispatch_bwd<kBF16, 128>(a, sl2, scale) : dispatch_bwd<kFP16, 128>(a, sl2, scale);
}

#endif  // FA_BWD_SMALL_D
