// Exact tiled attention forward for gfx950 (CDNA4, MI355X).
//
// The method is the online-softmax tiled attention of "Building a
// FlashAttention-2 Forward Kernel in Pure NumPy" (Architecture Overview;
// Step 3, the running max / correction factor / running sum update; Step 4,
// rescale the accumulator, add P V, divide by the running sum at the end),
// with the loop order of "Hands-on Build Guide: Tiled Self-Attention Kernel
// with Online Softmax in Pure NumPy" (Architecture Overview: one Q tile,
// K/V tiles streamed through it) and the causal tile skipping of "Python
// Attention Mechanisms Explained" (Causal Masking and Incremental Decoding).
//
// Work decomposition: one workgroup per (batch*head, Q tile); each wave owns
// 32 query rows.  16-bit kernel: 8 waves (256 rows), K/V tiles of 64 keys
// loaded straight from HBM into a 4-stage LDS ring (one barrier per tile).
// Role-split kernel (fa_fwd_rs: D = 256, D = 128, and small grids at D = 64):
// two waves per 32-row group, one running the scores and softmax, the other
// O += P V; 16 waves over 256 rows at D = 128, 8 over 128 rows otherwise.
// fp32 kernel: 4 waves (128 rows), K/V staged through registers into a
// double-buffered LDS stage; on grids with at most one such workgroup per CU,
// 32-row workgroups whose waves split each 128-key tile and merge at the end.
//
// Data layout inside a wave (16-bit types): the score tile is computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}: K (from LDS)
// is the A operand, the wave's Q fragment (registers, loaded once) is the B
// operand.  The 32x32 accumulator then holds, in lane l, query row l%32 and
// 16 keys 8*(r/4) + 4*(l/32) + r%4 (r = register 0..15): one query row lives
// in a lane pair (l, l^32), so the row max needs a single exchange across
// the half-waves and the row sum needs none until the end.  P^T is fed
// straight from those registers (rounded to bf16/fp16) as the B operand of
// O^T = V^T P^T, whose A operand comes from the row-major (swizzled) V tile
// in LDS through transposing reads (ds_read_b64_tr_b16).  O^T (fp32) stays
// in registers.  The fp32 path
// uses v_mfma_f32_32x32x2_f32 with the same accumulator layout, P stays
// fp32, and V stays row-major in LDS.
//
// Softmax runs in the log2 domain: t = s * scale * log2(e) (scale = 1/sqrt(D)
// unless given), p = exp2(t - m) on v_exp_f32; LSE = (m + log2 l) * ln 2 at
// the end.
//
// The library compiles this file twice.  Without FA_FWD_D256 it defines the
// fa_launch_fwd* entry points and every kernel up to D = 128; with
// FA_FWD_D256 it defines only the D = 256 launchers (fa_launch_fwd*_d256)
// and fa_fwd_rs, compiled with the MFMA accumulators in VGPRs, which the
// D <= 128 kernels do not want (fa_fwd_rs takes 191 VGPRs and no AGPRs in
// either form).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_device.h"
#include "fa_internal.h"

namespace {

constexpr int kThreads = 256;                     // 4 waves of 64 (fp32 kernel)
constexpr int kBR = 128;                          // query rows per workgroup (fp32 kernel)

// 16-bit kernel shape (fa_fwd_16, D <= 128): a workgroup of waves16<D>()
// waves owns 32 query rows per wave and streams K/V tiles of bc16<D>() keys
// through a 4-stage LDS ring (three tiles in flight while one is consumed;
// each stage holds a K tile and a V tile, 32 KB): 8 waves (256 rows, two
// waves per SIMD) and 64-key tiles, a tile being 32 MFMAs per wave at
// D = 128.  (D = 256 runs fa_fwd_rs below: there the Q fragment and fp32 O of
// 32 rows take more than half of a SIMD's registers.)
#ifndef FA_WAVES16
#define FA_WAVES16 8
#endif
template <int D>
constexpr int waves16() {
  static_assert(D <= 128, "D = 256 runs fa_fwd_rs");
  return FA_WAVES16;
}
// Software pipelining (step16p) pays only where a SIMD runs one wave, i.e.
// in the 4-wave form (small grids at D = 32, see dispatch16): with 8 waves
// the two waves of a SIMD already overlap one's softmax with the other's
// MFMAs, and the fixed interleave of step16p measured slower there (6% at
// D = 128, 22% at D = 64).
template <int D>
constexpr int bc16() {
  return 64;
}

// P = exp2(s sl2 + nm) of a lane's scores (16 per 32-key block), packed to
// 16 bits for the PV product; tl sums the fp32 P (bf16 only, for the LSE),
// tr the P as rounded (the normaliser; for fp16 also the LSE's sum, whose
// rounding error, at most 2^-11 relative, stays below the LSE tolerance).
template <int DT, int NB>
__device__ __forceinline__ void exp_tile(const f32x16 (&s)[NB], float sl2, float nm, u32x4 (&pf)[NB][2],
                                         float& tl, float& tr) {
  float ls0 = 0.f, ls1 = 0.f, lr0 = 0.f;
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][8 * hh + 2 * i], sl2, nm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][8 * hh + 2 * i + 1], sl2, nm));
        pf[n][hh][i] = pack2<DT>(p0, p1);
        if constexpr (DT == kBF16) {
          ls0 += p0;
          ls1 += p1;
        }
        lr0 = add_pair16<DT>(pf[n][hh][i], lr0);
      }
  tl = ls0 + ls1;
  tr = lr0;
}

// Which rule moves the reference max of the 8-wave tile (see tile16):
// the tile's P sums (no per-score max) where that pays: D = 128, and fp16 at
// D = 64, whose kernel still fits the 128 registers that let two workgroups
// share a CU (bf16 at D = 64, with its second sum, does not; and there the
// per-score max is kept).
template <int DT, int D>
constexpr bool sum_checked() {
  return D == 128 || (D == 64 && DT == kFP16);
}

// One K/V tile of the 16-bit kernel (stage `src`).  Tile j is complete in
// LDS since the previous tile's barrier (each barrier waits for the tile
// after its own), so the wave first reads the first K operands of its score
// MFMAs and only then waits for tile j+1 and meets the other waves, which
// hides the reads' latency behind the barrier.  Then it starts the loads of
// tile j+3 into `dst` (the stage of tile j-1, which every wave has finished
// with) and, if it needs tile j, runs S^T = K Q^T, the mask, the
// online-softmax update and O^T += V^T P^T.  `src` and `dst` are distinct
// __shared__ arrays, so the compiler knows the loads in flight never alias
// the operand reads.
template <int DT, int D, bool CAUSAL, int NW = waves16<D>()>
__device__ __forceinline__ void tile16(const u16* Kh, const u16* Vh, int kbytes, int j, int nt,
                                       const unsigned char* src, unsigned char* dst,
                                       const Wave16& w, const u32x4 (&qf)[D / 16],
                                       f32x16 (&oacc)[D / 32], float& mref, float& l, float& lr, float sl2) {
  constexpr int BC = bc16<D>();
  constexpr int TILEB = BC * D * 2;
  constexpr int NKK = D / 16, NDT = D / 32;
  constexpr int NB = BC / 32;  // 32-key score blocks per tile
  // The reference mref moves lazily: under the max rule only when a tile's
  // row max exceeds it by more than kTau (log2 units), so P = exp2(t - mref)
  // stays below 2^kTau; under the sum rule (sum_checked) only when a lane's
  // P sum exceeds 2^15.  O and l always share mref, so O / l and
  // mref + log2(l) are exact whatever mref is.
  constexpr float kTau = 8.0f;
  // S^T = K Q^T.  The K operands are read kPre MFMAs ahead of their use
  // (LDS latency, not bandwidth, bounds these reads); kPre also bounds the
  // LDS reads left in flight at the barrier (a 4-bit counter field).
  constexpr int NQK = NB * NKK, kPre = NKK < 8 ? NKK : 8;

  const int k0 = j * BC;
  const bool mine = k0 < w.wkend;
  const unsigned char* ks = src;
  const unsigned char* vs = src + TILEB;
  u32x4 ka[NQK];
  if (mine) {
#pragma unroll
    for (int i = 0; i < kPre; ++i) ka[i] = ks_operand<D>(ks, w, i);
  }
  // Loads complete in order: only tile j+2's may still be in flight; the
  // kPre reads just issued may be too (older LDS reads have completed).
  wait_tile_and_barrier<kPre>(j + 2 < nt ? loads_per_tile<D, NW, BC>(w.wave) : 0);
  if (j + 3 < nt) issue_tile16<D, NW, BC>(Kh, Vh, kbytes, j + 3, dst, w);

  if (mine) {
    f32x16 s[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) s[n] = f32x16{};
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      if (i + kPre < NQK) ka[i + kPre] = ks_operand<D>(ks, w, i + kPre);
      s[i / NKK] = mfma_32x32x16<DT>(ka[i], qf[i % NKK], s[i / NKK]);
    }
    // The first V^T operands of the PV are read now, so that the softmax
    // hides their latency (at D = 64 the PV is short, and fewer pay off).
    constexpr int KS = BC / 16;  // 16-key PV steps per output block
    constexpr int NPV = KS * NDT, vPre = D == 128 ? 8 : 4;
    u32x4 va[NPV];
#pragma unroll
    for (int i = 0; i < vPre; ++i) va[i] = vt_operand<D, BC>(vs, w, i);
    __builtin_amdgcn_sched_barrier(0);
    // Mask (diagonal and tail tiles only): key = k0 + 4*hf + off(n, r).
    if (k0 + BC - 1 > w.wklim) {
      const int lim = w.klim - (k0 + 4 * w.hf);
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[n][r] = (32 * n + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[n][r];
    }
    u32x4 pf[NB][2];
    if constexpr (sum_checked<DT, D>()) {
      // P = exp2(t - mref) with the current reference first: each P is at
      // most its lane's sum of 32 P, so the reference is moved (and the P
      // recomputed) only when such a sum exceeds kBound = 2^15 (P then fits
      // fp16 and nothing overflows), and on the wave's first tile.
      constexpr float kBound = 32768.0f;
      float tl = 0.f, tr = 0.f;
      bool redo = j == 0;
      if (!redo) {
        exp_tile<DT, NB>(s, sl2, -mref, pf, tl, tr);
        redo = __builtin_amdgcn_ballot_w64(!((DT == kBF16 ? tl : tr) <= kBound)) != 0;
      }
      if (redo) {
        float mx = s[0][0];
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
          for (int r = (n == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[n][r]);
        const float mnew = fmaxf(mref, pair_max(mx * sl2));
        const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
        l *= alpha;
        lr *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        mref = mnew;
        exp_tile<DT, NB>(s, sl2, -mref, pf, tl, tr);
      }
      l += DT == kBF16 ? tl : tr;
      lr += tr;
    } else {
      // Row max of the raw scores (scale > 0 commutes with max).
      float mx = s[0][0];
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = (n == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[n][r]);
      // Half-row max in the scaled log2 domain: a row's max exceeds mref + kTau
      // exactly when one of its halves does, so the lane-pair exchange is only
      // needed on the (rare) path that moves the reference.
      mx *= sl2;
      if (__builtin_amdgcn_ballot_w64(mx > mref + kTau)) {
        const float mnew = fmaxf(mref, pair_max(mx));
        const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
        l *= alpha;
        lr *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        mref = mnew;
      }
      const float nm = -mref;
      // l sums the fp32 P, for the LSE (its rounding to 16 bits would leave a
      // relative error of up to 2^-8 in the LSE of rows that see few keys).
      // bf16: lr sums the P as rounded for the PV product, and O is divided by
      // it, so that the weights applied to the V rows sum to one (a key that
      // dominates its row then passes its V row through exactly, where the
      // fp32 sum would leave P's rounding error, up to 2^-8 relative, on it:
      // with the output's own rounding that exceeded 2e-2 on peaky rows with
      // |O| >= 4).  fp16 rounds P 8 times more finely, and O is divided by l.
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][8 * hh + 2 * i], sl2, nm));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][8 * hh + 2 * i + 1], sl2, nm));
            pf[n][hh][i] = pack2<DT>(p0, p1);
            ls0 += p0;
            ls1 += p1;
            if constexpr (DT == kBF16) lr = add_pair16<DT>(pf[n][hh][i], lr);
          }
      l += ls0 + ls1;
    }
    // O^T += V^T P^T, V^T operands read vPre MFMAs ahead.
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + vPre < NPV) va[i + vPre] = vt_operand<D, BC>(vs, w, i + vPre);
      const int g16 = i % KS;
      oacc[i / KS] = mfma_32x32x16<DT>(va[i], pf[g16 >> 1][g16 & 1], oacc[i / KS]);
    }
  }
}

// Software-pipelined step j of the 16-bit kernel (used by the 4-wave form,
// where one wave per SIMD leaves no other wave to fill the matrix core while
// a wave runs its softmax; see the note above waves16/bc16).  On entry `s` holds the raw scores S(j) of
// tile j, computed by the previous step; the step meets the other waves
// (tile j+1 is then complete, and every wave is done with stage `dst`, tile
// j-1's), starts the loads of tile j+3 into `dst`, and then runs the softmax
// of S(j) with the score MFMAs of tile j+1 (from stage `nxt`) interleaved
// into it, so that the exponentials execute while the matrix core works,
// and last O^T += V^T P^T from stage `cur`.  On return `s` holds S(j+1).
// The sched_barrier after each MFMA and its softmax units fixes that order
// (left to the scheduler, the step measured 5% slower).
template <int DT, int D, bool CAUSAL, int NW = waves16<D>()>
__device__ __forceinline__ void step16p(const u16* Kh, const u16* Vh, int kbytes, int j, int nt,
                                        const unsigned char* cur, const unsigned char* nxt, unsigned char* dst,
                                        const Wave16& w, const u32x4 (&qf)[D / 16], f32x16 (&oacc)[D / 32],
                                        f32x16 (&s)[bc16<D>() / 32], float& mref, float& l, float& lr,
                                        float sl2) {
  constexpr int BC = bc16<D>();
  constexpr int TILEB = BC * D * 2;
  constexpr int NKK = D / 16, NDT = D / 32, NB = BC / 32, KS = BC / 16;
  constexpr int NQK = NB * NKK, NPV = KS * NDT;
  constexpr int NU = 4 * KS;  // units of softmax work: one pair of P values per lane each
  static_assert(NQK % NU == 0 || NU % NQK == 0, "units spread evenly over the score MFMAs");
  constexpr float kTau = 8.0f;  // as in tile16
  constexpr int kPre = 4, vPre = 4;

  wait_tile_and_barrier(j + 2 < nt ? loads_per_tile<D, NW, BC>(w.wave) : 0);
  if (j + 3 < nt) issue_tile16<D, NW, BC>(Kh, Vh, kbytes, j + 3, dst, w);
  const int k0 = j * BC;
  // The wave's last tile also scores stage `nxt` (stale data when tile j+1
  // is not needed or does not exist: the result is never used), which keeps
  // one path through the step.
  if (k0 < w.wkend) {
    const unsigned char* vs = cur + TILEB;
    u32x4 ka[NQK];
#pragma unroll
    for (int i = 0; i < kPre; ++i) ka[i] = ks_operand<D>(nxt, w, i);
    u32x4 va[NPV];
#pragma unroll
    for (int i = 0; i < vPre; ++i) va[i] = vt_operand<D, BC>(vs, w, (i % NDT) * KS + i / NDT);

    // Mask (diagonal and tail tiles only): key = k0 + 4*hf + off(n, r).
    if (k0 + BC - 1 > w.wklim) {
      const int lim = w.klim - (k0 + 4 * w.hf);
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[n][r] = (32 * n + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[n][r];
    }
    float mx = s[0][0];
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = (n == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[n][r]);
    mx *= sl2;
    if (__builtin_amdgcn_ballot_w64(mx > mref + kTau)) {
      const float mnew = fmaxf(mref, pair_max(mx));
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
      l *= alpha;
      lr *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
      mref = mnew;
    }
    const float nm = -mref;
    u32x4 pf[NB][2];
    float ls0 = 0.f, ls1 = 0.f;
    f32x16 sn[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) sn[n] = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
    // S(j+1) = K Q^T, with the units of the softmax of S(j) spread evenly
    // behind its MFMAs; unit u: P values 2q, 2q+1 of 16-key step g = u / 4
    // (block n = g / 2, half hh = g % 2), q = u % 4.
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      if (i + kPre < NQK) ka[i + kPre] = ks_operand<D>(nxt, w, i + kPre);
      sn[i / NKK] = mfma_32x32x16<DT>(ka[i], qf[i % NKK], sn[i / NKK]);
      // Units [u0, u1) follow MFMA i.
      const int u0 = (i * NU) / NQK, u1 = ((i + 1) * NU) / NQK;
#pragma unroll
      for (int u = u0; u < u1; ++u) {
        const int g = u >> 2, n = g >> 1, hh = g & 1, q = u & 3;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][8 * hh + 2 * q], sl2, nm));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][8 * hh + 2 * q + 1], sl2, nm));
        pf[n][hh][q] = pack2<DT>(p0, p1);
        ls0 += p0;
        ls1 += p1;
        if constexpr (DT == kBF16) lr = add_pair16<DT>(pf[n][hh][q], lr);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l += ls0 + ls1;
    // O^T += V^T P^T, 16-key step major (consecutive MFMAs use different
    // accumulators), V^T operands read vPre MFMAs ahead.
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const int ip = i + vPre;
      if (ip < NPV) va[ip] = vt_operand<D, BC>(vs, w, (ip % NDT) * KS + ip / NDT);
      const int g = i / NDT, dt = i % NDT;
      oacc[dt] = mfma_32x32x16<DT>(va[i], pf[g >> 1][g & 1], oacc[dt]);
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) s[n] = sn[n];
  }
}

// Workgroup -> (batch*head, Q tile, key range) of the forward kernels;
// false for a workgroup with nothing to do.
// VARLEN: workgroups go to the 8 XCDs round-robin by block id.  Each XCD
// sweeps all Q tiles of one head (heaviest first) before the next head, so
// that the tiles running together on its 32 CUs share that head's K/V in the
// XCD's L2 (with one head per Q tile at a time, the K/V of the long sequences
// of a packed batch overflowed it).  The grid rounds B*H up to a multiple of
// 8.
// SPLIT: range-major, then Q tiles heaviest first over all heads.
template <bool SPLIT, bool VARLEN>
__device__ __forceinline__ bool fwd_block(int nqt, int BH, int& bh, int& qt, int& split) {
  split = 0;
  if constexpr (VARLEN) {
    const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
    bh = xcd + 8 * (i / nqt);
    qt = nqt - 1 - i % nqt;
    return bh < BH;
  } else if constexpr (SPLIT) {
    const int per = BH * nqt;
    split = blockIdx.x / per;
    const int rem = blockIdx.x - split * per;
    bh = rem % BH;
    qt = nqt - 1 - rem / BH;
  } else {
    tile_of_block(nqt, BH, bh, qt);
  }
  return true;
}

// SPLIT: the grid also runs over key ranges of `split_len` keys; the
// workgroup of range s attends to keys [s split_len, (s+1) split_len) only
// and writes its normalised fp32 partial O_s and LSE_s (rows with no key in
// the range: O_s = 0, LSE_s = -inf) to Po / Pl, laid out [s][B*H][Nq][D] and
// [s][B*H][Nq]; merge_splits combines them.
// VARLEN: packed sequences of different lengths.  q, o are [H, tq, D], k, v
// [H, tk, D] and lse [H, tq]; sequence b owns query rows [cuq[b], cuq[b+1])
// and key rows [cuk[b], cuk[b+1]) (offsets clamped into [0, tq] / [0, tk]);
// BH = B*H, Nq = the longest sequence's query count (sets nqt).  Rows of a
// sequence without keys get O = 0 and LSE = -inf.
template <int DT, int D, bool CAUSAL, bool SPLIT = false, bool VARLEN = false, int NW = waves16<D>()>
__global__ __launch_bounds__(64 * NW, (D == 64 && NW == 8) ? 4 : 1) void fa_fwd_16(const u16* __restrict__ Qg,
                                                           const u16* __restrict__ Kg,
                                                           const u16* __restrict__ Vg,
                                                           u16* __restrict__ Og,
                                                           float* __restrict__ Lg, int BH, int Nq,
                                                           int Nk, int nqt, float sl2, int split_len,
                                                           float* __restrict__ Po, float* __restrict__ Pl,
                                                           const int* __restrict__ cuq, const int* __restrict__ cuk,
                                                           int H, int tq, int tk) {
  constexpr int BC = bc16<D>();          // keys per tile
  constexpr int ROWB = D * 2;             // bytes per row
  constexpr int TILEB = BC * ROWB;        // bytes per K (or V) tile
  constexpr int NKK = D / 16;             // MFMA steps over the head dimension
  constexpr int NDT = D / 32;             // 32-wide output column tiles
  static_assert(NW == waves16<D>() || (NW == 4 && !SPLIT && !VARLEN), "4-wave form: plain forward only");
  constexpr int BR = 32 * NW;              // query rows per workgroup

  // The LDS ring: tile j lives in stage j % 4 (a K tile followed by a V tile).
  __shared__ __attribute__((aligned(1024))) unsigned char stage0[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage1[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage2[2 * TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char stage3[2 * TILEB];

  Wave16 w;
  const int tid = threadIdx.x;
  w.lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  w.hf = w.lane >> 5;
  w.l32 = w.lane & 31;
  int bh, qt, split;
  if (!fwd_block<SPLIT, VARLEN>(nqt, BH, bh, qt, split)) return;
  const int q0 = qt * BR;
  // This head's rows: nq queries at Qh / Oh / Lh, NK keys at Kg + hr.ko.
  const HeadRows hr = head_rows<VARLEN>(bh, Nq, Nk, D, cuq, cuk, H, tq, tk);
  const int nq = hr.nq, NK = hr.nk;
  if (q0 >= nq) return;  // past this sequence's rows: the whole workgroup
  const u16* Qh = Qg + hr.qo;
  u16* Oh = Og + hr.qo;
  float* Lh = Lg + hr.so;
  const size_t koff = hr.ko;
  // This workgroup's keys: [kb, kb + nk) of the head (all of them unless
  // SPLIT); key indices below are relative to kb.
  const int kb = SPLIT ? split * split_len : 0;
  const int nk = SPLIT ? min(split_len, NK - kb) : NK;
  const u16* Kh = Kg + koff + (size_t)kb * D;
  const u16* Vh = Vg + koff + (size_t)kb * D;
  const int kbytes = nk * ROWB;

  const int kend = CAUSAL ? min(nk, min(q0 + BR, nq) - kb) : nk;  // keys [0, kend) are needed
  const int nt = kend > 0 ? (kend + BC - 1) / BC : 0;
  w.wq0 = q0 + 32 * w.wave;
  const int myq = w.wq0 + w.l32;
  // A wave whose rows all lie past Nq computes nothing.
  w.wkend = w.wq0 >= nq ? 0 : CAUSAL ? min(kend, w.wq0 + 32 - kb) : kend;
  w.klim = CAUSAL ? min(myq - kb, nk - 1) : nk - 1;
  w.wklim = CAUSAL ? min(w.wq0 - kb, nk - 1) : nk - 1;
  init_operand_offsets<D>(w);

  // Q fragment (B operand of S^T): lane holds Q[myq][16*kk + 8*hf .. +7];
  // rows past Nq read as zero.  Issued before the K/V loads: loads complete
  // in order, so waiting for a K/V tile also covers Q.
  u32x4 qf[NKK];
  {
    const auto rQ = make_rsrc_at(Qh, q0 * ROWB, nq * ROWB);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = __builtin_amdgcn_raw_buffer_load_b128(rQ, (32 * w.wave + w.l32) * ROWB + (16 * kk + 8 * w.hf) * 2,
                                                     0, 0);
  }
  // Tiles 0..2 into stages 0..2.
  if ((!SPLIT && !VARLEN) || nt > 0) issue_tile16<D, NW, BC>(Kh, Vh, kbytes, 0, stage0, w);
  if (nt > 1) issue_tile16<D, NW, BC>(Kh, Vh, kbytes, 1, stage1, w);
  if (nt > 2) issue_tile16<D, NW, BC>(Kh, Vh, kbytes, 2, stage2, w);

  float mref = kMinit, l = 0.f, lr = 0.f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};

  // Tile 0 must be complete before its first K operands are read.
  wait_tile_and_barrier(nt > 2 ? loads_per_tile<D, NW, BC>(w.wave) : 0);
  if constexpr (NW == 4) {
    // Pipelined: S(0) first, then each step finishes tile j and scores j+1.
    f32x16 s[BC / 32];
#pragma unroll
    for (int n = 0; n < BC / 32; ++n) s[n] = f32x16{};
    if (0 < w.wkend) {
#pragma unroll
      for (int i = 0; i < (BC / 32) * NKK; ++i)
        s[i / NKK] = mfma_32x32x16<DT>(ks_operand<D>(stage0, w, i), qf[i % NKK], s[i / NKK]);
    }
    for (int j = 0; j < nt; j += 4) {
      step16p<DT, D, CAUSAL, NW>(Kh, Vh, kbytes, j, nt, stage0, stage1, stage3, w, qf, oacc, s, mref, l, lr, sl2);
      if (j + 1 < nt) step16p<DT, D, CAUSAL, NW>(Kh, Vh, kbytes, j + 1, nt, stage1, stage2, stage0, w, qf, oacc, s, mref, l, lr, sl2);
      if (j + 2 < nt) step16p<DT, D, CAUSAL, NW>(Kh, Vh, kbytes, j + 2, nt, stage2, stage3, stage1, w, qf, oacc, s, mref, l, lr, sl2);
      if (j + 3 < nt) step16p<DT, D, CAUSAL, NW>(Kh, Vh, kbytes, j + 3, nt, stage3, stage0, stage2, w, qf, oacc, s, mref, l, lr, sl2);
    }
  } else {
    for (int j = 0; j < nt; j += 4) {
      tile16<DT, D, CAUSAL, NW>(Kh, Vh, kbytes, j, nt, stage0, stage3, w, qf, oacc, mref, l, lr, sl2);
      if (j + 1 < nt) tile16<DT, D, CAUSAL, NW>(Kh, Vh, kbytes, j + 1, nt, stage1, stage0, w, qf, oacc, mref, l, lr, sl2);
      if (j + 2 < nt) tile16<DT, D, CAUSAL, NW>(Kh, Vh, kbytes, j + 2, nt, stage2, stage1, w, qf, oacc, mref, l, lr, sl2);
      if (j + 3 < nt) tile16<DT, D, CAUSAL, NW>(Kh, Vh, kbytes, j + 3, nt, stage3, stage2, w, qf, oacc, mref, l, lr, sl2);
    }
  }

  const float lt = pair_sum(l);
  const float ltr = DT == kBF16 ? pair_sum(lr) : lt;
  if constexpr (SPLIT) {
    // fp32 partial of this key range (rows past Nq dropped by the range check).
    // Stores of 8 bytes, from two address registers so that they are not
    // merged into 16-byte stores: this compiler lets a VALU instruction
    // overwrite the data registers of a 16-byte store right after issuing it,
    // and on gfx950 the store then wrote corrupted data (seen on the first
    // dword, in the last four lanes of each 16).
    const bool none = !(lt > 0.f);
    const float inv = none ? 0.f : 1.0f / ltr;
    const size_t slot = (size_t)split * BH + bh;
    const auto rP = make_rsrc_at(Po + slot * Nq * D, q0 * D * 4, nq * D * 4);
    const int off0 = (32 * w.wave + w.l32) * D * 4 + 4 * w.hf * 4;
    int off1 = off0 + 8;
    asm volatile("" : "+v"(off1));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x2 v0 = {oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv};
        const f32x2 v1 = {oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv};
        const int col = (32 * dt + 8 * g) * 4;
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v0), rP, off0 + col, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v1), rP, off1 + col, 0, 0);
      }
    if (w.hf == 0) {
      const auto rL = make_rsrc_at(Pl + slot * Nq, q0 * 4, nq * 4);
      const float lse = none ? -INFINITY : (mref + __log2f(lt)) * kLn2;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse), rL, (32 * w.wave + w.l32) * 4, 0,
                                            0);
    }
    return;
  }
  // Epilogue: normalise by the combined half-row sums, round to 16 bits,
  // store (rows past Nq are dropped by the buffer range check).
  const bool none = VARLEN && !(lt > 0.f);  // a sequence without keys
  const float inv = none ? 0.f : 1.0f / ltr;
  const auto rO = make_rsrc_at(Oh, q0 * ROWB, nq * ROWB);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 v;
      v[0] = pack2<DT>(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
      v[1] = pack2<DT>(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
      __builtin_amdgcn_raw_buffer_store_b64(v, rO, (32 * w.wave + w.l32) * ROWB + (32 * dt + 8 * g + 4 * w.hf) * 2,
                                            0, 0);
    }
  if (w.hf == 0) {
    const auto rL = make_rsrc_at(Lh, q0 * 4, nq * 4);
    const float lse = none ? -INFINITY : (mref + __log2f(lt)) * kLn2;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse), rL, (32 * w.wave + w.l32) * 4, 0,
                                          0);
  }
}

// ---------------------------------------------------------------------------
// Role-split 16-bit kernel: D = 256, full grids at D = 128, small grids at
// D = 64 and 128.
// ---------------------------------------------------------------------------
// One workgroup of 2 NG waves per (batch*head, 32 NG query rows, key range).
// Waves g and g + NG share a SIMD and the 32 rows of group g.  Wave g, the
// score wave, holds the rows' Q fragment and runs S^T = K Q^T, the mask and
// the online-softmax update of each key tile, and leaves P (rounded to 16
// bits) in LDS; wave g + NG, the PV wave, holds the rows' fp32 O and one tile
// later rescales it (by the factor the score wave leaves, 1 when the
// reference did not move) and adds V^T P^T.  No wave holds both a Q fragment
// and an O accumulator, and one wave's softmax runs beside another's MFMAs.
//  * NG = 4 (8 waves, 128 rows): D = 256, where a wave holding both would
//    need more than half of a SIMD's registers, and grids too small to give
//    the 256-row kernel a workgroup per CU.  K and V tiles stream through
//    two 3-stage rings; in period p every wave meets the others once (K tile
//    p and V tile p-1 are then complete), starts the loads of V tile p+1 and
//    K tile p+2, and the score waves handle tile p while the PV waves handle
//    tile p-1.
//  * NG = 8 (16 waves, 256 rows, four waves per SIMD in 128 registers each):
//    D = 128 on full grids.  The LDS then holds a 3-stage K ring and a
//    2-stage V ring: V tile p is loaded in period p and read in period p+1.
// P and the rescale factors travel through double-buffered LDS areas.
template <int D, int NG>
struct RsShape {
  static constexpr int BC = D == 256 ? 32 : 64;  // keys per tile
  static constexpr int ROWB = D * 2, TILEB = BC * ROWB, NKK = D / 16, NDT = D / 32;
  static constexpr int NB = BC / 32, KS = BC / 16;  // 32-key blocks, 16-key PV steps
  static constexpr int NW = 2 * NG;                 // waves
  static constexpr int NPIECE = TILEB / 1024 / NW;  // 1 KB loads per wave and tile
  static constexpr int VST = NG == 8 ? 2 : 3;       // V ring stages
  // Loads a wave may leave in flight at a period's barrier: the previous
  // period's V and K tiles (VST = 3) or its K tile (VST = 2, whose V tile is
  // read in the period that follows).
  static constexpr int kWait = VST == 3 ? 2 * NPIECE : NPIECE;
  static constexpr int XG = KS * 64;         // u32x4 of P per group and buffer
  static constexpr int PRE = NG == 8 ? 2 : 8;  // operand read-ahead (MFMAs)
  static_assert(NPIECE >= 1 && TILEB % (1024 * NW) == 0, "whole 1 KB pieces for every wave");
  static_assert(kWait < 16, "vmcnt field");
};

// Meet the other waves once at most N of this wave's direct-to-LDS loads
// remain in flight (loads complete in order) and its LDS operations are done.
template <int N>
__device__ __forceinline__ void rs_wait_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);  // vmcnt(N), expcnt: no wait, lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One 1 KB direct-to-LDS load: 16 bytes a lane from byte `go` of `r`.
__device__ __forceinline__ void rs_piece(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int go) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, go, 0, 0, 0);
}

// This wave's 1 KB pieces of tile t of one [N, D] tensor.
template <int D, int NG>
__device__ __forceinline__ void rs_issue(const u16* Xh, int kbytes, int t, unsigned char* dst, const Wave16& w) {
  using S = RsShape<D, NG>;
  const auto r = make_rsrc_at(Xh, t * S::TILEB, kbytes);
#pragma unroll
  for (int I = 0; I < S::NPIECE; ++I) {
    const int G = w.wave + S::NW * I;
    rs_piece(r, dst + G * 1024, dma_src_off<D>(G, w.lane));
  }
}

// Score wave, tile j (K stage ks): S^T, mask, online softmax with the sum
// rule (the reference moves only when a lane's sum of its P exceeds 2^15,
// and on the first tile), then P to xo and O's rescale factor to fo.
template <int DT, int D, int NG>
__device__ __forceinline__ void rs_score(int j, const unsigned char* ks, u32x4* xo, float* fo, const Wave16& w,
                                         const u32x4 (&qf)[D / 16], float& mref, float& l, float& lr, float sl2) {
  using S = RsShape<D, NG>;
  constexpr int NB = S::NB, NKK = S::NKK, BC = S::BC, NQK = NB * NKK, PRE = NQK < S::PRE ? NQK : S::PRE;
  const int k0 = j * BC;
  if (k0 >= w.wkend) return;
  f32x16 s[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) s[n] = f32x16{};
  u32x4 ka[NQK];
#pragma unroll
  for (int i = 0; i < PRE; ++i) ka[i] = ks_operand<D>(ks, w, i);
#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    if (i + PRE < NQK) ka[i + PRE] = ks_operand<D>(ks, w, i + PRE);
    s[i / NKK] = mfma_32x32x16<DT>(ka[i], qf[i % NKK], s[i / NKK]);
  }
  // Mask (diagonal and tail tiles only): key = k0 + 4*hf + 32*n + 8*(r/4) + r%4.
  if (k0 + BC - 1 > w.wklim) {
    const int lim = w.klim - (k0 + 4 * w.hf);
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[n][r] = (32 * n + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[n][r];
  }
  constexpr float kBound = 32768.0f;
  u32x4 pf[NB][2];
  float tl = 0.f, tr = 0.f;
  float fac = 1.0f;
  bool redo = j == 0;
  if (!redo) {
    exp_tile<DT, NB>(s, sl2, -mref, pf, tl, tr);
    redo = __builtin_amdgcn_ballot_w64(!((DT == kBF16 ? tl : tr) <= kBound)) != 0;
  }
  if (redo) {
    float mx = s[0][0];
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int r = (n == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[n][r]);
    const float mnew = fmaxf(mref, pair_max(mx * sl2));
    fac = __builtin_amdgcn_exp2f(mref - mnew);
    l *= fac;
    lr *= fac;
    mref = mnew;
    exp_tile<DT, NB>(s, sl2, -mref, pf, tl, tr);
  }
  l += DT == kBF16 ? tl : tr;
  lr += tr;
#pragma unroll
  for (int g = 0; g < 2 * NB; ++g) xo[64 * g + w.lane] = pf[g >> 1][g & 1];
  fo[w.lane] = fac;
}

// PV wave, tile jj (V stage vs): rescale O where the factor differs from 1,
// then O^T += V^T P^T with the P from xi (16-key step g major, so
// consecutive MFMAs use different accumulators).
template <int DT, int D, int NG>
__device__ __forceinline__ void rs_pv(int jj, const unsigned char* vs, const u32x4* xi, const float* fi,
                                      const Wave16& w, f32x16 (&oacc)[D / 32]) {
  using S = RsShape<D, NG>;
  constexpr int NDT = S::NDT, KS = S::KS, BC = S::BC, NPV = KS * NDT, PRE = S::PRE;
  if (jj * BC >= w.wkend) return;
  u32x4 va[NPV];
#pragma unroll
  for (int i = 0; i < PRE; ++i) va[i] = vt_operand<D, BC>(vs, w, (i % NDT) * KS + i / NDT);
  u32x4 pk[KS];
#pragma unroll
  for (int g = 0; g < KS; ++g) pk[g] = xi[64 * g + w.lane];
  const float a = fi[w.lane];
  if (__builtin_amdgcn_ballot_w64(a != 1.0f)) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= a;
  }
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    const int ip = i + PRE;
    if (ip < NPV) va[ip] = vt_operand<D, BC>(vs, w, (ip % NDT) * KS + ip / NDT);
    oacc[i % NDT] = mfma_32x32x16<DT>(va[i], pk[i / NDT], oacc[i % NDT]);
  }
}

// Period p of one role (P6 = p mod 6: K stages p mod 3, V stages p mod VST,
// buffers p mod 2).  V tile p+VST-2 is loaded in period p.
template <int DT, int D, int NG, bool SCORE, int P6>
__device__ __forceinline__ void rs_period(int p, int nt, const u16* Kh, const u16* Vh, int kbytes,
                                          unsigned char* const (&kr)[3], unsigned char* const (&vr)[3],
                                          u32x4* const (&xb)[2],
                                          float* const (&fb)[2], const Wave16& w, const u32x4 (&qf)[D / 16],
                                          f32x16 (&oacc)[D / 32], float& mref, float& l, float& lr, float sl2) {
  using S = RsShape<D, NG>;
  constexpr int VST = S::VST;
  rs_wait_barrier<S::kWait>();
  rs_issue<D, NG>(Vh, kbytes, p + VST - 2, vr[(P6 + VST - 2) % VST], w);
  rs_issue<D, NG>(Kh, kbytes, p + 2, kr[(P6 + 2) % 3], w);
  if constexpr (SCORE) {
    if (p < nt) rs_score<DT, D, NG>(p, kr[P6 % 3], xb[P6 % 2], fb[P6 % 2], w, qf, mref, l, lr, sl2);
  } else {
    if (p >= 1) rs_pv<DT, D, NG>(p - 1, vr[(P6 + VST - 1) % VST], xb[(P6 + 1) % 2], fb[(P6 + 1) % 2], w, oacc);
  }
}

template <int DT, int D, int NG, bool SCORE>
__device__ __forceinline__ void rs_loop(int nt, const u16* Kh, const u16* Vh, int kbytes,
                                        unsigned char* const (&kr)[3], unsigned char* const (&vr)[3],
                                        u32x4* const (&xb)[2], float* const (&fb)[2], const Wave16& w,
                                        const u32x4 (&qf)[D / 16], f32x16 (&oacc)[D / 32], float& mref, float& l,
                                        float& lr, float sl2) {
  // K tiles 0 and 1 (and V tile 0 with three V stages); each period then
  // starts two more tiles.  Loads run past the last tile (reading zeros into
  // stages nobody reads), so that every period waits for the same count.
  rs_issue<D, NG>(Kh, kbytes, 0, kr[0], w);
  rs_issue<D, NG>(Kh, kbytes, 1, kr[1], w);
  if constexpr (RsShape<D, NG>::VST == 3) rs_issue<D, NG>(Vh, kbytes, 0, vr[0], w);
#define RS_PERIOD(P6) \
  rs_period<DT, D, NG, SCORE, P6>(p + P6, nt, Kh, Vh, kbytes, kr, vr, xb, fb, w, qf, oacc, mref, l, lr, sl2)
  for (int p = 0; p <= nt; p += 6) {
    RS_PERIOD(0);
    if (p + 1 <= nt) RS_PERIOD(1);
    if (p + 2 <= nt) RS_PERIOD(2);
    if (p + 3 <= nt) RS_PERIOD(3);
    if (p + 4 <= nt) RS_PERIOD(4);
    if (p + 5 <= nt) RS_PERIOD(5);
  }
#undef RS_PERIOD
  // The loads past the last tile complete before the workgroup's LDS is
  // released.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); lgkmcnt, expcnt: no wait
}

// SPLIT and VARLEN as in fa_fwd_16.
template <int DT, int D, int NG, bool CAUSAL, bool SPLIT = false, bool VARLEN = false>
__global__ __launch_bounds__(128 * NG, 1) void fa_fwd_rs(const u16* __restrict__ Qg, const u16* __restrict__ Kg,
                                                         const u16* __restrict__ Vg, u16* __restrict__ Og,
                                                         float* __restrict__ Lg, int BH, int Nq, int Nk, int nqt,
                                                         float sl2, int split_len, float* __restrict__ Po,
                                                         float* __restrict__ Pl, const int* __restrict__ cuq,
                                                         const int* __restrict__ cuk, int H, int tq, int tk) {
  using S = RsShape<D, NG>;
  constexpr int BR = 32 * NG, BC = S::BC, ROWB = S::ROWB, TILEB = S::TILEB, NKK = S::NKK, NDT = S::NDT, XG = S::XG;
  constexpr int VST = S::VST;
  // Ring stages aligned to their size so that none straddles a 64 KB
  // boundary (the operand reads address one 64 KB window each); as the most
  // aligned arrays they are also laid out first, within the first 96 KB.
  __shared__ __attribute__((aligned(TILEB))) unsigned char k0s[TILEB];
  __shared__ __attribute__((aligned(TILEB))) unsigned char k1s[TILEB];
  __shared__ __attribute__((aligned(TILEB))) unsigned char k2s[TILEB];
  __shared__ __attribute__((aligned(TILEB))) unsigned char v0s[TILEB];
  __shared__ __attribute__((aligned(TILEB))) unsigned char v1s[TILEB];
  __shared__ __attribute__((aligned(VST == 3 ? TILEB : 16))) unsigned char v2s[VST == 3 ? TILEB : 16];
  __shared__ u32x4 x0[NG * XG];
  __shared__ u32x4 x1[NG * XG];
  __shared__ float f0[NG * 64];
  __shared__ float f1[NG * 64];
  __shared__ float finv[NG * 64];

  Wave16 w;
  const int tid = threadIdx.x;
  w.lane = tid & 63;
  w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  w.hf = w.lane >> 5;
  w.l32 = w.lane & 31;
  int bh, qt, split;
  if (!fwd_block<SPLIT, VARLEN>(nqt, BH, bh, qt, split)) return;
  const int q0 = qt * BR;
  const HeadRows hr = head_rows<VARLEN>(bh, Nq, Nk, D, cuq, cuk, H, tq, tk);
  const int nq = hr.nq, NK = hr.nk;
  if (q0 >= nq) return;  // past this sequence's rows: the whole workgroup
  const u16* Qh = Qg + hr.qo;
  u16* Oh = Og + hr.qo;
  float* Lh = Lg + hr.so;
  const int kb = SPLIT ? split * split_len : 0;
  const int nk = SPLIT ? min(split_len, NK - kb) : NK;
  const u16* Kh = Kg + hr.ko + (size_t)kb * D;
  const u16* Vh = Vg + hr.ko + (size_t)kb * D;
  const int kbytes = nk * ROWB;
  const int kend = CAUSAL ? min(nk, min(q0 + BR, nq) - kb) : nk;
  const int nt = kend > 0 ? (kend + BC - 1) / BC : 0;
  const int grp = w.wave & (NG - 1);
  const bool score = w.wave < NG;
  w.wq0 = q0 + 32 * grp;
  const int myq = w.wq0 + w.l32;
  w.wkend = w.wq0 >= nq ? 0 : CAUSAL ? min(kend, w.wq0 + 32 - kb) : kend;
  w.klim = CAUSAL ? min(myq - kb, nk - 1) : nk - 1;
  w.wklim = CAUSAL ? min(w.wq0 - kb, nk - 1) : nk - 1;
  init_operand_offsets<D>(w);

  unsigned char* const kr[3] = {k0s, k1s, k2s};
  unsigned char* const vr[3] = {v0s, v1s, v2s};  // v2s: 3 V stages only
  u32x4* const xb[2] = {x0 + XG * grp, x1 + XG * grp};
  float* const fb[2] = {f0 + 64 * grp, f1 + 64 * grp};
  float* const fi = finv + 64 * grp;

  u32x4 qf[NKK];
  f32x16 oacc[NDT];
  float mref = kMinit, l = 0.f, lr = 0.f;
  if (score) {
    // Q fragment (B operand of S^T): lane holds Q[myq][16 kk + 8 hf .. +7];
    // rows past Nq read as zero.
    const auto rQ = make_rsrc_at(Qh, w.wq0 * ROWB, nq * ROWB);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[kk] = __builtin_amdgcn_raw_buffer_load_b128(rQ, w.l32 * ROWB + (16 * kk + 8 * w.hf) * 2, 0, 0);
    rs_loop<DT, D, NG, true>(nt, Kh, Vh, kbytes, kr, vr, xb, fb, w, qf, oacc, mref, l, lr, sl2);
    const float lt = pair_sum(l);
    const float ltr = DT == kBF16 ? pair_sum(lr) : lt;
    const bool none = (SPLIT || VARLEN) && !(lt > 0.f);
    fi[w.lane] = none ? 0.f : 1.0f / ltr;
    if (w.hf == 0) {
      const float lse = none ? -INFINITY : (mref + __log2f(lt)) * kLn2;
      const auto rL = SPLIT ? make_rsrc_at(Pl + ((size_t)split * BH + bh) * Nq, w.wq0 * 4, nq * 4)
                            : make_rsrc_at(Lh, w.wq0 * 4, nq * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse), rL, w.l32 * 4, 0, 0);
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
    rs_loop<DT, D, NG, false>(nt, Kh, Vh, kbytes, kr, vr, xb, fb, w, qf, oacc, mref, l, lr, sl2);
    __syncthreads();
    const float inv = fi[w.lane];
    if constexpr (SPLIT) {
      // fp32 partial of this key range, stored 8 bytes at a time from two
      // address registers (see fa_fwd_16).
      const size_t slot = (size_t)split * BH + bh;
      const auto rP = make_rsrc_at(Po + slot * Nq * D, w.wq0 * D * 4, nq * D * 4);
      const int off0 = w.l32 * D * 4 + 4 * w.hf * 4;
      int off1 = off0 + 8;
      asm volatile("" : "+v"(off1));
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x2 v0 = {oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv};
          const f32x2 v1 = {oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv};
          const int col = (32 * dt + 8 * g) * 4;
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v0), rP, off0 + col, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v1), rP, off1 + col, 0, 0);
        }
    } else {
      const auto rO = make_rsrc_at(Oh, w.wq0 * ROWB, nq * ROWB);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 v;
          v[0] = pack2<DT>(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
          v[1] = pack2<DT>(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
          __builtin_amdgcn_raw_buffer_store_b64(v, rO, w.l32 * ROWB + (32 * dt + 8 * g + 4 * w.hf) * 2, 0, 0);
        }
    }
  }
}

template <int DT, int D, int NG, bool CAUSAL, bool SPLIT, bool VARLEN = false>
int launch_rs(const FaLaunch& a, float sl2, int nsplit, int split_len, float* Po, float* Pl) {
  const int nqt = (int)((a.Nq + 32 * NG - 1) / (32 * NG));
  const int64_t heads = VARLEN ? (a.BH + 7) / 8 * 8 : a.BH;
  const dim3 grid((unsigned)(heads * nqt * nsplit)), block(128 * NG);
  return launch_kernel(fa_fwd_rs<DT, D, NG, CAUSAL, SPLIT, VARLEN>, grid, block, (hipStream_t)a.stream, (const u16*)a.q,
                       (const u16*)a.k, (const u16*)a.v, (u16*)a.o, a.lse, (int)a.BH, (int)a.Nq, (int)a.Nk, nqt,
                       sl2, split_len, Po, Pl, a.cu_q, a.cu_k, (int)a.H, (int)a.total_q, (int)a.total_k);
}

// ---------------------------------------------------------------------------
// fp32 kernel, D in {32, 64, 128}, v_mfma_f32_32x32x2_f32.  SPLIT and
// VARLEN as in fa_fwd_16 (the same workgroup mapping, key ranges, partial
// layout and packed layout).
// KS (key split inside the workgroup, for grids too small to give every SIMD
// a wave): the 4 waves share 32 query rows, the workgroup streams 128-key
// tiles and wave w attends to keys [32w, 32w + 32) of each, with its own
// running max, sum and O; at the end the waves' partial results are merged
// through LDS by the same associative update that merges key ranges
// (merge_splits).  No memory beyond the outputs is used.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool SPLIT = false, bool VARLEN = false, bool KS = false>
__global__ __launch_bounds__(kThreads, 1) void fa_fwd_32(const float* __restrict__ Qg,
                                                         const float* __restrict__ Kg,
                                                         const float* __restrict__ Vg,
                                                         float* __restrict__ Og,
                                                         float* __restrict__ Lg, int BH, int Nq,
                                                         int Nk, int nqt, float sl2, int split_len,
                                                         float* __restrict__ Po, float* __restrict__ Pl,
                                                         const int* __restrict__ cuq, const int* __restrict__ cuk,
                                                         int H, int tq, int tk) {
  static_assert(!(KS && (SPLIT || VARLEN)), "the key split runs on the plain forward only");
  constexpr int BC = KS ? 128 : (D <= 64) ? 64 : 32;  // keys per tile
  constexpr int NSUB = KS ? 1 : BC / 32;              // 32-key blocks per wave and tile
  constexpr int BRW = KS ? 32 : kBR;                  // query rows per workgroup
  constexpr int STR = D + 4;      // row stride (floats) of K and V in LDS
  constexpr int ST = BC * STR;    // floats per K (or V) stage
  constexpr int NSTG = (KS && D == 128) ? 1 : 2;  // LDS stages (one 128-key D = 128 stage takes 135 KB)
  constexpr int NDT = D / 32;
  constexpr int HALF = D / 2;     // lane half hf covers head columns [HALF*hf, HALF*hf + HALF)
  constexpr int CPT = BC * D / 4 / kThreads;  // 16-byte chunks per thread per tensor
  static_assert(CPT >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) float smem[NSTG * 2 * ST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  int bh, qt, split;
  if (!fwd_block<SPLIT, VARLEN>(nqt, BH, bh, qt, split)) return;
  const int q0 = qt * BRW;
  // This head's rows: nq queries at Q / Oh / Lh, NK keys at Kg + hr.ko.
  const HeadRows hr = head_rows<VARLEN>(bh, Nq, Nk, D, cuq, cuk, H, tq, tk);
  const int nq = hr.nq, NK = hr.nk;
  if (q0 >= nq) return;  // past this sequence's rows: the whole workgroup
  const float* Q = Qg + hr.qo;
  float* Oh = Og + hr.qo;
  float* Lh = Lg + hr.so;
  const size_t koff = hr.ko;
  // This workgroup's keys: [kb, kb + nk) of the head (all of them unless
  // SPLIT); key indices below are relative to kb.
  const int kb = SPLIT ? split * split_len : 0;
  const int nk = SPLIT ? min(split_len, NK - kb) : NK;
  const float* K = Kg + koff + (size_t)kb * D;
  const float* V = Vg + koff + (size_t)kb * D;

  const int kend = CAUSAL ? min(nk, min(q0 + BRW, nq) - kb) : nk;  // keys [0, kend) are needed
  const int nt = kend > 0 ? (kend + BC - 1) / BC : 0;
  const int wq0 = KS ? q0 : q0 + 32 * wave;
  const int kw = KS ? 32 * wave : 0;  // this wave's first key within a tile
  const int myq = wq0 + l32;
  // A wave whose rows all lie past Nq computes nothing.
  const int wkend = wq0 >= nq ? 0 : CAUSAL ? min(kend, wq0 + 32 - kb) : kend;

  // Q fragment: lane holds Q[myq][HALF*hf + c] for c = 0..HALF-1 (MFMA step c
  // pairs column c of the low half-wave with column HALF + c of the high).
  f32x4 qf[HALF / 4];
#pragma unroll
  for (int c = 0; c < HALF / 4; ++c)
    qf[c] = (myq < nq) ? *(const f32x4*)(Q + (size_t)myq * D + HALF * hf + 4 * c) : f32x4{0, 0, 0, 0};

  f32x4 kr[CPT], vr[CPT];
  auto load_tile = [&](int j) {
    const int k0 = j * BC;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kThreads * i;
      const int key = c / (D / 4), col = (c % (D / 4)) * 4;
      const bool ok = (k0 + key < nk);
      kr[i] = ok ? *(const f32x4*)(K + (size_t)(k0 + key) * D + col) : f32x4{0, 0, 0, 0};
      vr[i] = ok ? *(const f32x4*)(V + (size_t)(k0 + key) * D + col) : f32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int stage) {
    float* ks = smem + stage * 2 * ST;
    float* vs = ks + ST;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kThreads * i;
      const int key = c / (D / 4), col = (c % (D / 4)) * 4;
      *(f32x4*)(ks + key * STR + col) = kr[i];
      *(f32x4*)(vs + key * STR + col) = vr[i];
    }
  };

  float m = kMinit, l = 0.f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};

  if (nt > 0) load_tile(0);
  for (int j = 0; j < nt; ++j) {
    const int stage = NSTG == 2 ? (j & 1) : 0;
    if (NSTG == 1 && j > 0) __syncthreads();  // every wave is done with the one stage
    store_tile(stage);
    __syncthreads();
    if (j + 1 < nt) load_tile(j + 1);
    const int k0 = j * BC + kw;  // this wave's first key of the tile
    if (k0 < wkend) {
      const float* ks = smem + stage * 2 * ST + kw * STR;
      const float* vs = ks + ST;
      constexpr int BCW = 32 * NSUB;  // keys of the tile this wave attends to
      f32x16 s[NSUB];
#pragma unroll
      for (int n = 0; n < NSUB; ++n) {
        s[n] = f32x16{};
#pragma unroll
        for (int c = 0; c < HALF / 4; ++c) {
          const f32x4 a = *(const f32x4*)(ks + (32 * n + l32) * STR + HALF * hf + 4 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[n] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[c][e], s[n], 0, 0, 0);
        }
      }
      const bool need_mask = (k0 + BCW > nk) || (CAUSAL && (k0 + BCW - 1 > wq0 - kb));
      float mx = -INFINITY;
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = s[n][r] * sl2;
          if (need_mask) {
            const int key = k0 + 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= nk || (CAUSAL && key > myq - kb)) t = -INFINITY;
          }
          s[n][r] = t;
          mx = fmaxf(mx, t);
        }
      mx = fmaxf(mx, xor32(mx));
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      float rs = 0.f;
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[n][r] - mnew);
          s[n][r] = p;
          rs += p;
        }
      l = l * alpha + rs;
      m = mnew;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
      // O^T += V^T P^T: MFMA step r pairs key 8*(r/4) + r%4 (low half-wave)
      // with key 8*(r/4) + 4 + r%4 (high half-wave), the keys the lane holds.
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int n = 0; n < NSUB; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3);
            const float a = vs[key * STR + 32 * dt + l32];
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[n][r], oacc[dt], 0, 0, 0);
          }
    }
  }

  float lt = l + xor32(l);
  if constexpr (KS) {
    // Merge the four waves' (m, l, O) of the same rows: M = max m_w,
    // l = sum l_w 2^(m_w - M), O = sum O_w 2^(m_w - M) (each O_w unnormalised).
    // Wave w's O goes to LDS word ((w NDT + dt) 16 + r) 64 + lane; the
    // stage buffer is free once every wave has passed the barrier.
    __syncthreads();
    float* xo = smem;
    float* xm = smem + 4 * NDT * 16 * 64;
    float* xl = xm + 4 * 64;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[((wave * NDT + dt) * 16 + r) * 64 + lane] = oacc[dt][r];
    xm[wave * 64 + lane] = m;
    xl[wave * 64 + lane] = lt;
    __syncthreads();
    if (wave != 0) return;
    float mw[4];
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) mw[w2] = xm[w2 * 64 + lane];
    const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
    lt = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      const float c = __builtin_amdgcn_exp2f(mw[w2] - M);
      lt += c * xl[w2 * 64 + lane];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] += c * xo[((w2 * NDT + dt) * 16 + r) * 64 + lane];
    }
    m = M;
  }
  if (myq < nq) {
    // Rows without a key (an empty key range of SPLIT, a sequence without
    // keys of VARLEN): O = 0, LSE = -inf.
    const bool none = (SPLIT || VARLEN) && !(lt > 0.f);
    const float inv = none ? 0.f : 1.0f / lt;
    float* O;
    float* L;
    if constexpr (SPLIT) {
      const size_t slot = (size_t)split * BH + bh;
      O = Po + (slot * Nq + myq) * D;
      L = Pl + slot * Nq + myq;
    } else {
      O = Oh + (size_t)myq * D;
      L = Lh + myq;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hf;
        *(f32x4*)(O + d) = f32x4{oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv,
                                 oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv};
      }
    if (hf == 0) *L = none ? -INFINITY : (m + __log2f(lt)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool SPLIT, bool VARLEN = false, bool KS = false>
int launch32(const FaLaunch& a, float sl2, int nsplit, int split_len, float* Po, float* Pl) {
  const int nqt = (int)((a.Nq + (KS ? 32 : kBR) - 1) / (KS ? 32 : kBR));
  // VARLEN maps block ids per XCD (8 of them): round B*H up to a multiple of 8
  const int64_t heads = VARLEN ? (a.BH + 7) / 8 * 8 : a.BH;
  const dim3 grid((unsigned)(heads * nqt * nsplit)), block(kThreads);
  return launch_kernel(fa_fwd_32<D, CAUSAL, SPLIT, VARLEN, KS>, grid, block, (hipStream_t)a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, (int)a.BH,
                     (int)a.Nq, (int)a.Nk, nqt, sl2, split_len, Po, Pl, a.cu_q, a.cu_k, (int)a.H, (int)a.total_q,
                     (int)a.total_k);
}

template <int DT, int D, bool CAUSAL, bool SPLIT, bool VARLEN = false, int NW = waves16<D>()>
int launch16(const FaLaunch& a, float sl2, int nsplit, int split_len, float* Po, float* Pl) {
  constexpr int BR = 32 * NW;
  const int nqt = (int)((a.Nq + BR - 1) / BR);
  // VARLEN maps block ids per XCD (8 of them): round B*H up to a multiple of 8
  const int64_t heads = VARLEN ? (a.BH + 7) / 8 * 8 : a.BH;
  const dim3 grid((unsigned)(heads * nqt * nsplit)), block(64 * NW);
  return launch_kernel(fa_fwd_16<DT, D, CAUSAL, SPLIT, VARLEN, NW>, grid, block, (hipStream_t)a.stream,
                     (const u16*)a.q, (const u16*)a.k, (const u16*)a.v, (u16*)a.o, a.lse, (int)a.BH, (int)a.Nq,
                     (int)a.Nk, nqt, sl2, split_len, Po, Pl, a.cu_q, a.cu_k, (int)a.H, (int)a.total_q,
                     (int)a.total_k);
}

template <int DT, int D>
int dispatch16(const FaLaunch& a, float sl2) {
  // Fewer 256-row workgroups than CUs: 128-row workgroups, which double them.
  // D >= 64: the 8-wave role-split kernel (two waves per SIMD; 35-55% faster
  // than the 4-wave form on such grids, while on grids that fill the CUs it
  // lost 15-34% to the 256-row kernels).  D = 32 (a 64-key tile is 4 KB, too
  // little for eight waves' 1 KB loads): the 4-wave form (one wave per SIMD,
  // pipelined steps).  Otherwise 256-row workgroups: at D = 128 the 16-wave
  // role-split kernel (four waves per SIMD; 1-3% faster than fa_fwd_16, the
  // same results), at D <= 64 fa_fwd_16 (two workgroups per CU).
  constexpr int NW8 = waves16<D>();
  if (NW8 == 8 && a.BH * ((a.Nq + 32 * NW8 - 1) / (32 * NW8)) < a.cus) {
    if constexpr (D >= 64)
      return a.causal ? launch_rs<DT, D, 4, true, false>(a, sl2, 1, 0, nullptr, nullptr)
                      : launch_rs<DT, D, 4, false, false>(a, sl2, 1, 0, nullptr, nullptr);
    return a.causal ? launch16<DT, D, true, false, false, 4>(a, sl2, 1, 0, nullptr, nullptr)
                    : launch16<DT, D, false, false, false, 4>(a, sl2, 1, 0, nullptr, nullptr);
  }
  if constexpr (D == 128)
    return a.causal ? launch_rs<DT, D, 8, true, false>(a, sl2, 1, 0, nullptr, nullptr)
                    : launch_rs<DT, D, 8, false, false>(a, sl2, 1, 0, nullptr, nullptr);
  return a.causal ? launch16<DT, D, true, false>(a, sl2, 1, 0, nullptr, nullptr)
                  : launch16<DT, D, false, false>(a, sl2, 1, 0, nullptr, nullptr);
}

// Merge of the key-range partials: the numerically stable associative
// update that folds partial results into one output row ("Building a
// FlashAttention-2 Forward Kernel in Pure NumPy", Architecture Overview),
// exact through the partials' log-sum-exps:
//   LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s.
// D/4 lanes per row, four columns each.
template <int DT, int D>
__global__ __launch_bounds__(256) void merge_splits(const float* __restrict__ Po, const float* __restrict__ Pl,
                                                    void* __restrict__ Og, float* __restrict__ Lg, int64_t rows,
                                                    int nsplit) {
  constexpr int LPR = D / 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / LPR;
  const int c = (int)(t % LPR);
  if (row >= rows) return;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, Pl[s * rows + row]);
  float tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const float ls = Pl[s * rows + row];
    if (ls == -INFINITY) continue;  // no key of this range reaches the row
    const float wgt = __expf(ls - m);
    tot += wgt;
    const f32x4 o = *(const f32x4*)(Po + (s * rows + row) * D + 4 * c);
    acc += wgt * o;
  }
  const float inv = 1.0f / tot;
  if constexpr (DT == kFP16 || DT == kBF16) {
    u32x2 v;
    v[0] = pack2<DT>(acc[0] * inv, acc[1] * inv);
    v[1] = pack2<DT>(acc[2] * inv, acc[3] * inv);
    *(u32x2*)((u16*)Og + row * D + 4 * c) = v;
  } else {
    *(f32x4*)((float*)Og + row * D + 4 * c) = acc * inv;
  }
  if (c == 0) Lg[row] = m + __logf(tot);
}

template <int DT, int D>
int dispatch16_split(const FaLaunch& a, float sl2, int nsplit, int split_len) {
  const int64_t rows = a.BH * a.Nq;
  float* Po = (float*)a.workspace;
  float* Pl = Po + (size_t)nsplit * rows * D;
  const int st = a.causal ? launch16<DT, D, true, true>(a, sl2, nsplit, split_len, Po, Pl)
                          : launch16<DT, D, false, true>(a, sl2, nsplit, split_len, Po, Pl);
  if (st != 0) return st;
  const int64_t threads = rows * (D / 4);
  return launch_kernel(merge_splits<DT, D>, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       (hipStream_t)a.stream, (const float*)Po, (const float*)Pl, a.o, a.lse, rows, nsplit);
}

template <int D>
int dispatch32(const FaLaunch& a, float sl2) {
  // At most one 128-row workgroup per CU (one wave per SIMD): 32-row
  // workgroups that split their keys over the four waves instead, four times
  // the waves.  Measured: +25-33% at 256 workgroups (causal), 2.6x at 64;
  // at 512 workgroups the 128-row tiles win (the split re-reads each K/V
  // tile for every 32 rows).
  const bool ks = a.BH * ((a.Nq + kBR - 1) / kBR) <= a.cus;
  if (a.causal)
    return ks ? launch32<D, true, false, false, true>(a, sl2, 1, 0, nullptr, nullptr)
              : launch32<D, true, false>(a, sl2, 1, 0, nullptr, nullptr);
  return ks ? launch32<D, false, false, false, true>(a, sl2, 1, 0, nullptr, nullptr)
            : launch32<D, false, false>(a, sl2, 1, 0, nullptr, nullptr);
}

template <int D>
int dispatch32_split(const FaLaunch& a, float sl2, int nsplit, int split_len) {
  const int64_t rows = a.BH * a.Nq;
  float* Po = (float*)a.workspace;
  float* Pl = Po + (size_t)nsplit * rows * D;
  const int st = a.causal ? launch32<D, true, true>(a, sl2, nsplit, split_len, Po, Pl)
                          : launch32<D, false, true>(a, sl2, nsplit, split_len, Po, Pl);
  if (st != 0) return st;
  const int64_t threads = rows * (D / 4);
  return launch_kernel(merge_splits<0, D>, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       (hipStream_t)a.stream, (const float*)Po, (const float*)Pl, a.o, a.lse, rows, nsplit);
}

template <int D>
int dispatch32_varlen(const FaLaunch& a, float sl2) {
  return a.causal ? launch32<D, true, false, true>(a, sl2, 1, 0, nullptr, nullptr)
                  : launch32<D, false, false, true>(a, sl2, 1, 0, nullptr, nullptr);
}

template <int DT, int D>
int dispatch16_varlen(const FaLaunch& a, float sl2) {
  return a.causal ? launch16<DT, D, true, false, true>(a, sl2, 1, 0, nullptr, nullptr)
                  : launch16<DT, D, false, false, true>(a, sl2, 1, 0, nullptr, nullptr);
}

}  // namespace

#ifdef FA_FWD_D256

namespace {

template <int DT>
int dispatch_rs(const FaLaunch& a, float sl2) {
  return a.causal ? launch_rs<DT, 256, 4, true, false>(a, sl2, 1, 0, nullptr, nullptr)
                  : launch_rs<DT, 256, 4, false, false>(a, sl2, 1, 0, nullptr, nullptr);
}

template <int DT>
int dispatch_rs_split(const FaLaunch& a, float sl2, int nsplit, int split_len) {
  const int64_t rows = a.BH * a.Nq;
  float* Po = (float*)a.workspace;
  float* Pl = Po + (size_t)nsplit * rows * 256;
  const int st = a.causal ? launch_rs<DT, 256, 4, true, true>(a, sl2, nsplit, split_len, Po, Pl)
                          : launch_rs<DT, 256, 4, false, true>(a, sl2, nsplit, split_len, Po, Pl);
  if (st != 0) return st;
  const int64_t threads = rows * (256 / 4);
  return launch_kernel(merge_splits<DT, 256>, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       (hipStream_t)a.stream, (const float*)Po, (const float*)Pl, a.o, a.lse, rows, nsplit);
}

template <int DT>
int dispatch_rs_varlen(const FaLaunch& a, float sl2) {
  return a.causal ? launch_rs<DT, 256, 4, true, false, true>(a, sl2, 1, 0, nullptr, nullptr)
                  : launch_rs<DT, 256, 4, false, false, true>(a, sl2, 1, 0, nullptr, nullptr);
}

}  // namespace

int fa_launch_fwd_d256(const FaLaunch& a, float sl2) {
  return a.dtype == kBF16 ? dispatch_rs<kBF16>(a, sl2) : dispatch_rs<kFP16>(a, sl2);
}

int fa_launch_fwd_splitkv_d256(const FaLaunch& a, float sl2, int nsplit, int split_len) {
  return a.dtype == kBF16 ? dispatch_rs_split<kBF16>(a, sl2, nsplit, split_len)
                          : dispatch_rs_split<kFP16>(a, sl2, nsplit, split_len);
}

int fa_launch_fwd_varlen_d256(const FaLaunch& a, float sl2) {
  return a.dtype == kBF16 ? dispatch_rs_varlen<kBF16>(a, sl2) : dispatch_rs_varlen<kFP16>(a, sl2);
}

#else

int fa_launch_fwd_varlen(const FaLaunch& a) {
  const float sl2 = (float)(a.scale * 1.4426950408889634074);
  if (a.D == 256) return fa_launch_fwd_varlen_d256(a, sl2);
  switch (a.dtype) {
    case kBF16:
      return a.D == 32 ? dispatch16_varlen<kBF16, 32>(a, sl2)
           : a.D == 64 ? dispatch16_varlen<kBF16, 64>(a, sl2) : dispatch16_varlen<kBF16, 128>(a, sl2);
    case kFP16:
      return a.D == 32 ? dispatch16_varlen<kFP16, 32>(a, sl2)
           : a.D == 64 ? dispatch16_varlen<kFP16, 64>(a, sl2) : dispatch16_varlen<kFP16, 128>(a, sl2);
    default:
      return a.D == 32 ? dispatch32_varlen<32>(a, sl2)
           : a.D == 64 ? dispatch32_varlen<64>(a, sl2) : dispatch32_varlen<128>(a, sl2);
  }
}

int fa_launch_fwd_splitkv(const FaLaunch& a, int nsplit, int split_len) {
  const float sl2 = (float)(a.scale * 1.4426950408889634074);
  if (a.D == 256) return fa_launch_fwd_splitkv_d256(a, sl2, nsplit, split_len);
  switch (a.dtype) {
    case kBF16:
      return a.D == 32 ? dispatch16_split<kBF16, 32>(a, sl2, nsplit, split_len)
           : a.D == 64 ? dispatch16_split<kBF16, 64>(a, sl2, nsplit, split_len)
                       : dispatch16_split<kBF16, 128>(a, sl2, nsplit, split_len);
    case kFP16:
      return a.D == 32 ? dispatch16_split<kFP16, 32>(a, sl2, nsplit, split_len)
           : a.D == 64 ? dispatch16_split<kFP16, 64>(a, sl2, nsplit, split_len)
                       : dispatch16_split<kFP16, 128>(a, sl2, nsplit, split_len);
    default:
      return a.D == 32 ? dispatch32_split<32>(a, sl2, nsplit, split_len)
           : a.D == 64 ? dispatch32_split<64>(a, sl2, nsplit, split_len)
                       : dispatch32_split<128>(a, sl2, nsplit, split_len);
  }
}

int fa_launch_fwd(const FaLaunch& a) {
  // scale * log2(e), computed in double and rounded once.
  const float sl2 = (float)(a.scale * 1.4426950408889634074);
  if (a.D == 256) return fa_launch_fwd_d256(a, sl2);
  switch (a.dtype) {
    case kBF16:
      return a.D == 32 ? dispatch16<kBF16, 32>(a, sl2)
           : a.D == 64 ? dispatch16<kBF16, 64>(a, sl2) : dispatch16<kBF16, 128>(a, sl2);
    case kFP16:
      return a.D == 32 ? dispatch16<kFP16, 32>(a, sl2)
           : a.D == 64 ? dispatch16<kFP16, 64>(a, sl2) : dispatch16<kFP16, 128>(a, sl2);
    default:
      return a.D == 32 ? dispatch32<32>(a, sl2) : a.D == 64 ? dispatch32<64>(a, sl2) : dispatch32<128>(a, sl2);
  }
}

// Scratch of fa_fwd_splitkv_static, for callers that cannot allocate: the
// key-range partials go to this file-scope device array instead of a caller
// workspace.  Every device the library runs on holds its own copy, at its
// own address, until the process ends; all calls on one device share it.
// In host code `scratch` is only a stand-in for the device symbol: its
// device address is looked up once per device (fa_static_scratch) and only
// that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[FA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices];  // device address of `scratch`, per device
}  // namespace

int fa_static_scratch(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    scratch_addr[dev] = p;
  }
  *addr = scratch_addr[dev];
  return 0;
}

#endif  // FA_FWD_D256
