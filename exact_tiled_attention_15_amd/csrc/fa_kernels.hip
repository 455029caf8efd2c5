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
// Work decomposition: one workgroup of 4 waves per (batch*head, Q tile of
// 128 rows); each wave owns 32 query rows.  K/V tiles of 64 keys are
// streamed from HBM through registers into a double-buffered LDS stage (one
// barrier per tile).
//
// Data layout inside a wave (16-bit types): the score tile is computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}: K (from LDS)
// is the A operand, the wave's Q fragment (registers, loaded once) is the B
// operand.  The 32x32 accumulator then holds, in lane l, query row l%32 and
// 16 keys 8*(r/4) + 4*(l/32) + r%4 (r = register 0..15): one query row lives
// in a lane pair (l, l^32), so the row max needs a single exchange across
// the half-waves and the row sum needs none until the end.  P^T is fed
// straight from those registers (rounded to bf16/fp16) as the B operand of
// O^T = V^T P^T, whose A operand is read from a transposed, key-permuted
// copy of the V tile in LDS.  O^T (fp32) stays in registers.  The fp32 path
// uses v_mfma_f32_32x32x2_f32 with the same accumulator layout, P stays
// fp32, and V stays row-major in LDS.
//
// Softmax runs in the log2 domain: t = s * (log2(e)/sqrt(D)), p = exp2(t - m)
// on v_exp_f32; LSE = (m + log2 l) * ln 2 at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

namespace {

typedef unsigned short u16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kFP16 = 1, kBF16 = 2;  // fa_dtype codes (0 is fp32)
constexpr int kThreads = 256;                     // 4 waves of 64
constexpr int kBR = 128;                          // query rows per workgroup
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kMinit = -1.0e30f;  // finite start for the running max (no inf-inf)

template <int DT>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == kBF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Round two fp32 values to the 16-bit type (nearest even) and pack them,
// the first in the low half (one v_cvt_pk_{bf16,f16}_f32).
template <int DT>
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  const f32x2 x = {lo, hi};
  if constexpr (DT == kBF16) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2));
  } else {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(x, f16x2));
  }
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Lanes l and l^32 hold the two halves of one query row; these combine a
// per-lane value with its partner's (one ds_bpermute).  The gfx950
// permlane32 swap builtin is not used: this compiler returns the same
// register for both of its results.
__device__ __forceinline__ float pair_max(float x) { return fmaxf(x, xor32(x)); }
__device__ __forceinline__ float pair_sum(float x) { return x + xor32(x); }

// Smallest last-visible key over a wave's 32 rows: a 64-key tile starting at
// k0 needs masking when k0 + 63 exceeds it (causal diagonal, or past Nk).
__device__ __forceinline__ int klim_wave_max(int wq0, int Nk, bool causal) {
  return causal ? min(wq0, Nk - 1) : Nk - 1;
}

// Workgroup -> (batch*head, Q tile).  Q tiles are issued heaviest first
// (for causal attention the last Q tile sees the most keys), and all Q tiles
// of one head get the same block index modulo the head count, so that when
// that count is a multiple of 8 they land on the same XCD and share its L2
// for K/V.
__device__ __forceinline__ void tile_of_block(int nqt, int BH, int& bh, int& qt) {
  const int bid = blockIdx.x;
  bh = bid % BH;
  qt = nqt - 1 - bid / BH;
}

// ---------------------------------------------------------------------------
// 16-bit kernel (bf16 / fp16), D in {64, 128}, 64-key tiles.
// ---------------------------------------------------------------------------
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_16(const u16* __restrict__ Qg,
                                                         const u16* __restrict__ Kg,
                                                         const u16* __restrict__ Vg,
                                                         u16* __restrict__ Og,
                                                         float* __restrict__ Lg, int BH, int Nq,
                                                         int Nk, int nqt, float sl2) {
  constexpr int BC = 64;
  constexpr int KSTR = D + 8;     // K row stride (elements): +16 B breaks bank aliasing
  constexpr int VSTR = BC + 8;    // V^T row stride (elements)
  constexpr int KST = BC * KSTR;  // elements per K stage
  constexpr int VST = D * VSTR;   // elements per V^T stage
  constexpr int NKK = D / 16;     // MFMA steps over the head dimension
  constexpr int NDT = D / 32;     // 32-wide output column tiles
  constexpr int KPT = BC * D / 8 / kThreads;  // 16-byte K chunks per thread
  constexpr int VJOBS = (BC / 4) * (D / 8);   // 4-key x 8-column V blocks per tile
  static_assert(KPT >= 1 && VJOBS <= kThreads, "tile shape");

  __shared__ __attribute__((aligned(16))) u16 smem[2 * (KST + VST)];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hf = lane >> 5, l32 = lane & 31;
  int bh, qt;
  tile_of_block(nqt, BH, bh, qt);
  const int q0 = qt * kBR;
  const size_t qoff = (size_t)bh * Nq * D, koff = (size_t)bh * Nk * D;
  const u16* Q = Qg + qoff;
  const u16* K = Kg + koff;
  const u16* V = Vg + koff;

  const int kend = CAUSAL ? min(Nk, min(q0 + kBR, Nq)) : Nk;  // keys [0, kend) are needed
  const int nt = (kend + BC - 1) / BC;
  const bool ktail = (nt * BC > Nk);              // the last tile runs past Nk
  const int wq0 = q0 + 32 * wave;                  // this wave's first query row
  const int myq = wq0 + l32;                       // this lane's query row
  const int wkend = CAUSAL ? min(kend, wq0 + 32) : kend;  // keys this wave needs
  // last key this lane may see
  const int klim = CAUSAL ? min(myq, Nk - 1) : Nk - 1;

  // Q fragment: lane holds Q[myq][16*kk + 8*hf .. +7] for kk = 0..NKK-1.
  u32x4 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = (myq < Nq) ? *(const u32x4*)(Q + (size_t)myq * D + 16 * kk + 8 * hf) : u32x4{0, 0, 0, 0};
  }

  // Per-thread staging of the next K/V tile.
  u32x4 kr[KPT];
  u32x4 vr[4];
  const int g4 = tid & 15, db = tid >> 4;  // V job: keys 4*g4..+3, columns 8*db..+7
  const bool vjob = (VJOBS == kThreads) || (tid < VJOBS);
  const int krow0 = tid / (D / 8), kcol = (tid % (D / 8)) * 8;  // K chunk i: row krow0 + i*(256/(D/8))
  constexpr int KROWS_PER_PASS = kThreads / (D / 8);

  // Full tiles load unguarded; the tile that runs past Nk clamps the row and
  // zero-fills (zero V rows keep 0 * V finite for masked keys).
  auto load_tile = [&](int j, bool guard) {
    const int k0 = j * BC;
    if (!guard) {
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        kr[i] = *(const u32x4*)(K + (size_t)(k0 + krow0 + i * KROWS_PER_PASS) * D + kcol);
      if (vjob) {
#pragma unroll
        for (int r = 0; r < 4; ++r) vr[r] = *(const u32x4*)(V + (size_t)(k0 + 4 * g4 + r) * D + 8 * db);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int key = k0 + krow0 + i * KROWS_PER_PASS;
        const u32x4 x = *(const u32x4*)(K + (size_t)min(key, Nk - 1) * D + kcol);
        kr[i] = (key < Nk) ? x : u32x4{0, 0, 0, 0};
      }
      if (vjob) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 4 * g4 + r;
          const u32x4 x = *(const u32x4*)(V + (size_t)min(key, Nk - 1) * D + 8 * db);
          vr[r] = (key < Nk) ? x : u32x4{0, 0, 0, 0};
        }
      }
    }
  };

  // V^T positions inside a 16-key group: keys 0-3 -> 0-3, 8-11 -> 4-7,
  // 4-7 -> 8-11, 12-15 -> 12-15, so that the 8 keys one lane feeds to a PV
  // MFMA are contiguous.
  const int vpos = (g4 >> 2) * 16 + ((((g4 & 3) & 1) << 1) | ((g4 & 3) >> 1)) * 4;
  auto store_tile = [&](int stage) {
    u16* ks = smem + stage * (KST + VST);
    u16* vs = ks + KST;
#pragma unroll
    for (int i = 0; i < KPT; ++i) *(u32x4*)(ks + (krow0 + i * KROWS_PER_PASS) * KSTR + kcol) = kr[i];
    if (vjob) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned e01 = __builtin_amdgcn_perm(vr[1][j], vr[0][j], 0x05040100u);
        const unsigned e23 = __builtin_amdgcn_perm(vr[3][j], vr[2][j], 0x05040100u);
        const unsigned o01 = __builtin_amdgcn_perm(vr[1][j], vr[0][j], 0x07060302u);
        const unsigned o23 = __builtin_amdgcn_perm(vr[3][j], vr[2][j], 0x07060302u);
        *(u32x2*)(vs + (8 * db + 2 * j) * VSTR + vpos) = u32x2{e01, e23};
        *(u32x2*)(vs + (8 * db + 2 * j + 1) * VSTR + vpos) = u32x2{o01, o23};
      }
    }
  };

  // Running state.  mref is a reference maximum in the scaled log2 domain;
  // it is raised only when a tile's row max exceeds it by more than kTau, so
  // P = exp2(t - mref) stays below 2^kTau.  O and l always share mref, so the
  // final O / l and mref + log2(l) are exact whatever mref is.
  constexpr float kTau = 8.0f;
  float mref = kMinit, l = 0.f;
  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};

  load_tile(0, ktail && nt == 1);
  for (int j = 0; j < nt; ++j) {
    const int stage = j & 1;
    store_tile(stage);
    __syncthreads();
    if (j + 1 < nt) load_tile(j + 1, ktail && (j + 2 == nt));
    const int k0 = j * BC;
    if (k0 < wkend) {
      const u16* ks = smem + stage * (KST + VST);
      const u16* vs = ks + KST;
      f32x16 s[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        s[n] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const u32x4 a = *(const u32x4*)(ks + (32 * n + l32) * KSTR + 16 * kk + 8 * hf);
          s[n] = mfma_32x32x16<DT>(a, qf[kk], s[n]);
        }
      }
      // Mask (diagonal and tail tiles only): key = k0 + 4*hf + off(n, r).
      if ((k0 + BC - 1 > klim_wave_max(wq0, Nk, CAUSAL)) ) {
        const int lim = klim - (k0 + 4 * hf);
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[n][r] = (32 * n + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[n][r];
      }
      // Row max of the raw scores (scale > 0 commutes with max).
      float mx = s[0][0];
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = (n == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[n][r]);
      mx = pair_max(mx) * sl2;
      if (__builtin_amdgcn_ballot_w64(mx > mref + kTau)) {
        const float mnew = fmaxf(mref, mx);
        const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
        mref = mnew;
      }
      const float nm = -mref;
      u32x4 pf[2][2];
      // l sums the fp32 P (its rounding to 16 bits would leave a relative
      // error of up to 2^-9 in the LSE of rows that see few keys).
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][8 * hh + 2 * i], sl2, nm));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[n][8 * hh + 2 * i + 1], sl2, nm));
            pf[n][hh][i] = pack2<DT>(p0, p1);
            ls0 += p0;
            ls1 += p1;
          }
      l += ls0 + ls1;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const u32x4 a = *(const u32x4*)(vs + (32 * dt + l32) * VSTR + 32 * n + 16 * hh + 8 * hf);
            oacc[dt] = mfma_32x32x16<DT>(a, pf[n][hh], oacc[dt]);
          }
    }
  }

  // Epilogue: combine the two half-row sums, normalise, round, store.
  const float lt = pair_sum(l);
  if (myq < Nq) {
    const float inv = 1.0f / lt;
    u16* O = Og + qoff + (size_t)myq * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hf;
        u32x2 w;
        w[0] = pack2<DT>(oacc[dt][4 * g + 0] * inv, oacc[dt][4 * g + 1] * inv);
        w[1] = pack2<DT>(oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
        *(u32x2*)(O + d) = w;
      }
    if (hf == 0) Lg[(size_t)bh * Nq + myq] = (mref + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel, D in {64, 128}, v_mfma_f32_32x32x2_f32.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fa_fwd_32(const float* __restrict__ Qg,
                                                         const float* __restrict__ Kg,
                                                         const float* __restrict__ Vg,
                                                         float* __restrict__ Og,
                                                         float* __restrict__ Lg, int BH, int Nq,
                                                         int Nk, int nqt, float sl2) {
  constexpr int BC = (D == 64) ? 64 : 32;
  constexpr int NSUB = BC / 32;
  constexpr int STR = D + 4;      // row stride (floats) of K and V in LDS
  constexpr int ST = BC * STR;    // floats per K (or V) stage
  constexpr int NDT = D / 32;
  constexpr int HALF = D / 2;     // lane half hf covers head columns [HALF*hf, HALF*hf + HALF)
  constexpr int CPT = BC * D / 4 / kThreads;  // 16-byte chunks per thread per tensor
  static_assert(CPT >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) float smem[2 * 2 * ST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  int bh, qt;
  tile_of_block(nqt, BH, bh, qt);
  const int q0 = qt * kBR;
  const size_t qoff = (size_t)bh * Nq * D, koff = (size_t)bh * Nk * D;
  const float* Q = Qg + qoff;
  const float* K = Kg + koff;
  const float* V = Vg + koff;

  const int kend = CAUSAL ? min(Nk, min(q0 + kBR, Nq)) : Nk;
  const int nt = (kend + BC - 1) / BC;
  const int wq0 = q0 + 32 * wave;
  const int myq = wq0 + l32;
  const int wkend = CAUSAL ? min(kend, wq0 + 32) : kend;

  // Q fragment: lane holds Q[myq][HALF*hf + c] for c = 0..HALF-1 (MFMA step c
  // pairs column c of the low half-wave with column HALF + c of the high).
  f32x4 qf[HALF / 4];
#pragma unroll
  for (int c = 0; c < HALF / 4; ++c)
    qf[c] = (myq < Nq) ? *(const f32x4*)(Q + (size_t)myq * D + HALF * hf + 4 * c) : f32x4{0, 0, 0, 0};

  f32x4 kr[CPT], vr[CPT];
  auto load_tile = [&](int j) {
    const int k0 = j * BC;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + kThreads * i;
      const int key = c / (D / 4), col = (c % (D / 4)) * 4;
      const bool ok = (k0 + key < Nk);
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

  load_tile(0);
  for (int j = 0; j < nt; ++j) {
    const int stage = j & 1;
    store_tile(stage);
    __syncthreads();
    if (j + 1 < nt) load_tile(j + 1);
    const int k0 = j * BC;
    if (k0 < wkend) {
      const float* ks = smem + stage * 2 * ST;
      const float* vs = ks + ST;
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
      const bool need_mask = (k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > wq0));
      float mx = -INFINITY;
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = s[n][r] * sl2;
          if (need_mask) {
            const int key = k0 + 32 * n + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= Nk || (CAUSAL && key > myq)) t = -INFINITY;
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

  const float lt = l + xor32(l);
  if (myq < Nq) {
    const float inv = 1.0f / lt;
    float* O = Og + qoff + (size_t)myq * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * hf;
        *(f32x4*)(O + d) = f32x4{oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv,
                                 oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv};
      }
    if (hf == 0) Lg[(size_t)bh * Nq + myq] = (m + __log2f(lt)) * kLn2;
  }
}

template <typename KernelT, typename T>
int launch(KernelT kern, const FaLaunch& a, int nqt, float sl2) {
  const dim3 grid((unsigned)(a.BH * nqt)), block(kThreads);
  hipLaunchKernelGGL(kern, grid, block, 0, (hipStream_t)a.stream, (const T*)a.q, (const T*)a.k,
                     (const T*)a.v, (T*)a.o, a.lse, (int)a.BH, (int)a.Nq, (int)a.Nk, nqt, sl2);
  return (int)hipGetLastError();
}

template <int DT, int D>
int dispatch16(const FaLaunch& a, int nqt, float sl2) {
  if (a.causal) return launch<decltype(&fa_fwd_16<DT, D, true>), u16>(&fa_fwd_16<DT, D, true>, a, nqt, sl2);
  return launch<decltype(&fa_fwd_16<DT, D, false>), u16>(&fa_fwd_16<DT, D, false>, a, nqt, sl2);
}

template <int D>
int dispatch32(const FaLaunch& a, int nqt, float sl2) {
  if (a.causal) return launch<decltype(&fa_fwd_32<D, true>), float>(&fa_fwd_32<D, true>, a, nqt, sl2);
  return launch<decltype(&fa_fwd_32<D, false>), float>(&fa_fwd_32<D, false>, a, nqt, sl2);
}

}  // namespace

int fa_launch_fwd(const FaLaunch& a) {
  const int nqt = (int)((a.Nq + kBR - 1) / kBR);
  // log2(e)/sqrt(D), computed in double and rounded once.
  const float sl2 = (float)(1.4426950408889634074 / __builtin_sqrt((double)a.D));
  (void)hipGetLastError();  // clear a stale error so that the check below is ours
  switch (a.dtype) {
    case kBF16:
      return a.D == 64 ? dispatch16<kBF16, 64>(a, nqt, sl2) : dispatch16<kBF16, 128>(a, nqt, sl2);
    case kFP16:
      return a.D == 64 ? dispatch16<kFP16, 64>(a, nqt, sl2) : dispatch16<kFP16, 128>(a, nqt, sl2);
    default:
      return a.D == 64 ? dispatch32<64>(a, nqt, sl2) : dispatch32<128>(a, nqt, sl2);
  }
}
