// Device helpers shared by the gfx950 attention kernels (forward and
// backward): MFMA wrappers, 16-bit packing, buffer resources, the swizzled
// LDS tile layout with its direct-to-LDS loads and operand reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

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

// Add both 16-bit values of a packed pair (as packed by pack2) to `acc`:
// one v_dot2c_f32_{bf16,f16} against (1, 1).  The products are exact; the
// sum is an fp32 sum.
template <int DT>
__device__ __forceinline__ float add_pair16(unsigned pair, float acc) {
  if constexpr (DT == kBF16) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
  } else {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
  }
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Lanes l and l^32 hold the two halves of one query row; these combine a
// per-lane value with its partner's (one ds_bpermute).  The gfx950
// permlane32 swap builtin is not used: this compiler returns the same
// register for both of its results.
__device__ __forceinline__ float pair_max(float x) { return fmaxf(x, xor32(x)); }
__device__ __forceinline__ float pair_sum(float x) { return x + xor32(x); }

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

// The rows of one (batch, head) that a workgroup works on: nq queries and nk
// keys, and the offsets of the first query row (elements of q, o, dout, dq),
// key row (elements of k, v, dk, dv) and query statistic (lse, workspace).
// Dense tensors: [B*H, Nq, D] and [B*H, Nk, D].  Packed (VARLEN): sequence b
// owns query rows [cuq[b], cuq[b+1]) and key rows [cuk[b], cuk[b+1]) of
// [H, tq, D] / [H, tk, D] (offsets clamped into [0, tq] / [0, tk]).
struct HeadRows {
  int nq, nk;
  size_t qo, ko, so;
};

template <bool VARLEN>
__device__ __forceinline__ HeadRows head_rows(int bh, int Nq, int Nk, int D, const int* cuq, const int* cuk, int H,
                                              int tq, int tk) {
  HeadRows r;
  if constexpr (VARLEN) {
    const int b = bh / H, h = bh - b * H;
    const int qs = min(max(cuq[b], 0), tq), qe = min(max(cuq[b + 1], qs), tq);
    const int ks = min(max(cuk[b], 0), tk), ke = min(max(cuk[b + 1], ks), tk);
    r.nq = qe - qs;
    r.nk = ke - ks;
    r.qo = ((size_t)h * tq + qs) * D;
    r.ko = ((size_t)h * tk + ks) * D;
    r.so = (size_t)h * tq + qs;
  } else {
    r.nq = Nq;
    r.nk = Nk;
    r.qo = (size_t)bh * Nq * D;
    r.ko = (size_t)bh * Nk * D;
    r.so = (size_t)bh * Nq;
  }
  return r;
}

// ---------------------------------------------------------------------------
// 16-bit kernel (bf16 / fp16), D in {32, 64, 128}, 64-key tiles.
// ---------------------------------------------------------------------------
// Buffer resources for the ragged Nq / Nk tails.  Every buffer access here
// is a raw (stride 0) access whose scalar offset is 0: the resource's base
// is the start of the tile or row block being accessed, num_records the
// bytes of the tensor from there on, and the per-lane VGPR offset plus the
// instruction's immediate offset is range-checked against num_records:
// loads past it return 0 (into LDS too, for the direct-to-LDS form) and
// stores past it are dropped.
constexpr int kBufFlags = 0x00020000;  // gfx9 buffer descriptor word 3 (32-bit data format)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes > 0 ? bytes : 0, kBufFlags);
}
// The resource of the bytes [off, total) of a tensor at `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_at(const void* base, int off, int total) {
  return make_rsrc((const unsigned char*)base + off, total - off);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS tile layout for a BC x D tile of 16-bit values (K or V), in bytes.
// The gfx950 LDS serves 256 bytes per clock (64 banks of 4 bytes), so rows
// are taken in groups of 16 and 16-byte chunk c of the 16 rows shares one
// 256-byte line, at row slot (R % 16) XOR 4 (c % 4):
//   off(R, c) = (R / 16) * 32 D + 256 c + 16 ((R % 16) ^ (4 (c % 4))).
// A K-operand read (16 lanes = 16 rows x one chunk) and a transposing
// V-operand read (32 lanes = 4 rows x 4 chunks) then each cover one whole
// 256-byte line, and every read address is one of two per-lane bases plus
// a compile-time offset.

// Global byte offset (within a tile) of the 16 bytes that lane `lane` of
// the G-th 1 KB direct-to-LDS load must fetch so that LDS byte 1024 G +
// 16 lane ends up holding the chunk that the layout above puts there.
template <int D>
__device__ __forceinline__ int dma_src_off(int G, int lane) {
  const int o = G * 1024 + 16 * lane;
  const int rem = o % (32 * D);
  const int c = rem / 256;
  const int R = (o / (32 * D)) * 16 + (((rem % 256) / 16) ^ ((c & 3) << 2));
  return R * (2 * D) + c * 16;
}

// Per-wave constants of the 16-bit kernels.  The row/column fields are
// those of the forward kernel (rows = queries, streamed columns = keys).
struct Wave16 {
  int lane, hf, l32, wave;
  int wq0;    // first query row of the wave
  int wkend;  // keys [0, wkend) are needed by the wave
  int wklim;  // smallest last-visible key over the wave's rows
  int klim;   // last key this lane's row may see
  // LDS byte offsets of this lane's K-operand reads (even / odd kk) and of
  // its transposing V-operand reads (q = 0 / 1), each plain (lo) and plus
  // 64 KB (hi); see ks_operand.
  int kb_lo[2], kb_hi[2];
  int vb_lo[2], vb_hi[2];
};

constexpr int kStages = 4;  // LDS ring depth: three tiles in flight while one is consumed

// Wait until at most `later` of this wave's direct-to-LDS loads and LGKM
// of its LDS operations are still in flight (each counter completes in
// issue order), then meet the other waves.  s_waitcnt takes an immediate,
// hence the switch (`later` is wave-uniform, even and at most 12).
template <int LGKM = 0>
__device__ __forceinline__ void wait_tile_and_barrier(int later) {
  static_assert(LGKM >= 0 && LGKM < 16, "lgkmcnt field");
  constexpr int kBase = 0x070 | (LGKM << 8);  // expcnt: no wait; lgkmcnt(LGKM); vmcnt in the low bits
  asm volatile("" ::: "memory");
  switch (later) {
    case 12: __builtin_amdgcn_s_waitcnt(kBase | 12); break;
    case 10: __builtin_amdgcn_s_waitcnt(kBase | 10); break;
    case 8: __builtin_amdgcn_s_waitcnt(kBase | 8); break;
    case 6: __builtin_amdgcn_s_waitcnt(kBase | 6); break;
    case 4: __builtin_amdgcn_s_waitcnt(kBase | 4); break;
    case 2: __builtin_amdgcn_s_waitcnt(kBase | 2); break;
    default: __builtin_amdgcn_s_waitcnt(kBase); break;
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Number of 1 KB direct-to-LDS loads (both tensors together) that wave
// `wave` of NW issues per BC-row tile: the 1 KB pieces G = wave, wave + NW,
// ... of each tensor's tile.
template <int D, int NW, int BC = 64>
__device__ __forceinline__ int loads_per_tile(int wave) {
  constexpr int NG = BC * D * 2 / 1024;
  return 2 * ((NG - wave + NW - 1) / NW);
}

// Direct-to-LDS loads of BC-row tile t of two [N, D] tensors (K and V in
// the forward pass) into `dst` (first tensor) and `dst + BC D 2` (second):
// this wave's 1 KB pieces G = wave, wave + NW, ... of each.
template <int D, int NW, int BC = 64>
__device__ __forceinline__ void issue_tile16(const u16* Kh, const u16* Vh, int kbytes, int t,
                                             unsigned char* dst, const Wave16& w) {
  static_assert(BC % 16 == 0 && BC * D * 2 % 1024 == 0, "whole 16-row groups and 1 KB pieces");
  constexpr int TILEB = BC * D * 2;
  constexpr int NG = TILEB / 1024;
  const auto rk = make_rsrc_at(Kh, t * TILEB, kbytes);
  const auto rv = make_rsrc_at(Vh, t * TILEB, kbytes);
#pragma unroll
  for (int I = 0; I < (NG + NW - 1) / NW; ++I) {
    const int G = w.wave + NW * I;
    if (G < NG) {
      const int go = dma_src_off<D>(G, w.lane);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(dst + G * 1024), 16, go, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dst + TILEB + G * 1024), 16, go, 0, 0, 0);
    }
  }
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// LDS operand reads.  A ring stage may lie above 64 KB, past the reach of
// the ds_read immediate offset, so each lane's offsets exist twice, plain
// (lo) and plus 64 KB (hi), both kept opaque to the compiler; a read takes
// the copy that matches its stage's 64 KB window (`lds_bias`, a link-time
// constant), so that it is one base register plus an immediate below 64 KB,
// and its pointer still derives from the stage array, so the compiler still
// knows which array it reads (and that the loads in flight write others).
__device__ __forceinline__ unsigned lds_bias(const unsigned char* p) {
  return (unsigned)(uintptr_t)(const lds_u8*)p & 0xFFFF0000u;
}

// K operand of score MFMA i (block n = i / (D/16), step kk = i % (D/16)):
// row 32n + l32, chunk 2kk + hf of the tile.
template <int D>
__device__ __forceinline__ u32x4 ks_operand(const unsigned char* ks, const Wave16& w, int i) {
  const int n = i / (D / 16), kk = i % (D / 16);
  const unsigned bias = lds_bias(ks);
  const int base = bias ? w.kb_hi[kk & 1] : w.kb_lo[kk & 1];
  return *(const lds_u32x4*)((const lds_u8*)ks + (base + (n * 64 * D + (kk >> 1) * 1024 - (int)bias)));
}

// V^T operand of PV MFMA i of a BC-row tile (output block dt = i / (BC/16),
// keys 16 (i % (BC/16)), i.e. 32n + 16hh), from two transposing 64-bit reads.
template <int D, int BC = 64>
__device__ __forceinline__ u32x4 vt_operand(const unsigned char* vs, const Wave16& w, int i) {
  static_assert(BC == 32 || BC == 64, "one or two 32-key blocks");
  constexpr int KSH = BC == 64 ? 2 : 1;  // log2 of the 16-key steps per tile
  const int dt = i >> KSH, n = (i >> 1) & (BC / 32 - 1), hh = i & 1;
  const unsigned bias = lds_bias(vs);
  const int off = (2 * n + hh) * (32 * D) + dt * 1024 - (int)bias;
  const int b0 = bias ? w.vb_hi[0] : w.vb_lo[0], b1 = bias ? w.vb_hi[1] : w.vb_lo[1];
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((const lds_u8*)vs + (b0 + off)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((const lds_u8*)vs + (b1 + off)));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
}

// Lane offsets of the operand reads (set once per wave; w.lane, w.hf, w.l32
// must be set).  Row operand (ks_operand): row 32n + l32, chunk
// c = 2kk + hf, so the slot XOR (4 (c % 4)) depends on the parity of kk.
// Transposed operand (vt_operand): 16-lane group g reads rows
// 32n + 16hh + 8q + 4hf + i/4 at columns 32dt + 16g + 4(i%4), i = lane % 16,
// i.e. chunk 4dt + 2g + (i%4)/2 and half (i%2) of it.
template <int D>
__device__ __forceinline__ void init_operand_offsets(Wave16& w) {
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int c = 2 * par + w.hf;
    w.kb_lo[par] = (w.l32 >> 4) * (32 * D) + c * 256 + (((w.l32 & 15) ^ (c << 2)) << 4);
    w.kb_hi[par] = w.kb_lo[par] + 65536;
    asm volatile("" : "+v"(w.kb_lo[par]));
    asm volatile("" : "+v"(w.kb_hi[par]));
  }
  {
    const int vi = w.l32 & 15, vg = w.l32 >> 4;
    const int c = 2 * vg + ((vi & 3) >> 1);  // chunk within the 4-chunk (64-column) block
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      w.vb_lo[q] = c * 256 + (((8 * q + 4 * w.hf + (vi >> 2)) ^ (c << 2)) << 4) + 8 * (vi & 1);
      w.vb_hi[q] = w.vb_lo[q] + 65536;
      asm volatile("" : "+v"(w.vb_lo[q]));
      asm volatile("" : "+v"(w.vb_hi[q]));
    }
  }
}

// Host side: enqueue kernel<<<grid, block, 0, st>>>(args...) through
// hipLaunchKernel and return that launch's own status.  The runtime's
// last-error state (which may hold an error of the caller's earlier work) is
// not read or cleared, so a failure reported here is this launch's.
template <typename... P, typename... A>
int launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t st, A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
  std::tuple<P...> t{static_cast<P>(args)...};
  return std::apply(
      [&](auto&... p) {
        void* ptrs[] = {(void*)&p...};
        return (int)hipLaunchKernel((const void*)kernel, grid, block, ptrs, 0, st);
      },
      t);
}

}  // namespace
