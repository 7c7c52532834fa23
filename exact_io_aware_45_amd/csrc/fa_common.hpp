// fa_common.hpp -- device-side building blocks shared by the attention kernels
// (gfx950 / CDNA4 only).
//
// Register layouts of the two bf16 matrix instructions used here (measured on
// the device, lane l of a 64-wide wave, h = l / 32):
//   v_mfma_f32_32x32x16_bf16:  A[i][k]: i = l % 32, k = 8h + t   (t = 0..7)
//                              B[k][j]: j = l % 32, k = 8h + t
//                              C[i][j]: j = l % 32, i = 8(r/4) + 4h + r%4
//                              (r = 0..15 accumulator registers)
//   v_mfma_f32_16x16x32_bf16:  A[i][k]: i = l % 16, k = 8(l/16) + t
//                              B[k][j]: j = l % 16, k = 8(l/16) + t
//                              C[i][j]: j = l % 16, i = 4(l/16) + r
// ds_read_b64_tr_b16 (LDS transpose read): within each group of 16 lanes, lane
// i receives element (i % 4) of the 4-element chunk addressed by lane
// 4t + i/4, for t = 0..3.  If lane j = 4t + s of a group points at row
// (r0 + t), columns (c0 + 4s .. c0 + 4s + 3) of a row-major tile, lane i gets
// rows r0..r0+3 of column c0 + i: a column segment of the tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte LDS load (one MFMA operand of 8 bf16).
__device__ __forceinline__ bf16x8 lds_read8(const bf16* p) {
  return *(const FA_LDS bf16x8*)(p);
}

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane
// l's 16 bytes from `src` land at lds_base + 16 * l.  lds_base must be the
// same for every lane of the wave.  Completion is tracked by the vector
// memory counter; a workgroup barrier (which waits for it) publishes the data.
__device__ __forceinline__ void lds_load16(const bf16* src, bf16* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (FA_LDS void*)lds_base, 16, 0, 0);
}

// Direct HBM -> LDS copy of 4 bytes per lane (lane l's value lands at
// lds_base + 4 * l); same rules as lds_load16.
__device__ __forceinline__ void lds_load4(const float* src, float* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (FA_LDS void*)lds_base, 4, 0, 0);
}

// Transposed 8-byte LDS read (see the layout note at the top of the file).
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, r);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + x.x + x.y in fp32 (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float dot2_ones(bf16x2 x, float acc) {
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(x, ones, acc, false);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Reductions across the two halves of the wave (lanes l and l ^ 32), through
// ds_bpermute_b32.  (v_permlane32_swap would do this in one VALU op, but the
// ROCm 7.2 compiler miscompiles its second result when the two results are
// consumed separately -- it reuses the first result's register -- so it is
// not used.)
__device__ __forceinline__ float other_half(float x) {
  const int src = ((int)(threadIdx.x & 63) ^ 32) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float half_pair_max(float x) { return fmaxf(x, other_half(x)); }

__device__ __forceinline__ float half_pair_sum(float x) { return x + other_half(x); }

// Wait until every global load this wave has issued has returned
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their no-wait maxima).
// Used after loading register-resident operands before a loop, so that the
// loop's own prefetch loads are not waited on by the first use of those
// operands: the vector-memory counter retires in order.
__device__ __forceinline__ void wait_global_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// f32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                        float a5, float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16)a0; r[1] = (bf16)a1; r[2] = (bf16)a2; r[3] = (bf16)a3;
  r[4] = (bf16)a4; r[5] = (bf16)a5; r[6] = (bf16)a6; r[7] = (bf16)a7;
  return r;
}

// XOR swizzle of a row-major LDS tile with D bf16 per row (no padding),
// applied to the 16-byte chunk index: chunk q of row r is stored at chunk
// q ^ swz(r).  With the LDS seen as 64 banks of 4 bytes, it makes both
// access patterns the kernels use conflict-free:
//   * 16 consecutive rows reading the same chunk (ds_read_b128 operand rows);
//   * 4 consecutive rows (first row a multiple of 4) reading 4 consecutive
//     chunks (first a multiple of 4) -- half a wave of ds_read_b64_tr_b16.
// D = 128: a row is 16 chunks (256 B); swz(r) = 4(r%4) + (r/4)%4 maps the 16
// rows of an aligned group to 16 distinct chunks, and 4 aligned rows to 4
// distinct groups of 4 chunks.  D = 64: two rows share one 256-byte bank
// line; swz(r) = 4((r/2)%2) + (r/4)%4 does the same per row parity.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// The visible entries of one row or column of a tile mask (entry i at
// base[i * stride], i < n, nonzero = visible), read 64 entries at a time: one
// byte load per lane and a wave vote give a wave-uniform bitmask, so finding
// the next visible entry is a bit scan rather than a chain of dependent byte
// loads (each a full memory round trip).  Every lane of the wave must call
// next() together.
struct MaskScan {
  const uint8_t* base;
  long long stride;
  int n;
  int chunk;       // first entry of the cached 64 (a multiple of 64), -1: none
  uint64_t bits;   // bit j: entry chunk + j is visible

  __device__ MaskScan(const uint8_t* b, long long st, int count)
      : base(b), stride(st), n(count), chunk(-1), bits(0) {}

  // The first visible entry at or after i, or n if there is none.
  __device__ __forceinline__ int next(int i) {
    while (i < n) {
      const int c = i & ~63;
      if (c != chunk) {
        const int e = c + (int)(threadIdx.x & 63);
        const bool on = e < n && base[(size_t)e * stride] != 0;
        bits = __builtin_amdgcn_ballot_w64(on);
        chunk = c;
      }
      const uint64_t rest = bits >> (i - c);
      if (rest != 0) return i + (int)__builtin_ctzll(rest);
      i = c + 64;
    }
    return n;
  }
};

// Workgroup index -> work item, so that consecutive items stay on one XCD
// (the hardware deals workgroups to the 8 XCDs round-robin; each XCD has its
// own L2, and items of one head reuse the same K/V).  Falls back to identity
// when the count does not split evenly.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  constexpr int kXcd = 8;
  if (total % kXcd != 0) return wg;
  const int per = total / kXcd;
  return (wg % kXcd) * per + wg / kXcd;
}

// Work item w (an xcd_remap output) of a grid of `total` items, `ntile` tiles
// per head, for causal work whose cost falls with the tile's rank (rank 0 is
// the heaviest).  When each XCD's share holds whole heads, the share is
// ordered heaviest first across all its heads (every head's rank-0 tile, then
// every head's rank-1 tile, ...), so that the light tiles fill the tail;
// otherwise heaviest first within each head.
__device__ __forceinline__ void causal_order(int w, int total, int ntile, int& head, int& rank) {
  constexpr int kXcd = 8;
  if (total % kXcd == 0 && (total / kXcd) % ntile == 0) {
    const int per = total / kXcd, hpx = per / ntile, j = w % per;
    head = (w / per) * hpx + j % hpx;
    rank = j / hpx;
  } else {
    head = w / ntile;
    rank = w % ntile;
  }
}

}  // namespace fa
