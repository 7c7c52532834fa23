// fa_resident.hpp -- shared pieces of the d = 128 kernels whose workgroups
// stay resident (one per CU) and run a generated, register-pinned key loop
// between C++ set-up and epilogue: fa_fwd128.hip, fa_bwd_dq128.hip and
// fa_bwd_dkdv128.hip.
//
// The generated loop overwrites every vector register and most scalar ones,
// so the C++ around it re-derives what it needs in each round of the
// workgroup's item loop: lane values from the exec mask (`fresh_lane`), sizes
// and pointers through an opaque statement (`fresh`), which keeps the
// compiler from hoisting anything across the loop (and from spilling it).
// Direct loads issued here are inline assembly the compiler does not track,
// so it never waits on them by itself; the kernels wait explicitly.
#pragma once

#include <atomic>

#include "fa_common.hpp"

namespace fa {

// One direct HBM -> LDS load of 16 bytes per lane: lane l's bytes at
// gbase + voff land at LDS byte address m0 + 16 l.  The caller waits
// (s_waitcnt vmcnt) and synchronises before any wave reads them, and issues
// it only once every read of that LDS has returned.  The wait states before
// the load cover M0 and a base the vector unit may have just written to a
// scalar register (readfirstlane): the compiler adds none for the statement.
__device__ __forceinline__ void dma16_untracked(const void* gbase, uint32_t voff, uint32_t m0) {
  const uint64_t g = reinterpret_cast<uint64_t>(gbase);
  const uint64_t gs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(g >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)g);
  const uint32_t ms = (uint32_t)__builtin_amdgcn_readfirstlane((int)m0);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(ms), "v"(voff), "s"(gs)
               : "memory", "m0");
}

// The same with 4 bytes per lane: lane l's 4 bytes at gbase + voff land at
// LDS byte address m0 + 4 l.
__device__ __forceinline__ void dma4_untracked(const void* gbase, uint32_t voff, uint32_t m0) {
  const uint64_t g = reinterpret_cast<uint64_t>(gbase);
  const uint64_t gs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(g >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)g);
  const uint32_t ms = (uint32_t)__builtin_amdgcn_readfirstlane((int)m0);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(ms), "v"(voff), "s"(gs)
               : "memory", "m0");
}

// A vector value that is the same in every lane, as scalar bits (read from
// the first lane).  The wait states in front cover the hazard of reading a
// register the vector unit has just written: the compiler does not look
// inside the statement, so it inserts none of its own.
__device__ __forceinline__ uint32_t uniform_bits(float x) {
  uint32_t s;
  asm volatile("s_nop 4\n\tv_readfirstlane_b32 %0, %1" : "=s"(s) : "v"(x));
  return s;
}

// The lane index, recomputed where it is called (the statement is opaque).
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A wave-uniform value passed through an opaque statement.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+s"(x));
  return x;
}
__device__ __forceinline__ uint32_t fresh(uint32_t x) { return (uint32_t)fresh((int)x); }
__device__ __forceinline__ float fresh(float x) {
  return __builtin_bit_cast(float, fresh(__builtin_bit_cast(int, x)));
}
template <typename T>
__device__ __forceinline__ T* fresh(T* p) {
  const uint64_t x = reinterpret_cast<uint64_t>(p);
  return reinterpret_cast<T*>(((uint64_t)fresh((uint32_t)(x >> 32)) << 32) | fresh((uint32_t)x));
}

// Sizes of a launch, re-read in each round.
struct Shape {
  int N, H, Hkv, nq, total, nt;
  bool ragged;
};

template <int BR, int BC>
__device__ __forceinline__ Shape fresh_shape(int N, int B, int H, int Hkv) {
  Shape sh;
  sh.N = fresh(N);
  sh.H = fresh(H);
  sh.Hkv = fresh(Hkv);
  sh.nq = (sh.N + BR - 1) / BR;
  sh.total = sh.nq * fresh(B) * sh.H;
  sh.nt = (sh.N + BC - 1) / BC;
  sh.ragged = (sh.N % BC) != 0;
  return sh;
}

// A query tile of one head: BR rows from q0.
struct Item {
  int bh, q0;
};

// The workgroup stays resident and takes items in turn: round r's item is the
// one a one-item-per-workgroup launch would give to block b_r, where b_r walks
// this workgroup's XCD share (blocks b with b % 8 fixed) in a serpentine, so
// that causal items heavy early in one round pair with light ones in the next.
// False once the items are used up.
template <bool CAUSAL, int BR>
__device__ __forceinline__ bool resident_item(const Shape& sh, int r, Item& it) {
  const int G = fresh((int)gridDim.x), g = fresh((int)blockIdx.x);
  int b;
  if (G % 8 == 0 && sh.total % 8 == 0) {
    const int gx = G / 8, x = g % 8, k = g / 8;
    b = x + 8 * (r * gx + ((r & 1) ? gx - 1 - k : k));
  } else {
    b = r * G + ((r & 1) ? G - 1 - g : g);
  }
  if (b >= sh.total) return false;
  const int w = xcd_remap(b, sh.total);
  int bh = w / sh.nq, qt = w % sh.nq;
  if constexpr (CAUSAL) {
    int rank;
    causal_order(w, sh.total, sh.nq, bh, rank);
    qt = sh.nq - 1 - rank;
  }
  it.bh = __builtin_amdgcn_readfirstlane(bh);
  it.q0 = __builtin_amdgcn_readfirstlane(qt * BR);
  return true;
}

// Element offset of the K/V head that query head bh reads.
__device__ __forceinline__ size_t kv_head_offset(const Shape& sh, int bh, int D) {
  const int bkv = (bh / sh.H) * sh.Hkv + (bh % sh.H) / (sh.H / sh.Hkv);
  return (size_t)bkv * (size_t)sh.N * D;
}

// Direct loads of 64-row tile t (d = 128, bf16) of `src` into the 16 KiB LDS
// area at byte `lds`: wave w loads rows 16w .. 16w + 15, four rows per load,
// chunk q of row r to slot q ^ swz(r); rows past the sequence repeat its last
// row.
__device__ __forceinline__ void dma_tile128(const Shape& sh, int wave, const bf16* src, int t,
                                            uint32_t lds) {
  const int lane = fresh_lane();
  const int rows = min(64, sh.N - t * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * wave + 4 * i + (lane >> 4);
    const int col = 8 * ((lane & 15) ^ tile_swz<128>(row));
    dma16_untracked(src + (size_t)t * 64 * 128, (uint32_t)(min(row, rows - 1) * 128 + col) * 2u,
                    lds + 4096u * wave + 1024u * i);
  }
}

// Direct loads of one wave's 64 rows r0 .. r0 + 63 (d = 128, bf16) of a head
// into the 16 KiB LDS area at byte `lds`, chunk-swizzled like a tile (rows
// past the sequence repeat its last row).
__device__ __forceinline__ void dma_rows128(const Shape& sh, const bf16* head, int r0, uint32_t lds) {
  const int lane = fresh_lane();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 4 * i + (lane >> 4);
    const int col = 8 * ((lane & 15) ^ tile_swz<128>(row));
    dma16_untracked(head, (uint32_t)(min(r0 + row, sh.N - 1) * 128 + col) * 2u, lds + 1024u * i);
  }
}

// Direct loads of the 64 fp32 values of tile t of a per-row vector (one
// head's LSE or D) into 256 bytes of LDS at byte `lds` (rows past the
// sequence repeat its last row).
__device__ __forceinline__ void dma_vec64(const Shape& sh, const float* src, int t, uint32_t lds) {
  const int lane = fresh_lane();
  dma4_untracked(src + (size_t)t * 64, (uint32_t)(min(lane, sh.N - 1 - t * 64) * 4), lds);
}

// Resident workgroups: one per CU (each takes a whole CU's registers).
inline int resident_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace fa
