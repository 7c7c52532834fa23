// fa_fwd_fp8.hip -- exact attention forward with fp8 Q, K, V (OCP e4m3), gfx950.
//
// The same tiled, online-softmax forward as fa_fwd.hip ("FlashAttention."
// plate, opening section and "Never write the scores"), with both products on
// the 8-bit matrix instruction v_mfma_f32_32x32x64_f8f6f4, which does twice
// the bf16 work per cycle.  Lower-precision matrix inputs are the direction
// the plate's "Never write the scores" section names for the H100 generation
// of the method; the layouts here are gfx950's own.
//
// Numerics: the stored inputs are fp8 codes with one fp32 descale per tensor
// (real value = code * descale).  S = scale * (q_descale Q)(k_descale K)^T is
// exact products with fp32 accumulation; the descales fold into the softmax
// constant.  P is rounded to fp8 for the second product, stored shifted as
// exp2(s - m + 8) in [0, 256] so that typical weights stay in e4m3's normal
// range; the running maximum m is updated whenever it grows (no lazy
// threshold, which would let the shifted weights overflow e4m3's 448).  The
// row sum l is accumulated from the unrounded fp32 weights.  O is written in
// bf16, LSE in fp32.
//
// Operand layouts (measured on the device):
//   * the 32x32x64 instruction pairs byte t of lane (i + 32h) of A with byte t
//     of lane (j + 32h) of B; its accumulator layout is the one of the bf16
//     32x32 instruction (fa_common.hpp).  So the contraction index of byte t
//     of half h is ours to choose, as long as A and B agree;
//   * ds_read_b64_tr_b8: in each 16-lane group, lane 2e + s addresses row
//     r0 + e, bytes c0 + 8s .. + 7 of a row-major byte tile, and lane i
//     receives rows r0 .. r0 + 7 of column c0 + i (byte e = row r0 + e).
// S^T = K Q^T contracts over d with byte t of half h = d 64c + 32h + t, so A
// (K rows) and B (the wave's Q^T, in registers) are 32 contiguous bytes per
// lane.  O^T += V^T P^T contracts over the 64 keys of a tile in one
// instruction: byte t = 16kb + r of half h is key 32kb + 8(r/4) + 4h + r%4,
// which is exactly the key the lane's own S^T accumulator register r of key
// block kb holds, so P packs straight from the accumulators.  The V tile is
// stored with its rows permuted (key 32kb + 8g + 4h + e at row
// 32h + 16kb + 4g + e) so that each lane's keys are 32 consecutive rows:
// four transpose reads.
#include "fa_common.hpp"
#include "fa_internal.hpp"


namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned char u8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kPShift = 8.0f;  // log2 of the factor the stored weights carry
constexpr int kAcc = 4;          // independent partial maxima and sums per lane

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = e4m3 for A and B; scale exponents 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x4 lds_read16(const u8* p) { return *(const FA_LDS i32x4*)(p); }

__device__ __forceinline__ i32x2 lds_read_tr8(const u8* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2*)(const_cast<u8*>(p)));
}

__device__ __forceinline__ void dma16(const u8* src, u8* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (FA_LDS void*)lds_base, 16, 0, 0);
}

// XOR swizzles of the 16-byte chunk index (rows of D bytes, 64 banks of 4 B):
// k_swz keeps 16 consecutive K rows reading one chunk conflict-free; v_swz
// keeps the transpose reads (8 rows x 2 adjacent chunks per half wave)
// conflict-free.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? 2 * ((r >> 1) & 3) : 2 * ((r >> 2) & 1);
}

__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d) {
  int x = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, x, true);
}

// Four waves (128 query rows) per workgroup for both head sizes. d = 128 holds
// about 165 VGPRs, so three workgroups share a CU (three waves per SIMD); that
// leaves more waves to hide one wave's softmax behind another's MFMAs than two
// 8-wave workgroups would. d = 64 fits four per SIMD.
constexpr int kWaves = 4;

template <int D>
constexpr int kWavesPerSimd = D == 128 ? 3 : 4;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kWaves)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>, kWavesPerSimd<D>)))
void fwd_fp8_kernel(FwdArgs a) {
  constexpr int NW = kWaves;
  constexpr int kThreads = 64 * NW;
  constexpr int BR = 32 * NW;      // query rows per workgroup
  constexpr int BC = 64;           // keys per tile
  constexpr int NB = BC / 32;      // 32-key blocks per tile
  constexpr int DC = D / 64;       // contraction steps of S^T = K Q^T
  constexpr int DB = D / 32;       // 32-row blocks of O^T
  constexpr int CH = D / 16;       // 16-byte chunks per row
  constexpr int LOADS = BC * CH / kThreads;
  static_assert(BC * CH % kThreads == 0 && LOADS >= 1, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) u8 k_s0[BC * D];
  __shared__ __attribute__((aligned(16))) u8 k_s1[BC * D];
  __shared__ __attribute__((aligned(16))) u8 v_s0[BC * D];
  __shared__ __attribute__((aligned(16))) u8 v_s1[BC * D];

  const int N = a.N;
  const int nq = (N + BR - 1) / BR;
  const int total = nq * a.B * a.H;
  const int w = xcd_remap(blockIdx.x, total);
  int bh = w / nq, qt = w % nq;
  if constexpr (CAUSAL) {  // heaviest (last) query tiles first
    int rank;
    causal_order(w, total, nq, bh, rank);
    qt = nq - 1 - rank;
  }
  const int q0 = qt * BR;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const size_t head = (size_t)bh * (size_t)N * D;  // elements = bytes for fp8
  const u8* __restrict__ Q = reinterpret_cast<const u8*>(a.q) + head;
  const u8* __restrict__ K = reinterpret_cast<const u8*>(a.k) + head;
  const u8* __restrict__ V = reinterpret_cast<const u8*>(a.v) + head;
  bf16* __restrict__ O = reinterpret_cast<bf16*>(a.o) + head;

  // Q^T operand: query row qrow, d = 64c + 32h .. +31.
  const int qrow = q0 + 32 * wave + l32;
  const int qld = qrow < N ? qrow : N - 1;
  i32x8 qf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(Q + (size_t)qld * D + 64 * c + 32 * h);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(Q + (size_t)qld * D + 64 * c + 32 * h + 16);
    qf[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }

  const int nt = (N + BC - 1) / BC;
  const int qmax = min(q0 + BR, N) - 1;
  const int tend = CAUSAL ? min(nt, qmax / BC + 1) : nt;

  // HBM -> LDS direct loads: lane l of a wave's i-th load fills the 16 bytes
  // at LDS position p = (i * NW + wave) * 64 + l, i.e. row p / CH, slot p % CH.
  auto load_tile = [&](int t, u8* Ks, u8* Vs) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int base = (i * NW + wave) * 64;
      const int p = base + lane;
      const int row = p / CH;
      const int slot = p % CH;
      // K: natural row order.
      const size_t ks = (size_t)min(t * BC + row, N - 1) * D + 16 * (slot ^ k_swz<D>(row));
      dma16(K + ks, Ks + 16 * base);
      // V: LDS row `row` holds key 32kb + 8g + 4h + e for row = 32h + 16kb + 4g + e.
      const int key = 32 * ((row & 31) >> 4) + 8 * ((row & 15) >> 2) + 4 * (row >> 5) + (row & 3);
      const size_t vs = (size_t)min(t * BC + key, N - 1) * D + 16 * (slot ^ v_swz<D>(row));
      dma16(V + vs, Vs + 16 * base);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m_ref = -INFINITY;  // running maximum (log2 units) of the scores
  // Running sum of this lane's shifted weights, in kAcc independent parts
  // (one chain of dependent adds would stall every tile).
  float l_part[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) l_part[i] = 0.f;
  const float sl2 = a.scale * a.q_descale * a.k_descale * kLog2e;

  // Lane-invariant address parts.  K operand rows 32kb + l32, chunks
  // 4c + 2h (+1).  V^T transpose reads: rows 32h + 8q + tr_row, chunk
  // 2b + tr_half, bytes 8 tr_s.
  const int ksw = k_swz<D>(l32);
  const int tr_row = (lane & 15) >> 1;
  const int tr_half = (lane >> 4) & 1;
  const int tr_s = lane & 1;
  const int vsw = v_swz<D>(tr_row);  // equals v_swz of row 32h + 8q + tr_row

  auto tile_step = [&](int& t, const u8* Ks, const u8* Vs, u8* Kn, u8* Vn) {
    const int tn = t + 1;
    if (tn < tend) load_tile(tn, Kn, Vn);  // lands during this tile's math
    const int k0 = t * BC;
    if (!CAUSAL || k0 <= q0 + 32 * wave + 31) {
      f32x16 s[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const u8* kr = Ks + (32 * kb + l32) * D;
          const i32x4 lo = lds_read16(kr + 16 * ((4 * c + 2 * h) ^ ksw));
          const i32x4 hi = lds_read16(kr + 16 * ((4 * c + 2 * h + 1) ^ ksw));
          s[kb] = mfma_f8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qf[c], s[kb]);
        }
      }
      // Masking: causal tiles crossing this wave's diagonal, and the ragged tail.
      const bool diag = CAUSAL && (k0 + BC - 1 > q0 + 32 * wave);
      if (diag || k0 + BC > N) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
          }
      }
      // Online softmax (base 2), maximum updated whenever it grows.
      float mpart[kAcc];
#pragma unroll
      for (int i = 0; i < kAcc; ++i) mpart[i] = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mpart[r % kAcc] = fmaxf(mpart[r % kAcc], s[kb][r]);
      float mx = fmaxf(fmaxf(mpart[0], mpart[1]), fmaxf(mpart[2], mpart[3]));
      // The halves' maxima are exchanged only when some lane's maximum
      // exceeds the reference (the two halves hold keys of one query row).
      if (__builtin_amdgcn_ballot_w64(mx * sl2 > m_ref) != 0) {
        mx = half_pair_max(mx);
        const float m_new = fmaxf(m_ref, mx * sl2);
        if (m_new > m_ref) {
          const float alpha = fast_exp2(m_ref - m_new);
          m_ref = m_new;
#pragma unroll
          for (int i = 0; i < kAcc; ++i) l_part[i] *= alpha;
#pragma unroll
          for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        }
      }
      const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[kb][r], sl2, kPShift - mu));
          s[kb][r] = p;
          l_part[r % kAcc] += p;
        }
      // P^T operand: byte 16kb + r of this lane = weight s[kb][r].
      i32x8 pb;
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int kb = wd >> 2, r = 4 * (wd & 3);
        pb[wd] = pack4_fp8(s[kb][r], s[kb][r + 1], s[kb][r + 2], s[kb][r + 3]);
      }
      // O^T += V^T P^T over the tile's 64 keys.
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const int off = 16 * ((2 * b + tr_half) ^ vsw) + 8 * tr_s;
        i32x8 va;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x2 x = lds_read_tr8(Vs + (32 * h + 8 * q + tr_row) * D + off);
          va[2 * q] = x[0];
          va[2 * q + 1] = x[1];
        }
        oacc[b] = mfma_f8(va, pb, oacc[b]);
      }
    }
    __syncthreads();  // also drains this wave's direct loads of tile tn
    t = tn;
  };

  wait_global_loads();  // Q operands resident before the key loop
  int t = 0;
  if (t < tend) load_tile(t, k_s0, v_s0);
  __syncthreads();
  while (t < tend) {
    tile_step(t, k_s0, v_s0, k_s1, v_s1);
    if (t >= tend) break;
    tile_step(t, k_s1, v_s1, k_s0, v_s0);
  }

  // Epilogue: O = v_descale * acc / l (bf16), LSE in natural units.
  const float l_tot = half_pair_sum((l_part[0] + l_part[1]) + (l_part[2] + l_part[3]));
  const float inv = l_tot > 0.f ? a.v_descale / l_tot : 0.f;
  if (qrow < N) {
    if (h == 0)
      a.lse[(size_t)bh * N + qrow] =
          l_tot > 0.f ? (m_ref - kPShift + fast_log2(l_tot)) * kLn2 : -INFINITY;
    bf16* orow = O + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = to_bf16(oacc[b][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * g + 4 * h) = v4;
      }
  }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  constexpr int BR = 32 * kWaves;
  const int nq = (a.N + BR - 1) / BR;
  const long long grid = (long long)nq * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<D, true>), dim3((unsigned)grid), dim3(64 * kWaves), 0, s,
                       a);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<D, false>), dim3((unsigned)grid), dim3(64 * kWaves), 0,
                       s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t s) {
  if (a.mask || a.Hkv != a.H) return hipErrorInvalidValue;
  if (a.d == 128) return launch_d<128>(a, s);
  if (a.d == 64) return launch_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
