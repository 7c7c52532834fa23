// fa_bwd.hip -- exact attention backward, bf16 in / fp32 accumulate, gfx950.
//
// The probabilities are recomputed tile by tile from Q, K and the saved
// log-sum-exp instead of being stored ("FlashAttention." plate, "Never write
// the scores": the scores are recomputed in the backward pass).  The gradient
// formulas are the chain rule through P = softmax(S), S = scale Q K^T:
//   dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i (= sum_j P_ij dP_ij),
//   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Gradients are written in fp32: rounding them to bf16 alone would cost up
// to half a bf16 ulp (2^-6 for values in [4, 8), 2^-5 above 8), which is
// most of the 2e-2 absolute error budget the results are checked against.
//
// Grouped K/V heads (Hkv divides H; query head h reads K/V head h / (H/Hkv)):
// the gradient of a shared K/V head is the sum over the query heads that
// read it, accumulated inside one workgroup (the dK/dV workgroup loops over
// the group), so it stays deterministic.  A tile mask skips whole tiles in
// both passes: the dQ pass walks its mask row, the dK/dV pass its mask column.
//
// Three launches on the caller's stream, deterministic (no atomics):
//   1. bwd_delta: -D_i = -(dO_i . O_i) and LSE_i * log2(e) (fp32), into the
//      caller's workspace;
//   2. bwd_dkdv:  one workgroup per 128 keys loops over 64-query tiles of Q
//      and dO staged in LDS: S = Q K^T and
//      dP = dO V^T on MFMA (lane = key column), P = exp(S - LSE), dS, then
//      dV^T += dO^T P and dK^T += Q^T dS with dO^T / Q^T read from the
//      row-major LDS tiles by transpose reads.  d=64: each wave owns 32 keys,
//      K and V in registers.  d=128: two waves share 32 keys (K and V in LDS)
//      and split each query tile, and their partial sums meet in LDS;
//   3. bwd_dq:    one workgroup per 128 queries; each wave keeps 32 queries'
//      Q and dO in registers and loops over 64-key tiles of K and V, staged in
//      LDS by direct loads:
//      S^T = K Q^T, dP^T = V dO^T (lane = query column), dS^T, and
//      dQ^T += K^T dS^T with K^T read by transpose reads.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// Template modes: bit 0 = causal, bit 1 = tile mask.
enum Mode { kDense = 0, kCausal = 1, kSparse = 2, kSparseCausal = 3 };

// ---------------------------------------------------------------- D = dO.O
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(BwdArgs a, long long rows) {
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int RPB = kThreads / CH;    // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / CH;
  const int ch = threadIdx.x % CH;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 o = *reinterpret_cast<const bf16x8*>(
        reinterpret_cast<const bf16*>(a.o) + (size_t)row * D + 8 * ch);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(
        reinterpret_cast<const bf16*>(a.dout) + (size_t)row * D + 8 * ch);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, CH);
  if (row < rows && ch == 0) {
    a.delta[row] = -acc;   // negated: the d = 128 dK/dV loop starts its dP products from it
    a.lse2[row] = a.lse[row] * kLog2e;  // the dK/dV and dQ passes' exponent offset
  }
}

// ------------------------------------------------------------------ dK, dV
// NW waves per workgroup, 32 keys per wave; 64-query tiles of Q and dO are
// staged in swizzled LDS tiles (read row-wise for S = Q K^T and dP = dO V^T,
// and column-wise by transpose reads for dV^T += dO^T P and dK^T += Q^T dS).
template <int D, int NW>
struct DkdvTile {
  static constexpr int THREADS = 64 * NW;
  static constexpr int BK = 32 * NW;  // keys per workgroup
  static constexpr int BQ = 64;       // queries per loop step
  static constexpr int CH = D / 8;
  static constexpr int LOADS = BQ * CH / THREADS;  // direct loads per lane per tensor
  static constexpr int T_ELEMS = BQ * D;  // one tile (Q or dO), unpadded
  static_assert(BQ * CH % THREADS == 0, "tile must split evenly");
};

// Used for d=64: fp32 dK/dV accumulators (64 registers) and the K/V operands
// (32) stay resident at two waves per SIMD; 4-wave workgroups.
template <int D, int NW, int MODE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdArgs a) {
  using T = DkdvTile<D, NW>;
  constexpr bool CAUSAL = (MODE & kCausal) != 0;
  constexpr bool SPARSE = (MODE & kSparse) != 0;
  constexpr int DC = D / 16;
  constexpr int DB = D / 32;
  constexpr int QB = T::BQ / 32;

  __shared__ __attribute__((aligned(16))) bf16 tiles[2][2][T::T_ELEMS];  // [stage][Q|dO]
  __shared__ __attribute__((aligned(16))) float lse_s[2][T::BQ];
  __shared__ __attribute__((aligned(16))) float del_s[2][T::BQ];

  const int N = a.N;
  const int nkt = (N + T::BK - 1) / T::BK;
  const int total = nkt * a.B * a.Hkv * a.gsplit;
  const int w = xcd_remap(blockIdx.x, total);
  int bkv = w / nkt;  // (K/V head b * Hkv + hk) * gsplit + slice
  int kt = w % nkt;
  if constexpr (CAUSAL) causal_order(w, total, nkt, bkv, kt);  // small key tiles see the most queries
  const int slice = bkv % a.gsplit;
  bkv /= a.gsplit;
  const int kt0 = kt * T::BK;
  const int G = a.H / a.Hkv / a.gsplit;  // query heads of this slice
  // The slice's first query head.
  const int bq0 = (bkv / a.Hkv) * a.H + (bkv % a.Hkv) * (a.H / a.Hkv) + slice * G;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const size_t head = (size_t)bkv * N * D;
  const size_t qhead = (size_t)bq0 * N * D;
  const bf16* __restrict__ Q = reinterpret_cast<const bf16*>(a.q) + qhead;
  const bf16* __restrict__ K = reinterpret_cast<const bf16*>(a.k) + head;
  const bf16* __restrict__ V = reinterpret_cast<const bf16*>(a.v) + head;
  const bf16* __restrict__ dO = reinterpret_cast<const bf16*>(a.dout) + qhead;
  const float* __restrict__ LSE2 = a.lse2 + (size_t)bq0 * N;  // LSE * log2(e)
  const float* __restrict__ DEL = a.delta + (size_t)bq0 * N;

  // This wave's keys as B operands: K^T for S = Q K^T, V^T for dP = dO V^T.
  const int key = kt0 + 32 * wave + l32;
  const int kld = key < N ? key : N - 1;
  bf16x8 kf[DC], vf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    kf[c] = *reinterpret_cast<const bf16x8*>(K + (size_t)kld * D + 16 * c + 8 * h);
    vf[c] = *reinterpret_cast<const bf16x8*>(V + (size_t)kld * D + 16 * c + 8 * h);
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[b][r] = 0.f;
      dv[b][r] = 0.f;
    }

  const int nqt = (N + T::BQ - 1) / T::BQ;
  const int qt_begin = CAUSAL ? kt0 / T::BQ : 0;  // < nqt, since kt0 < N
  const float sl2 = a.scale * kLog2e;

  // The (query head g of the group, query tile qt) pairs this workgroup
  // visits, in order; with a tile mask, pairs whose mask entry
  // [qt * BQ / mb][kt0 / mb] is 0 are skipped (BK divides mb).
  const uint8_t* mcol = nullptr;
  int mb = 1, nmb = 1;
  if constexpr (SPARSE) {
    mb = a.mask_block;
    nmb = (N + mb - 1) / mb;
    mcol = a.mask + kt0 / mb;
  }
  MaskScan mscan(mcol, nmb, SPARSE ? nmb : 0);  // this workgroup's mask column
  struct Pos {
    int g, qt;
  };
  auto advance = [&](Pos p) {  // the first visited pair at or after p
    for (;;) {
      if (p.qt >= nqt) {
        p.qt = qt_begin;
        ++p.g;
      }
      if (p.g >= G) return p;
      if constexpr (SPARSE) {
        const int blk = (p.qt * T::BQ) / mb;
        const int vb = mscan.next(blk);
        if (vb == blk) return p;
        p.qt = (vb * mb) / T::BQ;  // first query tile of that block, or past the end
      } else {
        return p;
      }
    }
  };

  // HBM -> LDS direct loads of one 64-query tile of Q and dO (16-byte chunk q
  // of row r stored at chunk q ^ tile_swz(r)) plus its LSE and D rows.
  auto load_tile = [&](Pos p, int st) {
    const size_t ho = (size_t)p.g * N * D;
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int base = (i * NW + wave) * 64;
      const int lp = base + lane;
      const int row = lp / T::CH;
      const int q = (lp % T::CH) ^ tile_swz<D>(row);
      const size_t src = ho + (size_t)min(p.qt * T::BQ + row, N - 1) * D + 8 * q;
      lds_load16(Q + src, &tiles[st][0][8 * base]);
      lds_load16(dO + src, &tiles[st][1][8 * base]);
    }
    const size_t qr = (size_t)p.g * N + min(p.qt * T::BQ + lane, N - 1);
    if (wave == 0) lds_load4(LSE2 + qr, &lse_s[st][0]);
    if (wave == 1) lds_load4(DEL + qr, &del_s[st][0]);
  };

  // Per-lane swizzle terms.  Row-wise operand reads: row 32qb + l32, chunk
  // 2c + h.  Transpose reads: rows 32qb + 16cc + tr_row (+8), chunk
  // 4b + (tr_col >> 3), element (tr_col & 7) within the chunk.
  const int sw_row = tile_swz<D>(l32);
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int sw_lo = tile_swz<D>(tr_row), sw_hi = tile_swz<D>(tr_row + 8);
  const int tq = tr_col >> 3, te = tr_col & 7;
  auto tr_off = [&](int row, int sw, int b) {
    return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te;
  };

  wait_global_loads();  // K, V operands resident before the query loop
  Pos cur = advance(Pos{0, qt_begin});
  if (cur.g < G) load_tile(cur, 0);
  __syncthreads();
  int stage = 0;
  while (cur.g < G) {
    const Pos nxt = advance(Pos{cur.g, cur.qt + 1});
    if (nxt.g < G) load_tile(nxt, stage ^ 1);  // lands during this tile's math
    const bf16* Qs = tiles[stage][0];
    const bf16* Os = tiles[stage][1];
    const int q0 = cur.qt * T::BQ;
    const bool need_mask = (CAUSAL && q0 < kt0 + 32 * wave + 31) || (q0 + T::BQ > N);

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
      const int rrow = (32 * qb + l32) * D;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const int off = rrow + 8 * ((2 * c + h) ^ sw_row);
        s = mfma32(lds_read8(Qs + off), kf[c], s);
        dp = mfma32(lds_read8(Os + off), vf[c], dp);
      }
      // Issue order: operand reads two MFMAs ahead.
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 2 * DC - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      // s[r], dp[r]: query 32qb + 8(r/4) + 4h + r%4 of this tile, key `key`.
      // Masked and unmasked copies behind one wave-uniform branch.
      auto probs = [&](auto masked) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = 32 * qb + 8 * g + 4 * h;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_s[stage][ql]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&del_s[stage][ql]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float p = fast_exp2(fmaf(s[r], sl2, -l4[e]));
            if constexpr (decltype(masked)::value) {
              const int q = q0 + ql + e;
              if (q >= N || (CAUSAL && key > q)) p = 0.f;
            }
            s[r] = p;
            dp[r] = p * (dp[r] + d4[e]);
          }
        }
      };
      if (need_mask) probs(std::true_type{});
      else probs(std::false_type{});
      // dV^T += dO^T P ; dK^T += Q^T dS   (contraction over this block's queries)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const bf16x8 pb = pack8(s[8 * cc + 0], s[8 * cc + 1], s[8 * cc + 2], s[8 * cc + 3],
                                s[8 * cc + 4], s[8 * cc + 5], s[8 * cc + 6], s[8 * cc + 7]);
        const bf16x8 db = pack8(dp[8 * cc + 0], dp[8 * cc + 1], dp[8 * cc + 2], dp[8 * cc + 3],
                                dp[8 * cc + 4], dp[8 * cc + 5], dp[8 * cc + 6], dp[8 * cc + 7]);
        const int r_lo = 32 * qb + 16 * cc + tr_row;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const int o_lo = tr_off(r_lo, sw_lo, b), o_hi = tr_off(r_lo + 8, sw_hi, b);
          dv[b] = mfma32(cat8(lds_read_tr4(Os + o_lo), lds_read_tr4(Os + o_hi)), pb, dv[b]);
          dk[b] = mfma32(cat8(lds_read_tr4(Qs + o_lo), lds_read_tr4(Qs + o_hi)), db, dk[b]);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * 2, 0);
#pragma unroll
      for (int i = 0; i < 4 * DB - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __syncthreads();  // also drains this wave's direct loads of the next tile
    stage ^= 1;
    cur = nxt;
  }

  // dK^T, dV^T (fp32 out): lane holds key `key`, d = 32b + 8(r/4) + 4h + r%4.
  if (key < N) {
    const size_t kvsize = (size_t)a.B * a.Hkv * N * D;
    float* dkrow = (a.gsplit > 1 ? a.part + slice * kvsize : a.dk) + head + (size_t)key * D;
    float* dvrow =
        (a.gsplit > 1 ? a.part + (a.gsplit + slice) * kvsize : a.dv) + head + (size_t)key * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = dk[b][4 * g + e] * a.scale;
          v4[e] = dv[b][4 * g + e];
        }
        *reinterpret_cast<f32x4*>(dkrow + 32 * b + 8 * g + 4 * h) = k4;
        *reinterpret_cast<f32x4*>(dvrow + 32 * b + 8 * g + 4 * h) = v4;
      }
  }
}

// dK, dV for d = 128: 8-wave workgroups of 128 keys.  Waves w and w + 4 own
// the same 32 keys and take the two 32-query halves of every 64-query tile;
// their partial dK/dV are summed through LDS at the end in a fixed order, so
// the result stays deterministic.  K and V are read from an LDS copy instead
// of being held as register operands, which brings a wave under 256 registers
// (fp32 dK/dV accumulators 128, S and dP 32, loop-invariant LDS offsets 25):
// two waves share a SIMD, so one wave's exponentials overlap the other's
// matrix instructions.  LDS is one hand-laid-out array, so that every operand
// read is a loop-invariant offset register plus an immediate.
constexpr int kSplitKeys = 128;  // keys per workgroup (4 blocks of 32)

// Direct HBM -> LDS copies issued as inline assembly: the compiler does not
// track them, so it inserts no wait for them before LDS reads; the kernel
// waits (vmcnt) before the barrier that publishes each tile.
__device__ __forceinline__ void dma16_untracked(const void* src, unsigned lds_byte) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}
// Same, with a wave-uniform base address in scalar registers and a 32-bit
// per-lane byte offset (no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void dma16_sbase(const void* base, unsigned off, unsigned lds_byte) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_sbase(const void* base, unsigned off, unsigned lds_byte) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_untracked(const void* src, unsigned lds_byte) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

template <int D, int MODE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_split_kernel(BwdArgs a) {
  constexpr bool CAUSAL = (MODE & kCausal) != 0;
  constexpr bool SPARSE = (MODE & kSparse) != 0;
  constexpr int NW = 8;
  constexpr int BK = kSplitKeys;
  constexpr int BQ = 64;
  constexpr int CH = D / 8;
  constexpr int LOADS = BQ * CH / (64 * NW);
  constexpr int KV_LOADS = BK * CH / (64 * NW);
  constexpr int DC = D / 16;
  constexpr int DB = D / 32;
  static_assert(D == 128, "byte layout below is for d = 128");
  // LDS byte layout: stage s at 32 KB s = [Q tile 16 KB | dO tile 16 KB];
  // K at 64 KB, V at 96 KB (32 KB each); LSE * log2(e), D rows of stage s at
  // 128 KB + 512 s (+256 for D).  Stage offsets and the dO / V / D
  // displacements are compile-time constants that fold into the reads'
  // immediate offsets.
  constexpr unsigned kStage = 32768, kDO = 16384, kK = 65536, kV = 32768, kRows = 131072;
  __shared__ __attribute__((aligned(16))) char lds[kRows + 1024];

  const int N = a.N;
  const int nkt = (N + BK - 1) / BK;
  const int total = nkt * a.B * a.Hkv * a.gsplit;
  const int w = xcd_remap(blockIdx.x, total);
  int bkv = w / nkt;  // (K/V head) * gsplit + slice
  int kt = w % nkt;
  if constexpr (CAUSAL) causal_order(w, total, nkt, bkv, kt);
  const int slice = bkv % a.gsplit;
  bkv /= a.gsplit;
  const int kt0 = kt * BK;
  const int G = a.H / a.Hkv / a.gsplit;  // query heads of this slice
  const int bq0 = (bkv / a.Hkv) * a.H + (bkv % a.Hkv) * (a.H / a.Hkv) + slice * G;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kw = wave & 3;
  const int qh = wave >> 2;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const size_t head = (size_t)bkv * N * D;
  const size_t qhead = (size_t)bq0 * N * D;
  const bf16* __restrict__ Q = reinterpret_cast<const bf16*>(a.q) + qhead;
  const bf16* __restrict__ K = reinterpret_cast<const bf16*>(a.k) + head;
  const bf16* __restrict__ V = reinterpret_cast<const bf16*>(a.v) + head;
  const bf16* __restrict__ dO = reinterpret_cast<const bf16*>(a.dout) + qhead;
  const float* __restrict__ LSE2 = a.lse2 + (size_t)bq0 * N;  // LSE * log2(e)
  const float* __restrict__ DEL = a.delta + (size_t)bq0 * N;
  const unsigned lds0 = (unsigned)(size_t)(FA_LDS void*)lds;

  const int key = kt0 + 32 * kw + l32;

#pragma unroll
  for (int i = 0; i < KV_LOADS; ++i) {
    const int base = (i * NW + wave) * 64;
    const int lp = base + lane;
    const int row = lp / CH;
    const int q = (lp % CH) ^ tile_swz<D>(row);
    const size_t src = (size_t)min(kt0 + row, N - 1) * D + 8 * q;
    dma16_untracked(K + src, lds0 + kK + 16 * base);
    dma16_untracked(V + src, lds0 + kK + kV + 16 * base);
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[b][r] = 0.f;
      dv[b][r] = 0.f;
    }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt_begin = CAUSAL ? kt0 / BQ : 0;
  const float sl2 = a.scale * kLog2e;

  const uint8_t* mcol = nullptr;
  int mb = 1, nmb = 1;
  if constexpr (SPARSE) {
    mb = a.mask_block;
    nmb = (N + mb - 1) / mb;
    mcol = a.mask + kt0 / mb;
  }
  MaskScan mscan(mcol, nmb, SPARSE ? nmb : 0);  // this workgroup's mask column
  struct Pos {
    int g, qt;
  };
  auto advance = [&](Pos p) {
    for (;;) {
      if (p.qt >= nqt) {
        p.qt = qt_begin;
        ++p.g;
      }
      if (p.g >= G) return p;
      if constexpr (SPARSE) {
        const int blk = (p.qt * BQ) / mb;
        const int vb = mscan.next(blk);
        if (vb == blk) return p;
        p.qt = (vb * mb) / BQ;  // first query tile of that block, or past the end
      } else {
        return p;
      }
    }
  };

  // Per-lane byte offsets of the direct loads within a whole tile.
  unsigned loff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int lp = (i * NW + wave) * 64 + lane;
    const int row = lp / CH;
    loff[i] = 2 * (row * D + 8 * ((lp % CH) ^ tile_swz<D>(row)));
  }
  auto load_tile = [&](Pos p, unsigned st) {
    const size_t ho = (size_t)p.g * N * D;
    if ((p.qt + 1) * BQ <= N) {  // whole tile in range: scalar base + lane offsets
      const size_t t0 = ho + (size_t)p.qt * BQ * D;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const unsigned dst = lds0 + st * kStage + 16 * ((i * NW + wave) * 64);
        dma16_sbase(Q + t0, loff[i], dst);
        dma16_sbase(dO + t0, loff[i], dst + kDO);
      }
      const size_t r0 = (size_t)p.g * N + (size_t)p.qt * BQ;
      if (wave == 0) dma4_sbase(LSE2 + r0, 4 * lane, lds0 + kRows + 512 * st);
      if (wave == 1) dma4_sbase(DEL + r0, 4 * lane, lds0 + kRows + 512 * st + 256);
      return;
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int base = (i * NW + wave) * 64;
      const int lp = base + lane;
      const int row = lp / CH;
      const int q = (lp % CH) ^ tile_swz<D>(row);
      const size_t src = ho + (size_t)min(p.qt * BQ + row, N - 1) * D + 8 * q;
      dma16_untracked(Q + src, lds0 + st * kStage + 16 * base);
      dma16_untracked(dO + src, lds0 + st * kStage + kDO + 16 * base);
    }
    const size_t qr = (size_t)p.g * N + min(p.qt * BQ + lane, N - 1);
    if (wave == 0) dma4_untracked(LSE2 + qr, lds0 + kRows + 512 * st);
    if (wave == 1) dma4_untracked(DEL + qr, lds0 + kRows + 512 * st + 256);
  };

  // Loop-invariant per-lane byte offsets.  Row-wise reads: row 32qh + l32 of
  // the Q tile (K: row 32kw + l32), chunk (2c + h) ^ tile_swz(l32).
  const int sw_row = tile_swz<D>(l32);
  unsigned qoff[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) qoff[c] = (32 * qh + l32) * D * 2 + 16 * ((2 * c + h) ^ sw_row);
  // K rows sit a wave-uniform distance from this wave's Q rows (one scalar
  // add per K read instead of 8 more offset registers).
  unsigned kdelta = __builtin_amdgcn_readfirstlane(kK + 64 * D * (kw - qh));
  // Transpose reads: rows 32qh + 16cc + tr_row (+8), chunk 4b + (tr_col >> 3),
  // element tr_col & 7; the cc term is a constant 16-row step.
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int sw_lo = tile_swz<D>(tr_row), sw_hi = tile_swz<D>(tr_row + 8);
  const int tq = tr_col >> 3, te = tr_col & 7;
  unsigned troff[DB][2];
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    troff[b][0] = 2 * ((32 * qh + tr_row) * D + 8 * (((4 * b) ^ (sw_lo & 12)) | (tq ^ (sw_lo & 3))) + te);
    troff[b][1] = 2 * ((32 * qh + tr_row + 8) * D + 8 * (((4 * b) ^ (sw_hi & 12)) | (tq ^ (sw_hi & 3))) + te);
  }
  const unsigned rowoff = kRows + 4 * (32 * qh + 4 * h);

  auto rd8 = [&](unsigned off) { return *(const FA_LDS bf16x8*)(lds + off); };
  auto rdtr = [&](unsigned off) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(lds + off));
    return __builtin_bit_cast(bf16x4, r);
  };

  Pos cur = advance(Pos{0, qt_begin});
  if (cur.g < G) load_tile(cur, 0);
  wait_global_loads();
  __syncthreads();  // K/V and the first tile resident

  unsigned st = 0;  // current stage
  auto tile_step = [&]() {
    // so: byte offset of the current stage, loop-carried so that the
    // compiler cannot hoist one address register per stage out of the loop.
    const unsigned so = st * kStage;
    asm volatile("" : "+s"(kdelta));  // opaque per step, so K addresses are not hoisted
    const Pos nxt = advance(Pos{cur.g, cur.qt + 1});
    if (nxt.g < G) load_tile(nxt, st ^ 1);
    const int q0 = cur.qt * BQ + 32 * qh;
    const bool empty = (CAUSAL && q0 + 31 < kt0 + 32 * kw) || q0 >= N;
    if (!empty) {
      const bool need_mask = (CAUSAL && q0 < kt0 + 32 * kw + 31) || (q0 + 32 > N);
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const unsigned qa = qoff[c] + so;
        const unsigned ka = qoff[c] + kdelta;
        s = mfma32(rd8(qa), rd8(ka), s);
        dp = mfma32(rd8(qa + kDO), rd8(ka + kV), dp);
      }
      auto probs = [&](auto masked) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *(const FA_LDS f32x4*)(lds + rowoff + st * 512 + 32 * g);
          const f32x4 d4 = *(const FA_LDS f32x4*)(lds + rowoff + st * 512 + 256 + 32 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float p = fast_exp2(fmaf(s[r], sl2, -l4[e]));
            if constexpr (decltype(masked)::value) {
              const int q = q0 + 8 * g + 4 * h + e;
              if (q >= N || (CAUSAL && key > q)) p = 0.f;
            }
            s[r] = p;
            dp[r] = p * (dp[r] + d4[e]);
          }
        }
      };
      if (need_mask) probs(std::true_type{});
      else probs(std::false_type{});
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const bf16x8 pb = pack8(s[8 * cc + 0], s[8 * cc + 1], s[8 * cc + 2], s[8 * cc + 3],
                                s[8 * cc + 4], s[8 * cc + 5], s[8 * cc + 6], s[8 * cc + 7]);
        const bf16x8 db = pack8(dp[8 * cc + 0], dp[8 * cc + 1], dp[8 * cc + 2], dp[8 * cc + 3],
                                dp[8 * cc + 4], dp[8 * cc + 5], dp[8 * cc + 6], dp[8 * cc + 7]);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const unsigned lo = troff[b][0] + so + 16 * D * 2 * cc;
          const unsigned hi = troff[b][1] + so + 16 * D * 2 * cc;
          dv[b] = mfma32(cat8(rdtr(lo + kDO), rdtr(hi + kDO)), pb, dv[b]);
          dk[b] = mfma32(cat8(rdtr(lo), rdtr(hi)), db, dk[b]);
        }
      }
      // Transposed operand reads one MFMA ahead.  (The same order for the S
      // and dP products costs registers the kernel does not have.)
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * 2, 0);
#pragma unroll
      for (int i = 0; i < 4 * DB - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    wait_global_loads();
    __syncthreads();  // the next tile is resident; this one may be overwritten
    cur = nxt;
    st ^= 1;
  };
  while (cur.g < G) tile_step();

  float* xs = reinterpret_cast<float*>(lds + kK) + 4096 * kw;
  auto put = [&](const f32x16* acc) {
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[b][4 * g + e];
        *reinterpret_cast<f32x4*>(xs + 4 * ((4 * b + g) * 64 + lane)) = v4;
      }
  };
  auto add_store = [&](const f32x16* acc, float* out, float mul) {
    if (key >= N) return;
    float* row = out + head + (size_t)key * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 o4 = *reinterpret_cast<const f32x4*>(xs + 4 * ((4 * b + g) * 64 + lane));
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (acc[b][4 * g + e] + o4[e]) * mul;
        *reinterpret_cast<f32x4*>(row + 32 * b + 8 * g + 4 * h) = v4;
      }
  };
  const size_t kvsize = (size_t)a.B * a.Hkv * N * D;
  float* dkout = a.gsplit > 1 ? a.part + slice * kvsize : a.dk;
  float* dvout = a.gsplit > 1 ? a.part + (a.gsplit + slice) * kvsize : a.dv;
  if (qh == 1) put(dk);
  __syncthreads();
  if (qh == 0) add_store(dk, dkout, a.scale);
  __syncthreads();
  if (qh == 0) put(dv);
  __syncthreads();
  if (qh == 1) add_store(dv, dvout, 1.f);
}

// ---------------------------------------------------------------------- dQ
// 4 waves, 32 queries per wave; 64-key tiles of K and V in swizzled LDS
// tiles (K read row-wise for S^T = K Q^T and column-wise for dQ^T += K^T dS^T).
#ifndef FA_DQ_BK128
#define FA_DQ_BK128 64
#endif

template <int D>
struct DqTile {
  static constexpr int BQ = 128;  // queries per workgroup (4 waves x 32)
  static constexpr int BK = D == 128 ? FA_DQ_BK128 : 64;  // keys per loop step
  static constexpr int CH = D / 8;
  static constexpr int LOADS = BK * CH / kThreads;
  static constexpr int T_ELEMS = BK * D;
  static_assert(BK * CH % kThreads == 0, "tile must split evenly");
};

template <int D, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a) {
  using T = DqTile<D>;
  constexpr bool CAUSAL = (MODE & kCausal) != 0;
  constexpr bool SPARSE = (MODE & kSparse) != 0;
  constexpr int DC = D / 16;
  constexpr int DB = D / 32;
  constexpr int NB = T::BK / 32;

  // LDS byte layout: stage s at kStage * s = [K tile | V tile].  The stage
  // is a loop-carried byte offset and the V, key-block and cc displacements
  // are immediates, so each operand read is one offset register plus an
  // immediate.
  constexpr unsigned kTile = T::T_ELEMS * 2, kStage = 2 * kTile;
  __shared__ __attribute__((aligned(16))) char lds[2 * kStage];
  const unsigned lds0 = (unsigned)(size_t)(FA_LDS void*)lds;

  const int N = a.N;
  const int nqt = (N + T::BQ - 1) / T::BQ;
  const int total = nqt * a.B * a.H;
  const int w = xcd_remap(blockIdx.x, total);
  int bh = w / nqt, qt = w % nqt;
  if constexpr (CAUSAL) {  // heaviest (last) query tiles first
    int rank;
    causal_order(w, total, nqt, bh, rank);
    qt = nqt - 1 - rank;
  }
  const int q0 = qt * T::BQ;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const size_t head = (size_t)bh * N * D;
  const int bkv = (bh / a.H) * a.Hkv + (bh % a.H) / (a.H / a.Hkv);
  const size_t kvhead = (size_t)bkv * N * D;
  const bf16* __restrict__ Q = reinterpret_cast<const bf16*>(a.q) + head;
  const bf16* __restrict__ K = reinterpret_cast<const bf16*>(a.k) + kvhead;
  const bf16* __restrict__ V = reinterpret_cast<const bf16*>(a.v) + kvhead;
  const bf16* __restrict__ dO = reinterpret_cast<const bf16*>(a.dout) + head;

  const int qrow = q0 + 32 * wave + l32;
  const int qld = qrow < N ? qrow : N - 1;
  bf16x8 qf[DC], of[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    qf[c] = *reinterpret_cast<const bf16x8*>(Q + (size_t)qld * D + 16 * c + 8 * h);
    of[c] = *reinterpret_cast<const bf16x8*>(dO + (size_t)qld * D + 16 * c + 8 * h);
  }
  const float lse2 = a.lse2[(size_t)bh * N + qld];
  const float dlt = a.delta[(size_t)bh * N + qld];
  const float sl2 = a.scale * kLog2e;

  f32x16 dq[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[b][r] = 0.f;

  const int nt = (N + T::BK - 1) / T::BK;
  const int qmax = min(q0 + T::BQ, N) - 1;
  const int tend = CAUSAL ? min(nt, qmax / T::BK + 1) : nt;
  // With a tile mask, key tiles whose entry in this workgroup's mask row is 0
  // are skipped (BQ equals the mask tile, BK divides it).
  // Tile mask: this workgroup's row, over the blocks that cover [0, tend).
  const int mb = SPARSE ? a.mask_block : 1;
  const int nmb = (N + mb - 1) / mb;
  MaskScan mscan(SPARSE ? a.mask + (size_t)(q0 / mb) * nmb : nullptr, 1,
                 SPARSE ? (tend * T::BK + mb - 1) / mb : 0);
  // The first visited key tile at or after t (>= tend when none is left).
  auto next_tile = [&](int t) {
    if constexpr (SPARSE) {
      if (t < tend) {
        const int blk = (t * T::BK) / mb;
        const int vb = mscan.next(blk);
        if (vb != blk) t = (vb * mb) / T::BK;  // first tile of that block (BK divides mb)
      }
    }
    return t;
  };

  // HBM -> LDS direct loads of one key tile of K and V (chunk q of row r at
  // chunk q ^ tile_swz(r)): lane l of a wave's i-th load fills LDS position
  // p = (i * 4 + wave) * 64 + l, i.e. row p / CH, slot p % CH.
  unsigned loff[T::LOADS];
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int p = (i * 4 + wave) * 64 + lane;
    const int row = p / T::CH;
    loff[i] = 2 * (row * D + 8 * ((p % T::CH) ^ tile_swz<D>(row)));
  }
  auto load_tile = [&](int t, unsigned st) {
    if ((t + 1) * T::BK <= N) {  // whole tile in range: scalar base + lane offsets
      const size_t t0 = (size_t)t * T::BK * D;
#pragma unroll
      for (int i = 0; i < T::LOADS; ++i) {
        const unsigned dst = lds0 + st * kStage + 16 * ((i * 4 + wave) * 64);
        dma16_sbase(K + t0, loff[i], dst);
        dma16_sbase(V + t0, loff[i], dst + kTile);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int base = (i * 4 + wave) * 64;
      const int p = base + lane;
      const int row = p / T::CH;
      const int q = (p % T::CH) ^ tile_swz<D>(row);
      const size_t src = (size_t)min(t * T::BK + row, N - 1) * D + 8 * q;
      dma16_untracked(K + src, lds0 + st * kStage + 16 * base);
      dma16_untracked(V + src, lds0 + st * kStage + kTile + 16 * base);
    }
  };

  // Loop-invariant per-lane byte offsets: row-wise reads of row l32, chunk
  // (2c + h) ^ tile_swz(l32); transpose reads of rows tr_row (+8), chunk
  // 4b + (tr_col >> 3), element tr_col & 7.  The key block (32 rows), cc
  // (16 rows), V and stage terms are added as constants or once per step.
  const int sw_row = tile_swz<D>(l32);
  unsigned roff[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) roff[c] = 2 * (l32 * D + 8 * ((2 * c + h) ^ sw_row));
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int sw_lo = tile_swz<D>(tr_row), sw_hi = tile_swz<D>(tr_row + 8);
  const int tq = tr_col >> 3, te = tr_col & 7;
  unsigned troff[DB][2];
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    troff[b][0] = 2 * (tr_row * D + 8 * (((4 * b) ^ (sw_lo & 12)) | (tq ^ (sw_lo & 3))) + te);
    troff[b][1] = 2 * ((tr_row + 8) * D + 8 * (((4 * b) ^ (sw_hi & 12)) | (tq ^ (sw_hi & 3))) + te);
  }
  auto rd8 = [&](unsigned off) { return *(const FA_LDS bf16x8*)(lds + off); };
  auto rdtr = [&](unsigned off) {
    s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(lds + off));
    return __builtin_bit_cast(bf16x4, r);
  };

  wait_global_loads();  // Q, dO operands resident before the key loop
  int t = next_tile(0);
  if (t < tend) load_tile(t, 0);
  wait_global_loads();
  __syncthreads();
  unsigned st = 0;
  // One key tile: computes with stage st while the next visited tile lands in
  // the other stage.
  auto tile_step = [&]() {
    const unsigned so = st * kStage;
    const int tn = next_tile(t + 1);
    if (tn < tend) load_tile(tn, st ^ 1);
    const int k0 = t * T::BK;
    const bool need_mask = (CAUSAL && k0 + T::BK - 1 > q0 + 32 * wave) || (k0 + T::BK > N);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const unsigned off = roff[c] + so + 2 * 32 * D * kb;
        s = mfma32(rd8(off), qf[c], s);
        dp = mfma32(rd8(off + kTile), of[c], dp);
      }
      // Issue order: each operand read one MFMA ahead of its use.
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 2 * DC - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      // s[r], dp[r]: key k0 + 32kb + 8(r/4) + 4h + r%4, query qrow.  Masked
      // and unmasked copies behind one wave-uniform branch.
      auto grads = [&](auto masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(s[r], sl2, -lse2));
          if constexpr (decltype(masked)::value) {
            const int kk = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            if (kk >= N || (CAUSAL && kk > qrow)) p = 0.f;
          }
          dp[r] = p * (dp[r] + dlt);
        }
      };
      if (need_mask) grads(std::true_type{});
      else grads(std::false_type{});
      // dQ^T += K^T dS^T (contraction over this block's keys)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const bf16x8 db = pack8(dp[8 * cc + 0], dp[8 * cc + 1], dp[8 * cc + 2], dp[8 * cc + 3],
                                dp[8 * cc + 4], dp[8 * cc + 5], dp[8 * cc + 6], dp[8 * cc + 7]);
        const unsigned rb = so + 2 * (32 * kb + 16 * cc) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const bf16x8 ka = cat8(rdtr(troff[b][0] + rb), rdtr(troff[b][1] + rb));
          dq[b] = mfma32(ka, db, dq[b]);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * DB - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    wait_global_loads();
    __syncthreads();  // the next tile is resident; this one may be overwritten
    t = tn;
    st ^= 1;
  };
  while (t < tend) tile_step();

  if (qrow < N) {
    float* dqrow = a.dq + head + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = dq[b][4 * g + e] * a.scale;
        *reinterpret_cast<f32x4*>(dqrow + 32 * b + 8 * g + 4 * h) = v4;
      }
  }
}

// dK/dV workgroup size for d=64: 4 waves (128 keys) in every mode, so that a
// tile mask's 128-key column is one workgroup and short sequences still give
// two workgroups per CU (4 % faster than 8 waves at B8 H16 N1024 causal).
// (d=128 uses the 128-key split kernel in every mode.)
template <int D, int MODE>
constexpr int kDkdvWaves = 4;

// dK, dV = sum over the query-head slices' partials, in slot order (so the
// result does not depend on scheduling).  n4: float4 elements per tensor.
__global__ __launch_bounds__(256) void bwd_dkv_reduce_kernel(BwdArgs a, long long n4) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4* p = reinterpret_cast<const f32x4*>(a.part);
  f32x4 k4 = p[i], v4 = p[(long long)a.gsplit * n4 + i];
  for (int sl = 1; sl < a.gsplit; ++sl) {
    k4 += p[(long long)sl * n4 + i];
    v4 += p[(long long)(a.gsplit + sl) * n4 + i];
  }
  reinterpret_cast<f32x4*>(a.dk)[i] = k4;
  reinterpret_cast<f32x4*>(a.dv)[i] = v4;
}

template <int D, int MODE>
hipError_t launch_mode(const BwdArgs& a, hipStream_t s) {
  using TK = DkdvTile<D, kDkdvWaves<D, MODE>>;
  constexpr int BK = D == 128 ? kSplitKeys : TK::BK;  // keys per dK/dV workgroup
  static_assert(!(MODE & kSparse) || 128 % BK == 0, "dK/dV keys must fit one mask tile");
  static_assert(!(MODE & kSparse) || DqTile<D>::BQ == 128, "dQ rows must be one mask tile");
  const long long g1 = (long long)((a.N + BK - 1) / BK) * a.B * a.Hkv * a.gsplit;
  const long long g2 = (long long)((a.N + DqTile<D>::BQ - 1) / DqTile<D>::BQ) * a.B * a.H;
  if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if constexpr (D == 128) {
    if (!(MODE & kSparse) && dkdv128_applies(a)) {   // the resident kernel (fa_bwd_dkdv128.hip)
      const hipError_t e = launch_dkdv128(a, s);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL((bwd_dkdv_split_kernel<D, MODE>), dim3((unsigned)g1), dim3(512), 0, s, a);
    }
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, kDkdvWaves<D, MODE>, MODE>), dim3((unsigned)g1),
                       dim3(TK::THREADS), 0, s, a);
  }
  if (a.gsplit > 1) {
    const long long n4 = (long long)a.B * a.Hkv * a.N * D / 4;
    const long long g3 = (n4 + 255) / 256;
    if (g3 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_dkv_reduce_kernel, dim3((unsigned)g3), dim3(256), 0, s, a, n4);
  }
  if constexpr (D == 128 && !(MODE & kSparse)) {
    if (dq128_applies(a)) {   // the hand-scheduled resident kernel (fa_bwd_dq128.hip)
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_dq128(a, s);
    }
  }
  hipLaunchKernelGGL((bwd_dq_kernel<D, MODE>), dim3((unsigned)g2), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int RPB = kThreads / (D / 8);
  const long long g0 = (rows + RPB - 1) / RPB;
  if (g0 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.mask && a.mask_block != 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)g0), dim3(kThreads), 0, s, a, rows);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.mask) return a.causal ? launch_mode<D, kSparseCausal>(a, s) : launch_mode<D, kSparse>(a, s);
  return a.causal ? launch_mode<D, kCausal>(a, s) : launch_mode<D, kDense>(a, s);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  if (a.d == 128) return launch_d<128>(a, s);
  if (a.d == 64) return launch_d<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
