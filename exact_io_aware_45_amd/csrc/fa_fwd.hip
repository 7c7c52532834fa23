// fa_fwd.hip -- exact attention forward, bf16 in / fp32 accumulate, gfx950.
//
// What is computed: O = softmax(scale * Q K^T) V per (batch, head), with the
// row log-sum-exp saved for the backward pass.  The scores are produced and
// consumed tile by tile on chip and never written to HBM ("FlashAttention."
// plate, opening section and "Never write the scores"); the row softmax is
// the online (running max / running sum) form that folds one key tile at a
// time into the running output ("Flash Attention: IO-Aware Attention
// Computation", paragraph on fused kernels and the online softmax; the same
// plate's opening section).  Tiles that a tile mask marks irrelevant are
// skipped before any load ("Flash Attention: IO-Aware Attention Computation",
// paragraph on block-sparse attention; "FlashAttention: Fast and
// Memory-Efficient Exact Attention with IO-Awareness", Abstract).
//
// Work decomposition (MI355X-specific, not from the pages):
//   * one workgroup = 8 waves = 256 query rows of one head (4 waves = 128
//     rows for block-sparse, one mask row); each wave owns 32 query rows for
//     the whole key loop;
//   * K and V tiles of BC keys go HBM -> LDS with direct loads
//     (global_load_lds_dwordx4, no register round trip), double buffered:
//     the next tile's loads are in flight during the current tile's math,
//     and (dense d = 128) nothing waits for them before the tile's end;
//     The tiles are unpadded with an XOR swizzle of the 16-byte chunks, which
//     keeps both the K row reads and the V transpose reads conflict-free;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the
//     wave's Q held in registers), so that every lane owns one query column:
//     the row max and row sum are in-register plus one cross-half exchange;
//   * P goes from the S^T accumulators straight into the B operand of
//     O^T += V^T P^T; the V^T operand is read from the row-major V tile with
//     the LDS transpose read (ds_read_b64_tr_b16), in the key order the
//     accumulator layout dictates;
//   * exponentials in base 2 with scale*log2(e) folded into one FMA; the
//     running output is only rescaled when a row maximum grows by more than
//     2^8 (the final normalisation uses the same reference, so the result is
//     unchanged up to rounding);
//   * causal: only tiles that cross the diagonal are masked, tiles above it
//     are never visited, and the heaviest query tiles are scheduled first.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr int kAcc = 4;  // independent partial maxima and sums per lane

enum Mode { kDense = 0, kCausal = 1, kSparse = 2, kSparseCausal = 3 };

template <int D, int BC, int NW>
struct FwdTile {
  static constexpr int THREADS = 64 * NW;
  static constexpr int BR = 32 * NW;  // query rows per workgroup
  static constexpr int CH = D / 8;   // 16-byte chunks per row
  static constexpr int LOADS = BC * CH / THREADS;  // direct loads per lane per tile
  static constexpr int K_ELEMS = BC * D;  // unpadded rows, XOR-swizzled chunks
  static constexpr int V_ELEMS = BC * D;
  static constexpr int LDS_BYTES = 2 * (K_ELEMS + V_ELEMS) * 2;
  static_assert(BC * CH % THREADS == 0, "tile must split evenly over the workgroup");
};

// Waves per SIMD the register budget targets: d=128 needs about 215 VGPRs
// (two waves per SIMD); d=64 fits in 128 (four waves per SIMD).
template <int D>
constexpr int kWavesPerEU = D == 64 ? 4 : 2;

template <int D, int BC, int NW, int MODE>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(kWavesPerEU<D>, kWavesPerEU<D>)))
void fwd_bf16_kernel(FwdArgs a) {
  using T = FwdTile<D, BC, NW>;
  constexpr int kThreads = T::THREADS;
  constexpr int kBR = T::BR;
  constexpr bool kIsCausal = (MODE == kCausal || MODE == kSparseCausal);
  constexpr bool kIsSparse = (MODE == kSparse || MODE == kSparseCausal);
  constexpr int NB = BC / 32;  // 32-key blocks per tile
  constexpr int DC = D / 16;   // contraction steps of S^T = K Q^T
  constexpr int DB = D / 32;   // 32-row blocks of O^T

  // One LDS array per tensor and stage.  The compiler tracks the direct loads
  // into each array separately, so reading the current stage does not wait
  // for the loads of the next one (with a single array it waits for them
  // before the first read that might alias).
  __shared__ __attribute__((aligned(16))) bf16 k_s0[T::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 k_s1[T::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 v_s0[T::V_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 v_s1[T::V_ELEMS];

  const int N = a.N;
  const int nq = (N + kBR - 1) / kBR;
  const int total = nq * a.B * a.H;
  const int w = xcd_remap(blockIdx.x, total);
  int bh = w / nq, qt = w % nq;
  if constexpr (kIsCausal) {  // heaviest (last) query tiles first
    int rank;
    causal_order(w, total, nq, bh, rank);
    qt = nq - 1 - rank;
  }
  const int q0 = qt * kBR;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  // Query head bh = b * H + hq reads K/V head b * Hkv + hq / (H / Hkv).
  const size_t head = (size_t)bh * (size_t)N * D;
  const int bkv = (bh / a.H) * a.Hkv + (bh % a.H) / (a.H / a.Hkv);
  const size_t kvhead = (size_t)bkv * (size_t)N * D;
  const bf16* __restrict__ Q = reinterpret_cast<const bf16*>(a.q) + head;
  const bf16* __restrict__ K = reinterpret_cast<const bf16*>(a.k) + kvhead;
  const bf16* __restrict__ V = reinterpret_cast<const bf16*>(a.v) + kvhead;
  bf16* __restrict__ O = reinterpret_cast<bf16*>(a.o) + head;

  // Q^T operand of this wave: query row qrow, d = 16c + 8h .. +7.
  const int qrow = q0 + 32 * wave + l32;
  const int qld = qrow < N ? qrow : N - 1;
  bf16x8 qf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c)
    qf[c] = *reinterpret_cast<const bf16x8*>(Q + (size_t)qld * D + 16 * c + 8 * h);

  // Key tiles this workgroup visits: [0, tend), minus masked tiles.
  const int nt = (N + BC - 1) / BC;
  const int qmax = min(q0 + kBR, N) - 1;
  const int tend = kIsCausal ? min(nt, qmax / BC + 1) : nt;
  // Tile mask: this workgroup's row, over the blocks that cover [0, tend).
  const int mb = kIsSparse ? a.mask_block : 1;
  const int nmb = (N + mb - 1) / mb;
  MaskScan mscan(kIsSparse ? a.mask + (size_t)(q0 / mb) * nmb : nullptr, 1,
                 kIsSparse ? (tend * BC + mb - 1) / mb : 0);
  // The first visited tile at or after t (>= tend when none is left).
  auto next_tile = [&](int t) {
    if constexpr (kIsSparse) {
      if (t < tend) {
        const int blk = (t * BC) / mb;
        const int vb = mscan.next(blk);
        if (vb != blk) t = (vb * mb) / BC;  // first tile of that block (BC divides mb)
      }
    }
    return t;
  };

  // HBM -> LDS without a register round trip (global_load_lds_dwordx4):
  // lane l of a wave's i-th load fills the 16 bytes at LDS position
  // p = (i * NW + wave) * 64 + l of the tile, i.e. row p / CH, slot p % CH,
  // which holds the row's chunk slot ^ swz(row).
  auto load_tile = [&](int t, bf16* Ks, bf16* Vs) {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int base = (i * NW + wave) * 64;
      const int p = base + lane;
      const int row = p / T::CH;
      const int q = (p % T::CH) ^ tile_swz<D>(row);
      const size_t src = (size_t)min(t * BC + row, N - 1) * D + 8 * q;
      lds_load16(K + src, Ks + 8 * base);
      lds_load16(V + src, Vs + 8 * base);
    }
  };
  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m_ref = -INFINITY;  // reference maximum (log2 units) of the exponentials
  // Running sum over this lane's keys, as kAcc independent partial sums
  // (one chain of 32 dependent adds per tile would stall every tile; the
  // row maximum is likewise taken over kAcc partial maxima).
  float l_part[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) l_part[i] = 0.f;
  const float sl2 = a.scale * kLog2e;

  wait_global_loads();  // Q operands resident before the key loop
  int t = next_tile(0);
  if (t < tend) load_tile(t, k_s0, v_s0);
  __syncthreads();

  // Lane-invariant parts of the swizzled LDS addresses.  K operand rows:
  // row 32kb + l32, chunk 2c + h.  V^T transpose reads: rows
  // 32kb + 16cc + tr_row (+8), chunk 4b + (tr_col >> 3), element tr_col & 7.
  const int sw_row = tile_swz<D>(l32);
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int sw_lo = tile_swz<D>(tr_row), sw_hi = tile_swz<D>(tr_row + 8);
  const int tq = tr_col >> 3, te = tr_col & 7;
  auto tr_off = [&](int row, int sw, int b) {
    return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te;
  };

  // One key tile: computes with (Ks, Vs) while the next visited tile lands
  // in (Kn, Vn).
  auto tile_step = [&](const bf16* Ks, const bf16* Vs, bf16* Kn, bf16* Vn) {
    const int tn = next_tile(t + 1);
    if (tn < tend) load_tile(tn, Kn, Vn);

    const int k0 = t * BC;
    // A causal tile entirely above this wave's rows contributes nothing.
    if (!kIsCausal || k0 <= q0 + 32 * wave + 31) {

    // S^T = K Q^T for this tile: s[kb] holds keys k0 + 32kb + 8(r/4) + 4h + r%4
    // of query qrow.
    f32x16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    // The NB accumulation chains alternate; for dense d = 128 every operand
    // read is issued four matrix instructions ahead of its use.
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const bf16x8 ka = lds_read8(Ks + (32 * kb + l32) * D + 8 * ((2 * c + h) ^ sw_row));
        s[kb] = mfma32(ka, qf[c], s[kb]);
      }
    if constexpr (D == 128 && !kIsSparse) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < NB * DC - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }

    // Masking: causal tiles crossing this wave's diagonal, and the ragged tail.
    const bool diag = kIsCausal && (k0 + BC - 1 > q0 + 32 * wave);
    if (diag || k0 + BC > N) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= N || (kIsCausal && key > qrow)) s[kb][r] = -INFINITY;
        }
    }

    // Online softmax (base 2).
    float mpart[kAcc];
#pragma unroll
    for (int i = 0; i < kAcc; ++i) mpart[i] = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mpart[r % kAcc] = fmaxf(mpart[r % kAcc], s[kb][r]);
#pragma unroll
    for (int st = kAcc / 2; st > 0; st /= 2)
#pragma unroll
      for (int i = 0; i < st; ++i) mpart[i] = fmaxf(mpart[i], mpart[i + st]);
    float mx = mpart[0];
    // The two halves of the wave hold different keys of one query row, so the
    // reference must be their common maximum; but it only has to move when a
    // maximum exceeds it by more than the threshold.  The exchange between
    // the halves is done only when some lane of the wave sees that (rare once
    // the first tiles have set the reference).
    if (__builtin_amdgcn_ballot_w64(mx * sl2 > m_ref + kRescaleThreshold) != 0) {
      mx = half_pair_max(mx);
      const float m_new = fmaxf(m_ref, mx * sl2);
      if (m_new > m_ref + kRescaleThreshold) {
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
        const float p = fast_exp2(fmaf(s[kb][r], sl2, -mu));
        s[kb][r] = p;
        l_part[r % kAcc] += p;
      }

    // O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const bf16x8 pb = pack8(s[kb][8 * cc + 0], s[kb][8 * cc + 1], s[kb][8 * cc + 2],
                                s[kb][8 * cc + 3], s[kb][8 * cc + 4], s[kb][8 * cc + 5],
                                s[kb][8 * cc + 6], s[kb][8 * cc + 7]);
        const int r_lo = 32 * kb + 16 * cc + tr_row;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const bf16x4 lo = lds_read_tr4(Vs + tr_off(r_lo, sw_lo, b));
          const bf16x4 hi = lds_read_tr4(Vs + tr_off(r_lo + 8, sw_hi, b));
          oacc[b] = mfma32(cat8(lo, hi), pb, oacc[b]);
        }
      }
    }

    __syncthreads();  // also drains this wave's direct loads of tile tn
    t = tn;
  };
  if constexpr (D == 128 && !kIsSparse) {
    // Buffers named at compile time (two steps per trip), so that the reads
    // of one stage are known not to alias the loads into the other.
    while (t < tend) {
      tile_step(k_s0, v_s0, k_s1, v_s1);
      if (t >= tend) break;
      tile_step(k_s1, v_s1, k_s0, v_s0);
    }
  } else {
    // d = 64 keeps four waves per SIMD in 128 registers, and the tile-mask
    // scan adds registers too: the two-step loop does not fit there, so the
    // stage is chosen at run time.
    int stage = 0;
    while (t < tend) {
      tile_step(stage ? k_s1 : k_s0, stage ? v_s1 : v_s0, stage ? k_s0 : k_s1,
                stage ? v_s0 : v_s1);
      stage ^= 1;
    }
  }

  // Epilogue: O = acc / l (bf16), LSE = ln(sum) in natural units.
#pragma unroll
  for (int st = kAcc / 2; st > 0; st /= 2)
#pragma unroll
    for (int i = 0; i < st; ++i) l_part[i] += l_part[i + st];
  const float l_tot = half_pair_sum(l_part[0]);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qrow < N) {
    if (h == 0)
      a.lse[(size_t)bh * N + qrow] =
          l_tot > 0.f ? (m_ref + fast_log2(l_tot)) * kLn2 : -INFINITY;
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

template <int D, int BC, int NW, int MODE>
hipError_t launch_one(const FwdArgs& a, hipStream_t s) {
  using T = FwdTile<D, BC, NW>;
  const int nq = (a.N + T::BR - 1) / T::BR;
  const long long grid = (long long)nq * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, NW, MODE>), dim3((unsigned)grid), dim3(T::THREADS),
                     0, s, a);
  return hipGetLastError();
}

// Dense and causal: 8 waves (32 query rows each) share every staged K/V tile,
// unless the 8-wave grid would not give every CU two workgroups (or, causal,
// just two): then 4-wave workgroups, which double the grid and balance short
// causal rows better (B2 H16 N1024 d128: -23 %; B8 H16 N1024 d64 causal:
// -6 %; 5 % slower than 8 waves at B1 H32 N8192 d128).  Block-sparse: 4
// waves, so that one workgroup covers exactly one 128-row mask row.
constexpr long long kSmallGrid = 2 * 256;  // two 8-wave workgroups per CU

template <int D, int BC>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  if (a.mask) {
    if (a.causal) return launch_one<D, BC, 4, kSparseCausal>(a, s);
    return launch_one<D, BC, 4, kSparse>(a, s);
  }
  const long long grid8 = (long long)((a.N + 255) / 256) * a.B * a.H;
  const bool small = grid8 < kSmallGrid || (a.causal && grid8 == kSmallGrid);
  if (a.causal) {
    return small ? launch_one<D, BC, 4, kCausal>(a, s) : launch_one<D, BC, 8, kCausal>(a, s);
  }
  return small ? launch_one<D, BC, 4, kDense>(a, s) : launch_one<D, BC, 8, kDense>(a, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  if (fwd128_applies(a)) return launch_fwd128(a, s);
  if (fwd64_applies(a)) return launch_fwd64(a, s);
  if (a.d == 128) return launch_d<128, 64>(a, s);
  if (a.d == 64) return launch_d<64, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
