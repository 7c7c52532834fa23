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
//   * one workgroup = 4 waves = 128 query rows of one head; each wave owns 32
//     query rows for the whole key loop;
//   * K and V tiles of BC keys are staged HBM -> registers -> LDS, double
//     buffered, the next tile's global loads in flight during the current
//     tile's math;
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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;  // query rows per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

enum Mode { kDense = 0, kCausal = 1, kSparse = 2, kSparseCausal = 3 };

template <int D, int BC>
struct FwdTile {
  static constexpr int KP = D + 8;   // K row pitch in LDS (elements)
  static constexpr int VP = D + 32;  // V row pitch in LDS (elements)
  static constexpr int CH = D / 8;   // 16-byte chunks per row
  static constexpr int LOADS = BC * CH / kThreads;
  static constexpr int K_ELEMS = BC * KP;
  static constexpr int V_ELEMS = BC * VP;
  static constexpr int LDS_BYTES = 2 * (K_ELEMS + V_ELEMS) * 2;
  static_assert(BC * CH % kThreads == 0, "tile must split evenly over the workgroup");
};

template <int D, int BC, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(FwdArgs a) {
  using T = FwdTile<D, BC>;
  constexpr bool kIsCausal = (MODE == kCausal || MODE == kSparseCausal);
  constexpr bool kIsSparse = (MODE == kSparse || MODE == kSparseCausal);
  constexpr int NB = BC / 32;  // 32-key blocks per tile
  constexpr int DC = D / 16;   // contraction steps of S^T = K Q^T
  constexpr int DB = D / 32;   // 32-row blocks of O^T

  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (T::K_ELEMS + T::V_ELEMS)];

  const int N = a.N;
  const int nq = (N + kBR - 1) / kBR;
  const int total = nq * a.B * a.H;
  const int w = xcd_remap(blockIdx.x, total);
  const int bh = w / nq;
  const int qt = kIsCausal ? (nq - 1 - w % nq) : (w % nq);
  const int q0 = qt * kBR;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const size_t head = (size_t)bh * (size_t)N * D;
  const bf16* __restrict__ Q = reinterpret_cast<const bf16*>(a.q) + head;
  const bf16* __restrict__ K = reinterpret_cast<const bf16*>(a.k) + head;
  const bf16* __restrict__ V = reinterpret_cast<const bf16*>(a.v) + head;
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
  const uint8_t* mrow = nullptr;
  int mb = 1;
  if constexpr (kIsSparse) {
    mb = a.mask_block;
    const int nmb = (N + mb - 1) / mb;
    mrow = a.mask + (size_t)(q0 / mb) * nmb;
  }
  auto next_tile = [&](int t) {
    if constexpr (kIsSparse) {
      while (t < tend && !mrow[(t * BC) / mb]) ++t;
    }
    return t;
  };

  u32x4 kreg[T::LOADS], vreg[T::LOADS];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int idx = threadIdx.x + kThreads * i;
      const int row = idx / T::CH, ch = idx % T::CH;
      const int key = min(t * BC + row, N - 1);
      kreg[i] = *reinterpret_cast<const u32x4*>(K + (size_t)key * D + 8 * ch);
      vreg[i] = *reinterpret_cast<const u32x4*>(V + (size_t)key * D + 8 * ch);
    }
  };
  auto store_tile = [&](int stage) {
    bf16* Ks = smem + stage * T::K_ELEMS;
    bf16* Vs = smem + 2 * T::K_ELEMS + stage * T::V_ELEMS;
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
      const int idx = threadIdx.x + kThreads * i;
      const int row = idx / T::CH, ch = idx % T::CH;
      lds_write16(Ks + row * T::KP + 8 * ch, kreg[i]);
      lds_write16(Vs + row * T::VP + 8 * ch, vreg[i]);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m_ref = -INFINITY;  // reference maximum (log2 units) of the exponentials
  float l_run = 0.f;        // running sum over this lane's keys
  const float sl2 = a.scale * kLog2e;

  wait_global_loads();  // Q operands resident before the key loop
  int t = next_tile(0);
  if (t < tend) {
    load_tile(t);
    store_tile(0);
  }
  __syncthreads();
  int stage = 0;

  // Lane-invariant parts of the transpose-read address of V^T.
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  while (t < tend) {
    const int tn = next_tile(t + 1);
    if (tn < tend) load_tile(tn);

    const bf16* Ks = smem + stage * T::K_ELEMS;
    const bf16* Vs = smem + 2 * T::K_ELEMS + stage * T::V_ELEMS;
    const int k0 = t * BC;

    // S^T = K Q^T for this tile: s[kb] holds keys k0 + 32kb + 8(r/4) + 4h + r%4
    // of query qrow.
    f32x16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 ka = lds_read8(Ks + (32 * kb + l32) * T::KP + 16 * c + 8 * h);
        s[kb] = mfma32(ka, qf[c], s[kb]);
      }
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
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = half_pair_max(mx);
    const float m_new = fmaxf(m_ref, mx * sl2);
    if (m_new > m_ref + kRescaleThreshold) {
      const float alpha = fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
    }
    const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[kb][r], sl2, -mu));
        s[kb][r] = p;
        l_run += p;
      }

    // O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const bf16x8 pb = pack8(s[kb][8 * cc + 0], s[kb][8 * cc + 1], s[kb][8 * cc + 2],
                                s[kb][8 * cc + 3], s[kb][8 * cc + 4], s[kb][8 * cc + 5],
                                s[kb][8 * cc + 6], s[kb][8 * cc + 7]);
        const bf16* vrow = Vs + (32 * kb + 16 * cc + tr_row) * T::VP + tr_col;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const bf16x4 lo = lds_read_tr4(vrow + 32 * b);
          const bf16x4 hi = lds_read_tr4(vrow + 8 * T::VP + 32 * b);
          oacc[b] = mfma32(cat8(lo, hi), pb, oacc[b]);
        }
      }

    if (tn < tend) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    t = tn;
  }

  // Epilogue: O = acc / l (bf16), LSE = ln(sum) in natural units.
  const float l_tot = half_pair_sum(l_run);
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

template <int D, int BC, int MODE>
hipError_t launch_one(const FwdArgs& a, hipStream_t s) {
  const int nq = (a.N + kBR - 1) / kBR;
  const long long grid = (long long)nq * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, MODE>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

template <int D, int BC>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  if (a.mask) {
    if (a.causal) return launch_one<D, BC, kSparseCausal>(a, s);
    return launch_one<D, BC, kSparse>(a, s);
  }
  if (a.causal) return launch_one<D, BC, kCausal>(a, s);
  return launch_one<D, BC, kDense>(a, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  if (a.d == 128) return launch_d<128, 64>(a, s);
  if (a.d == 64) return launch_d<64, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
