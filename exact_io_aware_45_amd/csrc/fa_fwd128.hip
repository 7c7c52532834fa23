// fa_fwd128.hip -- exact attention forward for head dim 128, bf16 in / fp32
// accumulate, with a hand-scheduled main loop (gfx950).
//
// Same result as fwd_bf16_kernel (fa_fwd.hip): O = softmax(scale Q K^T) V per
// (batch, head) and the row log-sum-exp, the scores tiled through LDS and
// registers and never written to HBM ("FlashAttention." plate, opening section
// and "Never write the scores"; "Flash Attention: IO-Aware Attention
// Computation", paragraph on fused kernels and the online softmax).
//
// Work decomposition:
//   * one workgroup = 4 waves = 256 query rows of one head, one workgroup per
//     CU; each wave owns 64 rows (two 32-row blocks) for the whole key loop,
//     so each K or V^T operand read from LDS feeds two matrix instructions;
//   * K tiles are loaded two tiles ahead and V tiles one tile ahead, HBM ->
//     LDS by direct loads into double-buffered, XOR-swizzled stages;
//   * the whole key loop is a generated, hand-scheduled instruction stream
//     (fa_fwd128_loop.inc, from gen_fwd128.py) in which the products of the
//     next tile's scores and of the current tile's P V overlap the vector
//     work of the softmax; causal diagonal tiles and a ragged last tile are
//     masked there by one threshold compare per score.  The C++ below sets up
//     the Q operands, addresses and first loads, and writes O and the LSE.
#include "fa_common.hpp"
#include "fa_internal.hpp"
#include "fa_fwd128_loop.inc"

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int D = 128;
constexpr int BC = 64;          // keys per tile
constexpr int NW = 4;           // waves per workgroup
constexpr int BR = 64 * NW;     // query rows per workgroup
constexpr int TILE = BC * D;    // elements per K or V tile
constexpr int TILE_BYTES = TILE * 2;

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

template <bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd128_kernel(FwdArgs a) {
  // LDS: V stage 0, V stage 1, K stage 0, K stage 1 (16 KiB each; the
  // generated loop addresses this map directly), then the workgroup's 256
  // query rows as four 64-row tiles (read once into registers).  After the
  // loop each wave stages its normalised output rows in the first 64 KiB.
  __shared__ __attribute__((aligned(1024))) bf16 smem[8 * TILE];
  auto Vst = [&](int stage) { return smem + stage * TILE; };
  auto Kst = [&](int stage) { return smem + (2 + stage) * TILE; };
  auto Qst = [&](int i) { return smem + (4 + i) * TILE; };
  const uint32_t lds0 =
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS bf16*)smem));

  const int N = a.N;
  const int nq = (N + BR - 1) / BR;
  const int total = nq * a.B * a.H;
  const int w = xcd_remap(blockIdx.x, total);
  int bh = w / nq, qt = w % nq;
  if constexpr (CAUSAL) {
    int rank;
    causal_order(w, total, nq, bh, rank);
    qt = nq - 1 - rank;
  }
  const int q0 = qt * BR;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const size_t head = (size_t)bh * (size_t)N * D;
  const int bkv = (bh / a.H) * a.Hkv + (bh % a.H) / (a.H / a.Hkv);
  const size_t kvhead = (size_t)bkv * (size_t)N * D;
  const bf16* __restrict__ Q = reinterpret_cast<const bf16*>(a.q) + head;
  const bf16* __restrict__ K = reinterpret_cast<const bf16*>(a.k) + kvhead;
  const bf16* __restrict__ V = reinterpret_cast<const bf16*>(a.v) + kvhead;
  bf16* __restrict__ O = reinterpret_cast<bf16*>(a.o) + head;

  const int wrow0 = q0 + 64 * wave;

  // Key tiles [0, tend); from tile fm on every tile needs a mask (the
  // causal diagonal tiles and a partial last tile).
  const int nt = (N + BC - 1) / BC;
  const int qmax = min(q0 + BR, N) - 1;
  const int tend = CAUSAL ? min(nt, qmax / BC + 1) : nt;
  const bool ragged = (N % BC) != 0;
  int fm = tend;
  if (CAUSAL) fm = min(fm, q0 / BC);
  if (ragged) fm = min(fm, nt - 1);

  // Direct HBM -> LDS loads of one tile: this wave's i-th load fills LDS
  // slots p = (4i + wave) * 64 + lane (16 bytes each), row p / 16, slot
  // p % 16 holding the row's chunk slot ^ swz(row).  Rows past the end of
  // the sequence repeat the last row (their scores are masked).
  auto load_tile = [&](const bf16* src, int t, bf16* dst) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int base = (4 * i + wave) * 64;
      const int p = base + lane;
      const int row = p >> 4;
      const int q = (p & 15) ^ tile_swz<D>(row);
      lds_load16(src + (size_t)min(t * BC + row, N - 1) * D + 8 * q, dst + 8 * base);
    }
  };

  f32x16 o[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[rb][db][r] = 0.f;
  const float sl2 = a.scale * kLog2e;

  // Lane parts of the LDS operand addresses (byte addresses of stage 0).
  const int sw_row = tile_swz<D>(l32);
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int sw_lo = tile_swz<D>(tr_row), sw_hi = tile_swz<D>(tr_row + 8);
  const int tq = tr_col >> 3, te = tr_col & 7;
  auto tr_off = [&](int row, int sw, int b) {
    return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te;
  };
  u32x8 kaddr, vaddr;
#pragma unroll
  for (int c = 0; c < 8; ++c)
    kaddr[c] = lds0 + 2u * (2 * TILE + l32 * D + 8 * ((2 * c + h) ^ sw_row));
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    vaddr[2 * db] = lds0 + 2u * tr_off(tr_row, sw_lo, db);
    vaddr[2 * db + 1] = lds0 + 2u * tr_off(tr_row + 8, sw_hi, db);
  }
  // Direct-load offsets within a tile (wave w loads rows 16w .. 16w + 15,
  // four rows per load; load i carries instruction offset 1024 i, which
  // applies to both the global and the LDS address, so it is taken off
  // here), and for the partial last tile with its rows clamped to the
  // sequence (absolute: those loads move M0 instead).
  u32x4 goff, gtail;
  const int tlast = tend - 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = (4 * wave + i) * 64 + lane;
    const int row = p >> 4;
    const int col = 8 * ((p & 15) ^ tile_swz<D>(row));
    goff[i] = (uint32_t)(row * D + col) * 2u - 1024u * i;
    gtail[i] = (uint32_t)((min(tlast * BC + row, N - 1) - tlast * BC) * D + col) * 2u;
  }
  // Mask thresholds for tile fm: a score is masked when its key exceeds the
  // row's last visible key (the row itself when causal, N - 1 always).
  float thr[2];
  int thri[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = wrow0 + 32 * rb + l32;
    const int lim = CAUSAL ? min(row, N - 1) : N - 1;
    thri[rb] = lim - 4 * h - BC * fm;
    thr[rb] = __builtin_bit_cast(float, thri[rb]);
  }

  // Prologue: the workgroup's query rows, K_0, V_0 and K_1 in flight
  // together, all by coalesced direct loads into swizzled tiles.
#pragma unroll
  for (int i = 0; i < 4; ++i) load_tile(Q, q0 / BC + i, Qst(i));
  load_tile(K, 0, Kst(0));
  load_tile(V, 0, Vst(0));
  if (tend > 1) load_tile(K, 1, Kst(1));
  wait_global_loads();
  __syncthreads();

  // Q^T operands: row block rb holds query rows q0 + 64 wave + 32 rb + l32,
  // d = 16c + 8h .. +7 (rows past N - 1 repeat row N - 1; never stored).
  bf16x8 qf[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < 8; ++c)
      qf[rb][c] = lds_read8(Qst(wave) + (32 * rb + l32) * D + 8 * ((2 * c + h) ^ sw_row));

  // Scalar operands (wave-uniform values, moved to SGPRs explicitly).
  auto uni = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); };
  auto uni64 = [&](uint64_t x) {
    return ((uint64_t)uni((uint32_t)(x >> 32)) << 32) | uni((uint32_t)x);
  };
  const uint32_t m0k = uni(lds0 + 2 * TILE * 2 + wave * 4096);
  const uint32_t m0v = uni(lds0 + wave * 4096);
  const uint32_t cbits = uni(__builtin_bit_cast(uint32_t, sl2));
  uint64_t kptr = uni64(reinterpret_cast<uint64_t>(K + 2 * (size_t)TILE));
  uint64_t vptr = uni64(reinterpret_cast<uint64_t>(V + 1 * (size_t)TILE));
  // Loop control: iteration j processes tile j and loads K_{j+2} and
  // V_{j+1}; the partial last tile (loaded by iteration nt - 3 for K, nt - 2
  // for V) goes through the clamped offsets; iterations below `sfast` have
  // an unmasked next tile and two whole loads.
  const bool tail = ragged && tend == nt;
  const int kfull = tail ? nt - 1 : tend;
  uint32_t jt = 0;
  const uint32_t slast = uni((uint32_t)(tend - 1));
  const uint32_t skend = uni((uint32_t)max(0, tend - 2));
  const uint32_t sktail = uni(tail && nt >= 3 ? (uint32_t)(nt - 3) : ~0u);
  const uint32_t svtail = uni(tail && nt >= 2 ? (uint32_t)(nt - 2) : ~0u);
  const uint32_t sfm = uni((uint32_t)fm);
  const uint32_t sfast = uni((uint32_t)max(0, min(fm - 1, kfull - 2)));
  const uint32_t bperm = (uint32_t)((lane ^ 32) << 2);
  const float ninf = -INFINITY;
  float mneg0, mneg1, l0 = 0.f, l1 = 0.f;
  asm volatile(FA_FWD128_LOOP_ASM
               : "+{a[0:15]}"(o[0][0]), "+{a[16:31]}"(o[0][1]), "+{a[32:47]}"(o[0][2]),
                 "+{a[48:63]}"(o[0][3]), "+{a[64:79]}"(o[1][0]), "+{a[80:95]}"(o[1][1]),
                 "+{a[96:111]}"(o[1][2]), "+{a[112:127]}"(o[1][3]),
                 "={v212}"(mneg0), "={v213}"(mneg1), "+{v214}"(l0), "+{v215}"(l1),
                 "+{v249}"(thr[0]), "+{v250}"(thr[1]),
                 "+{s[60:61]}"(kptr), "+{s[62:63]}"(vptr), "+{s71}"(jt)
               : "{a[128:131]}"(qf[0][0]), "{a[132:135]}"(qf[0][1]),
                 "{a[136:139]}"(qf[0][2]), "{a[140:143]}"(qf[0][3]),
                 "{a[144:147]}"(qf[0][4]), "{a[148:151]}"(qf[0][5]),
                 "{a[152:155]}"(qf[0][6]), "{a[156:159]}"(qf[0][7]),
                 "{a[160:163]}"(qf[1][0]), "{a[164:167]}"(qf[1][1]),
                 "{a[168:171]}"(qf[1][2]), "{a[172:175]}"(qf[1][3]),
                 "{a[176:179]}"(qf[1][4]), "{a[180:183]}"(qf[1][5]),
                 "{a[184:187]}"(qf[1][6]), "{a[188:191]}"(qf[1][7]),
                 "{v[192:199]}"(kaddr), "{v[200:207]}"(vaddr), "{v[208:211]}"(goff),
                 "{v224}"(bperm), "{v251}"(ninf), "{v[252:255]}"(gtail),
                 "{s64}"(m0k), "{s65}"(m0v), "{s66}"(cbits), "{s67}"(slast), "{s68}"(skend),
                 "{s69}"(sktail), "{s70}"(sfm), "{s72}"(svtail), "{s82}"(sfast)
               : FA_FWD128_LOOP_CLOBBERS);
  const float m_ref[2] = {-mneg0, -mneg1};
  const float lsum[2] = {l0, l1};

  // Epilogue: O = acc / l (bf16), LSE = m + log2(l) in natural units.  The
  // loop ended with a barrier, so LDS is free: each wave writes its 64 rows
  // into its own tile with rows padded to 272 bytes (both the 8-byte writes
  // of 32 rows and the 16-byte reads of 4 whole rows then touch every bank
  // equally often), and stores whole rows, 1 KiB of consecutive rows per
  // store instruction.  Lane values are taken afresh from the exec mask (the
  // loop used every vector register).
  constexpr int OST = D + 8;
  const int el = __lane_id(), eh = el >> 5, e32 = el & 31;
  FA_LDS bf16* ost = (FA_LDS bf16*)(smem + wave * (64 * OST));
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int qrow = wrow0 + 32 * rb + e32;
    const float l_tot = lsum[rb] + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                                 (el ^ 32) << 2, __builtin_bit_cast(int, lsum[rb])));
    const float inv = __builtin_amdgcn_rcpf(l_tot);
    if (qrow < N && eh == 0) a.lse[(size_t)bh * N + qrow] = (m_ref[rb] + fast_log2(l_tot)) * kLn2;
    FA_LDS bf16* orow = ost + (32 * rb + e32) * OST + 4 * eh;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = to_bf16(o[rb][c >> 2][4 * (c & 3) + e] * inv);
      *reinterpret_cast<FA_LDS bf16x4*>(orow + 8 * c) = v4;
    }
  }
  const FA_LDS bf16* src = ost + (el >> 4) * OST + 8 * (el & 15);
  bf16* dst = O + (size_t)(wrow0 + (el >> 4)) * D + 8 * (el & 15);
  if (wrow0 + 64 <= N) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<bf16x8*>(dst + 4 * i * D) = *reinterpret_cast<const FA_LDS bf16x8*>(src + 4 * i * OST);
  } else {
    const int rows = N - wrow0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (4 * i + (el >> 4) < rows)
        *reinterpret_cast<bf16x8*>(dst + 4 * i * D) = *reinterpret_cast<const FA_LDS bf16x8*>(src + 4 * i * OST);
  }
}

}  // namespace

// Whether the hand-scheduled kernel takes this launch: head dim 128, no tile
// mask, and at least one 256-row workgroup per CU (smaller grids keep the
// 4-wave launch of fa_fwd.hip, which splits the rows finer).
bool fwd128_applies(const FwdArgs& a) {
  if (a.d != 128 || a.mask != nullptr) return false;
  const long long grid = (long long)((a.N + BR - 1) / BR) * a.B * a.H;
  return grid >= 256;
}

hipError_t launch_fwd128(const FwdArgs& a, hipStream_t s) {
  const long long grid = (long long)((a.N + BR - 1) / BR) * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.causal)
    hipLaunchKernelGGL((fwd128_kernel<true>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((fwd128_kernel<false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
