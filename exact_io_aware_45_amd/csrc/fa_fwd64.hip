// fa_fwd64.hip -- exact attention forward for head dim 64, bf16 in / fp32
// accumulate, with a hand-scheduled main loop (gfx950).
//
// Same result as fwd_bf16_kernel (fa_fwd.hip): O = softmax(scale Q K^T) V per
// (batch, head) and the row log-sum-exp, the scores tiled through LDS and
// registers and never written to HBM ("FlashAttention." plate, opening section
// and "Never write the scores"; "Flash Attention: IO-Aware Attention
// Computation", paragraph on fused kernels and the online softmax).
//
// The structure is the d = 128 kernel's (fa_fwd128.hip): resident
// workgroups taking query tiles in a serpentine over their XCD's share; 64
// query rows per wave for the whole key loop; K two tiles and V one tile
// ahead by direct loads; the key loop one generated statement
// (fa_fwd64_loop.inc, from gen_fwd128.py).  At d = 64 a 64-key tile is 16
// score and 16 P V products per wave against the same softmax as at
// d = 128, so the loop is bound by its vector work, which the generator
// spreads evenly over the products.
//
// Two shapes of workgroup: 4 waves over 256 rows, one workgroup per CU, or
// 2 waves over 128 rows, two per CU (56 KiB of LDS each; fa_fwd64w2_loop.inc,
// whose waves issue twice the direct loads).  Both keep one wave per SIMD.
// The 2-wave one serves causal launches of short sequences: its diagonal
// band costs two lockstep steps per item instead of four, for a few percent
// more K/V staging traffic per key.
#include "fa_common.hpp"
#include "fa_internal.hpp"
#include "fa_fwd64_loop.inc"
#include "fa_fwd64w2_loop.inc"
#include "fa_resident.hpp"

#include <algorithm>

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int D = 64;
constexpr int BC = 64;          // keys per tile
constexpr int TILE = BC * D;    // elements per K or V tile
constexpr int TILE_BYTES = TILE * 2;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Direct loads of 64-row tile t (d = 64, bf16) of `src` into the 8 KiB LDS
// area at byte `lds` by an NW-wave workgroup: wave w loads rows
// (64 / NW) w .. + 64 / NW - 1, eight rows (1 KiB) per load, chunk q of row r
// to slot q ^ swz(r); rows past the sequence repeat its last row.
template <int NW>
__device__ __forceinline__ void dma_tile64(const Shape& sh, int wave, const bf16* src, int t,
                                           uint32_t lds) {
  constexpr int RW = 64 / NW, NL = RW / 8;
  const int lane = fresh_lane();
  const int rows = min(64, sh.N - t * 64);
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int row = RW * wave + 8 * i + (lane >> 3);
    const int col = 8 * ((lane & 7) ^ tile_swz<D>(row));
    dma16_untracked(src + (size_t)t * TILE, (uint32_t)(min(row, rows - 1) * D + col) * 2u,
                    lds + 1024u * NL * wave + 1024u * i);
  }
}

// Direct loads of one wave's 64 query rows r0 .. r0 + 63 of a head into the
// 8 KiB LDS area at byte `lds`, chunk-swizzled like a tile.
__device__ __forceinline__ void dma_rows64(const Shape& sh, const bf16* head, int r0, uint32_t lds) {
  const int lane = fresh_lane();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 8 * i + (lane >> 3);
    const int col = 8 * ((lane & 7) ^ tile_swz<D>(row));
    dma16_untracked(head, (uint32_t)(min(r0 + row, sh.N - 1) * D + col) * 2u, lds + 1024u * i);
  }
}

// The generated statement with its operands: the loop of `LOOP`, whose
// direct-load offsets occupy v[208:GOFF_END] and v[252:GTAIL_END].
#define FWD64_LOOP_STMT(LOOP, GOFF_END, GTAIL_END) \
    asm volatile(LOOP##_ASM \
                 : "={a[0:15]}"(o[0][0]), "={a[16:31]}"(o[0][1]), "={a[32:47]}"(o[1][0]), \
                   "={a[48:63]}"(o[1][1]), \
                   "={v212}"(mneg0), "={v213}"(mneg1), "+{v214}"(l0), "+{v215}"(l1), \
                   "+{v249}"(thr[0]), "+{v250}"(thr[1]), \
                   "+{s[60:61]}"(kptr), "+{s[62:63]}"(vptr), "+{s71}"(jt) \
                 : "{a[128:131]}"(qf[0][0]), "{a[132:135]}"(qf[0][1]), \
                   "{a[136:139]}"(qf[0][2]), "{a[140:143]}"(qf[0][3]), \
                   "{a[144:147]}"(qf[1][0]), "{a[148:151]}"(qf[1][1]), \
                   "{a[152:155]}"(qf[1][2]), "{a[156:159]}"(qf[1][3]), \
                   "{v[192:195]}"(kaddr), "{v[200:203]}"(vaddr), "{v[208:" GOFF_END "]}"(goff), \
                   "{v224}"(bperm), "{v251}"(ninf), "{v[252:" GTAIL_END "]}"(gtail), \
                   "{s64}"(m0k), "{s65}"(m0v), "{s66}"(cbits), "{s67}"(slast), "{s68}"(skend), \
                   "{s69}"(sktail), "{s70}"(sfm), "{s72}"(svtail), "{s82}"(sfast), \
                   "{s83}"(swdiag) \
                 : LOOP##_CLOBBERS)

template <bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd64_kernel(FwdArgs a) {
  static_assert(NW == 4 || NW == 2, "4 or 2 waves per workgroup");
  constexpr int BR = 64 * NW;             // query rows per workgroup
  constexpr int NL = 8 / NW;              // direct loads per wave and K or V tile
  typedef __attribute__((ext_vector_type(NL))) uint32_t u32xl;
  // LDS, bytes: [0, 32K) V stage 0, V stage 1, K stage 0, K stage 1 (the
  // generated loop addresses these directly); then each wave's 64 query
  // rows (8 KiB), then each wave's output staging (32 rows, 4 KiB).
  __shared__ __attribute__((aligned(1024))) bf16 smem[(4 + NW) * TILE + NW * 2048];
  constexpr uint32_t KST0 = 2 * TILE_BYTES, QST0 = 4 * TILE_BYTES,
                     OST0 = (4 + NW) * TILE_BYTES;
  const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  auto shape = [&]() { return fresh_shape<BR, BC>(a.N, a.B, a.H, a.Hkv); };
  auto lds_base = [&]() {
    return fresh(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS bf16*)smem)));
  };
  auto item_of = [&](const Shape& sh, int r, Item& it) {
    return resident_item<CAUSAL, BR>(sh, r, it);
  };
  auto kv_off = [&](const Shape& sh, const Item& it) { return kv_head_offset(sh, it.bh, D); };
  auto tend_of = [&](const Shape& sh, const Item& it) {
    return CAUSAL ? min(sh.nt, (min(it.q0 + BR, sh.N) - 1) / BC + 1) : sh.nt;
  };
  auto dma_tile = [&](const Shape& sh, const bf16* src, int t, uint32_t stage) {
    dma_tile64<NW>(sh, fresh(wave0), src, t, lds_base() + stage);
  };
  auto dma_q = [&](const Shape& sh, const Item& it) {
    const int wave = fresh(wave0);
    dma_rows64(sh, fresh(reinterpret_cast<const bf16*>(a.q)) + (size_t)it.bh * (size_t)sh.N * D,
               it.q0 + 64 * wave, lds_base() + QST0 + (uint32_t)TILE_BYTES * wave);
  };
  auto dma_first_tiles = [&](const Shape& sh, const Item& it) {
    const size_t kv = kv_off(sh, it);
    const bf16* K = fresh(reinterpret_cast<const bf16*>(a.k)) + kv;
    const bf16* V = fresh(reinterpret_cast<const bf16*>(a.v)) + kv;
    dma_tile(sh, K, 0, KST0);
    dma_tile(sh, V, 0, 0);
    if (tend_of(sh, it) > 1) dma_tile(sh, K, 1, KST0 + TILE_BYTES);
  };

  Item cur;
  {
    const Shape sh = shape();
    if (!item_of(sh, 0, cur)) return;
    dma_q(sh, cur);
    dma_first_tiles(sh, cur);
  }
  wait_vmem();   // each wave reads only its own query rows before the next barrier

  for (int r = 0;; ++r) {
    const Shape sh = shape();
    const int wave = fresh(wave0);
    const int N = sh.N, nt = sh.nt;
    const uint32_t lds0 = lds_base();
    const int lane = fresh_lane();
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int q0 = cur.q0;
    const int wrow0 = q0 + 64 * wave;
    const size_t kv = kv_off(sh, cur);
    const bf16* __restrict__ K = fresh(reinterpret_cast<const bf16*>(a.k)) + kv;
    const bf16* __restrict__ V = fresh(reinterpret_cast<const bf16*>(a.v)) + kv;

    // Key tiles [0, tend); from tile fm on every tile needs a mask.
    const int tend = tend_of(sh, cur);
    int fm = tend;
    if (CAUSAL) fm = min(fm, q0 / BC);
    if (sh.ragged) fm = min(fm, nt - 1);

    // Q^T operands: row block rb holds query rows q0 + 64 wave + 32 rb + l32,
    // d = 16c + 8h .. +7.
    const int sw_row = tile_swz<D>(l32);
    bf16x8 qf[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        qf[rb][c] = lds_read8(smem + QST0 / 2 + wave * TILE + (32 * rb + l32) * D +
                              8 * ((2 * c + h) ^ sw_row));
    Item nxt;
    const bool more = item_of(sh, r + 1, nxt);

    // Lane parts of the LDS operand addresses (byte addresses of stage 0).
    const int tr_row = 4 * h + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int sw_lo = tile_swz<D>(tr_row), sw_hi = tile_swz<D>(tr_row + 8);
    const int tq = tr_col >> 3, te = tr_col & 7;
    auto tr_off = [&](int row, int sw, int b) {
      return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te;
    };
    u32x4 kaddr, vaddr;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kaddr[c] = lds0 + 2u * (2 * TILE + l32 * D + 8 * ((2 * c + h) ^ sw_row));
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      vaddr[2 * db] = lds0 + 2u * tr_off(tr_row, sw_lo, db);
      vaddr[2 * db + 1] = lds0 + 2u * tr_off(tr_row + 8, sw_hi, db);
    }
    // Direct-load offsets within a tile (as dma_tile64: eight rows per load;
    // load i carries instruction offset 1024 i, which applies to both the
    // global and the LDS address, so it is taken off here), and for the
    // partial last tile with its rows clamped.
    u32xl goff, gtail;
    const int tlast = tend - 1;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int row = 8 * NL * wave + 8 * i + (lane >> 3);
      const int col = 8 * ((lane & 7) ^ tile_swz<D>(row));
      goff[i] = (uint32_t)(row * D + col) * 2u - 1024u * i;
      gtail[i] = (uint32_t)((min(tlast * BC + row, N - 1) - tlast * BC) * D + col) * 2u;
    }
    // Mask thresholds for tile fm: a score is masked when its key exceeds the
    // row's last visible key (the row itself when causal, N - 1 always).
    float thr[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = wrow0 + 32 * rb + l32;
      const int lim = CAUSAL ? min(row, N - 1) : N - 1;
      thr[rb] = __builtin_bit_cast(float, lim - 4 * h - BC * fm);
    }

    auto uni = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); };
    auto uni64 = [&](uint64_t x) {
      return ((uint64_t)uni((uint32_t)(x >> 32)) << 32) | uni((uint32_t)x);
    };
    const uint32_t m0k = uni(lds0 + KST0 + wave * 1024 * NL);
    const uint32_t m0v = uni(lds0 + wave * 1024 * NL);
    const uint32_t cbits = uniform_bits(fresh(a.scale) * kLog2e);   // scale * log2(e)
    uint64_t kptr = uni64(reinterpret_cast<uint64_t>(K + 2 * (size_t)TILE));
    uint64_t vptr = uni64(reinterpret_cast<uint64_t>(V + 1 * (size_t)TILE));
    // Loop control, as in the d = 128 kernel: iteration j processes tile j
    // and loads K_{j+2} and V_{j+1}.
    const bool tail = sh.ragged && tend == nt;
    const int kfull = tail ? nt - 1 : tend;
    uint32_t jt = 0;
    const uint32_t slast = uni((uint32_t)(tend - 1));
    const uint32_t skend = uni((uint32_t)max(0, tend - 2));
    const uint32_t sktail = uni(tail && nt >= 3 ? (uint32_t)(nt - 3) : ~0u);
    const uint32_t svtail = uni(tail && nt >= 2 ? (uint32_t)(nt - 2) : ~0u);
    const uint32_t sfm = uni((uint32_t)fm);
    const uint32_t sfast = uni((uint32_t)max(0, min(fm - 1, kfull - 2)));
    // This wave's last tile holding a key it sees (causal: the tile of its
    // last row); past it the loop only loads and meets the barriers.
    const uint32_t swdiag =
        uni((uint32_t)(CAUSAL ? min(tend - 1, min(wrow0 + 63, N - 1) / BC) : tend - 1));
    const uint32_t bperm = (uint32_t)((lane ^ 32) << 2);
    const float ninf = -INFINITY;
    // This item's first K and V tiles and the previous output's stores
    // complete here; then the next item's query rows replace this one's,
    // which are in registers by now.
    wait_vmem();
    __syncthreads();
    if (more) {
      wait_lds();
      dma_q(sh, nxt);
    }
    f32x16 o[2][2];
    float mneg0, mneg1, l0 = 0.f, l1 = 0.f;
    if constexpr (NW == 4)
      FWD64_LOOP_STMT(FA_FWD64_LOOP, "209", "253");
    else
      FWD64_LOOP_STMT(FA_FWD64W2_LOOP, "211", "255");
    const float m_ref[2] = {-mneg0, -mneg1};
    const float lsum[2] = {l0, l1};

    // The loop ended with a barrier: the stages are free for the next item's
    // first tiles, which land while this item's output is written.
    const Shape sh2 = shape();
    if (more) dma_first_tiles(sh2, nxt);

    // Epilogue: O = acc / l (bf16), LSE = m + log2(l) in natural units.  Each
    // wave passes its rows through its own 4 KiB LDS area, 32 rows at a time
    // with chunk-swizzled rows, and stores 1 KiB of consecutive rows (eight)
    // per instruction.
    const int N2 = sh2.N;
    const int wave2 = fresh(wave0);
    const int el = fresh_lane(), eh = el >> 5, e32 = el & 31;
    FA_LDS char* ost = (FA_LDS char*)smem + OST0 + 4096 * wave2;
    const int wsw = tile_swz<D>(e32);
    const int rsub = el >> 3, rch = el & 7;
    const size_t ohead = (size_t)cur.bh * (size_t)N2;
    const int wrow2 = cur.q0 + 64 * wave2;
    typedef __attribute__((address_space(1))) bf16x8 gbf16x8;
    typedef __attribute__((address_space(1))) float gfloat;
    gbf16x8* orow0 = (gbf16x8*)(fresh(reinterpret_cast<bf16*>(a.o)) + (ohead + wrow2 + rsub) * D +
                                8 * rch);
    gfloat* lse = (gfloat*)(fresh(a.lse) + ohead);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int qrow = wrow2 + 32 * rb + e32;
      const float l_tot = lsum[rb] + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                                   (el ^ 32) << 2, __builtin_bit_cast(int, lsum[rb])));
      const float inv = __builtin_amdgcn_rcpf(l_tot);
      if (qrow < N2 && eh == 0) lse[qrow] = (m_ref[rb] + fast_log2(l_tot)) * kLn2;
      // element 4(c % 4) + e of o[rb][c / 4] is d = 8c + 4h + e: chunk c, bytes 8h ..
      FA_LDS char* wrow = ost + 128 * e32 + 8 * eh;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = to_bf16(o[rb][c >> 2][4 * (c & 3) + e] * inv);
        *reinterpret_cast<FA_LDS bf16x4*>(wrow + 16 * (c ^ wsw)) = v4;
      }
      bf16x8 v8[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * i + rsub;
        v8[i] = *reinterpret_cast<const FA_LDS bf16x8*>(ost + 128 * row + 16 * (rch ^ tile_swz<D>(row)));
      }
      // 1 KiB row groups: orow0 steps by 8 rows (64 of its elements) per i
      const int rows = N2 - (wrow2 + 32 * rb);
      if (rows >= 32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) orow0[(32 * rb + 8 * i) * (D / 8)] = v8[i];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (8 * i + rsub < rows) orow0[(32 * rb + 8 * i) * (D / 8)] = v8[i];
      }
    }
    if (!more) break;
    cur = nxt;
  }
}

}  // namespace

// Whether the hand-scheduled kernel takes this launch: head dim 64, no tile
// mask, and at least one 256-row query tile per CU.
bool fwd64_applies(const FwdArgs& a) {
  if (a.d != 64 || a.mask != nullptr) return false;
  const long long tiles = (long long)((a.N + 255) / 256) * a.B * a.H;
  return tiles >= 256;
}

namespace {

// Causal sequences up to this length take the 2-wave workgroups: their
// diagonal band is a large share of the steps (B8 H16 N1024: -7 % kernel
// time, N4096: -3 %; N16384: +1 %).
constexpr int kTwoWaveCausalMaxN = 4096;

template <bool CAUSAL, int NW>
hipError_t launch(const FwdArgs& a, hipStream_t s, int per_cu) {
  const long long items = (long long)((a.N + 64 * NW - 1) / (64 * NW)) * a.B * a.H;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const long long grid = std::min<long long>(items, (long long)per_cu * resident_cu_count());
  hipLaunchKernelGGL((fwd64_kernel<CAUSAL, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd64(const FwdArgs& a, hipStream_t s) {
  if (!a.causal) return launch<false, 4>(a, s, 1);
  if (a.N <= kTwoWaveCausalMaxN) return launch<true, 2>(a, s, 2);
  return launch<true, 4>(a, s, 1);
}

}  // namespace fa
