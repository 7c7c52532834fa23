// fa_bwd_dkdv128.hip -- the dK/dV pass of the backward for head dim 128, bf16
// inputs, fp32 dK and dV, with a hand-scheduled query loop (gfx950).
//
// Same result as bwd_dkdv_split_kernel (fa_bwd.hip): for every key the scores and their gradient are
// recomputed tile by tile from the saved log-sum-exp, never stored
// ("FlashAttention." plate, "Never write the scores"), and
//   dV = sum_i P_i^T dO_i,  dK = scale * sum_i dS_i^T Q_i,
//   dS = P (dP - D),  P = exp2(S c - L),
// with S = Q K^T, dP = dO V^T, L = LSE log2(e), c = scale log2(e) and
// D = rowsum(dO o O), which the delta pass stores negated (-D starts each
// dP product chain, so the products leave dP - D).
//
// Work decomposition:
//   * one workgroup = 4 waves = 128 keys of one K/V head, one resident
//     workgroup per CU taking 128-key items in turn (fa_resident.hpp; with a
//     causal mask the first key blocks, which see the most queries, go
//     first); each wave owns 32 keys: their K and V rows and their dK^T, dV^T
//     accumulators sit in the accumulation registers;
//   * with grouped K/V heads the item runs the query loop once per query
//     head of its group (or of its slice of the group: then it writes fp32
//     partial sums that bwd_dkv_reduce_kernel adds in slot order), the
//     accumulators passed on from one run to the next;
//   * Q and dO tiles (64 queries) load three tiles ahead, HBM -> LDS by
//     direct loads, into four stages each (a tile is read as rows for the
//     scores and, half a tile later, transposed for the gradients), and each
//     wave's copy of the tile's L and D values beside them;
//   * the query loop is one generated statement (fa_bwd_dkdv128_loop.inc,
//     from gen_bwd_dkdv128.py).  The C++ below loads the item's K and V rows,
//     sets up addresses and loop bounds, and stores dK and dV.
#include "fa_bwd_dkdv128_loop.inc"
#include "fa_common.hpp"
#include "fa_internal.hpp"
#include "fa_resident.hpp"

#include <algorithm>

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int D = 128;
constexpr int BQ = 64;           // queries per tile
constexpr int NW = 4;            // waves per workgroup
constexpr int BK = 32 * NW;      // keys per workgroup
constexpr int TILE = BQ * D;     // elements per Q or dO tile
constexpr int TILE_BYTES = TILE * 2;

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

template <bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv128_kernel(BwdArgs a) {
  // LDS, bytes: [0, 64K) Q stages 0-3, [64K, 128K) dO stages 0-3, [128K,
  // 136K) L/D stages 0-3 of 2 KiB (wave w's 64 L values at 512 w, its D
  // values 256 bytes further).  The generated loop addresses these directly.
  // After the loop, [32K w, 32K (w + 1)) stages wave w's dK and dV rows.
  __shared__ __attribute__((aligned(1024))) bf16 smem[8 * TILE + 4096];
  constexpr uint32_t OST0 = 4 * TILE_BYTES, LST0 = 8 * TILE_BYTES;
  const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto lds_base = [&]() {
    return fresh(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS bf16*)smem)));
  };
  // Items: 128-key blocks of each (K/V head, slice of its query heads).
  auto shape = [&]() { return fresh_shape<BK, BQ>(a.N, a.B, a.Hkv * a.gsplit, a.Hkv); };
  // Key block of an item: with a causal mask, item rank 0 (handed out first)
  // is key block 0, which sees every query.
  auto key0_of = [&](const Shape& sh, const Item& it) {
    return CAUSAL ? (sh.nq - 1) * BK - it.q0 : it.q0;
  };
  // Query head g of an item's (K/V head, slice): the group of K/V head
  // b Hkv + j is query heads b H + j H/Hkv .. + H/Hkv - 1, split in gsplit
  // slices of consecutive heads.
  auto qhead_of = [&](const Item& it, int g) {
    const int H = fresh(a.H), Hkv = fresh(a.Hkv), gs = fresh(a.gsplit);
    const int kvh = it.bh / gs, slice = it.bh % gs;
    const int G = H / Hkv;
    return (kvh / Hkv) * H + (kvh % Hkv) * G + slice * (G / gs) + g;
  };
  // Query head bq's tiles ts .. ts + 2 of the item into stages 0 .. 2, and
  // this wave's copy of their L and D values (the LDS they fill is free: the
  // statement before, or the previous item's epilogue, ended with a barrier
  // after their last read).
  auto dma_first_tiles = [&](const Shape& sh, const Item& it, int bq) {
    const int wave = fresh(wave0);
    const uint32_t lds0 = lds_base();
    const int ts = CAUSAL ? key0_of(sh, it) / BQ : 0;
    const int cnt = sh.nt - ts;
    const size_t head = (size_t)bq * (size_t)sh.N * D;
    const bf16* Q = fresh(reinterpret_cast<const bf16*>(a.q)) + head;
    const bf16* dO = fresh(reinterpret_cast<const bf16*>(a.dout)) + head;
    const float* lse2 = fresh(a.lse2) + (size_t)bq * sh.N;
    const float* del = fresh(a.delta) + (size_t)bq * sh.N;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      if (s < cnt) {
        dma_tile128(sh, wave, Q, ts + s, lds0 + s * TILE_BYTES);
        dma_tile128(sh, wave, dO, ts + s, lds0 + OST0 + s * TILE_BYTES);
        dma_vec64(sh, lse2, ts + s, lds0 + LST0 + 2048u * s + 512u * wave);
        dma_vec64(sh, del, ts + s, lds0 + LST0 + 2048u * s + 512u * wave + 256u);
      }
    }
  };

  // One run of the query loop: query head bq's tiles against the item's keys,
  // added to dk, dv.  Every per-lane value is derived here again, so that
  // nothing but the item, the accumulators and the K/V rows lives across the
  // statement, which overwrites most registers.
  auto run_query_loop = [&](const Item& it, int bq, f32x16 (&dk)[4], f32x16 (&dv)[4],
                            bf16x8 (&kf)[8], bf16x8 (&vf)[8]) {
    const Shape sh = shape();
    const int N = sh.N, nt = sh.nt;
    const int wave = fresh(wave0);
    const uint32_t lds0 = lds_base();
    const int k0 = key0_of(sh, it);
    const int ts = CAUSAL ? k0 / BQ : 0;
    const int cnt = nt - ts;
    const int lane = fresh_lane();
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int key = k0 + 32 * wave + l32;
    // Lane parts of the LDS operand addresses (byte addresses in Q stage 0
    // and dO stage 0, first 32-query half).
    const int sw_row = tile_swz<D>(l32);
    u32x8 raddr, draddr, taddr, tdaddr;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      raddr[c] = lds0 + 2u * (l32 * D + 8 * ((2 * c + h) ^ sw_row));
      draddr[c] = raddr[c] + OST0;
    }
    const int tr_row = 4 * h + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int sw_lo = tile_swz<D>(tr_row), sw_hi = tile_swz<D>(tr_row + 8);
    const int tq = tr_col >> 3, te = tr_col & 7;
    auto tr_off = [&](int row, int sw, int b) {
      return row * D + 8 * (((4 * b) ^ (sw & 12)) | (tq ^ (sw & 3))) + te;
    };
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      taddr[2 * db] = lds0 + 2u * tr_off(tr_row, sw_lo, db);
      taddr[2 * db + 1] = lds0 + 2u * tr_off(tr_row + 8, sw_hi, db);
      tdaddr[2 * db] = taddr[2 * db] + OST0;
      tdaddr[2 * db + 1] = taddr[2 * db + 1] + OST0;
    }
    const uint32_t laddr = lds0 + LST0 + 512u * wave + 16u * h;
    // Direct-load offsets within a tile (wave w loads rows 16w .. 16w + 15;
    // load i carries instruction offset 1024 i, taken off here), and for the
    // partial last tile with its rows clamped to the sequence; the same for
    // the L/D values (lane l loads row l).
    u32x4 goff, gtail;
    const int tlast = nt - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * i + (lane >> 4);
      const int col = 8 * ((lane & 15) ^ tile_swz<D>(row));
      goff[i] = (uint32_t)(row * D + col) * 2u - 1024u * i;
      gtail[i] = (uint32_t)((min(tlast * BQ + row, N - 1) - tlast * BQ) * D + col) * 2u;
    }
    const uint32_t loff = 4u * lane;
    const uint32_t ltail = 4u * (uint32_t)(min(tlast * BQ + lane, N - 1) - tlast * BQ);
    // Visibility: the score of query q and this lane's key is kept iff
    // 0 <= q - base < N - base (base = the key with a causal mask, else 0).
    // The loop forms q - base = off - (ta - 64 j - 32 half) for register
    // offset off = 8 (r / 4) + r % 4 of relative tile j.
    const int base = CAUSAL ? key : 0;
    const int ta = base - 4 * h - BQ * ts;
    const int range = max(N - base, 0);

    auto uni = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); };
    auto uni64 = [&](uint64_t x) {
      return ((uint64_t)uni((uint32_t)(x >> 32)) << 32) | uni((uint32_t)x);
    };
    const uint32_t m0q = uni(lds0 + wave * 4096);
    const uint32_t m0o = uni(lds0 + OST0 + wave * 4096);
    const uint32_t m0l = uni(lds0 + LST0 + wave * 512);
    const uint32_t cbits = uniform_bits(fresh(a.scale) * kLog2e);   // scale * log2(e)
    // Loop control, in tiles relative to ts: step j processes tile j and
    // loads tile j + 3; the partial last tile (loaded by step cnt - 4) goes
    // through the clamped offsets; tiles below `mlo` (the causal diagonal) and
    // from `mhi` on (the partial last tile) need a mask; steps mlo <= j <
    // sfast need none and load whole tiles.
    const int mlo = CAUSAL ? 2 : 0;
    const int mhi = sh.ragged ? cnt - 1 : cnt;
    uint32_t jt = 0;
    const uint32_t slast = uni((uint32_t)(cnt - 1));
    const uint32_t skend = uni((uint32_t)max(0, cnt - 3));
    const uint32_t stailj = uni(sh.ragged && cnt >= 4 ? (uint32_t)(cnt - 4) : ~0u);
    const uint32_t smlo = uni((uint32_t)mlo);
    const uint32_t smhi = uni((uint32_t)mhi);
    const uint32_t sfast = uni((uint32_t)max(0, mhi - 3));
    const uint32_t smask0 = uni((mlo > 0 || mhi == 0) ? 1u : 0u);
    const float ninf = -INFINITY;

    const size_t head = (size_t)bq * (size_t)N * D;
    const bf16* Q = fresh(reinterpret_cast<const bf16*>(a.q)) + head;
    const bf16* dO = fresh(reinterpret_cast<const bf16*>(a.dout)) + head;
    const float* lse2 = fresh(a.lse2) + (size_t)bq * N;
    const float* del = fresh(a.delta) + (size_t)bq * N;
    uint64_t qptr = uni64(reinterpret_cast<uint64_t>(Q + (size_t)(ts + 3) * TILE));
    uint64_t optr = uni64(reinterpret_cast<uint64_t>(dO + (size_t)(ts + 3) * TILE));
    uint64_t lptr = uni64(reinterpret_cast<uint64_t>(lse2 + (size_t)(ts + 3) * BQ));
    // The D load carries instruction offset 256 (its LDS area follows L's).
    uint64_t dptr = uni64(reinterpret_cast<uint64_t>(del + (size_t)(ts + 3) * BQ) - 256u);
    wait_vmem();
    __syncthreads();   // tiles 0 .. 2 are in LDS for every wave

    asm volatile(FA_BWD_DKDV128_LOOP_ASM
                 : "+{a[0:15]}"(dk[0]), "+{a[16:31]}"(dk[1]), "+{a[32:47]}"(dk[2]),
                   "+{a[48:63]}"(dk[3]), "+{a[64:79]}"(dv[0]), "+{a[80:95]}"(dv[1]),
                   "+{a[96:111]}"(dv[2]), "+{a[112:127]}"(dv[3]),
                   "+{s[60:61]}"(qptr), "+{s[62:63]}"(optr), "+{s[84:85]}"(lptr),
                   "+{s[86:87]}"(dptr), "+{s71}"(jt),
                   // unchanged by the statement; in-out so that they stay in
                   // place from one run to the next
                   "+{a[128:131]}"(kf[0]), "+{a[132:135]}"(kf[1]), "+{a[136:139]}"(kf[2]),
                   "+{a[140:143]}"(kf[3]), "+{a[144:147]}"(kf[4]), "+{a[148:151]}"(kf[5]),
                   "+{a[152:155]}"(kf[6]), "+{a[156:159]}"(kf[7]),
                   "+{a[160:163]}"(vf[0]), "+{a[164:167]}"(vf[1]), "+{a[168:171]}"(vf[2]),
                   "+{a[172:175]}"(vf[3]), "+{a[176:179]}"(vf[4]), "+{a[180:183]}"(vf[5]),
                   "+{a[184:187]}"(vf[6]), "+{a[188:191]}"(vf[7])
                 : "{v[160:167]}"(raddr), "{v[168:175]}"(draddr), "{v[176:183]}"(taddr),
                   "{v[184:191]}"(tdaddr), "{v192}"(laddr), "{v[196:199]}"(goff),
                   "{v[200:203]}"(gtail), "{v204}"(loff), "{v205}"(ltail), "{v206}"(ta),
                   "{v207}"(range), "{v208}"(ninf),
                   "{s64}"(m0q), "{s65}"(m0o), "{s66}"(cbits), "{s67}"(slast), "{s68}"(skend),
                   "{s69}"(stailj), "{s70}"(smlo), "{s72}"(smhi), "{s82}"(sfast), "{s88}"(m0l),
                   "{s89}"(smask0)
                 : FA_BWD_DKDV128_LOOP_CLOBBERS);
  };

  Item cur;
  {
    const Shape sh = shape();
    if (!resident_item<CAUSAL, BK>(sh, 0, cur)) return;
    dma_first_tiles(sh, cur, qhead_of(cur, 0));
  }

  for (int r = 0;; ++r) {
    const Shape sh = shape();
    Item nxt;
    const bool more = resident_item<CAUSAL, BK>(sh, r + 1, nxt);
    const int N = sh.N;
    const int wave = fresh(wave0);
    const int k0 = key0_of(sh, cur);
    const int kvh = cur.bh / fresh(a.gsplit);   // K/V head of the item
    const size_t kvhead = (size_t)kvh * (size_t)N * D;

    // This wave's K and V rows: lane (l32, h) holds key k0 + 32 wave + l32,
    // d = 16 c + 8 h .. +7 (keys past the sequence repeat its last one; their
    // dK and dV are never stored).
    const int lane = fresh_lane();
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int key = k0 + 32 * wave + l32;
    const size_t krow = kvhead + (size_t)min(key, N - 1) * D;
    const bf16* Kr = fresh(reinterpret_cast<const bf16*>(a.k)) + krow + 8 * h;
    const bf16* Vr = fresh(reinterpret_cast<const bf16*>(a.v)) + krow + 8 * h;
    bf16x8 kf[8], vf[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      kf[c] = *reinterpret_cast<const bf16x8*>(Kr + 16 * c);
      vf[c] = *reinterpret_cast<const bf16x8*>(Vr + 16 * c);
    }

    // The query loop once per query head of the item's group (slice), the
    // accumulators passed on from one run to the next.
    f32x16 dk[4], dv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) dk[i][e] = dv[i][e] = 0.f;
    const int heads = fresh(a.H) / fresh(a.Hkv) / fresh(a.gsplit);
    for (int g = 0; g < heads; ++g) {
      // The previous run ended with a barrier after its last LDS read.
      if (g > 0) dma_first_tiles(shape(), cur, qhead_of(cur, g));
      run_query_loop(cur, qhead_of(cur, g), dk, dv, kf, vf);
    }

    // Epilogue: dK = scale * acc, dV = acc, fp32.  Lane (l32, h) of block db
    // holds key l32, d = 32 db + 8 g + 4 h .. +3 in registers 4g .. 4g + 3:
    // stored as it is, every instruction would write 32 B pieces of 32 rows.
    // Each wave passes its 32 rows of dK and of dV through its own 32 KiB of
    // LDS instead (16-byte chunk q of row k at slot q ^ k, so that the writes
    // of 32 rows and the reads of 2 whole rows both spread over the banks)
    // and stores 1 KiB of two consecutive rows per instruction.
    const Shape sh2 = shape();
    const int wave2 = fresh(wave0);
    const int el = fresh_lane(), eh = el >> 5, e32 = el & 31;
    const float sc = fresh(a.scale);
    // dV passes through a multiply by an opaque 1 too: a plain copy out of the
    // accumulation registers is not lowered correctly (it becomes a vector
    // move with a 16-register source).
    const float one = fresh(1.0f);
    FA_LDS char* stg = (FA_LDS char*)smem + 32768 * wave2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x, y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = dk[db][4 * g + e] * sc;
          y[e] = dv[db][4 * g + e] * one;
        }
        const int slot = 16 * ((8 * db + 2 * g + eh) ^ e32);
        *reinterpret_cast<FA_LDS f32x4*>(stg + 512 * e32 + slot) = x;
        *reinterpret_cast<FA_LDS f32x4*>(stg + 16384 + 512 * e32 + slot) = y;
      }
    f32x4 rk[16], rv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 2 * i + eh;
      const int slot = 16 * (e32 ^ row);
      rk[i] = *reinterpret_cast<const FA_LDS f32x4*>(stg + 512 * row + slot);
      rv[i] = *reinterpret_cast<const FA_LDS f32x4*>(stg + 16384 + 512 * row + slot);
    }
    __syncthreads();   // every wave has its rows: the LDS takes the next item's tiles
    if (more) dma_first_tiles(sh2, nxt, qhead_of(nxt, 0));
    const int kw = key0_of(sh2, cur) + 32 * wave2;
    typedef __attribute__((address_space(1))) f32x4 gf32x4;
    // dK, dV of the K/V head, or (slices) partial slots slice and
    // gsplit + slice of `part`.
    const int gs2 = fresh(a.gsplit);
    const int kvh2 = cur.bh / gs2, slice2 = cur.bh % gs2;
    const size_t kvsize = (size_t)fresh(a.B) * (size_t)fresh(a.Hkv) * (size_t)sh2.N * D;
    const size_t row0 = ((size_t)kvh2 * sh2.N + kw + eh) * D + 4 * e32;
    float* dkbase = gs2 > 1 ? fresh(a.part) + (size_t)slice2 * kvsize : fresh(a.dk);
    float* dvbase = gs2 > 1 ? fresh(a.part) + (size_t)(gs2 + slice2) * kvsize : fresh(a.dv);
    gf32x4* dkp = (gf32x4*)(dkbase + row0);
    gf32x4* dvp = (gf32x4*)(dvbase + row0);
    const int rows = sh2.N - kw;   // rows of this wave inside the sequence
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (2 * i + eh < rows) {
        dkp[i * (2 * D / 4)] = rk[i];
        dvp[i * (2 * D / 4)] = rv[i];
      }
    }
    if (!more) break;
    cur = nxt;
  }
}

}  // namespace

// Whether the hand-scheduled dK/dV kernel takes this backward: head dim 128,
// no tile mask, at least one item (128 keys of one K/V head and slice) per
// CU.
bool dkdv128_applies(const BwdArgs& a) {
  if (a.d != 128 || a.mask != nullptr) return false;
  const long long items = (long long)((a.N + BK - 1) / BK) * a.B * a.Hkv * a.gsplit;
  return items >= 256;
}

hipError_t launch_dkdv128(const BwdArgs& a, hipStream_t s) {
  const long long items = (long long)((a.N + BK - 1) / BK) * a.B * a.Hkv * a.gsplit;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const long long grid = std::min<long long>(items, resident_cu_count());
  if (a.causal)
    hipLaunchKernelGGL((bwd_dkdv128_kernel<true>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dkdv128_kernel<false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
