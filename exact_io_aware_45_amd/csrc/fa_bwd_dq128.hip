// fa_bwd_dq128.hip -- the dQ pass of the backward for head dim 128, bf16
// inputs, fp32 dQ, with a hand-scheduled key loop (gfx950).
//
// Same result as bwd_dq_kernel (fa_bwd.hip): for every query row the scores
// and their gradient are recomputed tile by tile from the saved log-sum-exp,
// never stored ("FlashAttention." plate, "Never write the scores"), and
//   dQ = scale * sum_j dS_j K_j,  dS = P (dP - D),  P = exp2(S c - L),
// with S = Q K^T, dP = dO V^T, L = LSE log2(e), c = scale log2(e) and
// D = rowsum(dO o O), which the delta pass stores negated.
//
// Work decomposition:
//   * one workgroup = 4 waves = 256 query rows of one head, one resident
//     workgroup per CU taking 256-row items in turn (fa_resident.hpp); each
//     wave owns 64 rows (two 32-row blocks), its Q^T and dO^T operands and
//     its dQ^T accumulators sit in the 256 accumulation registers;
//   * K and V tiles (64 keys) load two tiles ahead, HBM -> LDS by direct
//     loads, K into four stages and V into two: K_j is read as rows for the
//     scores of tile j and transposed for its dQ products one half-tile later;
//   * the key loop is one generated statement (fa_bwd_dq128_loop.inc, from
//     gen_bwd_dq128.py) that overlaps each 32-key half's exponentials and dS
//     with the products of its neighbours.  The C++ below stages the item's
//     Q and dO rows through LDS into registers, sets up addresses, and stores
//     dQ through LDS in whole rows while the next item's first loads land.
#include "fa_bwd_dq128_loop.inc"
#include "fa_common.hpp"
#include "fa_internal.hpp"
#include "fa_resident.hpp"

#include <algorithm>

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int D = 128;
constexpr int BC = 64;           // keys per tile
constexpr int NW = 4;            // waves per workgroup
constexpr int BR = 64 * NW;      // query rows per workgroup
constexpr int TILE = BC * D;     // elements per K or V tile
constexpr int TILE_BYTES = TILE * 2;

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

template <bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq128_kernel(BwdArgs a) {
  // LDS, bytes: [0, 64K) K stages 0-3 and [64K, 96K) V stages 0-1 (the
  // generated loop addresses these directly); [96K, 160K) each wave's 64
  // query rows at the start of an item.  An item's dO rows pass through
  // [32K, 96K) before its first V tiles load there.  After the loop,
  // [32K w, 32K (w + 1)) stages wave w's dQ rows.
  __shared__ __attribute__((aligned(1024))) bf16 smem[10 * TILE];
  constexpr uint32_t VST0 = 4 * TILE_BYTES, QST0 = 6 * TILE_BYTES, DOST0 = 2 * TILE_BYTES;
  const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto lds_base = [&]() {
    return fresh(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FA_LDS bf16*)smem)));
  };

  auto shape = [&]() { return fresh_shape<BR, BC>(a.N, a.B, a.H, a.Hkv); };
  auto tend_of = [&](const Shape& sh, const Item& it) {
    return CAUSAL ? min(sh.nt, (min(it.q0 + BR, sh.N) - 1) / BC + 1) : sh.nt;
  };
  // An item's first loads: this wave's Q and dO rows and K tiles 0 and 1
  // (the LDS they fill is free: the previous item's loop and epilogue ended
  // with a barrier after their last read).
  auto dma_first = [&](const Shape& sh, const Item& it) {
    const int wave = fresh(wave0);
    const uint32_t lds0 = lds_base();
    const size_t head = (size_t)it.bh * (size_t)sh.N * D;
    const bf16* K = fresh(reinterpret_cast<const bf16*>(a.k)) + kv_head_offset(sh, it.bh, D);
    dma_rows128(sh, fresh(reinterpret_cast<const bf16*>(a.q)) + head, it.q0 + 64 * wave,
                lds0 + QST0 + 16384u * wave);
    dma_rows128(sh, fresh(reinterpret_cast<const bf16*>(a.dout)) + head, it.q0 + 64 * wave,
                lds0 + DOST0 + 16384u * wave);
    dma_tile128(sh, wave, K, 0, lds0);
    if (tend_of(sh, it) > 1) dma_tile128(sh, wave, K, 1, lds0 + TILE_BYTES);
  };

  Item cur;
  {
    const Shape sh = shape();
    if (!resident_item<CAUSAL, BR>(sh, 0, cur)) return;
    dma_first(sh, cur);
  }

  for (int r = 0;; ++r) {
    const Shape sh = shape();
    Item nxt;
    const bool more = resident_item<CAUSAL, BR>(sh, r + 1, nxt);
    const int N = sh.N, nt = sh.nt;
    const int wave = fresh(wave0);
    const uint32_t lds0 = lds_base();
    const int q0 = cur.q0;
    const int wrow0 = q0 + 64 * wave;
    const size_t kv = kv_head_offset(sh, cur.bh, D);
    const bf16* __restrict__ K = fresh(reinterpret_cast<const bf16*>(a.k)) + kv;
    const bf16* __restrict__ V = fresh(reinterpret_cast<const bf16*>(a.v)) + kv;
    const int tend = tend_of(sh, cur);
    int fm = tend;
    if (CAUSAL) fm = min(fm, q0 / BC);
    if (sh.ragged) fm = min(fm, nt - 1);

    const int lane = fresh_lane();
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int sw_row = tile_swz<D>(l32);
    // L and D of this lane's two rows (rows past the sequence repeat the last
    // one; their dQ is never stored).
    const float* lse2 = fresh(a.lse2) + (size_t)cur.bh * N;
    const float* del = fresh(a.delta) + (size_t)cur.bh * N;
    float lsel[2], dd[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = min(wrow0 + 32 * rb + l32, N - 1);
      lsel[rb] = lse2[row];
      dd[rb] = del[row];   // -D
    }
    wait_vmem();   // this wave's own rows (the K tiles are published by the barrier below)

    // Q^T and dO^T operands: row block rb holds rows wrow0 + 32 rb + l32,
    // d = 16c + 8h .. +7.
    bf16x8 qf[2][8], df[2][8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int e = (32 * rb + l32) * D + 8 * ((2 * c + h) ^ sw_row);
        qf[rb][c] = lds_read8(smem + QST0 / 2 + wave * TILE + e);
        df[rb][c] = lds_read8(smem + DOST0 / 2 + wave * TILE + e);
      }
    wait_lds();
    __syncthreads();   // every wave has its dO rows: V tiles 0 and 1 may overwrite them
    dma_tile128(sh, wave, V, 0, lds0 + VST0);
    if (tend > 1) dma_tile128(sh, wave, V, 1, lds0 + VST0 + TILE_BYTES);

    // Lane parts of the LDS operand addresses (byte addresses of K stage 0 and
    // V stage 0, key block 0).
    u32x8 raddr, vraddr, taddr;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      raddr[c] = lds0 + 2u * (l32 * D + 8 * ((2 * c + h) ^ sw_row));
      vraddr[c] = raddr[c] + VST0;
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
    }
    // Direct-load offsets within a tile (wave w loads rows 16w .. 16w + 15;
    // load i carries instruction offset 1024 i, taken off here), and for the
    // partial last tile with its rows clamped to the sequence.
    u32x4 goff, gtail;
    const int tlast = tend - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * i + (lane >> 4);
      const int col = 8 * ((lane & 15) ^ tile_swz<D>(row));
      goff[i] = (uint32_t)(row * D + col) * 2u - 1024u * i;
      gtail[i] = (uint32_t)((min(tlast * BC + row, N - 1) - tlast * BC) * D + col) * 2u;
    }
    // Mask thresholds: a score is masked when its key exceeds the row's last
    // visible key.  thr1 is the threshold of tile f, thr of tile f + 1, with
    // f the first tile whose step masks (max(fm - 1, 0)); tiles before fm
    // hold no invisible key, so masking them with these changes nothing.
    const int f = max(fm - 1, 0);
    float thr[2], thr1[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = wrow0 + 32 * rb + l32;
      const int lim = CAUSAL ? min(row, N - 1) : N - 1;
      thr1[rb] = __builtin_bit_cast(float, lim - 4 * h - BC * f);
      thr[rb] = __builtin_bit_cast(float, lim - 4 * h - BC * (f + 1));
    }

    auto uni = [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); };
    auto uni64 = [&](uint64_t x) {
      return ((uint64_t)uni((uint32_t)(x >> 32)) << 32) | uni((uint32_t)x);
    };
    const uint32_t m0k = uni(lds0 + wave * 4096);
    const uint32_t m0v = uni(lds0 + VST0 + wave * 4096);
    const uint32_t cbits = uniform_bits(fresh(a.scale) * kLog2e);   // scale * log2(e)
    uint64_t kptr = uni64(reinterpret_cast<uint64_t>(K + 2 * (size_t)TILE));
    uint64_t vptr = uni64(reinterpret_cast<uint64_t>(V + 2 * (size_t)TILE));
    // Loop control: step j processes tile j and loads tile j + 2 (K and V);
    // the partial last tile (loaded by step nt - 3) goes through the clamped
    // offsets; steps below `sfast` have an unmasked next tile and whole loads.
    const bool tail = sh.ragged && tend == nt;
    const int kfull = tail ? nt - 1 : tend;
    uint32_t jt = 0;
    const uint32_t slast = uni((uint32_t)(tend - 1));
    const uint32_t skend = uni((uint32_t)max(0, tend - 2));
    const uint32_t stailj = uni(tail && nt >= 3 ? (uint32_t)(nt - 3) : ~0u);
    const uint32_t sfm = uni((uint32_t)fm);
    const uint32_t sfast = uni((uint32_t)max(0, min(fm - 1, kfull - 2)));
    const float ninf = -INFINITY;
    wait_vmem();
    __syncthreads();   // K and V tiles 0 and 1 are in LDS for every wave

    f32x16 acc[2][4];
    asm volatile(FA_BWD_DQ128_LOOP_ASM
                 : "={a[0:15]}"(acc[0][0]), "={a[16:31]}"(acc[0][1]), "={a[32:47]}"(acc[0][2]),
                   "={a[48:63]}"(acc[0][3]), "={a[64:79]}"(acc[1][0]), "={a[80:95]}"(acc[1][1]),
                   "={a[96:111]}"(acc[1][2]), "={a[112:127]}"(acc[1][3]),
                   "+{v236}"(thr[0]), "+{v237}"(thr[1]), "+{v238}"(thr1[0]), "+{v239}"(thr1[1]),
                   "+{s[60:61]}"(kptr), "+{s[62:63]}"(vptr), "+{s71}"(jt)
                 : "{a[128:131]}"(qf[0][0]), "{a[132:135]}"(qf[0][1]),
                   "{a[136:139]}"(qf[0][2]), "{a[140:143]}"(qf[0][3]),
                   "{a[144:147]}"(qf[0][4]), "{a[148:151]}"(qf[0][5]),
                   "{a[152:155]}"(qf[0][6]), "{a[156:159]}"(qf[0][7]),
                   "{a[160:163]}"(qf[1][0]), "{a[164:167]}"(qf[1][1]),
                   "{a[168:171]}"(qf[1][2]), "{a[172:175]}"(qf[1][3]),
                   "{a[176:179]}"(qf[1][4]), "{a[180:183]}"(qf[1][5]),
                   "{a[184:187]}"(qf[1][6]), "{a[188:191]}"(qf[1][7]),
                   "{a[192:195]}"(df[0][0]), "{a[196:199]}"(df[0][1]),
                   "{a[200:203]}"(df[0][2]), "{a[204:207]}"(df[0][3]),
                   "{a[208:211]}"(df[0][4]), "{a[212:215]}"(df[0][5]),
                   "{a[216:219]}"(df[0][6]), "{a[220:223]}"(df[0][7]),
                   "{a[224:227]}"(df[1][0]), "{a[228:231]}"(df[1][1]),
                   "{a[232:235]}"(df[1][2]), "{a[236:239]}"(df[1][3]),
                   "{a[240:243]}"(df[1][4]), "{a[244:247]}"(df[1][5]),
                   "{a[248:251]}"(df[1][6]), "{a[252:255]}"(df[1][7]),
                   "{v[208:215]}"(raddr), "{v[216:223]}"(taddr), "{v224}"(lsel[0]),
                   "{v225}"(lsel[1]), "{v226}"(dd[0]), "{v227}"(dd[1]), "{v[228:231]}"(goff),
                   "{v[232:235]}"(gtail), "{v240}"(ninf), "{v[242:249]}"(vraddr),
                   "{s64}"(m0k), "{s65}"(m0v), "{s66}"(cbits), "{s67}"(slast), "{s68}"(skend),
                   "{s69}"(stailj), "{s70}"(sfm), "{s82}"(sfast)
                 : FA_BWD_DQ128_LOOP_CLOBBERS);

    // Epilogue: dQ = scale * acc, fp32.  Lane (l32, h) of block (rb, db)
    // holds row 32 rb + l32, d = 32 db + 8 g + 4 h .. +3 in registers 4g ..
    // 4g + 3: stored as it is, every instruction would write 32 B pieces of
    // 32 rows.  Each wave passes its 64 rows through its own 32 KiB of LDS
    // instead (16-byte chunk q of row k at slot q ^ (k mod 32), so that the
    // writes of 32 rows and the reads of 2 whole rows both spread over the
    // banks) and stores 1 KiB of two consecutive rows per instruction.
    const Shape sh2 = shape();
    const int wave2 = fresh(wave0);
    const int el = fresh_lane(), eh = el >> 5, e32 = el & 31;
    const float sc = fresh(a.scale);
    FA_LDS char* stg = (FA_LDS char*)smem + 32768 * wave2;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = acc[rb][db][4 * g + e] * sc;
          *reinterpret_cast<FA_LDS f32x4*>(stg + 512 * (32 * rb + e32) +
                                           16 * ((8 * db + 2 * g + eh) ^ e32)) = x;
        }
    f32x4 rq[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int row = 2 * i + eh;
      rq[i] = *reinterpret_cast<const FA_LDS f32x4*>(stg + 512 * row + 16 * (e32 ^ (row & 31)));
    }
    __syncthreads();   // every wave has its rows: the LDS takes the next item's first loads
    if (more) dma_first(sh2, nxt);
    const int wrow2 = cur.q0 + 64 * wave2;
    typedef __attribute__((address_space(1))) f32x4 gf32x4;
    gf32x4* dqp = (gf32x4*)(fresh(a.dq) + ((size_t)cur.bh * sh2.N + wrow2 + eh) * D + 4 * e32);
    const int rows = sh2.N - wrow2;   // rows of this wave inside the sequence
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (2 * i + eh < rows) dqp[i * (2 * D / 4)] = rq[i];
    if (!more) break;
    cur = nxt;
  }
}

}  // namespace

// Whether the hand-scheduled dQ kernel takes this backward: head dim 128,
// no tile mask, at least one 256-row item per CU.
bool dq128_applies(const BwdArgs& a) {
  if (a.d != 128 || a.mask != nullptr) return false;
  const long long items = (long long)((a.N + BR - 1) / BR) * a.B * a.H;
  return items >= 256;
}

hipError_t launch_dq128(const BwdArgs& a, hipStream_t s) {
  const long long items = (long long)((a.N + BR - 1) / BR) * a.B * a.H;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const long long grid = std::min<long long>(items, resident_cu_count());
  if (a.causal)
    hipLaunchKernelGGL((bwd_dq128_kernel<true>), dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq128_kernel<false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace fa
