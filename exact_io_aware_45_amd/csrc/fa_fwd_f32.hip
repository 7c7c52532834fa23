// fa_fwd_f32.hip -- exact attention forward in fp32 (inputs, arithmetic and
// outputs), for small problems that need fp32 accuracy.  Same definition and
// online softmax as the bf16 kernel ("FlashAttention." plate, opening section;
// "Flash Attention: IO-Aware Attention Computation", paragraph on fused
// kernels and the online softmax), on plain vector ALUs: the matrix cores'
// fp32 path is not needed at these sizes.
//
// These problems are latency-bound (one head of 128 rows is a handful of
// workgroups), so the work is spread thin:
//   * LPR = d / 16 lanes share a query row, each owning 16 of its d columns
//     (q and the running output in registers); a wave covers 64 / LPR rows;
//   * the eight waves of a workgroup take the same rows and split the keys:
//     wave w visits key chunks w, w + 8, w + 16, ... (KC keys each, read
//     straight from global memory: the whole head sits in cache), keeping its
//     own running maximum, sum and output;
//   * the eight partial states are merged at the end through LDS with the
//     same rule the online softmax uses between tiles: with M the largest
//     partial maximum, L = sum_w l_w e^(m_w - M) and O = sum_w o_w e^(m_w - M) / L.
// exp/log are the accurate libm-style device functions (expf/logf), not the
// hardware approximations.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = 16;  // d columns per lane
constexpr int KC = 4;      // keys per chunk

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a) {
  constexpr int LPR = D / kCols;    // lanes per query row
  constexpr int RPW = 64 / LPR;     // query rows per workgroup
  constexpr int F4 = kCols / 4;     // float4 per lane per key row
  // Partial states of every wave: kCols outputs, then m and l, per lane.
  __shared__ float part_s[kWaves][kCols + 2][64];

  const int N = a.N;
  const int nq = (N + RPW - 1) / RPW;
  const int bh = blockIdx.x / nq;
  const int q0 = (blockIdx.x % nq) * RPW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = q0 + lane / LPR;
  const int col0 = (lane % LPR) * kCols;
  const size_t head = (size_t)bh * N * D;
  const float* Q = reinterpret_cast<const float*>(a.q) + head;
  const float* K = reinterpret_cast<const float*>(a.k) + head;
  const float* V = reinterpret_cast<const float*>(a.v) + head;
  float* O = reinterpret_cast<float*>(a.o) + head;

  float q[kCols], o[kCols];
  const int qr = row < N ? row : N - 1;
#pragma unroll
  for (int i = 0; i < F4; ++i) {
    const float4 x = *reinterpret_cast<const float4*>(Q + (size_t)qr * D + col0 + 4 * i);
    q[4 * i] = x.x; q[4 * i + 1] = x.y; q[4 * i + 2] = x.z; q[4 * i + 3] = x.w;
  }
#pragma unroll
  for (int c = 0; c < kCols; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float scale = a.scale;

  const int qlast = min(q0 + RPW, N) - 1;
  const int kend = CAUSAL ? qlast + 1 : N;
  for (int k0 = wave * KC; k0 < kend; k0 += kWaves * KC) {
    float kr[KC][kCols], vr[KC][kCols];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const size_t off = (size_t)min(k0 + j, N - 1) * D + col0;
#pragma unroll
      for (int i = 0; i < F4; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(K + off + 4 * i);
        kr[j][4 * i] = x.x; kr[j][4 * i + 1] = x.y; kr[j][4 * i + 2] = x.z; kr[j][4 * i + 3] = x.w;
        const float4 y = *reinterpret_cast<const float4*>(V + off + 4 * i);
        vr[j][4 * i] = y.x; vr[j][4 * i + 1] = y.y; vr[j][4 * i + 2] = y.z; vr[j][4 * i + 3] = y.w;
      }
    }
    float s[KC];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < kCols; ++c) acc = fmaf(q[c], kr[j][c], acc);
#pragma unroll
      for (int st = 1; st < LPR; st *= 2) acc += __shfl_xor(acc, st, LPR);
      const int key = k0 + j;
      s[j] = (key < N && (!CAUSAL || key <= row)) ? acc * scale : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;  // nothing visible yet for this row
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < kCols; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const float p = expf(s[j] - m_new);
      l += p;
#pragma unroll
      for (int c = 0; c < kCols; ++c) o[c] = fmaf(p, vr[j][c], o[c]);
    }
    m = m_new;
  }

  // Merge the eight partial states of each (row, column group).
#pragma unroll
  for (int c = 0; c < kCols; ++c) part_s[wave][c][lane] = o[c];
  part_s[wave][kCols][lane] = m;
  part_s[wave][kCols + 1][lane] = l;
  __syncthreads();
  if (wave != 0) return;
  float mw[kWaves];
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = part_s[w][kCols][lane];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.f;
#pragma unroll
  for (int c = 0; c < kCols; ++c) o[c] = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = expf(mw[w] - M);  // 0 for a wave that saw no visible key
      L = fmaf(part_s[w][kCols + 1][lane], f, L);
#pragma unroll
      for (int c = 0; c < kCols; ++c) o[c] = fmaf(part_s[w][c][lane], f, o[c]);
    }
  }
  if (row < N) {
    const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
    for (int i = 0; i < F4; ++i) {
      float4 x;
      x.x = o[4 * i] * inv; x.y = o[4 * i + 1] * inv; x.z = o[4 * i + 2] * inv;
      x.w = o[4 * i + 3] * inv;
      *reinterpret_cast<float4*>(O + (size_t)row * D + col0 + 4 * i) = x;
    }
    if (col0 == 0) a.lse[(size_t)bh * N + row] = L > 0.f ? M + logf(L) : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  constexpr int RPW = 64 / (D / kCols);
  const long long grid = (long long)((a.N + RPW - 1) / RPW) * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.causal)
    hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  if (a.d == 64) return launch_d<64>(a, s);
  if (a.d == 128) return launch_d<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
