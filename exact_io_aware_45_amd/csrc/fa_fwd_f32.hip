// fa_fwd_f32.hip -- exact attention forward in fp32 (inputs, arithmetic and
// outputs), for small problems that need fp32 accuracy.  Same definition and
// online softmax as the bf16 kernel ("FlashAttention." plate, opening section;
// "Flash Attention: IO-Aware Attention Computation", paragraph on fused
// kernels and the online softmax), on plain vector ALUs: the matrix cores'
// fp32 path is not needed at these sizes.
//
// One workgroup = 64 query rows of one head; four lanes share a query row,
// each owning a quarter of the d columns of q and of the running output.
// K/V tiles of 32 keys are staged in LDS.  exp/log are the accurate libm-style
// device functions (expf/logf), not the hardware approximations.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int kRows = 64;
constexpr int kThreads = 4 * kRows;
constexpr int kKeys = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a) {
  constexpr int DQ = D / 4;  // columns per lane
  __shared__ float Ks[kKeys][D + 1];
  __shared__ float Vs[kKeys][D + 1];

  const int N = a.N;
  const int nq = (N + kRows - 1) / kRows;
  const int bh = blockIdx.x / nq;
  const int q0 = (blockIdx.x % nq) * kRows;
  const int row = q0 + threadIdx.x / 4;
  const int part = threadIdx.x % 4;
  const size_t head = (size_t)bh * N * D;
  const float* Q = reinterpret_cast<const float*>(a.q) + head;
  const float* K = reinterpret_cast<const float*>(a.k) + head;
  const float* V = reinterpret_cast<const float*>(a.v) + head;
  float* O = reinterpret_cast<float*>(a.o) + head;

  float q[DQ], o[DQ];
  const int qr = row < N ? row : N - 1;
#pragma unroll
  for (int c = 0; c < DQ; ++c) {
    q[c] = Q[(size_t)qr * D + part * DQ + c];
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float scale = a.scale;

  const int qlast = min(q0 + kRows, N) - 1;
  const int kend = CAUSAL ? qlast + 1 : N;
  for (int k0 = 0; k0 < kend; k0 += kKeys) {
    __syncthreads();
    for (int i = threadIdx.x; i < kKeys * D; i += kThreads) {
      const int r = i / D, c = i % D;
      const int key = min(k0 + r, N - 1);
      Ks[r][c] = K[(size_t)key * D + c];
      Vs[r][c] = V[(size_t)key * D + c];
    }
    __syncthreads();
    float s[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DQ; ++c) acc = fmaf(q[c], Ks[j][part * DQ + c], acc);
      acc += __shfl_xor(acc, 1, 4);
      acc += __shfl_xor(acc, 2, 4);
      const int key = k0 + j;
      s[j] = (key < N && (!CAUSAL || key <= row)) ? acc * scale : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;  // nothing visible yet for this row
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < DQ; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = expf(s[j] - m_new);
      l += p;
#pragma unroll
      for (int c = 0; c < DQ; ++c) o[c] = fmaf(p, Vs[j][part * DQ + c], o[c]);
    }
    m = m_new;
  }
  if (row < N) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int c = 0; c < DQ; ++c) O[(size_t)row * D + part * DQ + c] = o[c] * inv;
    if (part == 0) a.lse[(size_t)bh * N + row] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
  const long long grid = (long long)((a.N + kRows - 1) / kRows) * a.B * a.H;
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
