// bench_mfma_ceiling.hip -- how much bf16 MFMA throughput this GPU sustains.
//
// Built and run by `python bench.py --mfma-ceiling`.  Each wave repeats the
// matrix-core work of one attention tile (S = K Q^T as two chains of eight
// v_mfma_f32_32x32x16_bf16, conversion of S to bf16, O += V P as four chains),
// with every operand in registers: no memory traffic inside the loop.  It is
// run twice, on all-zero operands and on random bf16 operands, at 1-4 waves
// per SIMD.  The random-operand rate is the practical ceiling the attention
// kernels can approach: dense bf16 MFMA on random data draws enough power that
// the clock drops well below its 2.4 GHz maximum (the zero-operand run shows
// the same instruction stream at full clock).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);       \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

template <int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void tile_mfma(const bf16x8* in, float* out, int iters) {
  const int l = threadIdx.x & 63;
  bf16x8 q[8], v[4];
  for (int c = 0; c < 8; ++c) q[c] = in[(l + 8 * c) & 511];
  for (int c = 0; c < 4; ++c) v[c] = in[(l + 8 * c + 3) & 511];
  f32x16 o[4];
  for (int b = 0; b < 4; ++b)
    for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q[(c + kb) & 7], q[c], s[kb], 0, 0, 0);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        bf16x8 p;
        for (int e = 0; e < 8; ++e) p[e] = (__bf16)(s[kb][8 * cc + e] * 0.001f);
#pragma unroll
        for (int b = 0; b < 4; ++b)
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[b], p, o[b], 0, 0, 0);
      }
  }
  float t = 0.f;
  for (int b = 0; b < 4; ++b)
    for (int r = 0; r < 16; ++r) t += o[b][r];
  out[blockIdx.x * 256 + threadIdx.x] = t;
}

template <int WPE>
int run(const bf16x8* in, float* out, const char* data) {
  const int blocks = 256 * WPE, iters = 1024;  // every SIMD holds WPE waves
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL(tile_mfma<WPE>, dim3(blocks), dim3(256), 0, 0, in, out, iters);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e0));
  hipLaunchKernelGGL(tile_mfma<WPE>, dim3(blocks), dim3(256), 0, 0, in, out, iters);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double flops = (double)blocks * 4 * iters * 32 * 32768.0;
  printf("{\"data\": \"%s\", \"waves_per_simd\": %d, \"ms\": %.4f, \"tflops\": %.1f}\n", data, WPE,
         ms, flops / ms / 1e9);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return 0;
}

int main() {
  const int n = 512;
  bf16x8* in = nullptr;
  float* out = nullptr;
  CHECK(hipMalloc(&in, n * sizeof(bf16x8)));
  CHECK(hipMalloc(&out, (size_t)256 * 4 * 256 * sizeof(float)));
  for (int pass = 0; pass < 2; ++pass) {
    static unsigned short h[512 * 8];
    unsigned x = 12345u;
    for (int i = 0; i < n * 8; ++i) {
      x = x * 1664525u + 1013904223u;
      const float f = pass == 0 ? 0.f : ((x >> 8) & 0xffff) / 32768.0f - 1.0f;
      unsigned u;
      memcpy(&u, &f, 4);
      h[i] = (unsigned short)(u >> 16);
    }
    CHECK(hipMemcpy(in, h, sizeof(h), hipMemcpyHostToDevice));
    const char* data = pass == 0 ? "zeros" : "random";
    if (run<1>(in, out, data) || run<2>(in, out, data) || run<3>(in, out, data) ||
        run<4>(in, out, data))
      return 1;
  }
  CHECK(hipFree(in));
  CHECK(hipFree(out));
  return 0;
}
