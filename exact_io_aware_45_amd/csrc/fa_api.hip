// fa_api.hip -- the C ABI declared in include/fa.h: argument validation and
// dispatch to the kernel launchers.  No allocation; the only state is the
// fixed scratch array of fa_backward_noalloc and its per-device address.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.hpp"

// Scratch of fa_backward_noalloc: the backward workspace (D, then
// LSE * log2(e), one fp32 each per row) for callers that cannot allocate.
// Every GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` only names the array: its device address on each
// GPU comes from hipGetSymbolAddress, taken once per device with that device
// current (scratch_address below), and only that address is passed to
// kernels.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kVersion = 400;  // 0.4.0

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks shared by every entry point.  Sets *empty when there is no work.
int check_shape(int B, int H, int N, int d, float scale, bool* empty) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d <= 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  *empty = (B == 0 || H == 0 || N == 0);
  if (*empty) return FA_OK;
  // Every launch has at most one workgroup per 64 rows of each head; the
  // grid must fit in 31 bits.  (Element offsets are computed in 64 bits.)
  const long long heads = (long long)B * H;
  if (heads * ((N + 63) / 64) > 0x7fffffffLL) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int tensor_ok(const void* p) { return p != nullptr && aligned(p, 16); }

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Grouped K/V heads: Hkv must divide H (checked once the shape is non-empty).
int check_groups(int H, int Hkv) {
  if (Hkv < 1 || Hkv > H || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int forward_common(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Hkv, int N, int d, float scale, int causal, const uint8_t* mask,
                   int mask_block, bool f32, void* stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, scale, &empty);
  if (st != FA_OK || empty) return st;
  if ((st = check_groups(H, Hkv)) != FA_OK) return st;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o)) return FA_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal ? 1 : 0, mask, mask_block, Hkv,
                1.f, 1.f, 1.f};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // do not report an earlier, unrelated error
  return hip_status(f32 ? fa::launch_fwd_f32(a, s) : fa::launch_fwd_bf16(a, s));
}

bool positive_finite(float x) { return isfinite(x) && x > 0.f; }

size_t workspace_size(int B, int H, int N, int d) {
  bool empty = false;
  if (check_shape(B, H, N, d, 1.0f, &empty) != FA_OK || empty) return 0;
  const size_t rows = (size_t)B * H * N;
  return (2 * rows * sizeof(float) + 255) / 256 * 256;  // D, then LSE * log2(e)
}

// Grouped-head backward: every dK/dV workgroup covers 128 keys of one K/V
// head, so with few K/V heads the grid is small (MQA at B1 N8192: 64
// workgroups for 256 CUs).  Each group's query heads are then split into S
// slices (the smallest divisor of H / Hkv that gives 512 workgroups, else
// H / Hkv), each writing fp32 partial dK/dV that a reduction sums in order.
constexpr int kDkdvKeys = 128;
constexpr long long kDkdvWorkgroups = 512;

int gqa_slices(int B, int H, int Hkv, int N) {
  const int G = H / Hkv;
  const long long base = (long long)((N + kDkdvKeys - 1) / kDkdvKeys) * B * Hkv;
  for (int sl = 1; sl < G; ++sl)
    if (G % sl == 0 && base * sl >= kDkdvWorkgroups) return sl;
  return G;
}

// Extra workspace bytes for the slices' partials (0 when there is one slice).
size_t gqa_part_bytes(int B, int H, int Hkv, int N, int d) {
  const int S = gqa_slices(B, H, Hkv, N);
  if (S <= 1) return 0;
  return 256 + 2 * (size_t)S * B * Hkv * N * d * sizeof(float);  // + alignment slack
}

int backward_common(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, float* dq, float* dk, float* dv, void* workspace,
                    size_t workspace_bytes, int B, int H, int Hkv, int N, int d, float scale,
                    int causal, const uint8_t* mask, int mask_block, void* stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, scale, &empty);
  if (st != FA_OK || empty) return st;
  if ((st = check_groups(H, Hkv)) != FA_OK) return st;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o) || !tensor_ok(dout) ||
      !tensor_ok(dq) || !tensor_ok(dk) || !tensor_ok(dv))
    return FA_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  if (workspace == nullptr || !aligned(workspace, 4) ||
      workspace_bytes < workspace_size(B, H, N, d))
    return FA_ERR_INVALID_ARG;
  fa::BwdArgs a{q,  k,  v,  o,     dout,           lse,  dq,         dk, dv,
                static_cast<float*>(workspace), B, H, N, d, scale, causal ? 1 : 0,
                mask, mask_block, Hkv, nullptr, 1, nullptr};
  a.lse2 = a.delta + (size_t)B * H * N;
  if (Hkv != H) {
    const size_t base = workspace_size(B, H, N, d), part = gqa_part_bytes(B, H, Hkv, N, d);
    if (part > 0 && workspace_bytes >= base + part) {
      const uintptr_t p = (reinterpret_cast<uintptr_t>(workspace) + base + 255) & ~uintptr_t(255);
      a.gsplit = gqa_slices(B, H, Hkv, N);
      a.part = reinterpret_cast<float*>(p);
    }
  }
  (void)hipGetLastError();
  return hip_status(fa::launch_bwd_bf16(a, reinterpret_cast<hipStream_t>(stream)));
}

constexpr int kMaxDevices = 64;

// The device address of `scratch` on device `dev`.
int scratch_address(int dev, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return FA_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return FA_OK;
}

// Mask arguments: mask_block is checked first (so a bad block size is
// reported even for empty shapes), then a non-empty problem needs a mask.
int check_mask(int B, int H, int N, const uint8_t* block_mask, int mask_block) {
  if (mask_block != 128) return FA_ERR_UNSUPPORTED;
  if (B > 0 && H > 0 && N > 0 && block_mask == nullptr) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, void* stream) {
  return forward_common(q, k, v, o, lse, B, H, H, N, d, scale, causal, nullptr, 0, false,
                        stream);
}

int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                   int H, int N, int d, float scale, int causal, void* stream) {
  return forward_common(q, k, v, o, lse, B, H, H, N, d, scale, causal, nullptr, 0, true, stream);
}

int fa_forward_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, float scale, int causal,
                           const uint8_t* block_mask, int mask_block, void* stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, scale, &empty);
  if (st != FA_OK) return st;
  if ((st = check_mask(B, H, N, block_mask, mask_block)) != FA_OK) return st;
  return forward_common(q, k, v, o, lse, B, H, H, N, d, scale, causal, block_mask, mask_block,
                        false, stream);
}

int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int Hkv, int N, int d, float scale, int causal, void* stream) {
  if (Hkv < 0) return FA_ERR_INVALID_ARG;
  return forward_common(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, nullptr, 0, false,
                        stream);
}

int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int N, int d, float scale, float q_descale, float k_descale, float v_descale,
                   int causal, void* stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, scale, &empty);
  if (st != FA_OK) return st;
  if (!positive_finite(q_descale) || !positive_finite(k_descale) || !positive_finite(v_descale))
    return FA_ERR_INVALID_ARG;
  if (empty) return FA_OK;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o)) return FA_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal ? 1 : 0, nullptr, 0, H,
                q_descale, k_descale, v_descale};
  (void)hipGetLastError();
  return hip_status(fa::launch_fwd_fp8(a, reinterpret_cast<hipStream_t>(stream)));
}

size_t fa_backward_workspace_size(int B, int H, int N, int d) {
  return workspace_size(B, H, N, d);
}

size_t fa_backward_gqa_workspace_size(int B, int H, int Hkv, int N, int d) {
  bool empty = false;
  if (check_shape(B, H, N, d, 1.0f, &empty) != FA_OK || empty) return 0;
  if (check_groups(H, Hkv) != FA_OK) return 0;
  return workspace_size(B, H, N, d) + gqa_part_bytes(B, H, Hkv, N, d);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, float* dq, float* dk, float* dv, void* workspace,
                size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                void* stream) {
  return backward_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H,
                         N, d, scale, causal, nullptr, 0, stream);
}

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, float* dq, float* dk, float* dv,
                        int B, int H, int N, int d, float scale, int causal, void* stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, scale, &empty);
  if (st != FA_OK || empty) return st;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o) || !tensor_ok(dout) ||
      !tensor_ok(dq) || !tensor_ok(dk) || !tensor_ok(dv))
    return FA_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  if (workspace_size(B, H, N, d) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1;
  if ((s == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(s, &dev)) != hipSuccess)
    return FA_ERR_HIP;
  void* ws = nullptr;
  if ((st = scratch_address(dev, &ws)) != FA_OK) return st;
  return backward_common(q, k, v, o, dout, lse, dq, dk, dv, ws, FA_NOALLOC_SCRATCH_BYTES, B, H,
                         H, N, d, scale, causal, nullptr, 0, stream);
}

int fa_backward_blocksparse(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, float* dq, float* dk, float* dv,
                            void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                            float scale, int causal, const uint8_t* block_mask, int mask_block,
                            void* stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, scale, &empty);
  if (st != FA_OK) return st;
  if ((st = check_mask(B, H, N, block_mask, mask_block)) != FA_OK) return st;
  return backward_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, H,
                         N, d, scale, causal, block_mask, mask_block, stream);
}

int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, float* dq, float* dk, float* dv, void* workspace,
                    size_t workspace_bytes, int B, int H, int Hkv, int N, int d, float scale,
                    int causal, void* stream) {
  if (Hkv < 0) return FA_ERR_INVALID_ARG;
  return backward_common(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H,
                         Hkv, N, d, scale, causal, nullptr, 0, stream);
}

const char* fa_error_string(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or scale)";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration (head dim must be 64 or 128; mask block 128)";
    case FA_ERR_HIP: return "HIP runtime error at kernel launch";
    case FA_ERR_TOO_LARGE: return "problem too large for the fixed no-allocation scratch (B*H*N <= 1048576 rows)";
    default: return "unknown status";
  }
}

int fa_version(void) { return kVersion; }

int fa_runtime_version(void) {
  int v = -1;
  if (hipRuntimeGetVersion(&v) != hipSuccess) return -1;
  return v;
}

}  // extern "C"
