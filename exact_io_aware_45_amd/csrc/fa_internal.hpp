// fa_internal.hpp -- host-side launch interface between the C ABI (fa_api.hip)
// and the kernel translation units.  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Problem description shared by every forward launch.  Q, O are contiguous
// [B][H][N][d], K, V [B][Hkv][N][d] (Hkv divides H; query head h reads K/V
// head h / (H / Hkv)); lse is [B][H][N] fp32.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal;
  const uint8_t* mask;  // tile mask [nmb][nmb] or nullptr
  int mask_block;       // tile edge of the mask (keys and queries)
  int Hkv;
  // fp8 inputs only: the real value of a stored element is element * descale.
  float q_descale, k_descale, v_descale;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* delta;  // workspace: -D_i = -(dO_i . O_i), [B][H][N] fp32
  int B, H, N, d;
  float scale;
  int causal;
  const uint8_t* mask;  // tile mask [nmb][nmb] or nullptr
  int mask_block;
  int Hkv;  // K, V, dK, dV are [B][Hkv][N][d]; dK/dV sum over the H/Hkv query heads
  float* lse2;  // workspace: LSE_i * log2(e), [B][H][N] fp32 (written with D)
  // Grouped heads: each group's query heads are split into gsplit slices of
  // H / Hkv / gsplit heads, one dK/dV workgroup per slice; with gsplit > 1
  // the slices write fp32 partial dK (slots 0 .. gsplit-1) and dV (slots
  // gsplit .. 2 gsplit-1), each [B][Hkv][N][d], to `part`, and a reduction
  // sums them in slot order.
  int gsplit;
  float* part;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
bool fwd128_applies(const FwdArgs& a);
hipError_t launch_fwd128(const FwdArgs& a, hipStream_t s);
bool fwd64_applies(const FwdArgs& a);
hipError_t launch_fwd64(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s);
bool dq128_applies(const BwdArgs& a);
hipError_t launch_dq128(const BwdArgs& a, hipStream_t s);
bool dkdv128_applies(const BwdArgs& a);
hipError_t launch_dkdv128(const BwdArgs& a, hipStream_t s);

}  // namespace fa
