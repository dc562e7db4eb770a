// Internal launcher interface between the C ABI layer (fa_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa355 {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* kv_len;  // device int32[B] or nullptr
  int B, H, N, d;
  float scale_log2;  // scale * log2(e)
  int causal;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* kv_len;  // device int32[B] or nullptr
  float* dsum;            // workspace: D_i = rowsum(dO * O), fp32 [B][H][N]
  int B, H, N, d;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int causal;
};

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);

}  // namespace fa355
