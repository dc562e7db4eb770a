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
  int Hkv;           // K/V heads; query head h reads K/V head h / (H / Hkv)
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
  // workspace, written by the dQ pass and read by the dK/dV pass, per head nw rows
  // (N rounded up to 256; rows past N hold D = 0, lse2 = +inf):
  float* ws_d;  // D_i = rowsum(dO * O), fp32 [B][H][nw]
  float* ws_l;  // LSE_i * log2(e), +inf where the row has no admissible key, fp32 [B][H][nw]
  int nw;
  int B, H, N, d;
  int Hkv;           // K/V heads; query head h reads K/V head h / (H / Hkv)
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int causal;
  // grouped K/V heads with nsplit > 1: the query heads of a group are split over nsplit
  // workgroups per key block, which write fp32 partial dK, dV ([nsplit][B*Hkv][N][d]
  // each, dV right after dK) summed in a fixed order by a second kernel
  int nsplit;
  float* part;
};

// Key columns per dK/dV workgroup.
constexpr int kKvBlockKeys = 128;
// Workgroups a dK/dV launch aims for (two per CU); fewer key blocks x K/V heads than this
// split each group's query heads over several workgroups.
constexpr int kKvTargetBlocks = 512;

// Number of workgroups that share the query heads of one (key block, K/V head).
inline int kv_splits(int B, int H, int Hkv, int N) {
  if (Hkv >= H) return 1;
  const long long base = (long long)((N + kKvBlockKeys - 1) / kKvBlockKeys) * B * Hkv;
  const long long want = (kKvTargetBlocks + base - 1) / base;
  const int G = H / Hkv;
  return (int)(want < 1 ? 1 : (want > G ? G : want));
}

struct Fp8FwdArgs {
  const uint8_t* q8;   // E4M3 codes [B][H][N][d]
  const float* sq;     // Q block scales [B][H][ceil(N/64)]
  const uint8_t* k8;   // E4M3 codes [B][H][N][d]
  const float* sk;     // K block scales [B][H][ceil(N/64)]
  const uint8_t* v8t;  // E4M3 codes, transposed 64-key tiles [B][H][ceil(N/64)][d][64]
  const float* sv;     // V column scales [B][H][d]
  uint16_t* o;
  float* lse;
  const int32_t* kv_len;  // device int32[B] or nullptr
  int B, H, N, d;
  float scale_log2;  // scale * log2(e)
  int causal;
};

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);
hipError_t launch_forward_fp8(const Fp8FwdArgs& a, hipStream_t stream);
hipError_t launch_fp8_quantize_rows(const uint16_t* x, uint8_t* x8, float* scales, const float* signs,
                                    float post_scale, int B, int H, int N, int d, hipStream_t stream);
hipError_t launch_fp8_quantize_v(const uint16_t* v, uint8_t* v8t, float* scales, int B, int H, int N, int d,
                                 hipStream_t stream);
// passes: bit 0 = dQ pass (dq + row statistics), bit 1 = dK/dV pass
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream, int passes = 3);

}  // namespace fa355
