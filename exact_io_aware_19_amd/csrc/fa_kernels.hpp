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
  int B, H, N, d;    // N: query rows per head (of q, o, lse)
  int Nk;            // key rows per head (of k, v); N for the square problem
  int q_off;         // position of query row 0 in the key sequence (causal: key j is
                     // admissible for query row i iff j <= q_off + i); 0 for the square problem
  int Hkv;           // K/V heads; query head h reads K/V head h / (H / Hkv)
  float scale_log2;  // |scale| * log2(e) (log2(e) when scale = 0)
  int causal;
  // sign of the scale, applied to every dword of the Q fragments: q = (q & op_and) ^ op_xor
  uint32_t op_and, op_xor;
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
  float* ws_d;  // -D_i, D_i = rowsum(dO * O), fp32 [B][H][nw]
  float* ws_l;  // LSE_i * log2(e), +inf where the row has no admissible key, fp32 [B][H][nw]
  int nw;
  int B, H, N, d;
  int Hkv;           // K/V heads; query head h reads K/V head h / (H / Hkv)
  float scale;       // softmax scale (multiplies dQ and dK at the store)
  // scale * log2(e), with its sign: the backward recomputes P = exp2(S * scale_log2 -
  // LSE * log2(e)) from the saved LSE and needs no row maximum, so any finite scale
  // (zero and negative included) enters as it is
  float scale_log2;
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
  float scale_log2;  // |scale| * log2(e) (log2(e) when scale = 0)
  int causal;
  uint32_t op_and, op_xor;  // sign of the scale, applied to every dword of the Q codes
};

// The kernels multiply scores by a positive factor only (the row maximum must commute
// with scaling) and take the sign of the softmax scale from one operand held in
// registers: for scale < 0 its sign bits are flipped (exact: -S = (-Q) K^T), for
// scale = 0 it is zeroed (S = 0 exactly: uniform weights over the admissible keys).
// `sign_bits` has the sign bit of every element of one dword set.
struct ScaleSign {
  float scale_log2;
  uint32_t op_and, op_xor;
};
inline ScaleSign scale_sign(float scale, uint32_t sign_bits) {
  constexpr float kLog2eHost = 1.4426950408889634f;
  if (scale > 0.f) return {scale * kLog2eHost, 0xffffffffu, 0u};
  if (scale < 0.f) return {-scale * kLog2eHost, 0xffffffffu, sign_bits};
  return {kLog2eHost, 0u, 0u};
}
constexpr uint32_t kSignBitsBf16 = 0x80008000u;
constexpr uint32_t kSignBitsE4m3 = 0x80808080u;

// Small d = 128 grids: the forward and the dQ pass then run 128-row workgroups whose
// two wave groups take the two halves of the key range (merged in LDS), instead of one
// 256-row workgroup per CU.  `grid8` is the unsplit launch's workgroup count (256 query
// rows each).  Taken where that grid leaves at least half of the CUs idle, or, with the
// causal mask (whose row blocks differ in cost), where it is at most one workgroup per
// CU; measured slower on fuller grids (the split kernels do the same work per tile with
// more per-workgroup overhead and no ping-pong of the two wave groups).
inline bool split_small_grid(unsigned grid8, bool causal) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus <= 0)
    return false;
  return 2 * grid8 <= (unsigned)cus || (causal && grid8 <= (unsigned)cus);
}

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);
hipError_t launch_forward_fp8(const Fp8FwdArgs& a, hipStream_t stream);
hipError_t launch_fp8_quantize_rows(const uint16_t* x, uint8_t* x8, float* scales, const float* signs,
                                    float post_scale, int B, int H, int N, int d, hipStream_t stream);
hipError_t launch_fp8_quantize_v(const uint16_t* v, uint8_t* v8t, float* scales, int B, int H, int N, int d,
                                 hipStream_t stream);
// passes: bit 0 = dQ pass (dq + row statistics), bit 1 = dK/dV pass
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream, int passes = 3);

}  // namespace fa355
