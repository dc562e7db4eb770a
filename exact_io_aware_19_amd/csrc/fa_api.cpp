// C ABI of libfa355.so: host-side validation and dispatch.  Every check runs before
// any HIP call, so invalid calls return a negative status on any host (with or
// without a GPU) and enqueue nothing.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_kernels.hpp"

namespace {

// Library-owned scratch of the allocation-free backward: the row statistics the dQ pass
// writes and the dK/dV pass reads.  One copy per GPU, at its own address; host code
// uses only the address looked up by scratch_address(), never the array's name.
__device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the scratch array on the GPU of `stream` (the current GPU for the
// null stream), looked up once per GPU with that GPU current.
int scratch_address(fa_stream_t stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
  dev = cur;
  if (stream && hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return FA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return FA_ERR_LAUNCH;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return FA_ERR_LAUNCH;
    if (e != hipSuccess || !ptr) return FA_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  // B*H*N*d < 2^62 and the 1-D grid (query blocks x heads) fits 2^31
  const unsigned long long bh = (unsigned long long)B * (unsigned long long)H;
  if (bh > (1ull << 30)) return FA_ERR_SHAPE;
  const unsigned long long elems = bh * (unsigned long long)N * (unsigned long long)d;
  if (elems >= (1ull << 62)) return FA_ERR_SHAPE;
  // one head matrix ([N][d] bf16) is addressed through a 32-bit buffer resource
  if ((unsigned long long)N * (unsigned long long)d * 2ull >= (1ull << 32)) return FA_ERR_SHAPE;
  const unsigned long long qblocks = ((unsigned long long)N + 63) / 64;
  if (qblocks * bh >= (1ull << 31)) return FA_ERR_SHAPE;
  return FA_OK;
}

// any finite scale: negative and zero scales are carried by an operand's sign bits
int check_scale(float scale) { return isfinite(scale) ? FA_OK : FA_ERR_SCALE; }

int check_kv_heads(int H, int Hkv) { return (Hkv >= 1 && H % Hkv == 0) ? FA_OK : FA_ERR_KVHEADS; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Nk < 0: the square problem (Nk = N, query offset 0)
int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                 int d, float scale, int causal, const int32_t* kv_len, fa_stream_t stream, int Nk = -1,
                 int q_off = 0) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (Nk < 0) Nk = N;
  st = check_shape(B, H, Nk, d);
  if (st != FA_OK) return st;
  // causal positions q_off + row (+ a block) stay in int range
  if (q_off < 0 || (long long)q_off + N + 256 > 0x7fffffffLL) return FA_ERR_SHAPE;
  st = check_kv_heads(H, Hkv);
  if (st != FA_OK) return st;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u)) return FA_ERR_ALIGN;
  fa355::FwdArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.kv_len = kv_len;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.Nk = Nk;
  a.q_off = q_off;
  a.d = d;
  const fa355::ScaleSign sg = fa355::scale_sign(scale, fa355::kSignBitsBf16);
  a.scale_log2 = sg.scale_log2;
  a.op_and = sg.op_and;
  a.op_xor = sg.op_xor;
  a.causal = causal != 0;
  return fa355::launch_forward(a, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Rows per head in the backward workspace: N rounded up to the dQ pass's 256-row blocks.
int workspace_rows(int N) { return (N + 255) / 256 * 256; }

size_t stats_bytes(int B, int H, int N) {
  // -D_i and LSE_i * log2(e), fp32 [B][H][nw] each (a multiple of 2 KiB: the partials
  // that follow stay 256-byte aligned)
  return 2 * (size_t)B * H * workspace_rows(N) * 4;
}

size_t workspace_bytes(int B, int H, int Hkv, int N, int d) {
  // grouped K/V heads split over several workgroups: fp32 partial dK and dV per split
  const int ns = fa355::kv_splits(B, H, Hkv, N);
  const size_t parts = ns > 1 ? 2 * (size_t)ns * B * Hkv * N * d * 4 : 0;
  return stats_bytes(B, H, N) + parts;
}

int backward_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int causal,
                  const int32_t* kv_len, void* workspace, size_t ws_bytes, fa_stream_t stream, int passes = 3) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  st = check_kv_heads(H, Hkv);
  if (st != FA_OK) return st;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  if (!workspace || ws_bytes < workspace_bytes(B, H, Hkv, N, d)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 3u) || ((uintptr_t)workspace & 255u))
    return FA_ERR_ALIGN;
  fa355::BwdArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.kv_len = kv_len;
  a.nw = workspace_rows(N);
  a.ws_d = (float*)workspace;
  a.ws_l = (float*)workspace + (size_t)B * H * a.nw;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;  // signed: no row maximum in the backward
  a.causal = causal != 0;
  a.nsplit = fa355::kv_splits(B, H, Hkv, N);
  a.part = (float*)((char*)workspace + stats_bytes(B, H, N));
  return fa355::launch_backward(a, (hipStream_t)stream, passes) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, fa_stream_t stream) {
  return forward_impl(q, k, v, o, lse, B, H, H, N, d, scale, causal, nullptr, stream);
}

int fa_forward_kvlen(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                     float scale, int causal, const int32_t* kv_len, fa_stream_t stream) {
  return forward_impl(q, k, v, o, lse, B, H, H, N, d, scale, causal, kv_len, stream);
}

int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
                   int d, float scale, int causal, const int32_t* kv_len, fa_stream_t stream) {
  return forward_impl(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, kv_len, stream);
}

int fa_forward_offset(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                      int Nk, int d, float scale, int causal, int q_offset, const int32_t* kv_len,
                      fa_stream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (Nk < 1) return FA_ERR_SHAPE;  // (a negative Nk means the square problem internally)
  return forward_impl(q, k, v, o, lse, B, H, H, Nq, d, scale, causal, kv_len, stream, Nk, q_offset);
}

size_t fa_backward_workspace_size(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  return workspace_bytes(B, H, H, N, d);
}

size_t fa_backward_gqa_workspace_size(int B, int H, int H_kv, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK || check_kv_heads(H, H_kv) != FA_OK) return 0;
  return workspace_bytes(B, H, H_kv, N, d);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* workspace,
                size_t workspace_bytes_, fa_stream_t stream) {
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale, causal, nullptr, workspace,
                       workspace_bytes_, stream);
}

int fa_backward_kvlen(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                      const int32_t* kv_len, void* workspace, size_t workspace_bytes_, fa_stream_t stream) {
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale, causal, kv_len, workspace,
                       workspace_bytes_, stream);
}

int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int causal,
                    const int32_t* kv_len, void* workspace, size_t workspace_bytes_, fa_stream_t stream) {
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale, causal, kv_len, workspace,
                       workspace_bytes_, stream);
}

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                        int causal, const int32_t* kv_len, fa_stream_t stream) {
  // every argument check of fa_backward_kvlen, and the size limit, before any HIP call
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  if (workspace_bytes(B, H, H, N, d) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 3u))
    return FA_ERR_ALIGN;
  void* ws = nullptr;
  st = scratch_address(stream, &ws);
  if (st != FA_OK) return st;
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale, causal, kv_len, ws,
                       (size_t)FA_NOALLOC_SCRATCH_BYTES, stream);
}

int fa_backward_dq_pass(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                        int causal, const int32_t* kv_len, void* workspace, size_t workspace_bytes_,
                        fa_stream_t stream) {
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale, causal, kv_len, workspace,
                       workspace_bytes_, stream, 1);
}

int fa_backward_dkdv_pass(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                          int causal, const int32_t* kv_len, void* workspace, size_t workspace_bytes_,
                          fa_stream_t stream) {
  return backward_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale, causal, kv_len, workspace,
                       workspace_bytes_, stream, 2);
}

int fa_fp8_quantize_qk(const void* x, uint8_t* x8, float* scales, const float* signs, float post_scale, int B, int H,
                       int N, int d, fa_stream_t stream) {
  if (!x || !x8 || !scales) return FA_ERR_NULL;
  const int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!isfinite(post_scale) || !(post_scale > 0.f)) return FA_ERR_SCALE;
  if (!aligned16(x) || !aligned16(x8) || ((uintptr_t)scales & 3u) || ((uintptr_t)signs & 3u)) return FA_ERR_ALIGN;
  return fa355::launch_fp8_quantize_rows((const uint16_t*)x, x8, scales, signs, post_scale, B, H, N, d,
                                         (hipStream_t)stream) == hipSuccess
             ? FA_OK
             : FA_ERR_LAUNCH;
}

int fa_fp8_quantize_v(const void* v, uint8_t* v8t, float* scales, int B, int H, int N, int d, fa_stream_t stream) {
  if (!v || !v8t || !scales) return FA_ERR_NULL;
  const int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(v) || !aligned16(v8t) || ((uintptr_t)scales & 3u)) return FA_ERR_ALIGN;
  return fa355::launch_fp8_quantize_v((const uint16_t*)v, v8t, scales, B, H, N, d, (hipStream_t)stream) == hipSuccess
             ? FA_OK
             : FA_ERR_LAUNCH;
}

int fa_forward_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                   const uint8_t* v8t, const float* v_scale, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, const int32_t* kv_len, fa_stream_t stream) {
  if (!q8 || !q_scale || !k8 || !k_scale || !v8t || !v_scale || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  st = check_scale(scale);
  if (st != FA_OK) return st;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o) || ((uintptr_t)lse & 3u) ||
      ((uintptr_t)q_scale & 3u) || ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u))
    return FA_ERR_ALIGN;
  fa355::Fp8FwdArgs a;
  a.q8 = q8;
  a.sq = q_scale;
  a.k8 = k8;
  a.sk = k_scale;
  a.v8t = v8t;
  a.sv = v_scale;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.kv_len = kv_len;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  const fa355::ScaleSign sg = fa355::scale_sign(scale, fa355::kSignBitsE4m3);
  a.scale_log2 = sg.scale_log2;
  a.op_and = sg.op_and;
  a.op_xor = sg.op_xor;
  a.causal = causal != 0;
  return fa355::launch_forward_fp8(a, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: B, H or N < 1, or the problem is too large";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dim must be 64 or 128";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite (post_scale finite and > 0)";
    case FA_ERR_WORKSPACE:
      return "FA_ERR_WORKSPACE: workspace missing or too small (fa_backward_noalloc: problem beyond its scratch)";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not 16-byte aligned (lse 4, workspace 256)";
    case FA_ERR_KVHEADS: return "FA_ERR_KVHEADS: H_kv must be >= 1 and divide H";
    default: return "unknown fa_status";
  }
}

}  // extern "C"
