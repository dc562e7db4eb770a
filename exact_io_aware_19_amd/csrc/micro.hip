// Microbenchmarks of the gfx950 units the attention kernels are bound by: the bf16 MFMA
// rate the chip sustains (its clock under load included), the v_exp_f32 rate, LDS read
// bandwidth, fp32 global atomic throughput, MFMA/VALU co-execution on one SIMD and the issue
// rate of the forward's product order.  They measure the machine, not attention:
// the bench reports them beside the data-sheet peaks.  C ABI in include/fa_micro.h
// (libfa355_micro.so, a library of its own).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_micro.h"
#include "common.hpp"

namespace fa355 {
namespace {

constexpr int kMicroThreads = 256;  // 4 waves, one per SIMD
constexpr int kMicroBlocksPerCU = 2;

// Eight independent chains of v_mfma_f32_32x32x16_bf16 per wave; all SIMDs of the GPU run
// two such waves.  One product = 2*32*32*16 = 32768 FLOP.
__global__ __launch_bounds__(kMicroThreads, kMicroBlocksPerCU) void mfma_bf16_loop(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  // bf16 2^-10 (0x3A80) in every operand element: accumulators grow by 16 * 2^-20 per
  // product, far from overflow
  const u32x4 a = {0x3A803A80u, 0x3A803A80u, 0x3A803A80u, 0x3A803A80u};
  const u32x4 b = a;
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = mfma32(a, b, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[(size_t)blockIdx.x * kMicroThreads + tid] = s;
}

// Sixteen independent chains x <- exp2(-x) per lane (x stays in (0, 1]).
__global__ __launch_bounds__(kMicroThreads, kMicroBlocksPerCU) void exp_loop(float* __restrict__ out, int iters) {
  const int tid = threadIdx.x;
  float x[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = 0.25f + 0.03f * k + 1e-6f * tid;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += x[k];
  out[(size_t)blockIdx.x * kMicroThreads + tid] = s;
}

// 128-bit LDS reads: each wave reads 1 KiB contiguous per instruction (conflict free),
// eight reads in flight per lane, XOR-accumulated.  The window moves by 16 bytes per
// iteration so no read can be hoisted out of the loop; the largest byte read is
// 16*63 + 1024*3 + 16*63 + 4096*7 + 16 = 33776 < 40960.
constexpr uint32_t kMicroLdsBytes = 40960;
__global__ __launch_bounds__(kMicroThreads, kMicroBlocksPerCU) void lds_read_loop(float* __restrict__ out, int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char tile[kMicroLdsBytes];
  const int tid = threadIdx.x;
  for (uint32_t i = tid; i < kMicroLdsBytes / 16; i += kMicroThreads) {
    const u32x4 v = {i, i * 3u, i * 5u, i * 7u};
    lds_write128(tile, 16u * i, v);
  }
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint32_t base = 16u * (uint32_t)(tid & 63) + 1024u * (uint32_t)(tid >> 6);
  for (int i = 0; i < iters; ++i) {
    const uint32_t off = base + 16u * (uint32_t)(i & 63);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= lds_read128(tile, off + 4096u * (uint32_t)k);
  }
  out[(size_t)blockIdx.x * kMicroThreads + tid] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

// fp32 atomic adds of whole 64x128 tiles (32 KB), the pattern an atomic dQ accumulation
// would write: workgroup w adds `tiles` tiles at tile positions (w + t) % ntiles of buf.
__global__ __launch_bounds__(kMicroThreads) void atomic_tiles(float* __restrict__ buf, int ntiles, int tiles) {
  const int w = blockIdx.x;
  for (int t = 0; t < tiles; ++t) {
    float* tile = buf + (size_t)((w + t) % ntiles) * 64 * 128;
    for (int e = threadIdx.x; e < 64 * 128; e += kMicroThreads) atomicAdd(tile + e, 1.0f);
  }
}

// MFMA and VALU streams of different waves on one SIMD: 8-wave workgroups, one per CU,
// waves w and w + 4 on the same SIMD.  valu_kind 0, 1: waves 0-3 run the MFMA chains of
// mfma_bf16_loop (`mfma_iters` iterations) when mode bit 0 is set; waves 4-7 run 16
// independent chains per lane of `valu_iters` iterations when mode bit 1 is set:
// x <- exp2(-x) (valu_kind 0, v_exp_f32) or x <- fma(x, 0.999, 1e-4) (valu_kind 1,
// v_fma_f32).  valu_kind 2 (transcendental beside FMA): waves 0-3 run the exp chains
// (`mfma_iters` iterations, bit 0), waves 4-7 the FMA chains (`valu_iters`, bit 1).
// valu_kind 3 (both in one wave): waves 0-3 run the exp chains (`mfma_iters`, bit 0) and
// the FMA chains (`valu_iters`, bit 1) interleaved in one instruction stream; waves 4-7
// idle.  Timing the three modes shows how far the two streams overlap.
constexpr int kCoexThreads = 512;
__device__ __forceinline__ void exp_chains(float (&x)[16], int iters) {
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
  }
}
__device__ __forceinline__ void fma_chains(float (&x)[16], int iters) {
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 16; ++k) x[k] = __builtin_fmaf(x[k], 0.999f, 1e-4f);
  }
}
__device__ __forceinline__ float chain_sum(const float (&x)[16]) {
  float r = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) r += x[k];
  return r;
}
__global__ __launch_bounds__(kCoexThreads, 1) void coexec_loop(float* __restrict__ out, int mode, int valu_kind,
                                                               int mfma_iters, int valu_iters) {
  const int tid = threadIdx.x, w = tid >> 6;
  float* o = out + (size_t)blockIdx.x * kCoexThreads;
  float x[16], y[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) x[k] = y[k] = 0.25f + 0.03f * k + 1e-6f * (tid & 255);
  if (valu_kind == 3) {  // one wave, both streams interleaved
    if (w < 4) {
      int i = 0;
      if (mode == 3) {
        const int n = min(mfma_iters, valu_iters);
        for (; i < n; ++i) {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            x[k] = __builtin_amdgcn_exp2f(-x[k]);
            y[k] = __builtin_fmaf(y[k], 0.999f, 1e-4f);
          }
        }
      }
      if (mode & 1) exp_chains(x, mfma_iters - i);
      if (mode & 2) fma_chains(y, valu_iters - i);
      o[tid] = (mode & 1) ? chain_sum(x) : 0.f;
      o[256 + tid] = (mode & 2) ? chain_sum(y) : 0.f;
    }
    return;
  }
  float res = 0.f;
  if (w < 4) {
    if (mode & 1) {
      if (valu_kind == 2) {
        exp_chains(x, mfma_iters);
        res = chain_sum(x);
      } else {
        const u32x4 a = {0x3A803A80u, 0x3A803A80u, 0x3A803A80u, 0x3A803A80u};
        f32x16 acc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = f32x16{};
        for (int i = 0; i < mfma_iters; ++i) {
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[k] = mfma32(a, a, acc[k]);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int r = 0; r < 16; ++r) res += acc[k][r];
      }
    }
  } else if (mode & 2) {
    if (valu_kind == 0) exp_chains(x, valu_iters);
    else fma_chains(x, valu_iters);
    res = chain_sum(x);
  }
  o[tid] = res;
}

// Issue rate of 32 bf16 products per block in a given order, one wave per SIMD (a
// 256-thread workgroup per compute unit: 96 KiB of LDS keeps a second one off).  A
// operands are bf16 2^-10 (in registers, or in LDS for variant 3); accumulation chain k
// takes the B operand bf16 2^-10 (1 + k/128), so no two chains compute the same values
// (identical chains were merged by the compiler: 829 ticks per 32 products, below the
// 1024 the MFMA unit allows).  Lane 0 of each wave writes the s_memtime difference
// (shader-clock ticks) over the `iters` blocks.
//   0: 8 independent accumulation chains, 4 products each per block;
//   1: the forward's MFMA operation -- 16 P.V products over 4 accumulators (4 each),
//      then 16 score products over 2 accumulators (8 each, the first from C = 0);
//   2: as 1 with the scores over 4 accumulators (4 each, the first two from C = 0);
//   3: as 1 with every A operand read from LDS four products ahead (1 KiB per wave and
//      read, conflict free).
constexpr int kOrderLdsWords = 96 * 256;  // 96 KiB

__device__ __forceinline__ f32x16 mfma32_pinned(const u32x4& a, const u32x4& b, const f32x16& c) {
  const f32x16 d = mfma32(a, b, c);
  __builtin_amdgcn_sched_barrier(0);
  return d;
}

__global__ __launch_bounds__(kMicroThreads, 1) void mfma_order(unsigned long long* __restrict__ ticks,
                                                             float* __restrict__ sink, int variant, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t pad[kOrderLdsWords];
  const int tid = threadIdx.x;
  const u32x4 a = {0x3A803A80u, 0x3A803A80u, 0x3A803A80u, 0x3A803A80u};
  u32x4 b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t x = 0x3A80u + (uint32_t)k;  // bf16 2^-10 (1 + k/128)
    b[k] = u32x4{x | (x << 16), x | (x << 16), x | (x << 16), x | (x << 16)};
  }
  for (int e = tid; e < kOrderLdsWords; e += kMicroThreads) pad[e] = 0x3A803A80u;
  __syncthreads();
  f32x16 o[4], s[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[k] = f32x16{};
    s[k] = f32x16{};
  }
  float acc = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  if (variant == 0) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = mfma32_pinned(a, b[k], o[k]);
#pragma unroll
        for (int k = 0; k < 4; ++k) s[k] = mfma32_pinned(a, b[4 + k], s[k]);
      }
    }
  } else if (variant == 1) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = mfma32_pinned(a, b[db], o[db]);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32_pinned(a, b[4 + kb], kk == 0 ? f32x16{} : s[kb]);
      acc += s[0][0] + s[1][0];
    }
  } else if (variant == 2) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = mfma32_pinned(a, b[db], o[db]);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int x = kb + 2 * (kk & 1);
          s[x] = mfma32_pinned(a, b[4 + x], kk < 2 ? f32x16{} : s[x]);
        }
      acc += (s[0][0] + s[2][0]) + (s[1][0] + s[3][0]);
    }
  } else {
    // byte offsets: 16 * lane + 8192 * wave + 1024 * (j % 8) + 16 <= 32768 < 98304
    const unsigned char* base = (const unsigned char*)pad;
    const uint32_t lb = 16u * (tid & 63) + 8192u * (tid >> 6);
    for (int i = 0; i < iters; ++i) {
      u32x4 fr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) fr[j] = lds_read128(base, lb + 1024u * j);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const u32x4 av = fr[j & 3];
        if (j + 4 < 32) fr[j & 3] = lds_read128(base, lb + 1024u * ((j + 4) & 7));
        __builtin_amdgcn_sched_barrier(0);
        if (j < 16) {
          o[j & 3] = mfma32_pinned(av, b[j & 3], o[j & 3]);
        } else {
          const int kk = (j - 16) >> 1, kb = (j - 16) & 1;
          s[kb] = mfma32_pinned(av, b[4 + kb], kk == 0 ? f32x16{} : s[kb]);
        }
      }
      acc += s[0][0] + s[1][0];
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float r = acc;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += o[k][e] + s[k][e];
  sink[(size_t)blockIdx.x * kMicroThreads + tid] = r;
  if ((tid & 63) == 0) ticks[(size_t)blockIdx.x * 4 + (tid >> 6)] = t1 - t0;
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return n;
}


// One v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit scales) on one wave: C = A B^T
// + C0 for A, B of 32 rows x 64 bytes (row-major codes) and C0, C of 32 x 32 floats
// (row-major).  Operand layout: lane l supplies row l % 32 of A (and of B) and
// contraction slots 32 (l / 32) .. +31, one per byte; the accumulator element r of lane l
// is C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  Used to read the accumulation precision
// of the fp8 product.
typedef int i32x8m __attribute__((ext_vector_type(8)));
__global__ __launch_bounds__(64) void mfma_fp8_tile(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                    const float* __restrict__ c0, float* __restrict__ c) {
  const int l = threadIdx.x, row = l & 31, h = l >> 5;
  const uint32_t* ar = reinterpret_cast<const uint32_t*>(a + row * 64 + 32 * h);
  const uint32_t* br = reinterpret_cast<const uint32_t*>(b + row * 64 + 32 * h);
  i32x8m av, bv;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    av[k] = (int)ar[k];
    bv[k] = (int)br[k];
  }
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = c0[(8 * (r >> 2) + 4 * h + (r & 3)) * 32 + row];
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) c[(8 * (r >> 2) + 4 * h + (r & 3)) * 32 + row] = acc[r];
}

}  // namespace
}  // namespace fa355

extern "C" {

int fa_micro_grid_blocks(void) {
  const int n = fa355::cu_count();
  return n > 0 ? n * fa355::kMicroBlocksPerCU : -1;
}

int fa_micro_mfma_bf16(float* out, int blocks, int iters, fa_stream_t stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(fa355::mfma_bf16_loop, dim3(blocks), dim3(fa355::kMicroThreads), 0, (hipStream_t)stream, out,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int fa_micro_exp(float* out, int blocks, int iters, fa_stream_t stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(fa355::exp_loop, dim3(blocks), dim3(fa355::kMicroThreads), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int fa_micro_lds_read(float* out, int blocks, int iters, fa_stream_t stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(fa355::lds_read_loop, dim3(blocks), dim3(fa355::kMicroThreads), 0, (hipStream_t)stream, out,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int fa_micro_atomic_tiles(float* buf, int ntiles, int blocks, int tiles, fa_stream_t stream) {
  if (!buf || ntiles < 1 || blocks < 1 || tiles < 1) return -1;
  hipLaunchKernelGGL(fa355::atomic_tiles, dim3(blocks), dim3(fa355::kMicroThreads), 0, (hipStream_t)stream, buf,
                     ntiles, tiles);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int fa_micro_coexec(float* out, int blocks, int mode, int valu_kind, int mfma_iters, int valu_iters,
                    fa_stream_t stream) {
  if (!out || blocks < 1 || mode < 1 || mode > 3 || valu_kind < 0 || valu_kind > 3 || mfma_iters < 1 ||
      valu_iters < 1)
    return -1;
  hipLaunchKernelGGL(fa355::coexec_loop, dim3(blocks), dim3(fa355::kCoexThreads), 0, (hipStream_t)stream, out, mode,
                     valu_kind, mfma_iters, valu_iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int fa_micro_mfma_order(unsigned long long* ticks, float* sink, int blocks, int variant, int iters,
                        fa_stream_t stream) {
  if (!ticks || !sink || blocks < 1 || variant < 0 || variant > 3 || iters < 1) return -1;
  hipLaunchKernelGGL(fa355::mfma_order, dim3(blocks), dim3(fa355::kMicroThreads), 0, (hipStream_t)stream, ticks, sink,
                     variant, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int fa_micro_mfma_fp8_tile(const void* a, const void* b, const float* c0, float* c, fa_stream_t stream) {
  if (!a || !b || !c0 || !c) return -1;
  hipLaunchKernelGGL(fa355::mfma_fp8_tile, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a,
                     (const uint8_t*)b, c0, c);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
