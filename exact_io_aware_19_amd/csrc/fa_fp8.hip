// FP8 attention forward for gfx950 (MI355X), with its quantisers.
//
// The FlashAttention-3 generation runs the forward in FP8 with block quantisation and
// incoherent processing, FP8 inputs with FP32 accumulation ("FlashAttention" concept
// wiki page, section FA3 (3), and the cross-cutting insight on FP8 stability).  Here:
//   * Q and K: one fp32 scale per block of 64 rows of a head; optionally the rows are
//     first multiplied by diag(signs) and the unnormalised Walsh-Hadamard matrix
//     (incoherent processing: outliers are spread over all head-dimension columns, and
//     Q K^T only changes by the factor d, which goes into Q's scales);
//   * V: one fp32 scale per (head, column), written transposed per 64-key tile in the
//     key order the P V product consumes;
//   * the forward: S^T = K Q^T and O^T += V^T P^T on the gfx950 fp8 MFMA
//     (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales: 64-deep contraction, twice
//     the bf16 rate), P rounded to OCP E4M3 in registers.  The block scales of Q and K
//     fold into the softmax's one multiplier per tile, V's column scales into the final
//     normalisation, so quantisation costs no work in the inner loop.
// The online softmax, masks, tile skipping and block order are those of the bf16
// forward.  Format: OCP E4M3 (bias 7, largest finite 448, subnormals); conversions
// round to nearest even (v_cvt_pk_fp8_f32, checked on gfx950 against the format's
// definition), inputs clamped to +-448 first.
#include <float.h>
#include <type_traits>

#include "common.hpp"
#include "fa_kernels.hpp"

namespace fa355 {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.f;
constexpr int kTileKeys = 64;  // keys per K/V tile = rows per Q/K scale block
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // query rows per workgroup
// Conditional rescaling threshold and exponent bias (log2 units).  P = exp2(t - m + kBias)
// with the reference max m at most kTau below the true max: P < 2^(kTau + kBias) = 256
// stays inside E4M3's 448, and the largest P of a row is at least 2^kBias, which keeps
// the row's main terms out of E4M3's subnormal range (below 2^-6).
constexpr float kTau = 4.0f;
constexpr float kBias = 4.0f;
constexpr float kPLimit = 256.0f;  // 2^(kTau + kBias)

// fp8 x fp8 -> fp32, 32x32x64.  Operand layout (probed on gfx950): lane l supplies row
// (A) or column (B) l % 32 and contraction slots 32*(l/32) .. +31, one per byte; C as
// in the bf16 32x32x16 product.  Scale operands 0 select unit scales.
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 join8(const u32x4& lo, const u32x4& hi) {
  i32x8 r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// Four fp32 -> four E4M3 bytes (a in the lowest byte), round to nearest even.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float clamp_e4m3(float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Key of byte p (0..31) in half h of a 64-key tile, in the order the P V product
// consumes it: P's byte p of a lane in half h comes from C register r = p % 16 of the
// score block p / 16, which holds key 8*(r/4) + 4*h + r%4 of that 32-key block.
__device__ __forceinline__ constexpr int pv_key(int h, int p) {
  return 32 * (p >> 4) + 8 * ((p & 15) >> 2) + 4 * h + (p & 3);
}

// ---------------------------------------------------------------------------------
// Q / K block quantisation: one wave per block of 64 rows, one row per lane.
// ---------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void fp8_quant_rows_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ x8,
                                                             float* __restrict__ scales, const float* __restrict__ signs,
                                                             float post_scale, int N, int nb) {
  const int blk = (int)(blockIdx.x % (unsigned)nb);
  const size_t bh = blockIdx.x / (unsigned)nb;
  const int l = threadIdx.x;
  const int row = blk * kTileKeys + l;
  const bool ok = row < N;
  float y[D];
  const uint16_t* src = x + (bh * N + (ok ? row : 0)) * D;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    u32x4 t = *(const u32x4*)(src + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[8 * c + 2 * i] = ok ? bf16_lo(t[i]) : 0.f;
      y[8 * c + 2 * i + 1] = ok ? bf16_hi(t[i]) : 0.f;
    }
  }
  if (signs != nullptr) {
#pragma unroll
    for (int i = 0; i < D; ++i) y[i] *= signs[i];
    // fast Walsh-Hadamard butterflies, stage h = 1, 2, ..., D/2: (a, b) -> (a + b, a - b)
#pragma unroll
    for (int h = 1; h < D; h <<= 1)
#pragma unroll
      for (int i = 0; i < D; ++i)
        if ((i & h) == 0) {
          const float a = y[i], b = y[i + h];
          y[i] = a + b;
          y[i + h] = a - b;
        }
  }
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < D; ++i) am = fmaxf(am, fabsf(y[i]));
  am = wave_max(am);
  const float inv = am > 0.f ? kE4M3Max / am : 0.f;
  if (l == 0) scales[bh * nb + blk] = am > 0.f ? (am / kE4M3Max) * post_scale : 0.f;
  if (ok) {
    uint8_t* dst = x8 + (bh * N + row) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 out;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* v = y + 16 * c + 4 * i;
        out[i] = pack_fp8x4(clamp_e4m3(v[0] * inv), clamp_e4m3(v[1] * inv), clamp_e4m3(v[2] * inv),
                            clamp_e4m3(v[3] * inv));
      }
      *(u32x4*)(dst + 16 * c) = out;
    }
  }
}

// ---------------------------------------------------------------------------------
// V column quantisation, four launches:
//  0. zero the scale output;
//  1. column amax, 256 rows of one head per workgroup, merged with atomic max into the
//     scale output;
//  2. quantise and transpose one 64-key tile per workgroup: V8T[bh][tile][d][64] with
//     byte 32*h + p of row d = code of V[tile*64 + pv_key(h, p)][d] (zero past N);
//  3. amax -> scale = amax / 448 in place.
// (The zeroing is a kernel, not a memset, so the sequence may be captured in a graph.)
// ---------------------------------------------------------------------------------
// Column amax over 256 rows of one head per workgroup: 16-byte chunks, D/8 lanes per row
// (each row read as one contiguous segment), a tree over the rows in LDS, then one
// atomic max per column into amax (zeroed before; non-negative fp32 values order like
// their bit patterns, so the unsigned max is the float max and the result does not
// depend on the order of the workgroups).
constexpr int kColmaxRows = 256;
template <int D>
__global__ __launch_bounds__(256) void fp8_v_colmax_kernel(const uint16_t* __restrict__ v, float* __restrict__ amax,
                                                            int N, int nchunks) {
  constexpr int NCH = D / 8;            // lanes per row
  constexpr int RPP = 256 / NCH;        // rows per pass
  const int chunk = (int)(blockIdx.x % (unsigned)nchunks);
  const size_t bh = blockIdx.x / (unsigned)nchunks;
  const int t = threadIdx.x, ch = t % NCH, r0 = t / NCH;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* base = v + bh * N * D + 8 * ch;
  const int row_end = min(N, (chunk + 1) * kColmaxRows);
  for (int r = chunk * kColmaxRows + r0; r < row_end; r += RPP) {
    const u32x4 w = *(const u32x4*)(base + (size_t)r * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[2 * i] = fmaxf(m[2 * i], fabsf(bf16_lo(w[i])));
      m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(bf16_hi(w[i])));
    }
  }
  __shared__ float red[RPP][D + 4];
#pragma unroll
  for (int i = 0; i < 8; ++i) red[r0][8 * ch + i] = m[i];
  __syncthreads();
  for (int c = t; c < D; c += 256) {
    float x = 0.f;
    for (int r = 0; r < RPP; ++r) x = fmaxf(x, red[r][c]);
    atomicMax((unsigned int*)(amax + bh * D + c), __float_as_uint(x));
  }
}

__global__ __launch_bounds__(256) void fp8_zero_kernel(float* s, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) s[i] = 0.f;
}

template <int D>
__global__ __launch_bounds__(256) void fp8_v_quant_t_kernel(const uint16_t* __restrict__ v,
                                                             const float* __restrict__ amax,
                                                             uint8_t* __restrict__ v8t, int N, int ntiles) {
  const int tile = (int)(blockIdx.x % (unsigned)ntiles);
  const size_t bh = blockIdx.x / (unsigned)ntiles;
  const int t = threadIdx.x;
  __shared__ uint16_t vs[kTileKeys][D + 8];  // +8: rows 16 bytes apart in the bank map
  __shared__ float inv[D];
  for (int i = t; i < D; i += 256) {
    const float a = amax[bh * D + i];
    inv[i] = a > 0.f ? kE4M3Max / a : 0.f;
  }
  constexpr int NCH = D / 8;
  for (int u = t; u < kTileKeys * NCH; u += 256) {
    const int r = u / NCH, c = u % NCH;
    const int key = tile * kTileKeys + r;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (key < N) w = *(const u32x4*)(v + (bh * N + key) * D + 8 * c);
    *(u32x4*)&vs[r][8 * c] = w;
  }
  __syncthreads();
  // output row d holds 64 bytes = 4 units of 16; unit q: half h = q / 2, bytes p = 16*(q%2) + 0..15
  uint8_t* dst = v8t + (bh * ntiles + tile) * (size_t)(D * kTileKeys);
  for (int u = t; u < D * 4; u += 256) {
    const int d = u >> 2, q = u & 3, h = q >> 1;
    const float s = inv[d];
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = 16 * (q & 1) + 4 * i + j;
        const uint32_t bits = (uint32_t)vs[pv_key(h, p)][d] << 16;
        f[j] = clamp_e4m3(__builtin_bit_cast(float, bits) * s);
      }
      out[i] = pack_fp8x4(f[0], f[1], f[2], f[3]);
    }
    *(u32x4*)(dst + 16 * u) = out;
  }
}

__global__ __launch_bounds__(256) void fp8_amax_to_scale_kernel(float* s, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) s[i] = s[i] > 0.f ? s[i] / kE4M3Max : 0.f;
}

// ---------------------------------------------------------------------------------
// Forward.  One workgroup = 4 waves (one per SIMD) = 128 query rows, 32 per wave, and
// three workgroups per CU (166-168 registers per wave): the three waves that share a
// SIMD belong to different workgroups, so no barrier holds them in step and one's
// softmax runs beside another's products.  Measured (B=2, H=16, N=8192, d=128, one box):
// this straight tile loop at three waves per SIMD 0.60 ms, 3-4% less with the loop run
// in pairs of tiles (below); one 8-wave workgroup of 256 rows per CU 0.70; two 4-wave
// workgroups per CU with the next tile's score products issued under the softmax 0.65;
// an explicit phase-offset ping-pong of two wave groups 0.79.  K and V^T tiles of 64 keys (fp8) are double-buffered in LDS, filled by direct
// buffer -> LDS copies that overlap the previous tile's products.
//
// LDS tile layouts (16-byte units, XOR-swizzled so that the 16 lanes of an operand
// read hit 16 different bank groups):
//   K tile  [64 keys][D bytes]: unit (r, j) at r*U + (j ^ ((r / (16/U)) % U)), U = D/16
//   V^T tile [D][64 bytes]:     unit (d, j) at d*4 + (j ^ ((d / 4) % 4))
// ---------------------------------------------------------------------------------
template <int U>
__device__ __forceinline__ constexpr uint32_t k_unit(uint32_t r, uint32_t j) {
  return r * U + (j ^ ((r / (16 / U)) % U));
}
__device__ __forceinline__ constexpr uint32_t vt_unit(uint32_t d, uint32_t j) { return d * 4 + (j ^ ((d >> 2) & 3)); }

template <int D, bool CAUSAL, bool KVLEN>
__global__ __launch_bounds__(kThreads, 3) void fa_fwd_fp8_kernel(Fp8FwdArgs p) {
  constexpr int U = D / 16;                 // 16-byte units per K row
  constexpr int KT_UNITS = kTileKeys * U;   // K tile
  constexpr int VT_UNITS = D * 4;           // V^T tile
  constexpr int BUF_BYTES = (KT_UNITS + VT_UNITS) * 16;
  constexpr int NKK = D / 64;  // k-steps of S^T = K Q^T
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int COPIES = (KT_UNITS + VT_UNITS) / 64 / kWaves;  // copy instructions per wave per tile
  static_assert(COPIES * 64 * kWaves == KT_UNITS + VT_UNITS, "tile copy must split over the waves");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * BUF_BYTES];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, c = l & 31, h = l >> 5;
  const int BH = p.B * p.H;
  const int N = p.N;
  const int nqb = (N + kBM - 1) / kBM;
  const int ntk = (N + kTileKeys - 1) / kTileKeys;  // key tiles = scale blocks per head
  int blk, bh;
  block_order<!CAUSAL>((int)blockIdx.x, nqb, BH, blk, bh);
  const int qbi = CAUSAL ? (nqb - 1 - blk) : blk;
  const int b = bh / p.H;
  const size_t head = (size_t)bh * N * D;

  int kv_end = N;
  if constexpr (KVLEN) kv_end = min(max(p.kv_len[b], 0), N);
  const int q0 = qbi * kBM;
  const int qrow = q0 + w * kRowsPerWave + c;
  int kend = kv_end;
  if constexpr (CAUSAL) kend = min(kend, q0 + kBM);
  const int ntiles = (kend + kTileKeys - 1) / kTileKeys;
  int wave_kend = kend;
  if constexpr (CAUSAL) wave_kend = min(kend, q0 + w * kRowsPerWave + kRowsPerWave);

  if (ntiles == 0) {
    if (qrow < N) {
      f32x16 zero[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) zero[db] = f32x16{};
      store_ct_rows<D>(p.o + head, qrow, zero, 0.f, h);
      if (h == 0) p.lse[(size_t)bh * N + qrow] = -INFINITY;
    }
    return;
  }

  // Q fragments: B operand of S^T, query column c, head-dim bytes 64*kk + 32*h .. +31
  i32x8 qf[NKK];
  {
    const bool ok = qrow < N;
    const uint8_t* src = p.q8 + head + (size_t)(ok ? qrow : 0) * D + 32 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 lo = *(const u32x4*)(src + 64 * kk);
      const u32x4 hi = *(const u32x4*)(src + 64 * kk + 16);
      // sign of the scale: E4M3 sign bits flipped (scale < 0) or codes zeroed (scale = 0)
      qf[kk] = ok ? ((join8(lo, hi) & (int)p.op_and) ^ (int)p.op_xor) : i32x8{};
    }
  }
  // the wave's 32 rows lie in one 64-row scale block of Q
  const float sq = p.sq[(size_t)bh * ntk + min((q0 + w * kRowsPerWave) / kTileKeys, ntk - 1)];
  const float* sk = p.sk + (size_t)bh * ntk;

  const buf_rsrc kg = make_rsrc(p.k8 + head, (uint32_t)N * D);
  const buf_rsrc vg = make_rsrc(p.v8t + (size_t)bh * ntk * D * kTileKeys, (uint32_t)ntk * D * kTileKeys);
  // tile copy: instruction ii of wave w fills units [64*g, 64*g + 64), g = ii*kWaves + w, of
  // the buffer (K tile units first, then V^T units); lane l fills unit 64*g + l with the
  // 16 bytes the swizzle puts there
  auto copy_tile = [&](int j, unsigned char* buf) {
#pragma unroll
    for (int ii = 0; ii < COPIES; ++ii) {
      const int g = ii * kWaves + w;
      const int u = 64 * g + l;
      unsigned char* dst = buf + (size_t)__builtin_amdgcn_readfirstlane(64 * g) * 16;
      if (64 * g < KT_UNITS) {  // wave-uniform
        const int r = u / U, jj = (u % U) ^ ((r / (16 / U)) % U);
        const int row = min(j * kTileKeys + r, N - 1);
        buf2lds16(kg, (uint32_t)(row * D + 16 * jj), 0u, dst);
      } else {
        const int v = u - KT_UNITS;
        const int d = v >> 2, jj = (v & 3) ^ ((d >> 2) & 3);
        const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)j * (D * kTileKeys));
        buf2lds16(vg, (uint32_t)(d * 64 + 16 * jj), soff, dst);
      }
    }
  };
  // per-lane fragment byte offsets (the swizzle term depends only on the lane's row)
  uint32_t kfr[2][NKK][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int s = 0; s < 2; ++s) kfr[kb][kk][s] = k_unit<U>(32 * kb + c, 4 * kk + 2 * h + s) * 16;
  uint32_t vfr[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int s = 0; s < 2; ++s) vfr[db][s] = (KT_UNITS + vt_unit(32 * db + c, 2 * h + s)) * 16;

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // reference max (scaled log2 units), at most kTau below the true max
  float l_run = 0.f;        // this lane's half of the row sum of P (unrounded, biased by 2^kBias)
  const float sl_q = p.scale_log2 * sq;

  copy_tile(0, smem);
  wait_vmem();
  __syncthreads();
  // tiles run in pairs so that the LDS buffer of each tile is a compile-time constant:
  // fragment addresses are then per-lane bases plus immediate offsets
  auto tile_step = [&](int j, auto par_c) {
    constexpr int PAR = decltype(par_c)::value;
    unsigned char* cur = smem + PAR * BUF_BYTES;
    if (j + 1 < ntiles) copy_tile(j + 1, smem + (1 - PAR) * BUF_BYTES);
    const int kt0 = j * kTileKeys;
    if (kt0 < wave_kend) {
      // S^T = K_j Q^T, two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const i32x8 a = join8(lds_read128(cur, kfr[kb][kk][0]), lds_read128(cur, kfr[kb][kk][1]));
          s[kb] = mfma_fp8(a, qf[kk], s[kb]);
        }
      }
      // online softmax; the block scales of Q and K fold into the one multiplier (where
      // a scale is 0 the scores are exactly 0, and FLT_MIN keeps -inf masks at -inf)
      const float sl = fmaxf(sl_q * sk[j], FLT_MIN);
      bool need_mask = kt0 + kTileKeys > kv_end;
      if constexpr (CAUSAL) need_mask = need_mask || (kt0 + kTileKeys - 1 > q0 + w * kRowsPerWave);
      if (need_mask) {
        // the limit is opaque here: otherwise the compiler sees that no key is past it
        // on tiles that need no mask and runs the selects on every tile
        int lim = kv_end;
        asm volatile("" : "+s"(lim));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
            bool bad = key >= lim;
            if constexpr (CAUSAL) bad = bad || key > qrow;
            s[kb][r] = bad ? -INFINITY : s[kb][r];
          }
      }
      // P^T as the B operand: byte p of half h is key pv_key(h, p) = register p % 16 of
      // score block p / 16.  P is first formed against the current reference; each P is
      // at most its lane's share of the tile sum, so when no share exceeds 2^(kTau +
      // kBias) (and every row has a reference) the reference stays and the row max is
      // not needed; otherwise the row max over the raw scores (s keeps them) decides as
      // usual.  The sum runs in four partial chains, which keeps the registers within the
      // budget of three waves per SIMD.
      i32x8 pk;
      auto probs = [&](float m_ref) {
        const float m_use = m_ref - kBias;
        float t[4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int kb = i >> 2, r0 = 4 * (i & 3);
          float e[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) e[x] = fast_exp2(__builtin_fmaf(s[kb][r0 + x], sl, -m_use));
          pk[i] = (int)pack_fp8x4(e[0], e[1], e[2], e[3]);
          const float q = (e[0] + e[1]) + (e[2] + e[3]);
          t[i & 3] = i < 4 ? q : t[i & 3] + q;
        }
        return (t[0] + t[1]) + (t[2] + t[3]);
      };
      float lt = probs((m_run == -INFINITY) ? 0.f : m_run);
      if (__any(!(lt <= kPLimit) || m_run == -INFINITY)) {
        float mx = tree_max<2>(s);
        mx = half_max(mx) * sl;
        if (__any(mx > m_run + kTau)) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = fast_exp2(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db] *= alpha;
          lt = probs((m_run == -INFINITY) ? 0.f : m_run);
        }
      }
      l_run += lt;
      // O^T += V_j^T P^T
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const i32x8 a = join8(lds_read128(cur, vfr[db][0]), lds_read128(cur, vfr[db][1]));
        o[db] = mfma_fp8(a, pk, o[db]);
      }
    }
    wait_vmem();
    __syncthreads();
    };
  for (int j = 0; j < ntiles; j += 2) {
    tile_step(j, std::integral_constant<int, 0>{});
    if (j + 1 < ntiles) tile_step(j + 1, std::integral_constant<int, 1>{});
  }

  // epilogue: normalise once, apply V's column scales, store O and LSE
  const float l_tot = half_sum(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  if (qrow < N) {
    const float* sv = p.sv + (size_t)bh * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= sv[32 * db + 8 * (r >> 2) + 4 * h + (r & 3)];
    store_ct_rows<D>(p.o + head, qrow, o, inv, h);
    if (h == 0) p.lse[(size_t)bh * N + qrow] = empty ? -INFINITY : (m_run - kBias + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool KVLEN>
hipError_t launch_fp8_one(const Fp8FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.N + kBM - 1) / kBM;
  const unsigned grid = (unsigned)nqb * (unsigned)(a.B * a.H);
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, KVLEN>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_fp8(const Fp8FwdArgs& a, hipStream_t s) {
  const bool kv = a.kv_len != nullptr;
  if (a.causal) return kv ? launch_fp8_one<D, true, true>(a, s) : launch_fp8_one<D, true, false>(a, s);
  return kv ? launch_fp8_one<D, false, true>(a, s) : launch_fp8_one<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_forward_fp8(const Fp8FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return dispatch_fp8<128>(a, stream);
  return dispatch_fp8<64>(a, stream);
}

hipError_t launch_fp8_quantize_rows(const uint16_t* x, uint8_t* x8, float* scales, const float* signs,
                                    float post_scale, int B, int H, int N, int d, hipStream_t stream) {
  const int nb = (N + kTileKeys - 1) / kTileKeys;
  const unsigned grid = (unsigned)nb * (unsigned)(B * H);
  if (d == 128)
    hipLaunchKernelGGL(fp8_quant_rows_kernel<128>, dim3(grid), dim3(64), 0, stream, x, x8, scales, signs, post_scale,
                       N, nb);
  else
    hipLaunchKernelGGL(fp8_quant_rows_kernel<64>, dim3(grid), dim3(64), 0, stream, x, x8, scales, signs, post_scale,
                       N, nb);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_v(const uint16_t* v, uint8_t* v8t, float* scales, int B, int H, int N, int d,
                                 hipStream_t stream) {
  const int nt = (N + kTileKeys - 1) / kTileKeys;
  const unsigned bh = (unsigned)(B * H);
  const int nchunks = (N + kColmaxRows - 1) / kColmaxRows;
  const size_t n = (size_t)bh * d;
  hipLaunchKernelGGL(fp8_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, scales, n);
  if (d == 128) {
    hipLaunchKernelGGL(fp8_v_colmax_kernel<128>, dim3(bh * (unsigned)nchunks), dim3(256), 0, stream, v, scales, N,
                       nchunks);
    hipLaunchKernelGGL(fp8_v_quant_t_kernel<128>, dim3(bh * (unsigned)nt), dim3(256), 0, stream, v, scales, v8t, N,
                       nt);
  } else {
    hipLaunchKernelGGL(fp8_v_colmax_kernel<64>, dim3(bh * (unsigned)nchunks), dim3(256), 0, stream, v, scales, N,
                       nchunks);
    hipLaunchKernelGGL(fp8_v_quant_t_kernel<64>, dim3(bh * (unsigned)nt), dim3(256), 0, stream, v, scales, v8t, N,
                       nt);
  }
  hipLaunchKernelGGL(fp8_amax_to_scale_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, scales, n);
  return hipGetLastError();
}

}  // namespace fa355
