// Fused attention forward for gfx950 (MI355X).
//
// One workgroup = 8 waves (2 per SIMD) = 256 query rows; each wave owns 32 query rows
// for the whole kernel and streams key/value tiles of BN keys through LDS.  Per tile:
//   S^T = K_j Q^T        bf16 MFMA 32x32x16, fp32 accumulate (Q fragments stay in VGPRs)
//   online softmax       running row max m and row sum l in scaled-log2 units,
//                        earlier partials rescaled by exp2(m_old - m_new)
//   O^T += V_j^T P^T     P converted to bf16 in registers; V_j^T read from a
//                        transposed LDS copy
// so the N x N score matrix never leaves the chip ("FlashAttention" concept wiki page,
// section 定義 (1) tiling + online softmax; singularity-lens FA1 explainer, paragraphs
// on tiling and on the online softmax).  The output is normalised once at the end and
// only one log-sum-exp per row is stored (wiki page, FA2 (1): fewer non-matmul
// operations), which is all the backward pass needs to recompute P.
//
// Work is parallel over query blocks and heads (wiki page, FA2 (2)); each wave owns
// complete query rows so row statistics never cross waves (FA2 (3)).
#include "common.hpp"
#include "fa_kernels.hpp"

namespace fa355 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // query rows per workgroup

// K tile in LDS: [BN][D] bf16, 16-byte chunk c of row r stored at chunk c ^ swz_k(r).
// Reads (MFMA A operand) hit 16 consecutive rows at one logical chunk; the swizzle
// spreads them over 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ uint32_t swz_k(uint32_t row) {
  if constexpr (D == 128) return row & 15u;
  else return (row >> 1) & 7u;
}

// V^T tile in LDS: [D][BN] bf16 (row = head-dim index, 8 keys per 16-byte chunk).
// Reads hit 16 consecutive rows at one chunk; the 4x4-block transposed writes hit rows
// spaced by 4 -- the swizzle keeps both conflict-free.
template <int BN>
__device__ __forceinline__ uint32_t swz_v(uint32_t d) {
  if constexpr (BN == 64) return ((d >> 1) + (d >> 4)) & 7u;
  else return (d + (d >> 4)) & 15u;
}

// Row of K that lane c of the A operand supplies inside a 32-key block: bits 2 and 3
// of c swapped.  With it, score register r of lane (h = l/32) belongs to key
// 16*(r/8) + 8*h + (r%8), so each lane's eight consecutive score registers are eight
// consecutive keys -- exactly the k-slots that lane feeds to the P V^T product.
__device__ __forceinline__ uint32_t key_perm(uint32_t c) { return (c & ~12u) | ((c & 4u) << 1) | ((c & 8u) >> 1); }

template <int D, int BN, bool CAUSAL, bool KVLEN>
__global__ __launch_bounds__(kThreads) void fa_fwd_kernel(FwdArgs p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int KT_BYTES = BN * D * 2;  // one K tile, one V^T tile
  constexpr int NKB = BN / 32;          // 32-key blocks per tile
  constexpr int NDB = D / 32;           // 32-row blocks of the head dim
  constexpr int NKK = D / 16;           // k-steps of the QK^T contraction
  // LDS: K tiles at [0, 2*KT_BYTES), V^T tiles at [2*KT_BYTES, 4*KT_BYTES)
  auto kbuf = [&](int i) { return smem + i * KT_BYTES; };
  auto vbuf = [&](int i) { return smem + (2 + i) * KT_BYTES; };

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, c = l & 31, h = l >> 5;
  const int BH = p.B * p.H;
  const int nqb = (p.N + kBM - 1) / kBM;
  // Causal: heaviest query blocks first.  Consecutive workgroups take consecutive
  // heads, so every workgroup of one head lands on the same XCD when B*H % 8 == 0.
  const int qbi = CAUSAL ? (nqb - 1 - (int)(blockIdx.x / BH)) : (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / p.H;
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;
  const uint16_t* __restrict__ qg = p.q + head;
  const uint16_t* __restrict__ kg = p.k + head;
  const uint16_t* __restrict__ vg = p.v + head;

  int kv_end = N;
  if constexpr (KVLEN) kv_end = min(max(p.kv_len[b], 0), N);
  const int q0 = qbi * kBM;
  const int qrow = q0 + w * kRowsPerWave + c;  // this lane's query row
  int kend = kv_end;
  if constexpr (CAUSAL) kend = min(kend, q0 + kBM);
  const int ntiles = (kend + BN - 1) / BN;
  // last key any row of this wave may attend (exclusive bound for tile skipping)
  int wave_kend = kend;
  if constexpr (CAUSAL) wave_kend = min(kend, q0 + w * kRowsPerWave + kRowsPerWave);

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers for the whole kernel
  u32x4 qf[NKK];
  {
    const bool ok = qrow < N;
    const uint16_t* src = qg + (size_t)(ok ? qrow : 0) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 t = *(const u32x4*)(src + 16 * kk);
      qf[kk] = ok ? t : u32x4{0, 0, 0, 0};
    }
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled-log2 scores
  float l_run = 0.f;        // this lane's partial row sum (the other half-wave holds the rest)
  const float sl = p.scale_log2;

  // ---- tile loaders -------------------------------------------------------------
  // K: direct global->LDS copies, 16 B per lane, swizzle applied on the global side.
  auto load_k = [&](int tile, unsigned char* dst) {
    constexpr int CPR = D / 8;                       // 16-byte chunks per row
    constexpr int CHUNKS = BN * CPR;                 // per tile
    constexpr int PER_WAVE = CHUNKS / (kWaves * 64); // wave instructions
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int pos = (i * kWaves + w) * 64 + l;  // LDS chunk position
      const int row = pos / CPR, pc = pos % CPR;
      const int lc = pc ^ swz_k<D>(row);
      const int grow = min(tile * BN + row, N - 1);
      g2lds16(kg + (size_t)grow * D + lc * 8, dst + (size_t)(i * kWaves + w) * 64 * 16);
    }
  };
  // V: 4 keys x 4 head-dims per thread through registers, written transposed.
  constexpr int VBLK = (BN / 4) * (D / 4) / kThreads;  // 4x4 blocks per thread
  static_assert(VBLK >= 1, "tile too small");
  u32x2 vr[VBLK][4];
  auto fetch_v = [&](int tile) {
#pragma unroll
    for (int i = 0; i < VBLK; ++i) {
      const int vb = tid + i * kThreads;
      const int hsel = vb & 1, dq = (vb >> 1) % (D / 4), kc = (vb >> 1) / (D / 4);
      const int k0 = kc * 8 + hsel * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int grow = min(tile * BN + k0 + r, N - 1);
        vr[i][r] = *(const u32x2*)(vg + (size_t)grow * D + dq * 4);
      }
    }
  };
  auto store_vt = [&](unsigned char* dst) {
#pragma unroll
    for (int i = 0; i < VBLK; ++i) {
      const int vb = tid + i * kThreads;
      const int hsel = vb & 1, dq = (vb >> 1) % (D / 4), kc = (vb >> 1) / (D / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // column j of the 4x4 block: (V[k0..k0+3][d0+j])
        const uint32_t w0 = (j < 2) ? vr[i][0][0] : vr[i][0][1];
        const uint32_t w1 = (j < 2) ? vr[i][1][0] : vr[i][1][1];
        const uint32_t w2 = (j < 2) ? vr[i][2][0] : vr[i][2][1];
        const uint32_t w3 = (j < 2) ? vr[i][3][0] : vr[i][3][1];
        u32x2 out;
        if (j & 1) {
          out[0] = hi16_pair(w0, w1);
          out[1] = hi16_pair(w2, w3);
        } else {
          out[0] = lo16_pair(w0, w1);
          out[1] = lo16_pair(w2, w3);
        }
        const uint32_t d = dq * 4 + j;
        const uint32_t byte = d * (BN * 2) + ((kc ^ swz_v<BN>(d)) * 16) + hsel * 8;
        lds_write64(dst, byte, out);
      }
    }
  };

  if (ntiles == 0) {  // no admissible key for any row of this block (kv_len == 0)
    if (qrow < N) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * db + 8 * g + 4 * h;
          *(u32x2*)(p.o + head + (size_t)qrow * D + d0) = u32x2{0, 0};
        }
      if (h == 0) p.lse[(size_t)bh * N + qrow] = -INFINITY;
    }
    return;
  }

  // ---- prologue: tile 0 -------------------------------------------------------------
  load_k(0, kbuf(0));
  fetch_v(0);
  wait_vmem();
  store_vt(vbuf(0));
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const bool has_next = t + 1 < ntiles;
    if (has_next) {
      load_k(t + 1, kbuf(cur ^ 1));
      fetch_v(t + 1);
    }
    const int kt0 = t * BN;
    if (kt0 < wave_kend) {
      // ---- S^T = K Q^T for the BN keys of this tile
      f32x16 s[NKB];
      const unsigned char* kb_ = kbuf(cur);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        const uint32_t row = 32 * kb + key_perm(c);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const uint32_t lc = 2 * kk + h;
          const u32x4 a = lds_read128(kb_, row * (D * 2) + ((lc ^ swz_k<D>(row)) * 16));
          s[kb] = mfma32(a, qf[kk], s[kb]);
        }
      }
      // ---- mask (edge tiles only)
      bool need_mask = kt0 + BN > kv_end;
      if constexpr (CAUSAL) need_mask = need_mask || (kt0 + BN - 1 > q0 + w * kRowsPerWave);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + 32 * kb + 16 * (r >> 3) + 8 * h + (r & 7);
            bool bad = key >= kv_end;
            if constexpr (CAUSAL) bad = bad || key > qrow;
            if (bad) s[kb][r] = -INFINITY;
          }
      }
      // ---- online softmax (scaled-log2 units)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = half_max(mx);
      const float m_new = fmaxf(m_run, mx * sl);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      u32x4 pk[NKB][2];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = fast_exp2(__builtin_fmaf(s[kb][8 * sb + 2 * i], sl, -m_use));
            const float p1 = fast_exp2(__builtin_fmaf(s[kb][8 * sb + 2 * i + 1], sl, -m_use));
            // the row sum uses the unrounded fp32 P: the log-sum-exp the backward
            // recomputes P from must be accurate to fp32, not to bf16
            l_run += p0 + p1;
            pk[kb][sb][i] = pack_bf16x2(p0, p1);
          }
      // ---- O^T += V^T P^T
      const unsigned char* vb_ = vbuf(cur);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const uint32_t lc = 4 * kb + 2 * sb + h;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const uint32_t d = 32 * db + c;
            const u32x4 a = lds_read128(vb_, d * (BN * 2) + ((lc ^ swz_v<BN>(d)) * 16));
            o[db] = mfma32(a, pk[kb][sb], o[db]);
          }
        }
    }
    if (has_next) {
      wait_vmem();
      store_vt(vbuf(cur ^ 1));
    }
    __syncthreads();
  }

  // ---- epilogue: normalise once, store O and LSE
  const float l_tot = half_sum(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  if (qrow < N) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * h;
        u32x2 out;
        out[0] = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
        out[1] = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *(u32x2*)(p.o + head + (size_t)qrow * D + d0) = out;
      }
    if (h == 0) p.lse[(size_t)bh * N + qrow] = empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, int BN, bool CAUSAL, bool KVLEN>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  constexpr size_t lds = 4ull * BN * D * 2;
  auto kern = fa_fwd_kernel<D, BN, CAUSAL, KVLEN>;
  static bool attr_set = false;  // idempotent attribute, racing writers store the same value
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nqb = (a.N + kBM - 1) / kBM;
  const unsigned grid = (unsigned)nqb * (unsigned)(a.B * a.H);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int D, int BN>
hipError_t dispatch_masks(const FwdArgs& a, hipStream_t s) {
  const bool kv = a.kv_len != nullptr;
  if (a.causal) return kv ? launch_one<D, BN, true, true>(a, s) : launch_one<D, BN, true, false>(a, s);
  return kv ? launch_one<D, BN, false, true>(a, s) : launch_one<D, BN, false, false>(a, s);
}

}  // namespace

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return dispatch_masks<128, 64>(a, stream);
  return dispatch_masks<64, 128>(a, stream);
}

}  // namespace fa355
