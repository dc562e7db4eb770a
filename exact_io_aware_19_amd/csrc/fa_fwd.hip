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

template <int D, int BN, bool CAUSAL, bool KVLEN>
__global__ __launch_bounds__(kThreads) void fa_fwd_kernel(FwdArgs p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int TILE_BYTES = BN * D * 2;  // one K tile or one V^T tile
  constexpr int NKB = BN / 32;            // 32-key blocks per tile
  constexpr int NDB = D / 32;             // 32-row blocks of the head dim
  constexpr int NKK = D / 16;             // k-steps of the QK^T contraction
  // LDS: K tiles (natural) at [0, 2*TILE_BYTES), V^T tiles at [2*TILE_BYTES, 4*TILE_BYTES)
  auto kbuf = [&](int i) { return smem + i * TILE_BYTES; };
  auto vbuf = [&](int i) { return smem + (2 + i) * TILE_BYTES; };

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
  // keys past wave_kend are masked for every row of this wave (tile skipping)
  int wave_kend = kend;
  if constexpr (CAUSAL) wave_kend = min(kend, q0 + w * kRowsPerWave + kRowsPerWave);

  if (ntiles == 0) {  // no admissible key for any row of this block (kv_len == 0)
    if (qrow < N) {
      f32x16 zero[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) zero[db] = f32x16{};
      store_ct_rows<D>(p.o + head, qrow, zero, 0.f, h);
      if (h == 0) p.lse[(size_t)bh * N + qrow] = -INFINITY;
    }
    return;
  }

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

  TrTile<BN, D, kThreads> vt;
  const uint32_t kfrag = NatFrag<D>::base(c, h);  // K tile, A operand of S^T
  const uint32_t vfrag = TrFrag<BN>::base(c, h);  // V^T tile, A operand of O^T

  // ---- prologue: tile 0
  load_nat_tile<BN, D, kWaves>(kg, 0, N, kbuf(0), w, l);
  vt.fetch(vg, 0, N, tid);
  wait_vmem();
  vt.store(vbuf(0), tid);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const bool has_next = t + 1 < ntiles;
    if (has_next) {
      load_nat_tile<BN, D, kWaves>(kg, (t + 1) * BN, N, kbuf(cur ^ 1), w, l);
      vt.fetch(vg, (t + 1) * BN, N, tid);
    }
    const int kt0 = t * BN;
    if (kt0 < wave_kend) {
      // ---- S^T = K Q^T for the BN keys of this tile
      f32x16 s[NKB];
      const unsigned char* kb_ = kbuf(cur);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const u32x4 a = lds_read128(kb_, kfrag + kb * NatFrag<D>::BLK + kk * NatFrag<D>::KK);
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
            const int key = kt0 + 32 * kb + c_row(r, h);
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
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x4 a = lds_read128(vb_, vfrag + db * TrFrag<BN>::DB + (4 * kb + 2 * sb) * TrFrag<BN>::CH);
            o[db] = mfma32(a, pk[kb][sb], o[db]);
          }
        }
    }
    if (has_next) {
      wait_vmem();
      vt.store(vbuf(cur ^ 1), tid);
    }
    __syncthreads();
  }

  // ---- epilogue: normalise once, store O and LSE
  const float l_tot = half_sum(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  if (qrow < N) {
    store_ct_rows<D>(p.o + head, qrow, o, inv, h);
    if (h == 0) p.lse[(size_t)bh * N + qrow] = empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, int BN, bool CAUSAL, bool KVLEN>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  constexpr size_t lds = 4ull * BN * D * 2;
  auto kern = fa_fwd_kernel<D, BN, CAUSAL, KVLEN>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
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
