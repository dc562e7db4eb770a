// Attention backward for gfx950 (MI355X): gradients of L = sum(O * dO).
//
// The probabilities are never stored by the forward pass; both kernels recompute them
// on chip from Q, K and the saved per-row log-sum-exp ("FlashAttention" concept wiki
// page, section 定義 (2) recomputation; singularity-lens FA1 explainer, paragraph on
// recomputation).  With S the scaled scores, P = exp(S - LSE), dP = dO V^T,
// D_i = sum_k dO_ik O_ik and dS = P * (dP - D):
//     dV = P^T dO,   dK = scale * dS^T Q,   dQ = scale * dS K.
//
// dQ accumulation strategy: no atomics.  The pages single out the atomic additions of
// the backward pass as a cost (FlashAttention-4 summary, third optimisation; wiki page,
// FA4 (3)) and list the overhead of a deterministic backward as an open question (wiki
// page, 未解決の問い).  Here dQ is produced by its own query-outer pass that keeps the
// dQ rows in registers across all key tiles, and dK/dV by a key-outer pass that keeps
// its key columns' dK, dV in registers across all query tiles.  Each pass recomputes S
// and dP (7 products per tile pair instead of 5), in exchange every output is written
// exactly once, no dS tile is exchanged through LDS, and results are bitwise
// reproducible.
//
//   launch 1  fa_bwd_dq_kernel    (query-outer, 8 waves x 32 query rows)
//             D_i = rowsum(dO * O) -> workspace;  S^T = K Q^T, dP^T = V dO^T,
//             dS^T = P^T * (dP^T - D);  dQ^T += K^T dS^T
//   launch 2  fa_bwd_dkdv_kernel  (key-outer, 4 waves x 32 key columns)
//             S = Q K^T, dP = dO V^T, dS = P * (dP - D);
//             dV^T += dO^T P,  dK^T += Q^T dS
#include "common.hpp"
#include "fa_kernels.hpp"

namespace fa355 {

namespace {

// --------------------------------------------------------------------------------------
// launch 1: dQ (and D_i)
// --------------------------------------------------------------------------------------
constexpr int kDqWaves = 8;
constexpr int kDqThreads = kDqWaves * 64;
constexpr int kDqBM = kDqWaves * 32;  // query rows per workgroup

template <int D, int BN, bool CAUSAL, bool KVLEN>
__global__ __launch_bounds__(kDqThreads) void fa_bwd_dq_kernel(BwdArgs p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int NKB = BN / 32, NDB = D / 32, NKK = D / 16;
  // LDS: K natural x2, V natural x2, K^T x2
  auto kbuf = [&](int i) { return smem + i * TILE_BYTES; };
  auto vbuf = [&](int i) { return smem + (2 + i) * TILE_BYTES; };
  auto ktbuf = [&](int i) { return smem + (4 + i) * TILE_BYTES; };

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, c = l & 31, h = l >> 5;
  const int BH = p.B * p.H;
  const int nqb = (p.N + kDqBM - 1) / kDqBM;
  const int qbi = CAUSAL ? (nqb - 1 - (int)(blockIdx.x / BH)) : (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / p.H;
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;
  const buf_rsrc kg = make_rsrc(p.k + head, (uint32_t)N * D * 2);
  const buf_rsrc vg = make_rsrc(p.v + head, (uint32_t)N * D * 2);

  int kv_end = N;
  if constexpr (KVLEN) kv_end = min(max(p.kv_len[b], 0), N);
  const int q0 = qbi * kDqBM;
  const int qrow = q0 + w * 32 + c;
  const bool row_ok = qrow < N;
  int kend = kv_end;
  if constexpr (CAUSAL) kend = min(kend, q0 + kDqBM);
  const int ntiles = (kend + BN - 1) / BN;
  int wave_kend = kend;
  if constexpr (CAUSAL) wave_kend = min(kend, q0 + w * 32 + 32);

  // ---- per-row operands: Q and dO fragments (B operands), D_i, LSE
  u32x4 qf[NKK], dof[NKK];
  float di = 0.f;
  {
    const size_t off = head + (size_t)(row_ok ? qrow : 0) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 tq = *(const u32x4*)(p.q + off + 16 * kk);
      const u32x4 td = *(const u32x4*)(p.dout + off + 16 * kk);
      const u32x4 to = *(const u32x4*)(p.o + off + 16 * kk);
      qf[kk] = row_ok ? tq : u32x4{0, 0, 0, 0};
      dof[kk] = row_ok ? td : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        di = __builtin_fmaf(bf16_lo(to[e]), bf16_lo(td[e]), di);
        di = __builtin_fmaf(bf16_hi(to[e]), bf16_hi(td[e]), di);
      }
    }
    di = row_ok ? half_sum(di) : 0.f;
  }
  if (row_ok && h == 0) p.dsum[(size_t)bh * N + qrow] = di;
  float lse2 = INFINITY;  // P = exp2(s * scale * log2e - lse2); +inf gives P = 0
  if (row_ok) {
    const float ln = p.lse[(size_t)bh * N + qrow];
    lse2 = (ln == -INFINITY) ? INFINITY : ln * kLog2e;
  }

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

  if (ntiles == 0) {
    if (row_ok) store_ct_rows<D>(p.dq + head, qrow, dq, 0.f, h);
    return;
  }
  const float sl = p.scale_log2;
  TrTile<BN, D, kDqThreads> kt;
  const uint32_t nfrag = NatFrag<D>::base(c, h);  // K and V tiles, A operands of S^T and dP^T
  const uint32_t tfrag[2] = {TrFrag<BN>::base(c, h, 0), TrFrag<BN>::base(c, h, 1)};  // K^T tile, A operand of dQ^T

  load_nat_tile<BN, D, kDqWaves>(kg, 0, N, kbuf(0), w, l);
  load_nat_tile<BN, D, kDqWaves>(vg, 0, N, vbuf(0), w, l);
  kt.fetch(kg, 0, N, tid);
  wait_vmem();
  kt.store(ktbuf(0), tid);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const bool has_next = t + 1 < ntiles;
    if (has_next) {
      load_nat_tile<BN, D, kDqWaves>(kg, (t + 1) * BN, N, kbuf(cur ^ 1), w, l);
      load_nat_tile<BN, D, kDqWaves>(vg, (t + 1) * BN, N, vbuf(cur ^ 1), w, l);
      kt.fetch(kg, (t + 1) * BN, N, tid);
    }
    const int kt0 = t * BN;
    if (kt0 < wave_kend) {
      bool need_mask = kt0 + BN > kv_end;
      if constexpr (CAUSAL) need_mask = need_mask || (kt0 + BN - 1 > q0 + w * 32);
      // no running statistics in the backward: each 32-key block is finished on its own
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const uint32_t off = nfrag + kb * NatFrag<D>::BLK + kk * NatFrag<D>::KK;
          const u32x4 ak = lds_read128(kbuf(cur), off);
          s = mfma32(ak, qf[kk], s);
          const u32x4 av = lds_read128(vbuf(cur), off);
          dp = mfma32(av, dof[kk], dp);
        }
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + 32 * kb + c_row(r, h);
            bool bad = key >= kv_end;
            if constexpr (CAUSAL) bad = bad || key > qrow;
            if (bad) s[r] = -INFINITY;
          }
        }
        u32x4 dsk[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r0 = 8 * sb + 2 * i;
            const float p0 = fast_exp2(__builtin_fmaf(s[r0], sl, -lse2));
            const float p1 = fast_exp2(__builtin_fmaf(s[r0 + 1], sl, -lse2));
            dsk[sb][i] = pack_bf16x2(p0 * (dp[r0] - di), p1 * (dp[r0 + 1] - di));
          }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x4 a = lds_read128(ktbuf(cur), tfrag[db & 1] + db * TrFrag<BN>::DB + (4 * kb + 2 * sb) * TrFrag<BN>::CH);
            dq[db] = mfma32(a, dsk[sb], dq[db]);
          }
      }
    }
    if (has_next) {
      wait_vmem();
      kt.store(ktbuf(cur ^ 1), tid);
    }
    __syncthreads();
  }
  if (row_ok) store_ct_rows<D>(p.dq + head, qrow, dq, p.scale, h);
}

// --------------------------------------------------------------------------------------
// launch 2: dK, dV
// --------------------------------------------------------------------------------------
constexpr int kKvWaves = 4;
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kKvBN = kKvWaves * 32;  // key columns per workgroup

template <int D, int BM>
struct KvStage {
  static constexpr int TILE_BYTES = BM * D * 2;
  // Q natural, dO natural, Q^T, dO^T, then lse2[BM] and D[BM] (fp32)
  static constexpr int Q = 0, DO = TILE_BYTES, QT = 2 * TILE_BYTES, DOT = 3 * TILE_BYTES;
  static constexpr int LSE = 4 * TILE_BYTES, DSUM = 4 * TILE_BYTES + BM * 4;
  static constexpr int BYTES = 4 * TILE_BYTES + 2 * BM * 4;
};

template <int D, int BM, bool CAUSAL, bool KVLEN>
__global__ __launch_bounds__(kKvThreads) void fa_bwd_dkdv_kernel(BwdArgs p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  using St = KvStage<D, BM>;
  constexpr int NQB = BM / 32, NDB = D / 32, NKK = D / 16;
  auto stage = [&](int i) { return smem + i * St::BYTES; };

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, c = l & 31, h = l >> 5;
  const int BH = p.B * p.H;
  const int kbi = blockIdx.x / BH;  // causal: key block 0 sees the most queries, so it goes first
  const int bh = blockIdx.x % BH;
  const int b = bh / p.H;
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;
  const buf_rsrc qg = make_rsrc(p.q + head, (uint32_t)N * D * 2);
  const buf_rsrc dog = make_rsrc(p.dout + head, (uint32_t)N * D * 2);
  const float* __restrict__ lseg = p.lse + (size_t)bh * N;
  const float* __restrict__ dsg = p.dsum + (size_t)bh * N;

  int kv_end = N;
  if constexpr (KVLEN) kv_end = min(max(p.kv_len[b], 0), N);
  const int k0 = kbi * kKvBN;
  const int kw0 = k0 + w * 32;   // first key column of this wave
  const int kcol = kw0 + c;      // this lane's key column
  const bool col_store = kcol < N;
  const bool col_live = kcol < kv_end;

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  if (k0 >= kv_end) {  // every key of this block is padded away: exact zeros
    if (col_store) {
      store_ct_rows<D>(p.dk + head, kcol, dk, 0.f, h);
      store_ct_rows<D>(p.dv + head, kcol, dv, 0.f, h);
    }
    return;
  }

  // ---- this lane's key column: K and V fragments (B operands)
  u32x4 kf[NKK], vf[NKK];
  {
    const size_t off = head + (size_t)min(kcol, N - 1) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      kf[kk] = *(const u32x4*)(p.k + off + 16 * kk);
      vf[kk] = *(const u32x4*)(p.v + off + 16 * kk);
    }
  }

  const int i_first = CAUSAL ? (k0 / BM) : 0;
  const int i_last = (N + BM - 1) / BM;  // exclusive
  const float sl = p.scale_log2;
  TrTile<BM, D, kKvThreads> qt, dot;
  const uint32_t nfrag = NatFrag<D>::base(c, h);   // Q and dO tiles, A operands of S and dP
  const uint32_t tfrag[2] = {TrFrag<BM>::base(c, h, 0), TrFrag<BM>::base(c, h, 1)};  // Q^T, dO^T tiles: A of dK^T, dV^T

  // row statistics of one query tile: raw loads into registers now, converted only when
  // stored (using a loaded value early would wait on every load in flight)
  float st_lse = 0.f, st_d = 0.f;
  auto fetch_stats = [&](int i0) {
    if (tid < BM) {
      const int q = min(i0 + tid, N - 1);
      st_lse = lseg[q];
      st_d = dsg[q];
    }
  };
  auto store_stats = [&](unsigned char* st, int i0) {
    if (tid < BM) {
      // lse2 = +inf (P = 0) for rows past N and for rows with no admissible key
      const bool live = i0 + tid < N && st_lse != -INFINITY;
      ((float*)(st + St::LSE))[tid] = live ? st_lse * kLog2e : INFINITY;
      ((float*)(st + St::DSUM))[tid] = live ? st_d : 0.f;
    }
  };
  auto issue = [&](int i, unsigned char* st) {
    const int i0 = i * BM;
    load_nat_tile<BM, D, kKvWaves>(qg, i0, N, st + St::Q, w, l);
    load_nat_tile<BM, D, kKvWaves>(dog, i0, N, st + St::DO, w, l);
    qt.fetch(qg, i0, N, tid);
    dot.fetch(dog, i0, N, tid);
    fetch_stats(i0);
  };
  auto finish = [&](unsigned char* st, int i) {
    wait_vmem();
    qt.store(st + St::QT, tid);
    dot.store(st + St::DOT, tid);
    store_stats(st, i * BM);
  };

  issue(i_first, stage(0));
  finish(stage(0), i_first);
  __syncthreads();

  for (int i = i_first; i < i_last; ++i) {
    const int cur = (i - i_first) & 1;
    const bool has_next = i + 1 < i_last;
    if (has_next) issue(i + 1, stage(cur ^ 1));
    const int i0 = i * BM;
    unsigned char* st = stage(cur);
    // causal: skip tiles whose queries all precede this wave's first key
    if (!CAUSAL || i0 + BM - 1 >= kw0) {
      const int qoff0 = i0 + 8 * h - kcol;  // (query - key) of this lane's first row
      // Software pipeline over the 32-query blocks of the tile: the operand reads of
      // the next phase are issued before the math of the current one, so LDS latency
      // hides behind MFMA and VALU work of the same wave (one wave per SIMD here).
      u32x4 aq[NKK], ad[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        aq[kk] = lds_read128(st + St::Q, nfrag + kk * NatFrag<D>::KK);
        ad[kk] = lds_read128(st + St::DO, nfrag + kk * NatFrag<D>::KK);
      }
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          s = mfma32(aq[kk], kf[kk], s);
          dp = mfma32(ad[kk], vf[kk], dp);
        }
        // operands of dV^T / dK^T for this block, and statistics of its rows
        u32x4 ao[2][NDB], at[2][NDB];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const uint32_t off = tfrag[db & 1] + db * TrFrag<BM>::DB + (4 * qb + 2 * sb) * TrFrag<BM>::CH;
            ao[sb][db] = lds_read128(st + St::DOT, off);
            at[sb][db] = lds_read128(st + St::QT, off);
          }
        f32x4 lsv[2][2], dsv[2][2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          // the 8 query rows 32*qb + 16*sb + 8*h + 0..7 held by this lane
          const int rbase = 32 * qb + 16 * sb + 8 * h;
          lsv[sb][0] = *(const f32x4*)(st + St::LSE + rbase * 4);
          lsv[sb][1] = *(const f32x4*)(st + St::LSE + rbase * 4 + 16);
          dsv[sb][0] = *(const f32x4*)(st + St::DSUM + rbase * 4);
          dsv[sb][1] = *(const f32x4*)(st + St::DSUM + rbase * 4 + 16);
        }
        // next block's S/dP operands
        if (qb + 1 < NQB) {
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            aq[kk] = lds_read128(st + St::Q, nfrag + (qb + 1) * NatFrag<D>::BLK + kk * NatFrag<D>::KK);
            ad[kk] = lds_read128(st + St::DO, nfrag + (qb + 1) * NatFrag<D>::BLK + kk * NatFrag<D>::KK);
          }
        }
        // P = exp2(S * scale * log2e - LSE * log2e), dS = P * (dP - D)
        u32x4 pk[2], dsk[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r0 = 8 * sb + 2 * e;
            const float l0 = lsv[sb][e >> 1][(2 * e) & 3], l1 = lsv[sb][e >> 1][(2 * e + 1) & 3];
            const float d0 = dsv[sb][e >> 1][(2 * e) & 3], d1 = dsv[sb][e >> 1][(2 * e + 1) & 3];
            float p0 = fast_exp2(__builtin_fmaf(s[r0], sl, -l0));
            float p1 = fast_exp2(__builtin_fmaf(s[r0 + 1], sl, -l1));
            if constexpr (CAUSAL) {
              // key kcol is admissible for query q iff kcol <= q; qoff = q - kcol
              const int qoff = qoff0 + 32 * qb + 16 * sb + 2 * e;
              p0 = (qoff < 0) ? 0.f : p0;
              p1 = (qoff + 1 < 0) ? 0.f : p1;
            }
            pk[sb][e] = pack_bf16x2(p0, p1);
            dsk[sb][e] = pack_bf16x2(p0 * (dp[r0] - d0), p1 * (dp[r0 + 1] - d1));
          }
        // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            dv[db] = mfma32(ao[sb][db], pk[sb], dv[db]);
            dk[db] = mfma32(at[sb][db], dsk[sb], dk[db]);
          }
      }
    }
    if (has_next) finish(stage(cur ^ 1), i + 1);
    __syncthreads();
  }
  if (col_store) {
    // keys padded away for every query get exact zeros
    store_ct_rows<D>(p.dk + head, kcol, dk, col_live ? p.scale : 0.f, h);
    store_ct_rows<D>(p.dv + head, kcol, dv, col_live ? 1.f : 0.f, h);
  }
}

// --------------------------------------------------------------------------------------
template <typename K>
hipError_t set_lds(K kern, size_t lds) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <int D, int BN, int BM, bool CAUSAL, bool KVLEN>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  const unsigned bh = (unsigned)(a.B * a.H);
  {
    constexpr size_t lds = 6ull * BN * D * 2;
    auto kern = fa_bwd_dq_kernel<D, BN, CAUSAL, KVLEN>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((a.N + kDqBM - 1) / kDqBM) * bh;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kDqThreads), lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    constexpr size_t lds = 2ull * KvStage<D, BM>::BYTES;
    auto kern = fa_bwd_dkdv_kernel<D, BM, CAUSAL, KVLEN>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((a.N + kKvBN - 1) / kKvBN) * bh;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kKvThreads), lds, stream, a);
    return hipGetLastError();
  }
}

template <int D, int BN, int BM>
hipError_t dispatch_masks(const BwdArgs& a, hipStream_t s) {
  const bool kv = a.kv_len != nullptr;
  if (a.causal) return kv ? launch_bwd<D, BN, BM, true, true>(a, s) : launch_bwd<D, BN, BM, true, false>(a, s);
  return kv ? launch_bwd<D, BN, BM, false, true>(a, s) : launch_bwd<D, BN, BM, false, false>(a, s);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return dispatch_masks<128, 64, 64>(a, stream);
  return dispatch_masks<64, 128, 128>(a, stream);
}

}  // namespace fa355
