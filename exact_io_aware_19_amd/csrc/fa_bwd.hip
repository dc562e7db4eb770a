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
//             D_i = rowsum(dO * O), -D_i -> workspace;  S^T = K Q^T, dP^T = V dO^T,
//             dS^T = P^T * (dP^T - D);  dQ^T += K^T dS^T
//   launch 2  fa_bwd_dkdv_kernel  (key-outer, 4 waves x 32 key columns)
//             S = Q K^T, dP = dO V^T, dS = P * (dP - D);
//             dV^T += dO^T P,  dK^T += Q^T dS
#include <type_traits>

#include "common.hpp"
#include "fa_kernels.hpp"

namespace fa355 {

namespace {

// --------------------------------------------------------------------------------------
// launch 1: dQ (and D_i)
// --------------------------------------------------------------------------------------
constexpr int kDqWaves = 8;
constexpr int kDqThreads = kDqWaves * 64;
constexpr int kDqBM = kDqWaves * 32;  // query rows per workgroup (unsplit)

// G = 1: 8 waves x 32 query rows over the whole key range.  G = 2 (split, small d = 128
// grids, split_small_grid): 128 query rows per workgroup, waves 0-3 and 4-7 take the two
// halves of the key tiles through LDS tiles of their own, and the second group's dQ^T
// partial sums are added to the first group's through LDS at the end.  The workgroup
// count doubles and the causal mask's uneven row blocks halve: B=1, H=16, N=2048 causal
// 0.0711 -> 0.0562 ms, no mask 0.0805 -> 0.0635; B=2, H=16, N=2048 causal 0.0792 ->
// 0.0754 (one box); slower at d = 64 and on fuller grids.
template <int D, int BN, bool CAUSAL, bool KVLEN, int G>
__global__ __launch_bounds__(kDqThreads) void fa_bwd_dq_kernel(BwdArgs p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int NCH = D / 8;
  constexpr int NKB = BN / 32, NDB = D / 32, NKK = D / 16;
  constexpr int GW = kDqWaves / G;  // waves per group
  constexpr int GBM = GW * 32;      // query rows per workgroup
  const int tid = threadIdx.x;
  const int wg = tid >> 6, l = tid & 63, c = l & 31, h = l >> 5;
  const int grp = G == 1 ? 0 : wg / GW, w = G == 1 ? wg : wg % GW;
  // LDS per group: K x2, V x2 (swz4 layout), then the -D table; K^T operands are read
  // from the K tile transposed
  unsigned char* const gsm = smem + (size_t)grp * (4 * TILE_BYTES + GW * 32 * 16);
  auto kbuf = [&](int i) { return gsm + i * TILE_BYTES; };
  auto vbuf = [&](int i) { return gsm + (2 + i) * TILE_BYTES; };
  using Copy = SwzCopy<BN, D, GW, true>;

  const int BH = p.B * p.H;
  const int nqb = (p.N + GBM - 1) / GBM;
  // no mask: each XCD works through whole heads; causal: heaviest query blocks first
  int blk, bh;
  block_order<!CAUSAL>((int)blockIdx.x, nqb, BH, blk, bh);
  const int qbi = CAUSAL ? (nqb - 1 - blk) : blk;
  const int b = bh / p.H;
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;
  // grouped K/V heads: the H / Hkv query heads of a group share one K/V head
  const size_t kv_head = (size_t)(b * p.Hkv + (bh - b * p.H) / (p.H / p.Hkv)) * N * D;
  const buf_rsrc kg = make_rsrc(p.k + kv_head, (uint32_t)N * D * 2);
  const buf_rsrc vg = make_rsrc(p.v + kv_head, (uint32_t)N * D * 2);

  int kv_end = N;
  if constexpr (KVLEN) kv_end = min(max(p.kv_len[b], 0), N);
  const int q0 = qbi * GBM;
  const int qrow = q0 + w * 32 + c;
  const bool row_ok = qrow < N;
  int kend = kv_end;
  if constexpr (CAUSAL) kend = min(kend, q0 + GBM);
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
  float lse2 = INFINITY;  // P = exp2(s * scale * log2e - lse2); +inf gives P = 0
  if (row_ok) {
    const float ln = p.lse[(size_t)bh * N + qrow];
    lse2 = (ln == -INFINITY) ? INFINITY : ln * kLog2e;
  }
  // row statistics for the dK/dV pass (-D: its dP products start from it); the grid
  // covers exactly the nw padded rows
  if (h == 0 && (G == 1 || grp == 0)) {
    p.ws_d[(size_t)bh * p.nw + qrow] = -di;
    p.ws_l[(size_t)bh * p.nw + qrow] = lse2;
  }
  if constexpr (G == 2) {
    // the last block's second group fills the rows past the grid's (at most 128)
    if (h == 0 && grp == 1 && qbi == nqb - 1) {
      const int r = nqb * GBM + w * 32 + c;
      if (r < p.nw) {
        p.ws_d[(size_t)bh * p.nw + r] = -0.f;
        p.ws_l[(size_t)bh * p.nw + r] = INFINITY;
      }
    }
  }

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

  if (ntiles == 0) {
    if (row_ok && (G == 1 || grp == 0)) store_ct_rows<D>(p.dq + head, qrow, dq, 0.f, h);
    return;
  }
  const float sl = p.scale_log2;
  // -D of this lane's query four times over in LDS (16 bytes per query row, a region per
  // wave after the tiles): four 16-byte reads of it fill a dP^T accumulator, so the dP^T
  // products yield dP^T - D directly, with no subtraction per score (volatile: four
  // reads into the accumulator's registers, not one read and twelve register copies)
  unsigned char* const ndt = gsm + 4 * TILE_BYTES + w * 32 * 16;
  if (h == 0) {
    const uint32_t nd = __builtin_bit_cast(uint32_t, -di);
    lds_write128(ndt, 16 * c, u32x4{nd, nd, nd, nd});
  }
  auto neg_d = [&]() {
    f32x16 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = *(const volatile lds_u32x4*)((const __attribute__((address_space(3))) unsigned char*)ndt + 16 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = __builtin_bit_cast(float, (uint32_t)v[e]);
    }
    return x;
  };
  // Fragment bases.  S^T, dP^T: lane (c, h) reads K / V row 32*kb + row_perm(c), chunk
  // 2*kk + h; the swizzle depends on kk only through kk % 2.  dQ^T: the K^T operand
  // (rows d = 32*db + c, k-slots keys 16*sb + 8*h + 0..7 of block kb) comes from two
  // transposed reads of the K tile (keys +0..3, +4..7): lane s of 16-lane group g
  // addresses key 8*(g/2) + s/4 (+4 for the second read, an XOR of 64 in the byte
  // address), columns 16*(g%2) + 4*(s%4) .. +3.
  const uint32_t rp = row_perm(c);
  uint32_t nb[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) nb[x] = 16 * swz4_unit<NCH>(rp, 2 * x + h);
  const int tg = l >> 4, ts = l & 15;
  const uint32_t trb = 16 * swz4_unit<NCH>(8 * (tg >> 1) + (ts >> 2), 2 * (tg & 1) + ((ts & 3) >> 1)) + 8 * (ts & 1);
  constexpr uint32_t BLK16 = 16 * NCH * 16;  // bytes per 16 rows
  auto issue = [&](int t, int s) {
#pragma unroll
    for (int ii = 0; ii < Copy::PER_WAVE; ++ii) {
      // rows at or past the last admissible key repeat it: padded rows are never read
      Copy::issue(kg, t * BN, kv_end, kbuf(s), w, l, ii);
      Copy::issue(vg, t * BN, kv_end, vbuf(s), w, l, ii);
    }
  };

  // this group's tiles [jb, je); with G = 2 both groups run the first group's count of
  // iterations (the second group's last one is empty when the count is odd)
  const int half = G == 1 ? ntiles : (ntiles + 1) / 2;
  const int jb = G == 1 ? 0 : grp * half, je = G == 1 ? ntiles : min(ntiles, jb + half);
  if (jb < je) issue(jb, 0);
  wait_vmem();
  __syncthreads();

  for (int t = jb; t < jb + half; ++t) {
    const int cur = (t - jb) & 1;
    const bool has_next = t + 1 < je;
    if (has_next) issue(t + 1, cur ^ 1);
    const int kt0 = t * BN;
    if ((G == 1 || t < je) && kt0 < wave_kend) {
      bool need_mask = kt0 + BN > kv_end;
      if constexpr (CAUSAL) need_mask = need_mask || (kt0 + BN - 1 > q0 + w * 32);
      // No running statistics in the backward: each 32-key block is finished on its own.
      // Pairs of key blocks (a, b) run as one pinned stream of products with operand
      // fragments read kLook products ahead:
      //   S, dP (a) | S, dP (b) with P, dS (a) between the products | dQ (a) with P, dS (b)
      //   between them | dQ (b)
      // (each block's S products before its dP products, which start from -D)
      // so the elementwise work of one block overlaps the other block's products.
      auto pair = [&](auto kbp_c) {  // interior tiles only: no mask
        constexpr int KA = 2 * decltype(kbp_c)::value;
        constexpr int NSP = 2 * NKK, NQ = 2 * NDB, T = 2 * NSP + 2 * NQ;
        // one product ahead: two waves share each SIMD and hide each other's operand
        // reads; reading two ahead needed 6 more registers than the 256 the two waves
        // allow (spilled) and measured no faster
        constexpr int kLook = 1;
        f32x16 sc[2], dp[2];
        u32x4 dsk[2][2];
        // op t: [0, NSP) S/dP of a, [NSP, 2NSP) S/dP of b, then dQ of a, dQ of b
        auto aread = [&](int t) -> u32x4 {
          if (t < 2 * NSP) {  // S products of a block, then its dP products
            const int kb = KA + t / NSP, r = t % NSP, kk = r % NKK;
            return lds_read128((r >= NKK) ? vbuf(cur) : kbuf(cur), nb[kk & 1] + kb * 2 * BLK16 + (kk >> 1) * 64 * 16);
          }
          const int u = t - 2 * NSP, kb = KA + u / NQ, m = u % NQ, sb = m / NDB, db = m % NDB;
          const uint32_t off = (2 * kb + sb) * BLK16 + db * 4 * 16 * 16;
          const u32x2 a0 = lds_read_tr16(kbuf(cur), trb + off), a1 = lds_read_tr16(kbuf(cur), (trb ^ 64u) + off);
          return u32x4{a0[0], a0[1], a1[0], a1[1]};
        };
        // P, dS for rows 2e, 2e+1 of half sb of block x of the pair
        auto group = [&](int x, int g) {
          const int sb = g >> 2, e = g & 3, r0 = 8 * sb + 2 * e;
          const float p0 = fast_exp2(__builtin_fmaf(sc[x][r0], sl, -lse2));
          const float p1 = fast_exp2(__builtin_fmaf(sc[x][r0 + 1], sl, -lse2));
          dsk[x][sb][e] = pack_bf16x2(p0 * dp[x][r0], p1 * dp[x][r0 + 1]);
        };
        u32x4 fr[kLook];
#pragma unroll
        for (int t = 0; t < kLook; ++t) fr[t] = aread(t);
        static_for<T>([&](auto tc) {
          constexpr int t = decltype(tc)::value;
          const u32x4 a = fr[t % kLook];
          if constexpr (t + kLook < T) fr[t % kLook] = aread(t + kLook);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (t < 2 * NSP) {
            constexpr int x = t / NSP, r = t % NSP, kk = r % NKK;
            if constexpr (r == 0) dp[x] = neg_d();  // lands before the block's dP products
            if constexpr (r >= NKK) dp[x] = mfma32(a, dof[kk], dp[x]);
            else sc[x] = mfma32(a, qf[kk], kk == 0 ? f32x16{} : sc[x]);
            // P, dS of block a: its eight groups spread over the products of block b
            if constexpr (x == 1) {
              constexpr int G0 = (8 * r) / NSP, G1 = (8 * (r + 1)) / NSP;
              static_for<G1 - G0>([&](auto gc) { group(0, G0 + decltype(gc)::value); });
            }
          } else {
            constexpr int u = t - 2 * NSP, x = u / NQ, m = u % NQ, sb = m / NDB, db = m % NDB;
            dq[db] = mfma32(a, dsk[x][sb], dq[db]);
            // P, dS of block b: spread over the dQ products of block a
            if constexpr (x == 0) {
              constexpr int G0 = (8 * m) / NQ, G1 = (8 * (m + 1)) / NQ;
              static_for<G1 - G0>([&](auto gc) { group(1, G0 + decltype(gc)::value); });
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      };
      static_assert(NKB % 2 == 0, "key blocks run in pairs");
      if (!need_mask) {
        static_for<NKB / 2>([&](auto kbp) { pair(kbp); });
      } else {
        // edge tiles (causal diagonal, padding, ragged end): one block at a time
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          f32x16 s = f32x16{}, dp = neg_d();
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const uint32_t off = nb[kk & 1] + kb * 2 * BLK16 + (kk >> 1) * 64 * 16;
            s = mfma32(lds_read128(kbuf(cur), off), qf[kk], s);
            dp = mfma32(lds_read128(vbuf(cur), off), dof[kk], dp);
          }
          u32x4 dsk[2];
#pragma unroll
          for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r0 = 8 * sb + 2 * e;
              const int key0 = kt0 + 32 * kb + c_row(r0, h);
              bool bad0 = key0 >= kv_end, bad1 = key0 + 1 >= kv_end;
              if constexpr (CAUSAL) {
                bad0 = bad0 || key0 > qrow;
                bad1 = bad1 || key0 + 1 > qrow;
              }
              const float p0 = bad0 ? 0.f : fast_exp2(__builtin_fmaf(s[r0], sl, -lse2));
              const float p1 = bad1 ? 0.f : fast_exp2(__builtin_fmaf(s[r0 + 1], sl, -lse2));
              dsk[sb][e] = pack_bf16x2(p0 * dp[r0], p1 * dp[r0 + 1]);
            }
#pragma unroll
          for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const uint32_t off = (2 * kb + sb) * BLK16 + db * 4 * 16 * 16;
              const u32x2 a0 = lds_read_tr16(kbuf(cur), trb + off), a1 = lds_read_tr16(kbuf(cur), (trb ^ 64u) + off);
              dq[db] = mfma32(u32x4{a0[0], a0[1], a1[0], a1[1]}, dsk[sb], dq[db]);
            }
        }
      }
    }
    wait_vmem();
    __syncthreads();
  }
  if constexpr (G == 2) {
    // the second group's dQ^T partial sums through LDS (the tiles are free after the
    // loop's last barrier), added in a fixed order
    float* xq = (float*)smem + (size_t)(w * 64 + l) * (16 * NDB + 1);
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xq[16 * db + r] = dq[db][r];
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[db][r] += xq[16 * db + r];
  }
  if (row_ok) store_ct_rows<D>(p.dq + head, qrow, dq, p.scale, h);
}

// --------------------------------------------------------------------------------------
// launch 2: dK, dV
//
// One workgroup = 4 waves x 32 key columns; each wave keeps its keys' K and V fragments
// and its dK^T, dV^T accumulators in registers and streams the query tiles (BM rows).
// Per query tile the workgroup fetches Q and dO once, by direct global->LDS copies into
// swizzled natural tiles, and builds the transposed tiles Q^T, dO^T (A operands of dK^T
// and dV^T) from them in LDS with 8x8 register transpositions.  The per-row statistics
// (LSE * log2 e and -D) come from the dQ pass's workspace, also by direct copies; each
// 32-query block's dP products accumulate onto -D, so they yield dP - D directly.
//
// Software pipeline over query tiles: while tile i is reduced into dK^T, dV^T, the
// scores of tile i+1 (S, dP and from them P, dS in bf16) are computed, and tile i+2 is
// being fetched.  Inside an iteration the 32-query blocks are staggered so that the
// elementwise work on the scores of one block runs between the dK^T, dV^T products of
// the previous tile's block:
//   step q:  S, dP (i+1, q)  then  dV^T, dK^T (i, q)  alongside  P, dS (i+1, q)
// LDS: 2 x {Q, dO} natural, 2 x {Q^T, dO^T}, 3 x {lse2, -D}.
// --------------------------------------------------------------------------------------
constexpr int kKvWaves = 4;
constexpr int kKvThreads = kKvWaves * 64;
constexpr int kKvBN = kKvWaves * 32;  // key columns per workgroup
static_assert(kKvBN == kKvBlockKeys, "split planning assumes this many keys per workgroup");

template <int D, int BM>
struct KvLds {
  static constexpr int TILE = BM * D * 2;
  static constexpr int NAT = 0;         // slot s: Q at NAT + 2*s*TILE, dO right after
  static constexpr int TR = 4 * TILE;   // slot s: Q^T at TR + 2*s*TILE, dO^T right after
  // row statistics of tile t in slot (t - first tile) % 3: iteration i reads those of
  // tiles i and i+1 while the copy of tile i+2's lands, with no barrier in between
  static constexpr int ST = 8 * TILE;   // slot s: lse2[BM] at ST + 8*s*BM, -D[BM] right after
  static constexpr int BYTES = 8 * TILE + 3 * 8 * BM;
};

// Compile-time placement of the P, dS groups in the dK/dV stream (see the kernel).  A
// group runs in three stages on consecutive products (A: S, dP - D out of the
// accumulators and the exponent argument; B: exp2; C: products and bf16 packing), so no
// product slot carries a long dependent chain that would hold back the next product.
template <int NQB, int NS, int NR>
struct KvSched {
  static constexpr int NSTEP = NS + NR, T = NQB * NSTEP;
  // first stage of group u of block q of the scored tile: groups 0-3 on the block's
  // dK/dV products, 4-7 on the next block's S/dP products (-1: the last block's groups
  // 4-7, which run in the next iteration as carried groups of the reduced tile)
  static constexpr int OFF = NR >= 16 ? 1 : 0;
  static constexpr int min_(int a, int b) { return a < b ? a : b; }
  static constexpr int unit_op(int q, int u) {
    if (u < 4) return min_(q * NSTEP + NS + u * (NR / 4) + OFF, T - 6 + u);
    if (q + 1 < NQB) return (q + 1) * NSTEP + 1 + (u - 4) * (NS / 4);
    return -1;
  }
  static constexpr int carry_op(int u) { return 1 + (u - 4) * (NS / 4); }  // u = 4..7
  // group whose first stage runs after op t: 16*q + u for the scored tile, 1000 + u for
  // a carried group, -1 for none
  static constexpr int unit_at(int t) {
    if (t < 0) return -1;
    for (int u = 4; u < 8; ++u)
      if (carry_op(u) == t) return 1000 + u;
    for (int q = 0; q < NQB; ++q)
      for (int u = 0; u < 8; ++u)
        if (unit_op(q, u) == t) return 16 * q + u;
    return -1;
  }
  // number of groups starting before op t (ring index of a group's registers)
  static constexpr int seq(int t) {
    int n = 0;
    for (int x = 0; x < t; ++x) n += unit_at(x) >= 0;
    return n;
  }
  // every group starts on its own op and ends inside the iteration; at most three
  // groups are in flight (ring of three register sets, statistics read two ops ahead)
  static constexpr bool valid() {
    int starts[8 * NQB + 4] = {};
    int n = 0;
    for (int u = 4; u < 8; ++u) starts[n++] = carry_op(u);
    for (int q = 0; q < NQB; ++q)
      for (int u = 0; u < 8; ++u)
        if (unit_op(q, u) >= 0) starts[n++] = unit_op(q, u);
    for (int a = 0; a < n; ++a) {
      if (starts[a] < 0 || starts[a] + 2 >= T) return false;
      for (int b = 0; b < n; ++b)
        if (a != b && starts[a] == starts[b]) return false;
    }
    for (int a = 1; a < n; ++a)  // sort the starts
      for (int b = a; b > 0 && starts[b - 1] > starts[b]; --b) {
        const int x = starts[b];
        starts[b] = starts[b - 1];
        starts[b - 1] = x;
      }
    for (int k = 0; k + 3 < n; ++k)  // group k+3 reuses the registers of group k
      if (starts[k + 3] - 2 <= starts[k] + 1) return false;
    return true;
  }
};

template <int D, int BM, bool CAUSAL, bool KVLEN, bool GROUPED>
__global__ __launch_bounds__(kKvThreads) void fa_bwd_dkdv_kernel(BwdArgs p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  using L = KvLds<D, BM>;
  constexpr int NCH = D / 8, NCHT = BM / 8;
  constexpr int NQB = BM / 32, NDB = D / 32, NKK = D / 16;
  constexpr uint32_t NAT_QB = 32 * NCH * 16;  // bytes per 32 rows of a natural tile
  constexpr uint32_t TR_DB = 32 * NCHT * 16;  // bytes per 32 rows of a transposed tile
  auto nat_q = [&](int s) { return smem + L::NAT + 2 * s * L::TILE; };
  auto nat_d = [&](int s) { return smem + L::NAT + 2 * s * L::TILE + L::TILE; };
  auto tr_q = [&](int s) { return smem + L::TR + 2 * s * L::TILE; };
  auto tr_d = [&](int s) { return smem + L::TR + 2 * s * L::TILE + L::TILE; };
  auto st_l = [&](int s) { return smem + L::ST + 8 * s * BM; };
  auto st_d = [&](int s) { return smem + L::ST + 8 * s * BM + 4 * BM; };

  const int tid = threadIdx.x;
  // wave index as a scalar: tile copies then compute their LDS destinations in SALU
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, c = l & 31, h = l >> 5;
  // one workgroup per (key block, K/V head); with grouped heads it runs the query tiles
  // of every query head of its group in turn and sums their dK, dV in registers
  // (grouped heads split over nsplit workgroups: workgroup part s runs the group's query
  // heads [s*G/nsplit, (s+1)*G/nsplit) and writes fp32 partials)
  const int BHkv = p.B * p.Hkv;
  const int nsplit = GROUPED ? p.nsplit : 1;
  // no mask: each XCD works through whole heads; causal: key block 0 sees the most
  // queries, so it goes first
  const int nkb = (p.N + kKvBN - 1) / kKvBN;
  int kbi, hs;
  block_order<!CAUSAL>((int)blockIdx.x, nkb, BHkv * nsplit, kbi, hs);
  const int bhk = hs / nsplit, split = hs - bhk * nsplit;
  const int b = bhk / p.Hkv;
  const int N = p.N;
  const int G = GROUPED ? p.H / p.Hkv : 1;          // query heads per K/V head
  const int g_begin = split * G / nsplit, g_end = (split + 1) * G / nsplit;
  const int bq0 = b * p.H + (bhk - b * p.Hkv) * G;  // first query head of the group
  // fp32 partials of this workgroup's split (grouped, nsplit > 1)
  float* const part_dk = GROUPED ? p.part + ((size_t)split * BHkv + bhk) * N * D : nullptr;
  float* const part_dv = GROUPED ? part_dk + (size_t)nsplit * BHkv * N * D : nullptr;
  const size_t head = (size_t)bhk * N * D;          // K, V, dK, dV
  buf_rsrc qg, dog, wlg, wdg;
  auto set_query_head = [&](int g) {
    const size_t qhead = (size_t)(bq0 + g) * N * D;
    qg = make_rsrc(p.q + qhead, (uint32_t)N * D * 2);
    dog = make_rsrc(p.dout + qhead, (uint32_t)N * D * 2);
    wlg = make_rsrc(p.ws_l + (size_t)(bq0 + g) * p.nw, (uint32_t)p.nw * 4);
    wdg = make_rsrc(p.ws_d + (size_t)(bq0 + g) * p.nw, (uint32_t)p.nw * 4);
  };
  set_query_head(g_begin);

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
      if (nsplit > 1) {
        store_ct_rows_f32<D>(part_dk, kcol, dk, 0.f, h);
        store_ct_rows_f32<D>(part_dv, kcol, dv, 0.f, h);
      } else {
        store_ct_rows<D>(p.dk + head, kcol, dk, 0.f, h);
        store_ct_rows<D>(p.dv + head, kcol, dv, 0.f, h);
      }
    }
    return;
  }

  // ---- this lane's key column: K and V fragments (B operands of S and dP)
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

  // Fragment bases.  Natural tiles: lane (c, h) reads row 32*qb + row_perm(c), chunk
  // 2*kk + h; the swizzle depends on kk only through kk % 2.  Transposed tiles: lane
  // reads row 32*db + c, chunk 4*qb + 2*sb + h; the swizzle depends on sb.
  const uint32_t rp = row_perm(c);
  uint32_t nb[2], tb[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    nb[x] = 16 * swz_unit<NCH>(rp, 2 * x + h);
    tb[x] = 16 * swz_unit<NCHT>(c, 2 * x + h);
  }
  // This thread's 8x8 block of the transposition: matrix (waves 0-1 Q, 2-3 dO), row
  // block rc, chunk dc.  The low four lane bits run over (dc % 4, rc % 4): lane bits 3
  // and 0 give dc % 4, bits 1 and 2 give rc % 4 (of the assignments that keep both
  // the reads and the writes free of bank conflicts, measured on gfx950).
  constexpr int NDC4 = NCH / 4;
  const int hi = (l >> 4) + 4 * (w & 1);
  const int tdc = ((l >> 3) & 1) + 2 * (l & 1) + 4 * (hi % NDC4);
  const int trc = ((l >> 1) & 1) + 2 * ((l >> 2) & 1) + 4 * (hi / NDC4);
  const uint32_t t_rd = 16 * swz_unit<NCH>(8 * trc, tdc), t_wr = 16 * swz_unit<NCHT>(8 * tdc, trc);
  const bool t_dO = w >= 2;

  // Direct copies of tile `it` into tile slot s and statistics slot ss: item k <
  // 2*PER_WAVE is one 1 KB wave instruction of Q (k < PER_WAVE) or dO; item 2*PER_WAVE
  // the row statistics (lse2 on even waves, -D on odd ones; with BM = 64 waves 2-3
  // repeat what 0-1 copy).
  using Copy = SwzCopy<BM, D, kKvWaves>;
  constexpr int PER_WAVE = Copy::PER_WAVE;
  constexpr int NDMA = 2 * PER_WAVE + 1;
  auto dma_item = [&](int k, int it, int s, int ss) {
    const int i0 = it * BM;
    if (k < PER_WAVE) {
      Copy::issue(qg, i0, N, nat_q(s), w, l, k);
    } else if (k < 2 * PER_WAVE) {
      Copy::issue(dog, i0, N, nat_d(s), w, l, k - PER_WAVE);
    } else {
      constexpr int SW = BM / 64;  // wave instructions per statistic
      const int which = (w / SW) & 1, part = w % SW, row = i0 + part * 64 + l;
      buf2lds4(which ? wdg : wlg, (uint32_t)row * 4, 0, (which ? st_d(ss) : st_l(ss)) + part * 256);
    }
  };
  auto issue = [&](int it, int s, int ss) {
#pragma unroll
    for (int k = 0; k < NDMA; ++k) dma_item(k, it, s, ss);
  };
  // tile `it` needs the causal mask for this wave iff some query precedes some key
  // P = exp2(S * scale * log2e - lse2) and dS = P * (dP - D) for two query rows
  // (C registers r0, r0 + 1 of sc/dp; `qoff` = first row minus this lane's key)
  auto stat_pair = [&](const unsigned char* st, int row) {
    return __builtin_bit_cast(f32x2, *(const __attribute__((address_space(3))) u32x2*)(
                                          (const __attribute__((address_space(3))) unsigned char*)st + row * 4));
  };

  // ---- software pipeline --------------------------------------------------------
  // Iteration i reduces tile i (slot cs) into dK^T, dV^T while it scores tile i+1 (slot
  // ns), transposes tile i+1 and fetches tile i+2 into slot cs.  It is one flat, fully
  // unrolled stream of T products whose order is pinned with scheduling barriers:
  //   block q of 32 queries:  NS products S, dP (i+1, q)  then  NR products dV^T, dK^T (i, q)
  // with the other work slotted between products:
  //   - operand fragments are read kLook products ahead;
  //   - block q's S products come before its dP products, which start from -D of the
  //     block's rows, read from LDS a few products ahead;
  //   - P, dS of (i+1, q) in eight groups of two rows: groups 0-3 ride on the dV^T, dK^T
  //     products of block q, groups 4-7 on the S, dP products of block q+1 (those of the
  //     last block on the first block of the next iteration), so that every product
  //     slot carries about the same amount of VALU work; each group runs in three
  //     stages on consecutive products (placement in KvSched);
  //   - the direct copies of tile i+2 (every fifth product from 2: a burst of copies
  //     stalls instruction issue; early enough that their latency hides behind the
  //     iteration) and the transposition of tile i+1 (reads
  //     on products 0-7, one 8-row output on every seventh product from 8).
  // P, dS live in two register sets (tile being reduced / tile being scored) whose
  // roles swap every iteration; iterations run in pairs so the set index is a
  // compile-time constant and no register copies are needed.  S, dP are double
  // buffered by block parity.
  constexpr int NS = 2 * NKK, NR = 4 * NDB, NSTEP = NS + NR, T = NQB * NSTEP;
  constexpr int kLook = 6;  // measured: 4 -> 6 about 1% faster
  static_assert(NQB % 2 == 0, "S, dP buffers alternate by block parity");
  // side work spacing (measured): copies every kDmaStep products from 2, transposition
  // writes every kTxStep products from 8
  constexpr int kDmaStep = 5, kTxStep = 7;
  static_assert(8 + kTxStep * 7 < T && 2 + kDmaStep * (NDMA - 1) < T, "extra work must fit in the stream");
  u32x4 ps[2][NQB][2], dss[2][NQB][2];  // P, dS as bf16 pairs: [set][block][16-row half]
  f32x16 sbuf[2], dbuf[2];              // S, dP by block parity

  using Sch = KvSched<NQB, NS, NR>;
  static_assert(Sch::valid(), "P, dS group placement");

  // P = exp2(S * scale * log2e - lse2) and dS = P * (dP - D) for rows 2e, 2e+1 of
  // 16-row half sb of block q (dp holds dP - D), packed to bf16 pairs (not pipelined:
  // prologue, epilogue)
  auto group = [&](auto MASK, const f32x16& sc, const f32x16& dp, int q, int u, f32x2 l2, int tile,
                   u32x4 (&pd_p)[NQB][2], u32x4 (&pd_ds)[NQB][2]) {
    const int sb = u >> 2, e = u & 3, r0 = 8 * sb + 2 * e;
    const int qoff = tile * BM + 32 * q + 16 * sb + 8 * h + 2 * e - kcol;  // query - key of row 2e
    float p0 = fast_exp2(__builtin_fmaf(sc[r0], sl, -l2[0]));
    float p1 = fast_exp2(__builtin_fmaf(sc[r0 + 1], sl, -l2[1]));
    if constexpr (decltype(MASK)::value) {  // key kcol is admissible for query q iff kcol <= q
      p0 = (qoff < 0) ? 0.f : p0;
      p1 = (qoff + 1 < 0) ? 0.f : p1;
    }
    pd_p[q][sb][e] = pack_bf16x2(p0, p1);
    pd_ds[q][sb][e] = pack_bf16x2(p0 * dp[r0], p1 * dp[r0 + 1]);
  };
  auto stat_row = [&](int q, int u) { return 32 * q + 16 * (u >> 2) + 8 * h + 2 * (u & 3); };
  // -D of the 16 query rows whose dP this lane accumulates in block q (C registers 8*sb
  // + j hold row 32*q + 16*sb + 8*h + j): four 16-byte reads straight into the
  // accumulator the block's dP products start from
  auto neg_d = [&](const unsigned char* st, int q) {
    f32x16 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = lds_read128(st, 4 * (32 * q + 16 * (j >> 1) + 8 * h + 4 * (j & 1)));
      // (uint32_t) first: a bit cast straight from a vector element read element 0
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = __builtin_bit_cast(float, (uint32_t)v[e]);
    }
    return x;
  };

  // ---- prologue: fetch tiles i_first and i_first+1, transpose and score i_first
  auto prologue = [&]() {
  issue(i_first, 0, 0);
  issue(min(i_first + 1, i_last - 1), 1, 1);
  wait_vmem();
  __syncthreads();
  transpose8x8(t_dO ? nat_d(0) : nat_q(0), t_rd, t_dO ? tr_d(0) : tr_q(0), t_wr);
  {
    constexpr std::integral_constant<bool, CAUSAL> MK{};  // tile i_first always meets the diagonal
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      f32x16 sc, dp = neg_d(st_d(0), qb);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const uint32_t off = nb[kk & 1] + qb * NAT_QB + (kk >> 1) * 64 * 16;
        const u32x4 aq = lds_read128(nat_q(0), off), ad = lds_read128(nat_d(0), off);
        if (kk == 0) sc = mfma32_vz(aq, kf[kk]);
        else mfma32_vacc(sc, aq, kf[kk]);
        mfma32_vacc(dp, ad, vf[kk]);
      }
      mfma_valu_wait();
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (qb + 1 < NQB || u < 4)  // the last block's groups 4-7 are carried
          group(MK, sc, dp, qb, u, stat_pair(st_l(0), stat_row(qb, u)), i_first, ps[0], dss[0]);
      sbuf[qb & 1] = sc;
      dbuf[qb & 1] = dp;
    }
  }
  __syncthreads();
  };

  // ---- one iteration; PAR = set of the reduced tile, MC / MS = causal mask needed on
  // the reduced (carried groups) / scored tile
  auto iteration = [&](auto PARc, auto MC, auto MS, int i) {
    constexpr int PAR = decltype(PARc)::value;
    const int cs = (i - i_first) & 1, ns = cs ^ 1;
    // statistics slots of tiles i, i+1 (read here) and i+2 (copied here)
    const int r3 = (i - i_first) % 3;
    const int sc = r3, sn = r3 == 2 ? 0 : r3 + 1, s2 = r3 == 0 ? 2 : r3 - 1;
    const int it = i + 1, it2 = min(i + 2, i_last - 1);  // past the end: refetch, unused
    const unsigned char* t_src = t_dO ? nat_d(ns) : nat_q(ns);
    unsigned char* t_dst = t_dO ? tr_d(ns) : tr_q(ns);
    auto aread = [&](int t) -> u32x4 {
      const int q = t / NSTEP, r = t % NSTEP;
      if (r < NS) {  // S products, then dP products
        const int kk = r % NKK;
        return lds_read128((r >= NKK) ? nat_d(ns) : nat_q(ns), nb[kk & 1] + q * NAT_QB + (kk >> 1) * 64 * 16);
      }
      const int m = r - NS, sb = m / (2 * NDB), db = (m >> 1) % NDB;
      return lds_read128((m & 1) ? tr_q(cs) : tr_d(cs), tb[sb] + db * TR_DB + q * 64 * 16);
    };
    // statistics of the group whose first stage runs after op T0 (read two ops ahead)
    auto stat_read = [&](auto t_c, f32x2 (&l2)[3]) {
      constexpr int ua = Sch::unit_at(decltype(t_c)::value), n = Sch::seq(decltype(t_c)::value) % 3;
      constexpr bool carry = ua >= 1000;
      constexpr int q = carry ? NQB - 1 : ua / 16, u = carry ? ua - 1000 : ua % 16;
      l2[n] = stat_pair(carry ? st_l(sc) : st_l(sn), stat_row(q, u));
    };
    u32x4 fr[kLook];
#pragma unroll
    for (int t = 0; t < kLook; ++t) fr[t] = aread(t);
    u32x4 tx[8];
    // P, dS groups in flight, by group sequence number mod 3: lse2, stage A -> B
    // (exponent arguments, dP - D), stage B -> C (P)
    f32x2 sl2[3], ga[3], gd[3], gp[3];
    static_for<2>([&](auto tc) {
      if constexpr (Sch::unit_at(decltype(tc)::value) >= 0) stat_read(tc, sl2);
    });
    static_for<T>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      constexpr int q = t / NSTEP, r = t % NSTEP;
      const u32x4 a = fr[t % kLook];
      if constexpr (t + kLook < T) fr[t % kLook] = aread(t + kLook);
      if constexpr (t < 8) tx[t] = lds_read128(t_src, t_rd ^ (16u * t));
      if constexpr (t >= 8 && (t - 8) % kTxStep == 0 && (t - 8) / kTxStep < 8) {
        constexpr int jj = (t - 8) / kTxStep;
        u32x4 y;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
          y[pp] = (jj & 1) ? hi16_pair(tx[2 * pp][jj >> 1], tx[2 * pp + 1][jj >> 1])
                           : lo16_pair(tx[2 * pp][jj >> 1], tx[2 * pp + 1][jj >> 1]);
        lds_write128(t_dst, t_wr ^ (16u * jj), y);
      }
      if constexpr (t >= 2 && (t - 2) % kDmaStep == 0 && (t - 2) / kDmaStep < NDMA)
        dma_item((t - 2) / kDmaStep, it2, cs, s2);
      // -D into block q's dP accumulator: block 0's statistics landed before the last
      // barrier; block q+1's accumulator is free once the groups of the block before it
      // (same parity) have read it, by op 3 + 3*NS/4 of block q
      if constexpr (r == 0 && q == 0) dbuf[0] = neg_d(st_d(sn), 0);
      if constexpr (q + 1 < NQB && r == 4 + 3 * NS / 4) dbuf[(q + 1) & 1] = neg_d(st_d(sn), q + 1);
      if constexpr (t + 2 < T && Sch::unit_at(t + 2) >= 0)
        stat_read(std::integral_constant<int, t + 2>{}, sl2);
      // first read of block q's S, dP by VALU code: the products are inline assembly,
      // so the wait states after the last of them are explicit
      if constexpr (Sch::unit_at(t) >= 0 && Sch::unit_at(t) < 1000 && Sch::unit_at(t) % 16 == 0) mfma_valu_wait();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (r < NS) {
        // vector-register accumulators: the P, dS groups read them with VALU code
        if constexpr (r >= NKK) {
          mfma32_vacc(dbuf[q & 1], a, vf[r - NKK]);
        } else {
          if constexpr (r == 0) sbuf[q & 1] = mfma32_vz(a, kf[r]);
          else mfma32_vacc(sbuf[q & 1], a, kf[r]);
        }
      } else {
        constexpr int m = r - NS, sb = m / (2 * NDB), db = (m >> 1) % NDB;
        if constexpr (m & 1) dk[db] = mfma32(a, dss[PAR][q][sb], dk[db]);
        else dv[db] = mfma32(a, ps[PAR][q][sb], dv[db]);
      }
      // P, dS groups: stage C of the group started two ops ago, B of the one started
      // one op ago, A of the one starting now
      constexpr int uC = Sch::unit_at(t - 2), uB = Sch::unit_at(t - 1), uA = Sch::unit_at(t);
      if constexpr (uC >= 0) {
        constexpr int n = Sch::seq(t - 2) % 3;
        constexpr bool carry = uC >= 1000;
        constexpr int gq = carry ? NQB - 1 : uC / 16, gu = carry ? uC - 1000 : uC % 16;
        const uint32_t pv = pack_bf16x2(gp[n][0], gp[n][1]);
        const uint32_t dv_ = pack_bf16x2(gp[n][0] * gd[n][0], gp[n][1] * gd[n][1]);
        constexpr int set = carry ? PAR : (PAR ^ 1);
        ps[set][gq][gu >> 2][gu & 3] = pv;
        dss[set][gq][gu >> 2][gu & 3] = dv_;
      }
      if constexpr (uB >= 0) {
        constexpr int n = Sch::seq(t - 1) % 3;
        constexpr bool carry = uB >= 1000;
        constexpr int gq = carry ? NQB - 1 : uB / 16, gu = carry ? uB - 1000 : uB % 16;
        float p0 = fast_exp2(ga[n][0]), p1 = fast_exp2(ga[n][1]);
        constexpr bool mask = carry ? decltype(MC)::value : decltype(MS)::value;
        if constexpr (mask) {  // key kcol is admissible for query q iff kcol <= q
          const int qoff = (carry ? i : it) * BM + stat_row(gq, gu) - kcol;
          p0 = (qoff < 0) ? 0.f : p0;
          p1 = (qoff + 1 < 0) ? 0.f : p1;
        }
        gp[n] = f32x2{p0, p1};
      }
      if constexpr (uA >= 0) {
        constexpr int n = Sch::seq(t) % 3;
        constexpr bool carry = uA >= 1000;
        constexpr int gq = carry ? NQB - 1 : uA / 16, gu = carry ? uA - 1000 : uA % 16;
        constexpr int r0 = 8 * (gu >> 2) + 2 * (gu & 3);
        ga[n] = f32x2{__builtin_fmaf(sbuf[gq & 1][r0], sl, -sl2[n][0]), __builtin_fmaf(sbuf[gq & 1][r0 + 1], sl, -sl2[n][1])};
        gd[n] = f32x2{dbuf[gq & 1][r0], dbuf[gq & 1][r0 + 1]};
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    wait_vmem();
    __syncthreads();
  };
  // last tile: carried groups, then its dV^T, dK^T products (set 0)
  auto epilogue = [&](auto MC, int i) {
    const int cs = (i - i_first) & 1, sc = (i - i_first) % 3;
#pragma unroll
    for (int u = 4; u < 8; ++u)
      group(MC, sbuf[(NQB - 1) & 1], dbuf[(NQB - 1) & 1], NQB - 1, u, stat_pair(st_l(sc), stat_row(NQB - 1, u)), i,
            ps[0], dss[0]);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint32_t off = tb[sb] + db * TR_DB + qb * 64 * 16;
          dv[db] = mfma32(lds_read128(tr_d(cs), off), ps[0][qb][sb], dv[db]);
          dk[db] = mfma32(lds_read128(tr_q(cs), off), dss[0][qb][sb], dk[db]);
        }
  };
  auto copy_set = [&](int from, int to) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        ps[to][qb][sb] = ps[from][qb][sb];
        dss[to][qb][sb] = dss[from][qb][sb];
      }
  };
  // Causal: only tiles i_first and i_first+1 can hold queries before some key of the
  // workgroup (its first key is i_first * BM and it spans 128 keys), so the mask is
  // needed in the first two iterations at most; they run masked for every wave (the
  // mask is exact where it is not needed).
  constexpr std::integral_constant<bool, CAUSAL> C{};
  constexpr std::false_type F{};
  constexpr std::integral_constant<int, 0> P0{};
  constexpr std::integral_constant<int, 1> P1{};
  if constexpr (GROUPED) {
    // The query heads of the group run one after another, each through the whole
    // pipeline; dK, dV keep accumulating.  Causal: every iteration runs masked (exact
    // where no mask is needed), which keeps to two iteration variants.
    constexpr std::integral_constant<bool, CAUSAL> M{};
    for (int g = g_begin; g < g_end; ++g) {
      if (g > g_begin) {
        // the previous head's epilogue has read its last tiles before the copies refill them
        __syncthreads();
        set_query_head(g);
      }
      prologue();
      int i = i_first;
      for (; i + 2 < i_last; i += 2) {
        iteration(P0, M, M, i);
        iteration(P1, M, M, i + 1);
      }
      if (i + 1 < i_last) {
        iteration(P0, M, M, i);
        ++i;
        copy_set(1, 0);
      }
      epilogue(M, i);
    }
  } else {
    prologue();
    int i = i_first;
    bool last_masked = CAUSAL;  // mask state of the tile left for the epilogue
    if (i + 1 < i_last) {
      iteration(P0, C, C, i);  // reduces set 0, scores into set 1
      ++i;
      if (i + 1 < i_last) {
        iteration(P1, C, F, i);  // reduces set 1, scores into set 0
        ++i;
        last_masked = false;
        for (; i + 2 < i_last; i += 2) {
          iteration(P0, F, F, i);
          iteration(P1, F, F, i + 1);
        }
        if (i + 1 < i_last) {
          iteration(P0, F, F, i);
          ++i;
          copy_set(1, 0);
        }
      } else {
        copy_set(1, 0);
      }
    }
    if (CAUSAL && last_masked) epilogue(C, i);
    else epilogue(F, i);
  }
  if (col_store) {
    // keys padded away for every query get exact (+0) zeros: selected, not multiplied,
    // since whatever a padded key row holds (inf, NaN) went into its accumulators
    if (!col_live) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
      }
    }
    if (nsplit > 1) {
      store_ct_rows_f32<D>(part_dk, kcol, dk, col_live ? p.scale : 0.f, h);
      store_ct_rows_f32<D>(part_dv, kcol, dv, col_live ? 1.f : 0.f, h);
    } else {
      store_ct_rows<D>(p.dk + head, kcol, dk, col_live ? p.scale : 0.f, h);
      store_ct_rows<D>(p.dv + head, kcol, dv, col_live ? 1.f : 0.f, h);
    }
  }
}

// --------------------------------------------------------------------------------------
// launch 3 (grouped K/V heads split over several workgroups only): dK, dV = the sum of
// the nsplit fp32 partials, in split order (deterministic), rounded to bf16.  Eight
// consecutive elements per thread; the element count is a multiple of 8 (d is).
// --------------------------------------------------------------------------------------
constexpr int kReduceThreads = 256;

__global__ __launch_bounds__(kReduceThreads) void fa_bwd_kv_reduce_kernel(const float* __restrict__ part,
                                                                         uint16_t* __restrict__ dk,
                                                                         uint16_t* __restrict__ dv, size_t n,
                                                                         int nsplit) {
  const size_t e = ((size_t)blockIdx.x * kReduceThreads + threadIdx.x) * 8;  // over [dK | dV]
  if (e >= 2 * n) return;
  const bool is_v = e >= n;
  const size_t off = is_v ? e - n : e;
  const float* src = part + (is_v ? (size_t)nsplit * n : 0) + off;
  f32x4 a = *(const f32x4*)src, b4 = *(const f32x4*)(src + 4);
  for (int s = 1; s < nsplit; ++s) {
    a += *(const f32x4*)(src + (size_t)s * n);
    b4 += *(const f32x4*)(src + (size_t)s * n + 4);
  }
  const u32x4 out = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b4[0], b4[1]),
                     pack_bf16x2(b4[2], b4[3])};
  *(u32x4*)((is_v ? dv : dk) + off) = out;
}

// --------------------------------------------------------------------------------------
template <typename K>
hipError_t set_lds(K kern, size_t lds) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

template <int D, int BN, int BM, bool CAUSAL, bool KVLEN>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream, int passes) {
  const unsigned bh = (unsigned)(a.B * a.H);
  const unsigned dq_grid8 = (unsigned)((a.N + kDqBM - 1) / kDqBM) * bh;
  if ((passes & 1) && D == 128 && split_small_grid(dq_grid8, CAUSAL)) {
    constexpr size_t lds = 2 * (4ull * BN * D * 2 + (kDqWaves / 2) * 32 * 16);
    auto kern = fa_bwd_dq_kernel<D, BN, CAUSAL, KVLEN, D == 128 ? 2 : 1>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((a.N + kDqBM / 2 - 1) / (kDqBM / 2)) * bh;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kDqThreads), lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (passes & 1) {
    constexpr size_t lds = 4ull * BN * D * 2 + kDqWaves * 32 * 16;
    auto kern = fa_bwd_dq_kernel<D, BN, CAUSAL, KVLEN, 1>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(dq_grid8), dim3(kDqThreads), lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (passes & 2) {
    constexpr size_t lds = KvLds<D, BM>::BYTES;
    const bool grouped = a.Hkv != a.H;
    auto kern = grouped ? fa_bwd_dkdv_kernel<D, BM, CAUSAL, KVLEN, true>
                        : fa_bwd_dkdv_kernel<D, BM, CAUSAL, KVLEN, false>;
    hipError_t e = set_lds(kern, lds);
    if (e != hipSuccess) return e;
    const int nsplit = grouped ? a.nsplit : 1;
    const unsigned grid = (unsigned)((a.N + kKvBN - 1) / kKvBN) * (unsigned)(a.B * a.Hkv * nsplit);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kKvThreads), lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess || nsplit == 1) return e;
    const size_t n = (size_t)a.B * a.Hkv * a.N * D;
    const unsigned rgrid = (unsigned)((2 * n / 8 + kReduceThreads - 1) / kReduceThreads);
    hipLaunchKernelGGL(fa_bwd_kv_reduce_kernel, dim3(rgrid), dim3(kReduceThreads), 0, stream, a.part, a.dk, a.dv, n,
                       nsplit);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D, int BN, int BM>
hipError_t dispatch_masks(const BwdArgs& a, hipStream_t s, int ps) {
  const bool kv = a.kv_len != nullptr;
  if (a.causal) return kv ? launch_bwd<D, BN, BM, true, true>(a, s, ps) : launch_bwd<D, BN, BM, true, false>(a, s, ps);
  return kv ? launch_bwd<D, BN, BM, false, true>(a, s, ps) : launch_bwd<D, BN, BM, false, false>(a, s, ps);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream, int passes) {
  if (a.d == 128) return dispatch_masks<128, 64, 64>(a, stream, passes);
  return dispatch_masks<64, 128, 128>(a, stream, passes);
}

}  // namespace fa355
