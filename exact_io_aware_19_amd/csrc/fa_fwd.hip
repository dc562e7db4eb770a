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
#include <type_traits>

#include "common.hpp"
#include "fa_kernels.hpp"

namespace fa355 {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr int kBM = kWaves * kRowsPerWave;  // query rows per workgroup
// Conditional rescaling threshold in log2 units (FlashAttention-4 summary, second
// optimisation; wiki page, FA4 (2)): the reference max moves only when a row max grows
// by more than this, so un-normalised probabilities stay below 2^8.
constexpr float kRescaleTau = 8.0f;
constexpr float kRescaleLimit = 256.0f;  // 2^kRescaleTau
constexpr int kLdsTiles = 4;  // 2 K tiles + 2 V^T tiles

// P = exp2(s * scale * log2e - m_ref) of one lane's 16*NKB scores of a tile, packed to
// bf16 pairs (the B operand of O^T += V^T P^T); returns the lane's share of the tile's
// row sum, from the unrounded fp32 P (the log-sum-exp the backward recomputes P from
// must be accurate to fp32, not to bf16), as a tree (a serial chain would leave the
// VALU idle between dependent issues).
template <int NKB>
__device__ __forceinline__ float tile_probs(const f32x16 (&s)[NKB], float sl, float m_ref, u32x4 (&pk)[NKB][2]) {
  float t[8 * NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb][8 * sb + 2 * i], sl, -m_ref));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb][8 * sb + 2 * i + 1], sl, -m_ref));
        pk[kb][sb][i] = pack_bf16x2(p0, p1);
        t[8 * kb + 4 * sb + i] = p0 + p1;
      }
#pragma unroll
  for (int n = 4 * NKB; n >= 1; n >>= 1)
#pragma unroll
    for (int i = 0; i < n; ++i) t[i] = t[i] + t[i + n];
  return t[0];
}

// Online-softmax step of one tile for one wave: P of the tile's (masked) scores s into
// pk, and the row state -- reference max m_run in scaled-log2 units, this lane's partial
// row sum l_run, output accumulators o -- updated.  Conditional rescaling
// (FlashAttention-4 summary, second optimisation; wiki page, FA4 (2)): the reference
// moves only when some row max exceeds it by more than tau; results are exact for any
// reference (it cancels in O and is added back in the LSE) and tau bounds the
// un-normalised P by 2^tau.
//   GATED (the 8-wave kernel, whose softmax runs in a phase of its own): P is first
//   formed against the current reference; each P is at most its lane's share of the
//   tile sum, so when no share exceeds 2^tau (and every row has a reference) the
//   reference stays, P is final and the row max (a tree of three-input maxima over the
//   raw scores, which s still holds) is not needed; otherwise it decides as below.
//   Not gated (the small-grid kernel, whose products follow in the same wave and
//   overlap the exponentials): row max first, then P.
// Both give the same P, sums and outputs; they can differ only where P = 2^tau lies
// within rounding of the threshold, where either reference is exact.
template <bool GATED, int NKB, int NDB>
__device__ __forceinline__ void softmax_tile(const f32x16 (&s)[NKB], float sl, float& m_run, float& l_run,
                                             f32x16 (&o)[NDB], u32x4 (&pk)[NKB][2]) {
  float lt = 0.f;
  if constexpr (GATED) {
    lt = tile_probs<NKB>(s, sl, (m_run == -INFINITY) ? 0.f : m_run, pk);
    if (!__any(!(lt <= kRescaleLimit) || m_run == -INFINITY)) {
      l_run += lt;
      return;
    }
  }
  float mx = tree_max<NKB>(s);
  mx = half_max(mx) * sl;
  const bool moved = __any(mx > m_run + kRescaleTau);
  if (moved) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;
  }
  if (!GATED || moved) lt = tile_probs<NKB>(s, sl, (m_run == -INFINITY) ? 0.f : m_run, pk);
  l_run += lt;
}

// SPLIT (small d = 128 grids): 128 query rows per workgroup; both wave groups own the
// same rows (wave w: rows 32 * (w % 4) ..) and group g streams the g-th half of the key
// tiles through LDS rings of its own, one phase apart as above; at the end the second
// group's (m, l, O) is merged into the first's through LDS.  The schedule, the barriers
// and the per-tile work of each wave are those of the unsplit kernel.
template <int D, int BN, bool CAUSAL, bool KVLEN, bool SPLIT = false>
__global__ __launch_bounds__(kThreads) void fa_fwd_kernel(FwdArgs p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int TILE_BYTES = BN * D * 2;  // one K tile or one V^T tile
  constexpr int NKB = BN / 32;            // 32-key blocks per tile
  constexpr int NDB = D / 32;             // 32-row blocks of the head dim
  constexpr int NKK = D / 16;             // k-steps of the QK^T contraction
  constexpr int BM = SPLIT ? kBM / 2 : kBM;  // query rows per workgroup
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, c = l & 31, h = l >> 5;
  const int grp = w >> 2, wg = w & 3;  // wave group (one wave per SIMD) and wave in it
  const int wr = SPLIT ? wg : w;        // this wave's 32-row slice of the block
  // LDS: 2-deep rings of K tiles (natural) at [0, 2*TILE_BYTES) and of V^T tiles at
  // [2*TILE_BYTES, 4*TILE_BYTES) (SPLIT: a ring pair per wave group)
  unsigned char* const gsm = SPLIT ? smem + (size_t)grp * kLdsTiles * TILE_BYTES : smem;
  auto kbuf = [&](int i) { return gsm + i * TILE_BYTES; };
  auto vbuf = [&](int i) { return gsm + (2 + i) * TILE_BYTES; };

  const int BH = p.B * p.H;
  const int nqb = (p.N + BM - 1) / BM;
  // no mask: each XCD works through whole heads; causal: heaviest query blocks first
  int blk, bh;
  block_order<!CAUSAL>((int)blockIdx.x, nqb, BH, blk, bh);
  const int qbi = CAUSAL ? (nqb - 1 - blk) : blk;
  const int b = bh / p.H;
  const int N = p.N, Nk = p.Nk;
  const size_t head = (size_t)bh * N * D;
  // grouped K/V heads: the H / Hkv query heads of a group share one K/V head
  const size_t kv_head = (size_t)(b * p.Hkv + (bh - b * p.H) / (p.H / p.Hkv)) * Nk * D;
  const uint16_t* __restrict__ qg = p.q + head;
  const buf_rsrc kg = make_rsrc(p.k + kv_head, (uint32_t)Nk * D * 2);
  const buf_rsrc vg = make_rsrc(p.v + kv_head, (uint32_t)Nk * D * 2);

  int kv_end = Nk;
  if constexpr (KVLEN) kv_end = min(max(p.kv_len[b], 0), Nk);
  const int q0 = qbi * BM;
  const int qrow = q0 + wr * kRowsPerWave + c;  // this lane's query row
  // causal positions: query row i sits at key position q_off + i
  const int cq0 = q0 + p.q_off, cqrow = qrow + p.q_off;
  int kend = kv_end;
  if constexpr (CAUSAL) kend = min(kend, cq0 + BM);
  const int ntiles = (kend + BN - 1) / BN;
  // keys past wave_kend are masked for every row of this wave (tile skipping)
  int wave_kend = kend;
  if constexpr (CAUSAL) wave_kend = min(kend, cq0 + wr * kRowsPerWave + kRowsPerWave);
  // this group's tiles [jb, je); both groups run `nt` tile steps (SPLIT: the second
  // group's last one is empty when the count is odd)
  const int nt = SPLIT ? (ntiles + 1) / 2 : ntiles;
  const int jb = SPLIT ? grp * nt : 0, je = SPLIT ? min(ntiles, jb + nt) : ntiles;

  if (ntiles == 0) {  // no admissible key for any row of this block (kv_len == 0)
    if ((!SPLIT || grp == 0) && qrow < N) {
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
      const u32x4 t = *(const u32x4*)(src + 16 * kk);
      qf[kk] = ok ? ((t & p.op_and) ^ p.op_xor) : u32x4{0, 0, 0, 0};  // sign of the scale
    }
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // reference max of scaled-log2 scores (at most kRescaleTau below the true max)
  float l_run = 0.f;        // this lane's partial row sum (the other half-wave holds the rest)
  const float sl = p.scale_log2;

  // V^T: each group transposes half of every tile (SPLIT: each group all of its own)
  constexpr int NVH = SPLIT ? 2 : 1;
  VtHalf<BN, D> vh[NVH];
#pragma unroll
  for (int x = 0; x < NVH; ++x) vh[x].init(tid & 255, SPLIT ? x : grp);
  auto v_fetch = [&](int row0) {
#pragma unroll
    for (int x = 0; x < NVH; ++x) vh[x].fetch(vg, row0, kv_end);
  };
  auto v_store = [&](unsigned char* tile, int k) {  // k < 4 * NVH
    vh[k / 4].store(tile, k % 4);
  };
  // one wave-instruction of the K tile copy by wave group 0 (4 per wave)
  constexpr int KCOPY = BN * (D / 8) / (4 * 64);
  auto k_copy = [&](int row0, unsigned char* tile, int ii) {
    const int pos = (ii * 4 + wg) * 64 + l;  // unit index written by this lane
    const int blk = pos / (16 * (D / 8)), rem = pos % (16 * (D / 8));
    const int row = min(blk * 16 + (rem & 15), kv_end - 1 - row0);  // padded rows never read
    // the LDS destination (M0) and the tile offset (soffset) are wave-uniform
    const int slot = __builtin_amdgcn_readfirstlane(ii * 4 + wg);
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)row0 * (D * 2));
    buf2lds16(kg, (uint32_t)(row * (D * 2) + (rem >> 4) * 16), soff, tile + (size_t)slot * 64 * 16);
  };
  const uint32_t kfrag = NatFrag<D>::base(c, h);  // K tile, A operand of S^T
  const uint32_t vfrag[2] = {TrFrag<BN>::base(c, h, 0), TrFrag<BN>::base(c, h, 1)};  // V^T tile, A operand of O^T

  // ---- the two operations of the tile pipeline ------------------------------------
  u32x4 pk[NKB][2];  // P of the tile between its softmax and its P V product

  // MFMA operation for tile j: O += V_j^T P_j (P from the preceding softmax), then the
  // scores of tile j + 1 into `s`.  The operand fragments stream from LDS with a fixed
  // look-ahead: fragment i + kLook is requested before MFMA i issues, so each MFMA waits
  // only for a read issued kLook MFMAs (~kLook * 32 cycles) earlier.
  constexpr int NPV = NKB * 2 * NDB;  // P V^T MFMAs of one tile
  constexpr int NS = NKB * NKK;       // Q K^T MFMAs of one tile
  constexpr int kLook = 4;
  f32x16 s[NKB];  // scores of the next tile to go through the softmax
  auto mfma_stream = [&](auto first_c, auto count_c, const unsigned char* vb_, const unsigned char* kt, auto&& side) {
    constexpr int F = decltype(first_c)::value, M = decltype(count_c)::value;
    // flat MFMA index i: [0, NPV) = P V^T (kb, sb, db), [NPV, NPV+NS) = Q K^T (kk, kb)
    auto read_frag = [&](int i) -> u32x4 {
      if (i < NPV) {
        const int kb = i / (2 * NDB), sb = (i / NDB) % 2, db = i % NDB;
        return lds_read128(vb_, vfrag[db & 1] + db * TrFrag<BN>::DB + (4 * kb + 2 * sb) * TrFrag<BN>::CH);
      }
      const int kk = (i - NPV) / NKB, kb = (i - NPV) % NKB;
      return lds_read128(kt, kfrag + kb * NatFrag<D>::BLK + kk * NatFrag<D>::KK);
    };
    u32x4 fr[kLook];
#pragma unroll
    for (int i = 0; i < kLook && i < M; ++i) fr[i] = read_frag(F + i);
    static_for<M>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const u32x4 a = fr[i % kLook];
      if constexpr (i + kLook < M) fr[i % kLook] = read_frag(F + i + kLook);
      __builtin_amdgcn_sched_barrier(0);
      constexpr int fi = F + i;
      if constexpr (fi < NPV) {
        constexpr int kb = fi / (2 * NDB), sb = (fi / NDB) % 2, db = fi % NDB;
        o[db] = mfma32(a, pk[kb][sb], o[db]);
      } else {
        // kb fastest: the NKB accumulation chains alternate, so no MFMA waits on the
        // result of the one issued just before it
        constexpr int kk = (fi - NPV) / NKB, kb = (fi - NPV) % NKB;
        s[kb] = mfma32(a, qf[kk], kk == 0 ? f32x16{} : s[kb]);
      }
      side(std::integral_constant<int, i>{}, std::integral_constant<int, M>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // Tile movement rides on the MFMA operation: operation j of a wave group writes its
  // half of V_{j+1}^T (fetched into registers during its preceding softmax), and wave
  // group 0 also starts the copy of K_{j+2}.  Both spread over the MFMA stream, a few
  // products apart, so no wave stalls on a burst of memory instructions.
  //
  // The V^T stores are unconditional, so the stream has no branches: operation -1 stores
  // V_0 (fetched before the loop), and the store of the last operation rewrites a
  // buffer no later phase reads.  The K copy is chosen per stream at compile time.
  auto op_mfma = [&](int j) {  // j = -1: scores of the group's first tile only
    const bool do_pv = j >= 0 && jb + j < je && (jb + j) * BN < wave_kend;
    const int jn = j + 1;
    const bool do_s = jb + jn < je && (jb + jn) * BN < wave_kend;
    unsigned char* vnext = vbuf(jn & 1);
    unsigned char* knext = kbuf(j & 1);
    const int krow = (jb + j + 2) * BN;
    const unsigned char* vb_ = vbuf(j & 1);
    const unsigned char* kt = kbuf(jn & 1);
    auto run = [&](auto cpk) {
      constexpr bool CPK = decltype(cpk)::value;
      auto side = [&](auto ic, auto mc) {
        constexpr int i = decltype(ic)::value, SP = decltype(mc)::value / 16;
        // placement (measured): the V^T column stores late in a full stream (products
        // 24, 26, 28, 30 of 32; SPLIT: 8 stores from 16), the K copies one every four
        // products from 2
        constexpr int NVS = 4 * NVH;
        constexpr int V0 = SP == 2 ? 32 - 2 * NVS : 1, K0 = 2;
        if constexpr (i >= V0 && (i - V0) % 2 == 0 && (i - V0) / 2 < NVS) v_store(vnext, (i - V0) / 2);
        if constexpr (CPK && i >= K0 && (i - K0) % 4 == 0 && (i - K0) / 4 < KCOPY) k_copy(krow, knext, (i - K0) / 4);
      };
      if (do_pv && do_s) mfma_stream(std::integral_constant<int, 0>{}, std::integral_constant<int, NPV + NS>{}, vb_, kt, side);
      else if (do_pv) mfma_stream(std::integral_constant<int, 0>{}, std::integral_constant<int, NPV>{}, vb_, kt, side);
      else if (do_s) mfma_stream(std::integral_constant<int, NPV>{}, std::integral_constant<int, NS>{}, vb_, kt, side);
      else {
#pragma unroll
        for (int c4 = 0; c4 < 4 * NVH; ++c4) v_store(vnext, c4);
        if constexpr (CPK) {
#pragma unroll
          for (int ii = 0; ii < KCOPY; ++ii) k_copy(krow, knext, ii);
        }
      }
    };
    // K_{j+2}: wave group 0 copies it for both groups (SPLIT: each group its own)
    if ((SPLIT || grp == 0) && jb + j + 2 < je) run(std::true_type{});
    else run(std::false_type{});
  };

  // VALU operation for tile j: mask, online softmax with conditional rescaling, P -> pk.
  auto op_softmax = [&](int j) {
    const int kt0 = (jb + j) * BN;
    if (jb + j >= je || kt0 >= wave_kend) return;
    bool need_mask = kt0 + BN > kv_end;
    if constexpr (CAUSAL) need_mask = need_mask || (kt0 + BN - 1 > cq0 + wr * kRowsPerWave);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + 32 * kb + c_row(r, h);
          bool bad = key >= kv_end;
          if constexpr (CAUSAL) bad = bad || key > cqrow;
          s[kb][r] = bad ? -INFINITY : s[kb][r];
        }
    }
    softmax_tile<true, NKB, NDB>(s, sl, m_run, l_run, o, pk);
  };

  // ---- phase schedule ---------------------------------------------------------------
  // Every wave runs  [S_0] softmax_0 [PV_0,S_1] softmax_1 [PV_1,S_2] ...  Waves 0-3
  // (group 0) and 4-7 (group 1) hold one wave per SIMD each and run this sequence one
  // phase apart, so in every phase one wave of each SIMD issues MFMAs while the other
  // runs the softmax on the VALU.  Each phase ends with a workgroup barrier.
  // MFMA operation j (PV_j, S_{j+1}) runs in phase 2j+2 (group 0) and 2j+3 (group 1).
  // Tile movement:
  //   V_{j+1}: each group fetches its half into registers at the start of its softmax_j
  //            and writes it transposed during its MFMA operation j (phases 2j+2, 2j+3);
  //   K_{j+2}: group 0 starts the copy during its MFMA operation j (phase 2j+2) and
  //            waits for it at the end of its softmax_{j+1} (phase 2j+3).
  // Both land before the barrier that ends phase 2j+3, in buffers whose previous
  // contents (V_{j-1}, K_j) were last read in phase 2j+1, so both rings are two deep.
  // V_0 is fetched here and written by MFMA operation -1 (phases 0 and 1).
  if constexpr (SPLIT) {
    if (jb < je) {
      load_nat_tile<BN, D, 4>(kg, jb * BN, kv_end, kbuf(0), wg, l);
      v_fetch(jb * BN);
    }
  } else {
    load_nat_tile<BN, D, kWaves>(kg, 0, kv_end, kbuf(0), w, l);
    v_fetch(0);
  }
  wait_vmem();
  __syncthreads();
  // operation index of group 0 in phase ph is ph, of group 1 is ph - 1:
  //   op 0 = S_0, op 2j+1 = softmax_j, op 2j+2 = (PV_j, S_{j+1})
  for (int ph = 0; ph < 2 * nt + 2; ++ph) {
    const int op = ph - grp;
    if (op >= 0) {
      if (op & 1) {
        const int j = op >> 1;
        if (jb + j + 1 < je) v_fetch((jb + j + 1) * BN);
        op_softmax(j);
        if (SPLIT || grp == 0) wait_vmem();
      } else {
        op_mfma((op >> 1) - 1);
      }
    }
    lds_barrier();
  }
  if constexpr (SPLIT) {
    // merge: group 1 leaves (m, l, O) of each lane in LDS (the tiles are free after the
    // loop's last barrier); group 0 rescales both to the larger reference
    float* xo = (float*)smem + (size_t)(wg * 64 + l) * (16 * NDB + 2);
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[16 * db + r] = o[db][r];
      xo[16 * NDB] = m_run;
      xo[16 * NDB + 1] = l_run;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xo[16 * NDB], l1 = xo[16 * NDB + 1];
    const float mm = fmaxf(m_run, m1);
    const float mr = (mm == -INFINITY) ? 0.f : mm;
    const float a0 = fast_exp2(m_run - mr), a1 = fast_exp2(m1 - mr);
    m_run = mm;
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + xo[16 * db + r] * a1;
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

// ---------------------------------------------------------------------------------
// Small-grid forward: 4 waves (one per SIMD) = 128 query rows per workgroup, two
// workgroups per CU, a straight tile loop (copy tile j+1 | S_j, softmax, P V_j | store
// V_{j+1}^T | barrier).  Each wave computes exactly what it computes in the unsplit
// kernel above (same rows, tiles, order and arithmetic: outputs equal bit for bit,
// tested); the smaller workgroups fill the GPU better where the 8-wave grid is small.  Measured on one
// box (ms, 8-wave -> this kernel): BERT-shaped (8,16,512,64, padded) 0.0173 -> 0.0158,
// GPT-2-shaped causal (8,12,1024,64) 0.0331 -> 0.0288, (1,2,128,64) 0.0070 -> 0.0053;
// slower on large grids (d=128, N=8192: 1.06 -> 1.18; d=64, N=65536 causal: 9.86 ->
// 10.44) and at d=128, N=2048 (0.0725 -> 0.0815).
// ---------------------------------------------------------------------------------
constexpr int kW2 = 4;                    // waves per workgroup (one per SIMD)
constexpr int kBM2 = kW2 * kRowsPerWave;  // query rows per workgroup
template <int D, int BN, bool CAUSAL, bool KVLEN>
__global__ __launch_bounds__(kW2 * 64, 2) void fa_fwd_small_kernel(FwdArgs p) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int NKB = BN / 32, NDB = D / 32, NKK = D / 16;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, c = l & 31, h = l >> 5;
  auto kbuf = [&](int i) { return smem + i * TILE_BYTES; };
  auto vbuf = [&](int i) { return smem + (2 + i) * TILE_BYTES; };
  const int BH = p.B * p.H;
  const int nqb = (p.N + kBM2 - 1) / kBM2;
  int blk, bh;
  block_order<!CAUSAL>((int)blockIdx.x, nqb, BH, blk, bh);
  const int qbi = CAUSAL ? (nqb - 1 - blk) : blk;
  const int b = bh / p.H;
  const int N = p.N, Nk = p.Nk;
  const size_t head = (size_t)bh * N * D;
  const size_t kv_head = (size_t)(b * p.Hkv + (bh - b * p.H) / (p.H / p.Hkv)) * Nk * D;
  const uint16_t* __restrict__ qg = p.q + head;
  const buf_rsrc kg = make_rsrc(p.k + kv_head, (uint32_t)Nk * D * 2);
  const buf_rsrc vg = make_rsrc(p.v + kv_head, (uint32_t)Nk * D * 2);

  int kv_end = Nk;
  if constexpr (KVLEN) kv_end = min(max(p.kv_len[b], 0), Nk);
  const int q0 = qbi * kBM2;
  const int qrow = q0 + w * kRowsPerWave + c;
  const int cq0 = q0 + p.q_off, cqrow = qrow + p.q_off;  // causal positions
  int kend = kv_end;
  if constexpr (CAUSAL) kend = min(kend, cq0 + kBM2);
  const int ntiles = (kend + BN - 1) / BN;
  int wave_kend = kend;
  if constexpr (CAUSAL) wave_kend = min(kend, cq0 + w * kRowsPerWave + kRowsPerWave);

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

  u32x4 qf[NKK];
  {
    const bool ok = qrow < N;
    const uint16_t* src = qg + (size_t)(ok ? qrow : 0) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 t = *(const u32x4*)(src + 16 * kk);
      qf[kk] = ok ? ((t & p.op_and) ^ p.op_xor) : u32x4{0, 0, 0, 0};  // sign of the scale
    }
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float sl = p.scale_log2;

  VtHalf<BN, D> vh[2];
  vh[0].init(tid, 0);
  vh[1].init(tid, 1);
  const uint32_t kfrag = NatFrag<D>::base(c, h);
  const uint32_t vfrag[2] = {TrFrag<BN>::base(c, h, 0), TrFrag<BN>::base(c, h, 1)};

  load_nat_tile<BN, D, kW2>(kg, 0, kv_end, kbuf(0), w, l);
  vh[0].fetch(vg, 0, kv_end);
  vh[1].fetch(vg, 0, kv_end);
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    vh[0].store(vbuf(0), c4);
    vh[1].store(vbuf(0), c4);
  }
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const bool nxt = j + 1 < ntiles;
    if (nxt) {
      load_nat_tile<BN, D, kW2>(kg, (j + 1) * BN, kv_end, kbuf((j + 1) & 1), w, l);
      vh[0].fetch(vg, (j + 1) * BN, kv_end);
      vh[1].fetch(vg, (j + 1) * BN, kv_end);
    }
    const int kt0 = j * BN;
    if (kt0 < wave_kend) {
      const unsigned char* kt = kbuf(j & 1);
      f32x16 s[NKB];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const u32x4 a = lds_read128(kt, kfrag + kb * NatFrag<D>::BLK + kk * NatFrag<D>::KK);
          s[kb] = mfma32(a, qf[kk], kk == 0 ? f32x16{} : s[kb]);
        }
      bool need_mask = kt0 + BN > kv_end;
      if constexpr (CAUSAL) need_mask = need_mask || (kt0 + BN - 1 > cq0 + w * kRowsPerWave);
      if (need_mask) {
        // the limit is opaque here: otherwise the compiler sees that no key is past it
        // on tiles that need no mask and runs the selects on every tile
        int lim = kv_end;
        asm volatile("" : "+s"(lim));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + 32 * kb + c_row(r, h);
            bool bad = key >= lim;
            if constexpr (CAUSAL) bad = bad || key > cqrow;
            s[kb][r] = bad ? -INFINITY : s[kb][r];
          }
      }
      u32x4 pk[NKB][2];
      softmax_tile<false, NKB, NDB>(s, sl, m_run, l_run, o, pk);
      const unsigned char* vb_ = vbuf(j & 1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x4 a = lds_read128(vb_, vfrag[db & 1] + db * TrFrag<BN>::DB + (4 * kb + 2 * sb) * TrFrag<BN>::CH);
            o[db] = mfma32(a, pk[kb][sb], o[db]);
          }
    }
    if (nxt) {
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        vh[0].store(vbuf((j + 1) & 1), c4);
        vh[1].store(vbuf((j + 1) & 1), c4);
      }
    }
    wait_vmem();
    __syncthreads();
  }

  const float l_tot = half_sum(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  if (qrow < N) {
    store_ct_rows<D>(p.o + head, qrow, o, inv, h);
    if (h == 0) p.lse[(size_t)bh * N + qrow] = empty ? -INFINITY : (m_run + fast_log2(l_tot)) * kLn2;
  }
}

// Grids of the 8-wave kernel below this many workgroups (two per CU) run the small-grid
// kernel when d = 64 (where it measured faster; at d = 128 it did not).  At d = 128 the
// smallest grids (split_small_grid) run the 8-wave kernel's split form instead, 128 rows
// per workgroup with each wave group on half of the key tiles.  Measured (ms): a split on
// the 4-wave straight loop with the groups in lockstep against the unsplit kernel (one
// box): B=1, H=16, N=2048 causal 0.0598 -> 0.0476, no mask 0.0624 -> 0.0519; B=2, H=16,
// N=2048 causal 0.0660 -> 0.0628; this ping-pong split against that lockstep split
// (another box): 0.0473 -> 0.0433, 0.0538 -> 0.0496, 0.0643 -> 0.0601, and B=2, H=16,
// N=1024 causal 0.0293 -> 0.0281.  Splits measured slower at d = 64 and on fuller grids.
constexpr unsigned kSmallGrid = 512;

template <int D, int BN, bool CAUSAL, bool KVLEN>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  constexpr size_t lds = kLdsTiles * BN * D * 2;
  const unsigned bh = (unsigned)(a.B * a.H);
  const unsigned grid8 = (unsigned)((a.N + kBM - 1) / kBM) * bh;
  if constexpr (D == 128) {
    if (split_small_grid(grid8, CAUSAL)) {
      auto kern = fa_fwd_kernel<D, BN, CAUSAL, KVLEN, true>;
      const size_t lds2 = 2 * lds;
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
      if (e != hipSuccess) return e;
      const unsigned grid = (unsigned)((a.N + kBM / 2 - 1) / (kBM / 2)) * bh;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds2, stream, a);
      return hipGetLastError();
    }
  }
  if (D == 64 && grid8 < kSmallGrid) {
    auto kern = fa_fwd_small_kernel<D, BN, CAUSAL, KVLEN>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((a.N + kBM2 - 1) / kBM2) * bh;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kW2 * 64), lds, stream, a);
    return hipGetLastError();
  }
  auto kern = fa_fwd_kernel<D, BN, CAUSAL, KVLEN>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid8), dim3(kThreads), lds, stream, a);
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
