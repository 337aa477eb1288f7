// Fused exact attention forward for gfx950.
//
// The method ("From-scratch CUDA attention kernel reaches 94.4% of FlashAttention-4 on
// NVIDIA B200", section "How the kernel partitions its work"): one workgroup owns one
// tile of query rows, keeps it on chip, and streams the K/V tiles of its head past it;
// per K/V tile it forms the scores, updates a running row maximum and running row sum
// (the online softmax of "FlashStieltjes", section "The challenge"), rescales and adds
// P V into a private accumulator, and normalises once at the end.  The N x N score
// matrix never exists in memory.  Causal attention visits only the K/V tiles on or
// below the diagonal ("FlashAttention for Tesla P100", section "What it supports").
//
// gfx950 realisation:
//   * Large grids: workgroups of 4 waves that own 64 query rows each (256 rows, one wave
//     per SIMD), so every K or V^T fragment read from LDS feeds two MFMAs.  Otherwise a wave
//     owns 32 query rows, in workgroups of 8 waves (128 rows split over two wave groups that
//     take halves of the key range) or of 4 waves (128 rows).
//   * K/V tiles of BC = 64 keys are copied global -> LDS by direct loads into rings of
//     buffers, one or two tiles ahead of the compute, with no register staging.
//   * Scores are formed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16: each lane then
//     owns one query column, its row max and row sum are in-lane reductions plus one
//     v_permlane32_swap, and the bf16/fp16-rounded probabilities in registers are already
//     the B operand of O^T += V^T P^T.  V^T comes from the row-major V tile through
//     ds_read_b64_tr_b16.
//   * exp2 on the VALU with scale*log2(e) folded into one FMA per score.  The first tile
//     sets a reference max; later tiles form probabilities against it without a max, since
//     their row sum bounds each of them, and a rare tile over the bound is recomputed with
//     the reference moved.
#include "fa_device.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {

namespace {

constexpr int kFwdBC = 64;   // keys per K/V tile
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 of the largest probability)

// Work units of the softmax of one tile and one 32-query block, in dependency order: 16
// three-way maxima, the cross-lane reduction and reference update, 32 fused scale-subtract +
// exp2.  With QB query blocks per wave, unit u belongs to block u % QB and is unit u / QB of
// that block's list, so the blocks' chains interleave.
constexpr int kSmMax = 16, kSmRed = 16, kSmExp0 = 17, kSmUnits = 49;

// SPLIT = 2: the workgroup's waves form two groups that own the same query rows and split
// the K/V range in two contiguous halves (an on-chip split of the key range); each group runs
// the online softmax over its half and the halves merge through LDS at the end, exactly, by
// rescaling both to the larger running max.  Used where one query tile per workgroup leaves
// the CUs short of waves (small grids) or unevenly loaded (causal).
//
// PART: the key range of every query tile is also cut into `n_part` contiguous pieces, one
// workgroup each, and each workgroup writes its piece's normalised output and log-sum-exp as
// fp32 partials (Op, Lp) for a merge pass (merge_kernel).  A piece (or half) that holds no
// visible key for a row yields O = 0 and LSE = -inf there.
//
// QB: 32-query blocks per wave.  With QB = 2 every K or V^T fragment read from LDS feeds two
// MFMAs (one per block), which halves the LDS traffic per MFMA; a wave then needs about 400
// registers, so each SIMD runs one wave (4-wave workgroups of 256 query rows, one per CU).
template <typename TR, int HD, bool CAUSAL, int NW, int SPLIT, bool PART, int QB>
__global__ void __launch_bounds__(NW * 64, 8 / (NW * QB))
fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
           const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
           int Hq, int Hkv, int N, int n_qt, float c2, float scale, uint32_t qsign, int snake, int n_part,
           float* __restrict__ Op, float* __restrict__ Lp) {
  static_assert(SPLIT == 1 || SPLIT == 2, "one or two groups");
  static_assert(NW * QB == 4 || NW * QB == 8, "one or two workgroups per CU");
  constexpr int GW = NW / SPLIT;            // waves per group
  constexpr int RW = 32 * QB;               // query rows per wave
  constexpr int BR = GW * RW, BC = kFwdBC;  // query rows per workgroup, keys per tile
  constexpr int KST = HD / 16;              // k-steps of S^T over the head dim
  constexpr int DB = HD / 32;               // 32-row blocks of O^T
  constexpr int TILE = BC * HD * 2;         // bytes of one K or V tile
  constexpr int TI = TILE / 1024 / GW;      // 1 KB direct loads per wave per tile
  static_assert(TI * 1024 * GW == TILE, "tile must split into 1 KB loads over the waves");

  // K/V tiles are loaded DIST steps ahead into NB = DIST + 1 buffers each.  One workgroup per
  // CU has LDS to spare for two steps of lead; two workgroups per CU keep one, and so do the
  // two groups of a split workgroup.
  constexpr int DIST = (NW * QB == 8 && SPLIT == 1) ? 2 : 1, NB = DIST + 1;
  // The running max is not tracked per tile.  Probabilities are formed against the reference
  // max, and the row sum, computed anyway, bounds every one of them: while a lane's share of
  // the tile's sum stays <= 2^7, no probability exceeds 2^8 and nothing needs to be rescaled.
  // Otherwise (rare: a score far above the reference) the tile's scores are recomputed from
  // its K tile, still resident in one more K buffer, and the reference moves to their max.
  // This takes the 16 v_max3 and the cross-lane reduction per tile off the VALU.
  constexpr int NBK = NB + 1;
  // 64-row waves: O accumulators and Q fragments in AGPRs (mfma_av, mfma_va).
  constexpr bool AGPR = QB == 2;
  __shared__ __attribute__((aligned(1024))) char smem[SPLIT * (NBK + NB) * TILE];  // per group: K[NBK], V[NB]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / GW;  // group (0 when SPLIT = 1)
  const int wv = wave % GW;   // wave within the group
  const int c = lane & 31, g = lane >> 5;
  char* const sK = smem + grp * ((NBK + NB) * TILE);
  char* const sV = sK + NBK * TILE;

  int job = CAUSAL && !snake ? xcd_remap_interleaved(blockIdx.x, gridDim.x, n_qt * (PART ? n_part : 1))
                             : xcd_remap(blockIdx.x, gridDim.x);
  int part = 0;  // piece of the key range (PART)
  if constexpr (PART) {
    part = job % n_part;
    job /= n_part;
  }
  int qt = job % n_qt;
  const int bh = job / n_qt;
  if (CAUSAL) qt = causal_tile(qt, bh, n_qt, snake);
  const int hq = bh % Hq, b = bh / Hq;
  const int hkv = hq / (Hq / Hkv);
  const uint16_t* const Qh = Q + (size_t)bh * N * HD;
  const uint16_t* const Kh = K + ((size_t)b * Hkv + hkv) * N * HD;
  const uint16_t* const Vh = V + ((size_t)b * Hkv + hkv) * N * HD;

  const int qw0 = qt * BR + wv * RW;  // first query row of this wave
  int qi[QB];                         // the query row of this lane's column in each block
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qi[qb] = qw0 + qb * 32 + c;

  // K/V tiles the workgroup streams, and the prefix of them this wave computes on (causal
  // waves stop at their own diagonal; waves wholly past the last row compute nothing).
  int T = (N + BC - 1) / BC;
  if (CAUSAL) T = (min(N, (qt + 1) * BR) - 1) / BC + 1;
  int Tw = T;
  if (CAUSAL) Tw = (min(N, qw0 + RW) - 1) / BC + 1;
  if (qw0 >= N) Tw = 0;
  // This group's tiles [t0, t0 + Tg) (group 0 takes the larger half), the steps every wave
  // takes (the larger group's tile count + 1, one barrier each), and the number of the
  // group's tiles this wave computes on.  Only the wave's last tile Tw - 1 can need masks,
  // and when it lies in a group's range it is that group's last computed tile.
  const int tb = PART ? (int)((long long)T * part / n_part) : 0;  // this workgroup's piece [tb, te)
  const int te = PART ? (int)((long long)T * (part + 1) / n_part) : T;
  const int half = SPLIT == 2 ? (te - tb + 1) / 2 : te - tb;
  const int t0 = tb + (grp ? half : 0);
  const int Tg = grp ? te - tb - half : half;
  const int Twg = max(0, min(Tw - t0, Tg));

  // Direct loads of the group's tile t of K or V into `dst` (rows past the end read as zero,
  // which the masks then exclude).
  const BufRes rK = make_bufres(Kh, (uint32_t)N * HD * 2u), rV = make_bufres(Vh, (uint32_t)N * HD * 2u);
  uint32_t doff[TI];
#pragma unroll
  for (int r = 0; r < TI; ++r) {
    int row, col;
    sl_pos_to_rc<BC>((uint32_t)((wv * TI + r) * 64 + lane), row, col);
    doff[r] = (uint32_t)(row * HD + col) * 2u;
  }
  auto issue = [&](BufRes res, int t, char* dst) FA_INL {
#pragma unroll
    for (int r = 0; r < TI; ++r)
      dma_to_lds<16>(res, doff[r], (uint32_t)(t0 + t) * (BC * HD * 2), dst + (wv * TI + r) * 1024);
  };
  auto issue_first = [&]() FA_INL {
    if (0 < Tg) issue(rK, 0, sK);
    if constexpr (DIST == 2) {
      if (1 < Tg) issue(rK, 1, sK + TILE);
      issue(rV, 0, sV);
    }
  };
  // Q fragments: B operand of S^T = K Q^T (slot j of block qb, k-step kk = Q[qi[qb]][kk*16 + g*8 + j]).
  // Fragments bound for AGPRs are moved there as soon as they land, so their loads go first
  // (loads retire in order).
  if constexpr (!AGPR) issue_first();
  u32x4 qf[QB][KST];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kk = 0; kk < KST; ++kk)
      qf[qb][kk] = ld16_if(Qh + (size_t)qi[qb] * HD + kk * 16 + g * 8, qi[qb] < N) ^ qsign;
  if constexpr (AGPR) issue_first();

  // Per-lane LDS offsets.  K rows are read in the permuted order, so register i of an S^T
  // block is key (i/8)*16 + g*8 + i%8; one offset per k-step parity.
  const uint32_t koff[2] = {sl_off<BC>(perm_rows(c), g * 8), sl_off<BC>(perm_rows(c), 16 + g * 8)};
  const TrLane trl = tr_lane(lane);

  f32x16 acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
  if constexpr (AGPR) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kk = 0; kk < KST; ++kk) asm volatile("" : "+a"(qf[qb][kk]));  // Q moves to AGPRs once
    reg_fence(qf, true, true);
  }
  float m_run[QB];  // running (reference) max of raw scores for query qi[qb]
  float l_run[QB];  // this lane's share of the running sum of 2^((s - m) * c2)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_run[qb] = -INFINITY, l_run[qb] = 0.f;
  f32x16 p[2][QB];  // probabilities of the previous tile (key block, query block), waiting for P V

  // ---- the pieces of one pipeline step; step j computes S_j and its softmax while the
  //      MFMAs of P_{j-1} V_{j-1} run, so the exp2 work hides under matrix work.  Each MFMA
  //      is fenced together with a fixed share of the VALU work (and, once per fragment, the
  //      LDS read of the operand RD fragments ahead), so the two pipes stay interleaved.
  constexpr int RD = 5;
  // K fragment i (i = kb*KST + kk): key rows kb*32.., head-dim k-step kk.
  auto kfrag = [&](const char* tK, int i) FA_INL {
    const int kk = i % KST, kb = i / KST;
    return lds_ld128(tK + sl_off<BC>(kb * 32, (kk >> 1) * 32) + koff[kk & 1]);
  };
  // V^T fragment i (i = db*4 + kb*2 + t2).
  auto vfrag = [&](const char* tV, int i) FA_INL {
    const int db = i >> 2, kb = (i >> 1) & 1, t2 = i & 1;
    return lds_tr8(tV + sl_off<BC>(kb * 32 + t2 * 16, db * 32), trl);
  };
  // S^T_j = K_j Q^T (register i of block (kb, qb) holds key j*BC + kb*32 + (i/8)*16 + g*8 + i%8
  // against query qi[qb]), with valu(i * QB + qb) run under the MFMA of fragment i, block qb.
  // With PRE its first RD fragments arrive in `pre` (read during the phase before); with POST
  // its last RD steps, which have no fragment of their own left to read, read the next phase's
  // first fragments next(r) into `post`.  LASTNOP: the wait states the last MFMA carries (the
  // steady steps first read its result half a phase later).  pv() below takes the same options.
  auto scores = [&](auto pre_tag, auto post_tag, const char* __restrict__ tK, f32x16 (&s)[2][QB], auto&& valu,
                    const u32x4 (&pre)[RD], auto&& next, u32x4 (&post)[RD], auto nop_tag) FA_INL {
    constexpr bool PRE = decltype(pre_tag)::value, POST = decltype(post_tag)::value;
    constexpr int LASTNOP = decltype(nop_tag)::value;
    constexpr int NS = 2 * KST;
    u32x4 ring[RD + 1];
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      if constexpr (PRE)
        ring[i] = pre[i];
      else
        ring[i] = kfrag(tK, i);  // in use order, so each wait is partial
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + RD < NS)
        ring[(i + RD) % (RD + 1)] = kfrag(tK, i + RD);
      else if constexpr (POST)
        post[i + RD - NS] = next(i + RD - NS);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (!AGPR)
          s[i / KST][qb] = TR::mfma(ring[i % (RD + 1)], qf[qb][i % KST], s[i / KST][qb]);
        else if (i % KST == 0)  // (the loops are unrolled: one call remains per MFMA)
          mfma_va0<TR, kNopNone>(s[i / KST][qb], ring[i % (RD + 1)], qf[qb][i % KST]);
        else if (i == NS - 1 && qb == QB - 1)
          mfma_va<TR, LASTNOP>(s[i / KST][qb], ring[i % (RD + 1)], qf[qb][i % KST]);
        else
          mfma_va<TR, kNopNone>(s[i / KST][qb], ring[i % (RD + 1)], qf[qb][i % KST]);
        valu(i * QB + qb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (AGPR) reg_fence(s, false, false);
  };
  // O^T += V^T P^T (A = V^T: rows d, k = keys, read transposed from the V tile), with
  // valu(i * QB + qb) run under the MFMA of fragment i, block qb.
  auto pv = [&](auto pre_tag, auto post_tag, const char* __restrict__ tV, u32x4 (&pb)[2][2][QB], auto&& valu,
                const u32x4 (&pre)[RD], auto&& next, u32x4 (&post)[RD], auto nop_tag) FA_INL {
    constexpr bool PRE = decltype(pre_tag)::value, POST = decltype(post_tag)::value;
    constexpr int LASTNOP = decltype(nop_tag)::value;
    constexpr int NS = DB * 4;
    if constexpr (AGPR) {
      reg_fence(acc, true, false);
      reg_fence(reinterpret_cast<u32x4(&)[4][QB]>(pb), false, false);
    }
    u32x4 ring[RD + 1];
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      if constexpr (PRE)
        ring[i] = pre[i];
      else
        ring[i] = vfrag(tV, i);  // in use order, so each wait is partial
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + RD < NS)
        ring[(i + RD) % (RD + 1)] = vfrag(tV, i + RD);
      else if constexpr (POST)
        post[i + RD - NS] = next(i + RD - NS);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (AGPR) {  // (the loops are unrolled: one call remains per MFMA)
          f32x16& o = acc[qb][i >> 2];
          const u32x4 a = ring[i % (RD + 1)], b = pb[(i >> 1) & 1][i & 1][qb];
          if (i == 0 && qb == 0)
            mfma_av<TR, kNopBefore>(o, a, b);
          else if (i == NS - 1 && qb == QB - 1)
            mfma_av<TR, LASTNOP>(o, a, b);
          else
            mfma_av<TR, kNopNone>(o, a, b);
        }
        else
          acc[qb][i >> 2] = TR::mfma(ring[i % (RD + 1)], pb[(i >> 1) & 1][i & 1][qb], acc[qb][i >> 2]);
        valu(i * QB + qb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // Masks, needed only on a wave's last tile (the ragged end of the keys, or the tile that
  // holds this wave's diagonal): masked scores become -inf, so exp2 (with c2 > 0) makes
  // exact zeros.
  auto mask = [&](int j, f32x16 (&s)[2][QB]) FA_INL {
    const int kv0 = (t0 + j) * BC;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
          if (key >= N || (CAUSAL && key > qi[qb])) s[kb][qb][i] = -INFINITY;
        }
  };
  // One query block of S^T (the rare path): register i of r[kb][0] as in `scores`.
  auto scores_q = [&](const char* __restrict__ tK, int qb, f32x16 (&r)[2][1]) FA_INL {
#pragma unroll
    for (int i = 0; i < 2 * KST; ++i) {
      const u32x4 a = kfrag(tK, i);
      if constexpr (!AGPR)
        r[i / KST][0] = TR::mfma(a, qf[qb][i % KST], r[i / KST][0]);
      else if (i % KST == 0)
        mfma_va0<TR, kNopNone>(r[i / KST][0], a, qf[qb][i % KST]);
      else if (i == 2 * KST - 1)
        mfma_va<TR, kNopAfter>(r[i / KST][0], a, qf[qb][i % KST]);
      else
        mfma_va<TR, kNopNone>(r[i / KST][0], a, qf[qb][i % KST]);
    }
    if constexpr (AGPR) reg_fence(r, false, false);  // no read of r moves above the last MFMA
  };
  auto mask_q = [&](int j, int qb, f32x16 (&r)[2][1]) FA_INL {
    const int kv0 = (t0 + j) * BC;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kv0 + kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
        if (key >= N || (CAUSAL && key > qi[qb])) r[kb][0][i] = -INFINITY;
      }
  };
  // Online softmax in raw-score units (c2 = scale * log2(e) > 0), as units u of work (see
  // kSmUnits).  The full set (maxima, reduction, exp2) runs on a wave's first tile, where the
  // reference max is set (kRescaleLog2 only decides whether it moves there; it always does
  // from -inf); the steady steps run the exp2 units alone (see check / redo).  When the
  // reference moves, O is scaled by alpha before the next P V.
  bool need = false;  // uniform: O must be scaled by alpha before the next P V
  float alpha[QB], mx0[QB], mx1[QB], mb[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) alpha[qb] = 1.f, mx0[qb] = mx1[qb] = mb[qb] = 0.f;
  auto softmax_unit = [&](f32x16 (&s)[2][QB], int u) FA_INL {
    const int qb = u % QB, v = u / QB;
    if (v < kSmMax) {  // two running maxima, one per 32-key block, one v_max3 each step
      const int kb = v >> 3, e = (v & 7) * 2;
      float& m = kb ? mx1[qb] : mx0[qb];
      if ((v & 7) == 0)
        m = fmaxf(s[kb][qb][0], s[kb][qb][1]);
      else
        m = fmaxf(fmaxf(m, s[kb][qb][e]), s[kb][qb][e + 1]);
    } else if (v == kSmRed) {
      const float mx = pair_max(fmaxf(mx0[qb], mx1[qb]));
      const float m_new = fmaxf(m_run[qb], mx);  // finite: key 0 is visible to every row
      const bool nq = __builtin_amdgcn_ballot_w64((m_new - m_run[qb]) * c2 > kRescaleLog2) != 0;
      alpha[qb] = nq ? fast_exp2((m_run[qb] - m_new) * c2) : 1.f;
      m_run[qb] = nq ? m_new : m_run[qb];
      l_run[qb] *= alpha[qb];
      mb[qb] = m_run[qb] * c2;
      need = need || nq;
    } else {
      const int e = v - kSmExp0, kb = e >> 4, i = e & 15;
      s[kb][qb][i] = fast_exp2(fmaf(s[kb][qb][i], c2, -mb[qb]));
    }
  };
  auto softmax_all = [&](f32x16 (&s)[2][QB]) FA_INL {
#pragma unroll
    for (int u = 0; u < kSmUnits * QB; ++u) softmax_unit(s, u);
  };
  // P^T operands (slot j of (kb, t2, qb) = P for key kb*32 + t2*16 + g*8 + j) and the row sums,
  // as 16 units per query block: unit v of block qb packs pair v%4 of operand (v/8, (v/4)%2)
  // and adds its two values.  fp16 sums the rounded pair in one dot2 (relative rounding 2^-12,
  // far inside the LSE tolerance even for a row with one visible key); bf16 rounding (2^-9) is
  // not, so bf16 sums the fp32 values.
  // (The rare path rewrites every packed operand, so the compiler would sink the packing into
  // the common path after the check, where it runs between the two MFMA phases with the
  // matrix pipe idle; an empty asm statement that consumes each packed pair keeps it here.)
  float rs[QB];
  auto pack_unit = [&](u32x4 (&pb)[2][2][QB], int u) FA_INL {
    const int qb = u % QB, v = u / QB;
    const int kb = v >> 3, t2 = (v >> 2) & 1, pr = v & 3, e = t2 * 8 + pr * 2;
    uint32_t w = TR::pack(p[kb][qb][e], p[kb][qb][e + 1]);
    asm volatile("" : "+v"(w));
    pb[kb][t2][qb][pr] = w;
    if constexpr (std::is_same<TR, F16>::value)
      rs[qb] = TR::add_pair(pb[kb][t2][qb][pr], rs[qb]);
    else
      rs[qb] += p[kb][qb][e] + p[kb][qb][e + 1];
  };
  auto zero_rs = [&]() FA_INL {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) rs[qb] = -0.f;  // (x + -0 = x folds away)
  };
  // O *= alpha (rare).  Accumulators in AGPRs pass through VGPRs one block at a time, with
  // each move written out so that the accumulators are never allocated to VGPRs.
  auto scale_acc = [&]() FA_INL {
    // (the steady steps' last P V MFMA carries no wait states, so this rare reader waits;
    // the library's tests walk every path of the compiled code from each written-out MFMA)
    if constexpr (AGPR) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (AGPR) {
          f32x16 t;
          asm volatile("" : "=v"(t) : "0"(acc[qb][db]));
          t *= alpha[qb];
          asm volatile("" : "=a"(acc[qb][db]) : "0"(t));
        } else {
          acc[qb][db] *= alpha[qb];
        }
      }
    if constexpr (AGPR) reg_fence(acc, true, true);
  };

  // Pipeline step j (0 <= j <= T), one per K/V tile plus a drain: waits for K_j and V_{j-1},
  // loads K_{j+DIST} and V_{j+DIST-1}, then (by the kind of step) computes S_j and its softmax
  // and/or P_{j-1} V_{j-1}.  The LDS buffers are restrict-qualified parameters so that the
  // compiler can tell these reads from the direct loads in flight and does not make them wait.
  enum Kind { kFirst, kFirstMasked, kSteady, kSteadyMasked, kDrain, kIdle };
  // The rare path: P_{jp} (the previous tile, its K tile in tKp) is recomputed with
  // the reference moved to the tile's max; l is rescaled here and O (flagged by `need`) just
  // before P_{jp} V_{jp} is added.  One query block at a time, which keeps the path's registers
  // within those of the steady path.  Only the drain step's tile can need masks (`masked`).
  auto redo = [&](auto masked, const char* __restrict__ tKp, int jp, u32x4 (&pb)[2][2][QB]) FA_INL {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x16 r[2][1];
      r[0][0] = f32x16{};
      r[1][0] = f32x16{};
      scores_q(tKp, qb, r);
      if constexpr (decltype(masked)::value) mask_q(jp, qb, r);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, r[kb][0][i]);
      const float m_new = fmaxf(m_run[qb], pair_max(mx));
      alpha[qb] = fast_exp2((m_run[qb] - m_new) * c2);
      l_run[qb] *= alpha[qb];
      m_run[qb] = m_new;
      mb[qb] = m_new * c2;
      rs[qb] = -0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            const int e = t2 * 8 + pr * 2;
            const float x0 = fast_exp2(fmaf(r[kb][0][e], c2, -mb[qb]));
            const float x1 = fast_exp2(fmaf(r[kb][0][e + 1], c2, -mb[qb]));
            pb[kb][t2][qb][pr] = TR::pack(x0, x1);
            if constexpr (std::is_same<TR, F16>::value)
              rs[qb] = TR::add_pair(pb[kb][t2][qb][pr], rs[qb]);
            else
              rs[qb] += x0 + x1;
          }
    }
    need = true;
  };
  auto check = [&](auto masked, const char* __restrict__ tKp, int jp, u32x4 (&pb)[2][2][QB]) FA_INL {
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) over = over || !(rs[qb] <= 0x1p7f);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(over) != 0, 0)) redo(masked, tKp, jp, pb);
    if (need) {
      scale_acc();
      need = false;
    }
  };
  auto add_rs = [&]() FA_INL {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += rs[qb];
  };
  auto keep_p = [&](const f32x16 (&s)[2][QB]) FA_INL {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) p[kb][qb] = s[kb][qb];
  };

  // First K fragments of the next step's S phase, read during this step's last P V MFMAs
  // (two-step lead only: K_{j+1} is complete at step j's barrier).
  u32x4 kpre[RD];
  u32x4 unused[RD];
  auto no_next = [](int) FA_INL { return u32x4{0u, 0u, 0u, 0u}; };
  using Yes = std::true_type;
  using No = std::false_type;
  auto step = [&](auto kind_tag, const int j, char* __restrict__ nK, char* __restrict__ nV,
                  const char* __restrict__ tK, const char* __restrict__ tV,
                  const char* __restrict__ pK, const char* __restrict__ fK) FA_INL {
    constexpr Kind KIND = decltype(kind_tag)::value;
    // this wave's loads of K_j and V_{j-1} have landed, and with two steps of lead also K_{j+1}
    // (the load of V_j may stay in flight: loads retire in issue order) ...
    if constexpr (DIST == 2) {
      if (j < Tg)
        wait_vmcnt<TI>();
      else
        wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();
    }
    dma_barrier();  // ... and everyone's; everyone is also done with step j-1's buffers
    if (need) {       // the max moved in the previous step: rescale O (rare)
      scale_acc();
      need = false;
    }
    // The steady steps issue the next tiles' loads under their first S MFMAs (K after the first,
    // V after the third: 0.5-1% faster than after the second and fourth, and than any later pair).
    constexpr bool LATE_ISSUE = KIND == kSteady || KIND == kSteadyMasked;
    if constexpr (!LATE_ISSUE) {
      if (j + DIST < Tg) issue(rK, j + DIST, nK);
      if (j + DIST - 1 < Tg) issue(rV, j + DIST - 1, nV);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KIND == kSteady || KIND == kSteadyMasked) {
      // [S_j MFMAs | pack P_{j-1}]  [P_{j-1} V_{j-1} MFMAs | softmax of S_j]
      f32x16 s[2][QB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
      u32x4 pb[2][2][QB];
      zero_rs();
      // The steady steps run only the exp2 units of the softmax (FIRST = kSmExp0); the masks
      // of a masked tile come after its S MFMAs.
      // The units are spread evenly over the MFMAs of each phase.
      constexpr int NSM = 2 * KST * QB, NPV = DB * 4 * QB, FIRST = kSmExp0, NP = 16 * QB;
      u32x4 vpre[RD];
      auto packs = [&](int i) FA_INL {
        if (i == 0 && j + DIST < Tg) issue(rK, j + DIST, nK);
        if (i == 2 && j + DIST - 1 < Tg) issue(rV, j + DIST - 1, nV);
#pragma unroll
        for (int u = 0; u < NP; ++u)
          if (u * NSM / NP == i) pack_unit(pb, u);
      };
      auto vnext = [&](int r) FA_INL { return vfrag(tV, r); };
      // (the last S MFMA's result is first read half a phase later, unless the masks follow)
      constexpr int SNOP = KIND == kSteady ? kNopNone : kNopAfter;
      if constexpr (DIST == 2)
        scores(Yes{}, Yes{}, tK, s, packs, kpre, vnext, vpre, std::integral_constant<int, SNOP>{});
      else
        scores(No{}, Yes{}, tK, s, packs, unused, vnext, vpre, std::integral_constant<int, SNOP>{});
      check(std::false_type{}, pK, j - 1, pb);
      add_rs();
      if constexpr (KIND == kSteadyMasked) mask(j, s);
      // (the steady steps run exp2 units only, all of equal weight)
      constexpr int NX = (kSmUnits - FIRST) * QB;
      auto exps = [&](int i) FA_INL {
#pragma unroll
        for (int x = 0; x < NX; ++x)
          if (x * NPV / NX == i) softmax_unit(s, FIRST * QB + x);
      };
      // (the accumulators' next readers outside MFMAs, scale_acc and the drain, wait themselves)
      using NoWait = std::integral_constant<int, kNopNone>;
      if constexpr (DIST == 2 && KIND == kSteady)
        pv(Yes{}, Yes{}, tV, pb, exps, vpre, [&](int r) FA_INL { return kfrag(fK, r); }, kpre, NoWait{});
      else
        pv(Yes{}, No{}, tV, pb, exps, vpre, no_next, unused, NoWait{});
      keep_p(s);
    } else if constexpr (KIND == kFirst || KIND == kFirstMasked) {
      f32x16 s[2][QB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
      scores(No{}, No{}, tK, s, [](int) FA_INL {}, unused, no_next, unused,
             std::integral_constant<int, kNopAfter>{});
      if constexpr (KIND == kFirstMasked) mask(j, s);
      softmax_all(s);
      need = false;  // O is still zero
      keep_p(s);
      if constexpr (DIST == 2 && KIND == kFirst) {  // the next step computes S: K_1 is complete
#pragma unroll
        for (int r = 0; r < RD; ++r) kpre[r] = kfrag(fK, r);
      }
    } else if constexpr (KIND == kDrain) {
      u32x4 pb[2][2][QB];
      zero_rs();
#pragma unroll
      for (int u = 0; u < 16 * QB; ++u) pack_unit(pb, u);
      check(std::true_type{}, pK, j - 1, pb);
      add_rs();
      pv(No{}, No{}, tV, pb, [](int) FA_INL {}, unused, no_next, unused,
         std::integral_constant<int, kNopAfter>{});
    }
  };

  // Buffer rings: step j reads K_j from kc and V_{j-1} from vp and fills kd with K_{j+DIST}
  // and vd with V_{j+DIST-1}; with DIST = 2, kf holds K_{j+1} and vf holds V_j in flight; kp
  // keeps K_{j-1} for the rare path.
  char* kc = sK;
  char* kf = sK + TILE;
  char* kd = sK + (NB - 1) * TILE;
  char* kp = sK + (NBK - 1) * TILE;
  char* vp = sV + (NB - 1) * TILE;
  char* vf = sV;
  char* vd = sV + (DIST - 1) * TILE;
  auto run = [&](auto kind_tag, int j) FA_INL {
    step(kind_tag, j, kd, vd, kc, vp, kp, kf);
    char* t;
    if constexpr (DIST == 2) {
      t = kp, kp = kc, kc = kf, kf = kd, kd = t;
      t = vp, vp = vf, vf = vd, vd = t;
    } else {
      t = kp, kp = kc, kc = kd, kd = t;
      t = vp, vp = vd, vd = t;
    }
  };
  using KFirst = std::integral_constant<Kind, kFirst>;
  using KFirstMasked = std::integral_constant<Kind, kFirstMasked>;
  using KSteady = std::integral_constant<Kind, kSteady>;
  using KSteadyMasked = std::integral_constant<Kind, kSteadyMasked>;
  using KDrain = std::integral_constant<Kind, kDrain>;
  using KIdle = std::integral_constant<Kind, kIdle>;
  // Every wave takes exactly half + 1 steps (one barrier each); the group's last computed
  // tile is the only one that can need masks.
  if (Twg == 0) {
    for (int j = 0; j <= half; ++j) run(KIdle{}, j);
  } else {
    if (Twg == 1)
      run(KFirstMasked{}, 0);
    else
      run(KFirst{}, 0);
    for (int j = 1; j < Twg - 1; ++j) run(KSteady{}, j);
    if (Twg >= 2) run(KSteadyMasked{}, Twg - 1);
    run(KDrain{}, Twg);
    for (int j = Twg + 1; j <= half; ++j) run(KIdle{}, j);
  }
  if constexpr (AGPR) reg_fence(acc, true, false);
  if (need) scale_acc();

  // ---- split workgroups: group 1 hands its (O, running max, running sum) to the group-0 wave
  // that owns the same rows, through LDS (the K/V buffers are free once every wave has passed
  // the barrier).  Both halves are rescaled to the larger max: exp2 of (m_h - m) * c2, which is
  // 0 for a half that saw no key (m_h = -inf).
  constexpr int XB = 16 * DB + 2, XW = QB * XB;  // floats per lane and block: O, max, sum
  if constexpr (SPLIT == 2) {
    static_assert(GW * 64 * XW * 4 <= (int)sizeof(smem), "exchange must fit in the K/V buffers");
    float* const xs = reinterpret_cast<float*>(smem) + wv * (64 * XW) + lane;
    lds_barrier();
    if (grp == 1) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) xs[(qb * XB + db * 16 + i) * 64] = acc[qb][db][i];
        xs[(qb * XB + 16 * DB) * 64] = m_run[qb];
        xs[(qb * XB + 16 * DB + 1) * 64] = l_run[qb];
      }
    }
    lds_barrier();
    if (grp == 1) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m1 = xs[(qb * XB + 16 * DB) * 64], l1 = xs[(qb * XB + 16 * DB + 1) * 64];
      const float m = fmaxf(m_run[qb], m1);
      // (equal maxima take weight 1, which also keeps two empty halves, m = -inf, NaN-free)
      const float a0 = m_run[qb] == m ? 1.f : fast_exp2((m_run[qb] - m) * c2);
      const float a1 = m1 == m ? 1.f : fast_exp2((m1 - m) * c2);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[qb][db][i] = acc[qb][db][i] * a0 + xs[(qb * XB + db * 16 + i) * 64] * a1;
      l_run[qb] = l_run[qb] * a0 + l1 * a1;
      m_run[qb] = m;
    }
  }

  // ---- epilogue: normalise, write O (input dtype, RNE) and LSE (natural log, fp32)
  if constexpr (PART) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = pair_sum(l_run[qb]);
      if (qi[qb] >= N) continue;
      // fp32 partials of piece `part`; a row with no visible key in the piece: O = 0, LSE = -inf
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const size_t rows = (size_t)(gridDim.x / (n_part * n_qt)) * N;  // B * Hq * N
      const size_t row = (size_t)part * rows + (size_t)bh * N + qi[qb];
      float* const orow = Op + row * HD;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d = db * 32 + i4 * 8 + g * 4;
          const f32x4 w = {acc[qb][db][i4 * 4 + 0] * inv, acc[qb][db][i4 * 4 + 1] * inv,
                           acc[qb][db][i4 * 4 + 2] * inv, acc[qb][db][i4 * 4 + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + d) = w;
        }
      if (g == 0) Lp[row] = l_tot > 0.f ? m_run[qb] * scale + __logf(l_tot) : -INFINITY;
    }
  } else {
    // O rows go out through LDS, whole rows per store instruction (stage_row, store_staged).
    char* ob;
    if constexpr (SPLIT == 2) {
      ob = smem + wv * (64 * XW * 4);  // the hand-off region this wave has just read
    } else {
      lds_store_barrier();             // every wave is done with the K/V buffers
      ob = sK + wv * (RW * HD * 2);
    }
    static_assert(RW * HD * 2 <= (SPLIT == 2 ? 64 * XW * 4 : NBK * TILE / GW), "O rows must fit the region");
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = pair_sum(l_run[qb]);
      const float inv = 1.f / l_tot;
      u32x2 w[DB][4];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          w[db][i4] = u32x2{TR::pack(acc[qb][db][i4 * 4 + 0] * inv, acc[qb][db][i4 * 4 + 1] * inv),
                            TR::pack(acc[qb][db][i4 * 4 + 2] * inv, acc[qb][db][i4 * 4 + 3] * inv)};
      stage_row<HD>(ob, qb * 32 + c, g, w);
      if (qi[qb] < N && g == 0) LSE[(size_t)bh * N + qi[qb]] = m_run[qb] * scale + __logf(l_tot);
    }
    store_staged<HD * 2, RW>(ob, O + ((size_t)bh * N + qw0) * HD, N - qw0, lane);
  }
}

// 128-query grids that split the key range inside the workgroup: causal grids, whose tiles
// carry uneven work, and grids too small to give every CU two 4-wave workgroups.
inline bool fwd_split_kv(const FwdArgs& a) {
  return a.causal || a.B * a.Hq * ((a.N + 127) / 128) < 512;
}

template <typename TR, int HD, bool CAUSAL, int NW, int SPLIT, bool PART = false, int QB = 1>
hipError_t launch_fwd_nw(const FwdArgs& a) {
  constexpr int BR = NW / SPLIT * 32 * QB;
  const int n_qt = (int)((a.N + BR - 1) / BR);
  const int n_part = PART ? a.n_part : 1;
  const long long blocks = a.B * a.Hq * (long long)n_qt * n_part;
  // c2 must be > 0 so that exp2(-inf * c2) is an exact 0 for masked scores; a zero scale
  // becomes 2^-100, for which every exp2 rounds to exactly 1 (uniform weights).  A negative
  // scale runs as |scale| on -Q (qsign flips the sign bit of every 16-bit element of the Q
  // fragments): the scaled scores, and so O and LSE, are unchanged.
  const float as = fabsf(a.scale);
  const float c2 = as > 0.f ? as * kLog2e : 0x1p-100f;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_kernel<TR, HD, CAUSAL, NW, SPLIT, PART, QB>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                     a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                     (int)a.Hq, (int)a.Hkv, (int)a.N, n_qt, c2, as, qsign, (int)grid_fits(blocks, 8 / (NW * QB)), n_part,
                     a.o_part, a.lse_part);
  return hipGetLastError();
}

// 256-query workgroups (one per CU) halve the K/V traffic from L2 per query; they run as 4
// waves of 64 query rows, which also halves the LDS reads per MFMA (measured: 1.4-2% faster
// than 8 waves of 32 rows at N >= 8192, the same at N = 4096; the forward is power-bound).
// Smaller grids use 128-query tiles: as 8-wave workgroups that split the key range over two
// wave groups (one per CU), which keeps two waves on every SIMD and evens out causal work, or
// as 4-wave workgroups (two per CU).  A causal D = 64 grid that runs in one round takes 64-query
// tiles instead, split over two groups of two waves, two workgroups per CU (80 KiB of LDS
// each): its causal_tile order hands every CU a heavy and a light tile, where 128-query tiles
// would give each CU one tile of very unequal work (measured: 8% less time at GQA N = 2048).
template <typename TR, int HD, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a) {
  const long long big = a.B * a.Hq * ((a.N + 255) / 256);
  if (big >= 512) return launch_fwd_nw<TR, HD, CAUSAL, 4, 1, false, 2>(a);
  if constexpr (HD == 64 && CAUSAL)
    if (grid_fits(a.B * a.Hq * ((a.N + 63) / 64), 2)) return launch_fwd_nw<TR, HD, CAUSAL, 4, 2>(a);
  if (fwd_split_kv(a)) return launch_fwd_nw<TR, HD, CAUSAL, 8, 2>(a);
  return launch_fwd_nw<TR, HD, CAUSAL, 4, 1>(a);
}

template <typename TR>
hipError_t launch_fwd_dt(const FwdArgs& a) {
  if (a.D == 64) return a.causal ? launch_fwd_t<TR, 64, true>(a) : launch_fwd_t<TR, 64, false>(a);
  return a.causal ? launch_fwd_t<TR, 128, true>(a) : launch_fwd_t<TR, 128, false>(a);
}

// Key-range pieces always run as split 128-query workgroups: the grids that need pieces are
// the ones too small for anything else.
template <typename TR>
hipError_t launch_fwd_part_dt(const FwdArgs& a) {
  if (a.D == 64)
    return a.causal ? launch_fwd_nw<TR, 64, true, 8, 2, true>(a) : launch_fwd_nw<TR, 64, false, 8, 2, true>(a);
  return a.causal ? launch_fwd_nw<TR, 128, true, 8, 2, true>(a) : launch_fwd_nw<TR, 128, false, 8, 2, true>(a);
}

// ---------------------------------------------------------------- merge of partials
// Attention over a union of disjoint key sets from the results over each set: with m the
// largest partial LSE, w_s = exp(LSE_s - m), LSE = m + log(sum_s w_s) and
// O = sum_s (w_s / sum_s w_s) O_s.  A part with LSE_s = -inf (no key) has weight 0.  One
// thread handles 8 columns of one row; parts are summed in index order (deterministic).
template <typename TR, int HD>
__global__ void __launch_bounds__(256)
merge_kernel(const float* __restrict__ Op, const float* __restrict__ Lp, int n_part, long long rows,
             uint16_t* __restrict__ O, float* __restrict__ LSE) {
  constexpr int TPR = HD / 8;
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int d0 = (threadIdx.x % TPR) * 8;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int s = 0; s < n_part; ++s) m = fmaxf(m, Lp[s * rows + row]);
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
  float wsum = 0.f;
  if (m > -INFINITY) {
    for (int s = 0; s < n_part; ++s) {
      const float w = __expf(Lp[s * rows + row] - m);
      const float* src = Op + ((size_t)s * rows + row) * HD + d0;
      o0 += w * *reinterpret_cast<const f32x4*>(src);
      o1 += w * *reinterpret_cast<const f32x4*>(src + 4);
      wsum += w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *reinterpret_cast<u32x4*>(O + row * HD + d0) =
      u32x4{TR::pack(o0[0] * inv, o0[1] * inv), TR::pack(o0[2] * inv, o0[3] * inv),
            TR::pack(o1[0] * inv, o1[1] * inv), TR::pack(o1[2] * inv, o1[3] * inv)};
  if (d0 == 0) LSE[row] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

template <typename TR, int HD>
hipError_t launch_merge_t(const MergeArgs& a) {
  constexpr int RPB = 256 / (HD / 8);
  hipLaunchKernelGGL((merge_kernel<TR, HD>), dim3((unsigned)((a.rows + RPB - 1) / RPB)), dim3(256), 0, a.stream,
                     a.o_part, a.lse_part, a.n_part, a.rows, static_cast<uint16_t*>(a.o), a.lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.f32) return launch_fwd_f32(a);
  if (a.n_part > 1) return a.bf16 ? launch_fwd_part_dt<Bf16>(a) : launch_fwd_part_dt<F16>(a);
  return a.bf16 ? launch_fwd_dt<Bf16>(a) : launch_fwd_dt<F16>(a);
}

hipError_t launch_merge(const MergeArgs& a) {
  if (a.bf16) return a.D == 64 ? launch_merge_t<Bf16, 64>(a) : launch_merge_t<Bf16, 128>(a);
  return a.D == 64 ? launch_merge_t<F16, 64>(a) : launch_merge_t<F16, 128>(a);
}

// Pieces of the key range for fa_fwd_splitkv when the caller leaves the choice to the library:
// grids that already fill the CUs take none (1); smaller ones take enough pieces for one split
// 128-query workgroup per CU (measured: more pieces cost more in partial traffic and merging
// than they gain), while every half-piece keeps at least four 64-key tiles.
int fwd_auto_parts(long long B, long long Hq, long long N, long long D, bool causal) {
  (void)D;
  if (B * Hq * ((N + 255) / 256) >= 512) return 1;
  const long long tiles = B * Hq * ((N + 127) / 128);
  const long long T = (N + 63) / 64 / (causal ? 2 : 1);
  long long parts = (256 + tiles - 1) / tiles;
  parts = parts < T / 8 ? parts : T / 8;
  return (int)(parts < 1 ? 1 : (parts > 64 ? 64 : parts));
}

}  // namespace fa
