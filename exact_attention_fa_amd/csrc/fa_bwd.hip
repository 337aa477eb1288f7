// Fused exact attention backward for gfx950: preprocess, dK/dV pass, dQ pass, postprocess.
//
// The method: P is recomputed from the saved log-sum-exp, then
//   dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dK = scale * dS^T Q, dQ = scale * dS K
// with D = rowsum(dO * O).  The score-gradient step is a cancellation, so dP and dS stay
// in fp32 and only the MFMA operands are rounded to the input type ("FlashAttention for
// Tesla P100", section "Documentation": the choice of precision is made per product).  That
// page's backward accumulates dQ with atomics and also ships a no-atomic variant ("Layout"
// table); here dQ comes from its own query-stationary pass with no atomics, which recomputes
// S and dP (three products instead of one, but no fp32 atomic traffic, no dS round trip
// through LDS and a bitwise-deterministic result).
//
// dK/dV pass: a workgroup (4 waves) owns 128 keys of one query head, a wave owns 32 of them;
// its K and V rows stay in registers.  64-query tiles of Q and dO, with the per-row
// LSE*log2(e) and D, stream through a triple-buffered LDS by direct global->LDS loads issued
// two tiles ahead (first read one tile ahead, by the pipelined S/dP).  Per query tile, per wave and per 32-query block: S = Q K^T and dP = dO V^T on
// v_mfma_f32_32x32x16 with the key as the accumulator column, so each lane owns one key;
// register 8t+j of the block is query 16t + 8g + j (row permutation of the Q/dO operand),
// which is exactly the k-slot order of the A operand of dV += P^T dO and dK += dS^T Q, so
// the rounded P and dS feed those MFMAs from registers; the dO and Q B operands come through
// ds_read_b64_tr_b16.
// Grouped-query attention: the grid runs over query heads; when Hq > Hkv each workgroup
// writes fp32 per-query-head dK/dV partials that the postprocess sums over the group
// (deterministic), otherwise it writes dK/dV directly.
#include "fa_device.h"
#include "fa_launch.h"

#include <type_traits>

namespace fa {

namespace {

constexpr int kThreads = 256;

#define FA_HIP_TRY(expr)                       \
  do {                                         \
    const hipError_t _e = (expr);              \
    if (_e != hipSuccess) return _e;           \
  } while (0)
constexpr int kBwdBKV = 128;  // keys per workgroup (32 per wave)
constexpr int kBwdBQ = 64;    // query rows per streamed tile
constexpr int kDqBC = 32;     // dQ kernel: keys per K/V tile

// ---------------------------------------------------------------- preprocess
// Dl[row] = -D[row] = -sum_d dO[row][d] * O[row][d] (fp32, stored negated: it is the
// accumulator input of the dK/dV pass's dP MFMAs) and L2[row] = LSE[row] * log2(e) (the
// exponent offset of the base-2 recompute of P).  HBM-bound: HD/8 threads share a row, 16
// bytes of O and of dO each; a thread keeps the loads of kPreRows rows in flight, and at most
// kPreBlocks workgroups stride over the rows (streaming reads on this GPU reach their best
// rate with a few thousand resident workgroups, not one short-lived workgroup per 64 rows).
// The loads are non-temporal (each byte is read once): 11% faster than ordinary loads at
// 131 MiB and at 1 GiB.  (Four rows in flight per thread were 4% faster still at 131 MiB but
// halve the workgroups of small grids, which then ran slower.)
constexpr int kPreRows = 2, kPreBlocks = 2048;
__device__ __forceinline__ u32x4 ld16_stream_if(const void* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)) : z;
}
template <typename TR, int HD>
__global__ void __launch_bounds__(kThreads)
bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
               const float* __restrict__ LSE, float* __restrict__ Dl, float* __restrict__ L2, long long rows) {
  constexpr int TPR = HD / 8;          // threads per row, 8 elements each
  constexpr int RPP = kThreads / TPR;  // rows per pass of the block
  const int part = threadIdx.x % TPR;
  const long long stride = (long long)gridDim.x * RPP * kPreRows;
  for (long long row0 = (long long)blockIdx.x * RPP * kPreRows + threadIdx.x / TPR; row0 - threadIdx.x / TPR < rows;
       row0 += stride) {
    u32x4 o[kPreRows], d[kPreRows];
#pragma unroll
    for (int u = 0; u < kPreRows; ++u) {
      const long long row = row0 + (long long)u * RPP;  // each pass reads RPP consecutive rows
      const bool ok = row < rows;
      o[u] = ld16_stream_if(O + (ok ? row : 0) * HD + part * 8, ok);
      d[u] = ld16_stream_if(dO + (ok ? row : 0) * HD + part * 8, ok);
    }
#pragma unroll
    for (int u = 0; u < kPreRows; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = fmaf(TR::lo(o[u][w]), TR::lo(d[u][w]), acc);
        acc = fmaf(TR::hi(o[u][w]), TR::hi(d[u][w]), acc);
      }
#pragma unroll
      for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      const long long row = row0 + (long long)u * RPP;
      if (row < rows && part == 0) {
        Dl[row] = -acc;
        L2[row] = LSE[row] * kLog2e;
      }
    }
  }
}

// ---------------------------------------------------------------- dK, dV
// Key-stationary: a workgroup (4 waves) owns 128 keys of one query head, a wave owns 32.  The
// wave's K and V rows are loaded once into registers (the B operands of S = Q K^T and
// dP = dO V^T; in AGPRs, with the dK/dV accumulators).  64-query tiles of Q and dO with their
// LSE*log2(e) and D stream through a triple-buffered LDS by direct loads issued two tiles
// ahead, one barrier per tile.  Work is
// done in units of 32 queries, software-pipelined inside the wave: while the MFMAs of S and
// dP of unit u+1 run, the VALU forms P and dS of unit u; then the MFMAs of dV += P^T dO and
// dK += dS^T Q of unit u run with dO and Q read transposed from LDS.  Query rows past the
// end read as zero (Q = dO = 0 and LSE = D = 0), which makes their dS and dO rows zero: they
// add nothing, so only the causal diagonal needs masks.
template <typename TR, int HD, bool CAUSAL, bool PARTIAL>
__global__ void __launch_bounds__(kThreads, 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ L2, const float* __restrict__ Dl, uint16_t* __restrict__ dK,
                uint16_t* __restrict__ dV, float* __restrict__ dKp, float* __restrict__ dVp, int Hq, int Hkv,
                int N, int n_kt, float c2, float scale, uint32_t ksign, int snake, int n_qp) {
  constexpr int BKV = kBwdBKV, BQ = kBwdBQ;
  constexpr int KST = HD / 16, DB = HD / 32;
  constexpr int QT_BYTES = BQ * HD * 2;
  constexpr int QI = QT_BYTES / 1024 / 4;   // 1 KB direct loads per wave for one Q (or dO) tile
  static_assert(QI * 4096 == QT_BYTES, "tiles must split into 1 KB loads");
  constexpr int NBUF = 3;
  constexpr int RD = 4;                     // LDS operand reads issued this many MFMAs ahead

  // NBUF slots, each [Q tile | dO tile | BQ floats LSE*log2(e) | BQ floats D].
  constexpr int SLOT = 2 * QT_BYTES + 2 * BQ * 4;
  constexpr int OFF_DO = QT_BYTES, OFF_L = 2 * QT_BYTES, OFF_D = 2 * QT_BYTES + BQ * 4;
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;

  int job = CAUSAL && !snake ? xcd_remap_interleaved(blockIdx.x, gridDim.x, n_kt * n_qp)
                             : xcd_remap(blockIdx.x, gridDim.x);
  // Small grids cut the query range of each key block into n_qp pieces, one workgroup each,
  // whose partials the postprocess sums (PARTIAL).
  const int piece = job % n_qp;
  job /= n_qp;
  // causal: low kt has the most query tiles
  const int kt = CAUSAL ? n_kt - 1 - causal_tile(job % n_kt, job / n_kt, n_kt, snake) : job % n_kt;
  const int bh = job / n_kt;
  const int hq = bh % Hq, b = bh / Hq;
  const int hkv = hq / (Hq / Hkv);
  const size_t kvoff = ((size_t)b * Hkv + hkv) * N * HD;
  const uint16_t* const Qh = Q + (size_t)bh * N * HD;
  const uint16_t* const dOh = dO + (size_t)bh * N * HD;
  const float* const L2h = L2 + (size_t)bh * N;
  const float* const Dh = Dl + (size_t)bh * N;

  const int kv0 = kt * BKV;
  const int kw0 = kv0 + wave * 32;  // this wave's first key
  const int key = kw0 + c;          // the key this lane's accumulator column belongs to
  const int n_qt_all = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kv0 / BQ : 0;  // earlier query tiles see none of these keys
  // this workgroup's query tiles [q_lo, n_qt): piece `piece` of [qt0, n_qt_all)
  const int q_lo = qt0 + (int)((long long)(n_qt_all - qt0) * piece / n_qp);
  const int n_qt = qt0 + (int)((long long)(n_qt_all - qt0) * (piece + 1) / n_qp);

  // Direct loads of one 64-query tile of Q, dO, L2 and D into buffer slot `sl`.
  const uint32_t rowb = (uint32_t)N * HD * 2u;
  const BufRes rQ = make_bufres(Qh, rowb), rdO = make_bufres(dOh, rowb);
  const BufRes rL = make_bufres(L2h, (uint32_t)N * 4u), rD = make_bufres(Dh, (uint32_t)N * 4u);
  uint32_t qvo[QI];
#pragma unroll
  for (int r = 0; r < QI; ++r) {
    int row, col;
    sl_pos_to_rc<BQ>((uint32_t)((wave * QI + r) * 64 + lane), row, col);
    qvo[r] = (uint32_t)(row * HD + col) * 2u;
  }
  auto issue = [&](int qt, char* dst) FA_INL {
    const uint32_t q0 = (uint32_t)qt * BQ;
#pragma unroll
    for (int r = 0; r < QI; ++r) {
      const int blk = wave * QI + r;
      dma_to_lds<16>(rQ, qvo[r], q0 * (HD * 2), dst + blk * 1024);
      dma_to_lds<16>(rdO, qvo[r], q0 * (HD * 2), dst + OFF_DO + blk * 1024);
    }
    if (wave == 0) dma_to_lds<4>(rL, (uint32_t)lane * 4u, q0 * 4u, dst + OFF_L);
    if (wave == 1) dma_to_lds<4>(rD, (uint32_t)lane * 4u, q0 * 4u, dst + OFF_D);
  };
  if (q_lo < n_qt) issue(q_lo, smem);
  if (q_lo + 1 < n_qt) issue(q_lo + 1, smem + SLOT);

  // K and V rows of this lane's key as B operands: slot j of k-step kk = K[key][kk*16 + g*8 + j]
  // (zero past the end: those keys' dK/dV are never stored).  For a negative softmax scale
  // ksign negates K, so that S c2 (c2 > 0) is still the scaled score; dK takes the signed scale.
  // They are only ever MFMA B operands and stay in AGPRs, as do the dK/dV accumulators, which
  // only MFMAs touch until the epilogue (written-out MFMAs, see fa_device.h); S and dP land in
  // VGPRs for the VALU.
  u32x4 kv[2][KST];  // [0] K, [1] V
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) {
    kv[0][kk] = ld16_if(K + kvoff + (size_t)key * HD + kk * 16 + g * 8, key < N) ^ ksign;
    kv[1][kk] = ld16_if(V + kvoff + (size_t)key * HD + kk * 16 + g * 8, key < N);
  }
  reg_fence(kv, true, true);

  // Per-lane LDS offsets: Q/dO rows in the permuted order, so register i of a unit's S/dP
  // block is query (i/8)*16 + g*8 + i%8; one offset per k-step parity.
  const uint32_t qoff[2] = {sl_off<BQ>(perm_rows(c), g * 8), sl_off<BQ>(perm_rows(c), 16 + g * 8)};
  const TrLane trl = tr_lane(lane);

  f32x16 acc[2][DB];  // [0] dK, [1] dV
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    acc[0][db] = f32x16{};
    acc[1][db] = f32x16{};
  }

  // ---- pipeline pieces.  A unit is (query tile qt, block qb): queries qt*BQ + qb*32 + 0..31,
  //      held in the LDS slot `sl` of its tile.  One wave runs per SIMD, so nothing else
  //      covers the latency of a phase's first LDS reads: each phase's first RD operand
  //      fragments, and a unit's per-query values, are read during the phase before.
  // Operand fragment i of S = Q K^T / dP = dO V^T (i = kk*2 + (0: Q, 1: dO)) of block qb.
  auto sdp_frag = [&](const char* sl, int qb, int i) FA_INL {
    const int kk = i >> 1;
    const uint32_t o = sl_off<BQ>(qb * 32, (kk >> 1) * 32) + qoff[kk & 1];
    return lds_ld128(sl + ((i & 1) ? OFF_DO : 0) + o);
  };
  // Operand fragment i of dV += P^T dO / dK += dS^T Q (i = (db*2 + t2)*2 + (0: dO, 1: Q)),
  // read transposed.
  auto dvdk_frag = [&](const char* sl, int qb, int i) FA_INL {
    const int db = i >> 2, t2 = (i >> 1) & 1;
    const uint32_t o = sl_off<BQ>(qb * 32 + t2 * 16, db * 32);
    return lds_tr8(sl + ((i & 1) ? 0 : OFF_DO) + o, trl);
  };
  // S and dP of a unit (16 MFMAs), with valu(i) under MFMA i.  Its first RD fragments come in
  // `pre`; in the last RD steps, where none of its own remain to be read, it reads the next
  // phase's first fragments (next(r), r < RD) into `post`.
  auto sdp = [&](const char* sl, int qb, f32x16& s, f32x16& dp, const u32x4 (&pre)[RD], auto&& next,
                 u32x4 (&post)[RD], auto&& valu) FA_INL {
    constexpr int NS = 2 * KST;
    u32x4 ring[RD + 1];
#pragma unroll
    for (int i = 0; i < RD; ++i) ring[i] = pre[i];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + RD < NS)
        ring[(i + RD) % (RD + 1)] = sdp_frag(sl, qb, i + RD);
      else
        post[i + RD - NS] = next(i + RD - NS);
      __builtin_amdgcn_sched_barrier(0);
      if (i & 1)  // (the loops are unrolled: one call remains per MFMA)
        mfma_va<TR, kNopNone>(dp, ring[i % (RD + 1)], kv[1][i >> 1]);
      else if (i == 0)
        mfma_va0<TR, kNopNone>(s, ring[i % (RD + 1)], kv[0][0]);
      else
        mfma_va<TR, kNopNone>(s, ring[i % (RD + 1)], kv[0][i >> 1]);
      valu(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Per-query values of a unit as this lane's accumulator registers see them: register i is
  // query qb*32 + (i/8)*16 + g*8 + i%8, so four 16-byte reads give all sixteen in order.
  // LSE*log2(e) feeds P; -D (stored negated by the preprocess) is the accumulator input of the
  // dP MFMAs, which then produce dP - D directly.
  auto rowvals = [&](const char* sl, int qb) FA_INL {
    const float* tL = reinterpret_cast<const float*>(sl + OFF_L);
    f32x4 l[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) l[t] = *reinterpret_cast<const f32x4*>(tL + qb * 32 + (t >> 1) * 16 + g * 8 + (t & 1) * 4);
    return f32x16{l[0][0], l[0][1], l[0][2], l[0][3], l[1][0], l[1][1], l[1][2], l[1][3],
                  l[2][0], l[2][1], l[2][2], l[2][3], l[3][0], l[3][1], l[3][2], l[3][3]};
  };
  auto neg_d = [&](const char* sl, int qb) FA_INL {
    const float* tD = reinterpret_cast<const float*>(sl + OFF_D);
    f32x4 d[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) d[t] = *reinterpret_cast<const f32x4*>(tD + qb * 32 + (t >> 1) * 16 + g * 8 + (t & 1) * 4);
    return f32x16{d[0][0], d[0][1], d[0][2], d[0][3], d[1][0], d[1][1], d[1][2], d[1][3],
                  d[2][0], d[2][1], d[2][2], d[2][3], d[3][0], d[3][1], d[3][2], d[3][3]};
  };
  // P = exp2(S c2 - LSE log2 e) and dS = P (dP - D) of one unit as 16 work units (one query
  // register each; dp already holds dP - D), packed into the A operands of dV += P^T dO and
  // dK += dS^T Q.  A unit runs in three stages, each on its own register of s (the exponent,
  // then P, then dS and the packing), so that consecutive MFMA steps can carry stages of
  // different units: with one wave per SIMD, a dependent chain inside one step would stall
  // the in-order issue.
  auto pds_a = [&](f32x16& s, const f32x16& l2, int i) FA_INL { s[i] = fmaf(s[i], c2, -l2[i]); };
  auto pds_b = [&](f32x16& s, int i) FA_INL { s[i] = fast_exp2(s[i]); };
  auto pds_c = [&](f32x16& s, const f32x16& dp, u32x4 (&pa)[2], u32x4 (&dsa)[2], float (&pt)[2], float (&dt)[2],
                   int i) FA_INL {
    const int t2 = i >> 3, j = i & 7;
    const float p = s[i];
    const float ds = p * dp[i];
    if (j & 1) {
      pa[t2][j >> 1] = TR::pack(pt[0], p);
      dsa[t2][j >> 1] = TR::pack(dt[0], ds);
    } else {
      pt[0] = p;
      dt[0] = ds;
    }
  };
  // Causal mask of a unit whose queries start at q0: keys after the query get -inf.
  auto mask = [&](f32x16& s, int q0) FA_INL {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = q0 + (i >> 3) * 16 + g * 8 + (i & 7);
      if (key > q) s[i] = -INFINITY;
    }
  };
  // dV += P^T dO and dK += dS^T Q of a unit (16 MFMAs).  Its first RD fragments come in `pre`;
  // `ahead()` runs after the first MFMA (the reads for the next unit), and in the last RD steps
  // it reads the next phase's first fragments (next(r)) into `post`, if HAS_POST.
  // `rare` (the last unit, which runs outside the loop): the register allocator may move
  // accumulator blocks there with v_accvgpr copies just before the MFMA that reads them, so
  // every MFMA of that unit waits 2 first.  `tail`: the epilogue follows.
  auto dvdk = [&](auto rare_tag, auto tail_tag, auto has_post_tag, const char* sl, int qb, const u32x4 (&pa)[2],
                  const u32x4 (&dsa)[2], const u32x4 (&pre)[RD], auto&& ahead, auto&& next,
                  u32x4 (&post)[RD]) FA_INL {
    constexpr int NS = 4 * DB;
    u32x4 ring[RD + 1];
#pragma unroll
    for (int i = 0; i < RD; ++i) ring[i] = pre[i];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + RD < NS)
        ring[(i + RD) % (RD + 1)] = dvdk_frag(sl, qb, i + RD);
      else if constexpr (decltype(has_post_tag)::value)
        post[i + RD - NS] = next(i + RD - NS);
      __builtin_amdgcn_sched_barrier(0);
      const int db = i >> 2, t2 = (i >> 1) & 1;
      const u32x4 a = (i & 1) ? dsa[t2] : pa[t2];
      f32x16& o = acc[(i & 1) ? 0 : 1][db];
      // (P and dS were packed by the VALU just before the first MFMA; after the last one of the
      // tail unit the epilogue reads the accumulators)
      constexpr bool RARE = decltype(rare_tag)::value, TAIL = decltype(tail_tag)::value;
      const bool before = i == 0 || RARE, after = TAIL && i == NS - 1;
      if (before && after)
        mfma_av<TR, kNopBoth>(o, a, ring[i % (RD + 1)]);
      else if (before)
        mfma_av<TR, kNopBefore>(o, a, ring[i % (RD + 1)]);
      else if (after)
        mfma_av<TR, kNopAfter>(o, a, ring[i % (RD + 1)]);
      else
        mfma_av<TR, kNopNone>(o, a, ring[i % (RD + 1)]);
      if (i == 0) ahead();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Pipeline state carried from unit to unit: the LSE*log2(e) values of the current unit, -D
  // of the next one (the dP accumulator input of its S/dP phase) and the first fragments of
  // that phase.
  f32x16 l2c, ndc;
  u32x4 sdp_pre[RD];

  // One pipeline iteration for unit u = (qt, qb) in slot `sl`: [S/dP of unit u+1 (slot `nsl`) |
  // P, dS of unit u] then [dV, dK of unit u | reads for units u+1 and u+2 (slot `n2sl`)].
  // (cs, cdp) hold u's S/dP, (ns, ndp) receive u+1's.  HAS_NEXT2: unit u+2 exists.
  auto unit = [&](bool masked, auto has_next_tag, auto has_next2_tag, int qt, int qb, const char* sl,
                  const char* nsl, const char* n2sl, f32x16& cs, f32x16& cdp, f32x16& ns, f32x16& ndp) FA_INL {
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    constexpr bool HAS_NEXT2 = decltype(has_next2_tag)::value;
    const f32x16 l2 = l2c;
    if (CAUSAL && masked) mask(cs, qt * BQ + qb * 32);  // (uniform)
    u32x4 pa[2], dsa[2], dvdk_pre[RD];
    float pt[2], dt[2];
    if constexpr (HAS_NEXT) {
      ndp = ndc;
      // unit w finishes at MFMA step h = w * 2 * KST / 16; its exponent and exp2 run one and
      // two steps earlier (clamped to the first step)
      sdp(nsl, qb ^ 1, ns, ndp, sdp_pre, [&](int r) FA_INL { return dvdk_frag(sl, qb, r); }, dvdk_pre,
          [&](int i) FA_INL {
#pragma unroll
            for (int w = 0; w < 16; ++w) {
              const int h = w * 2 * KST / 16;  // (a unit's stages in order when clamped together)
              if ((h >= 2 ? h - 2 : 0) == i) pds_a(cs, l2, w);
              if ((h >= 1 ? h - 1 : 0) == i) pds_b(cs, w);
              if (h == i) pds_c(cs, cdp, pa, dsa, pt, dt, w);
            }
          });
    } else {
#pragma unroll
      for (int w = 0; w < 16; ++w) pds_a(cs, l2, w);
#pragma unroll
      for (int w = 0; w < 16; ++w) pds_b(cs, w);
#pragma unroll
      for (int w = 0; w < 16; ++w) pds_c(cs, cdp, pa, dsa, pt, dt, w);
#pragma unroll
      for (int r = 0; r < RD; ++r) dvdk_pre[r] = dvdk_frag(sl, qb, r);
    }
    // during dV/dK of u: the LSE values of u+1 and -D of u+2, then u+2's first S/dP fragments
    // (unit u+2 has block qb, in slot n2sl)
    dvdk(std::integral_constant<bool, !HAS_NEXT>{}, std::integral_constant<bool, !HAS_NEXT>{}, has_next2_tag, sl, qb,
         pa, dsa, dvdk_pre,
         [&]() FA_INL {
           if constexpr (HAS_NEXT) l2c = rowvals(nsl, qb ^ 1);
           if constexpr (HAS_NEXT2) ndc = neg_d(n2sl, qb);
         },
         [&](int r) FA_INL { return sdp_frag(n2sl, qb, r); }, sdp_pre);
  };

  // Per query tile: wait for its successor's loads and let every wave see them (everyone is
  // then also done with the tile two back, whose slot the next loads refill), then two units.
  // The slots are restrict-qualified parameters so that the compiler can tell these reads
  // from the direct loads in flight and does not make them wait.  Unit (qt, 1)'s successors
  // (qt+1, 0) and (qt+1, 1) are in the next tile's slot, which has been complete since this
  // tile's barrier.
  f32x16 s0, dp0, s1, dp1;
  // causal: the first two tiles hold this workgroup's diagonal; every later tile is entirely
  // below it
  const int qt_m = CAUSAL ? min(n_qt, qt0 + 2) : q_lo;
  auto tile = [&](auto last_tag, int qt, char* __restrict__ cur, char* __restrict__ nxt,
                  char* __restrict__ dst) FA_INL {
    constexpr bool LAST = decltype(last_tag)::value;
    const bool masked = qt < qt_m;
    wait_vmcnt<0>();
    lds_barrier();
    if (qt + 2 < n_qt) issue(qt + 2, dst);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (LAST) {
      unit(masked, std::true_type{}, std::false_type{}, qt, 0, cur, cur, nxt, s0, dp0, s1, dp1);
      unit(masked, std::false_type{}, std::false_type{}, qt, 1, cur, nxt, nxt, s1, dp1, s0, dp0);
    } else {
      unit(masked, std::true_type{}, std::true_type{}, qt, 0, cur, cur, nxt, s0, dp0, s1, dp1);
      unit(masked, std::true_type{}, std::true_type{}, qt, 1, cur, nxt, nxt, s1, dp1, s0, dp0);
    }
  };

  if (q_lo < n_qt) {
    // prologue: S/dP of the first unit, and the reads the first iteration starts from
    wait_vmcnt<0>();
    lds_barrier();
    s0 = f32x16{};
    dp0 = neg_d(smem, 0);
    u32x4 pre[RD];
#pragma unroll
    for (int r = 0; r < RD; ++r) pre[r] = sdp_frag(smem, 0, r);
    sdp(smem, 0, s0, dp0, pre, [&](int r) FA_INL { return sdp_frag(smem, 1, r); }, sdp_pre, [](int) FA_INL {});
    l2c = rowvals(smem, 0);
    ndc = neg_d(smem, 1);
    char* c0 = smem;
    char* c1 = smem + SLOT;
    char* c2 = smem + 2 * SLOT;
    auto run = [&](auto last_tag, int qt) FA_INL {
      tile(last_tag, qt, c0, c1, c2);
      char* t = c0;
      c0 = c1;
      c1 = c2;
      c2 = t;
    };
    int qt = q_lo;
    for (; qt < n_qt - 1; ++qt) run(std::false_type{}, qt);
    run(std::true_type{}, qt);
  }

  // ---- epilogue: register i of acc[.][db] <-> key kw0 + (i/4)*8 + g*4 + i%4, column db*32 + c
  // (each store instruction covers 64 or 128 contiguous bytes of two rows; staging the rows
  // through LDS for whole-row stores, as the forward and dQ passes do, measured no faster)
  reg_fence(acc, true, false);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr_ = kw0 + (i >> 2) * 8 + g * 4 + (i & 3);
      if (kr_ >= N) continue;
      const int d = db * 32 + c;
      if (PARTIAL) {
        const size_t off = (((size_t)bh * n_qp + piece) * N + kr_) * HD + d;
        dKp[off] = acc[0][db][i] * scale;
        dVp[off] = acc[1][db][i];
      } else {
        const size_t off = kvoff + (size_t)kr_ * HD + d;
        dK[off] = (uint16_t)(TR::pack(acc[0][db][i] * scale, 0.f) & 0xffffu);
        dV[off] = (uint16_t)(TR::pack(acc[1][db][i], 0.f) & 0xffffu);
      }
    }
}

// ---------------------------------------------------------------- dK/dV partial sums
// dK/dV of KV head (b, hkv) = sum over its `grp` query heads of the fp32 partials
// (dK partials already carry the softmax scale).  Item i covers 8 consecutive elements.
template <typename TR>
__device__ FA_INL void post_dkdv_item(long long i, const float* __restrict__ dKp, const float* __restrict__ dVp,
                                      uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int grp,
                                      long long head8) {
  const long long bkv = i / head8, rem = i % head8;
  f32x4 ka = {0.f, 0.f, 0.f, 0.f}, kb = ka, va = ka, vb = ka;
  for (int h = 0; h < grp; ++h) {
    const long long src = ((bkv * grp + h) * head8 + rem) * 8;
    ka += *reinterpret_cast<const f32x4*>(dKp + src);
    kb += *reinterpret_cast<const f32x4*>(dKp + src + 4);
    va += *reinterpret_cast<const f32x4*>(dVp + src);
    vb += *reinterpret_cast<const f32x4*>(dVp + src + 4);
  }
  *reinterpret_cast<u32x4*>(dK + i * 8) =
      u32x4{TR::pack(ka[0], ka[1]), TR::pack(ka[2], ka[3]), TR::pack(kb[0], kb[1]), TR::pack(kb[2], kb[3])};
  *reinterpret_cast<u32x4*>(dV + i * 8) =
      u32x4{TR::pack(va[0], va[1]), TR::pack(va[2], va[3]), TR::pack(vb[0], vb[1]), TR::pack(vb[2], vb[3])};
}

// ---------------------------------------------------------------- dQ
// Query-stationary: a workgroup owns 64, 128 or 256 query rows (32 per wave) of one head and
// streams 32-key tiles of K and V of its KV head through LDS (direct loads issued DIST tiles
// ahead into DIST + 1 K buffers and DIST V buffers, DIST = 3, or 2 where two workgroups of
// D = 128 share a CU; one barrier per tile).  Per tile j, per wave:
//   S^T = K Q^T and dP^T = V dO^T  (K, V rows from LDS; Q and dO fragments in registers)
//   dS^T = exp2(S^T c2 - LSE log2 e) * (dP^T - D)        (fp32, one query per lane)
//   dQ^T += K^T dS^T  (K^T read transposed from the K tile; the rounded dS^T registers are
//                      the B operand thanks to the permuted K rows)
// software-pipelined inside the wave: the VALU work of tile j runs under the MFMAs of S^T and
// dP^T of tile j+1, then the dQ MFMAs of tile j follow.  Keys past the end read as zero rows
// of K and V, so their dS^T K terms vanish; only the causal diagonal needs masks.  Every dQ
// element is produced by exactly one lane: no atomics, bitwise deterministic.
// SPLIT = 2: two wave groups own the same query rows and take the two halves of the key range,
// each with its own LDS buffers; group 1 hands its dQ^T partial to group 0 through LDS at the
// end (one fixed-order addition, still deterministic).
// PART: small grids also cut each query tile's key range into n_kp pieces, one workgroup
// each; a piece writes its unscaled fp32 dQ partial (dQp) and bwd_dq_sum_kernel adds them.
// SUMS: the workgroups also run the grouped-query dK/dV partial sums (post_dkdv_item) after
// their own dQ rows, each an interval of the n8post items: on a one-round causal grid weighted
// by n_qt - qt towards the light tiles, which finish early, else equal.  (fa_bwd uses this in
// place of the separate postprocess launch where the grid has no key-range pieces.)
// ROWS: the pass forms its rows' D and LSE*log2(e) itself, from O, dO and the LSE, and stores
// them (-D and LSE*log2(e)) for the dK/dV pass that follows it, in place of the preprocess
// launch.  The sum runs in the preprocess kernel's order (the same per-16-byte FMA chains, the
// same pairwise tree), so both routes give the same bits.  (fa_bwd runs the dQ pass first this
// way wherever the dK/dV pass writes no partials.)
template <typename TR, int HD, bool CAUSAL, int NW, int SPLIT, bool PART, bool SUMS, bool ROWS, int DIST>
__global__ void __launch_bounds__(NW * 64, 8 / NW)
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
              const float* __restrict__ L2, const float* __restrict__ Dl, uint16_t* __restrict__ dQ,
              int Hq, int Hkv, int N, int n_qt, float c2, float scale, uint32_t qsign, int snake, int n_kp,
              float* __restrict__ dQp, const float* __restrict__ dKp, const float* __restrict__ dVp,
              uint16_t* __restrict__ dKo, uint16_t* __restrict__ dVo, int pgrp, long long head8, long long n8post,
              const uint16_t* __restrict__ Oin, const float* __restrict__ LSEin, float* __restrict__ L2o,
              float* __restrict__ Dlo) {
  static_assert(SPLIT == 1 || SPLIT == 2, "one or two groups");
  static_assert(!(SUMS && PART), "the fused partial sums run on grids without key-range pieces");
  static_assert(!(SUMS && ROWS), "the partial sums follow a dK/dV pass, the row values precede one");
  constexpr int GW = NW / SPLIT;            // waves per group
  constexpr int BR = GW * 32, BC = kDqBC;  // query rows per workgroup (32 per wave), keys per tile
  constexpr int KST = HD / 16;              // k-steps over the head dim
  constexpr int DB = HD / 32;               // 32-row blocks of dQ^T
  constexpr int TILE = BC * HD * 2;         // bytes of one K or V tile
  constexpr int TI = TILE / 1024 / GW;      // 1 KB direct loads per wave per tile
  static_assert(TI * 1024 * GW == TILE, "tile must split into 1 KB loads over the waves");
  static_assert(DIST == 2 || DIST == 3, "loads two or three tiles ahead");
  constexpr int NK = DIST + 1, NV = DIST;  // K tiles j..j+DIST, V tiles j+1..j+DIST
  constexpr int RD = 3;                     // LDS operand reads issued this many MFMAs ahead

  __shared__ __attribute__((aligned(1024))) char smem[SPLIT * (NK + NV) * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / GW;  // group (0 when SPLIT = 1)
  const int wv = wave % GW;   // wave within the group
  const int c = lane & 31, g = lane >> 5;

  int job = CAUSAL && !snake ? xcd_remap_interleaved(blockIdx.x, gridDim.x, n_qt * (PART ? n_kp : 1))
                             : xcd_remap(blockIdx.x, gridDim.x);
  int part = 0;  // piece of the key range (PART)
  if constexpr (PART) {
    part = job % n_kp;
    job /= n_kp;
  }
  int qt = job % n_qt;
  const int bh = job / n_qt;
  if (CAUSAL) qt = causal_tile(qt, bh, n_qt, snake);
  const int hq = bh % Hq, b = bh / Hq;
  const int hkv = hq / (Hq / Hkv);
  const uint16_t* const Kh = K + ((size_t)b * Hkv + hkv) * N * HD;
  const uint16_t* const Vh = V + ((size_t)b * Hkv + hkv) * N * HD;

  const int qw0 = qt * BR + wv * 32;  // first query row of this wave
  const int qi = qw0 + c;             // the query of this lane's accumulator column

  // Key tiles the workgroup streams, and the prefix this wave computes on (causal waves stop
  // at the tile holding their diagonal; waves wholly past the last row compute nothing).
  int T = (N + BC - 1) / BC;
  if (CAUSAL) T = (min(N, (qt + 1) * BR) - 1) / BC + 1;
  int Tw = T;
  if (CAUSAL) Tw = (min(N, qw0 + 32) - 1) / BC + 1;
  if (qw0 >= N) Tw = 0;
  // This group's tiles [t0, t0 + Tg) (group 0 takes the larger half), the steps every wave
  // takes (the larger group's tile count), and how many of the group's tiles this wave
  // computes on; the wave's diagonal tile Tw - 1, when in the group's range, is its last.
  const int tb = PART ? (int)((long long)T * part / n_kp) : 0;  // this workgroup's piece [tb, te)
  const int te = PART ? (int)((long long)T * (part + 1) / n_kp) : T;
  const int half = SPLIT == 2 ? (te - tb + 1) / 2 : te - tb;
  const int t0 = tb + (grp ? half : 0);
  const int Tg = grp ? te - tb - half : half;
  const int Twg = max(0, min(Tw - t0, Tg));

  // Direct loads of K/V tile t (keys past the end read as zero).
  const BufRes rK = make_bufres(Kh, (uint32_t)N * HD * 2u), rV = make_bufres(Vh, (uint32_t)N * HD * 2u);
  uint32_t kvo[TI];
#pragma unroll
  for (int r = 0; r < TI; ++r) {
    int row, col;
    sl_pos_to_rc<BC>((uint32_t)((wv * TI + r) * 64 + lane), row, col);
    kvo[r] = (uint32_t)(row * HD + col) * 2u;
  }
  auto issue_k = [&](int t, char* dK_) FA_INL {
#pragma unroll
    for (int r = 0; r < TI; ++r)
      dma_to_lds<16>(rK, kvo[r], (uint32_t)(t0 + t) * (BC * HD * 2), dK_ + (wv * TI + r) * 1024);
  };
  auto issue_v = [&](int t, char* dV_) FA_INL {
#pragma unroll
    for (int r = 0; r < TI; ++r)
      dma_to_lds<16>(rV, kvo[r], (uint32_t)(t0 + t) * (BC * HD * 2), dV_ + (wv * TI + r) * 1024);
  };
  auto issue = [&](int t, char* dK_, char* dV_) FA_INL {
    issue_k(t, dK_);
    issue_v(t, dV_);
  };
  char* const kb0 = smem + grp * ((NK + NV) * TILE);  // K buffers kb0 + i*TILE, i < NK
  char* const vb0 = kb0 + NK * TILE;                   // V buffers vb0 + i*TILE, i < NV
  // the group's tiles t < DIST go to K buffer t and V buffer t
#pragma unroll
  for (int t = 0; t < DIST; ++t)
    if (t < Tg) issue(t, kb0 + t * TILE, vb0 + t * TILE);

  // B operands: slot j of k-step kk = Q[qi][kk*16 + g*8 + j] and dO[qi][...]
  const size_t rowoff = (size_t)bh * N * HD + (size_t)qi * HD;
  u32x4 qf[KST], of[KST];
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) {
    qf[kk] = ld16_if(Q + rowoff + kk * 16 + g * 8, qi < N) ^ qsign;  // -Q for a negative scale
    of[kk] = ld16_if(dO + rowoff + kk * 16 + g * 8, qi < N);
  }
  float l2, nd;  // LSE*log2(e) and -D of this lane's query
  if constexpr (ROWS) {
    // D = sum_d dO O over the row: 16-byte chunk p = kk*2 + g of the row is this lane's
    // fragment kk (the other half of the row is in lane ^ 32).  Each chunk is one FMA chain in
    // element order, then the chunks pair up as chunk p with chunk p ^ 2^m for m = 3, 2, 1
    // (HD = 128) or 2, 1 (HD = 64), in this lane, and m = 0 with the partner lane: the
    // preprocess kernel's shuffle tree, term for term.
    u32x4 ofr[KST];
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) ofr[kk] = ld16_if(Oin + rowoff + kk * 16 + g * 8, qi < N);
    float cs[KST];
#pragma unroll
    for (int kk = 0; kk < KST; ++kk) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = fmaf(TR::lo(ofr[kk][w]), TR::lo(of[kk][w]), acc);
        acc = fmaf(TR::hi(ofr[kk][w]), TR::hi(of[kk][w]), acc);
      }
      cs[kk] = acc;
    }
#pragma unroll
    for (int st = KST / 2; st >= 1; st >>= 1)
#pragma unroll
      for (int kk = 0; kk < st; ++kk) cs[kk] += cs[kk + st];
    const float dsum = pair_sum(cs[0]);
    l2 = qi < N ? LSEin[(size_t)bh * N + qi] * kLog2e : 0.f;
    nd = qi < N ? -dsum : 0.f;
    // one writer per query: group 0, key piece 0, the lane of the row's first half
    if (qi < N && g == 0 && grp == 0 && (!PART || part == 0)) {
      L2o[(size_t)bh * N + qi] = l2;
      Dlo[(size_t)bh * N + qi] = nd;
    }
  } else {
    l2 = qi < N ? L2[(size_t)bh * N + qi] : 0.f;
    nd = qi < N ? Dl[(size_t)bh * N + qi] : 0.f;
  }
  // On the large grids (one group per workgroup) every dP^T accumulator of a tile starts at -D
  // (all 16 registers of a lane hold its query's value), so the MFMAs yield dP^T - D directly
  // (dQ pass 1.8-2% faster there; the split-key workgroups measured 2-3% slower with it).
  constexpr bool DP_FROM_ND = SPLIT == 1;
  f32x16 ndv;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndv[i] = DP_FROM_ND ? nd : 0.f;

  const uint32_t koff[2] = {sl_off<BC>(perm_rows(c), g * 8), sl_off<BC>(perm_rows(c), 16 + g * 8)};
  const TrLane trl = tr_lane(lane);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // ---- pipeline pieces
  // S^T and dP^T of one tile (register i <-> key (i/8)*16 + g*8 + i%8), with valu(i) run
  // under MFMA i.
  // dQ^T fragment i of tile tK (i = db*2 + t2): K^T read transposed.
  auto qfrag = [&](const char* tK, int i) FA_INL {
    return lds_tr8(tK + sl_off<BC>((i & 1) * 16, (i >> 1) * 32), trl);
  };
  // With POST the last RD steps read the dQ phase's first fragments (of tile pK) into post.
  auto sdp = [&](auto post_tag, const char* tK, const char* tV, f32x16& s, f32x16& dp, auto&& valu,
                 const char* pK, u32x4 (&post)[RD]) FA_INL {
    constexpr bool POST = decltype(post_tag)::value;
    auto frag = [&](int i) FA_INL {  // i = kk*2 + (0: K, 1: V)
      const int kk = i >> 1;
      return lds_ld128(((i & 1) ? tV : tK) + sl_off<BC>(0, (kk >> 1) * 32) + koff[kk & 1]);
    };
    u32x4 ring[RD + 1];
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      ring[i] = frag(i);  // in use order, so each wait is partial
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 2 * KST; ++i) {
      if (i + RD < 2 * KST)
        ring[(i + RD) % (RD + 1)] = frag(i + RD);
      else if constexpr (POST)
        post[i + RD - 2 * KST] = qfrag(pK, i + RD - 2 * KST);
      __builtin_amdgcn_sched_barrier(0);
      if (i & 1)
        dp = TR::mfma(ring[i % (RD + 1)], of[i >> 1], dp);
      else
        s = TR::mfma(ring[i % (RD + 1)], qf[i >> 1], s);
      valu(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // dS^T of tile j as 16 work units (one key register each), packed into the B operand of
  // dQ^T += K^T dS^T.  Causal masks (keys after the query) on the wave's last tile only.
  auto ds_unit = [&](auto masked_tag, int j, const f32x16& s, const f32x16& dp, u32x4 (&dsb)[2], float& dt,
                     int i) FA_INL {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float sv = s[i];
    if constexpr (MASKED) {
      const int key = (t0 + j) * BC + (i >> 3) * 16 + g * 8 + (i & 7);
      if (key > qi) sv = -INFINITY;
    }
    const float ds = fast_exp2(fmaf(sv, c2, -l2)) * (DP_FROM_ND ? dp[i] : dp[i] + nd);
    if (i & 1)
      dsb[i >> 3][(i & 7) >> 1] = TR::pack(dt, ds);
    else
      dt = ds;
  };
  // dQ^T += K^T dS^T of one tile (2*DB MFMAs), A operand read transposed from the K tile.
  auto dqm = [&](auto pre_tag, const char* tK, const u32x4 (&dsb)[2], const u32x4 (&pre)[RD]) FA_INL {
    constexpr bool PRE = decltype(pre_tag)::value;
    auto frag = [&](int i) FA_INL { return qfrag(tK, i); };  // i = db*2 + t2
    constexpr int NS = 2 * DB;
    u32x4 ring[RD + 1];
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      if constexpr (PRE)
        ring[i] = pre[i];
      else
        ring[i] = frag(i);  // in use order, so each wait is partial
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + RD < NS) ring[(i + RD) % (RD + 1)] = frag(i + RD);
      __builtin_amdgcn_sched_barrier(0);
      acc[i >> 1] = TR::mfma(ring[i % (RD + 1)], dsb[i & 1], acc[i >> 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Step j (0 <= j < T): wait for tile j+1 (with DIST = 3, tile j+2 may stay in flight), let
  // every wave see it (everyone is then also done with step j-1, whose buffers the next loads
  // refill), load tile j+DIST, then [S^T/dP^T of tile j+1 | dS^T of tile j] and dQ of tile j.
  // (cs, cdp) hold tile j's S^T/dP^T, (ns, ndp) receive tile j+1's.  The LDS buffers are
  // restrict-qualified parameters so that the compiler can tell these reads from the loads in
  // flight.
  enum Kind { kSteady, kLast, kLastMasked, kIdle };
  auto step = [&](auto kind_tag, const int j, const char* __restrict__ tK, const char* __restrict__ nK,
                  const char* __restrict__ nV, char* __restrict__ dK_, char* __restrict__ dV_, f32x16& cs,
                  f32x16& cdp, f32x16& ns, f32x16& ndp) FA_INL {
    constexpr Kind KIND = decltype(kind_tag)::value;
    if (DIST == 3 && j + 2 < Tg)
      wait_vmcnt<2 * TI>();
    else
      wait_vmcnt<0>();
    dma_barrier();
    if constexpr (KIND != kSteady)
      if (j + DIST < Tg) issue(j + DIST, dK_, dV_);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 dsb[2];
    float dt;
    u32x4 qpre[RD];
    if constexpr (KIND == kSteady) {
      ns = f32x16{};
      ndp = ndv;
      // the next tile's loads go out under the first MFMAs (K after the first, V after the third:
      // 0.3-0.7% faster than both after the second).  Where two waves share a SIMD, the one in
      // its S/dP phase (MFMAs interleaved with the dS VALU work) issues first; the one in its
      // dQ phase, MFMAs only, fills the gaps (0.8-1.1% faster than equal priority, and than the
      // reverse order).
      __builtin_amdgcn_s_setprio(1);
      sdp(std::true_type{}, nK, nV, ns, ndp, [&](int i) FA_INL {
        if (i == 0 && j + DIST < Tg) issue_k(j + DIST, dK_);
        if (i == 2 && j + DIST < Tg) issue_v(j + DIST, dV_);
#pragma unroll
        for (int w = 0; w < 16; ++w)
          if (w * 2 * KST / 16 == i) ds_unit(std::false_type{}, j, cs, cdp, dsb, dt, w);
      }, tK, qpre);
      __builtin_amdgcn_s_setprio(0);
      dqm(std::true_type{}, tK, dsb, qpre);
    } else if constexpr (KIND == kLast || KIND == kLastMasked) {
#pragma unroll
      for (int w = 0; w < 16; ++w) ds_unit(std::bool_constant<KIND == kLastMasked>{}, j, cs, cdp, dsb, dt, w);
      dqm(std::false_type{}, tK, dsb, qpre);
    }
  };

  // Buffer rings: kr = K tiles j .. j+DIST-1 and the slot for j+DIST; vr = V tiles
  // j+1 .. j+DIST-1 and the slot for j+DIST (tile 0's V buffer, free after the prologue).
  char* kr[NK];
  char* vr[NV];
#pragma unroll
  for (int i = 0; i < NK; ++i) kr[i] = kb0 + i * TILE;
#pragma unroll
  for (int i = 0; i < NV; ++i) vr[i] = vb0 + ((i + 1) % NV) * TILE;
  f32x16 sa, dpa, sb, dpb;
  auto run = [&](auto kind_tag, int j, f32x16& cs, f32x16& cdp, f32x16& ns, f32x16& ndp) FA_INL {
    step(kind_tag, j, kr[0], kr[1], vr[0], kr[NK - 1], vr[NV - 1], cs, cdp, ns, ndp);
    char* const t = kr[0];
#pragma unroll
    for (int i = 0; i + 1 < NK; ++i) kr[i] = kr[i + 1];
    kr[NK - 1] = t;
    char* const u = vr[0];
#pragma unroll
    for (int i = 0; i + 1 < NV; ++i) vr[i] = vr[i + 1];
    vr[NV - 1] = u;
  };
  using KSteady = std::integral_constant<Kind, kSteady>;
  using KLast = std::integral_constant<Kind, CAUSAL ? kLastMasked : kLast>;
  using KIdle = std::integral_constant<Kind, kIdle>;

  // prologue: tile 0 resident (tiles 1 .. DIST-1 may stay in flight), S^T/dP^T of tile 0
  if (DIST == 3 && Tg > 2)
    wait_vmcnt<4 * TI>();
  else if (Tg > 1)
    wait_vmcnt<2 * TI>();
  else
    wait_vmcnt<0>();
  dma_barrier();
  if (Twg > 0) {
    sa = f32x16{};
    dpa = ndv;
    u32x4 unused[RD];
    sdp(std::false_type{}, kb0, vb0, sa, dpa, [](int) FA_INL {}, kb0, unused);
  }
  // Every wave takes exactly `half` steps (one barrier each); the group's last computed tile
  // is the only one that can need masks.
  int j = 0;
  for (; j + 2 <= Twg - 1; j += 2) {
    run(KSteady{}, j, sa, dpa, sb, dpb);
    run(KSteady{}, j + 1, sb, dpb, sa, dpa);
  }
  if (j < Twg - 1) {
    run(KSteady{}, j, sa, dpa, sb, dpb);
    ++j;
    run(KLast{}, j, sb, dpb, sa, dpa);
    ++j;
  } else if (j == Twg - 1) {
    run(KLast{}, j, sa, dpa, sb, dpb);
    ++j;
  }
  for (; j < half; ++j) run(KIdle{}, j, sa, dpa, sb, dpb);

  // ---- split workgroups: group 1 hands its dQ^T partial to the group-0 wave that owns the
  // same rows, through LDS (free once every wave has passed the barrier).
  if constexpr (SPLIT == 2) {
    static_assert(GW * 64 * 16 * DB * 4 <= (int)sizeof(smem), "exchange must fit in the K/V buffers");
    float* const xs = reinterpret_cast<float*>(smem) + wv * (64 * 16 * DB) + lane;
    lds_barrier();
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) xs[(db * 16 + i) * 64] = acc[db][i];
    }
    lds_barrier();
    if (grp == 1) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] += xs[(db * 16 + i) * 64];
  }

  // ---- epilogue: register i of acc[db] <-> dQ[qi][db*32 + (i/4)*8 + g*4 + i%4]
  if constexpr (PART) {
    if (qi < N) {
      float* const prow = dQp + (((size_t)bh * n_kp + part) * N + qi) * HD;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<f32x4*>(prow + db * 32 + i4 * 8 + g * 4) =
              f32x4{acc[db][i4 * 4 + 0], acc[db][i4 * 4 + 1], acc[db][i4 * 4 + 2], acc[db][i4 * 4 + 3]};
    }
    return;
  }
  // dQ rows go out through LDS, whole rows per store instruction (stage_row, store_staged).
  // Eight waves of one group need more than the K/V buffers hold: they stage the two halves
  // of their columns one after the other.
  constexpr int PASSES = SPLIT == 2 || GW * 32 * HD * 2 <= (int)sizeof(smem) ? 1 : 2;
  constexpr int HDP = HD / PASSES;  // columns per pass
  char* qs;
  if constexpr (SPLIT == 2) {
    qs = smem + wv * (64 * 16 * DB * 4);  // the hand-off region this wave has just read
  } else {
    lds_store_barrier();                  // every wave is done with the K/V buffers
    qs = smem + wv * (32 * HDP * 2);
  }
  static_assert(32 * HDP * 2 <= (SPLIT == 2 ? 64 * 16 * DB * 4 : (int)sizeof(smem) / GW), "dQ rows must fit the region");
  u32x2 w[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      w[db][i4] = u32x2{TR::pack(acc[db][i4 * 4 + 0] * scale, acc[db][i4 * 4 + 1] * scale),
                        TR::pack(acc[db][i4 * 4 + 2] * scale, acc[db][i4 * 4 + 3] * scale)};
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    stage_row<HDP>(qs, c, g, reinterpret_cast<const u32x2(&)[HDP / 32][4]>(w[p * (DB / PASSES)]));
    store_staged<HDP * 2, 32, HD * 2>(qs, dQ + ((size_t)bh * N + qw0) * HD + p * HDP, N - qw0, lane);
  }

  if constexpr (SUMS) {
    constexpr int NT = (SPLIT == 2 ? GW : NW) * 64;  // the threads still here (group 1 has left)
    const long long heads = gridDim.x / n_qt;      // B * Hq
    long long lo, hi;
    if (CAUSAL && snake) {
      // weights n_qt - t for tile t of every head, in (head, tile) order
      const long long wh = (long long)n_qt * (n_qt + 1) / 2;
      const long long pre = (long long)bh * wh + (long long)qt * n_qt - (long long)qt * (qt - 1) / 2;
      const long long tot = heads * wh;
      lo = n8post * pre / tot;
      hi = n8post * (pre + n_qt - qt) / tot;
    } else {
      const long long j = (long long)bh * n_qt + qt;
      lo = n8post * j / gridDim.x;
      hi = n8post * (j + 1) / gridDim.x;
    }
    for (long long i = lo + tid; i < hi; i += NT) post_dkdv_item<TR>(i, dKp, dVp, dKo, dVo, pgrp, head8);
  }
}

// ---------------------------------------------------------------- postprocess
// dK/dV of KV head (b, hkv) = sum over its `grp` query heads of the fp32 partials, one
// item per thread (post_dkdv_item).
template <typename TR>
__global__ void __launch_bounds__(kThreads)
bwd_post_dkdv_kernel(const float* __restrict__ dKp, const float* __restrict__ dVp,
                     uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int grp,
                     long long head8, long long n8) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n8) return;
  post_dkdv_item<TR>(i, dKp, dVp, dK, dV, grp, head8);
}

// dQ of row (bh, n) = scale * the sum, in piece order, of its n_kp fp32 partials.
template <typename TR, int HD>
__global__ void __launch_bounds__(kThreads)
bwd_dq_sum_kernel(const float* __restrict__ dQp, uint16_t* __restrict__ dQ, int n_kp, int N, float scale,
                  long long n8) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n8) return;
  constexpr int C8 = HD / 8;
  const long long row = i / C8, bh = row / N, n = row % N;
  const int d0 = (int)(i % C8) * 8;
  f32x4 a = {0.f, 0.f, 0.f, 0.f}, c = a;
  for (int p = 0; p < n_kp; ++p) {
    const float* src = dQp + ((bh * n_kp + p) * N + n) * HD + d0;
    a += *reinterpret_cast<const f32x4*>(src);
    c += *reinterpret_cast<const f32x4*>(src + 4);
  }
  *reinterpret_cast<u32x4*>(dQ + i * 8) =
      u32x4{TR::pack(a[0] * scale, a[1] * scale), TR::pack(a[2] * scale, a[3] * scale),
            TR::pack(c[0] * scale, c[1] * scale), TR::pack(c[2] * scale, c[3] * scale)};
}

// ---------------------------------------------------------------- launchers

template <typename TR, int HD>
hipError_t pre_t(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  const long long rows = a.B * a.Hq * a.N;
  constexpr int RPB = kThreads / (HD / 8) * kPreRows;
  const long long need = (rows + RPB - 1) / RPB;
  const long long blocks = need < kPreBlocks ? need : kPreBlocks;
  hipLaunchKernelGGL((bwd_pre_kernel<TR, HD>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout), a.lse,
                     reinterpret_cast<float*>(a.ws + w.delta), reinterpret_cast<float*>(a.ws + w.lse2), rows);
  return hipGetLastError();
}

// c2 must be > 0 so that exp2(-inf * c2) is an exact 0 for masked scores; a zero scale
// becomes 2^-100, for which every exp2 rounds to exactly 1 (uniform weights).  A negative scale
// runs as |scale| with the stationary operand of S negated (sign_bits flips the sign bit of
// every 16-bit element): the scaled scores are unchanged, and the gradients dQ and dK are
// multiplied by the signed scale.
inline float exp2_factor(float scale) {
  const float as = fabsf(scale);
  return as > 0.f ? as * kLog2e : 0x1p-100f;
}
inline uint32_t sign_bits(float scale) { return scale < 0.f ? 0x80008000u : 0u; }

template <typename TR, int HD, bool CAUSAL, bool PARTIAL>
hipError_t dkdv_t(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  const int n_kt = (int)((a.N + kBwdBKV - 1) / kBwdBKV);
  const long long blocks = a.B * a.Hq * (long long)n_kt * w.n_qp;
  float* const dkp = PARTIAL ? reinterpret_cast<float*>(a.ws + w.dk_part) : nullptr;
  float* const dvp = PARTIAL ? reinterpret_cast<float*>(a.ws + w.dv_part) : nullptr;
  hipLaunchKernelGGL((bwd_dkdv_kernel<TR, HD, CAUSAL, PARTIAL>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout),
                     reinterpret_cast<const float*>(a.ws + w.lse2), reinterpret_cast<const float*>(a.ws + w.delta),
                     static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), dkp, dvp, (int)a.Hq, (int)a.Hkv,
                     (int)a.N, n_kt, exp2_factor(a.scale), a.scale, sign_bits(a.scale), (int)grid_fits(blocks, 1),
                     w.n_qp);
  return hipGetLastError();
}

template <typename TR, int HD>
hipError_t dkdv_hd(const BwdArgs& a) {
  const bool partial = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D).partial_dkdv;
  if (a.causal) return partial ? dkdv_t<TR, HD, true, true>(a) : dkdv_t<TR, HD, true, false>(a);
  return partial ? dkdv_t<TR, HD, false, true>(a) : dkdv_t<TR, HD, false, false>(a);
}

template <typename TR, int HD, bool CAUSAL, int NW, int SPLIT, bool PART = false, bool POST = false,
          bool ROWS = false, int DIST = 3>
hipError_t dq_nw(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  constexpr int BR = NW / SPLIT * 32;
  const int n_qt = (int)((a.N + BR - 1) / BR);
  const int n_kp = PART ? w.n_kp : 1;
  const long long blocks = a.B * a.Hq * (long long)n_qt * n_kp;
  float* const dqp = PART ? reinterpret_cast<float*>(a.ws + w.dq_part) : nullptr;
  // (POST: the grouped-query dK/dV partial sums ride along, as in post_t; ROWS: the pass forms
  // the row values the preprocess would have stored, and stores them)
  const long long kv8 = POST ? a.B * a.Hkv * a.N * a.D / 8 : 0;
  float* const lse2 = reinterpret_cast<float*>(a.ws + w.lse2);
  float* const delta = reinterpret_cast<float*>(a.ws + w.delta);
  hipLaunchKernelGGL((bwd_dq_kernel<TR, HD, CAUSAL, NW, SPLIT, PART, POST, ROWS, DIST>), dim3((unsigned)blocks),
                     dim3(NW * 64), 0, a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout),
                     ROWS ? nullptr : lse2, ROWS ? nullptr : delta,
                     static_cast<uint16_t*>(a.dq), (int)a.Hq, (int)a.Hkv, (int)a.N, n_qt, exp2_factor(a.scale),
                     a.scale, sign_bits(a.scale), (int)grid_fits(blocks, 8 / NW), n_kp, dqp,
                     POST ? reinterpret_cast<const float*>(a.ws + w.dk_part) : nullptr,
                     POST ? reinterpret_cast<const float*>(a.ws + w.dv_part) : nullptr,
                     POST ? static_cast<uint16_t*>(a.dk) : nullptr, POST ? static_cast<uint16_t*>(a.dv) : nullptr,
                     (int)(a.Hq / a.Hkv) * w.n_qp, a.N * a.D / 8, kv8,
                     ROWS ? static_cast<const uint16_t*>(a.o) : nullptr, ROWS ? a.lse : nullptr,
                     ROWS ? lse2 : nullptr, ROWS ? delta : nullptr);
  if constexpr (PART) {
    FA_HIP_TRY(hipGetLastError());
    const long long n8 = a.B * a.Hq * a.N * a.D / 8;
    hipLaunchKernelGGL((bwd_dq_sum_kernel<TR, HD>), dim3((unsigned)((n8 + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, a.stream, dqp, static_cast<uint16_t*>(a.dq), n_kp, (int)a.N, a.scale, n8);
  }
  return hipGetLastError();
}

// 256-query workgroups (8 waves, one workgroup per CU) halve the K/V traffic from L2 per
// query, which lowers the power the pass draws and lets the clock rise; D = 64 tiles are too
// small to split over 8 waves.  Smaller grids use 128-query tiles: 8-wave workgroups that split
// the key range over two wave groups (causal grids, whose tiles carry uneven work, and grids
// too small to give every CU two 4-wave workgroups), else 4-wave workgroups, two per CU.  A
// causal grid that runs in one round takes 64-query tiles, split over two groups of two waves,
// two workgroups per CU (at D = 128 with loads two tiles ahead, so that two fit the LDS): its
// causal_tile order hands every CU a heavy and a light tile.
// With `post` (fa_bwd, when the dK/dV pass wrote partials) the pass also runs their sums
// unless its grid takes key-range pieces; *fused says whether it did.  With `rows` (fa_bwd,
// when the dK/dV pass writes no partials) the pass runs first and forms the row values itself.
enum class DqMode { kPlain, kPost, kRows };
template <typename TR, int HD, bool CAUSAL, int NW, int SPLIT, bool PART = false, int DIST = 3>
hipError_t dq_mode(const BwdArgs& a, DqMode m) {
  if constexpr (!PART)
    if (m == DqMode::kPost) return dq_nw<TR, HD, CAUSAL, NW, SPLIT, false, true, false, DIST>(a);
  if (m == DqMode::kRows) return dq_nw<TR, HD, CAUSAL, NW, SPLIT, PART, false, true, DIST>(a);
  return dq_nw<TR, HD, CAUSAL, NW, SPLIT, PART, false, false, DIST>(a);
}
template <typename TR, int HD, bool CAUSAL>
hipError_t dq_t(const BwdArgs& a, DqMode m, bool* fused) {
  const long long big = a.B * a.Hq * ((a.N + 255) / 256);
  const bool pieces = bwd_key_pieces(a.B, a.Hq, a.N, a.D) > 1;
  if (m == DqMode::kPost && pieces) m = DqMode::kPlain;
  *fused = m == DqMode::kPost;
  if constexpr (HD == 128)
    if (big >= 512) return dq_mode<TR, HD, CAUSAL, 8, 1>(a, m);
  if (pieces) return dq_mode<TR, HD, CAUSAL, 8, 2, true>(a, m);
  if constexpr (CAUSAL)
    if (grid_fits(a.B * a.Hq * ((a.N + 63) / 64), 2)) return dq_mode<TR, HD, CAUSAL, 4, 2, false, HD == 128 ? 2 : 3>(a, m);
  if (a.causal || a.B * a.Hq * ((a.N + 127) / 128) < 512) return dq_mode<TR, HD, CAUSAL, 8, 2>(a, m);
  return dq_mode<TR, HD, CAUSAL, 4, 1>(a, m);
}

template <typename TR>
hipError_t dq_dt(const BwdArgs& a, DqMode m, bool* fused) {
  if (a.D == 64) return a.causal ? dq_t<TR, 64, true>(a, m, fused) : dq_t<TR, 64, false>(a, m, fused);
  return a.causal ? dq_t<TR, 128, true>(a, m, fused) : dq_t<TR, 128, false>(a, m, fused);
}

template <typename TR>
hipError_t post_t(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  if (!w.partial_dkdv) return hipSuccess;  // dK and dV were written directly
  const long long kv8 = a.B * a.Hkv * a.N * a.D / 8;
  hipLaunchKernelGGL((bwd_post_dkdv_kernel<TR>), dim3((unsigned)((kv8 + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, a.stream, reinterpret_cast<const float*>(a.ws + w.dk_part),
                     reinterpret_cast<const float*>(a.ws + w.dv_part), static_cast<uint16_t*>(a.dk),
                     static_cast<uint16_t*>(a.dv), (int)(a.Hq / a.Hkv) * w.n_qp, a.N * a.D / 8, kv8);
  return hipGetLastError();
}

}  // namespace

// Query-range pieces of the dK/dV pass: a grid that gives the CUs too few workgroups cuts each
// key block's query range into pieces whose fp32 partials the postprocess sums.  Grouped-query
// heads write partials anyway, so there the pieces also even out the causal spread of work
// between key blocks: enough for two workgroups per workgroup slot (one slot per CU at D = 128,
// two at D = 64; measured +3-6% on causal GQA training steps at N = 2048-4096).  Each piece
// keeps at least eight 64-query tiles.
int bwd_query_pieces(long long B, long long Hq, long long Hkv, long long N, long long D) {
  const long long grid = B * Hq * ((N + kBwdBKV - 1) / kBwdBKV);
  const long long target = Hq != Hkv ? (D == 64 ? 1024 : 512) : 256;
  if (grid >= target) return 1;
  long long p = (target + grid - 1) / grid;
  const long long cap = (N + kBwdBQ - 1) / kBwdBQ / 8;
  p = p < cap ? p : cap;
  return (int)(p < 1 ? 1 : (p > 64 ? 64 : p));
}

// Key-range pieces of the dQ pass where it runs as split 128-query workgroups (one per CU),
// each half-piece keeping at least four 32-key tiles.
int bwd_key_pieces(long long B, long long Hq, long long N, long long D) {
  if (D == 128 && B * Hq * ((N + 255) / 256) >= 512) return 1;
  const long long grid = B * Hq * ((N + 127) / 128);
  if (grid >= 256) return 1;
  long long p = (256 + grid - 1) / grid;
  const long long cap = (N + kDqBC - 1) / kDqBC / 8;
  p = p < cap ? p : cap;
  return (int)(p < 1 ? 1 : (p > 64 ? 64 : p));
}

hipError_t launch_bwd_preprocess(const BwdArgs& a) {
  if (a.f32) return launch_bwd_preprocess_f32(a);
  if (a.bf16) return a.D == 64 ? pre_t<Bf16, 64>(a) : pre_t<Bf16, 128>(a);
  return a.D == 64 ? pre_t<F16, 64>(a) : pre_t<F16, 128>(a);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
  if (a.f32) return launch_bwd_dkdv_f32(a);
  if (a.bf16) return a.D == 64 ? dkdv_hd<Bf16, 64>(a) : dkdv_hd<Bf16, 128>(a);
  return a.D == 64 ? dkdv_hd<F16, 64>(a) : dkdv_hd<F16, 128>(a);
}

hipError_t launch_bwd_dq(const BwdArgs& a) {
  if (a.f32) return launch_bwd_dq_f32(a);
  bool fused = false;
  return a.bf16 ? dq_dt<Bf16>(a, DqMode::kPlain, &fused) : dq_dt<F16>(a, DqMode::kPlain, &fused);
}

hipError_t launch_bwd_dq_post(const BwdArgs& a) {
  if (a.f32) {
    FA_HIP_TRY(launch_bwd_dq_f32(a));
    return launch_bwd_postprocess(a);
  }
  const DqMode m = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D).partial_dkdv ? DqMode::kPost : DqMode::kPlain;
  bool fused = false;
  FA_HIP_TRY(a.bf16 ? dq_dt<Bf16>(a, m, &fused) : dq_dt<F16>(a, m, &fused));
  return fused ? hipSuccess : launch_bwd_postprocess(a);
}

hipError_t launch_bwd_dq_rows(const BwdArgs& a) {
  bool fused = false;
  return a.bf16 ? dq_dt<Bf16>(a, DqMode::kRows, &fused) : dq_dt<F16>(a, DqMode::kRows, &fused);
}

hipError_t launch_bwd_postprocess(const BwdArgs& a) {
  if (a.f32) return hipSuccess;  // the fp32 dK/dV pass writes dk/dv directly
  return a.bf16 ? post_t<Bf16>(a) : post_t<F16>(a);
}

}  // namespace fa
