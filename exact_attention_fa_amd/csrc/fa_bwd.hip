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
// the K and V tiles stay in LDS.  64-query tiles of Q and dO, with the per-row LSE*log2(e)
// and D, stream through a double-buffered LDS by direct global->LDS loads issued one tile
// ahead.  Per query tile, per wave and per 32-query block: S = Q K^T and dP = dO V^T on
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
constexpr int kBwdBKV = 128;  // keys per workgroup (32 per wave)
constexpr int kBwdBQ = 64;    // query rows per streamed tile
constexpr int kDqBR = 128;    // dQ kernel: query rows per workgroup (32 per wave)
constexpr int kDqBC = 64;     // dQ kernel: keys per K/V tile

// ---------------------------------------------------------------- preprocess
// D[row] = sum_d dO[row][d] * O[row][d] (fp32) and L2[row] = LSE[row] * log2(e) (the
// exponent offset of the base-2 recompute of P).
template <typename TR, int HD>
__global__ void __launch_bounds__(kThreads)
bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
               const float* __restrict__ LSE, float* __restrict__ Dl, float* __restrict__ L2, long long rows) {
  constexpr int TPR = HD / 8;          // threads per row, 8 elements each
  constexpr int RPB = kThreads / TPR;  // rows per block
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = ld16(O + row * HD + part * 8);
    const u32x4 d = ld16(dO + row * HD + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(TR::lo(o[w]), TR::lo(d[w]), acc);
      acc = fmaf(TR::hi(o[w]), TR::hi(d[w]), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    Dl[row] = acc;
    L2[row] = LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------- dK, dV
template <typename TR, int HD, bool CAUSAL, bool PARTIAL>
__global__ void __launch_bounds__(kThreads, 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ L2, const float* __restrict__ Dl, uint16_t* __restrict__ dK,
                uint16_t* __restrict__ dV, float* __restrict__ dKp, float* __restrict__ dVp, int Hq, int Hkv,
                int N, int n_kt, float c2, float scale) {
  constexpr int BKV = kBwdBKV, BQ = kBwdBQ;
  constexpr int KST = HD / 16, DB = HD / 32;
  constexpr int KT_BYTES = BKV * HD * 2;
  constexpr int QT_BYTES = BQ * HD * 2;
  constexpr int KI = KT_BYTES / 1024 / 4;   // 1 KB direct loads per wave for the K tile
  constexpr int QI = QT_BYTES / 1024 / 4;   // ... for one Q (or dO) tile
  static_assert(KI * 4096 == KT_BYTES && QI * 4096 == QT_BYTES, "tiles must split into 1 KB loads");

  __shared__ __attribute__((aligned(1024))) char smem[2 * KT_BYTES + 4 * QT_BYTES + 4 * BQ * 4];
  char* const sK = smem;
  char* const sV = sK + KT_BYTES;
  char* const sQ = sV + KT_BYTES;          // two buffers
  char* const sdO = sQ + 2 * QT_BYTES;     // two buffers
  char* const sL = sdO + 2 * QT_BYTES;     // two buffers of BQ floats: LSE * log2(e)
  char* const sD = sL + 2 * BQ * 4;        // two buffers of BQ floats: D

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;

  const int job = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = job % n_kt;  // causal: low kt has the most query tiles and comes first
  const int bh = job / n_kt;
  const int hq = bh % Hq, b = bh / Hq;
  const int hkv = hq / (Hq / Hkv);
  const size_t kvoff = ((size_t)b * Hkv + hkv) * N * HD;
  const uint16_t* const Kh = K + kvoff;
  const uint16_t* const Vh = V + kvoff;
  const uint16_t* const Qh = Q + (size_t)bh * N * HD;
  const uint16_t* const dOh = dO + (size_t)bh * N * HD;
  const float* const L2h = L2 + (size_t)bh * N;
  const float* const Dh = Dl + (size_t)bh * N;

  const int kv0 = kt * BKV;
  const int kw0 = kv0 + wave * 32;  // this wave's first key
  const int key = kw0 + c;          // the key this lane's accumulator column belongs to
  const int n_qt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kv0 / BQ : 0;  // earlier query tiles see none of these keys

  // Direct loads of one 64-query tile of Q, dO, L2 and D into buffer `buf`.  Rows past the
  // end read as zero (their scores are masked).
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
  auto issue = [&](int qt, char* dQt, char* ddO, char* dL, char* dD) {
    const uint32_t q0 = (uint32_t)qt * BQ;
#pragma unroll
    for (int r = 0; r < QI; ++r) {
      const int blk = wave * QI + r;
      dma_to_lds<16>(rQ, qvo[r], q0 * (HD * 2), dQt + blk * 1024);
      dma_to_lds<16>(rdO, qvo[r], q0 * (HD * 2), ddO + blk * 1024);
    }
    if (wave == 0) dma_to_lds<4>(rL, (uint32_t)lane * 4u, q0 * 4u, dL);
    if (wave == 1) dma_to_lds<4>(rD, (uint32_t)lane * 4u, q0 * 4u, dD);
  };

  // K and V tiles -> LDS for the whole kernel (keys past the end read as zero; their scores
  // are masked), then the first query tile.
  {
    const BufRes rK = make_bufres(Kh, rowb), rV = make_bufres(Vh, rowb);
#pragma unroll
    for (int r = 0; r < KI; ++r) {
      const int blk = wave * KI + r;
      int row, col;
      sl_pos_to_rc<BKV>((uint32_t)(blk * 64 + lane), row, col);
      const uint32_t vo = (uint32_t)(row * HD + col) * 2u;
      dma_to_lds<16>(rK, vo, (uint32_t)kv0 * (HD * 2), sK + blk * 1024);
      dma_to_lds<16>(rV, vo, (uint32_t)kv0 * (HD * 2), sV + blk * 1024);
    }
  }
  if (qt0 < n_qt) issue(qt0, sQ, sdO, sL, sD);

  // Per-lane LDS offsets (all reads below add compile-time tile offsets to these).
  const uint32_t poff[2] = {sl_off<64>(c, g * 8), sl_off<64>(c, 16 + g * 8)};                   // row c
  const uint32_t qoff[2] = {sl_off<64>(perm_rows(c), g * 8), sl_off<64>(perm_rows(c), 16 + g * 8)};  // permuted
  const TrLane trl = tr_lane(lane);

  wait_vmcnt<0>();
  lds_barrier();
  // B operands of S = Q K^T and dP = dO V^T for k-step kk: slot j = K/V[key][kk*16 + g*8 + j]

  f32x16 dKa[DB], dVa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dKa[db] = f32x16{};
    dVa[db] = f32x16{};
  }

  // One 64-query tile: recompute S and P, form dP and dS, accumulate dV and dK.  Register i of the accumulators of query block qb is
  // query q0 + qb*32 + (i/8)*16 + g*8 + i%8 (permuted Q/dO rows), key `key`; that order is
  // the k-slot order of the A operands of dV = P^T dO and dK = dS^T Q.  The MASKED body
  // handles the causal diagonal and ragged edges; the other one is straight-line code so the
  // two query blocks' MFMAs and softmax work can be interleaved by the scheduler.
  auto tile = [&](auto masked_tag, const int q0, const char* tQ, const char* tdO, const float* tL,
                  const float* tD, const char* tK, const char* tV) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // ---- S = Q K^T and dP = dO V^T for both query blocks, k-step by k-step
    struct Ops1 {
      u32x4 kf, vf, q[2], o[2];
    };
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    pipelined<KST, 2>(
        [&](int kk) {
          Ops1 f;
          const uint32_t ko = sl_off<BKV>(wave * 32, (kk >> 1) * 32) + poff[kk & 1];
          f.kf = lds_ld128(tK + ko);
          f.vf = lds_ld128(tV + ko);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const uint32_t o = sl_off<BQ>(qb * 32, (kk >> 1) * 32) + qoff[kk & 1];
            f.q[qb] = lds_ld128(tQ + o);
            f.o[qb] = lds_ld128(tdO + o);
          }
          return f;
        },
        [&](int, const Ops1& f) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            s[qb] = TR::mfma(f.q[qb], f.kf, s[qb]);
            dp[qb] = TR::mfma(f.o[qb], f.vf, dp[qb]);
          }
        });

    // ---- P = exp2(S c2 - LSE log2 e), dS = P (dP - D); rounded copies are the A operands of
    //      dV += P^T dO and dK += dS^T Q.
    u32x4 pa[2][2], dsa[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qb0 = q0 + qb * 32;
      if (MASKED) {
        // masked scores become -inf, so exp2 (with c2 > 0) makes them exact zeros
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qb0 + (i >> 3) * 16 + g * 8 + (i & 7);
          if (key >= N || q >= N || (CAUSAL && key > q)) s[qb][i] = -INFINITY;
        }
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int r0 = qb * 32 + t2 * 16 + g * 8;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(tL + r0);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(tL + r0 + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(tD + r0);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(tD + r0 + 4);
        float p[8], ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = t2 * 8 + j;
          const float lse2 = j < 4 ? l0[j] : l1[j - 4];
          const float dd = j < 4 ? d0[j] : d1[j - 4];
          p[j] = fast_exp2(fmaf(s[qb][i], c2, -lse2));
          ds[j] = p[j] * (dp[qb][i] - dd);
        }
        pa[qb][t2] = u32x4{TR::pack(p[0], p[1]), TR::pack(p[2], p[3]), TR::pack(p[4], p[5]), TR::pack(p[6], p[7])};
        dsa[qb][t2] = u32x4{TR::pack(ds[0], ds[1]), TR::pack(ds[2], ds[3]), TR::pack(ds[4], ds[5]),
                            TR::pack(ds[6], ds[7])};
      }
    }

    // ---- dV += P^T dO, dK += dS^T Q; B operands read transposed from the dO / Q tiles
    struct Ops2 {
      u32x4 o, q;
    };
    pipelined<2 * DB * 2, 2>(
        [&](int i) {
          const int qb = i / (2 * DB), db = (i / 2) % DB, t2 = i % 2;
          const uint32_t o = sl_off<BQ>(qb * 32 + t2 * 16, db * 32);
          return Ops2{lds_tr8(tdO + o, trl), lds_tr8(tQ + o, trl)};
        },
        [&](int i, const Ops2& f) {
          const int qb = i / (2 * DB), db = (i / 2) % DB, t2 = i % 2;
          dVa[db] = TR::mfma(pa[qb][t2], f.o, dVa[db]);
          dKa[db] = TR::mfma(dsa[qb][t2], f.q, dKa[db]);
        });
  };

  // One query tile: wait for its loads, prefetch the next, compute.  The LDS buffers are
  // restrict-qualified parameters so that the compiler can tell this tile's reads from the
  // direct loads filling the next tile and does not make them wait.
  auto step = [&](auto masked_tag, const int qt, char* __restrict__ nQ, char* __restrict__ ndO,
                  char* __restrict__ nL, char* __restrict__ nD, const char* __restrict__ tQ,
                  const char* __restrict__ tdO, const char* __restrict__ tL, const char* __restrict__ tD,
                  const char* __restrict__ tK, const char* __restrict__ tV) {
    const int q0 = qt * BQ;
    if (qt > qt0) {
      wait_vmcnt<0>();  // this tile's direct loads (issued one tile ago) have landed
      lds_barrier();    // ... for every wave; every wave is also done with the previous tile
    }
    if (qt + 1 < n_qt) issue(qt + 1, nQ, ndO, nL, nD);
    __builtin_amdgcn_sched_barrier(0);
    tile(masked_tag, q0, tQ, tdO, reinterpret_cast<const float*>(tL), reinterpret_cast<const float*>(tD), tK, tV);
  };

  // Query tiles [qt_a, qt_b) need no mask for any wave of the workgroup (the key tile is
  // whole, the query tile is whole and lies entirely below the diagonal); the others take
  // the masked body.  Three single-body loops keep the accumulators in fixed registers.
  int qt_a = qt0, qt_b = qt0;
  if (kv0 + BKV <= N) {
    qt_a = CAUSAL ? min(n_qt, (kv0 + BKV - 1) / BQ + 1) : qt0;  // first tile with q0 >= kv0 + BKV - 1
    qt_b = max(qt_a, N / BQ);                                   // tiles before the ragged tail
  }
  char* cQ = sQ;
  char* cdO = sdO;
  char* cL = sL;
  char* cD = sD;
  char* nQ = sQ + QT_BYTES;
  char* ndO = sdO + QT_BYTES;
  char* nL = sL + BQ * 4;
  char* nD = sD + BQ * 4;
  auto run = [&](auto masked_tag, int qt) {
    step(masked_tag, qt, nQ, ndO, nL, nD, cQ, cdO, cL, cD, sK, sV);
    char* t;
    t = cQ, cQ = nQ, nQ = t;
    t = cdO, cdO = ndO, ndO = t;
    t = cL, cL = nL, nL = t;
    t = cD, cD = nD, nD = t;
  };
  for (int qt = qt0; qt < qt_a; ++qt) run(std::true_type{}, qt);
  for (int qt = qt_a; qt < qt_b; ++qt) run(std::false_type{}, qt);
  for (int qt = max(qt_a, qt_b); qt < n_qt; ++qt) run(std::true_type{}, qt);

  // ---- epilogue: register i of dKa/dVa[db] <-> key kw0 + (i/4)*8 + g*4 + i%4, column db*32 + c
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr_ = kw0 + (i >> 2) * 8 + g * 4 + (i & 3);
      if (kr_ >= N) continue;
      const int d = db * 32 + c;
      if (PARTIAL) {
        const size_t off = ((size_t)bh * N + kr_) * HD + d;
        dKp[off] = dKa[db][i] * scale;
        dVp[off] = dVa[db][i];
      } else {
        const size_t off = kvoff + (size_t)kr_ * HD + d;
        dK[off] = (uint16_t)(TR::pack(dKa[db][i] * scale, 0.f) & 0xffffu);
        dV[off] = (uint16_t)(TR::pack(dVa[db][i], 0.f) & 0xffffu);
      }
    }
}

// ---------------------------------------------------------------- dQ
// Query-stationary: a workgroup owns 128 query rows (32 per wave) of one head and streams
// the K/V tiles of its KV head through a double-buffered LDS, exactly like the forward.  Per
// 64-key tile, per wave:
//   S^T = K Q^T and dP^T = V dO^T  (K, V rows from LDS; Q and dO fragments in registers)
//   P^T = exp2(S^T c2 - LSE log2 e),  dS^T = P^T * (dP^T - D)      (fp32, one query per lane)
//   dQ^T += K^T dS^T  (K^T read transposed from the K tile; the rounded dS^T registers are
//                      the B operand thanks to the permuted K rows)
// Every dQ element is produced by exactly one lane: no atomics, bitwise deterministic.
template <typename TR, int HD, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2)
bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
              const float* __restrict__ L2, const float* __restrict__ Dl, uint16_t* __restrict__ dQ,
              int Hq, int Hkv, int N, int n_qt, float c2, float scale) {
  constexpr int BR = kDqBR, BC = kDqBC;
  constexpr int KST = HD / 16;              // k-steps over the head dim
  constexpr int DB = HD / 32;               // 32-row blocks of dQ^T
  constexpr int TILE = BC * HD * 2;         // bytes of one K or V tile
  constexpr int TI = TILE / 1024 / 4;       // 1 KB direct loads per wave per tile
  static_assert(TI * 4096 == TILE, "tile must split into 1 KB loads over 4 waves");

  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // K[2], V[2]
  char* const sK = smem;
  char* const sV = smem + 2 * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;

  const int job = xcd_remap(blockIdx.x, gridDim.x);
  int qt = job % n_qt;
  const int bh = job / n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;  // heaviest query tiles first
  const int hq = bh % Hq, b = bh / Hq;
  const int hkv = hq / (Hq / Hkv);
  const uint16_t* const Kh = K + ((size_t)b * Hkv + hkv) * N * HD;
  const uint16_t* const Vh = V + ((size_t)b * Hkv + hkv) * N * HD;

  const int qw0 = qt * BR + wave * 32;  // first query row of this wave
  const int qi = qw0 + c;               // the query of this lane's accumulator column

  int kv_end = (N + BC - 1) / BC;
  if (CAUSAL) kv_end = (min(N, (qt + 1) * BR) - 1) / BC + 1;

  // Direct loads of K/V tile t (keys past the end read as zero; their scores are masked).
  const BufRes rK = make_bufres(Kh, (uint32_t)N * HD * 2u), rV = make_bufres(Vh, (uint32_t)N * HD * 2u);
  uint32_t kvo[TI];
#pragma unroll
  for (int r = 0; r < TI; ++r) {
    int row, col;
    sl_pos_to_rc<BC>((uint32_t)((wave * TI + r) * 64 + lane), row, col);
    kvo[r] = (uint32_t)(row * HD + col) * 2u;
  }
  auto issue = [&](int t, char* dK_, char* dV_) {
#pragma unroll
    for (int r = 0; r < TI; ++r) {
      const int blk = wave * TI + r;
      dma_to_lds<16>(rK, kvo[r], (uint32_t)t * (BC * HD * 2), dK_ + blk * 1024);
      dma_to_lds<16>(rV, kvo[r], (uint32_t)t * (BC * HD * 2), dV_ + blk * 1024);
    }
  };
  issue(0, sK, sV);

  // B operands: slot j of k-step kk = Q[qi][kk*16 + g*8 + j] and dO[qi][...]
  const size_t rowoff = (size_t)bh * N * HD + (size_t)qi * HD;
  u32x4 qf[KST], of[KST];
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) {
    qf[kk] = ld16_if(Q + rowoff + kk * 16 + g * 8, qi < N);
    of[kk] = ld16_if(dO + rowoff + kk * 16 + g * 8, qi < N);
  }
  const float l2 = qi < N ? L2[(size_t)bh * N + qi] : 0.f;
  const float dd = qi < N ? Dl[(size_t)bh * N + qi] : 0.f;

  const uint32_t koff[2] = {sl_off<BC>(perm_rows(c), g * 8), sl_off<BC>(perm_rows(c), 16 + g * 8)};
  const TrLane trl = tr_lane(lane);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  auto step = [&](const int t, char* __restrict__ nK, char* __restrict__ nV, const char* __restrict__ tK,
                  const char* __restrict__ tV) {
    if (t + 1 < kv_end) issue(t + 1, nK, nV);
    const int kv0 = t * BC;
    if (CAUSAL && kv0 > qw0 + 31) return;  // tile lies above the diagonal for this wave

    // ---- S^T = K Q^T, dP^T = V dO^T: register i of block kb is key kv0 + kb*32 + (i/8)*16 + g*8 + i%8
    struct Ops {
      u32x4 k[2], v[2];
    };
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    pipelined<KST, 1>(
        [&](int kk) {
          Ops f;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const uint32_t o = sl_off<BC>(kb * 32, (kk >> 1) * 32) + koff[kk & 1];
            f.k[kb] = lds_ld128(tK + o);
            f.v[kb] = lds_ld128(tV + o);
          }
          return f;
        },
        [&](int kk, const Ops& f) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            s[kb] = TR::mfma(f.k[kb], qf[kk], s[kb]);
            dp[kb] = TR::mfma(f.v[kb], of[kk], dp[kb]);
          }
        });

    if ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0)) {
      // masked scores become -inf, so exp2 (with c2 > 0) makes them exact zeros
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
          if (key >= N || (CAUSAL && key > qi)) s[kb][i] = -INFINITY;
        }
    }

    // ---- dS^T = P^T (dP^T - D), rounded to the B operand of dQ^T += K^T dS^T
    u32x4 dsb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        float ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = t2 * 8 + j;
          ds[j] = fast_exp2(fmaf(s[kb][i], c2, -l2)) * (dp[kb][i] - dd);
        }
        dsb[kb][t2] = u32x4{TR::pack(ds[0], ds[1]), TR::pack(ds[2], ds[3]), TR::pack(ds[4], ds[5]),
                            TR::pack(ds[6], ds[7])};
      }

    // ---- dQ^T += K^T dS^T  (A = K^T: rows d, k = keys, read transposed from the K tile)
    pipelined<DB * 4, 2>(
        [&](int i) {
          const int db = i >> 2, kb = (i >> 1) & 1, t2 = i & 1;
          return lds_tr8(tK + sl_off<BC>(kb * 32 + t2 * 16, db * 32), trl);
        },
        [&](int i, const u32x4& a) {
          const int db = i >> 2, kb = (i >> 1) & 1, t2 = i & 1;
          acc[db] = TR::mfma(a, dsb[kb][t2], acc[db]);
        });
  };

  // Unrolled by two so that each half sees fixed buffers (even tiles in buffer 0).
  for (int t = 0; t < kv_end; t += 2) {
    wait_vmcnt<0>();
    lds_barrier();
    step(t, sK + TILE, sV + TILE, sK, sV);
    if (t + 1 < kv_end) {
      wait_vmcnt<0>();
      lds_barrier();
      step(t + 1, sK, sV, sK + TILE, sV + TILE);
    }
  }

  // ---- epilogue: dQ = scale * acc; register i of acc[db] is column db*32 + (i/4)*8 + g*4 + i%4
  if (qi < N) {
    uint16_t* const drow = dQ + rowoff;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + i4 * 8 + g * 4;
        const u32x2 w = {TR::pack(acc[db][i4 * 4 + 0] * scale, acc[db][i4 * 4 + 1] * scale),
                         TR::pack(acc[db][i4 * 4 + 2] * scale, acc[db][i4 * 4 + 3] * scale)};
        *reinterpret_cast<u32x2*>(drow + d) = w;
      }
  }
}

// ---------------------------------------------------------------- postprocess
// dK/dV of KV head (b, hkv) = sum over its `grp` query heads of the fp32 partials
// (dK partials already carry the softmax scale).
template <typename TR>
__global__ void __launch_bounds__(kThreads)
bwd_post_dkdv_kernel(const float* __restrict__ dKp, const float* __restrict__ dVp,
                     uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int grp,
                     long long head8, long long n8) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n8) return;
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

// ---------------------------------------------------------------- launchers

template <typename TR, int HD>
hipError_t pre_t(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  const long long rows = a.B * a.Hq * a.N;
  constexpr int RPB = kThreads / (HD / 8);
  const long long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_pre_kernel<TR, HD>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout), a.lse,
                     reinterpret_cast<float*>(a.ws + w.delta), reinterpret_cast<float*>(a.ws + w.lse2), rows);
  return hipGetLastError();
}

// c2 must be > 0 so that exp2(-inf * c2) is an exact 0 for masked scores; a zero scale
// becomes 2^-100, for which every exp2 rounds to exactly 1 (uniform weights).
inline float exp2_factor(float scale) { return scale > 0.f ? scale * kLog2e : 0x1p-100f; }

template <typename TR, int HD, bool CAUSAL, bool PARTIAL>
hipError_t dkdv_t(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  const int n_kt = (int)((a.N + kBwdBKV - 1) / kBwdBKV);
  const long long blocks = a.B * a.Hq * (long long)n_kt;
  float* const dkp = PARTIAL ? reinterpret_cast<float*>(a.ws + w.dk_part) : nullptr;
  float* const dvp = PARTIAL ? reinterpret_cast<float*>(a.ws + w.dv_part) : nullptr;
  hipLaunchKernelGGL((bwd_dkdv_kernel<TR, HD, CAUSAL, PARTIAL>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout),
                     reinterpret_cast<const float*>(a.ws + w.lse2), reinterpret_cast<const float*>(a.ws + w.delta),
                     static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), dkp, dvp, (int)a.Hq, (int)a.Hkv,
                     (int)a.N, n_kt, exp2_factor(a.scale), a.scale);
  return hipGetLastError();
}

template <typename TR, int HD>
hipError_t dkdv_hd(const BwdArgs& a) {
  const bool partial = a.Hq != a.Hkv;
  if (a.causal) return partial ? dkdv_t<TR, HD, true, true>(a) : dkdv_t<TR, HD, true, false>(a);
  return partial ? dkdv_t<TR, HD, false, true>(a) : dkdv_t<TR, HD, false, false>(a);
}

template <typename TR, int HD, bool CAUSAL>
hipError_t dq_t(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  const int n_qt = (int)((a.N + kDqBR - 1) / kDqBR);
  const long long blocks = a.B * a.Hq * (long long)n_qt;
  hipLaunchKernelGGL((bwd_dq_kernel<TR, HD, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout),
                     reinterpret_cast<const float*>(a.ws + w.lse2), reinterpret_cast<const float*>(a.ws + w.delta),
                     static_cast<uint16_t*>(a.dq), (int)a.Hq, (int)a.Hkv, (int)a.N, n_qt, exp2_factor(a.scale),
                     a.scale);
  return hipGetLastError();
}

template <typename TR>
hipError_t dq_dt(const BwdArgs& a) {
  if (a.D == 64) return a.causal ? dq_t<TR, 64, true>(a) : dq_t<TR, 64, false>(a);
  return a.causal ? dq_t<TR, 128, true>(a) : dq_t<TR, 128, false>(a);
}

template <typename TR>
hipError_t post_t(const BwdArgs& a) {
  if (a.Hq == a.Hkv) return hipSuccess;  // dK and dV were written directly
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  const long long kv8 = a.B * a.Hkv * a.N * a.D / 8;
  hipLaunchKernelGGL((bwd_post_dkdv_kernel<TR>), dim3((unsigned)((kv8 + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, a.stream, reinterpret_cast<const float*>(a.ws + w.dk_part),
                     reinterpret_cast<const float*>(a.ws + w.dv_part), static_cast<uint16_t*>(a.dk),
                     static_cast<uint16_t*>(a.dv), (int)(a.Hq / a.Hkv), a.N * a.D / 8, kv8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const BwdArgs& a) {
  if (a.bf16) return a.D == 64 ? pre_t<Bf16, 64>(a) : pre_t<Bf16, 128>(a);
  return a.D == 64 ? pre_t<F16, 64>(a) : pre_t<F16, 128>(a);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a) {
  if (a.bf16) return a.D == 64 ? dkdv_hd<Bf16, 64>(a) : dkdv_hd<Bf16, 128>(a);
  return a.D == 64 ? dkdv_hd<F16, 64>(a) : dkdv_hd<F16, 128>(a);
}

hipError_t launch_bwd_dq(const BwdArgs& a) { return a.bf16 ? dq_dt<Bf16>(a) : dq_dt<F16>(a); }

hipError_t launch_bwd_postprocess(const BwdArgs& a) {
  return a.bf16 ? post_t<Bf16>(a) : post_t<F16>(a);
}

}  // namespace fa
