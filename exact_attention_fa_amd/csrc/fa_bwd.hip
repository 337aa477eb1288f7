// Fused exact attention backward for gfx950: preprocess, main, postprocess.
//
// The method: P is recomputed from the saved log-sum-exp, then
//   dV = P^T dO, dP = dO V^T, dS = P * (dP - D), dK = scale * dS^T Q, dQ = scale * dS K
// with D = rowsum(dO * O).  The score-gradient step is a cancellation, so dP and dS stay
// in fp32 and only the MFMA operands are rounded to the input type ("FlashAttention for
// Tesla P100", section "Documentation": the choice of precision is made per product).
// The page's backward also reads dQ through atomics by default, with a no-atomic variant
// ("Layout" table); this file uses fp32 atomics into a workspace accumulator.
//
// gfx950 realisation of the main kernel: a workgroup (4 waves) owns 128 keys of one
// query head, a wave owns 32 of them.  K and V fragments of those keys stay in registers
// (and the K tile also in LDS).  64-query tiles of Q and dO, with the per-row LSE*log2(e)
// and D, stream through double-buffered LDS by direct global->LDS loads issued one tile
// ahead, so no registers are spent on staging.  Per query tile, per wave and per 32-query
// block:
//   S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16 with the key as the accumulator
//   column, so each lane owns one key; register 8t+j of the block is query 16t + 8g + j
//   (row permutation of the Q/dO operand).  That register order is exactly the k-slot
//   order of the A operand of dV += P^T dO and dK += dS^T Q, so the rounded P and dS feed
//   those MFMAs from registers; the dO and Q B operands come through ds_read_b64_tr_b16.
//   dS^T is written to LDS; after a barrier the four waves split dQ += dS K of the tile
//   (both operands read transposed) and add it into the fp32 accumulator with hardware
//   float atomics.  Barriers wait for LDS traffic only, so the atomics stay in flight.
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

// ---------------------------------------------------------------- preprocess
// D[row] = sum_d dO[row][d] * O[row][d] (fp32), L2[row] = LSE[row] * log2(e) (the exponent
// offset of the base-2 recompute of P) and dQacc[row][:] = 0.
template <typename TR, int HD>
__global__ void __launch_bounds__(kThreads)
bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
               const float* __restrict__ LSE, float* __restrict__ Dl, float* __restrict__ L2,
               float* __restrict__ dQacc, long long rows) {
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
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(dQacc + row * HD + part * 8) = z;
    *reinterpret_cast<f32x4*>(dQacc + row * HD + part * 8 + 4) = z;
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    Dl[row] = acc;
    L2[row] = LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------- main
template <typename TR, int HD, bool CAUSAL, bool PARTIAL>
__global__ void __launch_bounds__(kThreads, 1)
bwd_main_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ L2, const float* __restrict__ Dl,
                float* __restrict__ dQacc, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                float* __restrict__ dKp, float* __restrict__ dVp, int Hq, int Hkv, int N, int n_kt,
                float c2, float scale) {
  constexpr int BKV = kBwdBKV, BQ = kBwdBQ;
  constexpr int KST = HD / 16, DB = HD / 32;
  constexpr int KT_BYTES = BKV * HD * 2;
  constexpr int QT_BYTES = BQ * HD * 2;
  constexpr int ST_BYTES = BKV * BQ * 2;
  constexpr int KI = KT_BYTES / 1024 / 4;   // 1 KB direct loads per wave for the K tile
  constexpr int QI = QT_BYTES / 1024 / 4;   // ... for one Q (or dO) tile
  constexpr int NATOM = (DB / 2) * 16;      // dQ atomics a wave issues per query tile
  static_assert(KI * 4096 == KT_BYTES && QI * 4096 == QT_BYTES, "tiles must split into 1 KB loads");

  __shared__ __attribute__((aligned(1024))) char smem[KT_BYTES + 4 * QT_BYTES + ST_BYTES + 4 * BQ * 4];
  char* const sK = smem;
  char* const sQ = sK + KT_BYTES;          // two buffers
  char* const sdO = sQ + 2 * QT_BYTES;     // two buffers
  char* const sdS = sdO + 2 * QT_BYTES;    // dS^T: rows = the workgroup's keys, columns = queries
  char* const sL = sdS + ST_BYTES;         // two buffers of BQ floats: LSE * log2(e)
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
  float* const dQh = dQacc + (size_t)bh * N * HD;

  const int kv0 = kt * BKV;
  const int kw0 = kv0 + wave * 32;  // this wave's first key
  const int key = kw0 + c;          // the key this lane's accumulator column belongs to
  const int n_qt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kv0 / BQ : 0;  // earlier query tiles see none of these keys

  // Direct loads of one 64-query tile of Q, dO, L2 and D into buffer `buf`.  Rows past the
  // end read row N-1 (finite data that the masks then zero out).
  auto issue = [&](int qt, int buf) {
    const int q0 = qt * BQ;
#pragma unroll
    for (int r = 0; r < QI; ++r) {
      const int blk = wave * QI + r;
      int row, col;
      sl_pos_to_rc<BQ>((uint32_t)(blk * 64 + lane), row, col);
      const size_t src = (size_t)min(q0 + row, N - 1) * HD + col;
      dma_to_lds<16>(Qh + src, sQ + buf * QT_BYTES + blk * 1024);
      dma_to_lds<16>(dOh + src, sdO + buf * QT_BYTES + blk * 1024);
    }
    if (wave == 0) dma_to_lds<4>(L2h + min(q0 + lane, N - 1), sL + buf * BQ * 4);
    if (wave == 1) dma_to_lds<4>(Dh + min(q0 + lane, N - 1), sD + buf * BQ * 4);
  };

  // K tile -> LDS (for dQ += dS K) and the first query tile; V fragments straight into
  // registers (B operand of dP = dO V^T: slot j of k-step kk = V[key][kk*16 + g*8 + j]).
#pragma unroll
  for (int r = 0; r < KI; ++r) {
    const int blk = wave * KI + r;
    int row, col;
    sl_pos_to_rc<BKV>((uint32_t)(blk * 64 + lane), row, col);
    dma_to_lds<16>(Kh + (size_t)min(kv0 + row, N - 1) * HD + col, sK + blk * 1024);
  }
  if (qt0 < n_qt) issue(qt0, 0);
  u32x4 vr[KST];
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) vr[kk] = ld16_if(Vh + (size_t)key * HD + kk * 16 + g * 8, key < N);

  // Per-lane LDS offsets (all reads below add compile-time tile offsets to these).
  const uint32_t poff[2] = {sl_off<64>(c, g * 8), sl_off<64>(c, 16 + g * 8)};                   // row c
  const uint32_t qoff[2] = {sl_off<64>(perm_rows(c), g * 8), sl_off<64>(perm_rows(c), 16 + g * 8)};  // permuted
  const TrLane trl = tr_lane(lane);

  wait_vmcnt<0>();
  lds_barrier();
  u32x4 kr[KST];  // B operand of S = Q K^T
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) kr[kk] = lds_ld128(sK + sl_off<BKV>(wave * 32, (kk >> 1) * 32) + poff[kk & 1]);

  f32x16 dKa[DB], dVa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dKa[db] = f32x16{};
    dVa[db] = f32x16{};
  }

  // One 64-query tile: recompute S and P, form dP and dS, accumulate dV and dK, and leave
  // dS^T in LDS for the dQ product.  Register i of the accumulators of query block qb is
  // query q0 + qb*32 + (i/8)*16 + g*8 + i%8 (permuted Q/dO rows), key `key`; that order is
  // the k-slot order of the A operands of dV = P^T dO and dK = dS^T Q.  The MASKED body
  // handles the causal diagonal and ragged edges; the other one is straight-line code so the
  // two query blocks' MFMAs and softmax work can be interleaved by the scheduler.
  auto tile = [&](auto masked_tag, const int q0, const char* tQ, const char* tdO, const float* tL,
                  const float* tD) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
      if (MASKED && CAUSAL && q0 + qb * 32 + 31 < kw0) continue;  // all above the diagonal
#pragma unroll
      for (int kk = 0; kk < KST; ++kk)
        s[qb] = TR::mfma(lds_ld128(tQ + sl_off<BQ>(qb * 32, (kk >> 1) * 32) + qoff[kk & 1]), kr[kk], s[qb]);
#pragma unroll
      for (int kk = 0; kk < KST; ++kk)
        dp[qb] = TR::mfma(lds_ld128(tdO + sl_off<BQ>(qb * 32, (kk >> 1) * 32) + qoff[kk & 1]), vr[kk], dp[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qb0 = q0 + qb * 32;
      char* const dsrow = sdS + sl_off<BKV>(wave * 32, qb * 32);
      if (MASKED && CAUSAL && qb0 + 31 < kw0) {
        // every key of this wave lies above the diagonal for these 32 queries: dS = 0
        const u32x4 z = {0u, 0u, 0u, 0u};
        lds_st128(dsrow + poff[0], z);
        lds_st128(dsrow + poff[1], z);
        continue;
      }
      if (MASKED) {
        // masked scores become -inf, so exp2 (with c2 > 0) makes them exact zeros
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qb0 + (i >> 3) * 16 + g * 8 + (i & 7);
          if (key >= N || q >= N || (CAUSAL && key > q)) s[qb][i] = -INFINITY;
        }
      }
      u32x4 pa[2], dsa[2];
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
        pa[t2] = u32x4{TR::pack(p[0], p[1]), TR::pack(p[2], p[3]), TR::pack(p[4], p[5]), TR::pack(p[6], p[7])};
        dsa[t2] = u32x4{TR::pack(ds[0], ds[1]), TR::pack(ds[2], ds[3]), TR::pack(ds[4], ds[5]),
                        TR::pack(ds[6], ds[7])};
        lds_st128(dsrow + poff[t2], dsa[t2]);
      }
      // dV += P^T dO, dK += dS^T Q (the rounded P / dS registers are the A operands)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          dVa[db] = TR::mfma(pa[t2], lds_tr8(tdO + sl_off<BQ>(qb * 32 + t2 * 16, db * 32), trl), dVa[db]);
          dKa[db] = TR::mfma(dsa[t2], lds_tr8(tQ + sl_off<BQ>(qb * 32 + t2 * 16, db * 32), trl), dKa[db]);
        }
    }
  };

  for (int qt = qt0; qt < n_qt; ++qt) {
    const int q0 = qt * BQ;
    const int buf = (qt - qt0) & 1;
    if (qt > qt0) {
      // This tile's direct loads were issued before the previous tile's NATOM atomics;
      // vector-memory operations retire in order, so this waits for the loads only.
      wait_vmcnt<NATOM>();
      lds_barrier();
    }
    if (qt + 1 < n_qt) issue(qt + 1, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    const char* const tQ = sQ + buf * QT_BYTES;
    const char* const tdO = sdO + buf * QT_BYTES;
    const float* const tL = reinterpret_cast<const float*>(sL + buf * BQ * 4);
    const float* const tD = reinterpret_cast<const float*>(sD + buf * BQ * 4);
    if ((kw0 + 32 > N) || (q0 + BQ > N) || (CAUSAL && q0 < kw0 + 31))
      tile(std::true_type{}, q0, tQ, tdO, tL, tD);
    else
      tile(std::false_type{}, q0, tQ, tdO, tL, tD);

    lds_barrier();  // dS^T of all four waves is in LDS

    // dQ[q0 .. q0+63] += dS K: wave -> 32 queries x HD/2 columns
    {
      const int qb = wave & 1;
#pragma unroll
      for (int dbi = 0; dbi < DB / 2; ++dbi) {
        const int db = (wave >> 1) * (DB / 2) + dbi;
        f32x16 dq = f32x16{};
#pragma unroll
        for (int ks = 0; ks < BKV / 16; ++ks)
          dq = TR::mfma(lds_tr8(sdS + sl_off<BKV>(ks * 16, qb * 32), trl),
                        lds_tr8(sK + sl_off<BKV>(ks * 16, db * 32), trl), dq);
        float* const dst = dQh + (size_t)(q0 + qb * 32 + g * 4) * HD + db * 32 + c;
        if (q0 + BQ <= N) {
#pragma unroll
          for (int i = 0; i < 16; ++i) unsafeAtomicAdd(dst + ((i >> 2) * 8 + (i & 3)) * HD, dq[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int q = q0 + qb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
            if (q < N) unsafeAtomicAdd(dst + ((i >> 2) * 8 + (i & 3)) * HD, dq[i]);
          }
        }
      }
    }
  }

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

// ---------------------------------------------------------------- postprocess
// dQ = dtype(scale * dQacc), 8 elements per thread.
template <typename TR>
__global__ void __launch_bounds__(kThreads)
bwd_post_dq_kernel(const float* __restrict__ dQacc, uint16_t* __restrict__ dQ, long long n8, float scale) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *reinterpret_cast<const f32x4*>(dQacc + i * 8);
  const f32x4 b = *reinterpret_cast<const f32x4*>(dQacc + i * 8 + 4);
  const u32x4 w = {TR::pack(a[0] * scale, a[1] * scale), TR::pack(a[2] * scale, a[3] * scale),
                   TR::pack(b[0] * scale, b[1] * scale), TR::pack(b[2] * scale, b[3] * scale)};
  *reinterpret_cast<u32x4*>(dQ + i * 8) = w;
}

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
                     reinterpret_cast<float*>(a.ws + w.delta), reinterpret_cast<float*>(a.ws + w.lse2),
                     reinterpret_cast<float*>(a.ws + w.dq_acc), rows);
  return hipGetLastError();
}

template <typename TR, int HD, bool CAUSAL, bool PARTIAL>
hipError_t main_t(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  const int n_kt = (int)((a.N + kBwdBKV - 1) / kBwdBKV);
  const long long blocks = a.B * a.Hq * (long long)n_kt;
  float* const dkp = PARTIAL ? reinterpret_cast<float*>(a.ws + w.dk_part) : nullptr;
  float* const dvp = PARTIAL ? reinterpret_cast<float*>(a.ws + w.dv_part) : nullptr;
  hipLaunchKernelGGL((bwd_main_kernel<TR, HD, CAUSAL, PARTIAL>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     a.stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout),
                     reinterpret_cast<const float*>(a.ws + w.lse2), reinterpret_cast<const float*>(a.ws + w.delta),
                     reinterpret_cast<float*>(a.ws + w.dq_acc),
                     static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), dkp, dvp, (int)a.Hq,
                     (int)a.Hkv, (int)a.N, n_kt, a.scale > 0.f ? a.scale * kLog2e : 0x1p-100f, a.scale);
  return hipGetLastError();
}

template <typename TR>
hipError_t post_t(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  const long long n8 = a.B * a.Hq * a.N * a.D / 8;
  hipLaunchKernelGGL((bwd_post_dq_kernel<TR>), dim3((unsigned)((n8 + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     a.stream, reinterpret_cast<const float*>(a.ws + w.dq_acc), static_cast<uint16_t*>(a.dq), n8,
                     a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.Hq == a.Hkv) return e;
  const long long kv8 = a.B * a.Hkv * a.N * a.D / 8;
  hipLaunchKernelGGL((bwd_post_dkdv_kernel<TR>), dim3((unsigned)((kv8 + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, a.stream, reinterpret_cast<const float*>(a.ws + w.dk_part),
                     reinterpret_cast<const float*>(a.ws + w.dv_part), static_cast<uint16_t*>(a.dk),
                     static_cast<uint16_t*>(a.dv), (int)(a.Hq / a.Hkv), a.N * a.D / 8, kv8);
  return hipGetLastError();
}

template <typename TR, int HD>
hipError_t main_hd(const BwdArgs& a) {
  const bool partial = a.Hq != a.Hkv;
  if (a.causal) return partial ? main_t<TR, HD, true, true>(a) : main_t<TR, HD, true, false>(a);
  return partial ? main_t<TR, HD, false, true>(a) : main_t<TR, HD, false, false>(a);
}

}  // namespace

hipError_t launch_bwd_preprocess(const BwdArgs& a) {
  if (a.bf16) return a.D == 64 ? pre_t<Bf16, 64>(a) : pre_t<Bf16, 128>(a);
  return a.D == 64 ? pre_t<F16, 64>(a) : pre_t<F16, 128>(a);
}

hipError_t launch_bwd_main(const BwdArgs& a) {
  if (a.bf16) return a.D == 64 ? main_hd<Bf16, 64>(a) : main_hd<Bf16, 128>(a);
  return a.D == 64 ? main_hd<F16, 64>(a) : main_hd<F16, 128>(a);
}

hipError_t launch_bwd_postprocess(const BwdArgs& a) {
  return a.bf16 ? post_t<Bf16>(a) : post_t<F16>(a);
}

}  // namespace fa
