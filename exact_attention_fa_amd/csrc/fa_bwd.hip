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
// query head, a wave owns 32 of them.  K and V of those keys stay in registers (and K
// also in LDS), and 64-query tiles of Q and dO stream through LDS, prefetched one tile
// ahead.  Per query tile, per wave:
//   S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16 with the key as the accumulator
//   column, so each lane owns one key; register 8t+j of a 32-query block is query
//   16t + 8g + j (row permutation of the Q/dO operand).  That register order is exactly
//   the k-slot order of the A operand of dV = P^T dO and dK = dS^T Q, so P and dS feed
//   those MFMAs from registers; the dO and Q B operands come through ds_read_b64_tr_b16.
//   dS^T is written to LDS once; after a barrier the four waves split dQ += dS K of the
//   tile (both operands read transposed) and add it to the fp32 accumulator atomically.
// Grouped-query attention: the grid runs over query heads; when Hq > Hkv each workgroup
// writes fp32 per-query-head dK/dV partials that the postprocess sums over the group
// (deterministic), otherwise it writes dK/dV directly.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBwdBKV = 128;  // keys per workgroup (32 per wave)
constexpr int kBwdBQ = 64;    // query rows per streamed tile

// ---------------------------------------------------------------- preprocess
// D[row] = sum_d dO[row][d] * O[row][d] (fp32) and dQacc[row][:] = 0.
template <typename TR, int HD>
__global__ void __launch_bounds__(kThreads)
bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
               float* __restrict__ Dl, float* __restrict__ dQacc, long long rows) {
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
  if (row < rows && part == 0) Dl[row] = acc;
}

// ---------------------------------------------------------------- main
template <typename TR, int HD, bool CAUSAL, bool PARTIAL>
__global__ void __launch_bounds__(kThreads, 1)
bwd_main_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ LSE, const float* __restrict__ Dl,
                float* __restrict__ dQacc, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                float* __restrict__ dKp, float* __restrict__ dVp, int Hq, int Hkv, int N, int n_kt,
                float c2, float scale) {
  constexpr int BKV = kBwdBKV, BQ = kBwdBQ;
  constexpr int KST = HD / 16, DB = HD / 32;
  constexpr int CPR = HD / 8;                 // 16-byte chunks per row
  constexpr int KCH = BKV * CPR / kThreads;   // K-tile chunks per thread
  constexpr int QCH = BQ * CPR / kThreads;    // Q/dO-tile chunks per thread
  constexpr int KT_BYTES = BKV * HD * 2;
  constexpr int QT_BYTES = BQ * HD * 2;
  constexpr int ST_BYTES = BKV * BQ * 2;
  static_assert(KCH * kThreads == BKV * CPR && QCH * kThreads == BQ * CPR, "uneven tile split");

  __shared__ __attribute__((aligned(1024))) char smem[KT_BYTES + 2 * QT_BYTES + ST_BYTES + 2 * BQ * 4];
  char* const sK = smem;
  char* const sQ = sK + KT_BYTES;
  char* const sdO = sQ + QT_BYTES;
  char* const sdS = sdO + QT_BYTES;  // dS^T: rows = the workgroup's keys, columns = queries
  float* const sL = reinterpret_cast<float*>(sdS + ST_BYTES);  // LSE * log2(e)
  float* const sD = sL + BQ;                                     // D

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  const float* const LSEh = LSE + (size_t)bh * N;
  const float* const Dh = Dl + (size_t)bh * N;
  float* const dQh = dQacc + (size_t)bh * N * HD;

  const int kv0 = kt * BKV;
  const int kw0 = kv0 + wave * 32;  // this wave's first key
  const int key = kw0 + c;          // the key this lane's accumulator column belongs to

  // K tile -> LDS (read transposed by dQ += dS K); V straight into registers.
#pragma unroll
  for (int r = 0; r < KCH; ++r) {
    const int cid = tid + kThreads * r;
    const int row = cid / CPR, ch = cid % CPR;
    lds_write8<HD>(sK, row, ch * 8, ld16_if(Kh + (size_t)(kv0 + row) * HD + ch * 8, kv0 + row < N));
  }
  u32x4 vr[KST];  // B operand of dP = dO V^T: slot j of k-step kk = V[key][kk*16 + g*8 + j]
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) vr[kk] = ld16_if(Vh + (size_t)key * HD + kk * 16 + g * 8, key < N);
  __syncthreads();
  u32x4 kr[KST];  // B operand of S = Q K^T
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) kr[kk] = lds_read8<HD>(sK, wave * 32 + c, kk * 16 + g * 8);

  f32x16 dKa[DB], dVa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dKa[db] = f32x16{};
    dVa[db] = f32x16{};
  }

  const int n_qt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kv0 / BQ : 0;  // earlier query tiles see none of these keys

  u32x4 qreg[QCH], oreg[QCH];
  float lreg = 0.f;
  auto gload = [&](int qt) {
    const int q0 = qt * BQ;
#pragma unroll
    for (int r = 0; r < QCH; ++r) {
      const int cid = tid + kThreads * r;
      const int row = cid / CPR, ch = cid % CPR;
      const int q = q0 + row;
      qreg[r] = ld16_if(Qh + (size_t)q * HD + ch * 8, q < N);
      oreg[r] = ld16_if(dOh + (size_t)q * HD + ch * 8, q < N);
    }
    if (tid < BQ) {
      const int q = q0 + tid;
      lreg = q < N ? LSEh[q] * kLog2e : 0.f;
    } else if (tid < 2 * BQ) {
      const int q = q0 + tid - BQ;
      lreg = q < N ? Dh[q] : 0.f;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int r = 0; r < QCH; ++r) {
      const int cid = tid + kThreads * r;
      const int row = cid / CPR, ch = cid % CPR;
      lds_write8<HD>(sQ, row, ch * 8, qreg[r]);
      lds_write8<HD>(sdO, row, ch * 8, oreg[r]);
    }
    if (tid < BQ) sL[tid] = lreg;
    else if (tid < 2 * BQ) sD[tid - BQ] = lreg;
  };

  // Recompute P and form dS for the 64-query tile in LDS; register i of query block qb
  // <-> query q0 + qb*32 + (i/8)*16 + g*8 + i%8, key `key`.  P and dS come back rounded
  // to the input type as A operands (k-slot j of (qb, t2) = query q0 + qb*32 + t2*16 + g*8
  // + j), and dS^T is also written to LDS for the dQ product.
  auto p_ds = [&](const bool masked, const int q0, u32x4 (&pa)[2][2], u32x4 (&dsa)[2][2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KST; ++kk)
        s = TR::mfma(lds_read8<HD>(sQ, qb * 32 + perm_rows(c), kk * 16 + g * 8), kr[kk], s);
#pragma unroll
      for (int kk = 0; kk < KST; ++kk)
        dp = TR::mfma(lds_read8<HD>(sdO, qb * 32 + perm_rows(c), kk * 16 + g * 8), vr[kk], dp);
      // masked scores become -inf, so exp2 (with c2 > 0) makes them exact zeros
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = q0 + qb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
          if (key >= N || q >= N || (CAUSAL && key > q)) s[i] = -INFINITY;
        }
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int r0 = qb * 32 + t2 * 16 + g * 8;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(sL + r0);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(sL + r0 + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(sD + r0);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(sD + r0 + 4);
        float p[8], ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = t2 * 8 + j;
          const float lse2 = j < 4 ? l0[j] : l1[j - 4];
          const float dd = j < 4 ? d0[j] : d1[j - 4];
          const float pv = fast_exp2(fmaf(s[i], c2, -lse2));
          p[j] = pv;
          ds[j] = pv * (dp[i] - dd);
        }
        pa[qb][t2] = u32x4{TR::pack(p[0], p[1]), TR::pack(p[2], p[3]), TR::pack(p[4], p[5]),
                           TR::pack(p[6], p[7])};
        dsa[qb][t2] = u32x4{TR::pack(ds[0], ds[1]), TR::pack(ds[2], ds[3]), TR::pack(ds[4], ds[5]),
                            TR::pack(ds[6], ds[7])};
        lds_write8<BQ>(sdS, wave * 32 + c, r0, dsa[qb][t2]);
      }
    }
  };

  if (qt0 < n_qt) gload(qt0);
  for (int qt = qt0; qt < n_qt; ++qt) {
    const int q0 = qt * BQ;
    __syncthreads();  // previous tile's LDS reads are finished
    lstore();
    __syncthreads();
    if (qt + 1 < n_qt) gload(qt + 1);

    // Masks only on the tiles that cross the diagonal or a ragged edge; the common case is
    // compiled without any mask code.
    u32x4 pa[2][2], dsa[2][2];
    p_ds((kw0 + 32 > N) || (q0 + BQ > N) || (CAUSAL && q0 < kw0 + 31), q0, pa, dsa);

    // ---- dV += P^T dO and dK += dS^T Q (the rounded P / dS registers are the A operands)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const u32x4 bo = lds_read_tr8<HD>(sdO, qb * 32 + t2 * 16, db * 32, lane);
          dVa[db] = TR::mfma(pa[qb][t2], bo, dVa[db]);
          const u32x4 bq = lds_read_tr8<HD>(sQ, qb * 32 + t2 * 16, db * 32, lane);
          dKa[db] = TR::mfma(dsa[qb][t2], bq, dKa[db]);
        }

    __syncthreads();  // dS^T of all four waves is in LDS

    // ---- dQ[q0 .. q0+63] += dS K: wave -> 32 queries x HD/2 columns
    {
      const int qb = wave & 1;
#pragma unroll
      for (int dbi = 0; dbi < DB / 2; ++dbi) {
        const int db = (wave >> 1) * (DB / 2) + dbi;
        f32x16 dq = f32x16{};
#pragma unroll
        for (int ks = 0; ks < BKV / 16; ++ks) {
          const u32x4 a = lds_read_tr8<BQ>(sdS, ks * 16, qb * 32, lane);
          const u32x4 bk = lds_read_tr8<HD>(sK, ks * 16, db * 32, lane);
          dq = TR::mfma(a, bk, dq);
        }
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
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout),
                     reinterpret_cast<float*>(a.ws + w.delta), reinterpret_cast<float*>(a.ws + w.dq_acc), rows);
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
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout), a.lse,
                     reinterpret_cast<const float*>(a.ws + w.delta), reinterpret_cast<float*>(a.ws + w.dq_acc),
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
