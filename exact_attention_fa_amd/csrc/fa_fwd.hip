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
//   * 256 threads = 4 waves; a wave owns 32 query rows (BR = 128 rows per workgroup).
//   * K/V tiles of BC = 64 keys are copied global -> LDS by direct loads into a double
//     buffer, one tile ahead of the compute, with no register staging.
//   * Scores are formed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16: each lane then
//     owns one query column, its row max and row sum are in-lane reductions plus one
//     v_permlane32_swap, and the bf16/fp16-rounded probabilities in registers are already
//     the B operand of O^T += V^T P^T.  V^T comes from the row-major V tile through
//     ds_read_b64_tr_b16.
//   * exp2 on the VALU with scale*log2(e) folded into one FMA per score; the running max
//     is moved (and O, l rescaled) only when it grows by more than 2^8.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kFwdBR = 128;  // query rows per workgroup
constexpr int kFwdBC = 64;   // keys per K/V tile
constexpr int kThreads = 256;
constexpr float kRescaleLog2 = 8.f;  // lazy-rescale threshold (log2 of the largest probability)

template <typename TR, int HD, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2)
fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
           const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
           int Hq, int Hkv, int N, int n_qt, float c2, float scale) {
  constexpr int BR = kFwdBR, BC = kFwdBC;
  constexpr int KST = HD / 16;              // k-steps of S^T over the head dim
  constexpr int DB = HD / 32;               // 32-row blocks of O^T
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
  const uint16_t* const Qh = Q + (size_t)bh * N * HD;
  const uint16_t* const Kh = K + ((size_t)b * Hkv + hkv) * N * HD;
  const uint16_t* const Vh = V + ((size_t)b * Hkv + hkv) * N * HD;

  const int qw0 = qt * BR + wave * 32;  // first query row of this wave
  const int qi = qw0 + c;               // the query row this lane's column belongs to

  int kv_end = (N + BC - 1) / BC;
  if (CAUSAL) kv_end = (min(N, (qt + 1) * BR) - 1) / BC + 1;

  // Direct loads of K/V tile t into buffer `buf`; keys past the end read key N-1 (finite
  // data that the masks then exclude).
  auto issue = [&](int t, char* dK, char* dV) {
#pragma unroll
    for (int r = 0; r < TI; ++r) {
      const int blk = wave * TI + r;
      int row, col;
      sl_pos_to_rc<BC>((uint32_t)(blk * 64 + lane), row, col);
      const size_t src = (size_t)min(t * BC + row, N - 1) * HD + col;
      dma_to_lds<16>(Kh + src, dK + blk * 1024);
      dma_to_lds<16>(Vh + src, dV + blk * 1024);
    }
  };
  issue(0, sK, sV);

  // Q fragments: B operand of S^T = K Q^T (slot j of k-step kk = Q[qi][kk*16 + g*8 + j]).
  u32x4 qf[KST];
#pragma unroll
  for (int kk = 0; kk < KST; ++kk) qf[kk] = ld16_if(Qh + (size_t)qi * HD + kk * 16 + g * 8, qi < N);

  // Per-lane LDS offsets.  K rows are read in the permuted order, so register i of an S^T
  // block is key (i/8)*16 + g*8 + i%8; one offset per k-step parity.
  const uint32_t koff[2] = {sl_off<BC>(perm_rows(c), g * 8), sl_off<BC>(perm_rows(c), 16 + g * 8)};
  const TrLane trl = tr_lane(lane);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;  // running (reference) max of raw scores for query qi
  float l_run = 0.f;        // this lane's share of the running sum of 2^((s - m) * c2)

  // One K/V tile.  The LDS buffers are restrict-qualified parameters so that the compiler
  // can tell the reads of tile t from the direct loads filling tile t+1 and does not make
  // the reads wait for those loads.
  auto step = [&](const int t, char* __restrict__ nK, char* __restrict__ nV, const char* __restrict__ tK,
                  const char* __restrict__ tV) {
    if (t + 1 < kv_end) issue(t + 1, nK, nV);

    const int kv0 = t * BC;
    if (CAUSAL && kv0 > qw0 + 31) return;  // tile lies above the diagonal for this wave

    // ---- S^T = K Q^T: register i of block kb holds key kv0 + kb*32 + (i/8)*16 + g*8 + i%8
    f32x16 s[2] = {f32x16{}, f32x16{}};
    pipelined<KST, 2>(
        [&](int kk) {
          struct {
            u32x4 k[2];
          } f;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) f.k[kb] = lds_ld128(tK + sl_off<BC>(kb * 32, (kk >> 1) * 32) + koff[kk & 1]);
          return f;
        },
        [&](int kk, const auto& f) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) s[kb] = TR::mfma(f.k[kb], qf[kk], s[kb]);
        });

    // ---- masks only on the ragged last tile and tiles crossing the diagonal (a uniform
    //      branch): masked scores become -inf, so exp2 (with c2 > 0) makes exact zeros.
    if ((kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
          if (key >= N || (CAUSAL && key > qi)) s[kb][i] = -INFINITY;
        }
    }

    // ---- online softmax in raw-score units (c2 = scale * log2(e) > 0).  The reference max
    //      moves only when the tile max exceeds it by more than 2^kRescaleLog2 in the exp2
    //      domain (always on the first tile); otherwise probabilities up to 2^kRescaleLog2
    //      accumulate against the stale reference, exact because O and l share it.
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx);  // finite: key 0 of tile 0 is visible to every row
    const bool grow = (m_run == -INFINITY) || ((m_new - m_run) * c2 > kRescaleLog2);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * c2);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float mb = m_run * c2;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[kb][i], c2, -mb));
        s[kb][i] = p;
        rs += p;
      }
    l_run += rs;

    // ---- P^T operands: slot j of (kb, t2) = P for key kv0 + kb*32 + t2*16 + g*8 + j
    u32x4 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int i0 = t2 * 8;
        pb[kb][t2] = u32x4{TR::pack(s[kb][i0 + 0], s[kb][i0 + 1]), TR::pack(s[kb][i0 + 2], s[kb][i0 + 3]),
                           TR::pack(s[kb][i0 + 4], s[kb][i0 + 5]), TR::pack(s[kb][i0 + 6], s[kb][i0 + 7])};
      }

    // ---- O^T += V^T P^T  (A = V^T: rows d, k = keys, read transposed from the V tile)
    pipelined<DB * 4, 2>(
        [&](int i) {
          const int db = i >> 2, kb = (i >> 1) & 1, t2 = i & 1;
          return lds_tr8(tV + sl_off<BC>(kb * 32 + t2 * 16, db * 32), trl);
        },
        [&](int i, const u32x4& a) {
          const int db = i >> 2, kb = (i >> 1) & 1, t2 = i & 1;
          acc[db] = TR::mfma(a, pb[kb][t2], acc[db]);
        });
  };

  // Unrolled by two so that each half sees fixed buffers (even tiles in buffer 0).
  for (int t = 0; t < kv_end; t += 2) {
    wait_vmcnt<0>();  // this wave's share of tile t has landed
    lds_barrier();    // ... and everyone's; everyone is also done with tile t-1
    step(t, sK + TILE, sV + TILE, sK, sV);
    if (t + 1 < kv_end) {
      wait_vmcnt<0>();
      lds_barrier();
      step(t + 1, sK, sV, sK + TILE, sV + TILE);
    }
  }

  // ---- epilogue: normalise, write O (input dtype, RNE) and LSE (natural log, fp32)
  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / l_tot;
  if (qi < N) {
    uint16_t* const orow = O + (size_t)bh * N * HD + (size_t)qi * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = db * 32 + i4 * 8 + g * 4;
        const u32x2 w = {TR::pack(acc[db][i4 * 4 + 0] * inv, acc[db][i4 * 4 + 1] * inv),
                         TR::pack(acc[db][i4 * 4 + 2] * inv, acc[db][i4 * 4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    if (g == 0) LSE[(size_t)bh * N + qi] = m_run * scale + __logf(l_tot);
  }
}

template <typename TR, int HD, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a) {
  const int n_qt = (int)((a.N + kFwdBR - 1) / kFwdBR);
  const long long blocks = a.B * a.Hq * (long long)n_qt;
  // c2 must be > 0 so that exp2(-inf * c2) is an exact 0 for masked scores; a zero scale
  // becomes 2^-100, for which every exp2 rounds to exactly 1 (uniform weights).
  const float c2 = a.scale > 0.f ? a.scale * kLog2e : 0x1p-100f;
  hipLaunchKernelGGL((fwd_kernel<TR, HD, CAUSAL>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                     (int)a.Hq, (int)a.Hkv, (int)a.N, n_qt, c2, a.scale);
  return hipGetLastError();
}

template <typename TR>
hipError_t launch_fwd_dt(const FwdArgs& a) {
  if (a.D == 64) return a.causal ? launch_fwd_t<TR, 64, true>(a) : launch_fwd_t<TR, 64, false>(a);
  return a.causal ? launch_fwd_t<TR, 128, true>(a) : launch_fwd_t<TR, 128, false>(a);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
  return a.bf16 ? launch_fwd_dt<Bf16>(a) : launch_fwd_dt<F16>(a);
}

}  // namespace fa
