// Fp32-input path: the same attention, forward and backward, for float32 Q, K, V (and dO),
// with float32 outputs.  It is a verification path (gradient checking against the 16-bit
// kernels, as "FlashAttention for Tesla P100" keeps an fp32-accumulate build and
// "FlashNystrom" section "Scope" keeps fp32 D=128 for checking), so it favours a plain,
// obviously ordered structure over throughput: fp32 FMAs on the VALU, no MFMA.
//
//   forward   one query row per thread (q and the O accumulator in registers); 32-key K/V
//             tiles staged in LDS and read as broadcasts; the online softmax updates its
//             running max and sum once per tile.
//   dQ        one query row per thread: s = q.k, dp = dO.v, dS = P (dP - D), dQ += dS k.
//   dK, dV    two lanes per key (lanes c and c + 32 of a wave): one holds k and the dK
//             accumulator, the other v and the dV accumulator.  For each query, each lane
//             dots its own vector with q (resp. dO), the pair swaps the two dot products
//             (v_permlane32_swap), and both form P and dS; then dK += dS q and dV += P dO.
//             A workgroup loops over every query head of its KV head's group, so GQA needs
//             no partials.
// D and LSE*log2(e) come from the preprocess, in the backward workspace like the 16-bit path
// (-D stored negated).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kF32Threads = 256;
constexpr int kF32BC = 32;  // keys (forward, dQ) or queries (dK/dV) per LDS tile

// Cooperative copy of `rows` rows of HD floats (rows past `valid` read as zero) into LDS.
template <int HD>
__device__ __forceinline__ void stage_rows(float* __restrict__ dst, const float* __restrict__ src, int rows,
                                           int valid) {
  constexpr int V4 = HD / 4;
  for (int e = threadIdx.x; e < rows * V4; e += kF32Threads) {
    const int r = e / V4, c4 = e % V4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r < valid) v = *reinterpret_cast<const f32x4*>(src + (size_t)r * HD + c4 * 4);
    *reinterpret_cast<f32x4*>(dst + r * HD + c4 * 4) = v;
  }
}

template <int HD>
__device__ __forceinline__ float dot_lds(const float (&x)[HD], const float* __restrict__ row) {
  float a = 0.f;
#pragma unroll
  for (int d = 0; d < HD; d += 4) {
    const f32x4 r = *reinterpret_cast<const f32x4*>(row + d);
    a = fmaf(x[d], r[0], a);
    a = fmaf(x[d + 1], r[1], a);
    a = fmaf(x[d + 2], r[2], a);
    a = fmaf(x[d + 3], r[3], a);
  }
  return a;
}

template <int HD>
__device__ __forceinline__ void axpy_lds(float (&y)[HD], float w, const float* __restrict__ row) {
#pragma unroll
  for (int d = 0; d < HD; d += 4) {
    const f32x4 r = *reinterpret_cast<const f32x4*>(row + d);
    y[d] = fmaf(w, r[0], y[d]);
    y[d + 1] = fmaf(w, r[1], y[d + 1]);
    y[d + 2] = fmaf(w, r[2], y[d + 2]);
    y[d + 3] = fmaf(w, r[3], y[d + 3]);
  }
}

// ---------------------------------------------------------------- forward
template <int HD, bool CAUSAL>
__global__ void __launch_bounds__(kF32Threads, 1)
f32_fwd_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
               float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int N, int n_qt, float c2,
               float scale) {
  __shared__ __attribute__((aligned(16))) float sK[kF32BC * HD];
  __shared__ __attribute__((aligned(16))) float sV[kF32BC * HD];
  const int qt = blockIdx.x % n_qt, bh = blockIdx.x / n_qt;
  const int hq = bh % Hq, b = bh / Hq, hkv = hq / (Hq / Hkv);
  const float* const Kh = K + ((size_t)b * Hkv + hkv) * N * HD;
  const float* const Vh = V + ((size_t)b * Hkv + hkv) * N * HD;
  const int q0 = qt * kF32Threads;
  const int qi = q0 + threadIdx.x;
  const bool row_ok = qi < N;

  float q[HD], o[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    q[d] = row_ok ? Q[((size_t)bh * N + qi) * HD + d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;  // running max of c2-scaled scores, running sum against it

  const int kend = CAUSAL ? min(N, q0 + kF32Threads) : N;  // keys any row of the block sees
  for (int k0 = 0; k0 < kend; k0 += kF32BC) {
    const int nk = min(kF32BC, N - k0);
    __syncthreads();
    stage_rows<HD>(sK, Kh + (size_t)k0 * HD, kF32BC, nk);
    stage_rows<HD>(sV, Vh + (size_t)k0 * HD, kF32BC, nk);
    __syncthreads();
    if (!row_ok) continue;
    float t[kF32BC];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32BC; ++j) {
      const int key = k0 + j;
      const bool vis = key < N && (!CAUSAL || key <= qi);
      t[j] = vis ? dot_lds<HD>(q, sK + j * HD) * c2 : -INFINITY;
      mt = fmaxf(mt, t[j]);
    }
    if (mt == -INFINITY) continue;  // no visible key in this tile (causal rows)
    const float m_new = fmaxf(m, mt);
    const float alpha = exp2f(m - m_new);  // 0 on the first visible tile (m = -inf)
    l *= alpha;
#pragma unroll
    for (int d = 0; d < HD; ++d) o[d] *= alpha;
    m = m_new;
#pragma unroll
    for (int j = 0; j < kF32BC; ++j) {
      const float p = exp2f(t[j] - m);
      l += p;
      axpy_lds<HD>(o, p, sV + j * HD);
    }
  }
  if (row_ok) {
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < HD; ++d) O[((size_t)bh * N + qi) * HD + d] = o[d] * inv;
    // m is in log2 units of the scaled scores: LSE = (m + log2 l) ln 2
    LSE[(size_t)bh * N + qi] = (m + log2f(l)) * kLn2;
  }
  (void)scale;
}

// ---------------------------------------------------------------- backward
// -D = -rowsum(dO * O) and LSE * log2(e), one thread per row.
template <int HD>
__global__ void __launch_bounds__(kF32Threads)
f32_bwd_pre_kernel(const float* __restrict__ O, const float* __restrict__ dO, const float* __restrict__ LSE,
                   float* __restrict__ Dl, float* __restrict__ L2, long long rows) {
  const long long r = (long long)blockIdx.x * kF32Threads + threadIdx.x;
  if (r >= rows) return;
  float a = 0.f;
#pragma unroll 8
  for (int d = 0; d < HD; ++d) a = fmaf(O[r * HD + d], dO[r * HD + d], a);
  Dl[r] = -a;
  L2[r] = LSE[r] * kLog2e;
}

// dQ: one query row per thread.
template <int HD, bool CAUSAL>
__global__ void __launch_bounds__(kF32Threads, 1)
f32_bwd_dq_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                  const float* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dl,
                  float* __restrict__ dQ, int Hq, int Hkv, int N, int n_qt, float c2, float scale) {
  __shared__ __attribute__((aligned(16))) float sK[kF32BC * HD];
  __shared__ __attribute__((aligned(16))) float sV[kF32BC * HD];
  const int qt = blockIdx.x % n_qt, bh = blockIdx.x / n_qt;
  const int hq = bh % Hq, b = bh / Hq, hkv = hq / (Hq / Hkv);
  const float* const Kh = K + ((size_t)b * Hkv + hkv) * N * HD;
  const float* const Vh = V + ((size_t)b * Hkv + hkv) * N * HD;
  const int q0 = qt * kF32Threads;
  const int qi = q0 + threadIdx.x;
  const bool row_ok = qi < N;
  float q[HD], g[HD], acc[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    q[d] = row_ok ? Q[((size_t)bh * N + qi) * HD + d] : 0.f;
    g[d] = row_ok ? dO[((size_t)bh * N + qi) * HD + d] : 0.f;
    acc[d] = 0.f;
  }
  const float l2 = row_ok ? L2[(size_t)bh * N + qi] : 0.f;
  const float nd = row_ok ? Dl[(size_t)bh * N + qi] : 0.f;  // -D
  const int kend = CAUSAL ? min(N, q0 + kF32Threads) : N;
  for (int k0 = 0; k0 < kend; k0 += kF32BC) {
    const int nk = min(kF32BC, N - k0);
    __syncthreads();
    stage_rows<HD>(sK, Kh + (size_t)k0 * HD, kF32BC, nk);
    stage_rows<HD>(sV, Vh + (size_t)k0 * HD, kF32BC, nk);
    __syncthreads();
    if (!row_ok) continue;
    for (int j = 0; j < kF32BC; ++j) {
      const int key = k0 + j;
      if (key >= N || (CAUSAL && key > qi)) continue;
      const float p = exp2f(dot_lds<HD>(q, sK + j * HD) * c2 - l2);
      const float ds = p * (dot_lds<HD>(g, sV + j * HD) + nd);
      axpy_lds<HD>(acc, ds, sK + j * HD);
    }
  }
  if (row_ok) {
#pragma unroll
    for (int d = 0; d < HD; ++d) dQ[((size_t)bh * N + qi) * HD + d] = acc[d] * scale;
  }
}

// dK, dV: a workgroup owns 128 keys of one KV head (a key per lane pair) and loops over the
// queries of every query head of the group.
template <int HD, bool CAUSAL>
__global__ void __launch_bounds__(kF32Threads, 1)
f32_bwd_dkdv_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                    const float* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dl,
                    float* __restrict__ dK, float* __restrict__ dV, int Hq, int Hkv, int N, int n_kt, float c2,
                    float scale) {
  constexpr int KPB = kF32Threads / 2;  // keys per workgroup
  __shared__ __attribute__((aligned(16))) float sQ[kF32BC * HD];
  __shared__ __attribute__((aligned(16))) float sG[kF32BC * HD];
  __shared__ float sL[kF32BC], sD[kF32BC];
  const int kt = blockIdx.x % n_kt, bkv = blockIdx.x / n_kt;
  const int b = bkv / Hkv, hkv = bkv % Hkv, grp = Hq / Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5;                       // 0: K side, 1: V side
  const int key = kt * KPB + wave * 32 + (lane & 31);
  const bool key_ok = key < N;
  const float* const own = (half ? V : K) + ((size_t)bkv * N + key) * HD;
  float x[HD], acc[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    x[d] = key_ok ? own[d] : 0.f;
    acc[d] = 0.f;
  }
  const int kmin = kt * KPB;  // causal: queries before the block's first key see none of it
  const int qstart = CAUSAL ? (kmin / kF32BC) * kF32BC : 0;
  for (int h = 0; h < grp; ++h) {
    const int bh = b * Hq + hkv * grp + h;
    for (int q0 = qstart; q0 < N; q0 += kF32BC) {
      const int nq = min(kF32BC, N - q0);
      __syncthreads();
      stage_rows<HD>(sQ, Q + ((size_t)bh * N + q0) * HD, kF32BC, nq);
      stage_rows<HD>(sG, dO + ((size_t)bh * N + q0) * HD, kF32BC, nq);
      if (threadIdx.x < kF32BC) {
        const bool ok = (int)threadIdx.x < nq;
        sL[threadIdx.x] = ok ? L2[(size_t)bh * N + q0 + threadIdx.x] : 0.f;
        sD[threadIdx.x] = ok ? Dl[(size_t)bh * N + q0 + threadIdx.x] : 0.f;
      }
      __syncthreads();
      const float* const arows = half ? sG : sQ;  // q for the K side, dO for the V side
      for (int i = 0; i < nq; ++i) {
        const int qi = q0 + i;
        // own dot product (s on the K side, dP on the V side), then swap with the partner
        const float mine = dot_lds<HD>(x, arows + i * HD);
        // v_permlane32_swap(u, u): the first result holds lane l - 32's value in the upper
        // half, the second holds lane l + 32's value in the lower half
        const uint32_t u = __float_as_uint(mine);
        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        const float other = __uint_as_float(half ? sw[0] : sw[1]);
        const float s = half ? other : mine, dp = half ? mine : other;
        const bool vis = key_ok && (!CAUSAL || key <= qi);
        const float p = vis ? exp2f(s * c2 - sL[i]) : 0.f;
        const float ds = p * (dp + sD[i]);
        axpy_lds<HD>(acc, half ? p : ds, arows + i * HD);  // dV += P dO  /  dK += dS q
      }
    }
  }
  if (key_ok) {
    float* const dst = (half ? dV : dK) + ((size_t)bkv * N + key) * HD;
    const float f = half ? 1.f : scale;
#pragma unroll
    for (int d = 0; d < HD; ++d) dst[d] = acc[d] * f;
  }
}

// ---------------------------------------------------------------- launchers
// The fp32 kernels keep their running max in c2-scaled units and mask with explicit -inf, so a
// negative scale needs no special case; a zero scale becomes 2^-100 (every exp2 rounds to 1).
inline float f32_c2(float scale) { return scale != 0.f ? scale * kLog2e : 0x1p-100f; }

template <int HD, bool CAUSAL>
hipError_t f32_fwd_t(const FwdArgs& a) {
  const int n_qt = (int)((a.N + kF32Threads - 1) / kF32Threads);
  hipLaunchKernelGGL((f32_fwd_kernel<HD, CAUSAL>), dim3((unsigned)(a.B * a.Hq * n_qt)), dim3(kF32Threads), 0,
                     a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, (int)a.Hq, (int)a.Hkv,
                     (int)a.N, n_qt, f32_c2(a.scale), a.scale);
  return hipGetLastError();
}

template <int HD>
hipError_t f32_pre_t(const BwdArgs& a, const BwdWorkspace& w) {
  const long long rows = a.B * a.Hq * a.N;
  hipLaunchKernelGGL((f32_bwd_pre_kernel<HD>), dim3((unsigned)((rows + kF32Threads - 1) / kF32Threads)),
                     dim3(kF32Threads), 0, a.stream, static_cast<const float*>(a.o), static_cast<const float*>(a.dout),
                     a.lse, reinterpret_cast<float*>(a.ws + w.delta), reinterpret_cast<float*>(a.ws + w.lse2), rows);
  return hipGetLastError();
}

template <int HD, bool CAUSAL>
hipError_t f32_dq_t(const BwdArgs& a, const BwdWorkspace& w) {
  const int n_qt = (int)((a.N + kF32Threads - 1) / kF32Threads);
  hipLaunchKernelGGL((f32_bwd_dq_kernel<HD, CAUSAL>), dim3((unsigned)(a.B * a.Hq * n_qt)), dim3(kF32Threads), 0,
                     a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<const float*>(a.dout),
                     reinterpret_cast<const float*>(a.ws + w.lse2), reinterpret_cast<const float*>(a.ws + w.delta),
                     static_cast<float*>(a.dq), (int)a.Hq, (int)a.Hkv, (int)a.N, n_qt, f32_c2(a.scale), a.scale);
  return hipGetLastError();
}

template <int HD, bool CAUSAL>
hipError_t f32_dkdv_t(const BwdArgs& a, const BwdWorkspace& w) {
  const int n_kt = (int)((a.N + kF32Threads / 2 - 1) / (kF32Threads / 2));
  hipLaunchKernelGGL((f32_bwd_dkdv_kernel<HD, CAUSAL>), dim3((unsigned)(a.B * a.Hkv * n_kt)), dim3(kF32Threads), 0,
                     a.stream, static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<const float*>(a.dout),
                     reinterpret_cast<const float*>(a.ws + w.lse2), reinterpret_cast<const float*>(a.ws + w.delta),
                     static_cast<float*>(a.dk), static_cast<float*>(a.dv), (int)a.Hq, (int)a.Hkv, (int)a.N, n_kt,
                     f32_c2(a.scale), a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  if (a.D == 64) return a.causal ? f32_fwd_t<64, true>(a) : f32_fwd_t<64, false>(a);
  return a.causal ? f32_fwd_t<128, true>(a) : f32_fwd_t<128, false>(a);
}

hipError_t launch_bwd_preprocess_f32(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  return a.D == 64 ? f32_pre_t<64>(a, w) : f32_pre_t<128>(a, w);
}

hipError_t launch_bwd_dkdv_f32(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  if (a.D == 64) return a.causal ? f32_dkdv_t<64, true>(a, w) : f32_dkdv_t<64, false>(a, w);
  return a.causal ? f32_dkdv_t<128, true>(a, w) : f32_dkdv_t<128, false>(a, w);
}

hipError_t launch_bwd_dq_f32(const BwdArgs& a) {
  const BwdWorkspace w = bwd_workspace_layout(a.B, a.Hq, a.Hkv, a.N, a.D);
  if (a.D == 64) return a.causal ? f32_dq_t<64, true>(a, w) : f32_dq_t<64, false>(a, w);
  return a.causal ? f32_dq_t<128, true>(a, w) : f32_dq_t<128, false>(a, w);
}

}  // namespace fa
