// Backward pass of exact tiled attention on gfx950.
//
// No probability matrix is read back from memory: every score block is
// rebuilt from Q, K and the per-row lse saved by the forward pass, and the
// gradients are computed block by block and accumulated (Brenndoerfer,
// "FlashAttention Algorithm > Recomputation Strategy", "What Gets Stored vs
// Recomputed"; dmarx anthology record SOTA-087, "Why recomputation is cheaper
// here than storing").
//
// Three kernels on one stream:
//   1. bwd_pre: D_i = dO_i . o_i (float32) and zeroing of the float32 dQ
//      accumulator.  Because each row of the softmax Jacobian satisfies
//      sum_j P_ij dP_ij = dO_i . o_i, the Jacobian product collapses to
//      dS_ij = P_ij (dP_ij - D_i).
//   2. bwd_main: one workgroup keeps a block of 128 keys (K_j, V_j) resident
//      and sweeps the query blocks.  Per query block it recomputes
//      S^T = K Q^T and dP^T = V dO^T on the matrix cores (a lane owns one
//      query, so lse_i and D_i are per-lane scalars), forms P and dS, parks
//      them in LDS, accumulates dV += P^T dO and dK += dS^T Q in registers,
//      and adds dQ += dS K into the float32 accumulator with hardware float
//      atomics (the dQ contributions of different key blocks meet only
//      there; the choice over a separate dQ pass keeps the executed matrix
//      work at five products per score block).
//   3. bwd_post: dq = scale * accumulator, converted to the output type.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBwdBK = 128;
constexpr int kBwdThreads = 256;

// ---------------------------------------------------------------------------
// 1. D_i = dO_i . o_i, and dq_acc = 0.  CPR threads cooperate on one row.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = D / EPC;  // 16-byte chunks per row: 8, 16 or 32
  const long long rows = (long long)a.B * a.H * a.N;
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  const T* O = reinterpret_cast<const T*>(a.o);
  const T* dO = reinterpret_cast<const T*>(a.dO);
  // Every thread of a row group runs the same trip count, so the shuffles
  // below always see all CPR lanes of the group.
  for (long long t = gtid; t < ((rows * CPR + stride - 1) / stride) * stride; t += stride) {
    const long long row = t / CPR;
    const int part = (int)(t % CPR);
    float dot = 0.f;
    const bool in = row < rows;
    if (in) {
      const uint4 ov = *reinterpret_cast<const uint4*>(O + row * D + part * EPC);
      const uint4 dv = *reinterpret_cast<const uint4*>(dO + row * D + part * EPC);
      const T* op = reinterpret_cast<const T*>(&ov);
      const T* dp = reinterpret_cast<const T*>(&dv);
#pragma unroll
      for (int e = 0; e < EPC; ++e) dot = fmaf((float)op[e], (float)dp[e], dot);
      float* acc = a.dq_acc + row * D + part * EPC;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) *reinterpret_cast<f32x4*>(acc + e) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, CPR);
    if (in && part == 0) {
      const int pos = (int)(row % a.N);
      const int b = (int)(row / ((long long)a.H * a.N));
      const int L = clamp_len(a.seqlens, b, a.N);
      a.delta[row] = pos < L ? dot : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. Key-block-resident recompute of P and dS, dV/dK accumulation, dQ atomics.
template <typename T, int D, bool CAUSAL, int BQ>
__global__ __launch_bounds__(kBwdThreads) void bwd_main_kernel(BwdArgs a) {
  constexpr int BK = kBwdBK, NT = kBwdThreads;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int STR = D + PAD;    // row stride of K, Q, dO tiles
  constexpr int PSTR = BK + PAD;  // row stride of the P and dS tiles ([query][key])
  constexpr int NC = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NQT = BQ / 32;
  __shared__ __attribute__((aligned(16))) T sK[BK * STR];
  __shared__ __attribute__((aligned(16))) T sQ[BQ * STR];
  __shared__ __attribute__((aligned(16))) T sdO[BQ * STR];
  __shared__ __attribute__((aligned(16))) T sP[BQ * PSTR];
  __shared__ __attribute__((aligned(16))) T sdS[BQ * PSTR];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, n = lane & 31;
  const int BH = a.B * a.H;
  const int kb = blockIdx.x / BH;  // causal: low key blocks see the most queries and go first
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H;
  const int L = clamp_len(a.seqlens, b, a.N);
  const size_t hoff = (size_t)bh * a.N * D;
  const T* Qg = reinterpret_cast<const T*>(a.q) + hoff;
  const T* Kg = reinterpret_cast<const T*>(a.k) + hoff;
  const T* Vg = reinterpret_cast<const T*>(a.v) + hoff;
  const T* dOg = reinterpret_cast<const T*>(a.dO) + hoff;
  T* dKg = reinterpret_cast<T*>(a.dk) + hoff;
  T* dVg = reinterpret_cast<T*>(a.dv) + hoff;
  float* dQacc = a.dq_acc + hoff;
  const float* LSE = a.lse + (size_t)bh * a.N;
  const float* Dv = a.delta + (size_t)bh * a.N;

  const int k0 = kb * BK;
  const int kw0 = k0 + 32 * w;  // this wave's first key

  if (k0 >= L) {
    // Whole key block is padding: its gradients are zero.
    for (int idx = tid; idx < BK * D; idx += NT) {
      const int r = k0 + idx / D;
      if (r < a.N) {
        dKg[(size_t)r * D + idx % D] = (T)0.f;
        dVg[(size_t)r * D + idx % D] = (T)0.f;
      }
    }
    return;
  }

  // This wave's 32 keys and values as A fragments (rows = keys).
  Frag<T> kf[NC], vf[NC];
  {
    const int kr = kw0 + n;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[c] = kr < a.N ? ld8(Kg + (size_t)kr * D + 16 * c + 8 * h) : zero_frag<T>();
      vf[c] = kr < a.N ? ld8(Vg + (size_t)kr * D + 16 * c + 8 * h) : zero_frag<T>();
    }
  }
  {
    TileCopy<T, BK, D, NT> ck;
    ck.load(Kg, k0, a.N, tid);
    ck.template store<STR>(sK, tid);
  }

  f32x16 dKacc[NDT], dVacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    dKacc[t] = zero16();
    dVacc[t] = zero16();
  }
  const float c2 = a.scale * kLog2e;
  const int qb_begin = CAUSAL ? k0 / BQ : 0;
  const int qb_end = (L + BQ - 1) / BQ;

  for (int qb = qb_begin; qb < qb_end; ++qb) {
    const int q0 = qb * BQ;
    {
      TileCopy<T, BQ, D, NT> cq, cd;
      cq.load(Qg, q0, a.N, tid);
      cd.load(dOg, q0, a.N, tid);
      cq.template store<STR>(sQ, tid);
      cd.template store<STR>(sdO, tid);
    }
    float lse2[NQT], dq_[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int qq = q0 + 32 * qt + n;
      lse2[qt] = qq < L ? LSE[qq] * kLog2e : 0.f;
      dq_[qt] = qq < L ? Dv[qq] : 0.f;
    }
    __syncthreads();

#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        mma16(s, kf[c], ld8(sQ + (32 * qt + n) * STR + 16 * c + 8 * h));
        mma16(dp, vf[c], ld8(sdO + (32 * qt + n) * STR + 16 * c + 8 * h));
      }
      const int qq = q0 + 32 * qt + n;
      const bool qvalid = qq < L;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        float pv[4], dsv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * gi + j;
          const int key = kw0 + acc_row(i, h);
          const bool ok = qvalid && key < L && (!CAUSAL || key <= qq);
          const float p = ok ? exp2_fast(fmaf(s[i], c2, -lse2[qt])) : 0.f;
          pv[j] = p;
          dsv[j] = p * (dp[i] - dq_[qt]);
        }
        const int off = (32 * qt + n) * PSTR + 32 * w + 8 * gi + 4 * h;
        st4(sP + off, pv[0], pv[1], pv[2], pv[3]);
        st4(sdS + off, dsv[0], dsv[1], dsv[2], dsv[3]);
      }
    }
    // dV += P^T dO and dK += dS^T Q over this wave's own 32 keys (its own
    // LDS columns, written above by this same wave).
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int qc = 0; qc < BQ / 16; ++qc) {
        mma16(dVacc[t], ld_col_frag<false>(sP, PSTR, 16 * qc, 32 * w, lane),
              ld_col_frag<false>(sdO, STR, 16 * qc, 32 * t, lane));
        mma16(dKacc[t], ld_col_frag<false>(sdS, PSTR, 16 * qc, 32 * w, lane),
              ld_col_frag<false>(sQ, STR, 16 * qc, 32 * t, lane));
      }
    __syncthreads();  // every wave's dS columns are in LDS

    // dQ (block of BQ queries x D) = dS (BQ x 128 keys) K (128 x D); the
    // 32x32 output tiles are dealt round-robin to the waves.
    for (int tile = w; tile < NQT * NDT; tile += 4) {
      const int qt = tile / NDT, t = tile % NDT;
      f32x16 acc = zero16();
#pragma unroll
      for (int c = 0; c < BK / 16; ++c)
        mma16(acc, ld8(sdS + (32 * qt + n) * PSTR + 16 * c + 8 * h), ld_col_frag<false>(sK, STR, 16 * c, 32 * t, lane));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qq = q0 + 32 * qt + acc_row(i, h);
        if (qq < L) unsafeAtomicAdd(dQacc + (size_t)qq * D + 32 * t + n, acc[i]);
      }
    }
    __syncthreads();  // LDS tiles are rewritten by the next query block
  }

#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw0 + acc_row(i, h);
      if (key < a.N) {
        const bool ok = key < L;
        dKg[(size_t)key * D + 32 * t + n] = (T)(ok ? dKacc[t][i] * a.scale : 0.f);
        dVg[(size_t)key * D + 32 * t + n] = (T)(ok ? dVacc[t][i] : 0.f);
      }
    }
}

// ---------------------------------------------------------------------------
// 3. dq = scale * dq_acc in the output type (rows past L hold zeros already).
template <typename T>
__global__ __launch_bounds__(256) void bwd_post_kernel(const float* __restrict__ acc, T* __restrict__ dq,
                                                       long long n4, float scale) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(acc + 4 * i);
    st4(dq + 4 * i, v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
  }
}

unsigned grid_for(long long work, int threads) {
  long long g = (work + threads - 1) / threads;
  if (g > 65536LL * 8) g = 65536LL * 8;
  return (unsigned)(g < 1 ? 1 : g);
}

template <typename T, int D, bool CAUSAL, int BQ>
hipError_t launch_one(const BwdArgs& a, hipStream_t stream) {
  constexpr int CPR = D * (int)sizeof(T) / 16;
  const long long rows = (long long)a.B * a.H * a.N;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(grid_for(rows * CPR, 256)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkb = (a.N + kBwdBK - 1) / kBwdBK;
  const long long grid = (long long)nkb * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_main_kernel<T, D, CAUSAL, BQ>), dim3((unsigned)grid), dim3(kBwdThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n4 = rows * D / 4;
  hipLaunchKernelGGL((bwd_post_kernel<T>), dim3(grid_for(n4, 256)), dim3(256), 0, stream, a.dq_acc,
                     reinterpret_cast<T*>(a.dq), n4, a.scale);
  return hipGetLastError();
}

template <typename T, int D, int BQ>
hipError_t launch_mask(const BwdArgs& a, bool causal, hipStream_t stream) {
  return causal ? launch_one<T, D, true, BQ>(a, stream) : launch_one<T, D, false, BQ>(a, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int d, int dtype, bool causal, hipStream_t stream) {
  if (dtype == 0) return d == 64 ? launch_mask<bf16, 64, 64>(a, causal, stream) : launch_mask<bf16, 128, 64>(a, causal, stream);
  return d == 64 ? launch_mask<float, 64, 64>(a, causal, stream) : launch_mask<float, 128, 32>(a, causal, stream);
}

}  // namespace fa
