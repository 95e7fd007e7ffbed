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
//   1. bwd_pre:  D_i = dO_i . o_i (float32).  Because each row of the softmax
//      Jacobian satisfies sum_j P_ij dP_ij = dO_i . o_i, the Jacobian
//      product collapses to dS_ij = P_ij (dP_ij - D_i).
//   2. bwd_dkdv: one workgroup keeps a block of 128 keys (K_j, V_j) resident
//      and sweeps the query blocks, recomputing S = Q K^T and dP = dO V^T and
//      accumulating dV += P^T dO and dK += dS^T Q in registers.
//   3. bwd_dq:   one workgroup keeps a block of 128 queries resident and sweeps
//      the key blocks, recomputing S and dP once more and accumulating
//      dQ += dS K in registers.
// dQ is reduced by this separate pass, not by float atomics from stage 2:
// device-scope float atomics are resolved beyond the per-XCD L2 caches, and
// at 4 bytes per (key block, query, dim) their request rate, not the two
// extra matrix products per score block, bounds the pass.  Stages 2 and 3
// are independent once D exists.  Everything is deterministic.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// 1. D_i = dO_i . o_i.  CPR threads cooperate on one row.
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
// 2. dK, dV.  Each wave owns 32 keys and computes S = Q K^T for 32-query
// tiles, so a lane owns one key and holds 16 queries of a tile in registers.
// P and dS then feed dV += P^T dO and dK += dS^T Q straight from registers
// (the contraction runs over the queries held in-register; dO and Q are read
// as column fragments in the matching order).  Query blocks are double
// buffered: the next block's Q, dO, lse and D are fetched into registers
// while the current one is computed, then parked in the idle buffer.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, (sizeof(T) == 2 && D == 64) ? 2 : 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BK = 128, NT = kThreads;
  constexpr int BQ = (sizeof(T) == 4 && D == 128) ? 32 : 64;  // fp32 d=128 keeps its registers
  constexpr int NC = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NQT = BQ / 32;
  __shared__ __attribute__((aligned(16))) T sQ[2][BQ * D];   // swizzled Tile<T, D>
  __shared__ __attribute__((aligned(16))) T sdO[2][BQ * D];
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];  // lse * log2(e); +inf for rows >= L
  __shared__ __attribute__((aligned(16))) float sD[2][BQ];  // D_i; 0 for rows >= L

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
  const float* LSE = a.lse + (size_t)bh * a.N;
  const float* Dv = a.delta + (size_t)bh * a.N;

  const int k0 = kb * BK;
  const int kw0 = k0 + 32 * w;  // this wave's first key
  const int key = kw0 + n;      // this lane's key
  const bool key_ok = key < L;

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

  // This wave's keys and values as B fragments (columns = keys).
  Frag<T> kf[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    kf[c] = key < a.N ? ld8(Kg + (size_t)key * D + 16 * c + 8 * h) : zero_frag<T>();
    vf[c] = key < a.N ? ld8(Vg + (size_t)key * D + 16 * c + 8 * h) : zero_frag<T>();
  }

  const float c2 = a.scale * kLog2e;
  const int qb_begin = CAUSAL ? k0 / BQ : 0;
  const int qb_end = (L + BQ - 1) / BQ;

  // The prefetch keeps the raw loaded values; any arithmetic on them waits
  // for the load, and the in-order memory counter would then also wait for
  // the Q and dO tiles issued with it.  They are converted when parked.
  TileCopy<T, BQ, D, NT> cq, cd;
  float raw_l = 0.f, raw_d = 0.f;
  int pre_q0 = 0;
  auto fetch = [&](int qb) {
    pre_q0 = qb * BQ;
    cq.load(Qg, pre_q0, a.N, tid);
    cd.load(dOg, pre_q0, a.N, tid);
    if (tid < BQ) {
      const int qq = min(pre_q0 + tid, L - 1);  // L >= 1 here
      raw_l = LSE[qq];
      raw_d = Dv[qq];
    }
  };
  auto park = [&](int buf) {
    cq.store(sQ[buf], tid);
    cd.store(sdO[buf], tid);
    if (tid < BQ) {
      const bool in = pre_q0 + tid < L;
      sL[buf][tid] = in ? raw_l * kLog2e : INFINITY;
      sD[buf][tid] = in ? raw_d : 0.f;
    }
  };
  if (qb_begin < qb_end) {
    fetch(qb_begin);
    park(0);
  }
  // Every load issued so far (kf, vf and the first block) has landed; waiting
  // here lets the loop's matrix products read kf and vf without waiting on
  // the in-order memory counter, which would also cover the prefetch.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();

  f32x16 dKacc[NDT], dVacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    dKacc[t] = zero16();
    dVacc[t] = zero16();
  }

  for (int qb = qb_begin; qb < qb_end; ++qb) {
    const int buf = (qb - qb_begin) & 1;
    const int q0 = qb * BQ;
    const bool more = qb + 1 < qb_end;
    if (more) fetch(qb + 1);
    const T* Qs = sQ[buf];
    const T* dOs = sdO[buf];
    // Masking is needed only where the block crosses the diagonal of this
    // wave's keys or the wave holds padded keys.
    const bool edge = (CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > L);

#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        mma16(s, ld_row_frag<T, D>(Qs, 32 * qt + n, 16 * c + 8 * h), kf[c]);
        mma16(dp, ld_row_frag<T, D>(dOs, 32 * qt + n, 16 * c + 8 * h), vf[c]);
      }
      if (edge) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qq = q0 + 32 * qt + acc_row(i, h);
          if (!key_ok || (CAUSAL && key > qq)) s[i] = -INFINITY;
        }
      }
      float p[16], ds[16];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[buf][32 * qt + 8 * gi + 4 * h]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sD[buf][32 * qt + 8 * gi + 4 * h]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * gi + j;
          p[i] = exp2_fast(fmaf(s[i], c2, -l4[j]));
          ds[i] = p[i] * (dp[i] - d4[j]);
        }
      }
      // Registers 8cc..8cc+7 enumerate queries 16cc..16cc+15 of this tile in
      // the PERM order, so they are directly the contraction operand.
      Frag<T> pf[2], dsf[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[cc][e] = (T)p[8 * cc + e];
          dsf[cc][e] = (T)ds[8 * cc + e];
        }
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          mma16(dVacc[t], pf[cc], ld_col_frag<true, T, D>(dOs, 32 * qt + 16 * cc, 32 * t, lane));
          mma16(dKacc[t], dsf[cc], ld_col_frag<true, T, D>(Qs, 32 * qt + 16 * cc, 32 * t, lane));
        }
    }
    if (more) park(buf ^ 1);
    __syncthreads();  // the next query block is in LDS; this one is no longer read
  }

  // dV / dK tiles: lane = head-dim column, registers = keys.
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kr = kw0 + acc_row(i, h);
      if (kr < a.N) {
        const bool ok = kr < L;
        dKg[(size_t)kr * D + 32 * t + n] = (T)(ok ? dKacc[t][i] * a.scale : 0.f);
        dVg[(size_t)kr * D + 32 * t + n] = (T)(ok ? dVacc[t][i] : 0.f);
      }
    }
}

// ---------------------------------------------------------------------------
// 3. dQ.  The forward kernel's structure: 4 waves x 32 queries, key/value
// blocks of 64 streamed through LDS.  Each wave computes S^T = K Q^T and
// dP^T = V dO^T (a lane owns one query, so lse_i and D_i are per-lane
// scalars), forms dS^T in registers and accumulates dQ^T += K^T dS^T with
// dS^T as the contraction operand straight from registers.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, (sizeof(T) == 2 && D == 64) ? 2 : 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BQ = 128, BK = 64, NT = kThreads;
  constexpr int NC = D / 16;
  constexpr int NDT = D / 32;
  __shared__ __attribute__((aligned(16))) T sK[2][BK * D];  // swizzled Tile<T, D>
  __shared__ __attribute__((aligned(16))) T sV[2][BK * D];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, n = lane & 31;
  const int BH = a.B * a.H;
  const int nqb = (a.N + BQ - 1) / BQ;
  const int qb = CAUSAL ? (nqb - 1 - (int)(blockIdx.x / BH)) : (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H;
  const int L = clamp_len(a.seqlens, b, a.N);
  const size_t hoff = (size_t)bh * a.N * D;
  const T* Qg = reinterpret_cast<const T*>(a.q) + hoff;
  const T* Kg = reinterpret_cast<const T*>(a.k) + hoff;
  const T* Vg = reinterpret_cast<const T*>(a.v) + hoff;
  const T* dOg = reinterpret_cast<const T*>(a.dO) + hoff;
  T* dQg = reinterpret_cast<T*>(a.dq) + hoff;
  const float* LSE = a.lse + (size_t)bh * a.N;
  const float* Dv = a.delta + (size_t)bh * a.N;

  const int q0w = qb * BQ + w * 32;
  const int qrow = q0w + n;
  int kend = L;
  if (CAUSAL) kend = min(kend, min(a.N, (qb + 1) * BQ));
  int kend_w = L;
  if (CAUSAL) kend_w = min(kend_w, q0w + 32);
  const bool wave_live = q0w < L;
  const bool row_ok = qrow < L;

  Frag<T> qf[NC], df[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qf[c] = (qrow < a.N) ? ld8(Qg + (size_t)qrow * D + 16 * c + 8 * h) : zero_frag<T>();
    df[c] = (qrow < a.N) ? ld8(dOg + (size_t)qrow * D + 16 * c + 8 * h) : zero_frag<T>();
  }
  // Rows past L get lse = +inf (every probability 0) and D = 0.
  const float lse2 = row_ok ? LSE[qrow] * kLog2e : INFINITY;
  const float dq_i = row_ok ? Dv[qrow] : 0.f;
  const float c2 = a.scale * kLog2e;

  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = zero16();

  const int nkb = (kend + BK - 1) / BK;
  TileCopy<T, BK, D, NT> ck, cv;
  if (nkb > 0) {
    ck.load(Kg, 0, a.N, tid);
    cv.load(Vg, 0, a.N, tid);
  }
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    ck.store(sK[buf], tid);
    cv.store(sV[buf], tid);
    __syncthreads();
    if (kb + 1 < nkb) {
      ck.load(Kg, (kb + 1) * BK, a.N, tid);
      cv.load(Vg, (kb + 1) * BK, a.N, tid);
    }
    const int k0 = kb * BK;
    if (wave_live && k0 < kend_w) {
      const T* kt = sK[buf];
      const T* vt = sV[buf];
      f32x16 s[2] = {zero16(), zero16()}, dp[2] = {zero16(), zero16()};
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          mma16(s[t], ld_row_frag<T, D>(kt, t * 32 + n, 16 * c + 8 * h), qf[c]);
          mma16(dp[t], ld_row_frag<T, D>(vt, t * 32 + n, 16 * c + 8 * h), df[c]);
        }
      // Masked scores become -inf (probability exactly 0); only blocks that
      // cross the padding boundary or the diagonal take this branch.
      if ((k0 + BK > L) || (CAUSAL && k0 + BK - 1 > q0w)) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * t + acc_row(i, h);
            if (key >= L || (CAUSAL && key > qrow)) s[t][i] = -INFINITY;
          }
      }
      Frag<T> dsf[4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2_fast(fmaf(s[t][i], c2, -lse2));
          dsf[2 * t + (i >> 3)][i & 7] = (T)(p * (dp[t][i] - dq_i));
        }
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) mma16(acc[t], ld_col_frag<true, T, D>(kt, 16 * c, 32 * t, lane), dsf[c]);
    }
  }

  if (qrow < a.N) {
    const float sc = row_ok ? a.scale : 0.f;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        st4(dQg + (size_t)qrow * D + 32 * t + 8 * gi + 4 * h, acc[t][4 * gi] * sc, acc[t][4 * gi + 1] * sc,
            acc[t][4 * gi + 2] * sc, acc[t][4 * gi + 3] * sc);
  }
}

unsigned grid_for(long long work, int threads) {
  long long g = (work + threads - 1) / threads;
  if (g > 65536LL * 8) g = 65536LL * 8;
  return (unsigned)(g < 1 ? 1 : g);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_one(int stage, const BwdArgs& a, hipStream_t stream) {
  constexpr int CPR = D * (int)sizeof(T) / 16;
  const long long rows = (long long)a.B * a.H * a.N;
  if (stage == 1) {
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(grid_for(rows * CPR, 256)), dim3(256), 0, stream, a);
  } else {
    const long long grid = (long long)((a.N + 127) / 128) * a.B * a.H;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (stage == 2)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mask(int stage, const BwdArgs& a, bool causal, hipStream_t stream) {
  return causal ? launch_one<T, D, true>(stage, a, stream) : launch_one<T, D, false>(stage, a, stream);
}

}  // namespace

hipError_t launch_bwd_stage(int stage, const BwdArgs& a, int d, int dtype, bool causal, hipStream_t stream) {
  if (dtype == 0)
    return d == 64 ? launch_mask<bf16, 64>(stage, a, causal, stream) : launch_mask<bf16, 128>(stage, a, causal, stream);
  return d == 64 ? launch_mask<float, 64>(stage, a, causal, stream) : launch_mask<float, 128>(stage, a, causal, stream);
}

}  // namespace fa
