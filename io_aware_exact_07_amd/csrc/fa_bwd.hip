// Backward pass of exact tiled attention on gfx950.
//
// No probability matrix is read back from memory: every score block is
// rebuilt from Q, K and the per-row lse saved by the forward pass, and the
// gradients are computed block by block and accumulated (Brenndoerfer,
// "FlashAttention Algorithm > Recomputation Strategy", "What Gets Stored vs
// Recomputed"; dmarx anthology record SOTA-087, "Why recomputation is cheaper
// here than storing").
//
// Two kernels on one stream:
//   1. bwd_pre:  -D_i = -(dO_i . o_i) (float32).  Because each row of the
//      softmax Jacobian satisfies sum_j P_ij dP_ij = dO_i . o_i, the Jacobian
//      product collapses to dS_ij = P_ij (dP_ij - D_i).
//   2. bwd_grad: two lists of blocks.  A dK/dV block keeps 128 keys (K_j, V_j)
//      resident and sweeps the query blocks, recomputing S = Q K^T and
//      dP = dO V^T and accumulating dV += P^T dO and dK += dS^T Q in
//      registers.  A dQ block keeps 128 queries resident and sweeps the key
//      blocks, recomputing S and dP once more and accumulating dQ += dS K in
//      registers.  One launch runs either list alone or both interleaved.
// dQ is reduced by its own block list, not by float atomics from the dK/dV
// blocks: device-scope float atomics are resolved beyond the per-XCD L2
// caches, and at 4 bytes per (key block, query, dim) their request rate, not
// the two extra matrix products per score block, bounds the pass.  The two
// lists are independent once D exists.  Everything is deterministic.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_place.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// 1. Row vectors for the gradient stages, over Npad rows per head:
//    delta[i] = -(dO_i . o_i) and lse2[i] = lse_i * log2(e) for rows i < L;
//    delta = 0 and lse2 = +inf (every probability of the row 0) for padded
//    rows and for the rows that round the head up to whole 128-row blocks.
//    CPR threads cooperate on one row.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CHUNKS = D / EPC;  // 16-byte chunks per row: 8, 12, 16, 24 or 32
  constexpr int CPR = CHUNKS <= 8 ? 8 : CHUNKS <= 16 ? 16 : 32;  // lanes per row (power of two)
  const int Np = padded_rows(a.N);
  const long long rows = (long long)a.B * a.H * Np;
  const long long gtid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  const T* O = reinterpret_cast<const T*>(a.o);
  const T* dO = reinterpret_cast<const T*>(a.dO);
  // Every thread of a row group runs the same trip count, so the shuffles
  // below always see all CPR lanes of the group.
  for (long long t = gtid; t < ((rows * CPR + stride - 1) / stride) * stride; t += stride) {
    const long long prow = t / CPR;  // row in the padded layout
    const int part = (int)(t % CPR);
    const long long bh = prow / Np;
    const int pos = (int)(prow % Np);
    const int L = prow < rows ? clamp_len(a.seqlens, (int)(bh / a.H), a.N) : 0;
    const bool in = prow < rows && pos < L;
    float dot = 0.f;
    if (in && part < CHUNKS) {
      const long long row = bh * a.N + pos;
      const uint4 ov = *reinterpret_cast<const uint4*>(O + row * D + part * EPC);
      const uint4 dv = *reinterpret_cast<const uint4*>(dO + row * D + part * EPC);
      const T* op = reinterpret_cast<const T*>(&ov);
      const T* dp = reinterpret_cast<const T*>(&dv);
#pragma unroll
      for (int e = 0; e < EPC; ++e) dot = fmaf((float)op[e], (float)dp[e], dot);
    }
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, CPR);
    if (prow < rows && part == 0) {
      a.delta[prow] = in ? -dot : 0.f;  // stored negated: the dP products accumulate onto it
      a.lse2[prow] = in ? a.lse[bh * a.N + pos] * kLog2e : INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV.  Each wave owns 32 keys and computes S = Q K^T for 32-query
// tiles, so a lane owns one key and holds 16 queries of a tile in registers.
// P and dS then feed dV += P^T dO and dK += dS^T Q straight from registers
// (the contraction runs over the queries held in-register; dO and Q are read
// as column fragments in the matching order).  Query blocks stream through S
// LDS stages filled by direct HBM -> LDS copies issued S-1 blocks ahead: the
// Q and dO tiles, plus the block's lse2 and -D row vectors.
template <typename T, int D, int OCC>
struct DkdvShape {
  static constexpr int BK = 128;
  // Query rows per block and pipeline stages.  bf16 d=64 takes 128-row
  // blocks (half the barriers per score tile) in two stages, which still
  // fits two workgroups per CU; fp32 d=96, 128 take 32 rows to keep their
  // registers, and so does bf16 d=128 at OCC = 2 waves per SIMD.
  static constexpr bool WIDE = sizeof(T) == 2 && D == 64;
  static constexpr int BQ = WIDE ? 128 : ((sizeof(T) == 4 && D > 64) || (D == 128 && OCC == 2)) ? 32 : 64;
  static constexpr int S = WIDE ? 2 : 3;
  static_assert(BQ / 2 <= 64, "one wave copies a block's lse2 and -D rows, 4 floats per lane");
  static constexpr int TILE = BQ * D * (int)sizeof(T);               // bytes of one Q or dO tile
  static constexpr int STAGE = 2 * TILE + 2 * BQ * 4;                // Q, dO, lse2 | D
  static constexpr int LDS = S * STAGE;
};

// One key block (BK keys of head bh): dK and dV.  `lds` holds S stages of
// [Q tile | dO tile | lse2 | D].
template <typename T, int D, bool CAUSAL, int OCC>
__device__ __forceinline__ void dkdv_block(const BwdArgs& a, const int kb, const int bh, char* lds) {
  using SH = DkdvShape<T, D, OCC>;
  constexpr int BK = SH::BK, NT = kThreads;
  constexpr int BQ = SH::BQ;
  constexpr int NC = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NQT = BQ / 32;
  // Three pipeline stages: Q and dO tiles (swizzled Tile<T, D>) and the
  // block's lse2 | D row vectors, filled by direct HBM -> LDS copies issued
  // two blocks ahead.
  constexpr int S = SH::S;
  auto qst = [&](auto STG) -> T* { return reinterpret_cast<T*>(lds + decltype(STG)::value * SH::STAGE); };
  auto ost = [&](auto STG) -> T* { return reinterpret_cast<T*>(lds + decltype(STG)::value * SH::STAGE + SH::TILE); };
  auto rst = [&](auto STG) -> float* {
    return reinterpret_cast<float*>(lds + decltype(STG)::value * SH::STAGE + 2 * SH::TILE);
  };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, n = lane & 31;
  const int b = bh / a.H;
  const int L = clamp_len(a.seqlens, b, a.N);
  const size_t hoff = (size_t)bh * a.N * D;
  const T* Qg = reinterpret_cast<const T*>(a.q) + hoff;
  const T* Kg = reinterpret_cast<const T*>(a.k) + hoff;
  const T* Vg = reinterpret_cast<const T*>(a.v) + hoff;
  const T* dOg = reinterpret_cast<const T*>(a.dO) + hoff;
  T* dKg = reinterpret_cast<T*>(a.dk) + hoff;
  T* dVg = reinterpret_cast<T*>(a.dv) + hoff;
  const size_t roff = (size_t)bh * padded_rows(a.N);
  const float* L2g = a.lse2 + roff;
  const float* Dg = a.delta + roff;

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
  // Every load so far has landed; the loop's matrix products then never wait
  // on the in-order memory counter for kf and vf.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  const float c2 = a.scale * kLog2e;
  const int qb_begin = CAUSAL ? k0 / BQ : 0;
  const int qb_end = (L + BQ - 1) / BQ;

  TileDma<T, BQ, D, NT> dma;
  dma.init(tid);
  // Wave 0 also copies the row vectors: lanes [0, BQ/4) take lse2, lanes
  // [BQ/4, BQ/2) take D, into one 2*BQ-float stage array.
  constexpr int VM_OTHERS = 2 * TileDma<T, BQ, D, NT>::PER;
  constexpr int VM_WAVE0 = VM_OTHERS + 1;
  auto issue = [&](int qb, auto STG) {
    const int q0 = qb * BQ;
    dma.issue(Qg, q0, a.N, qst(STG), tid);
    dma.issue(dOg, q0, a.N, ost(STG), tid);
    if (w == 0 && lane < BQ / 2) {
      const float* src = lane < BQ / 4 ? L2g + q0 + 4 * lane : Dg + q0 + 4 * (lane - BQ / 4);
      dma16(src, rst(STG));
    }
  };
  static_for<S - 1>([&](auto J) {
    if (qb_begin + J < qb_end) issue(qb_begin + J, J);
  });

  f32x16 dKacc[NDT], dVacc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    dKacc[t] = zero16();
    dVacc[t] = zero16();
  }

  FragAddr<T, D> fr;
  fr.init(lane);
  // One query block from pipeline stage STG (compile-time, so every LDS
  // address is a precomputed per-lane offset plus an immediate).
  auto block = [&](const int qb, auto STG) {
    constexpr int buf = decltype(STG)::value;
    constexpr int nxt = (buf + S - 1) % S;
    // Block qb has landed once at most the later blocks' copies are pending.
    if (w == 0) wait_blocks<S - 2, VM_WAVE0>(qb_end - 1 - qb);
    else wait_blocks<S - 2, VM_OTHERS>(qb_end - 1 - qb);
    barrier_lds();  // block qb visible to all waves; stage nxt no longer read
    if (qb + S - 1 < qb_end) issue(qb + S - 1, std::integral_constant<int, nxt>());
    const int q0 = qb * BQ;
    const T* Qs = qst(STG);
    const T* dOs = ost(STG);
    const float* Rs = rst(STG);
    // Masking is needed only where the block crosses the diagonal of this
    // wave's keys or the wave holds padded keys (padded query rows carry
    // lse2 = +inf and D = 0).
    // The two versions of the tile loop keep the masking branch out of the
    // loop body, so the scheduler can overlap one tile's matrix products with
    // the other tile's exponentials.
    auto tiles = [&](auto EDGE) {
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      // A query tile whose queries all precede this wave's keys (in the
      // diagonal block, the first w tiles of wave w) has P = 0 and dS = 0
      // everywhere: its products would add exact zeros, so they are skipped.
      if constexpr (CAUSAL && decltype(EDGE)::value) {
        if (q0 + 32 * qt + 31 < kw0) continue;
      }
      // dP starts from -D of each query row, so the product leaves dP - D.
      f32x16 s = zero16(), dp;
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(Rs + BQ + 32 * qt + 8 * gi + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[4 * gi + j] = d4[j];
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        mma16(s, fr.row(Qs, qt, c), kf[c]);
        mma16(dp, fr.row(dOs, qt, c), vf[c]);
      }
      if constexpr (decltype(EDGE)::value) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qq = q0 + 32 * qt + acc_row(i, h);
          if (!key_ok || (CAUSAL && key > qq)) s[i] = -INFINITY;
        }
      }
      float p[16], ds[16];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(Rs + 32 * qt + 8 * gi + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * gi + j;
          p[i] = exp2_fast(fmaf(s[i], c2, -l4[j]));
          ds[i] = p[i] * dp[i];
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
          mma16(dVacc[t], pf[cc], fr.col(dOs, 32 * qt + 16 * cc, t));
          mma16(dKacc[t], dsf[cc], fr.col(Qs, 32 * qt + 16 * cc, t));
        }
    }
    };
    if ((CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > L)) tiles(std::true_type());
    else tiles(std::false_type());
  };
  for (int qb = qb_begin; qb < qb_end; qb += S)
    static_for<S>([&](auto J) {
      if (qb + J < qb_end) block(qb + J, J);
    });

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
template <typename T, int D>
struct DqShape {
  static constexpr int BQ = 128, BK = 64;
  static constexpr int S = (sizeof(T) == 2 && D == 64) ? 3 : 2;  // pipeline stages
  static constexpr int TILE = BK * D * (int)sizeof(T);            // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;
  static constexpr int LDS = S * STAGE;
};

// One query block (BQ queries of head bh): dQ.  `lds` holds S stages of
// [K tile | V tile].  GMAX = 32-key tiles whose scores are live at once: the
// whole block, or one tile at a time where the register budget is halved.
template <typename T, int D, bool CAUSAL, int GMAX>
__device__ __forceinline__ void dq_block(const BwdArgs& a, const int qb, const int bh, char* lds) {
  using SH = DqShape<T, D>;
  constexpr int BQ = SH::BQ, BK = SH::BK, NT = kThreads;
  constexpr int NC = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NKT = BK / 32;  // 32-key tiles per block
  // Pipeline stages as in the forward kernel: K/V blocks copied HBM -> LDS
  // S-1 blocks ahead.
  constexpr int S = SH::S;
  auto kst = [&](auto STG) -> T* { return reinterpret_cast<T*>(lds + decltype(STG)::value * SH::STAGE); };
  auto vst = [&](auto STG) -> T* { return reinterpret_cast<T*>(lds + decltype(STG)::value * SH::STAGE + SH::TILE); };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, n = lane & 31;
  const int b = bh / a.H;
  const int L = clamp_len(a.seqlens, b, a.N);
  const size_t hoff = (size_t)bh * a.N * D;
  const T* Qg = reinterpret_cast<const T*>(a.q) + hoff;
  const T* Kg = reinterpret_cast<const T*>(a.k) + hoff;
  const T* Vg = reinterpret_cast<const T*>(a.v) + hoff;
  const T* dOg = reinterpret_cast<const T*>(a.dO) + hoff;
  T* dQg = reinterpret_cast<T*>(a.dq) + hoff;
  const size_t roff = (size_t)bh * padded_rows(a.N);

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
  // Padded and past-the-end rows carry lse2 = +inf (every probability 0), D = 0.
  const float lse2 = a.lse2[roff + qrow];
  const float ndq_i = a.delta[roff + qrow];  // -D of this lane's query
  // dP^T starts from -D (every register of a lane is the same query), so the
  // product leaves dP - D; the copy is loop-invariant.  At bf16 d>64 the
  // two-wave register budget has no room for it, and -D is added after the
  // product instead (in every launch mode, so they round alike).
  constexpr bool NDQ_IN_MMA = !(sizeof(T) == 2 && D > 64);
  f32x16 ndq16;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndq16[i] = ndq_i;
  const float c2 = a.scale * kLog2e;
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = zero16();

  const int nkb = (kend + BK - 1) / BK;
  FragAddr<T, D> fr;
  fr.init(lane);
  TileDma<T, BK, D, NT> dma;
  dma.init(tid);
  constexpr int VM_PER_BLOCK = 2 * TileDma<T, BK, D, NT>::PER;
  auto issue = [&](int kb, T* kd, T* vd) {
    dma.issue(Kg, kb * BK, a.N, kd, tid);
    dma.issue(Vg, kb * BK, a.N, vd, tid);
  };
  static_for<S - 1>([&](auto J) {
    if (J < nkb) issue(J, kst(J), vst(J));
  });
  // One key/value block from pipeline stage STG (compile-time, so every LDS
  // address is a precomputed per-lane offset plus an immediate).
  auto block = [&](const int kb, auto STG) {
    constexpr int buf = decltype(STG)::value;
    constexpr int nxt = (buf + S - 1) % S;
    wait_blocks<S - 2, VM_PER_BLOCK>(nkb - 1 - kb);
    barrier_lds();  // block kb visible to all waves; stage nxt no longer read
    if (kb + S - 1 < nkb) issue(kb + S - 1, kst(std::integral_constant<int, nxt>()), vst(std::integral_constant<int, nxt>()));
    const int k0 = kb * BK;
    if (!(wave_live && k0 < kend_w)) return;
    const T* kt = kst(STG);
    const T* vt = vst(STG);
    // Two versions of the block body keep the masking branch out of it, so
    // the scheduler can overlap one tile's exponentials with the other
    // tile's matrix products.
    // `ntile` of the block's 32-key tiles take part; the rest are wholly
    // masked for this wave (past the sequence end or above its queries), so
    // their products would add exact zeros and are skipped.
    auto body = [&](auto EDGE, auto GGc, const int ntile) {
    constexpr int G = decltype(GGc)::value;  // tiles whose scores are live at once
    static_assert(NKT % G == 0, "tile groups must divide the block");
#pragma unroll
    for (int g0 = 0; g0 < NKT; g0 += G) {
      if (g0 >= ntile) break;
      f32x16 s[G], dp[G];
#pragma unroll
      for (int t = 0; t < G; ++t) {
        s[t] = zero16();
        dp[t] = NDQ_IN_MMA ? ndq16 : zero16();
      }
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          mma16(s[t], fr.row(kt, g0 + t, c), qf[c]);
          mma16(dp[t], fr.row(vt, g0 + t, c), df[c]);
        }
      // Masked scores become -inf (probability exactly 0); only blocks that
      // cross the padding boundary or the diagonal take this version.
      if constexpr (decltype(EDGE)::value) {
#pragma unroll
        for (int t = 0; t < G; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * (g0 + t) + acc_row(i, h);
            if (key >= L || (CAUSAL && key > qrow)) s[t][i] = -INFINITY;
          }
      }
      Frag<T> dsf[2 * G];
#pragma unroll
      for (int t = 0; t < G; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2_fast(fmaf(s[t][i], c2, -lse2));
          dsf[2 * t + (i >> 3)][i & 7] = (T)(NDQ_IN_MMA ? p * dp[t][i] : p * (dp[t][i] + ndq_i));
        }
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int c = 0; c < 2 * G; ++c) mma16(acc[t], fr.col(kt, 32 * g0 + 16 * c, t), dsf[c]);
    }
    };
    if ((k0 + BK > L) || (CAUSAL && k0 + BK - 1 > q0w)) {
      // Tiles wholly above this wave's queries are skipped under the causal
      // mask; tiles wholly past the sequence end only where two tiles are
      // grouped (one at a time, the extra branch costs registers at d > 64).
      int live = NKT;
      if (CAUSAL || GMAX > 1) live = min(live, (L - k0 + 31) / 32);
      if (CAUSAL) live = min(live, (q0w + 63 - k0) / 32);
      if (GMAX > 1 && live < NKT) body(std::true_type(), std::integral_constant<int, 1>(), live);
      else body(std::true_type(), std::integral_constant<int, GMAX>(), live);
    } else {
      body(std::false_type(), std::integral_constant<int, GMAX>(), NKT);
    }
  };
  for (int kb = 0; kb < nkb; kb += S)
    static_for<S>([&](auto J) {
      if (kb + J < nkb) block(kb + J, J);
    });

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

// ---------------------------------------------------------------------------
// Waves per SIMD the register budget targets: two at bf16 (at d>64 the dQ
// body then holds one 32-key tile's scores at a time, and at d=128 the dK/dV
// body takes 32-row query blocks and spills a few registers), except for the
// dK/dV-only launch at bf16 d=128, whose 64-row blocks run faster at one wave
// with 256 VGPRs and 160 AGPRs.  One wave at fp32.
template <typename T, int D, int MODE>
constexpr int grad_occupancy() {
  return (sizeof(T) == 2 && (D <= 96 || MODE != 1)) ? 2 : 1;
}

// Gradient kernel.  MODE 1: dK/dV blocks only; MODE 2: dQ blocks only;
// MODE 0: both job lists in one launch.  With a causal mask the work of a
// block ranges from one block-step to N/64, and a lone launch of either list
// has its heaviest blocks longer than the average per resident workgroup.
// Interleaving the two independent lists heaviest-first (rank r of each list
// in turn, every head) doubles the work per slot so the greedy dispatch
// balances it.  In MODE 0 both bodies share one LDS allocation; a single-list
// launch takes only its own body's, so a dQ-only launch is not held to the
// footprint of the dK/dV stages.
template <typename T, int D, bool CAUSAL, int MODE>
__global__ __launch_bounds__(kThreads, (grad_occupancy<T, D, MODE>())) void bwd_grad_kernel(BwdArgs a) {
  constexpr int OCC = grad_occupancy<T, D, MODE>();
  using KV = DkdvShape<T, D, OCC>;
  using QS = DqShape<T, D>;
  constexpr int LDS = MODE == 1 ? KV::LDS : MODE == 2 ? QS::LDS : (KV::LDS > QS::LDS ? KV::LDS : QS::LDS);
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  const int BH = a.B * a.H;
  const int nb = (a.N + 127) / 128;  // 128-row blocks: key blocks of dK/dV, query blocks of dQ
  // Work item of this workgroup: a head and a block level, heaviest level
  // first (causal: low key blocks, high query blocks).  A single-list launch
  // keeps each head's blocks on as few XCDs as the balance allows, so the
  // tiles they all stream (Q and dO for dK/dV, K and V for dQ) are read into
  // one L2.  MODE 0 interleaves the lists rank by rank over all heads
  // instead: there the dK/dV and dQ blocks of a head stream different
  // tensors, so placing them together shares nothing, and this order spreads
  // each XCD's lists over the fewest heads of either kind (measured: fewer
  // bytes and a shorter launch on the long-context workload).
  int bh, level;
  bool dkdv = MODE == 1;
  if (MODE == 0) {
    const int i = blockIdx.x;
    const int r = i / (2 * BH), j = i % (2 * BH);
    dkdv = j < BH;
    bh = dkdv ? j : j - BH;
    level = nb - 1 - r;
  } else {
    place_workgroup(make_placement(BH, nb), blockIdx.x, 0, bh, level);
  }
  if (dkdv) {
    if constexpr (MODE != 2) dkdv_block<T, D, CAUSAL, OCC>(a, nb - 1 - level, bh, lds);
  } else {
    if constexpr (MODE != 1) dq_block<T, D, CAUSAL, (OCC == 2 && D > 64) ? 1 : QS::BK / 32>(a, level, bh, lds);
  }
}

unsigned grid_for(long long work, int threads) {
  long long g = (work + threads - 1) / threads;
  if (g > 65536LL * 8) g = 65536LL * 8;
  return (unsigned)(g < 1 ? 1 : g);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_one(int stage, const BwdArgs& a, hipStream_t stream) {
  constexpr int CHUNKS = D * (int)sizeof(T) / 16;
  constexpr int CPR = CHUNKS <= 8 ? 8 : CHUNKS <= 16 ? 16 : 32;
  const long long rows = (long long)a.B * a.H * padded_rows(a.N);
  if (stage == 1) {
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(grid_for(rows * CPR, 256)), dim3(256), 0, stream, a);
  } else {
    const long long grid = (long long)((a.N + 127) / 128) * a.B * a.H;
    if (2 * grid > 0x7fffffffLL) return hipErrorInvalidValue;
    if (stage == 2)
      hipLaunchKernelGGL((bwd_grad_kernel<T, D, CAUSAL, 1>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else if (stage == 3)
      hipLaunchKernelGGL((bwd_grad_kernel<T, D, CAUSAL, 2>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_grad_kernel<T, D, CAUSAL, 0>), dim3((unsigned)(2 * grid)), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_mask(int stage, const BwdArgs& a, bool causal, hipStream_t stream) {
  return causal ? launch_one<T, D, true>(stage, a, stream) : launch_one<T, D, false>(stage, a, stream);
}

}  // namespace

hipError_t launch_bwd_stage(int stage, const BwdArgs& a, int d, int dtype, bool causal, hipStream_t stream) {
  if (dtype == 0) {
    if (d == 64) return launch_mask<bf16, 64>(stage, a, causal, stream);
    if (d == 96) return launch_mask<bf16, 96>(stage, a, causal, stream);
    return launch_mask<bf16, 128>(stage, a, causal, stream);
  }
  if (d == 64) return launch_mask<float, 64>(stage, a, causal, stream);
  if (d == 96) return launch_mask<float, 96>(stage, a, causal, stream);
  return launch_mask<float, 128>(stage, a, causal, stream);
}

}  // namespace fa
