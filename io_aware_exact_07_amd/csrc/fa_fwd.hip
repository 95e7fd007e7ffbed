// Forward pass of exact tiled attention on gfx950.
//
// One workgroup = 4 waves = 128 query rows of one (batch, head); each wave
// owns 32 rows.  Key/value blocks of 64 rows are streamed through LDS (a
// pipeline of direct HBM -> LDS copies, one barrier per block) and every
// block of scores lives
// only in registers: it is produced by the matrix cores, folded into the
// running max / normaliser / output accumulator, and dropped (dmarx anthology
// record SOTA-087, "Why recomputation is cheaper here than storing": the score
// block is consumed on chip and never written out; "Condition": the softmax is
// computed blockwise with the online running-maximum formulation).
//
// Orientation: each wave computes S^T = K Q^T, so a lane owns one query and
// holds that query's scores for 16 keys of each 32-key tile; the row max and
// row sum are in-lane reductions plus one exchange with the lane 32 apart.
// The output is accumulated transposed (O^T += V^T P^T) so that the running
// rescale factor of a query is a per-lane scalar, and the probability tile is
// fed to the matrix core straight from registers (the V^T fragment is read
// with the matching key order).
//
// Saved per row: lse = m*scale + ln(l), one float32, which is everything the
// backward pass needs besides Q, K, V, O (Brenndoerfer, "FlashAttention
// Algorithm > Recomputation Strategy", "What Gets Stored vs Recomputed": the
// running max m and normaliser L; stored here as their combination).
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_place.h"

namespace fa {

namespace {

constexpr int kFwdBQ = 128;
constexpr int kFwdBK = 64;
constexpr int kFwdThreads = 256;
constexpr float kSlack = 8.0f;  // probabilities are formed relative to a max at most 2^8 stale
constexpr int kCUs = 256;        // compute units of an MI355X: workgroups g and g + kCUs share a CU

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, (sizeof(T) == 2 ? 2 : 1)) void fwd_kernel(FwdArgs a) {
  constexpr int BQ = kFwdBQ, BK = kFwdBK, NT = kFwdThreads;
  constexpr int NC = D / 16;   // contraction chunks over the head dimension
  constexpr int NDT = D / 32;  // 32-wide output tiles over the head dimension
  // Pipeline depth: blocks kb+1 .. kb+S-1 are in flight while block kb is
  // computed, which covers the HBM/L2 round trip at d=64.
  // Each stage is its own LDS array so the compiler can tell that copies
  // into one stage never alias reads of another.
  constexpr int S = (sizeof(T) == 2 && D == 64) ? 3 : 2;
  static_assert(S >= 2 && S <= 3, "two or three pipeline stages");
  constexpr int TS = BK * D, TS2 = S > 2 ? BK * D : 8;
  __shared__ __attribute__((aligned(16))) T sK0[TS];  // swizzled Tile<T, D> layout
  __shared__ __attribute__((aligned(16))) T sV0[TS];
  __shared__ __attribute__((aligned(16))) T sK1[TS];
  __shared__ __attribute__((aligned(16))) T sV1[TS];
  __shared__ __attribute__((aligned(16))) T sK2[TS2];
  __shared__ __attribute__((aligned(16))) T sV2[TS2];
  auto kst = [&](auto STG) -> T* {
    if constexpr (decltype(STG)::value == 0) return sK0;
    else if constexpr (decltype(STG)::value == 1) return sK1;
    else return sK2;
  };
  auto vst = [&](auto STG) -> T* {
    if constexpr (decltype(STG)::value == 0) return sV0;
    else if constexpr (decltype(STG)::value == 1) return sV1;
    else return sV2;
  };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, n = lane & 31;
  const int BH = a.B * a.H;
  const int nqb = (a.N + BQ - 1) / BQ;
  // Which query block of which head this workgroup takes: heads stay on as
  // few XCDs as the balance allows, so their K/V tiles are shared in one L2,
  // and each XCD runs its blocks heaviest first (causal work grows with the
  // query block index).  Workgroups g and g + kCUs share a compute unit, so
  // under the causal mask every other group of kCUs is reversed to pair heavy
  // with light blocks there.  At bf16 d = 64 and 96 a compute unit holds three
  // workgroups (g + 2*kCUs too); the pairing then balances two of the three,
  // which measured the same as a three-way balance, because a causal launch's
  // span is set by its heaviest blocks rather than by compute-unit load.
  int bh, qb;
  place_workgroup(make_placement(BH, nqb), blockIdx.x, CAUSAL ? kCUs / 8 : 0, bh, qb);
  const int b = bh / a.H;
  const int L = clamp_len(a.seqlens, b, a.N);
  const size_t hoff = (size_t)bh * a.N * D;
  const T* Q = reinterpret_cast<const T*>(a.q) + hoff;
  const T* K = reinterpret_cast<const T*>(a.k) + hoff;
  const T* V = reinterpret_cast<const T*>(a.v) + hoff;
  T* O = reinterpret_cast<T*>(a.o) + hoff;
  float* LSE = a.lse + (size_t)bh * a.N;

  const int q0w = qb * BQ + w * 32;  // first query row of this wave
  const int qrow = q0w + n;          // this lane's query row
  int kend = L;                      // keys needed by the workgroup
  if (CAUSAL) kend = min(kend, min(a.N, (qb + 1) * BQ));
  int kend_w = L;                    // keys needed by this wave
  if (CAUSAL) kend_w = min(kend_w, q0w + 32);
  const bool wave_live = q0w < L;

  Frag<T> qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qf[c] = (qrow < a.N) ? ld8(Q + (size_t)qrow * D + 16 * c + 8 * h) : zero_frag<T>();

  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = zero16();
  float m = -1e30f;   // running max of raw scores (finite sentinel: no inf-inf)
  float lsum = 0.f;   // this lane's half of the running normaliser
  const float c2 = a.scale * kLog2e;

  // The query fragments have landed before any copy is issued, so the loop's
  // matrix products never wait on the in-order memory counter for them.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  const int nkb = (kend + BK - 1) / BK;
  FragAddr<T, D> fr;
  fr.init(lane);
  TileDma<T, BK, D, NT> dma;
  dma.init(tid);
  constexpr int VM_PER_BLOCK = 2 * TileDma<T, BK, D, NT>::PER;
  auto issue = [&](int kb, T* kd, T* vd) {
    dma.issue(K, kb * BK, a.N, kd, tid);
    dma.issue(V, kb * BK, a.N, vd, tid);
  };
  static_for<S - 1>([&](auto J) {
    if (J < nkb) issue(J, kst(J), vst(J));
  });
  // One key/value block from pipeline stage STG (compile-time, so every LDS
  // address below is a precomputed per-lane offset plus an immediate).
  auto block = [&](const int kb, auto STG) {
    constexpr int buf = decltype(STG)::value;
    constexpr int nxt = (buf + S - 1) % S;
    // Block kb has landed once at most the later blocks' copies are pending.
    wait_blocks<S - 2, VM_PER_BLOCK>(nkb - 1 - kb);
    barrier_lds();  // block kb visible to all waves; stage nxt no longer read
    if (kb + S - 1 < nkb) issue(kb + S - 1, kst(std::integral_constant<int, nxt>()), vst(std::integral_constant<int, nxt>()));
    const int k0 = kb * BK;
    if (!(wave_live && k0 < kend_w)) return;
    const T* kt = kst(STG);
    const T* vt = vst(STG);
    f32x16 s[2] = {zero16(), zero16()};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < NC; ++c) mma16(s[t], fr.row(kt, t, c), qf[c]);

    if ((k0 + BK > L) || (CAUSAL && k0 + BK - 1 > q0w)) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * t + acc_row(i, h);
          if (key >= L || (CAUSAL && key > qrow)) s[t][i] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
    mx = pair_max(mx);
    // The reference max m only moves when some lane's block max exceeds it
    // by more than kSlack (base-2 units), so exponents stay <= kSlack and
    // the rescale of the accumulator is skipped for most blocks.  The
    // result is unchanged: lse and o use the same m consistently.
    if (__builtin_amdgcn_ballot_w64(mx * c2 > m * c2 + kSlack) != 0) {
      const float mnew = fmaxf(m, mx);
      const float alpha = exp2_fast((m - mnew) * c2);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < NDT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] *= alpha;
    }
    const float mc = m * c2;
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2_fast(fmaf(s[t][i], c2, -mc));
        s[t][i] = p;
        rs += p;
      }
    lsum += rs;

    // P^T as contraction operand: chunk c covers keys 16c..16c+15 of the
    // block, registers 8*(c%2)..+7 of tile c/2 (the PERM key order).
    Frag<T> pf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[c][e] = (T)s[c >> 1][8 * (c & 1) + e];
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) mma16(acc[t], fr.col(vt, 16 * c, t), pf[c]);
  };
  for (int kb = 0; kb < nkb; kb += S)
    static_for<S>([&](auto J) {
      if (kb + J < nkb) block(kb + J, J);
    });

  const float ltot = pair_sum(lsum);
  if (qrow < a.N) {
    const bool valid = qrow < L;
    const float inv = valid ? 1.f / ltot : 0.f;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        st4(O + (size_t)qrow * D + 32 * t + 8 * gi + 4 * h, acc[t][4 * gi] * inv, acc[t][4 * gi + 1] * inv,
            acc[t][4 * gi + 2] * inv, acc[t][4 * gi + 3] * inv);
    if (h == 0) LSE[qrow] = valid ? (m * a.scale + log2_fast(ltot) * kLn2) : -INFINITY;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.N + kFwdBQ - 1) / kFwdBQ;
  const long long grid = (long long)nqb * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL>), dim3((unsigned)grid), dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int d, int dtype, bool causal, hipStream_t stream) {
  if (dtype == 0) {
    if (d == 64) return causal ? launch_one<bf16, 64, true>(a, stream) : launch_one<bf16, 64, false>(a, stream);
    if (d == 96) return causal ? launch_one<bf16, 96, true>(a, stream) : launch_one<bf16, 96, false>(a, stream);
    return causal ? launch_one<bf16, 128, true>(a, stream) : launch_one<bf16, 128, false>(a, stream);
  }
  if (d == 64) return causal ? launch_one<float, 64, true>(a, stream) : launch_one<float, 64, false>(a, stream);
  if (d == 96) return causal ? launch_one<float, 96, true>(a, stream) : launch_one<float, 96, false>(a, stream);
  return causal ? launch_one<float, 128, true>(a, stream) : launch_one<float, 128, false>(a, stream);
}

}  // namespace fa
