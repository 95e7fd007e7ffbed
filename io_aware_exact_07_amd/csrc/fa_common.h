// Device helpers shared by the attention kernels (gfx950 / CDNA4 only).
//
// Matrix-core conventions used everywhere (v_mfma_f32_32x32x16_bf16; the
// fp32 path issues eight v_mfma_f32_32x32x2_f32 per 16-wide chunk with the
// same register arrangement):
//   A fragment  lane l: row m = l % 32, contraction k = 8*(l/32) + e, e = 0..7
//   B fragment  lane l: col n = l % 32, contraction k = 8*(l/32) + e
//   C/D tile    lane l: col n = l % 32, register i: row acc_row(i, l/32)
// A "row fragment" is 8 contraction-contiguous elements of one row, read with
// one 16-byte LDS load.  A "column fragment" holds 8 contraction indices that
// are 8 different rows of a row-major LDS tile; for bf16 it is gathered with
// two ds_read_b64_tr_b16, whose lane mapping is: within each group of 16
// lanes, lane 4r+s supplies the address of 4 contiguous elements of row r
// (columns 4s..4s+3 of a 16-column strip) and lane j receives column j of
// rows 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <utility>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left unconstrained
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct FragOf;
template <> struct FragOf<bf16> { using type = bf16x8; };
template <> struct FragOf<float> { using type = f32x8; };
template <typename T> using Frag = typename FragOf<T>::type;

// Row of the 32x32 accumulator held in register i by lanes of half h.
__device__ __forceinline__ constexpr int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

__device__ __forceinline__ void mma16(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// 8 contiguous elements at p (16-byte aligned for bf16, 32-byte span for fp32).
__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 ld8(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) { r[e] = a[e]; r[e + 4] = b[e]; }
  return r;
}
template <typename T> __device__ __forceinline__ Frag<T> zero_frag() {
  Frag<T> z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (T)0.f;
  return z;
}

// Row-major LDS tile of D-element rows without padding; 16-byte chunks are
// XOR-swizzled per row so that both access patterns the kernels use are free
// of bank conflicts on the 64-bank LDS:
//   (a) 16 lanes read the same logical chunk of 16 consecutive rows
//       (row fragments, ds_read_b128);
//   (b) 32 lanes read 4 consecutive chunks of 4 consecutive rows, rows and
//       chunks aligned to 4 (column fragments, ds_read_b64_tr_b16).
// With 128-byte rows (8 chunks) the row's XOR key takes bits 1..3 of the
// row so that rows 2 apart differ in bit 2; with 256- or 512-byte rows it
// makes the 4 rows of (b) differ in bits 2..3.  Each key is a permutation
// over 16 consecutive rows, which (a) needs.  Rows of 12 or 24 chunks (head
// dimension 96) rotate the chunks by (row/4) % 4 instead: consecutive rows
// then start 12 or 24 chunks apart, so rows r and r+1 already fall 4 or 8
// chunk slots apart and the rotation separates the four 4-row groups.  Every
// key repeats every 16 rows, so adding whole 16-row blocks to a fragment's
// row never changes its column placement.
template <typename T, int D>
struct Tile {
  static constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;         // chunks per row
  static constexpr bool ROT = CPR % 12 == 0;
  static_assert(CPR == 8 || CPR == 12 || CPR == 16 || CPR == 24 || CPR == 32, "unsupported row length");
  __device__ __forceinline__ static int swz(int row) {
    return CPR == 8 ? ((((row >> 1) & 1) << 2) | ((row >> 2) & 3)) : (((row & 3) << 2) | ((row >> 2) & 3));
  }
  // Physical chunk of logical chunk j in `row`, and the inverse.
  __device__ __forceinline__ static int phys(int row, int j) {
    if constexpr (ROT) return (j + ((row >> 2) & 3)) % CPR;
    else return j ^ swz(row);
  }
  __device__ __forceinline__ static int logical(int row, int pc) {
    if constexpr (ROT) return (pc + CPR - ((row >> 2) & 3)) % CPR;
    else return pc ^ swz(row);
  }
  // Element offset of (row, col); col % EPC is preserved.
  __device__ __forceinline__ static int off(int row, int col) {
    return row * D + phys(row, col / EPC) * EPC + (col % EPC);
  }
};

// Row fragment: 8 contiguous columns col..col+7 (col a multiple of 8) of one row.
template <typename T, int D>
__device__ __forceinline__ Frag<T> ld_row_frag(const T* base, int row, int col) {
  if constexpr (sizeof(T) == 2) {
    return ld8(base + Tile<T, D>::off(row, col));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(base + Tile<T, D>::off(row, col));
    const f32x4 b = *reinterpret_cast<const f32x4*>(base + Tile<T, D>::off(row, col + 4));
    Frag<T> r;
#pragma unroll
    for (int e = 0; e < 4; ++e) { r[e] = a[e]; r[e + 4] = b[e]; }
    return r;
  }
}

// Column fragment: the lane receives column col0 + (lane % 32) of 8 rows.
// PERM = false: register e holds row k0 + 8*h + e               (h = lane/32)
// PERM = true:  register e holds row k0 + 8*(e/4) + 4*h + e%4
// The PERM order is the order in which a 32x32 accumulator's registers
// 8c..8c+7 enumerate its rows 16c..16c+15, so an accumulator converted to T
// can feed a matrix core directly as the contraction operand against this
// fragment.
template <bool PERM, typename T, int D>
__device__ __forceinline__ Frag<T> ld_col_frag(const T* base, int k0, int col0, int lane) {
  const int h = lane >> 5;
  if constexpr (sizeof(T) == 2) {
    const int g = lane >> 4, r = (lane >> 2) & 3, s = lane & 3;
    const int col = col0 + 16 * (g & 1) + 4 * s;
    bf16x8 out;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = PERM ? (k0 + 8 * t + 4 * h + r) : (k0 + 8 * h + 4 * t + r);
      const bf16* p = base + Tile<T, D>::off(row, col);
      s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
      bf16x4 vb = __builtin_bit_cast(bf16x4, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * t + e] = vb[e];
    }
    return out;
  } else {
    const int col = col0 + (lane & 31);
    f32x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = PERM ? (k0 + 8 * (e >> 2) + 4 * h + (e & 3)) : (k0 + 8 * h + e);
      out[e] = base[Tile<T, D>::off(row, col)];
    }
    return out;
  }
}

// Per-lane element offsets of every fragment a kernel reads from a Tile<T, D>,
// computed once.  The parts of a fragment address that vary inside the loops
// (the 32-row tile index of a row fragment, the 16-row block of a column
// fragment, the double-buffer slot) are multiples of whole rows, which the
// swizzle does not see, so they stay compile-time immediates of the LDS
// instructions.
//   row(base, r32, c): row fragment of row 32*r32 + (lane % 32), columns
//                      16c + 8h .. +7 (h = lane / 32)
//   col(base, k0, dt): PERM column fragment of rows k0.. (k0 a multiple of
//                      16), columns 32*dt + (lane % 32)
template <typename T, int D>
struct FragAddr;

template <int D>
struct FragAddr<bf16, D> {
  using TL = Tile<bf16, D>;
  static constexpr int NC = D / 16, NDT = D / 32;
  int rofs[NC];
  int cofs[2][NDT];
  __device__ __forceinline__ void init(int lane) {
    const int h = lane >> 5, n = lane & 31;
    const int g = lane >> 4, r = (lane >> 2) & 3, s = lane & 3;
#pragma unroll
    for (int c = 0; c < NC; ++c) rofs[c] = TL::off(n, 16 * c + 8 * h);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) cofs[t][dt] = TL::off(8 * t + 4 * h + r, 32 * dt + 16 * (g & 1) + 4 * s);
  }
  __device__ __forceinline__ bf16x8 row(const bf16* base, int r32, int c) const {
    return ld8(base + rofs[c] + 32 * r32 * D);
  }
  __device__ __forceinline__ bf16x8 col(const bf16* base, int k0, int dt) const {
    bf16x8 out;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16* p = base + cofs[t][dt] + k0 * D;
      s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
      bf16x4 vb = __builtin_bit_cast(bf16x4, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * t + e] = vb[e];
    }
    return out;
  }
};

// fp32 (parity path): addresses computed at each use.
template <int D>
struct FragAddr<float, D> {
  int lane_;
  __device__ __forceinline__ void init(int lane) { lane_ = lane; }
  __device__ __forceinline__ f32x8 row(const float* base, int r32, int c) const {
    return ld_row_frag<float, D>(base, 32 * r32 + (lane_ & 31), 16 * c + 8 * (lane_ >> 5));
  }
  __device__ __forceinline__ f32x8 col(const float* base, int k0, int dt) const {
    return ld_col_frag<true, float, D>(base, k0, 32 * dt, lane_);
  }
};

// Store 4 consecutive values (converted to T) at p.
__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// Exchange with the lane 32 apart: returns {x, partner} in some order, so
// max/sum of the pair is the same on both halves.
__device__ __forceinline__ float pair_max(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// One global_load_lds_dwordx4: every active lane copies 16 bytes from its
// `src` to dst + 16 * lane, where dst (wave-uniform) goes in M0.  Issued
// through asm so that the compiler's LDS-DMA tracking, which cannot tell the
// pipeline stages apart and would wait for every copy in flight before any
// LDS read, stays out; callers wait with explicit vmcnt before a barrier.
// M0 is reserved to the compiler, which on gfx950 sets it only right before
// the few instructions that read it (none of which these kernels use), so
// overwriting it here is safe; the clobber entry documents it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)(dst));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(m0), "v"(src)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// One global_load_lds_dwordx4 in its scalar-base form: every active lane
// copies the 16 bytes at base + off (base wave-uniform in SGPRs, off a
// 32-bit per-lane byte offset) to LDS address m0 + 16 * lane.  Same
// synchronisation contract as dma16.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16s(const void* base, unsigned off, unsigned m0) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(m0), "v"(off), "s"(base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)(p);
}

// Direct HBM -> LDS copy (global_load_lds_dwordx4) of rows [r0, r0+R) of a
// row-major [nrows][D] array into a swizzled Tile<T, D>.  Each instruction
// moves 64 lanes x 16 bytes into a contiguous 1 KB span of LDS (lane l
// writes bytes 16l..16l+15 of the span), so lane l of wave w, instruction u,
// fills physical chunk P = (u*NW + w)*64 + l and loads the global chunk that
// the swizzle maps there.  The source is addressed as a scalar row base plus
// a loop-invariant per-lane byte offset, so a block's copies cost no vector
// address arithmetic.  Rows >= nrows re-read row nrows-1 (finite data the
// kernels mask out).  Completion is tracked by the wave's vmcnt; the data is
// visible to other waves after a workgroup barrier.
template <typename T, int R, int D, int NT>
struct TileDma {
  static constexpr int EPC = 16 / sizeof(T);
  static constexpr int CPR = D / EPC;
  static constexpr int NW = NT / 64;
  static constexpr int RB = D * (int)sizeof(T);  // bytes per row
  static constexpr int TOTAL = R * CPR;
  static_assert(TOTAL % NT == 0, "tile must split evenly over the threads");
  static constexpr int PER = TOTAL / NT;  // instructions per thread per tile
  unsigned voff[PER];                     // byte offset of this lane's chunk from row r0
  int prow[PER];                          // tile row of that chunk
  int wu;                                 // wave index, wave-uniform
  __device__ __forceinline__ void init(int tid) {
    const int lane = tid & 63;
    wu = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int P = (u * NW + wu) * 64 + lane;
      const int row = P / CPR, pc = P % CPR;
      prow[u] = row;
      voff[u] = (unsigned)(row * RB + Tile<T, D>::logical(row, pc) * 16);
    }
  }
  // Requires r0 < nrows.
  __device__ __forceinline__ void issue(const T* g, int r0, int nrows, const T* lds, int /*tid*/) const {
    const char* base = reinterpret_cast<const char*>(g) + (size_t)r0 * RB;
    const unsigned dst = lds_addr(lds);
    const bool inside = r0 + R <= nrows;
    const int last = nrows - 1 - r0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      unsigned off = voff[u];
      if (!inside) off -= (unsigned)((prow[u] - min(prow[u], last)) * RB);
      dma16s(base, off, dst + (unsigned)((u * NW + wu) * 64 * 16));
    }
  }
};

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// instructions (lgkmcnt(0)) but not for its outstanding global loads, so
// direct-to-LDS copies of later pipeline stages stay in flight across it.
// (A fenced barrier would also wait for every outstanding LDS DMA.)  The
// empty asm statements keep the compiler from moving memory accesses across.
// Callers wait for the DMA a stage needs with an explicit vmcnt before it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediate for vmcnt(n) (n < 64) with expcnt and lgkmcnt unconstrained.
__device__ __forceinline__ constexpr int wait_vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Waits until at most min(K, avail) blocks of PER copy instructions each are
// still pending for this wave (vmcnt takes an immediate, so the run-time
// count selects among the compile-time ones).
template <int K, int PER>
__device__ __forceinline__ void wait_blocks(int avail) {
  if constexpr (K <= 0) {
    __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(0));
  } else {
    static_assert(K * PER < 64, "vmcnt holds at most 63");
    if (avail >= K) __builtin_amdgcn_s_waitcnt(wait_vmcnt_imm(K * PER));
    else wait_blocks<K - 1, PER>(avail);
  }
}

// f(std::integral_constant<int, J>()) for J = 0 .. N-1, unrolled.
template <int N, typename F, int... J>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>()), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>());
}

__device__ __forceinline__ int clamp_len(const int32_t* seqlens, int b, int N) {
  if (!seqlens) return N;
  int L = seqlens[b];
  return L < 0 ? 0 : (L > N ? N : L);
}

}  // namespace fa
