// Calibration microbenchmarks for the rooflines the attention kernels are
// measured against, run on the GPU at hand (device 0).  Prints one JSON line.
//
//   mfma      independent v_mfma_f32_32x32x16_bf16 chains: sustained bf16 dense
//             matrix rate (the ceiling a real kernel can approach)
//   exp, fma  independent v_exp_f32 / v_fma_f32 chains: vector-ALU rates of the
//             softmax's two kinds of instruction
//   mix       one wave alternating one product with four exponentials (no data
//             dependence between them): how far the matrix core and the vector
//             ALU overlap inside a wave
//   split     the same work in 8-wave groups, waves 0-3 doing only products and
//             waves 4-7 only exponentials; waves w and w+4 share SIMD w, so
//             this is how far two waves of one SIMD overlap the two pipes
//   lds_frag  the attention kernels' LDS fragment reads on a swizzled
//             128 x 64 bf16 tile, 2 four-wave groups per CU: row fragments
//             (ds_read_b128) and transposed column fragments
//             (ds_read_b64_tr_b16), bytes per ns per CU
//   mfma_lds  8-wave groups, waves 0-3 products, waves 4-7 conflict-free
//             ds_read_b128 reads: whether LDS reads slow the products of
//             another wave on the same SIMD
//   placement where a 1536-group launch lands: XCD of group g (hardware
//             register) against g % 8, and whether g and g + 256 share a
//             compute unit
//   lds       ds_read_b128 from conflict-free addresses: LDS read bandwidth
//   copy      1 GiB device-to-device copy: HBM bandwidth (read + write bytes)
//   atomic    device-scope float atomic adds spread over 32 MiB: the rate a
//             dQ reduction by atomics would have to live with
//
// Every kernel indexes its buffers inside their sizes (checked on the host
// against the grid before launch) and every loop has a fixed trip count.
#include <hip/hip_runtime.h>

#include "fa_common.h"

#include <algorithm>
#include <utility>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

#define CHECK(x)                                                                          \
  do {                                                                                    \
    hipError_t e_ = (x);                                                                  \
    if (e_ != hipSuccess) {                                                               \
      std::printf("{\"error\": \"%s at %s:%d\"}\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      std::exit(1);                                                                       \
    }                                                                                     \
  } while (0)

__device__ __forceinline__ bf16x8 frag(float seed) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (__bf16)(seed * (float)(i + 1));
  return f;
}

__device__ __forceinline__ float sum16(const f32x16& c) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c[i];
  return s;
}

// 8 products per iteration on 4 independent accumulators.
__global__ __launch_bounds__(kThreads) void k_mfma(float* out, int iters, float seed) {
  const bf16x8 a = frag(seed), b = frag(seed * 0.5f);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  out[blockIdx.x * kThreads + threadIdx.x] = sum16(c0) + sum16(c1) + sum16(c2) + sum16(c3);
}

// 32 vector instructions per iteration on 8 independent registers.
template <bool EXP>
__global__ __launch_bounds__(kThreads) void k_valu(float* out, int iters, float seed) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = -seed * (float)(i + 1);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = EXP ? __builtin_amdgcn_exp2f(x[i]) : fmaf(x[i], 0.999f, seed);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

// Issue order is fixed with volatile asm: the compiler would otherwise group
// the products.  No instruction reads a register another one in flight writes,
// except a product's accumulator by the next product on it (the matrix core
// forwards that), and the accumulators are read only after the trailing nops.
#define MF(c) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b))
#define EX(x) asm volatile("v_exp_f32 %0, %0" : "+v"(x))

// MODE 0: each wave alternates 1 product and 4 exponentials (8 and 32 per
// iteration).  MODE 1: even waves 16 products, odd waves 64 exponentials per
// iteration (the same total work per pair of waves).
template <int MODE>
__global__ __launch_bounds__(2 * kThreads) void k_overlap(float* out, int iters, float seed) {
  const bf16x8 a = frag(seed), b = frag(seed * 0.5f);
  f32x16 c0 = {}, c1 = {};
  float e0 = -seed, e1 = -2 * seed, e2 = -3 * seed, e3 = -4 * seed, e4 = -5 * seed, e5 = -6 * seed,
        e6 = -7 * seed, e7 = -8 * seed;
  const bool odd = MODE == 1 ? (threadIdx.x >> 6) >= 4 : false;  // MODE 1: 8-wave groups, waves 4-7
  for (int it = 0; it < iters; ++it) {
    if (MODE == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        MF(c0); EX(e0); EX(e1); EX(e2); EX(e3);
        MF(c1); EX(e4); EX(e5); EX(e6); EX(e7);
      }
    } else if (odd) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        EX(e0); EX(e1); EX(e2); EX(e3); EX(e4); EX(e5); EX(e6); EX(e7);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) { MF(c0); MF(c1); }
    }
  }
  // The products' results are read only after these wait states.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1));
  out[blockIdx.x * blockDim.x + threadIdx.x] = e0 + e1 + e2 + e3 + e4 + e5 + e6 + e7 + sum16(c0) + sum16(c1);
}

// 8 ds_read_b128 per iteration per lane from a 64 KiB buffer; lanes read
// consecutive 16-byte chunks, so every read is conflict-free.
__global__ __launch_bounds__(kThreads) void k_lds(unsigned* out, int iters) {
  __shared__ uint4 buf[4096];
  for (int i = threadIdx.x; i < 4096; i += kThreads) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint4 v = buf[(threadIdx.x + r * kThreads + it * 64) & 4095];
      acc.x ^= v.x;
      acc.y += v.y;
      acc.z ^= v.z;
      acc.w += v.w;
    }
  }
  out[blockIdx.x * kThreads + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

// LDS fragment reads as the attention kernels issue them: a swizzled
// 128 x 64 bf16 tile (fa::Tile), ROW = 8 row fragments (ds_read_b128) or
// COL = 16 transposed reads (ds_read_b64_tr_b16) per iteration, every address
// a fa::FragAddr offset inside the tile.
template <bool ROW>
__global__ __launch_bounds__(kThreads, 2) void k_lds_frag(float* out, int iters) {
  __shared__ __attribute__((aligned(16))) fa::bf16 tile[2 * 128 * 64];
  for (int i = threadIdx.x; i < 2 * 128 * 64; i += kThreads) tile[i] = (fa::bf16)(float)((i * 7) % 13);
  __syncthreads();
  fa::FragAddr<fa::bf16, 64> fr;
  fr.init(threadIdx.x & 63);
  float acc = 0.f;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");  // keep the reads inside the loop
    fa::bf16x8 x = {};
    const int q = it & 3;
    if (ROW) {
#pragma unroll
      for (int c = 0; c < 4; ++c) { x += fr.row(tile, q, c); x += fr.row(tile + 128 * 64, q, c); }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) { x += fr.col(tile, 32 * q + 16 * cc, t); x += fr.col(tile + 128 * 64, 32 * q + 16 * cc, t); }
    }
    acc += (float)x[0] + (float)x[7];
  }
  out[blockIdx.x * kThreads + threadIdx.x] = acc;
}

// 8-wave groups: waves 0-3 issue independent products (MODE 0 and 1), waves
// 4-7 conflict-free ds_read_b128 (MODE 1 and 2).
template <int MODE>
__global__ __launch_bounds__(2 * kThreads) void k_mfma_lds(float* out, int iters, float seed) {
  __shared__ uint4 buf[1024];
  for (int i = threadIdx.x; i < 1024; i += 2 * kThreads) buf[i] = make_uint4(i, i + 1, i + 2, i + 3);
  __syncthreads();
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float r = 0.f;
  if (w < 4 && MODE != 2) {
    const bf16x8 a = frag(seed), b = frag(seed * 0.5f);
    f32x16 c0 = {}, c1 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 4; ++u) { MF(c0); MF(c1); }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c0), "+v"(c1));
    r = sum16(c0) + sum16(c1);
  } else if (w >= 4 && MODE != 0) {
    uint4 acc = make_uint4(0, 0, 0, 0);
    for (int it = 0; it < iters; ++it) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint4 v = buf[(lane + 64 * j + it) & 1023];
        acc.x ^= v.x; acc.y += v.y; acc.z ^= v.z; acc.w += v.w;
      }
    }
    r = (float)(acc.x + acc.y + acc.z + acc.w);
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}
#undef MF
#undef EX

// Placement: each group records its XCD id and hardware id (SE, SH, CU
// fields) and spins for a fixed number of clocks so that all groups of the
// launch are resident together, as the first round of a real launch is.
__global__ __launch_bounds__(kThreads) void k_place(uint2* out, long long spin) {
  unsigned xcc, hwid;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hwid));
  const long long t0 = clock64();
  while (clock64() - t0 < spin) {
  }
  if (threadIdx.x == 0) out[blockIdx.x] = make_uint2(xcc, hwid);
}

__global__ __launch_bounds__(kThreads) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads) dst[i] = src[i];
}

// Each thread adds `per` values; consecutive lanes hit consecutive words, as a
// dQ tile's lanes would.
__global__ __launch_bounds__(kThreads) void k_atomic(float* acc, size_t words, int per) {
  const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (int j = 0; j < per; ++j) unsafeAtomicAdd(acc + (t + (size_t)j * stride) % words, 1.0f);
}

template <typename F>
float time_ms(F&& launch, int reps = 5) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  launch();  // warm-up
  CHECK(hipGetLastError());
  std::vector<float> t;
  for (int r = 0; r < reps; ++r) {
    CHECK(hipEventRecord(e0));
    launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    t.push_back(ms);
  }
  CHECK(hipGetLastError());
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  std::sort(t.begin(), t.end());
  return t[t.size() / 2];
}

}  // namespace

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const int waves_per_simd = 2;
  const int grid = cus * waves_per_simd;  // 4-wave workgroups: waves_per_simd waves on each SIMD
  const long long waves = (long long)grid * (kThreads / 64);
  const long long simds = 4LL * cus;
  float* out = nullptr;
  CHECK(hipMalloc(&out, (size_t)grid * kThreads * sizeof(float)));  // one word per thread of every kernel below

  const int it_m = 4000, it_v = 4000, it_o = 2000, it_l = 4000;
  const float t_mfma = time_ms([&] { hipLaunchKernelGGL(k_mfma, dim3(grid), dim3(kThreads), 0, 0, out, it_m, 1e-3f); });
  const float t_exp = time_ms([&] { hipLaunchKernelGGL(k_valu<true>, dim3(grid), dim3(kThreads), 0, 0, out, it_v, 1e-3f); });
  const float t_fma = time_ms([&] { hipLaunchKernelGGL(k_valu<false>, dim3(grid), dim3(kThreads), 0, 0, out, it_v, 1e-3f); });
  const float t_mix = time_ms([&] { hipLaunchKernelGGL(k_overlap<0>, dim3(grid), dim3(kThreads), 0, 0, out, it_o, 1e-3f); });
  // split: one 8-wave group per CU (waves_per_simd = 2 waves on each SIMD, one of each kind)
  const float t_split = time_ms([&] { hipLaunchKernelGGL(k_overlap<1>, dim3(cus), dim3(2 * kThreads), 0, 0, out, it_o, 1e-3f); });
  const int it_f = 4000;
  const float t_row = time_ms([&] { hipLaunchKernelGGL(k_lds_frag<true>, dim3(grid), dim3(kThreads), 0, 0, out, it_f); });
  const float t_col = time_ms([&] { hipLaunchKernelGGL(k_lds_frag<false>, dim3(grid), dim3(kThreads), 0, 0, out, it_f); });
  const double frag_bytes = (double)grid * kThreads * it_f * 128;  // 128 bytes per lane per iteration in both kinds
  const int it_ml = 8000;
  const float t_ml_p = time_ms([&] { hipLaunchKernelGGL(k_mfma_lds<0>, dim3(cus), dim3(2 * kThreads), 0, 0, out, it_ml, 1e-3f); });
  const float t_ml_b = time_ms([&] { hipLaunchKernelGGL(k_mfma_lds<1>, dim3(cus), dim3(2 * kThreads), 0, 0, out, it_ml, 1e-3f); });
  const float t_ml_l = time_ms([&] { hipLaunchKernelGGL(k_mfma_lds<2>, dim3(cus), dim3(2 * kThreads), 0, 0, out, it_ml, 1e-3f); });

  const int pgrid = 6 * cus;
  uint2* place = nullptr;
  CHECK(hipMalloc(&place, (size_t)pgrid * sizeof(uint2)));
  hipLaunchKernelGGL(k_place, dim3(pgrid), dim3(kThreads), 0, 0, place, 2000000LL);
  CHECK(hipGetLastError());
  std::vector<uint2> ph(pgrid);
  CHECK(hipMemcpy(ph.data(), place, (size_t)pgrid * sizeof(uint2), hipMemcpyDeviceToHost));
  CHECK(hipFree(place));
  // HW_ID fields: CU bits 11:8, SH bit 12, SE bits 15:13 (identify a CU within its XCD)
  auto cu_of = [&](int g) { return std::make_pair(ph[g].x, (ph[g].y >> 8) & 0xff); };
  int xcd_mod8 = 0, same_cu = 0;
  for (int g = 0; g < pgrid; ++g) xcd_mod8 += (int)ph[g].x == g % 8;
  for (int g = 0; g + 256 < pgrid; ++g) same_cu += cu_of(g) == cu_of(g + 256);
  const float t_lds = time_ms([&] { hipLaunchKernelGGL(k_lds, dim3(grid), dim3(kThreads), 0, 0, reinterpret_cast<unsigned*>(out), it_l); });

  // Products per wave: it*8; exponentials per wave: it*32 (mix and split alike).
  const double mfma_flops = (double)waves * it_m * 8 * (2.0 * 32 * 32 * 16);
  const double mfma_ns = t_mfma * 1e6 / ((double)waves / simds * it_m * 8);        // per product per SIMD
  const double exp_ns = t_exp * 1e6 / ((double)waves / simds * it_v * 32);          // per wave instruction per SIMD
  const double fma_ns = t_fma * 1e6 / ((double)waves / simds * it_v * 32);
  const double o_mfma = (double)waves / simds * it_o * 8 * mfma_ns * 1e-6;          // ms the products alone take
  const double o_exp = (double)waves / simds * it_o * 32 * exp_ns * 1e-6;           // ms the exponentials alone take
  const double lds_bytes = (double)grid * kThreads * it_l * 8 * 16;

  const size_t copy_bytes = 1ull << 30;
  const size_t n4 = copy_bytes / sizeof(uint4);
  uint4 *src = nullptr, *dst = nullptr;
  CHECK(hipMalloc(&src, copy_bytes));
  CHECK(hipMalloc(&dst, copy_bytes));
  CHECK(hipMemset(src, 1, copy_bytes));
  const float t_copy = time_ms([&] { hipLaunchKernelGGL(k_copy, dim3(cus * 32), dim3(kThreads), 0, 0, src, dst, n4); });
  CHECK(hipFree(src));
  CHECK(hipFree(dst));

  const size_t words = (32ull << 20) / sizeof(float);
  const int per = 64;
  const int agrid = cus * 16;
  float* acc = nullptr;
  CHECK(hipMalloc(&acc, words * sizeof(float)));
  CHECK(hipMemset(acc, 0, words * sizeof(float)));
  const float t_atomic = time_ms([&] { hipLaunchKernelGGL(k_atomic, dim3(agrid), dim3(kThreads), 0, 0, acc, words, per); });
  const double atomics = (double)agrid * kThreads * per;
  CHECK(hipFree(acc));
  CHECK(hipFree(out));

  std::printf(
      "{\"device\": \"%s\", \"compute_units\": %d, \"waves_per_simd\": %d, "
      "\"mfma_bf16_tflops\": %.1f, \"mfma_ns_per_product\": %.3f, "
      "\"exp_ns_per_wave_instr\": %.3f, \"fma_ns_per_wave_instr\": %.3f, "
      "\"mix_over_longer\": %.3f, \"split_over_longer\": %.3f, "
      "\"lds_read_tbs\": %.1f, \"lds_bytes_per_cu_ns\": %.1f, "
      "\"lds_row_frag_bytes_per_cu_ns\": %.1f, \"lds_col_frag_bytes_per_cu_ns\": %.1f, "
      "\"mfma_with_lds_reader_over_longer\": %.3f, "
      "\"placement\": {\"groups\": %d, \"xcd_is_group_mod_8\": %.4f, \"group_and_group_plus_256_share_cu\": %.4f}, "
      "\"hbm_copy_tbs\": %.2f, \"atomic_f32_gops\": %.1f, "
      "\"ms\": {\"mfma\": %.4f, \"exp\": %.4f, \"fma\": %.4f, \"mix\": %.4f, \"split\": %.4f, \"lds\": %.4f, "
      "\"copy\": %.4f, \"atomic\": %.4f, \"lds_row_frag\": %.4f, \"lds_col_frag\": %.4f, "
      "\"mfma_alone\": %.4f, \"lds_alone\": %.4f, \"mfma_with_lds\": %.4f}}\n",
      prop.gcnArchName, cus, waves_per_simd, mfma_flops / (t_mfma * 1e9), mfma_ns, exp_ns, fma_ns,
      t_mix / std::max(o_mfma, o_exp), t_split / std::max(o_mfma, o_exp), lds_bytes / (t_lds * 1e9),
      lds_bytes / (t_lds * 1e6) / cus, frag_bytes / (t_row * 1e6) / cus, frag_bytes / (t_col * 1e6) / cus,
      t_ml_b / std::max(t_ml_p, t_ml_l), pgrid, (double)xcd_mod8 / pgrid, (double)same_cu / (pgrid - 256),
      2.0 * copy_bytes / (t_copy * 1e9), atomics / (t_atomic * 1e6), t_mfma, t_exp,
      t_fma, t_mix, t_split, t_lds, t_copy, t_atomic, t_row, t_col, t_ml_p, t_ml_l, t_ml_b);
  return 0;
}
