// Roofline calibration microbenchmarks for gfx950 (a standalone executable, not part of
// libattn.so).  Each kernel runs a fixed, bounded amount of work per wave over the whole chip;
// rates are derived from hipEvent timings.  Results feed the roofline figures used to judge the
// attention forward kernel: dense bf16 MFMA rate, v_exp_f32 and v_fma_f32 issue rates, whether
// transcendental and MFMA work overlap on one SIMD, LDS read bandwidth and HBM copy bandwidth.
//
//   make micro && ./micro
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                               \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));          \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

constexpr int kIters = 4096;

// 4 independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave.
__global__ __launch_bounds__(256) void mfma_rate(float *out, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (threadIdx.x + i));
    b[i] = (__bf16)(seed * (i + 1));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < kIters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == 1234.5f) out[threadIdx.x] = s;
}

// The same MFMA stream, 4x longer, with the shader clock measured inside the kernel: thread 0 of
// each workgroup records the elapsed s_memtime cycles (core clock) and s_memrealtime ticks
// (constant wall clock) around its loop.
__global__ __launch_bounds__(256) void mfma_clock(unsigned long long *clk, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (threadIdx.x + i));
    b[i] = (__bf16)(seed * (i + 1));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < 4 * kIters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = (r1 - r0) + (s == 1234.5f);
  }
}

// 8 independent chains of v_exp_f32 per lane.
__global__ __launch_bounds__(256) void exp_rate(float *out, float seed) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i) * 1e-3f;
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) - 1.0f;
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  if (s == 1234.5f) out[threadIdx.x] = s;
}

// 8 independent chains of v_fma_f32 per lane.
__global__ __launch_bounds__(256) void fma_rate(float *out, float seed) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i);
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], 0.999f, 0.001f);
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  if (s == 1234.5f) out[threadIdx.x] = s;
}

// Even waves run the MFMA loop, odd waves the exp loop: two waves share each SIMD.
__global__ __launch_bounds__(512) void mixed_rate(float *out, float seed) {
  const int wave = threadIdx.x >> 6;
  float s = 0.f;
  if (wave & 1) {
    float x[8];
    for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i) * 1e-3f;
    for (int it = 0; it < kIters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) - 1.0f;
    }
    for (int i = 0; i < 8; ++i) s += x[i];
  } else {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(seed * (threadIdx.x + i));
      b[i] = (__bf16)(seed * (i + 1));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < kIters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  }
  if (s == 1234.5f) out[threadIdx.x] = s;
}

// ds_read_b128 from a 32 KB LDS array: each lane reads a 16-byte chunk of its own row (pitch
// 272 bytes, the forward kernel's K layout), 8 reads per iteration at different offsets.
__global__ __launch_bounds__(256) void lds_rate(float *out, float seed) {
  __shared__ __attribute__((aligned(16))) float lds[64 * 68];
  for (int i = threadIdx.x; i < 64 * 68; i += 256) lds[i] = seed * i;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const float *base = &lds[(lane & 31) * 68 + (lane >> 5) * 4];
  f32x4 acc = {};
  for (int it = 0; it < kIters; ++it) {
    asm volatile("" ::: "memory");  // the reads are loop-invariant: force them every iteration
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x4 v = *(const f32x4 *)(base + 8 * k + ((it & 1) << 11));
      acc += v;
    }
  }
  if (acc[0] + acc[1] + acc[2] + acc[3] == 1234.5f) out[threadIdx.x] = acc[0];
}

// Dependent v_fma_f32 chain in one wave (latency): 64 dependent FMAs per iteration.
__global__ __launch_bounds__(64) void fma_latency(float *out, float seed) {
  float x = seed * threadIdx.x;
  for (int it = 0; it < kIters / 16; ++it) {
#pragma unroll
    for (int i = 0; i < 64; ++i) x = fmaf(x, 0.999f, 0.001f);
  }
  if (x == 1234.5f) out[threadIdx.x] = x;
}

// Interleaved independent exp and fma chains in one wave: do the transcendental and FMA work
// overlap?
__global__ __launch_bounds__(256) void expfma_rate(float *out, float seed) {
  float x[8], y[8];
  for (int i = 0; i < 8; ++i) {
    x[i] = seed * (threadIdx.x + i) * 1e-3f;
    y[i] = seed * (threadIdx.x + 2 * i);
  }
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = __builtin_amdgcn_exp2f(x[i]);
      y[i] = fmaf(y[i], 0.999f, 0.001f);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i] + y[i];
  if (s == 1234.5f) out[threadIdx.x] = s;
}

// Even waves MFMA, odd waves FMA.
__global__ __launch_bounds__(512) void mixed_fma(float *out, float seed) {
  const int wave = threadIdx.x >> 6;
  float s = 0.f;
  if (wave & 1) {
    float x[8];
    for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i);
    for (int it = 0; it < kIters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i], 0.999f, 0.001f);
    }
    for (int i = 0; i < 8; ++i) s += x[i];
  } else {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(seed * (threadIdx.x + i));
      b[i] = (__bf16)(seed * (i + 1));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < kIters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  }
  if (s == 1234.5f) out[threadIdx.x] = s;
}

// Read-only stream: 8 independent 16-byte loads in flight per lane, XOR-folded.
__global__ __launch_bounds__(256) void read_kernel(const f32x4 *__restrict__ src, size_t n,
                                                   float *out) {
  constexpr int UN = 8;
  f32x4 acc = {};
  const size_t stride = (size_t)gridDim.x * 256 * UN;
  for (size_t base = (size_t)blockIdx.x * 256 * UN + threadIdx.x; base < n; base += stride) {
    f32x4 v[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) v[u] = (base + u * 256 < n) ? src[base + u * 256] : f32x4{};
#pragma unroll
    for (int u = 0; u < UN; ++u) acc += v[u];
  }
  if (acc[0] + acc[1] + acc[2] + acc[3] == 1234.5f) out[blockIdx.x & 4095] = acc[0];  // out holds 4096 floats
}

// 4 KB blocks (256 x 16 bytes) read in the order perm gives, one workgroup per block.
__global__ __launch_bounds__(256) void read_blocks_kernel(const f32x4 *__restrict__ src,
                                                          const int *perm, int nblk, float *out) {
  f32x4 acc = {};
  for (int bb = blockIdx.x; bb < nblk; bb += gridDim.x) acc += src[(size_t)perm[bb] * 256 + threadIdx.x];
  if (acc[0] + acc[1] + acc[2] + acc[3] == 1234.5f) out[blockIdx.x & 4095] = acc[0];  // out holds 4096 floats
}

__global__ __launch_bounds__(256) void copy_kernel(const f32x4 *__restrict__ src,
                                                   f32x4 *__restrict__ dst, size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    dst[i] = src[i];
}

template <typename F>
float time_ms(F launch, int reps) {
  hipEvent_t a, b;
  CHECK(hipEventCreate(&a));
  CHECK(hipEventCreate(&b));
  launch();
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(a));
  for (int r = 0; r < reps; ++r) launch();
  CHECK(hipEventRecord(b));
  CHECK(hipEventSynchronize(b));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, a, b));
  CHECK(hipEventDestroy(a));
  CHECK(hipEventDestroy(b));
  return ms / reps;
}

int main() {
  hipDeviceProp_t p;
  CHECK(hipGetDeviceProperties(&p, 0));
  const int cus = p.multiProcessorCount;
  printf("device %s, %d CUs, clock %.0f MHz\n", p.gcnArchName, cus, p.clockRate / 1e3);
  float *out;
  CHECK(hipMalloc(&out, 4096 * sizeof(float)));
  const float seed = 1e-3f;

  // One workgroup of 4 waves per CU -> 1 wave per SIMD; 2 per CU -> 2 waves per SIMD.
  for (int wg_per_cu = 1; wg_per_cu <= 2; ++wg_per_cu) {
    const int grid = cus * wg_per_cu * 8;
    float ms = time_ms([&] { mfma_rate<<<grid, 256>>>(out, seed); }, 5);
    const double flops = (double)grid * 4 * kIters * 4 * 32768.0;
    printf("mfma bf16 32x32x16, %d wave/SIMD: %.1f TFLOP/s (%.2f cycles/MFMA/SIMD at 2.4 GHz)\n",
           wg_per_cu, flops / ms / 1e9, ms * 1e-3 * 2.4e9 / ((double)grid * 4 * kIters * 4 / (cus * 4)));
    ms = time_ms([&] { exp_rate<<<grid, 256>>>(out, seed); }, 5);
    double ops = (double)grid * 256 * kIters * 8;
    printf("v_exp_f32, %d wave/SIMD: %.1f Gop/s = %.2f lane-ops/clk/CU at 2.4 GHz\n", wg_per_cu,
           ops / ms / 1e6, ops / (ms * 1e-3) / 2.4e9 / cus);
    ms = time_ms([&] { fma_rate<<<grid, 256>>>(out, seed); }, 5);
    printf("v_fma_f32, %d wave/SIMD: %.1f Gop/s = %.2f lane-ops/clk/CU at 2.4 GHz\n", wg_per_cu,
           ops / ms / 1e6, ops / (ms * 1e-3) / 2.4e9 / cus);
  }
  // The core clock under sustained MFMA load (one wave per SIMD), from inside the kernel.
  {
    int wall_khz = 0;
    CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0));
    const int grid = cus;
    unsigned long long *clk;
    CHECK(hipMalloc(&clk, 2 * grid * sizeof(unsigned long long)));
    const float ms = time_ms([&] { mfma_clock<<<grid, 256>>>(clk, seed); }, 3);
    std::vector<unsigned long long> h(2 * grid);
    CHECK(hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
    std::vector<double> mhz, cyc;
    for (int g = 0; g < grid; ++g) {
      mhz.push_back((double)h[2 * g] / (double)h[2 * g + 1] * wall_khz / 1e3);
      cyc.push_back((double)h[2 * g] / (4.0 * kIters * 4));
    }
    std::sort(mhz.begin(), mhz.end());
    std::sort(cyc.begin(), cyc.end());
    const double flops = (double)grid * 4 * 4 * kIters * 4 * 32768.0;
    printf("core clock under MFMA load (s_memtime / s_memrealtime at %d kHz): median %.0f MHz "
           "(min %.0f, max %.0f); %.2f core cycles per 32x32x16 MFMA; %.1f TFLOP/s\n",
           wall_khz, mhz[grid / 2], mhz[0], mhz[grid - 1], cyc[grid / 2], flops / ms / 1e9);
    CHECK(hipFree(clk));
  }
  // Throughput-bound VALU: 4 waves per SIMD (four 256-thread workgroups per CU).
  {
    const int grid = cus * 4;
    float ms = time_ms([&] { fma_rate<<<grid * 4, 256>>>(out, seed); }, 5);
    double ops = (double)grid * 1024 * kIters * 8;
    printf("v_fma_f32, 4 wave/SIMD: %.2f lane-ops/clk/CU (%.2f cycles per wave64 instruction per SIMD)\n",
           ops / (ms * 1e-3) / 2.4e9 / cus, 64.0 * 4 / (ops / (ms * 1e-3) / 2.4e9 / cus));
    ms = time_ms([&] { exp_rate<<<grid * 4, 256>>>(out, seed); }, 5);
    printf("v_exp_f32 (+1 sub each), 4 wave/SIMD: %.2f exp lane-ops/clk/CU\n", ops / (ms * 1e-3) / 2.4e9 / cus);
    ms = time_ms([&] { expfma_rate<<<grid * 4, 256>>>(out, seed); }, 5);
    printf("exp + fma interleaved, 4 wave/SIMD: %.2f (exp+fma) lane-ops/clk/CU\n", 2 * ops / (ms * 1e-3) / 2.4e9 / cus);
    ms = time_ms([&] { fma_latency<<<cus * 4, 64>>>(out, seed); }, 3);
    printf("dependent v_fma_f32 chain, 1 wave: %.2f cycles per FMA\n", ms * 1e-3 * 2.4e9 / ((double)(kIters / 16) * 64));
  }
  {
    const int grid = cus * 8;
    const float ms_mf = time_ms([&] { mixed_fma<<<grid, 512>>>(out, seed); }, 5);
    const float ms_f = time_ms([&] { fma_rate<<<grid, 256>>>(out, seed); }, 5);
    const float ms_mm = time_ms([&] { mfma_rate<<<grid, 256>>>(out, seed); }, 5);
    printf("overlap: mfma wave + fma wave per SIMD %.3f ms vs mfma alone %.3f ms, fma alone %.3f ms\n",
           ms_mf, ms_mm, ms_f);
  }
  {
    const int grid = cus * 8;
    const float ms_mix = time_ms([&] { mixed_rate<<<grid, 512>>>(out, seed); }, 5);
    const float ms_m = time_ms([&] { mfma_rate<<<grid, 256>>>(out, seed); }, 5);
    const float ms_e = time_ms([&] { exp_rate<<<grid, 256>>>(out, seed); }, 5);
    printf("overlap: mfma wave + exp wave per SIMD %.3f ms vs mfma alone %.3f ms, exp alone %.3f "
           "ms (sum %.3f)\n", ms_mix, ms_m, ms_e, ms_m + ms_e);
  }
  {
    const int grid = cus * 2 * 8;
    const float ms = time_ms([&] { lds_rate<<<grid, 256>>>(out, seed); }, 5);
    const double bytes = (double)grid * 256 * kIters * 8 * 16;
    printf("LDS ds_read_b128: %.1f TB/s = %.1f B/clk/CU at 2.4 GHz\n", bytes / ms / 1e9,
           bytes / (ms * 1e-3) / 2.4e9 / cus);
  }
  {
    const size_t n = (size_t)1 << 26;  // 1 GiB of f32x4
    f32x4 *a, *b;
    CHECK(hipMalloc(&a, n * sizeof(f32x4)));
    CHECK(hipMalloc(&b, n * sizeof(f32x4)));
    CHECK(hipMemset(a, 0, n * sizeof(f32x4)));
    const float ms = time_ms([&] { copy_kernel<<<cus * 16, 256>>>(a, b, n); }, 10);
    printf("HBM copy 1 GiB: %.1f GB/s (read + write)\n", 2.0 * n * sizeof(f32x4) / ms / 1e6);
    const float ms_r = time_ms([&] { read_kernel<<<cus * 8, 256>>>(a, n, out); }, 10);
    printf("HBM read 1 GiB: %.1f GB/s (8 loads in flight per lane)\n", n * sizeof(f32x4) / ms_r / 1e6);
    const int nblk = (int)(n / 256);
    std::vector<int> hp(nblk);
    for (int i = 0; i < nblk; ++i) hp[i] = i;
    unsigned x = 12345u;  // Fisher-Yates with a fixed LCG: a reproducible block order
    for (int i = nblk - 1; i > 0; --i) {
      x = x * 1664525u + 1013904223u;
      std::swap(hp[i], hp[x % (unsigned)(i + 1)]);
    }
    int *perm;
    CHECK(hipMalloc(&perm, nblk * sizeof(int)));
    CHECK(hipMemcpy(perm, hp.data(), nblk * sizeof(int), hipMemcpyHostToDevice));
    const float ms_p = time_ms([&] { read_blocks_kernel<<<cus * 32, 256>>>(a, perm, nblk, out); }, 10);
    printf("HBM read 1 GiB as 4 KB blocks in a random order: %.1f GB/s\n",
           n * sizeof(f32x4) / ms_p / 1e6);
    CHECK(hipFree(perm));
    CHECK(hipFree(a));
    CHECK(hipFree(b));
  }
  CHECK(hipFree(out));
  return 0;
}
