// Roofline calibration microbenchmarks for gfx950 (a standalone executable, not part of
// libattn.so).  Each kernel runs a fixed, bounded amount of work per wave.  The issue-rate
// kernels time themselves in core cycles (s_memtime inside the kernel, the median over the
// workgroups) at a stated number of waves per SIMD: one 4-wave workgroup per CU places one wave
// on each SIMD, so a grid of k workgroups per CU runs k waves per SIMD.  The bandwidth kernels
// are timed with hipEvents.  Results feed the roofline figures used to assess the attention
// forward kernel: the MFMA rate and the core clock under it, the cost of transcendental and FMA
// instructions alone and mixed, the forward kernel's per-score probability work, how matrix-core
// and vector waves share a SIMD, how far one wave overlaps its own MFMAs with vector work, the
// rate of a dependent MFMA chain, LDS read bandwidth and HBM bandwidth.
//
//   make micro && ./micro_bench
#include <hip/hip_runtime.h>

#include <algorithm>
#include <utility>
#include <vector>

#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

#define CHECK(x)                                                               \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));          \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)

constexpr int kIters = 2048;
constexpr int kHwRegSimdId = (4) | (4 << 6) | ((2 - 1) << 11);  // HW_ID bits 4..5: SIMD id

// 4 independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave; core cycles (s_memtime)
// and 100 MHz wall-clock ticks (s_memrealtime) over the loop.
__global__ __launch_bounds__(256) void mfma_cycles(u64 *clk, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (threadIdx.x + i));
    b[i] = (__bf16)(seed * (i + 1));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const u64 t0 = __builtin_amdgcn_s_memtime();
  const u64 r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < kIters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  const u64 t1 = __builtin_amdgcn_s_memtime();
  const u64 r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = (r1 - r0) + (s == 1234.5f);
  }
}

// One loop iteration of vector instructions, written as a single asm block so that the compiler
// keeps the order: 8 independent registers x for transcendentals, 16 independent y for FMAs.
//   KIND 0: 8 v_exp_f32      KIND 1: 8 v_rcp_f32      KIND 2: 16 v_fma_f32
//   KIND 3: 8 x (v_exp_f32, v_fma_f32, v_fma_f32), interleaved
#define VOPS                                                                                    \
  "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),         \
      "+v"(x[7]), "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]),     \
      "+v"(y[6]), "+v"(y[7]), "+v"(y[8]), "+v"(y[9]), "+v"(y[10]), "+v"(y[11]), "+v"(y[12]),  \
      "+v"(y[13]), "+v"(y[14]), "+v"(y[15])
#define T8(op)                                                                                  \
  op " %0, %0\n" op " %1, %1\n" op " %2, %2\n" op " %3, %3\n" op " %4, %4\n" op " %5, %5\n" op \
     " %6, %6\n" op " %7, %7\n"
#define F(r) "v_fma_f32 %" #r ", %" #r ", %24, %25\n"
#define F16 F(8) F(9) F(10) F(11) F(12) F(13) F(14) F(15) F(16) F(17) F(18) F(19) F(20) F(21) F(22) F(23)
#define EFF(e, f0, f1) "v_exp_f32 %" #e ", %" #e "\n" F(f0) F(f1)
#define EFF8                                                                                    \
  EFF(0, 8, 9) EFF(1, 10, 11) EFF(2, 12, 13) EFF(3, 14, 15) EFF(4, 16, 17) EFF(5, 18, 19)       \
  EFF(6, 20, 21) EFF(7, 22, 23)

template <int KIND>
__device__ __forceinline__ void valu_iter(float (&x)[8], float (&y)[16], float fa, float fb) {
  if constexpr (KIND == 0) asm volatile(T8("v_exp_f32") : VOPS : "v"(fa), "v"(fb));
  if constexpr (KIND == 1) asm volatile(T8("v_rcp_f32") : VOPS : "v"(fa), "v"(fb));
  if constexpr (KIND == 2) asm volatile(F16 : VOPS : "v"(fa), "v"(fb));
  if constexpr (KIND == 3) asm volatile(EFF8 : VOPS : "v"(fa), "v"(fb));
}

template <int KIND>
__global__ __launch_bounds__(256) void valu_cycles(float *out, u64 *cyc, float seed) {
  float x[8], y[16];
  for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i) * 1e-3f;
  for (int i = 0; i < 16; ++i) y[i] = seed * (threadIdx.x + 2 * i);
  const u64 t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kIters; ++it) valu_iter<KIND>(x, y, 0.999f, 0.001f);
  const u64 t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int i = 0; i < 8; ++i) s += x[i];
  for (int i = 0; i < 16; ++i) s += y[i];
  if (s == 1234.5f) out[threadIdx.x] = s;
  if (threadIdx.x == 0) cyc[blockIdx.x] = (t1 - t0) / kIters;
}

// Dependent v_fma_f32 chain in one wave (latency): 64 dependent FMAs per iteration.
__global__ __launch_bounds__(64) void fma_latency(float *out, u64 *cyc, float seed) {
  float x = seed * threadIdx.x;
  const u64 t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kIters / 16; ++it) {
#pragma unroll
    for (int i = 0; i < 64; ++i) x = fmaf(x, 0.999f, 0.001f);
  }
  const u64 t1 = __builtin_amdgcn_s_memtime();
  if (x == 1234.5f) out[threadIdx.x] = x;
  if (threadIdx.x == 0) cyc[blockIdx.x] = (t1 - t0) / (kIters / 16 * 64);
}

// The per-score vector work of the forward kernel's softmax phase: 32 independent scores per
// lane per iteration (one lane's share of a 64-key tile), each turned into a probability that is
// summed and packed to fp16 as the P V operand.  SOFTCAP: u = 1 / (1 + 2^(c x)), a running
// minimum of u (the tile maximum of the capped score) and p = 2^(A - B u): three
// transcendentals per score.  Otherwise a running maximum and p = 2^(x - A): one.  The scores
// are made opaque each iteration so that nothing is hoisted out of the loop.
template <bool SOFTCAP>
__global__ __launch_bounds__(256) void prob_chain(float *out, u64 *cyc, float seed) {
  typedef __fp16 h2 __attribute__((ext_vector_type(2)));
  constexpr int kRounds = 512;
  float s[32];
  for (int j = 0; j < 32; ++j) s[j] = seed * (threadIdx.x + j);
  const float c = 0.0961f, A = 43.2f, B = 86.5f;
  float l = 0.f, mx = 0.f;
  const u64 t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kRounds; ++it) {
#pragma unroll
    for (int j = 0; j < 32; ++j) asm volatile("" : "+v"(s[j]));
    float t = SOFTCAP ? __builtin_inff() : -__builtin_inff(), sum = 0.f;
    float p[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (SOFTCAP) {
        const float u = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(s[j] * c));
        t = fminf(t, u);
        p[j] = __builtin_amdgcn_exp2f(fmaf(u, -B, A));
      } else {
        t = fmaxf(t, s[j]);
        p[j] = __builtin_amdgcn_exp2f(s[j] - A);
      }
      sum += p[j];
    }
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
      const h2 pk = __builtin_amdgcn_cvt_pkrtz(p[j], p[j + 1]);
      asm volatile("" ::"v"(pk));
    }
    l += sum;
    mx += t;
  }
  const u64 t1 = __builtin_amdgcn_s_memtime();
  if (l + mx == 1234.5f) out[threadIdx.x] = l;
  if (threadIdx.x == 0) cyc[blockIdx.x] = (t1 - t0) / kRounds;
}

// Two waves per SIMD (one 8-wave workgroup per CU) with different roles: on each SIMD the wave
// with the lower wave number (SIMD id from HW_ID) runs the MFMA loop of mfma_cycles, the other
// one a vector loop (KIND of valu_cycles: 0 exp, 2 fma) for twice as many iterations.  ROLES
// selects which of the two run (1: matrix only, 2: vector only, 3: both).  cyc gets each wave's
// core cycles, with bit 63 set for the matrix role.
template <int KIND, int ROLES>
__global__ __launch_bounds__(512) void pair_cycles(float *out, u64 *cyc, float seed) {
  __shared__ int simd_of[8];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) simd_of[wave] = __builtin_amdgcn_s_getreg(kHwRegSimdId) & 3;
  __syncthreads();
  int rank = 0;
  for (int w = 0; w < wave; ++w) rank += simd_of[w] == simd_of[wave];
  const bool mat = __builtin_amdgcn_readfirstlane(rank) == 0;
  u64 dt = 0;
  float s = 0.f;
  if (mat && (ROLES & 1)) {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(seed * (threadIdx.x + i));
      b[i] = (__bf16)(seed * (i + 1));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const u64 t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < kIters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    dt = __builtin_amdgcn_s_memtime() - t0;
  } else if (!mat && (ROLES & 2)) {
    float x[8], y[16];
    for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i) * 1e-3f;
    for (int i = 0; i < 16; ++i) y[i] = seed * (threadIdx.x + 2 * i);
    const u64 t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < 2 * kIters; ++it) valu_iter<KIND>(x, y, 0.999f, 0.001f);
    for (int i = 0; i < 8; ++i) s += x[i];
    for (int i = 0; i < 16; ++i) s += y[i];
    dt = __builtin_amdgcn_s_memtime() - t0;
  }
  if (s == 1234.5f) out[threadIdx.x] = s;
  if (lane == 0) cyc[blockIdx.x * 8 + wave] = dt | ((u64)mat << 63);
}

// One wave per SIMD that interleaves its own MFMAs with independent vector work: each of the 4
// MFMAs of an iteration (4 accumulator chains) is followed by NV independent v_fma_f32 (EXP:
// v_exp_f32) on registers no MFMA touches.  If the wave overlaps the two, an iteration takes the
// 4 MFMAs' 128 cycles until the vector instructions alone take longer.
template <int NV, bool EXP>
__global__ __launch_bounds__(256) void mixed_cycles(float *out, u64 *cyc, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (threadIdx.x + i));
    b[i] = (__bf16)(seed * (i + 1));
  }
  f32x16 c[4] = {};
  float y[4 * NV + 1];
  for (int i = 0; i < 4 * NV + 1; ++i) y[i] = -seed * (threadIdx.x + 2 * i);
  const u64 t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      c[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[m], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        float &v = y[m * NV + k];
        v = EXP ? __builtin_amdgcn_exp2f(v) : fmaf(v, 0.999f, 0.001f);
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    }
  }
  const u64 t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int m = 0; m < 4; ++m)
    for (int i = 0; i < 16; ++i) s += c[m][i];
  for (int i = 0; i < 4 * NV + 1; ++i) s += y[i];
  if (s == 1234.5f) out[threadIdx.x] = s;
  if (threadIdx.x == 0) cyc[blockIdx.x] = (t1 - t0) / kIters;
}

// One wave per SIMD issuing 8 MFMAs per iteration into NC accumulator chains (NC = 1: every MFMA
// takes the previous one's result as its accumulator).
template <int NC>
__global__ __launch_bounds__(256) void chain_cycles(float *out, u64 *cyc, float seed) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (threadIdx.x + i));
    b[i] = (__bf16)(seed * (i + 1));
  }
  f32x16 c[NC] = {};
  const u64 t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) c[m % NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[m % NC], 0, 0, 0);
  }
  const u64 t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int m = 0; m < NC; ++m)
    for (int i = 0; i < 16; ++i) s += c[m][i];
  if (s == 1234.5f) out[threadIdx.x] = s;
  if (threadIdx.x == 0) cyc[blockIdx.x] = (t1 - t0) / kIters;
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
  for (int it = 0; it < 2 * kIters; ++it) {
    asm volatile("" ::: "memory");  // the reads are loop-invariant: force them every iteration
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x4 v = *(const f32x4 *)(base + 8 * k + ((it & 1) << 11));
      acc += v;
    }
  }
  if (acc[0] + acc[1] + acc[2] + acc[3] == 1234.5f) out[threadIdx.x] = acc[0];
}

// ds_read_b64_tr_b16 (the transposing 8-byte read) with the backward kernels' operand pattern:
// a 32-row tile of pitch 272 bytes, rows placed with index bits 0-1 and 2-3 swapped; per
// iteration 16 reads = the 8 transposed 32x16 fragments of a 32 x 128 tile (two 16-row halves x
// four 32-column blocks), alternating between two tiles.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
__global__ __launch_bounds__(256) void lds_tr_rate(float *out, float seed) {
  constexpr int P = 136;  // row pitch in 2-byte elements
  __shared__ __attribute__((aligned(16))) unsigned short lds[2 * 32 * P];
  for (int i = threadIdx.x; i < 2 * 32 * P; i += 256) lds[i] = (unsigned short)(seed * i);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int q = lane & 3, m = (lane >> 2) & 3, g = lane >> 4;
  const int col = 16 * (q & 1) + 8 * (g & 1) + 4 * (q >> 1);
  int off[2];
  for (int u = 0; u < 2; ++u) {
    int r = 8 * (g >> 1) + m + 4 * u;                  // row before the two placements
    r = (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);  // pi: bits 2 and 3 swapped
    r = (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);   // LDS placement: bit pairs 0-1, 2-3 swapped
    off[u] = r * P + col;  // <= 15 * 136 + 28; with the offsets below < 32 * 136 per tile
  }
  int acc = 0;
  for (int it = 0; it < 2 * kIters; ++it) {
    asm volatile("" ::: "memory");  // the reads are loop-invariant: force them every iteration
    const unsigned short *t = &lds[(it & 1) * 32 * P];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int d0 = 0; d0 < 4; ++d0)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16 *)&t[off[u] + 16 * kk * P + 32 * d0]);
          acc += v[0] ^ v[1] ^ v[2] ^ v[3];
        }
  }
  if (acc == 12345) out[threadIdx.x] = (float)acc;
}

// Do LDS reads and MFMAs overlap?  Eight waves per CU (two per SIMD), each iteration a wave
// issues 8 MFMAs (4 accumulator chains; operands in registers) and/or 8 KB of LDS reads whose
// results no MFMA uses: TR = 16 ds_read_b64_tr_b16 with the backward kernels' addresses, else
// 8 ds_read_b128 of 16-byte row chunks.  MODE 1: MFMAs only, 2: reads only, 3: both, the
// reads issued before the MFMAs of the iteration.  Core cycles per iteration: if the two
// overlap, MODE 3 takes the longer of MODE 1 and 2; if not, their sum.
template <int MODE, bool TR, bool AGPR = false>
__global__ __launch_bounds__(512) void lds_mfma_cycles(float *out, u64 *cyc, float seed) {
  constexpr int P = 136;
  __shared__ __attribute__((aligned(16))) unsigned short lds[2 * 32 * P];
  for (int i = threadIdx.x; i < 2 * 32 * P; i += 512) lds[i] = (unsigned short)(seed * i);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane & 3, m = (lane >> 2) & 3, g = lane >> 4;
  const int col = 16 * (q & 1) + 8 * (g & 1) + 4 * (q >> 1);
  int off[2];
  for (int u = 0; u < 2; ++u) {
    int r = 8 * (g >> 1) + m + 4 * u;
    r = (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
    r = (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
    off[u] = r * P + col;  // as in lds_tr_rate: every read stays inside its 32 x 136 tile
  }
  const int roff = (lane & 31) * P + (lane >> 5) * 8;  // row reads: <= 31 * 136 + 8 + 7 * 16 + 7
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (threadIdx.x + i));
    b[i] = (__bf16)(seed * (i + 1));
  }
  f32x16 c[4] = {};
  int acc = 0;
  const u64 t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kIters; ++it) {
    asm volatile("" ::: "memory");
    const unsigned short *t = &lds[(it & 1) * 32 * P];
    if constexpr (MODE & 2) {
      if constexpr (TR) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int d0 = 0; d0 < 4; ++d0)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_v4i16 *)&t[off[u] + 16 * kk * P + 32 * d0]);
              acc += v[0] ^ v[1] ^ v[2] ^ v[3];
            }
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const v8i16 v = *(const v8i16 *)&t[roff + 16 * k];  // 16-byte aligned
          acc += v[0] ^ v[1] ^ v[2] ^ v[3] ^ v[4] ^ v[5] ^ v[6] ^ v[7];
        }
      }
    }
    if constexpr (MODE & 1) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          if constexpr (AGPR)  // accumulators held in AGPRs (the MFMA result form before gfx90a)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c[mm]) : "v"(a), "v"(b));
          else
            c[mm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[mm], 0, 0, 0);
        }
    }
  }
  const u64 dt = __builtin_amdgcn_s_memtime() - t0;
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c[0][i] + c[1][i] + c[2][i] + c[3][i];
  if (s == 1234.5f || acc == 12345) out[threadIdx.x] = s;
  if (lane == 0) cyc[blockIdx.x * 8 + wave] = dt;
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

// Runs launch twice (the first warms up) and returns the n values it left in cyc.
template <typename F>
std::vector<u64> cycles(F launch, const u64 *cyc, int n) {
  for (int r = 0; r < 2; ++r) {
    launch();
    CHECK(hipDeviceSynchronize());
  }
  std::vector<u64> h(n);
  CHECK(hipMemcpy(h.data(), cyc, n * sizeof(u64), hipMemcpyDeviceToHost));
  return h;
}

double median(std::vector<double> v) {
  if (v.empty()) return 0.0;
  std::sort(v.begin(), v.end());
  return v[v.size() / 2];
}

template <typename F>
double median_cycles(F launch, const u64 *cyc, int n) {
  const std::vector<u64> h = cycles(launch, cyc, n);
  return median(std::vector<double>(h.begin(), h.end()));
}

int main() {
  hipDeviceProp_t p;
  CHECK(hipGetDeviceProperties(&p, 0));
  const int cus = p.multiProcessorCount;
  printf("device %s, %d CUs, clock %.0f MHz\n", p.gcnArchName, cus, p.clockRate / 1e3);
  float *out;
  CHECK(hipMalloc(&out, 4096 * sizeof(float)));
  u64 *cyc;  // 8 entries per workgroup, for up to 4 workgroups per CU
  CHECK(hipMalloc(&cyc, 8 * 4 * cus * sizeof(u64)));
  const float seed = 1e-3f;

  // The MFMA issue rate and the core clock under it, one and two waves per SIMD.
  {
    int wall_khz = 0;
    CHECK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, 0));
    for (int wps = 1; wps <= 2; ++wps) {
      const int grid = cus * wps;
      const float ms = time_ms([&] { mfma_cycles<<<grid, 256>>>(cyc, seed); }, 3);
      std::vector<u64> h(2 * grid);
      CHECK(hipMemcpy(h.data(), cyc, h.size() * sizeof(u64), hipMemcpyDeviceToHost));
      std::vector<double> mhz, per;
      for (int g = 0; g < grid; ++g) {
        mhz.push_back((double)h[2 * g] / (double)h[2 * g + 1] * wall_khz / 1e3);
        per.push_back((double)h[2 * g] / (4.0 * kIters) / wps);
      }
      const double flops = (double)grid * 4 * 4 * kIters * 32768.0;
      std::sort(mhz.begin(), mhz.end());
      printf("mfma bf16 32x32x16, %d wave/SIMD: %.2f core cycles per MFMA per SIMD; core clock "
             "median %.0f MHz (min %.0f, max %.0f; s_memtime against s_memrealtime at %d kHz); "
             "%.1f TFLOP/s\n",
             wps, median(per), mhz[grid / 2], mhz[0], mhz[grid - 1], wall_khz, flops / ms / 1e9);
    }
  }
  // Vector instruction cost per SIMD, one, two and four waves per SIMD.
  for (int wps = 1; wps <= 4; wps *= 2) {
    const int grid = cus * wps;
    const double e = median_cycles([&] { valu_cycles<0><<<grid, 256>>>(out, cyc, seed); }, cyc, grid);
    const double r = median_cycles([&] { valu_cycles<1><<<grid, 256>>>(out, cyc, seed); }, cyc, grid);
    const double f = median_cycles([&] { valu_cycles<2><<<grid, 256>>>(out, cyc, seed); }, cyc, grid);
    const double m = median_cycles([&] { valu_cycles<3><<<grid, 256>>>(out, cyc, seed); }, cyc, grid);
    printf("%d wave/SIMD, core cycles per wave64 instruction per SIMD: v_exp_f32 %.2f, v_rcp_f32 "
           "%.2f, v_fma_f32 %.2f; 1 exp + 2 fma interleaved %.2f per group (%.2f apart)\n",
           wps, e / 8 / wps, r / 8 / wps, f / 16 / wps, m / 8 / wps, (e + f) / 8 / wps);
  }
  {
    const double l = median_cycles([&] { fma_latency<<<cus * 4, 64>>>(out, cyc, seed); }, cyc, cus * 4);
    printf("dependent v_fma_f32 chain, 1 wave: %.2f core cycles per FMA\n", l);
  }
  // Softmax-phase vector work per score.
  for (int wps = 1; wps <= 4; wps *= 2) {
    const int grid = cus * wps;
    const double sc = median_cycles([&] { prob_chain<true><<<grid, 256>>>(out, cyc, seed); }, cyc, grid);
    const double pl = median_cycles([&] { prob_chain<false><<<grid, 256>>>(out, cyc, seed); }, cyc, grid);
    printf("probability per score, %d wave/SIMD: soft-cap %.1f, plain %.1f core cycles per SIMD\n",
           wps, sc / 32 / wps, pl / 32 / wps);
  }
  // One matrix-core wave and one vector wave per SIMD: each role's core cycles, together and
  // with the other role idle.
  {
    const int grid = cus, n = 8 * grid;
    auto roles = [&](auto launch) {
      const std::vector<u64> h = cycles(launch, cyc, n);
      std::vector<double> mt, vt;
      for (u64 x : h) {
        const double c = (double)(x & ~(1ull << 63));
        if (c == 0) continue;  // an idle role
        ((x >> 63) ? mt : vt).push_back(c);
      }
      return std::make_pair(median(mt), median(vt));
    };
    const std::pair<double, double> eb = roles([&] { pair_cycles<0, 3><<<grid, 512>>>(out, cyc, seed); });
    const std::pair<double, double> em = roles([&] { pair_cycles<0, 1><<<grid, 512>>>(out, cyc, seed); });
    const std::pair<double, double> ev = roles([&] { pair_cycles<0, 2><<<grid, 512>>>(out, cyc, seed); });
    printf("one mfma wave + one exp wave per SIMD, core cycles: together mfma %.0f, exp %.0f; "
           "alone mfma %.0f, exp %.0f\n", eb.first, eb.second, em.first, ev.second);
    const std::pair<double, double> fb = roles([&] { pair_cycles<2, 3><<<grid, 512>>>(out, cyc, seed); });
    const std::pair<double, double> fm = roles([&] { pair_cycles<2, 1><<<grid, 512>>>(out, cyc, seed); });
    const std::pair<double, double> fv = roles([&] { pair_cycles<2, 2><<<grid, 512>>>(out, cyc, seed); });
    printf("one mfma wave + one fma wave per SIMD, core cycles: together mfma %.0f, fma %.0f; "
           "alone mfma %.0f, fma %.0f\n", fb.first, fb.second, fm.first, fv.second);
  }
  // One wave per SIMD: a dependent MFMA chain against independent ones.
  {
    const int grid = cus;
    auto per = [&](auto launch) { return median_cycles(launch, cyc, grid) / 8.0; };
    printf("1 wave/SIMD, core cycles per MFMA with 1, 2, 4 accumulator chains: %.1f %.1f %.1f\n",
           per([&] { chain_cycles<1><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { chain_cycles<2><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { chain_cycles<4><<<grid, 256>>>(out, cyc, seed); }));
  }
  // One wave per SIMD overlapping its own MFMAs with independent vector instructions.
  {
    const int grid = cus;
    auto per = [&](auto launch) { return median_cycles(launch, cyc, grid) / 4.0; };
    printf("1 wave/SIMD, core cycles per MFMA followed by n independent vector instructions:\n"
           "  fma n=0..8: %.1f %.1f %.1f %.1f %.1f\n  exp n=1..4: %.1f %.1f %.1f %.1f\n",
           per([&] { mixed_cycles<0, false><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { mixed_cycles<2, false><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { mixed_cycles<4, false><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { mixed_cycles<6, false><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { mixed_cycles<8, false><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { mixed_cycles<1, true><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { mixed_cycles<2, true><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { mixed_cycles<3, true><<<grid, 256>>>(out, cyc, seed); }),
           per([&] { mixed_cycles<4, true><<<grid, 256>>>(out, cyc, seed); }));
  }
  {
    const int grid = cus * 2 * 8;
    const float ms = time_ms([&] { lds_rate<<<grid, 256>>>(out, seed); }, 5);
    const double bytes = (double)grid * 256 * 2 * kIters * 8 * 16;
    printf("LDS ds_read_b128: %.1f TB/s = %.1f B/clk/CU at 2.4 GHz\n", bytes / ms / 1e9,
           bytes / (ms * 1e-3) / 2.4e9 / cus);
  }
  {
    const int grid = cus * 2 * 8;
    const float ms = time_ms([&] { lds_tr_rate<<<grid, 256>>>(out, seed); }, 5);
    const double bytes = (double)grid * 256 * 2 * kIters * 16 * 8;
    printf("LDS ds_read_b64_tr_b16: %.1f TB/s = %.1f B/clk/CU at 2.4 GHz\n", bytes / ms / 1e9,
           bytes / (ms * 1e-3) / 2.4e9 / cus);
  }
  {
    // one 8-wave workgroup per CU; cycles per iteration (median over the waves)
    const int grid = cus;
    auto per = [&](auto launch) { return median_cycles(launch, cyc, grid * 8) / kIters; };
    printf("2 wave/SIMD, core cycles per iteration of 8 MFMAs and/or 8 KB of LDS reads per wave: "
           "MFMA %.0f; ds_read_b64_tr_b16 %.0f, both %.0f; ds_read_b128 %.0f, both %.0f\n",
           per([&] { lds_mfma_cycles<1, true><<<grid, 512>>>(out, cyc, seed); }),
           per([&] { lds_mfma_cycles<2, true><<<grid, 512>>>(out, cyc, seed); }),
           per([&] { lds_mfma_cycles<3, true><<<grid, 512>>>(out, cyc, seed); }),
           per([&] { lds_mfma_cycles<2, false><<<grid, 512>>>(out, cyc, seed); }),
           per([&] { lds_mfma_cycles<3, false><<<grid, 512>>>(out, cyc, seed); }));
    printf("  the same with the MFMA accumulators in AGPRs: MFMA %.0f; ds_read_b64_tr_b16 both %.0f; "
           "ds_read_b128 both %.0f\n",
           per([&] { lds_mfma_cycles<1, true, true><<<grid, 512>>>(out, cyc, seed); }),
           per([&] { lds_mfma_cycles<3, true, true><<<grid, 512>>>(out, cyc, seed); }),
           per([&] { lds_mfma_cycles<3, false, true><<<grid, 512>>>(out, cyc, seed); }));
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
  CHECK(hipFree(cyc));
  CHECK(hipFree(out));
  return 0;
}
