// Measured peaks of the GPU for the access patterns and the MFMA shape that
// the MSA kernels use; bench.py prints them next to the published peaks.
//
//  * HBM, sequential: 16-byte coalesced reads, writes and a copy over 8 GiB
//    (the combine's slab reads are sequential).
//  * HBM, random 4 KB chunks over a 16 GiB footprint: reads, writes, and a
//    1:1 mix (the attention kernel gathers 4 KB query rows and stores 4 KB
//    partial-output pieces at scattered places).
//  * MFMA: back-to-back v_mfma_f32_32x32x16_bf16 on register operands, four
//    independent accumulators per wave, every SIMD busy (the clock the chip
//    sustains under that load sets the ceiling).  Two operand kinds: a few
//    fixed low-entropy patterns, and random unit-scale bf16 fragments that
//    change from one MFMA to the next, as real Q and K tiles do; the matrix
//    cores draw more power on the latter and the clock drops accordingly.
//
// Every index is reduced modulo its buffer, so all accesses stay inside the
// allocations.  Prints one JSON line.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "peaks: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// SplitMix64 finaliser (Steele, Lea, Flood, OOPSLA 2014).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

constexpr int kThreads = 256;  // a workgroup access round is 4 KB
constexpr int kUnroll = 16;    // independent 4 KB accesses in flight per workgroup

// Sequential: round r of workgroup g covers pieces (g * R + r) * 16 + u,
// u < 16, each 4 KB; the 16 loads of a round are issued before any is used.
template <int MODE>  // 0 read, 1 write, 2 copy (read a, write b)
__global__ __launch_bounds__(kThreads) void seq_kernel(u32x4* a, u32x4* b, uint64_t npieces,
                                                       int rounds, u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int r = 0; r < rounds; ++r) {
    const uint64_t p0 = (static_cast<uint64_t>(blockIdx.x) * rounds + r) * kUnroll;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t i = ((p0 + u) % npieces) * kThreads + threadIdx.x;
      if (MODE == 0 || MODE == 2) v[u] = a[i];
      if (MODE == 1) a[i] = u32x4{static_cast<uint32_t>(i), 1u, 2u, 3u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t i = ((p0 + u) % npieces) * kThreads + threadIdx.x;
      if (MODE == 0) acc ^= v[u];
      if (MODE == 2) b[i] = v[u];
    }
  }
  if (MODE == 0 && acc[0] == 0x12345678u && acc[1] == 0x9abcdefu) sink[threadIdx.x] = acc;
}

// Random 4 KB chunks: access u of round r of workgroup g touches chunk
// hash(id) mod n, id = (g * R + r) * 16 + u.
template <int MODE>  // 0 read, 1 write, 2 read one chunk and write another
__global__ __launch_bounds__(kThreads) void rand_kernel(u32x4* a, uint64_t nchunks, int rounds,
                                                        u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int r = 0; r < rounds; ++r) {
    const uint64_t id0 = (static_cast<uint64_t>(blockIdx.x) * rounds + r) * kUnroll;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint64_t c = mix64(id0 + u) % nchunks;
      if (MODE == 0 || MODE == 2) v[u] = a[c * kThreads + threadIdx.x];
      if (MODE == 1) a[c * kThreads + threadIdx.x] = u32x4{static_cast<uint32_t>(id0 + u), 1u, 2u, 3u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (MODE == 0) acc ^= v[u];
      if (MODE == 2) a[(mix64((id0 + u) ^ 0x5DEECE66Dull) % nchunks) * kThreads + threadIdx.x] = v[u];
    }
  }
  if (MODE == 0 && acc[0] == 0x12345678u && acc[1] == 0x9abcdefu) sink[threadIdx.x] = acc;
}

// Random operands: 8 A and 8 B fragments per lane, bf16 values of random
// sign and magnitude in [0.25, 1), cycled so that consecutive MFMAs see
// different data.
__device__ __forceinline__ bf16x8 random_fragment(uint64_t seed) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint64_t z = mix64(seed * 4 + i);
    const uint32_t lo = 0x3E00u | (static_cast<uint32_t>(z) & 0x81FFu);
    const uint32_t hi = 0x3E00u | (static_cast<uint32_t>(z >> 32) & 0x81FFu);
    r[i] = lo | (hi << 16);
  }
  return __builtin_bit_cast(bf16x8, r);
}

__global__ __launch_bounds__(kThreads) void mfma_rand_kernel(int iters, float* sink) {
  const uint64_t t = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = random_fragment(t * 16 + j);
    b[j] = random_fragment(t * 16 + 8 + j);
  }
  f32x16 c[4] = {};
  for (int i = 0; i < iters; i += 64) {  // iters: a multiple of 64
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(3 * j + r) & 7], c[j & 3], 0, 0, 0);
    }
  }
  const float s = c[0][0] + c[1][1] + c[2][2] + c[3][3];
  if (s == 1.2345f) sink[t % kThreads] = s;
}

__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float* sink) {
  const int t = threadIdx.x;
  u32x4 ra = {static_cast<uint32_t>(t) * 0x3F803F80u, 0x3F003F00u, 0x3E803E80u, 0x3F803F80u};
  u32x4 rb = {0x3F803F80u, static_cast<uint32_t>(t) | 0x3E003E00u, 0x3F003F00u, 0x3E803E80u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra), b = __builtin_bit_cast(bf16x8, rb);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c3, 0, 0, 0);
  }
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  if (s == 1.2345f) sink[t] = s;
}

template <typename F>
static float time_ms(F launch, int reps) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  launch();  // warmup
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e0, 0));
  for (int i = 0; i < reps; ++i) launch();
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return ms / reps;
}

int main() {
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  const uint64_t seq_bytes = 8ull << 30, rand_bytes = 16ull << 30;
  u32x4 *a, *b, *sink;
  CHECK(hipMalloc(&a, rand_bytes));
  CHECK(hipMalloc(&b, seq_bytes));
  CHECK(hipMalloc(&sink, kThreads * sizeof(u32x4)));
  CHECK(hipMemset(a, 0, rand_bytes));
  CHECK(hipMemset(b, 0, seq_bytes));

  // Sequential: each launch streams the whole 8 GiB region once.
  const uint64_t npieces = seq_bytes / (kThreads * 16);
  const unsigned sgrid = static_cast<unsigned>(cus) * 8;
  const int srounds = static_cast<int>((npieces + static_cast<uint64_t>(sgrid) * kUnroll - 1) /
                                       (static_cast<uint64_t>(sgrid) * kUnroll));
  const double sb = static_cast<double>(sgrid) * srounds * kUnroll * kThreads * 16;
  const float t_rd = time_ms([&] { hipLaunchKernelGGL(seq_kernel<0>, dim3(sgrid), dim3(kThreads), 0, 0, a, b, npieces, srounds, sink); }, 3);
  const float t_wr = time_ms([&] { hipLaunchKernelGGL(seq_kernel<1>, dim3(sgrid), dim3(kThreads), 0, 0, a, b, npieces, srounds, sink); }, 3);
  const float t_cp = time_ms([&] { hipLaunchKernelGGL(seq_kernel<2>, dim3(sgrid), dim3(kThreads), 0, 0, a, b, npieces, srounds, sink); }, 3);

  // Random: 16 GiB of 4 KB accesses per stream and launch over the 16 GiB footprint.
  const uint64_t nchunks = rand_bytes / (kThreads * 16);
  const int rounds = 32;
  const unsigned rgrid = static_cast<unsigned>(cus) * 32;
  const double rb = static_cast<double>(rgrid) * rounds * kUnroll * kThreads * 16;  // per stream
  const float t_rr = time_ms([&] { hipLaunchKernelGGL(rand_kernel<0>, dim3(rgrid), dim3(kThreads), 0, 0, a, nchunks, rounds, sink); }, 3);
  const float t_rw = time_ms([&] { hipLaunchKernelGGL(rand_kernel<1>, dim3(rgrid), dim3(kThreads), 0, 0, a, nchunks, rounds, sink); }, 3);
  const float t_rm = time_ms([&] { hipLaunchKernelGGL(rand_kernel<2>, dim3(rgrid), dim3(kThreads), 0, 0, a, nchunks, rounds, sink); }, 3);

  const int iters = 8192;
  const unsigned mgrid = static_cast<unsigned>(cus) * 2;  // 8 waves per CU, two per SIMD
  const float t_mf = time_ms([&] { hipLaunchKernelGGL(mfma_kernel, dim3(mgrid), dim3(kThreads), 0, 0, iters, reinterpret_cast<float*>(sink)); }, 3);
  const double mflop = static_cast<double>(mgrid) * (kThreads / 64) * iters * 4 * (32.0 * 32 * 16 * 2);
  const float t_mr = time_ms([&] { hipLaunchKernelGGL(mfma_rand_kernel, dim3(mgrid), dim3(kThreads), 0, 0, 4 * iters, reinterpret_cast<float*>(sink)); }, 3);

  printf("{\"hbm_seq_read_GBs\": %.1f, \"hbm_seq_write_GBs\": %.1f, \"hbm_copy_GBs\": %.1f, "
         "\"hbm_rand4k_read_GBs\": %.1f, \"hbm_rand4k_write_GBs\": %.1f, \"hbm_rand4k_mixed_GBs\": %.1f, "
         "\"mfma_bf16_TFLOPs\": %.1f, \"mfma_bf16_random_TFLOPs\": %.1f}\n",
         sb / t_rd / 1e6, sb / t_wr / 1e6, 2 * sb / t_cp / 1e6, rb / t_rr / 1e6, rb / t_rw / 1e6,
         2 * rb / t_rm / 1e6, mflop / t_mf / 1e9, mflop / t_mr / 1e9);
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  CHECK(hipFree(sink));
  return 0;
}
