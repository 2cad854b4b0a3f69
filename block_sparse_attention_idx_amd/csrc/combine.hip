// Split-K log-sum-exp merge of the KV-outer partial outputs
// ("MiniMax Sparse Attention (MSA)", Deep Dive > KV-Outer Sparse Attention,
// step 6: the combine kernel normalises the partial buffer by a split-K
// log-sum-exp merge).  For query i and head h of group r, over the slots s
// whose block id is valid:
//     LSE = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - LSE) * Obar_s.
// A slot is valid when its id lies in [0, floor(i / B_k)], the same test the
// inversion applies: the attention pass never writes the partials of any
// other slot (-1 padding, or an out-of-range id the inversion skipped and
// counted), so those partials are never read.
//
// A pure streaming kernel.  The partials of one (query, group) are one
// contiguous k * G * d_h bf16 slab; a workgroup of 256 threads owns
// 4096 / (G * d_h) (query, group) pairs at a time and every thread 8 output
// dimensions of one head.  The slot loop is unrolled at compile time so all
// of a thread's slab loads (16 bytes each, non-temporal: the partials are
// read exactly once) are in flight together; the selection row and the lse
// values are read first, the weights computed once per (query, head).
// Output rows (a query's G heads of group r) are contiguous 16-byte stores,
// non-temporal like the loads: nothing in the pass reads O again, and cached
// write-back stores measured 6% slower over the passes of a 128K prefill.
// (Non-temporal stores only pay for whole lines; the 4-byte lse values stay
// ordinary stores.)
// Each XCD streams one contiguous share of the partial buffer.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kCombThreads = 256;

template <int G, int KMAX>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const int32_t* __restrict__ block_idx, const uint16_t* __restrict__ o_part,
    const float* __restrict__ lse_part, int64_t N, int H_kv, int k, int64_t q_begin,
    int64_t q_count, int64_t rows_total, int bks, uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int TPQ = 16 * G;              // threads per (query, group)
  constexpr int QPW = kCombThreads / TPQ;  // (query, group) pairs per workgroup
  const int t = threadIdx.x;
  // Workgroups are dealt round-robin to the kXcds XCDs; the grid is a
  // multiple of kXcds and XCD x takes the x-th contiguous share of the
  // (query, group) slabs, so each XCD streams its own region of the partial
  // buffer (measured: steadier and faster than interleaving the XCDs).
  const int64_t per = gridDim.x / kXcds;
  const int64_t wgi = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  // flat (query, group) index: f = seq * q_count + row, seq = batch * H_kv + r
  const int64_t f = wgi * QPW + t / TPQ;
  if (f >= rows_total) return;
  const int64_t seq = f / q_count, row = f % q_count;
  const int g = (t % TPQ) >> 4, dc = t & 15;
  const int64_t bat = seq / H_kv;
  const int r = static_cast<int>(seq % H_kv);
  const int32_t* sel = block_idx + f * k;
  const int64_t base = f * k;  // slot 0 of this (query, group)
  // the row's local block: the largest id a slot may hold (bks < 0: rows of
  // one decode step, whose ids the library itself wrote, are not checked)
  const uint32_t lmax = bks < 0 ? 0x7FFFFFFFu : static_cast<uint32_t>((q_begin + row) >> bks);

  bool valid[KMAX];
  float l[KMAX];
  u32x4 v[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) valid[s] = s < k && static_cast<uint32_t>(sel[s]) <= lmax;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    v[s] = u32x4{0u, 0u, 0u, 0u};
    if (valid[s])
      v[s] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(o_part + ((base + s) * G + g) * kDh + dc * 8));
  }
#pragma unroll
  for (int s = 0; s < KMAX; ++s) l[s] = valid[s] ? lse_part[(base + s) * G + g] : -__builtin_huge_valf();

  constexpr float kLog2e = 1.4426950408889634f;
  float mx = -__builtin_huge_valf();
#pragma unroll
  for (int s = 0; s < KMAX; ++s) mx = fmaxf(mx, l[s]);
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    l[s] = valid[s] ? __builtin_amdgcn_exp2f((l[s] - mx) * kLog2e) : 0.f;
    sum += l[s];
  }
  // a row left with no valid slot (a caller's selection may hold none) gets
  // O = 0 and LSE = -inf
  const float inv = sum > 0.f ? 1.f / sum : 0.f;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    const float w = l[s] * inv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += w * __uint_as_float(v[s][j] << 16);
      acc[2 * j + 1] += w * __uint_as_float(v[s][j] & 0xFFFF0000u);
    }
  }
  const int64_t orow = (bat * N + q_begin + row) * (static_cast<int64_t>(H_kv) * G) + r * G + g;
  __builtin_nontemporal_store(
      u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
            pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])},
      reinterpret_cast<u32x4*>(o + orow * kDh + dc * 8));
  if (lse && dc == 0) lse[orow] = mx + __builtin_amdgcn_logf(sum) * 0.69314718055994531f;
}

template <int G, int KMAX>
hipError_t launch_gk(const int32_t* block_idx, const uint16_t* o_part, const float* lse_part,
                     int batch, int64_t N, int H_kv, int k, int64_t q_begin, int64_t q_count,
                     int bks, uint16_t* o, float* lse, hipStream_t stream) {
  constexpr int QPW = kCombThreads / (16 * G);
  const int64_t rows_total = static_cast<int64_t>(batch) * H_kv * q_count;
  const int64_t nx = (rows_total + QPW - 1) / QPW;
  const int64_t grid = (nx + kXcds - 1) / kXcds * kXcds;  // see the kernel
  hipLaunchKernelGGL((combine_kernel<G, KMAX>), dim3(static_cast<unsigned>(grid)),
                     dim3(kCombThreads), 0, stream, block_idx, o_part, lse_part, N, H_kv, k,
                     q_begin, q_count, rows_total, bks, o, lse);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const int32_t* block_idx, const uint16_t* o_part, const float* lse_part,
                    int batch, int64_t N, int H_kv, int k, int64_t q_begin, int64_t q_count,
                    int bks, uint16_t* o, float* lse, hipStream_t stream) {
  if (k <= 4)
    return launch_gk<G, 4>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, bks, o, lse, stream);
  if (k <= 8)
    return launch_gk<G, 8>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, bks, o, lse, stream);
  if (k <= 16)
    return launch_gk<G, 16>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, bks, o, lse, stream);
  return launch_gk<G, 32>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, bks, o, lse, stream);
}

}  // namespace

hipError_t launch_combine(const int32_t* block_idx, const uint16_t* o_part, const float* lse_part,
                          int batch, int64_t N, int H_kv, int G, int k, int64_t q_begin,
                          int64_t q_count, uint16_t* o, float* lse, hipStream_t stream, int bk) {
  int bks = -1;
  if (bk > 0) {
    bks = 0;
    while ((1 << bks) < bk) ++bks;
    if ((1 << bks) != bk) return hipErrorInvalidValue;
  }
  switch (G) {
    case 1: return launch_g<1>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, bks, o, lse, stream);
    case 2: return launch_g<2>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, bks, o, lse, stream);
    case 4: return launch_g<4>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, bks, o, lse, stream);
    case 8: return launch_g<8>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, bks, o, lse, stream);
    case 16: return launch_g<16>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, bks, o, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
