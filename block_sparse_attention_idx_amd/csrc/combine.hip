// Split-K log-sum-exp merge of the KV-outer partial outputs
// ("MiniMax Sparse Attention (MSA)", Deep Dive > KV-Outer Sparse Attention,
// step 6: the combine kernel normalises the partial buffer by a split-K
// log-sum-exp merge).  For query i and head h of group r, over the slots s
// whose block id is valid:
//     LSE = ln sum_s exp(lse_s),   O = sum_s exp(lse_s - LSE) * Obar_s.
//
// A pure streaming kernel: the partials of one (query, group) are one
// contiguous k * G * d_h bf16 slab, read once with 16-byte loads; each thread
// owns 8 output dimensions of one head.  Output rows (a query's G heads of
// group r) are contiguous 16-byte stores.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kCombThreads = 256;

template <int G>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    const int32_t* __restrict__ block_idx, const uint16_t* __restrict__ o_part,
    const float* __restrict__ lse_part, int64_t N, int H_kv, int k, int64_t q_begin,
    int64_t q_count, uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int TPQ = 16 * G;              // threads per (query, group)
  constexpr int QPW = kCombThreads / TPQ;  // queries per workgroup
  const int t = threadIdx.x;
  const int64_t seq = blockIdx.y;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * QPW + t / TPQ;
  if (row >= q_count) return;
  const int g = (t % TPQ) >> 4, dc = t & 15;
  const int64_t bat = seq / H_kv;
  const int r = static_cast<int>(seq % H_kv);
  const int32_t* sel = block_idx + (seq * q_count + row) * k;
  const int64_t base = (seq * q_count + row) * k;  // slot 0 of this (query, group)

  float mx = -__builtin_huge_valf();
  for (int s = 0; s < k; ++s)
    if (sel[s] >= 0) mx = fmaxf(mx, lse_part[(base + s) * G + g]);
  constexpr float kLog2e = 1.4426950408889634f;
  float sum = 0.f;
  for (int s = 0; s < k; ++s)
    if (sel[s] >= 0) sum += __builtin_amdgcn_exp2f((lse_part[(base + s) * G + g] - mx) * kLog2e);
  const float inv = 1.f / sum;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < k; ++s) {
    if (sel[s] < 0) continue;
    const float w = __builtin_amdgcn_exp2f((lse_part[(base + s) * G + g] - mx) * kLog2e) * inv;
    const u32x4 v = *reinterpret_cast<const u32x4*>(o_part + ((base + s) * G + g) * kDh + dc * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += w * __uint_as_float(v[j] << 16);
      acc[2 * j + 1] += w * __uint_as_float(v[j] & 0xFFFF0000u);
    }
  }
  const int64_t orow = (bat * N + q_begin + row) * (static_cast<int64_t>(H_kv) * G) + r * G + g;
  *reinterpret_cast<u32x4*>(o + orow * kDh + dc * 8) =
      u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
            pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  if (lse && dc == 0) lse[orow] = mx + __builtin_amdgcn_logf(sum) * 0.69314718055994531f;
}

template <int G>
hipError_t launch_g(const int32_t* block_idx, const uint16_t* o_part, const float* lse_part,
                    int batch, int64_t N, int H_kv, int k, int64_t q_begin, int64_t q_count,
                    uint16_t* o, float* lse, hipStream_t stream) {
  constexpr int QPW = kCombThreads / (16 * G);
  const int64_t nx = (q_count + QPW - 1) / QPW;
  hipLaunchKernelGGL(combine_kernel<G>, dim3(static_cast<unsigned>(nx), batch * H_kv),
                     dim3(kCombThreads), 0, stream, block_idx, o_part, lse_part, N, H_kv, k,
                     q_begin, q_count, o, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const int32_t* block_idx, const uint16_t* o_part, const float* lse_part,
                          int batch, int64_t N, int H_kv, int G, int k, int64_t q_begin,
                          int64_t q_count, uint16_t* o, float* lse, hipStream_t stream) {
  switch (G) {
    case 1: return launch_g<1>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, o, lse, stream);
    case 2: return launch_g<2>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, o, lse, stream);
    case 4: return launch_g<4>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, o, lse, stream);
    case 8: return launch_g<8>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, o, lse, stream);
    case 16: return launch_g<16>(block_idx, o_part, lse_part, batch, N, H_kv, k, q_begin, q_count, o, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
