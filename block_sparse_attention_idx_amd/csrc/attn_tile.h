// LDS tile layout and K/V staging shared by the query-outer attention kernels
// (dense baseline and decode).  One K/V block of one head (128 keys x 128
// dims, bf16) occupies a kBufBytes buffer: K row-major, then V transposed,
// rows padded to 272 bytes, staged by a 512-thread workgroup through
// registers.  The layout is the one the score and P V MFMA fragments of those
// kernels read:
//  * K row-major, 272 B per key row: a 16-lane phase of 16-byte reads of rows
//    n .. n + 15 starts at distinct 4-bank groups;
//  * V^T row d stored at position 2 (d mod 64) + d / 64, and bits 0 and 1 of
//    the 8-byte key-chunk index kc (four keys) swapped, so that the eight keys
//    one lane feeds to a P^T step lie in one 16-byte chunk and the 32 rows one
//    operand read touches are consecutive.
#pragma once

#include "msa_internal.h"

namespace msa {
namespace tile {

constexpr int kStr = 272;                        // padded LDS row of K, V^T and output tiles
constexpr int kVtOff = kBk * kStr;               // V^T after K in a buffer
constexpr int kBufBytes = kVtOff + kDh * kStr;   // one block: 69,632 B
constexpr int kStageThreads = 512;               // threads that stage one block

__device__ __forceinline__ int dvt_row(int d) { return ((d & 63) << 1) | (d >> 6); }
__device__ __forceinline__ int dvt_off(int d, int kc) {
  const int kcp = (kc & ~3) | ((kc & 1) << 1) | ((kc & 2) >> 1);
  return dvt_row(d) * kStr + kcp * 8;
}

__device__ __forceinline__ uint32_t bf16_of(const u32x4& w, int dd) {
  const uint32_t x = w[dd >> 1];
  return (dd & 1) ? (x >> 16) : (x & 0xFFFFu);
}

// Lanes n and n + 32 hold the two halves of one row; v_permlane32_swap
// exchanges the half-waves.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One K/V block of one head in flight through registers: thread t (of 512)
// holds 16-byte chunks t % 16 of keys t / 16 + 32 p (K) and the 8 dims
// 8 (t / 32) .. + 7 of keys 4 (t % 32) .. + 3 (V, transposed when written).
struct KVRegs {
  u32x4 k[4];
  u32x4 v[4];
};

// Keys at or past nvalid are read from row nvalid - 1 (every load stays in
// bounds) and replaced by zeros when stored.
__device__ __forceinline__ void kv_load(KVRegs& R, const uint8_t* __restrict__ kb,
                                        const uint8_t* __restrict__ vb, int64_t rstride, int nvalid,
                                        int tid) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int key = (tid >> 4) + 32 * p, c = tid & 15;
    R.k[p] = *reinterpret_cast<const u32x4*>(kb + min(key, nvalid - 1) * rstride + c * 16);
  }
  const int kc = tid & 31, dg = tid >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    R.v[j] = *reinterpret_cast<const u32x4*>(vb + min(4 * kc + j, nvalid - 1) * rstride + dg * 16);
}

__device__ __forceinline__ void kv_store(const KVRegs& R, uint8_t* buf, int nvalid, int tid) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int key = (tid >> 4) + 32 * p, c = tid & 15;
    const u32x4 w = key < nvalid ? R.k[p] : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(buf + key * kStr + c * 16) = w;
  }
  const int kc = tid & 31, dg = tid >> 5;
  u32x4 row[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) row[j] = 4 * kc + j < nvalid ? R.v[j] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    const int d = 8 * dg + dd;
    const u32x2 w = {bf16_of(row[0], dd) | (bf16_of(row[1], dd) << 16),
                     bf16_of(row[2], dd) | (bf16_of(row[3], dd) << 16)};
    *reinterpret_cast<u32x2*>(buf + kVtOff + dvt_off(d, kc)) = w;
  }
}

}  // namespace tile
}  // namespace msa
