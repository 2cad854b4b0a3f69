// Internal declarations shared by the MSA HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBk = 128;   // tokens per key block
constexpr int kDh = 128;   // head dimension of Q, K, V
constexpr int kXcds = 8;   // MI355X: workgroups are dealt round-robin to 8 XCDs

// Attention workgroup: kAttnWaves = 8 waves, two per SIMD, one 32-row MFMA
// tile each, so a pass is kPassRows (query, head) rows = kPassRows / G
// entries.  (Four waves, one per SIMD with all 512 registers, measured
// slower.)
constexpr int kAttnWaves = 8;
constexpr int kPassRows = 32 * kAttnWaves;


// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D[32x32] += A[32x16] * B[16x32] in bf16 with fp32 accumulation.
// Lane l supplies A row (l % 32) and B column (l % 32), reduction slots
// 8 * (l / 32) .. + 7; it receives D column (l % 32), rows
// 8 * (e / 4) + 4 * (l / 32) + (e % 4) for accumulator element e.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max(a, b, c) as one v_max3_f32.  With NaNs excluded (-fno-honor-nans) the
// compiler treats fmaxf as associative and rebalances a running maximum over
// pairs into pairwise maxima plus v_max3 (three instructions per four values
// instead of two); a chain of these keeps the running form.  Exact, so the
// result is the same whatever the order.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Pack two fp32 into two bf16 (round to nearest even) in one u32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// OCP e4m3fn code -> bf16 bits of (value * 2^-8), exact, in integer
// arithmetic.  The code's bits are placed into an fp16 (exponent bias 15
// instead of 7, so the value is scaled by 2^-8; fp16 subnormals carry the e4m3
// subnormals), widened to fp32 and truncated to bf16 (at most 4 significant
// bits, so no rounding happens).
__device__ __forceinline__ uint32_t e4m3_to_bf16_scaled(uint32_t c) {
  uint16_t h = static_cast<uint16_t>(((c & 0x80u) << 8) | ((c & 0x7Fu) << 7));
  float f = static_cast<float>(__builtin_bit_cast(_Float16, h));
  return __float_as_uint(f) >> 16;
}

// The same for 4 codes (one u32) -> 4 bf16 (two u32), in integer arithmetic.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4_int(uint32_t w) {
  u32x2 r;
  r[0] = e4m3_to_bf16_scaled(w & 0xFF) | (e4m3_to_bf16_scaled((w >> 8) & 0xFF) << 16);
  r[1] = e4m3_to_bf16_scaled((w >> 16) & 0xFF) | (e4m3_to_bf16_scaled(w >> 24) << 16);
  return r;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the HIP error of the launch.

// Index branch.  block_idx rows: [batch][H_kv][q_count][k].  force_first /
// window > 1 also force block 0 and the window - 1 blocks before the local one.
hipError_t launch_index_topk(const uint16_t* q_idx, const uint16_t* k_idx, int batch, int64_t N,
                             int H_kv, int d_idx, int k, int64_t q_begin, int64_t q_count,
                             int32_t* block_idx, hipStream_t stream, int force_first = 0,
                             int window = 1, int bk = kBk);

// FLOP-matched sliding-window selection: block 0 and the k - 1 blocks ending
// at the local one (all of 0 .. L when L < k), ascending, -1 padded.
hipError_t launch_window_select(int batch, int H_kv, int k, int64_t q_begin, int64_t q_count,
                                int32_t* block_idx, hipStream_t stream, int bk = kBk);

// Inversion scratch layout (all offsets in 4-byte words, 256-byte aligned).
// Bins are (seq, block), ordered seq-major, so a seq owns B_c consecutive
// bins.  The attention work list is a flat array of passes in bin order: each
// holds up to EPP = kPassRows / G consecutive entries of one bin, so no pass
// spans two bins.
struct SchedLayout {
  int64_t nbins;       // batch * H_kv * B_c
  int64_t B_c;         // key blocks visible to the range
  int64_t T64;         // 64-row query tiles of the range
  int64_t EPP;         // entries per pass
  int64_t max_passes;  // capacity of the pass list
  int64_t off_tot;     // per-bin totals [nbins]
  int64_t off_bad;     // per-tile out-of-range counts [batch * H_kv * T64]
  int64_t off_segp;    // first pass of each bin [nbins + 1]
  int64_t off_pass;    // pass descriptors [max_passes]
  int64_t off_cnt;     // per-(seq, tile, bin) counts, then column prefixes
  int64_t words;       // total size in words
};
// Header words at the start of the scratch buffer.
enum { kHdrEntries = 0, kHdrBad = 1, kHdrPasses = 2, kHdrWords = 64 };

// One attention pass: entries [start, start + cnt) of blk_entries, all in
// bin (seq, blk).
struct PassDesc {
  int32_t start, cnt, seq, blk;
};

// bk: tokens per key block (32, 64 or 128).
SchedLayout sched_layout(int batch, int H_kv, int G, int k, int64_t q_begin, int64_t q_count,
                         int bk = kBk);

hipError_t launch_invert(const int32_t* block_idx, int batch, int H_kv, int G, int k,
                         int64_t q_begin, int64_t q_count, int32_t* blk_offsets,
                         int32_t* blk_entries, int32_t* sched, hipStream_t stream, int bk = kBk);

// Multiply-high reciprocal of a slot count d <= 32 (exact for 31-bit
// dividends): n / d == umulhi(n, magic) >> shift for d >= 2.
void kdiv_params(int d, uint32_t* magic, int* shift);

// H_sel selection groups of G query heads each; group r reads K/V head
// r >> kv_shift (H_kv = H_sel >> kv_shift: the ratio is a power of two).
hipError_t launch_sparse_attn(const void* q, const void* k, const void* v, bool fp8, int batch,
                              int64_t N, int H_sel, int G, int kv_shift, int kslots, float scale_log2,
                              float out_scale, const int32_t* blk_offsets,
                              const int32_t* blk_entries, const int32_t* sched, int64_t q_begin,
                              int64_t q_count, uint16_t* o_part, float* lse_part,
                              hipStream_t stream, int bk = kBk);

// Slots whose id is outside [0, floor(i / bk)] (i the query's position) are
// left out, like the inversion leaves them out; bk = 0 checks only id >= 0.
hipError_t launch_combine(const int32_t* block_idx, const uint16_t* o_part, const float* lse_part,
                          int batch, int64_t N, int H_kv, int G, int k, int64_t q_begin,
                          int64_t q_count, uint16_t* o, float* lse, hipStream_t stream, int bk);

// Dense causal GQA attention (bf16), query rows [q_begin, q_begin + q_count):
// o [batch][N][H_q][d_h], lse [batch][N][H_q] (natural log; may be null).
hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int batch,
                             int64_t N, int H_kv, int G, int64_t q_begin, int64_t q_count,
                             float scale_log2, uint16_t* o, float* lse, hipStream_t stream);

// Decode: one query per sequence (its last token) against cached K, V, K^idx;
// lens (device, [batch], may be null = N for all) gives each sequence's
// length within the N cache slots.
// H_sel selection groups (index heads) of G query heads, group r reading K/V
// head r >> kv_shift.  q [batch][H_q][d_h], q_idx [batch][H_sel][d_idx],
// caches as for the prefill; scores [batch][H_sel][ceil(N / B_k)] fp32,
// block_idx [batch][H_sel][k], o_part [batch][H_sel][k][G][d_h],
// lse_part [batch][H_sel][k][G] are scratch (block_idx is also an output);
// o [batch][H_q][d_h], lse [batch][H_q] or null.
hipError_t launch_decode(const uint16_t* q, const uint16_t* q_idx, const uint16_t* k, const uint16_t* v,
                         const uint16_t* k_idx, int batch, int64_t N, int H_sel, int G, int kv_shift, int d_idx,
                         int kslots, float scale_log2, float* scores, int32_t* block_idx,
                         uint16_t* o_part, float* lse_part, uint16_t* o, float* lse,
                         hipStream_t stream, int bk = kBk, const int32_t* lens = nullptr);

// Backward pass over one query range [q_begin, q_begin + q_count) with 128-token
// blocks.  block_idx holds the range's selection rows [batch][H_sel][q_count][k]
// and entries / sched the inversion launch_invert built from them.  dk_acc,
// dv_acc [batch][N][H_kv][d_h] and dki_acc [batch][N][d_idx] are fp32
// accumulators (atomically added to); dq [batch][N][H_q][d_h], dq_idx
// [batch][N][H_sel][d_idx] (bf16) and kl [batch][H_sel][N] receive the range's
// rows.  The rest is scratch: dlt [batch][N][H_q], lsei_part, kl_part
// [slots], lsei2 [batch][H_sel][q_count], dq_part [slots][G][d_h] (bf16),
// dqi_part [slots][d_idx].  index = false skips the index branch.
struct BwdArgs {
  const uint16_t *q, *k_ptr, *v, *dout, *o, *q_idx, *k_idx;
  const float* lse;
  const int32_t *block_idx, *entries, *sched;
  int batch;
  int64_t N;
  int H_sel, G, kv_shift, k, d_idx;
  int64_t q_begin, q_count;
  float scale, idx_scale, kl_weight;
  bool index;
  float *dlt, *lsei_part, *lsei2, *dqi_part, *kl_part, *dk_acc, *dv_acc, *dki_acc, *kl;
  float* tch;  // teacher rows per entry [slot][key], written by the main branch for the index branch
  uint16_t *dq_part, *dq, *dq_idx;
};
hipError_t launch_backward_chunk(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream);
hipError_t launch_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t stream);

}  // namespace msa
