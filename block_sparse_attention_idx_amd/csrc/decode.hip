// MSA decode: one new query per sequence (its last token, position len - 1)
// against cached K, V and K^idx of its len tokens (len = N for every
// sequence, or per-sequence lengths in caches of N slots).
//
// What is computed (the same definitions as the prefill, for row i = N - 1):
//  * index branch ("MiniMax Sparse Attention (MSA)", Deep Dive > Index Branch
//    Architecture and Exp-Free TopK Kernel; Training Stability Mechanisms):
//    every earlier key block b < L = floor((N - 1) / B_k) scores
//    max_{j in b} Q^idx[r] . K^idx[j] (unscaled, fp32 sums of exact bf16
//    products); the k - 1 best blocks join the local block L;
//  * main branch ("MiniMax Sparse Attention", sec. 2.1-2.2): the G query
//    heads of group r attend with exact softmax to the tokens of the
//    selected blocks (all of them visible: the query is the last token);
//  * the per-block partials are merged by log-sum-exp ("MiniMax Sparse
//    Attention (MSA)", Deep Dive > KV-Outer Sparse Attention, step 6) with
//    the prefill's combine kernel.
// The decode form is the query-stationary one ("Optimizing MiniMax M3 Sparse
// Attention on NVIDIA Blackwell", sec. 1: with one query the tile height is
// the GQA factor), split over the selected blocks so that every block is read
// by its own workgroup.
//
// gfx950 design.  Decode is bound by HBM, and the index scan dominates: it
// reads the whole K^idx cache (256 B per token at d_idx = 128), while the main
// branch reads k blocks of K and V per group.
//  * Scores: waves stride over the (sequence, block) pairs; a wave scores one
//    block for all groups at once with v_mfma_f32_32x32x16_bf16 (keys on the
//    row dimension, the H_sel <= 32 index query heads on the columns), the
//    block's K^idx fragments loaded straight from memory, all 32 KB requested
//    before the first MFMA (each 256-byte row is read by two lanes, 16 bytes
//    per step); the block max is an in-lane max plus one half-wave exchange.
//    Block scores go to a small fp32 buffer [batch][H_sel][B].
//  * Top-k: one workgroup per (sequence, group); each thread keeps the best
//    (score, block) keys of its strided share in VGPRs, then the lists are
//    merged pairwise (a bitonic merge in registers per round, the partner
//    list read from LDS).  A 64-bit key (order-preserving score bits, then the
//    complemented block id) makes "higher score, then smaller id" a plain
//    unsigned comparison.
//  * Partials: one 512-thread workgroup per (sequence, group, slot) stages
//    the selected K/V block into LDS (the shared tile layout) and one wave
//    computes S^T = K Q^T for the G heads, the softmax and O^T = V^T P^T.
#include <limits.h>

#include "attn_tile.h"
#include "msa_internal.h"

namespace msa {
namespace {

using namespace tile;

constexpr int kScoreWaves = 4;  // key blocks per scoring workgroup

// Tokens of sequence b: its entry of the per-sequence lengths (clamped to
// [1, N]), or the cache length N for all when there are none.
__device__ __forceinline__ int64_t seq_len_of(const int32_t* __restrict__ lens, int b, int64_t N) {
  if (lens == nullptr) return N;
  const int64_t l = lens[b];
  return l < 1 ? 1 : (l > N ? N : l);
}

// Order-preserving map of an fp32 score (no NaN) onto uint32.
__device__ __forceinline__ uint32_t ord_score(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// KT: 32-key tiles per key block (blocks of 32 KT tokens).
template <int DIDX, int KT>
__global__ __launch_bounds__(64 * kScoreWaves) void decode_scores_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, int64_t N, int H_sel,
    int L, int B, int batch, const int32_t* __restrict__ lens, float* __restrict__ scores) {
  constexpr int STEPS = DIDX / 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31, h = lane >> 5;
  const int64_t items = static_cast<int64_t>(batch) * L;  // (sequence, block) pairs
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kScoreWaves;
  // Each wave strides over the pairs; consecutive waves take consecutive
  // blocks of one sequence.  No barrier in this kernel.
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * kScoreWaves + wave; it < items; it += nwaves) {
    const int bat = static_cast<int>(it / L), blk = static_cast<int>(it % L);
    // blocks from this sequence's own local block on are not candidates
    if (lens != nullptr && blk >= static_cast<int>((seq_len_of(lens, bat, N) - 1) / (32 * KT))) continue;
    // All 4 key tiles' A fragments (row 32 mt + n, dims 16 ks + 8 h .. + 7)
    // are requested before any is used.
    const uint16_t* kb = k_idx + (static_cast<int64_t>(bat) * N + static_cast<int64_t>(blk) * (32 * KT) + n) * DIDX + 8 * h;
    u32x4 kf[KT][STEPS];
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) {
#pragma unroll
      for (int ks = 0; ks < STEPS; ++ks)
        kf[mt][ks] = *reinterpret_cast<const u32x4*>(kb + 32 * mt * DIDX + 16 * ks);
    }
    // B operand: column n = index query head n (zero past H_sel).
    const uint16_t* qrow = q_idx + (static_cast<int64_t>(bat) * H_sel + min(n, H_sel - 1)) * DIDX;
    bf16x8 qf[STEPS];
#pragma unroll
    for (int ks = 0; ks < STEPS; ++ks) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * h);
      qf[ks] = as_bf16x8(n < H_sel ? w : u32x4{0u, 0u, 0u, 0u});
    }
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < STEPS; ++ks) acc = mfma32x32x16(as_bf16x8(kf[mt][ks]), qf[ks], acc);
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[e]);
    }
    mx = halves_max(mx);
    if (h == 0 && n < H_sel) scores[(static_cast<int64_t>(bat) * H_sel + n) * B + blk] = mx;
  }
}

constexpr int kTopkBatch = 8;  // candidates a thread requests before inserting
// Threads of the top-k workgroup: few merge rounds matter more than short
// per-thread scans (each round is a 64-bit bitonic merge in every active lane).
template <int KP>
constexpr int topk_threads() { return 256; }

// Insert key x into the descending list v[0..KP) (v[KP - 1] the smallest).
template <int KP>
__device__ __forceinline__ void insert_desc(uint64_t (&v)[KP], uint64_t x) {
#pragma unroll
  for (int j = 0; j < KP; ++j) {
    const uint64_t t = v[j];
    const bool sw = x > t;
    v[j] = sw ? x : t;
    x = sw ? t : x;
  }
}

// KP (a power of two >= k - 1) best keys per thread, then log2(threads) merge
// rounds: list t takes the best KP of lists t and t + s.  A thread first
// requests all its candidates (up to kTopkBatch per pass), then inserts them,
// so the score loads are not serialised behind the insertions.  A merge is
// compile-time indexed: the elementwise max of one descending list and the
// other reversed holds the KP largest keys as a bitonic sequence, which a
// bitonic merge sorts descending.  Partner lists go through LDS entry-major
// (conflict-free).
template <int KP>
__global__ __launch_bounds__(topk_threads<KP>()) void decode_topk_kernel(const float* __restrict__ scores,
                                                                         int L_all, int B, int k,
                                                                         const int32_t* __restrict__ lens,
                                                                         int64_t N, int H_sel, int bk,
                                                                         int32_t* __restrict__ block_idx) {
  constexpr int kTopkThreads = topk_threads<KP>();
  __shared__ uint64_t lists[KP * kTopkThreads / 2];
  const int seq = blockIdx.x;  // batch * H_sel + r
  // this sequence's local block
  const int L = lens == nullptr ? L_all : static_cast<int>((seq_len_of(lens, seq / H_sel, N) - 1) / bk);
  const int t = threadIdx.x;
  const float* row = scores + static_cast<int64_t>(seq) * B;

  uint64_t v[KP];
#pragma unroll
  for (int j = 0; j < KP; ++j) v[j] = 0;  // below every real key
  for (int b0 = t; b0 < L; b0 += kTopkThreads * kTopkBatch) {
    float sc[kTopkBatch];
#pragma unroll
    for (int u = 0; u < kTopkBatch; ++u) {
      const int b = b0 + u * kTopkThreads;
      sc[u] = row[b < L ? b : 0];
    }
#pragma unroll
    for (int u = 0; u < kTopkBatch; ++u) {
      const int b = b0 + u * kTopkThreads;
      const uint64_t key = b < L ? (static_cast<uint64_t>(ord_score(sc[u])) << 32) |
                                       (0xFFFFFFFFu - static_cast<uint32_t>(b))
                                 : 0;
      if (key > v[KP - 1]) insert_desc<KP>(v, key);
    }
  }
  for (int s = kTopkThreads / 2; s > 0; s >>= 1) {
    if (t >= s && t < 2 * s) {
#pragma unroll
      for (int j = 0; j < KP; ++j) lists[j * (kTopkThreads / 2) + (t - s)] = v[j];
    }
    __syncthreads();
    if (t < s) {
      uint64_t m[KP];
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const uint64_t x = v[j], y = lists[(KP - 1 - j) * (kTopkThreads / 2) + t];
        m[j] = x > y ? x : y;
      }
#pragma unroll
      for (int st = KP / 2; st > 0; st >>= 1) {
#pragma unroll
        for (int i = 0; i < KP; ++i) {
          if ((i & st) == 0) {
            const uint64_t x = m[i], y = m[i + st];
            m[i] = x > y ? x : y;
            m[i + st] = x > y ? y : x;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < KP; ++j) v[j] = m[j];
    }
    __syncthreads();
  }
  if (t == 0) {
    // Ascending ids of the k - 1 best (fewer when there are fewer earlier
    // blocks), then L, then -1.  Odd-even transposition sort, compile-time
    // indices.
    int ids[KP];
    int nv = 0;
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      ids[j] = (v[j] != 0 && j < k - 1) ? static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(v[j])) : INT_MAX;
      nv += ids[j] != INT_MAX ? 1 : 0;
    }
#pragma unroll
    for (int round = 0; round < KP; ++round) {
#pragma unroll
      for (int i = round & 1; i + 1 < KP; i += 2) {
        const int a = ids[i], c = ids[i + 1];
        ids[i] = min(a, c);
        ids[i + 1] = max(a, c);
      }
    }
    int32_t* dst = block_idx + static_cast<int64_t>(seq) * k;
#pragma unroll
    for (int j = 0; j <= KP; ++j) {
      if (j < k) dst[j] = j < nv ? ids[j < KP ? j : 0] : (j == nv ? L : -1);
    }
  }
}

// Partial attention of the G heads of group r over selected slot s.
template <int G>
__global__ __launch_bounds__(kStageThreads, 1) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t N, int H_sel, int kv_shift, int kslots, int bk, const int32_t* __restrict__ lens, float scale_log2,
    const int32_t* __restrict__ block_idx,
    uint16_t* __restrict__ o_part, float* __restrict__ lse_part) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kBufBytes];
  const int64_t item = blockIdx.x;  // (seq, slot)
  const int64_t seq = item / kslots;
  const int blk = block_idx[item];
  if (blk < 0) return;  // uniform: empty slot, skipped by the combine
  const int bat = static_cast<int>(seq / H_sel), r = static_cast<int>(seq % H_sel);
  const int H_kv = H_sel >> kv_shift;  // selection group r reads K/V head r >> kv_shift
  const int tid = threadIdx.x;
  // Blocks of bk <= 128 tokens sit at the start of the 128-key tile; the keys
  // after them (and past the sequence end) are zero and hidden below.
  const int nvalid = static_cast<int>(min<int64_t>(bk, seq_len_of(lens, bat, N) - static_cast<int64_t>(blk) * bk));
  const int64_t rstride = static_cast<int64_t>(H_kv) * kDh * 2;
  const int64_t row0 = (static_cast<int64_t>(bat) * N + static_cast<int64_t>(blk) * bk) * H_kv + (r >> kv_shift);
  KVRegs R;
  kv_load(R, reinterpret_cast<const uint8_t*>(k) + row0 * kDh * 2,
          reinterpret_cast<const uint8_t*>(v) + row0 * kDh * 2, rstride, nvalid, tid);
  kv_store(R, lds, nvalid, tid);
  __syncthreads();
  if (tid >= 64) return;  // one wave computes (no barrier follows)

  const int lane = tid, n = lane & 31, h = lane >> 5;
  const int H_q = H_sel * G;
  // B operand: column n = head r G + n (zero past G).
  const uint16_t* qrow = q + (static_cast<int64_t>(bat) * H_q + r * G + min(n, G - 1)) * kDh;
  u32x4 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * h);
    qf[ks] = n < G ? w : u32x4{0u, 0u, 0u, 0u};
  }
  // S^T = K Q^T: acc[mt] holds keys 32 mt + 8 (e / 4) + 4 h + (e % 4) of head n.
  const uint8_t* kfr = lds + n * kStr + h * 16;
  f32x16 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      acc[mt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(kfr + 32 * mt * kStr + 32 * ks)),
                             as_bf16x8(qf[ks]), acc[mt]);
  }
  // Keys past the end of the sequence (a partial last block) are hidden; the
  // query is the last token, so every other key is visible.
  if (nvalid < kBk) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int el = 0; el < 16; ++el) {
        const int key = 32 * mt + 8 * (el >> 2) + 4 * h + (el & 3);
        if (key >= nvalid) acc[mt][el] = -__builtin_huge_valf();
      }
    }
  }
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int el = 0; el < 16; ++el) m = fmaxf(m, acc[mt][el]);
  }
  const float mb = halves_max(m) * scale_log2;
  bf16x8 pf[8];
  float l = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mt][8 * e2 + 2 * j], scale_log2, -mb));
        const float pb = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mt][8 * e2 + 2 * j + 1], scale_log2, -mb));
        w[j] = pack_bf16x2(pa, pb);
        l += pa + pb;
      }
      pf[2 * mt + e2] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
    }
  }
  l = halves_sum(l);
  const float inv = __builtin_amdgcn_rcpf(l);
  // O^T = V^T P^T: lane (n, h) receives dims 64 h + 16 dt + e of head n.
  const int dsel = 64 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  const uint8_t* vfr = lds + kVtOff + dvt_row(dsel) * kStr + h * 16;
  uint16_t* orow = o_part + (item * G + min(n, G - 1)) * kDh + 64 * h;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    f32x16 oa = {};
#pragma unroll
    for (int st = 0; st < 8; ++st)
      oa = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(vfr + 32 * dt * kStr + 32 * st)), pf[st], oa);
    if (n < G) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int b8 = 8 * hf;
        *reinterpret_cast<u32x4*>(orow + 16 * dt + 8 * hf) =
            u32x4{pack_bf16x2(oa[b8 + 0] * inv, oa[b8 + 1] * inv), pack_bf16x2(oa[b8 + 2] * inv, oa[b8 + 3] * inv),
                  pack_bf16x2(oa[b8 + 4] * inv, oa[b8 + 5] * inv), pack_bf16x2(oa[b8 + 6] * inv, oa[b8 + 7] * inv)};
      }
    }
  }
  if (h == 0 && n < G) lse_part[item * G + n] = (mb + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
}

template <int KP>
hipError_t launch_topk(const float* scores, int nseq, int L, int B, int k, const int32_t* lens, int64_t N,
                       int H_sel, int bk, int32_t* block_idx, hipStream_t stream) {
  hipLaunchKernelGGL(decode_topk_kernel<KP>, dim3(static_cast<unsigned>(nseq)), dim3(topk_threads<KP>()), 0,
                     stream, scores, L, B, k, lens, N, H_sel, bk, block_idx);
  return hipGetLastError();
}

template <int G>
hipError_t launch_partial(const uint16_t* q, const uint16_t* k, const uint16_t* v, int batch, int64_t N,
                          int H_sel, int kv_shift, int kslots, int bk, const int32_t* lens, float scale_log2,
                          const int32_t* block_idx,
                          uint16_t* o_part, float* lse_part, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(batch) * H_sel * kslots;
  hipLaunchKernelGGL(decode_partial_kernel<G>, dim3(static_cast<unsigned>(items)), dim3(kStageThreads), 0,
                     stream, q, k, v, N, H_sel, kv_shift, kslots, bk, lens, scale_log2, block_idx, o_part, lse_part);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const uint16_t* q, const uint16_t* q_idx, const uint16_t* k, const uint16_t* v,
                         const uint16_t* k_idx, int batch, int64_t N, int H_sel, int G, int kv_shift, int d_idx,
                         int kslots, float scale_log2, float* scores, int32_t* block_idx,
                         uint16_t* o_part, float* lse_part, uint16_t* o, float* lse,
                         hipStream_t stream, int bk, const int32_t* lens) {
  const int B = static_cast<int>((N + bk - 1) / bk);
  // the local block of a full-length sequence; blocks 0 .. L - 1 are scored
  // (a shorter sequence scores only the blocks before its own local block)
  const int L = static_cast<int>((N - 1) / bk);
  const int nseq = batch * H_sel;
  hipError_t e = hipSuccess;
  if (L > 0) {
    // A few waves per SIMD, each striding over many blocks.
    const int64_t items = static_cast<int64_t>(batch) * L;
    int64_t wgs = (items + kScoreWaves - 1) / kScoreWaves;
    if (wgs > 1024) wgs = 1024;
    const dim3 g(static_cast<unsigned>(wgs)), t(64 * kScoreWaves);
#define MSA_DEC_SCORES(D, KT) \
  hipLaunchKernelGGL((decode_scores_kernel<D, KT>), g, t, 0, stream, q_idx, k_idx, N, H_sel, L, B, batch, lens, scores)
    if (d_idx == 64) {
      if (bk == 32) MSA_DEC_SCORES(64, 1);
      else if (bk == 64) MSA_DEC_SCORES(64, 2);
      else MSA_DEC_SCORES(64, 4);
    } else {
      if (bk == 32) MSA_DEC_SCORES(128, 1);
      else if (bk == 64) MSA_DEC_SCORES(128, 2);
      else MSA_DEC_SCORES(128, 4);
    }
#undef MSA_DEC_SCORES
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int km = kslots - 1;
  if (km <= 1) e = launch_topk<1>(scores, nseq, L, B, kslots, lens, N, H_sel, bk, block_idx, stream);
  else if (km <= 2) e = launch_topk<2>(scores, nseq, L, B, kslots, lens, N, H_sel, bk, block_idx, stream);
  else if (km <= 4) e = launch_topk<4>(scores, nseq, L, B, kslots, lens, N, H_sel, bk, block_idx, stream);
  else if (km <= 8) e = launch_topk<8>(scores, nseq, L, B, kslots, lens, N, H_sel, bk, block_idx, stream);
  else if (km <= 16) e = launch_topk<16>(scores, nseq, L, B, kslots, lens, N, H_sel, bk, block_idx, stream);
  else e = launch_topk<32>(scores, nseq, L, B, kslots, lens, N, H_sel, bk, block_idx, stream);
  if (e != hipSuccess) return e;
  switch (G) {
    case 1: e = launch_partial<1>(q, k, v, batch, N, H_sel, kv_shift, kslots, bk, lens, scale_log2, block_idx, o_part, lse_part, stream); break;
    case 2: e = launch_partial<2>(q, k, v, batch, N, H_sel, kv_shift, kslots, bk, lens, scale_log2, block_idx, o_part, lse_part, stream); break;
    case 4: e = launch_partial<4>(q, k, v, batch, N, H_sel, kv_shift, kslots, bk, lens, scale_log2, block_idx, o_part, lse_part, stream); break;
    case 8: e = launch_partial<8>(q, k, v, batch, N, H_sel, kv_shift, kslots, bk, lens, scale_log2, block_idx, o_part, lse_part, stream); break;
    case 16: e = launch_partial<16>(q, k, v, batch, N, H_sel, kv_shift, kslots, bk, lens, scale_log2, block_idx, o_part, lse_part, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // One query row per sequence: the combine's output rows [batch][1][H_q].
  return launch_combine(block_idx, o_part, lse_part, batch, 1, H_sel, G, kslots, 0, 1, o, lse, stream, 0);
}

}  // namespace msa
