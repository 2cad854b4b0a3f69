// KV-outer block-sparse attention (main branch of MSA).
//
// What is computed ("MiniMax Sparse Attention", sec. 2.2 and 4.2;
// "MiniMax Sparse Attention (MSA)", Deep Dive > KV-Outer Sparse Attention):
// for every (sequence, group r, key block b) bin of the inverted index, the K
// and V rows of block b (head r) are staged in LDS once, and every (query i,
// head g of group r) that selected the block gets the block's partial softmax
// attention over its causally visible tokens:
//     Obar = sum_j softmax(s)_j V_j,  lse = ln sum_j exp(s_j),
//     s_j = scale * Q[i, rG+g] . K[j, r],  j in block b, j <= i.
// The causal mask only bites when b is the query's own block.  One (Obar, lse)
// pair per (query, slot, head) goes to the partial buffers, merged afterwards
// by the combine kernel.
//
// gfx950 design:
//  * Persistent grid, one workgroup of 8 waves per CU (two waves per SIMD).
//    The work list is a flat array of pass descriptors (entry start, count,
//    group, block) built by the inversion, ordered (sequence, block); the
//    workgroups take the sequences in order and each takes an equal
//    contiguous share of every sequence's passes: every workgroup gets the
//    same work whatever the block popularity, and a K/V block is staged only
//    when consecutive passes change block.
//  * A pass is 256 (query, head) rows: 256 / G entries x G heads (a query's G
//    heads are contiguous in Q, 256 B each); each wave owns one 32-row MFMA
//    column tile.  K (row-major) and V (transposed) live in padded LDS
//    (68 KB), shared by the 8 waves.
//  * S^T = K_b * Q^T with v_mfma_f32_32x32x16_bf16 (keys on the row
//    dimension): every lane holds 64 of the 128 keys of one (query, head) row,
//    so the row max and row sum need one half-wave exchange, and the
//    probabilities feed O^T = V^T * P^T directly as the MFMA B operand with no
//    shuffle (the reduction slots of each P^T step are exactly the keys that
//    lane already holds).  The V^T operand rows are permuted so that every
//    lane ends up with 64 contiguous output dimensions of its row.
//  * The partial outputs go through an 8.5 KB LDS tile per wave: written in
//    the MFMA layout (lane = row), read back row-contiguous, and stored 1 KB
//    contiguous per instruction (non-temporal), so L2 receives whole 128-byte
//    lines rather than 16-byte pieces of 64 different rows.
//  * Software pipeline over passes: while pass p computes, the Q rows of pass
//    p+1 are gathered into registers and the entry of pass p+2 is read; the
//    scores of pass p+1 follow pass p's P V.  One register set each for Q and
//    the scores (194 VGPRs in the bf16 kernel), which leaves the scheduler
//    room to keep LDS fragment reads ahead of their MFMAs.  Every memory
//    operation of the loop is issued unconditionally, so the compiler's
//    in-order vmcnt waits never have to cover the stores or the loads just
//    issued.
//  * Softmax in base 2 (v_exp_f32) with the scale folded into one FMA, its
//    exponentials interleaved with the P V MFMAs of the previous key step.  fp8
//    (OCP e4m3) inputs: the scores come from v_mfma_scale_f32_32x32x64_f8f6f4
//    on the Q and K codes (exact products, K kept as codes in LDS), V is
//    widened exactly to bf16 when staged (P V stays a bf16 product), and the
//    per-tensor scales are folded into the softmax scale and the output scale.
#include "attn_tile.h"
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kWaves = kAttnWaves;
constexpr int kThreads = 64 * kWaves;

// LDS layouts.  Rows are padded rather than swizzled so that every fragment
// read of a lane is one base address plus a compile-time offset (no per-read
// address registers).  K and V^T use the shared tile layout (attn_tile.h):
//  * K row-major, 272 B per key row: a 16-lane phase of 16-byte reads of rows
//    n .. n + 15 starts at banks 4n + const, all distinct.
//  * V^T, 272 B per output-dimension row, row d stored at position
//    2 (d mod 64) + d / 64, so that the 32 rows one operand read touches
//    (d in 0..15 and 64..79, plus 16 dt) are 32 consecutive rows.  Within a
//    row, bits 2 and 3 of the key index are swapped: the 8 keys
//    16 s + 8 h' + 4 a + b (h', a, b: lane half, chunk, key in chunk) that
//    one lane feeds to P^T step s, keys 16 s + 8 a + 4 h' + b, lie in one
//    16-byte chunk.
//  * Output tile, 272 B per row: 16-byte writes of rows n .. n + 15 and
//    16-byte reads of the 16 chunks of one row are both conflict free.
constexpr int kKStride = tile::kStr;
// fp8: K stays as e4m3 codes, 144 B per key row (128 codes + 16 B): the
// 16-byte reads of rows n .. n + 15 start at banks 36 n mod 64, all distinct.
constexpr int kK8Stride = 144;
constexpr int kVStride = tile::kStr;
constexpr int kOStride = tile::kStr;

__device__ __forceinline__ int k_lds_off(int key, int c) {  // 16-byte chunk c of key row
  return key * kKStride + c * 16;
}

using tile::bf16_of;
using tile::dvt_off;
using tile::dvt_row;
using tile::halves_max;
using tile::halves_sum;

// Stage K (row-major) and V (transposed) of one block of one head into LDS,
// with the kThreads threads of the workgroup.
template <bool FP8>
__device__ __forceinline__ void stage_kv(const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb,
                                         int64_t rstride, int nvalid, uint8_t* k_lds,
                                         uint8_t* vt_lds) {
  // Staging is rare (once per run of passes on a block); an opaque copy of the
  // thread id keeps the compiler from hoisting its per-lane addresses out of
  // the caller's loop, where they would stay live across every pass.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  // Rows past the end of the sequence (a partial last block) are read from the
  // last valid row and replaced by zeros, so every load is issued at once.
  if constexpr (!FP8) {
    // 128 keys x 16 chunks of 16 bytes
    constexpr int R = kBk * 16 / kThreads;
    u32x4 w[R];
#pragma unroll
    for (int p = 0; p < R; ++p) {
      const int key = (tid >> 4) + (kThreads / 16) * p, c = tid & 15;
      w[p] = *reinterpret_cast<const u32x4*>(kb + min(key, nvalid - 1) * rstride + c * 16);
    }
#pragma unroll
    for (int p = 0; p < R; ++p) {
      const int key = (tid >> 4) + (kThreads / 16) * p, c = tid & 15;
      if (key >= nvalid) w[p] = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(k_lds + k_lds_off(key, c)) = w[p];
    }
  } else {
    // 128 keys x 8 chunks of 16 codes
    constexpr int R = kBk * 8 / kThreads;
    u32x4 wk[R];
#pragma unroll
    for (int p = 0; p < R; ++p) {
      const int key = (tid >> 3) + (kThreads / 8) * p, cc = tid & 7;
      wk[p] = *reinterpret_cast<const u32x4*>(kb + min(key, nvalid - 1) * rstride + cc * 16);
    }
#pragma unroll
    for (int p = 0; p < R; ++p) {
      const int key = (tid >> 3) + (kThreads / 8) * p, cc = tid & 7;
      *reinterpret_cast<u32x4*>(k_lds + key * kK8Stride + cc * 16) = key < nvalid ? wk[p] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // V: item (dg, kc) transposes the 8 dims 8 dg .. 8 dg + 7 of keys
  // 4 kc .. 4 kc + 3 into four-key chunks of V^T rows; 16 x 32 items.
#pragma unroll
  for (int it = 0; it < 512 / kThreads; ++it) {
    const int item = tid + kThreads * it;
    const int kc = item & 31, dg = item >> 5;
    u32x4 rows[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = min(4 * kc + j, nvalid - 1);
      if constexpr (!FP8) {
        rows[j] = *reinterpret_cast<const u32x4*>(vb + key * rstride + dg * 16);
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(vb + key * rstride + dg * 8);
        rows[j] = u32x4{w[0], w[1], 0u, 0u};
      }
    }
    u32x4 row[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (4 * kc + j >= nvalid) {
        row[j] = u32x4{0u, 0u, 0u, 0u};
      } else if constexpr (!FP8) {
        row[j] = rows[j];
      } else {
        const u32x2 a = e4m3x4_to_bf16x4_int(rows[j][0]), b = e4m3x4_to_bf16x4_int(rows[j][1]);
        row[j] = u32x4{a[0], a[1], b[0], b[1]};
      }
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int d = 8 * dg + dd;
      const u32x2 v = {bf16_of(row[0], dd) | (bf16_of(row[1], dd) << 16),
                       bf16_of(row[2], dd) | (bf16_of(row[3], dd) << 16)};
      *reinterpret_cast<u32x2*>(vt_lds + dvt_off(d, kc)) = v;
    }
  }
}

// Q fragments (B operand of S^T) of one row, kept as loaded, so a prefetch is
// never waited on before its pass: bf16 dims 16 ks + 8 h .. + 7 (8 x 16 B),
// fp8 codes as below.  V is widened once per staging with integer arithmetic
// (the conversion instruction there made the compiler spill).
template <bool FP8>
struct QFrag;
template <>
struct QFrag<false> {
  u32x4 w[8];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ qr, int h) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) w[ks] = *reinterpret_cast<const u32x4*>(qr + (16 * ks + 8 * h) * 2);
  }
  __device__ __forceinline__ bf16x8 get(int ks) const { return as_bf16x8(w[ks]); }
};
// fp8: the codes of dims 64 s + 32 h .. + 31 (s = 0, 1), the B operand of
// one v_mfma_scale_f32_32x32x64_f8f6f4 each.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ i32x8 as_i32x8(const u32x4& a, const u32x4& b) {
  return i32x8{static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]), static_cast<int>(a[3]),
               static_cast<int>(b[0]), static_cast<int>(b[1]), static_cast<int>(b[2]), static_cast<int>(b[3])};
}
template <>
struct QFrag<true> {
  u32x4 w[4];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ qr, int h) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      w[2 * s] = *reinterpret_cast<const u32x4*>(qr + 64 * s + 32 * h);
      w[2 * s + 1] = *reinterpret_cast<const u32x4*>(qr + 64 * s + 32 * h + 16);
    }
  }
  __device__ __forceinline__ i32x8 get8(int s) const { return as_i32x8(w[2 * s], w[2 * s + 1]); }
};

// BKS: log2 of the key block size.  Blocks of 32 or 64 tokens (the paper's
// block-size ablation) stage their tokens into the 128-key tile with zeros
// after them; the key tiles past the block are left out of the scores, the
// softmax and P V at compile time.
template <int G, bool FP8, int BKS>
__global__ __launch_bounds__(kThreads, 1) void sparse_attn_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    int64_t N, int H_sel, int kv_shift, int kslots, uint32_t kdiv_magic, int kdiv_shift, float scale_log2,
    float out_scale, const int32_t* __restrict__ entries, const int32_t* __restrict__ segp,
    const PassDesc* __restrict__ passes, int B_c, int nseqs, int q_begin, int q_count,
    uint16_t* __restrict__ o_part, float* __restrict__ lse_part) {
  constexpr int EB = FP8 ? 1 : 2;  // bytes per Q/K/V element
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kBk * kKStride];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[kDh * kVStride];
  __shared__ __attribute__((aligned(16))) uint8_t o_lds[kWaves * 32 * kOStride];
  __shared__ __attribute__((aligned(8))) int64_t orow_lds[kWaves * 32];

  // This workgroup's passes: the sequences (seq = batch * H_sel + group) in
  // order, and in each one contiguous, equal share of its passes.
  // next_pass() returns the next pass index, or -1 when the shares are
  // exhausted (and from then on).
  int it_seq = -1, it_p = 0, it_end = 0;
  auto next_pass = [&]() -> int {
    if (++it_p < it_end) return it_p;
    while (++it_seq < nseqs) {
      const int a = segp[it_seq * B_c];
      const int64_t np = segp[(it_seq + 1) * B_c] - a;
      const int s0 = a + static_cast<int>(np * blockIdx.x / gridDim.x);
      const int s1 = a + static_cast<int>(np * (blockIdx.x + 1) / gridDim.x);
      if (s0 < s1) {
        it_p = s0;
        it_end = s1;
        return s0;
      }
    }
    return -1;
  };
  const int i0 = next_pass();
  if (i0 < 0) return;  // uniform

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int H_q = H_sel * G;

  // Output dimension of V^T operand row n in d-tile 0 (d-tile dt adds 16 dt;
  // see the output step below), and the lane's fragment base addresses.
  const int dsel = 64 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  const uint8_t* k_base = k_lds + n * kKStride + h * 16;
  const uint8_t* v_base = vt_lds + dvt_row(dsel) * kVStride + h * 16;
  uint8_t* o_tile = o_lds + wave * 32 * kOStride;
  int64_t* orow_tile = orow_lds + wave * 32;
  const int rho = 32 * wave + n;     // this lane's row of the pass
  const int e_row = rho / G, g_row = rho % G;

  // Per-lane row of a pass.  An entry holds qrow * k + slot; the division by
  // k is a multiply-high by the host's round-up reciprocal.  A row past the
  // pass's entries takes the pass's first entry (same head): it recomputes
  // that row bit for bit, so its stores repeat that row's stores.
  struct RowRef {
    const uint8_t* q;  // the row's Q vector
    int64_t orow;      // partial-output row (seq, qrow, slot, g)
    int i;             // query position
  };
  auto row_ent = [&](const PassDesc& D) {  // raw entry word
    return static_cast<uint32_t>(entries[D.start + (e_row < D.cnt ? e_row : 0)]);
  };
  auto row_dec = [&](uint32_t ent, int seq) {
    RowRef rr;
    const uint32_t qrow = kslots == 1 ? ent : (__umulhi(ent, kdiv_magic) >> kdiv_shift);
    const uint32_t slot = ent - qrow * static_cast<uint32_t>(kslots);
    rr.i = q_begin + static_cast<int>(qrow);
    rr.orow = ((static_cast<int64_t>(seq) * q_count + qrow) * kslots + slot) * G + g_row;
    const int bat = seq / H_sel, r = seq - bat * H_sel;
    rr.q = static_cast<const uint8_t*>(qp) +
           ((static_cast<int64_t>(bat) * N + rr.i) * H_q + r * G + g_row) * static_cast<int64_t>(kDh) * EB;
    return rr;
  };

  auto stage = [&](const PassDesc& D) {
    const int64_t key0 = static_cast<int64_t>(D.blk) << BKS;
    // selection group r reads K/V head r >> kv_shift of the H_sel >> kv_shift heads
    const int bat = D.seq / H_sel, r = D.seq - bat * H_sel;
    const int H_kv = H_sel >> kv_shift;
    const int64_t rstride = static_cast<int64_t>(H_kv) * kDh * EB;
    const int64_t row0 = (static_cast<int64_t>(bat) * N + key0) * H_kv + (r >> kv_shift);
    stage_kv<FP8>(static_cast<const uint8_t*>(kp) + row0 * kDh * EB,
                  static_cast<const uint8_t*>(vp) + row0 * kDh * EB, rstride,
                  static_cast<int>(min<int64_t>(int64_t(1) << BKS, N - key0)), k_lds, vt_lds);
  };

  // S^T = K_b Q^T of one pass: acc[mt] holds keys 32mt + 8(e/4) + 4h + (e%4)
  // of this lane's row.
  // For fp8 the reduction step is the outer loop, so each widened Q fragment
  // is used by its four MFMAs and dies; for bf16 (no widening) the key tile.
  auto scores = [&](const QFrag<FP8>& q, f32x16(&acc)[4]) {
    // row 32 mt + n, 16-byte chunk 2 ks + h
    auto kfrag = [&](int mt, int ks) {
      return as_bf16x8(*reinterpret_cast<const u32x4*>(k_base + 32 * mt * kKStride + 32 * ks));
    };
    if constexpr (FP8) {
      // The e4m3 codes go straight into v_mfma_scale_f32_32x32x64_f8f6f4
      // (exact products, fp32 sums): lane (n, h) supplies key 32 mt + n and
      // row n with the same 32 dims 64 s + 32 h .. + 31, and both operands
      // carry the block scale 2^-8 (E8M0 code 119), the factor the widening
      // to bf16 applies to each value, so the scores are those of the bf16
      // path up to the order of the fp32 sums.
      const uint8_t* k8 = k_lds + n * kK8Stride + 32 * h;
      auto kfrag8 = [&](int mt, int s2) {
        const uint8_t* p = k8 + 32 * mt * kK8Stride + 64 * s2;
        return as_i32x8(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 16));
      };
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x16{};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const i32x8 qk = q.get8(s2);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kfrag8(mt, s2), qk, acc[mt], 0, 0, 0, 119,
                                                                    0, 119);
      }
    } else {
      // Rolling K fragments: the register that fed MFMA (mt, ks) is refilled
      // with fragment (mt + 1, ks) right after it, so every read has a whole
      // tile of MFMAs (8 x 32 cycles) to land; scheduling barriers keep each
      // read beside its MFMA (left alone, the scheduler sinks every read next
      // to its use and each MFMA waits out an LDS round trip).
      bf16x8 kf[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = kfrag(0, ks);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        acc[mt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          acc[mt] = mfma32x32x16(kf[ks], q.get(ks), acc[mt]);
          __builtin_amdgcn_sched_barrier(0);
          if (mt + 1 < 4) kf[ks] = kfrag(mt + 1, ks);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // The causal mask only bites in a query's own block, so it runs on a
  // wave-uniform branch taken by the few passes that hold such a row.  Key
  // 32mt + 8(e/4) + 4h + (e%4) is hidden when it lies past the query; the
  // lane part 4h moves to the limit so that the comparisons take constants.
  // The opaque statement keeps the branch a branch (not a select executed by
  // every pass), and the mask is a bit select on the sign of lim - key, which
  // needs no scalar condition registers.
  auto mask_own = [&](f32x16(&acc)[4], const RowRef& rr, int blk) {
    constexpr int BK = 1 << BKS;
    constexpr int MT = BK / 32;  // key tiles that hold the block's tokens
    // Smaller blocks: the zero keys BK .. 127 after the block are hidden in
    // every pass (compile-time tiles).
#pragma unroll
    for (int mt = MT; mt < 4; ++mt) acc[mt] = f32x16{} - __builtin_huge_valf();
    const bool own = blk == (rr.i >> BKS);
    if (__any(own)) {
      asm volatile("" ::: "memory");
      const int lim = (own ? rr.i - (blk << BKS) : BK - 1) - 4 * h;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int el = 0; el < 16; ++el) {
          const uint32_t hide = static_cast<uint32_t>((lim - (32 * mt + 8 * (el >> 2) + (el & 3))) >> 31);
          acc[mt][el] = __uint_as_float((__float_as_uint(acc[mt][el]) & ~hide) | (0xFF800000u & hide));
        }
      }
    }
  };

  // Softmax and O^T = V^T P^T in one walk over the keys.  Row maximum on the
  // raw scores, then the scale folded into one FMA before exp2; the row sum
  // adds the fp32 probabilities in key order, so lse is the exact
  // log-sum-exp up to fp32 rounding.  The two half-waves hold the two halves
  // of every row and swap partial results with one v_permlane32_swap.
  // P^T fragments (B operand of O^T = V^T P^T): step st = 2 mt + e2 covers
  // keys 32mt + 16e2 + 8(j/4) + 4h + (j%4), accumulator elements 8e2 .. +7.
  // Key tiles past a smaller block hold no keys: their probabilities are zero
  // and neither the softmax nor P V visits them.
  // After the maximum, fenced slot (st, dt) issues the P V MFMA of dims tile
  // dt on P step st and turns probability pair dt of step st + 1, so the
  // exponentials run beside the matrix cores; each V fragment is read two
  // slots ahead.  Lane (n, h) receives dims 64h + 16dt + el of its row and
  // writes them, scaled by 1/l, to the wave's tile: in the last key step each
  // dims tile goes out beside the next tile's MFMA (l is complete by then).
  constexpr int kMT = (1 << BKS) / 32;
  auto softmax_pv = [&](const f32x16(&acc)[4], float& lse2) {
    float m0 = -__builtin_huge_valf(), m1 = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
#pragma unroll
      for (int el = 0; el < 16; el += 4) {
        m0 = max3f(m0, acc[mt][el], acc[mt][el + 1]);
        m1 = max3f(m1, acc[mt][el + 2], acc[mt][el + 3]);
      }
    }
    // Rounded once and opaque: otherwise the compiler may contract the
    // product into the lse sum below (one fma instead of a multiply and an
    // add), which moves lse by an ulp depending on the schedule around it.
    float mb = halves_max(fmaxf(m0, m1)) * scale_log2;  // scale_log2 > 0
    asm volatile("" : "+v"(mb));
    constexpr int NS = 2 * kMT;  // P steps of 16 keys
    float l0 = 0.f, l1 = 0.f;
    // probability pair j of step st: keys of accumulator elements 8 e2 + 2j, + 1
    auto pair = [&](int st, int j) {
      const int mt = st >> 1, e2 = st & 1;
      const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mt][8 * e2 + 2 * j], scale_log2, -mb));
      const float pb = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[mt][8 * e2 + 2 * j + 1], scale_log2, -mb));
      l0 += pa;
      l1 += pb;
      return pack_bf16x2(pa, pb);
    };
    // V^T fragment i = 4 st + dt: row dsel + 16 dt (stored at dvt_row(dsel) +
    // 32 dt); keys 16 st + 8 h .. + 7, one 16-byte chunk in the permuted order
    auto vread = [&](int i) {
      return *reinterpret_cast<const u32x4*>(v_base + 32 * (i & 3) * kVStride + 32 * (i >> 2));
    };
    uint32_t w[2][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[0][j] = pair(0, j);
    u32x4 vr[3];
    vr[0] = vread(0);
    vr[1] = vread(1);
    f32x16 oa[4] = {};
    float inv = 0.f;
    auto out_tile = [&](int dt) {
      uint8_t* dst = o_tile + n * kOStride + 128 * h + 32 * dt;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int b8 = 8 * hf;
        *reinterpret_cast<u32x4*>(dst + 16 * hf) =
            u32x4{pack_bf16x2(oa[dt][b8 + 0] * inv, oa[dt][b8 + 1] * inv),
                  pack_bf16x2(oa[dt][b8 + 2] * inv, oa[dt][b8 + 3] * inv),
                  pack_bf16x2(oa[dt][b8 + 4] * inv, oa[dt][b8 + 5] * inv),
                  pack_bf16x2(oa[dt][b8 + 6] * inv, oa[dt][b8 + 7] * inv)};
      }
    };
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      if (st == NS - 1) {
        // every probability has been added: the row's l, 1/l and lse
        const float l = halves_sum(l0 + l1);
        inv = out_scale * __builtin_amdgcn_rcpf(l);
        lse2 = mb + __builtin_amdgcn_logf(l);
      }
      const bf16x8 pfs = as_bf16x8(u32x4{w[st & 1][0], w[st & 1][1], w[st & 1][2], w[st & 1][3]});
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int i = 4 * st + dt;
        if (i + 2 < 4 * NS) vr[(i + 2) % 3] = vread(i + 2);
        oa[dt] = mfma32x32x16(as_bf16x8(vr[i % 3]), pfs, oa[dt]);
        if (st + 1 < NS) w[(st + 1) & 1][dt] = pair(st + 1, dt);
        else if (dt > 0) out_tile(dt - 1);  // its last MFMA was the slot before
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    out_tile(3);
  };

  // ---- software pipeline over passes: at the start of pass p the entry of
  // pass p+2 is read and the Q rows of pass p+1 are gathered (a whole pass of
  // latency each), then pass p runs its softmax, P V and stores, and pass
  // p+1's scores end the step.  One Q register set and one accumulator set
  // serve every pass (an earlier two-pass-ahead form with alternating register
  // sets sat at the 256-register limit, which cost its schedule the room to
  // keep LDS reads ahead of the MFMAs and spilled the fp8 kernel).  Past the
  // end of the work the last pass stands in (its loads are valid and their
  // results unused).
  const int i1 = next_pass();
  bool have1 = i1 >= 0;
  int j_last = have1 ? i1 : i0;  // furthest pass looked up (a valid index)
  PassDesc D0 = passes[i0];
  PassDesc D1 = passes[j_last];
  RowRef rr0 = row_dec(row_ent(D0), D0.seq);
  RowRef rr1 = row_dec(row_ent(D1), D1.seq);
  QFrag<FP8> q;
  f32x16 acc[4];
  q.load(rr0.q, h);
  stage(D0);
  __syncthreads();
  scores(q, acc);

  for (;;) {
    // ---- entry of pass p+2 and the Q rows of pass p+1 (unconditionally)
    const int i2 = have1 ? next_pass() : -1;
    const bool have2 = i2 >= 0;
    if (have2) j_last = i2;
    const PassDesc D2 = passes[j_last];
    const uint32_t raw2 = row_ent(D2);
    q.load(rr1.q, h);

    // ---- pass p: causal mask, softmax and O^T = V^T P^T into the wave's
    // tile, then out
    mask_own(acc, rr0, D0.blk);
    float lse2;
    if (h == 0) orow_tile[n] = rr0.orow;
    softmax_pv(acc, lse2);
    // (both half-waves hold the same m and l; their stores coincide)
    lse_part[rr0.orow] = lse2 * 0.69314718055994531f;
    // The wave's 32 rows leave row-contiguous: instruction j stores rows
    // 4j .. 4j + 3, lane L the 16-byte chunk L % 16 of row 4j + L / 16.  LDS
    // operations of a wave complete in order, so the tile is read back after
    // it was written, and rewritten only after this readback.  The partials
    // are read once, much later, by the combine: the stores are non-temporal.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 4 * j + (lane >> 4), chunk = lane & 15;
      const u32x4 v = *reinterpret_cast<const u32x4*>(o_tile + row * kOStride + chunk * 16);
      const int64_t orow = orow_tile[row];
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(o_part + orow * kDh + chunk * 8));
    }
    if (!have1) break;

    // ---- pass p+1: stage its block when it changes, then its scores
    if (D1.seq != D0.seq || D1.blk != D0.blk) {
      __syncthreads();
      stage(D1);
      __syncthreads();
    }
    scores(q, acc);

    // ---- advance the pass descriptors and row references
    D0 = D1;
    D1 = D2;
    rr0 = rr1;
    rr1 = row_dec(raw2, D2.seq);
    have1 = have2;
  }
}

// Persistent workgroups per CU (135 KB of LDS each).
constexpr int kAttnWgPerCu = 1;

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

}  // namespace

// Round-up reciprocal of d in [2, 32] for 31-bit dividends (Granlund and
// Montgomery, "Division by invariant integers using multiplication", PLDI 1994,
// Thm. 4.2 with N = 31): with l = ceil(log2 d) and m = floor(2^(31+l) / d) + 1,
// 2^(31+l) < m d <= 2^(31+l) + 2^l, so n / d = (m n) >> (31 + l), i.e.
// umulhi(n, m) >> (l - 1), for every 0 <= n < 2^31; m < 2^32 for d >= 2.
void kdiv_params(int d, uint32_t* magic, int* shift) {
  if (d <= 1) {
    *magic = 0;
    *shift = 0;
    return;
  }
  int l = 0;
  while ((1 << l) < d) ++l;
  *magic = static_cast<uint32_t>(((uint64_t(1) << (31 + l)) / static_cast<uint64_t>(d)) + 1);
  *shift = l - 1;
}

namespace {

template <int G, int BKS>
hipError_t launch_g(const void* q, const void* k, const void* v, bool fp8, int batch, int64_t N,
                    int H_sel, int kv_shift, int kslots, float scale_log2, float out_scale,
                    const int32_t* blk_entries, const int32_t* sched, int64_t q_begin,
                    int64_t q_count, uint16_t* o_part, float* lse_part, hipStream_t stream) {
  const SchedLayout s = sched_layout(batch, H_sel, G, kslots, q_begin, q_count, 1 << BKS);
  // Never more workgroups than passes, so every workgroup has work when the
  // range is small.
  int64_t grid = static_cast<int64_t>(device_cus()) * kAttnWgPerCu;
  const int64_t min_passes = (static_cast<int64_t>(batch) * H_sel * q_count * kslots + s.EPP - 1) / s.EPP;
  if (min_passes < grid) grid = min_passes;
  if (grid < 1) grid = 1;
  uint32_t magic = 0;
  int shift = 0;
  kdiv_params(kslots, &magic, &shift);
  // fp8 runs with 128-token blocks only (the entry point rejects the rest)
  auto kern = (fp8 && BKS == 7) ? sparse_attn_kernel<G, true, 7> : sparse_attn_kernel<G, false, BKS>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream, q, k, v,
                     N, H_sel, kv_shift, kslots, magic, shift, scale_log2, out_scale, blk_entries,
                     sched + s.off_segp, reinterpret_cast<const PassDesc*>(sched + s.off_pass),
                     static_cast<int>(s.B_c), static_cast<int>(batch * H_sel),
                     static_cast<int>(q_begin), static_cast<int>(q_count), o_part, lse_part);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const void* q, const void* k, const void* v, bool fp8, int batch,
                              int64_t N, int H_sel, int G, int kv_shift, int kslots, float scale_log2,
                              float out_scale, const int32_t* /*blk_offsets: the pass list carries them*/,
                              const int32_t* blk_entries, const int32_t* sched, int64_t q_begin,
                              int64_t q_count, uint16_t* o_part, float* lse_part,
                              hipStream_t stream, int bk) {
#define MSA_ATTN_CASE(GG)                                                                           \
  case GG:                                                                                          \
    if (bk == 32)                                                                                   \
      return launch_g<GG, 5>(q, k, v, fp8, batch, N, H_sel, kv_shift, kslots, scale_log2, out_scale, \
                             blk_entries, sched, q_begin, q_count, o_part, lse_part, stream);       \
    if (bk == 64)                                                                                   \
      return launch_g<GG, 6>(q, k, v, fp8, batch, N, H_sel, kv_shift, kslots, scale_log2, out_scale, \
                             blk_entries, sched, q_begin, q_count, o_part, lse_part, stream);       \
    return launch_g<GG, 7>(q, k, v, fp8, batch, N, H_sel, kv_shift, kslots, scale_log2, out_scale,   \
                           blk_entries, sched, q_begin, q_count, o_part, lse_part, stream);
  switch (G) {
    MSA_ATTN_CASE(1)
    MSA_ATTN_CASE(2)
    MSA_ATTN_CASE(4)
    MSA_ATTN_CASE(8)
    MSA_ATTN_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef MSA_ATTN_CASE
}

}  // namespace msa
