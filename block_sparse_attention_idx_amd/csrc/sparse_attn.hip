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
//    The (query, slot) entries are taken in segment order -- (sequence, query
//    window, block), see invert.hip -- and that sequence is cut into one equal
//    contiguous share per workgroup: every workgroup gets the same number of
//    entries whatever the block popularity, and stages a K/V block only when
//    its share moves to the next segment.
//  * A pass is 256 (query, head) rows: 256 / G entries x G heads (a query's G
//    heads are contiguous in Q, 256 B each); each wave owns one 32-row MFMA
//    column tile.  K (row-major) and V (transposed) live in padded LDS
//    (67 KB), shared by the 8 waves.
//  * S^T = K_b * Q^T with v_mfma_f32_32x32x16_bf16 (keys on the row
//    dimension): every lane holds 64 of the 128 keys of one (query, head) row,
//    so the row max and row sum need one half-wave exchange, and the
//    probabilities feed O^T = V^T * P^T directly as the MFMA B operand with no
//    shuffle (the reduction slots of each P^T step are exactly the keys that
//    lane already holds).  The V^T operand rows are permuted so that every
//    lane ends up with 64 contiguous output dimensions of its row.
//  * The partial outputs go through an 8.5 KB LDS tile per wave: written in
//    the MFMA layout (lane = row), read back row-contiguous, and stored 1 KB
//    contiguous per instruction, so L2 receives whole 128-byte lines rather
//    than 16-byte pieces of 64 different rows.
//  * Software pipeline over passes: the Q rows of the next pass are gathered
//    into registers and the entries of the pass after it are read while the
//    current pass computes.  Every memory operation of the loop is issued
//    unconditionally, so the compiler's in-order vmcnt waits never have to
//    cover the stores or the loads just issued.
//  * Softmax in base 2 (v_exp_f32) with the scale folded into one FMA; fp8
//    (OCP e4m3) inputs are widened exactly to bf16 when used and the
//    per-tensor scales are folded into the softmax scale and the output scale.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kPassRows = 32 * kWaves;  // (query, head) rows per pass

// LDS layouts.  Rows are padded rather than swizzled so that every fragment
// read of a lane is one base address plus a compile-time offset (no per-read
// address registers):
//  * K row-major, 272 B per key row: a 16-lane phase of 16-byte reads of rows
//    n .. n + 15 starts at banks 4n + const, all distinct.
//  * V^T, 264 B per output-dimension row, row d stored at position
//    2 (d mod 64) + d / 64: the 32 rows one 8-byte read touches
//    (d in 0..15 and 64..79, plus 16 dt) land on 32 distinct even banks.
//  * Output tile, 272 B per row: 16-byte writes of rows n .. n + 15 and
//    16-byte reads of the 16 chunks of one row are both conflict free.
constexpr int kKStride = 272;
constexpr int kVStride = 264;
constexpr int kOStride = 272;

__device__ __forceinline__ int k_lds_off(int key, int c) {  // 16-byte chunk c of key row
  return key * kKStride + c * 16;
}

__device__ __forceinline__ int vt_row(int d) { return ((d & 63) << 1) | (d >> 6); }

__device__ __forceinline__ int vt_lds_off(int d, int kc) {  // 8-byte chunk kc (4 keys) of row d
  return vt_row(d) * kVStride + kc * 8;
}

__device__ __forceinline__ uint32_t half_of(const u32x4& w, int dd) {
  const uint32_t x = w[dd >> 1];
  return (dd & 1) ? (x >> 16) : (x & 0xFFFFu);
}

// Stage K (row-major) and V (transposed) of one block of one head into LDS.
template <bool FP8>
__device__ __forceinline__ void stage_kv(const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb,
                                         int64_t rstride, int nvalid, uint8_t* k_lds,
                                         uint8_t* vt_lds) {
  // Staging is rare (once per segment); an opaque copy of the thread id keeps
  // the compiler from hoisting its per-lane addresses out of the caller's
  // loop, where they would stay live across every pass.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  // Rows past the end of the sequence (a partial last block) are read from the
  // last valid row and replaced by zeros, so every load is issued at once.
  if constexpr (!FP8) {
    u32x4 w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int key = (tid >> 4) + 32 * p, c = tid & 15;
      w[p] = *reinterpret_cast<const u32x4*>(kb + min(key, nvalid - 1) * rstride + c * 16);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int key = (tid >> 4) + 32 * p, c = tid & 15;
      if (key >= nvalid) w[p] = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(k_lds + k_lds_off(key, c)) = w[p];
    }
  } else {
    u32x4 wk[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int key = (tid >> 3) + 64 * p, cc = tid & 7;
      wk[p] = *reinterpret_cast<const u32x4*>(kb + min(key, nvalid - 1) * rstride + cc * 16);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int key = (tid >> 3) + 64 * p, cc = tid & 7;
      const u32x4 w = key < nvalid ? wk[p] : u32x4{0u, 0u, 0u, 0u};
      const u32x2 a = e4m3x4_to_bf16x4(w[0]), b = e4m3x4_to_bf16x4(w[1]);
      const u32x2 c2 = e4m3x4_to_bf16x4(w[2]), d2 = e4m3x4_to_bf16x4(w[3]);
      *reinterpret_cast<u32x4*>(k_lds + k_lds_off(key, 2 * cc)) = u32x4{a[0], a[1], b[0], b[1]};
      *reinterpret_cast<u32x4*>(k_lds + k_lds_off(key, 2 * cc + 1)) = u32x4{c2[0], c2[1], d2[0], d2[1]};
    }
  }
  // V: thread (dg, kc) transposes the 8 dims 8 dg .. 8 dg + 7 of keys
  // 4 kc .. 4 kc + 3 into four-key chunks of V^T rows.
  const int kc = tid & 31, dg = tid >> 5;
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
      const u32x2 a = e4m3x4_to_bf16x4(rows[j][0]), b = e4m3x4_to_bf16x4(rows[j][1]);
      row[j] = u32x4{a[0], a[1], b[0], b[1]};
    }
  }
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    const int d = 8 * dg + dd;
    const u32x2 v = {half_of(row[0], dd) | (half_of(row[1], dd) << 16),
                     half_of(row[2], dd) | (half_of(row[3], dd) << 16)};
    *reinterpret_cast<u32x2*>(vt_lds + vt_lds_off(d, kc)) = v;
  }
}

// Q fragments (B operand of S^T) of one row, dims 16 ks + 8 h .. + 8, kept as
// loaded (bf16: 8 x 16 B; fp8: 8 x 8 B of codes) and widened when used, so a
// prefetch is never waited on before its pass.
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
template <>
struct QFrag<true> {
  u32x2 w[8];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ qr, int h) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) w[ks] = *reinterpret_cast<const u32x2*>(qr + 16 * ks + 8 * h);
  }
  __device__ __forceinline__ bf16x8 get(int ks) const {
    const u32x2 a = e4m3x4_to_bf16x4(w[ks][0]), b = e4m3x4_to_bf16x4(w[ks][1]);
    return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
  }
};

struct AttnSched {
  int64_t B_c, T64, TW, nW;
  int64_t off_ckey, off_cpre, off_cnt;
};

template <int G, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void sparse_attn_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    int64_t N, int H_kv, int kslots, uint32_t kdiv_magic, int kdiv_shift, float scale_log2,
    float out_scale, const int32_t* __restrict__ blk_offsets, const int32_t* __restrict__ entries,
    const int32_t* __restrict__ sched, AttnSched sv, int64_t q_begin, int64_t q_count,
    uint16_t* __restrict__ o_part, float* __restrict__ lse_part) {
  constexpr int EPP = kPassRows / G;  // entries per pass
  constexpr int EB = FP8 ? 1 : 2;     // bytes per Q/K/V element
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kBk * kKStride];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[kDh * kVStride];
  __shared__ __attribute__((aligned(16))) uint8_t o_lds[kWaves * 32 * kOStride];
  __shared__ __attribute__((aligned(8))) int64_t orow_lds[kWaves * 32];
  __shared__ int s_seg;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int H_q = H_kv * G;
  const int32_t* ckey = sched + sv.off_ckey;
  const int32_t* cpre = sched + sv.off_cpre;
  const int32_t* ccnt = sched + sv.off_cnt;

  // This workgroup's share [p0, p1) of the entries in segment order.
  const int64_t T = sched[kHdrEntries];
  const int64_t nsegc = sched[kHdrSegs];
  const int64_t p0 = T * blockIdx.x / gridDim.x;
  const int64_t p1 = T * (blockIdx.x + 1) / gridDim.x;
  if (p0 >= p1) return;
  if (tid == 0) {  // last non-empty segment starting at or before p0
    int64_t lo = 0, hi = nsegc - 1;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) >> 1;
      if (cpre[mid] <= p0) lo = mid; else hi = mid - 1;
    }
    s_seg = static_cast<int>(lo);
  }
  __syncthreads();

  // Segment cursor (uniform across the workgroup).
  int64_t c = s_seg;
  int64_t seg_end = 0, eoff = 0, seq_q = 0;
  int seq = 0, blk = 0;
  const uint8_t* seg_q = nullptr;  // Q rows of this segment's (batch, group)
  auto open_segment = [&](int64_t cc) {
    const int key = ckey[cc];
    const int B_c = static_cast<int>(sv.B_c), nW = static_cast<int>(sv.nW);
    blk = key % B_c;
    const int sw = key / B_c;
    seq = sw / nW;
    const int64_t t0 = static_cast<int64_t>(sw % nW) * sv.TW;
    // entry index = position + eoff
    eoff = static_cast<int64_t>(blk_offsets[static_cast<int64_t>(seq) * (B_c + 1) + blk]) +
           ccnt[(seq * sv.T64 + t0) * sv.B_c + blk] - cpre[cc];
    seg_end = cpre[cc + 1];
    seq_q = static_cast<int64_t>(seq) * q_count;
    const int bat = seq / H_kv, r = seq % H_kv;
    seg_q = static_cast<const uint8_t*>(qp) +
            (static_cast<int64_t>(bat) * N * H_q + r * G) * static_cast<int64_t>(kDh) * EB;
  };
  open_segment(c);

  // Output dimension of V^T operand row n in d-tile 0 (d-tile dt adds 16 dt;
  // see the output step below), and the lane's fragment base addresses.
  const int dsel = 64 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  const uint8_t* k_base = k_lds + n * kKStride + h * 16;
  const uint8_t* v_base = vt_lds + vt_row(dsel) * kVStride + h * 8;
  uint8_t* o_tile = o_lds + wave * 32 * kOStride;
  int64_t* orow_tile = orow_lds + wave * 32;
  const int rho = 32 * wave + n;     // this lane's row of the pass
  const int e_row = rho / G, g_row = rho % G;

  // Per-lane row descriptor of a pass.  An entry holds qrow * k + slot; the
  // division by k is a multiply-high by the host's round-up reciprocal.  A row
  // past the pass's entries takes the pass's first entry (same head): it
  // recomputes that row bit for bit, so its stores repeat that row's stores.
  struct RowRef {
    const uint8_t* q;  // the row's Q vector
    int64_t orow;      // partial-output row (seq, qrow, slot, g)
    int64_t i;         // query position
  };
  auto row_ent = [&](int64_t pos, int cnt) {  // raw entry word
    return static_cast<uint32_t>(entries[pos + eoff + (e_row < cnt ? e_row : 0)]);
  };
  auto row_dec = [&](uint32_t ent) {  // with the cursor at the pass's segment
    RowRef rr;
    const uint32_t qrow = kslots == 1 ? ent : (__umulhi(ent, kdiv_magic) >> kdiv_shift);
    const uint32_t slot = ent - qrow * static_cast<uint32_t>(kslots);
    rr.i = q_begin + qrow;
    rr.orow = ((seq_q + qrow) * kslots + slot) * G + g_row;
    rr.q = seg_q + (rr.i * H_q + g_row) * static_cast<int64_t>(kDh) * EB;
    return rr;
  };

  // ---- software pipeline over passes: while pass p computes, the Q rows of
  // pass p+1 are in flight and the entries of pass p+2 are being read.  A pass
  // never spans two segments; the segment cursor always sits at the furthest
  // pass looked up.
  struct Pass {
    int64_t pos;  // first position (segment order)
    int cnt;      // entries
    int seq, blk;
  };
  auto next_pass = [&](int64_t at, Pass& P) -> bool {
    if (at >= p1) return false;
    if (at >= seg_end) {
      // (with a consistent work list the next segment starts exactly here)
      if (c + 1 >= nsegc) return false;
      open_segment(++c);
    }
    P.pos = at;
    P.cnt = static_cast<int>(min<int64_t>(EPP, min(seg_end, p1) - at));
    P.seq = seq;
    P.blk = blk;
    return P.cnt > 0;
  };

  Pass P0, P1{}, P2{};
  RowRef rr0, rr1;
  uint32_t raw2 = 0;  // pass p+2's entry word, decoded one iteration later
  QFrag<FP8> qf, qn;
  if (!next_pass(p0, P0)) return;  // uniform
  rr0 = row_dec(row_ent(P0.pos, P0.cnt));
  bool have1 = next_pass(P0.pos + P0.cnt, P1);
  if (have1) rr1 = row_dec(row_ent(P1.pos, P1.cnt));
  qf.load(rr0.q, h);
  // Settle the first pass's gather here, once: inside the loop qf is always a
  // copy of an already-waited prefetch.
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) asm volatile("" ::"v"(qf.w[ks]));
  int64_t staged = -1;

  while (true) {
    // ---- stage K and V of this pass's block if not resident
    const int64_t bin = static_cast<int64_t>(P0.seq) * sv.B_c + P0.blk;
    const int64_t key0 = static_cast<int64_t>(P0.blk) * kBk;
    if (bin != staged) {
      __syncthreads();
      const int64_t bat = P0.seq / H_kv;
      const int r = P0.seq % H_kv;
      const int64_t rstride = static_cast<int64_t>(H_kv) * kDh * EB;
      const uint8_t* kb = static_cast<const uint8_t*>(kp) + ((bat * N + key0) * H_kv + r) * kDh * EB;
      const uint8_t* vb = static_cast<const uint8_t*>(vp) + ((bat * N + key0) * H_kv + r) * kDh * EB;
      stage_kv<FP8>(kb, vb, rstride, static_cast<int>(min<int64_t>(kBk, N - key0)), k_lds, vt_lds);
      __syncthreads();
      staged = bin;
    }

    // ---- read pass p+2's entry and gather pass p+1's Q row (unconditionally:
    // a missing pass reads entry 0 / this pass's row and ignores it)
    const bool have2 = have1 && next_pass(P1.pos + P1.cnt, P2);
    raw2 = static_cast<uint32_t>(entries[have2 ? P2.pos + eoff + (e_row < P2.cnt ? e_row : 0) : 0]);
    qn.load(have1 ? rr1.q : rr0.q, h);

    // ---- S^T = K_b Q^T: acc[mt] holds keys 32mt + 8(e/4) + 4h + (e%4) of this row
    f32x16 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      acc[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        // row 32 mt + n, 16-byte chunk 2 ks + h
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(k_base + 32 * mt * kKStride + 32 * ks));
        acc[mt] = mfma32x32x16(kf, qf.get(ks), acc[mt]);
      }
    }

    // ---- softmax.  The causal mask only bites in a query's own block, so it
    // runs on a wave-uniform branch taken by the few passes that hold such a
    // row.  The maximum is taken on the raw scores and the scale is folded
    // into one FMA before exp2; the row sum adds the fp32 probabilities, so
    // lse is the exact log-sum-exp up to fp32 rounding.
    const bool own = P0.blk == (rr0.i >> 7);
    if (__any(own)) {
      const int limit = own ? static_cast<int>(rr0.i - key0) : kBk - 1;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int el = 0; el < 16; ++el) {
          const int key = 32 * mt + 8 * (el >> 2) + 4 * h + (el & 3);
          if (key > limit) acc[mt][el] = -__builtin_huge_valf();
        }
      }
    }
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int el = 0; el < 16; el += 2) m = fmaxf(m, fmaxf(acc[mt][el], acc[mt][el + 1]));
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    const float mb = m * scale_log2;  // scale_log2 > 0: the max commutes with it
    float l = 0.f;
    // P^T fragments (B operand of O^T = V^T P^T): step st = 2 mt + e2 covers
    // keys 32mt + 16e2 + 8(j/4) + 4h + (j%4), accumulator elements 8e2 .. +7.
    bf16x8 pf[8];
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
    l += __shfl_xor(l, 32);
    const float inv = out_scale / l;
    const float lse2 = mb + __builtin_amdgcn_logf(l);

    // ---- O^T = V^T P^T, one 32-dim tile at a time; lane (n, h) receives dims
    // 64h + 16dt + el of its row and writes them to the wave's output tile.
    if (h == 0) orow_tile[n] = rr0.orow;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x16 oa = {};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        // row dsel + 16 dt (stored at vt_row(dsel) + 32 dt), 8-byte chunks
        // c1 = 4 st + h = 8 mt + 4 e2 + h and c1 + 2
        const uint8_t* vp8 = v_base + 32 * dt * kVStride + 32 * st;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vp8);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vp8 + 16);
        oa = mfma32x32x16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pf[st], oa);
      }
      uint8_t* dst = o_tile + n * kOStride + 128 * h + 32 * dt;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int b8 = 8 * hf;
        *reinterpret_cast<u32x4*>(dst + 16 * hf) =
            u32x4{pack_bf16x2(oa[b8 + 0] * inv, oa[b8 + 1] * inv),
                  pack_bf16x2(oa[b8 + 2] * inv, oa[b8 + 3] * inv),
                  pack_bf16x2(oa[b8 + 4] * inv, oa[b8 + 5] * inv),
                  pack_bf16x2(oa[b8 + 6] * inv, oa[b8 + 7] * inv)};
      }
    }
    // (both half-waves hold the same m and l; their stores coincide)
    lse_part[rr0.orow] = lse2 * 0.69314718055994531f;
    // ---- the wave's 32 rows leave row-contiguous: instruction j stores rows
    // 4j .. 4j + 3, lane L the 16-byte chunk L % 16 of row 4j + L / 16.  LDS
    // operations of a wave complete in order, so the tile is read back after
    // it was written, and rewritten only after this readback.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 4 * j + (lane >> 4), chunk = lane & 15;
      const u32x4 v = *reinterpret_cast<const u32x4*>(o_tile + row * kOStride + chunk * 16);
      const int64_t orow = orow_tile[row];
      *reinterpret_cast<u32x4*>(o_part + orow * kDh + chunk * 8) = v;
    }
    if (!have1) break;

    // ---- rotate the pipeline (the cursor still sits at pass p+2's segment)
    P0 = P1;
    P1 = P2;
    rr0 = rr1;
    if (have2) rr1 = row_dec(raw2);
    qf = qn;
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

template <int G>
hipError_t launch_g(const void* q, const void* k, const void* v, bool fp8, int batch, int64_t N,
                    int H_kv, int kslots, float scale_log2, float out_scale,
                    const int32_t* blk_offsets, const int32_t* blk_entries, const int32_t* sched,
                    int64_t q_begin, int64_t q_count, uint16_t* o_part, float* lse_part,
                    hipStream_t stream) {
  const SchedLayout s = sched_layout(batch, H_kv, q_begin, q_count);
  const AttnSched sv{s.B_c, s.T64, s.TW, s.nW, s.off_ckey, s.off_cpre, s.off_cnt};
  // Never more workgroups than passes, so every workgroup has work when the
  // range is small.
  const int64_t entries_max = static_cast<int64_t>(batch) * H_kv * q_count * kslots;
  const int64_t passes = (entries_max + (kPassRows / G) - 1) / (kPassRows / G);
  int64_t grid = static_cast<int64_t>(device_cus()) * kAttnWgPerCu;
  if (passes < grid) grid = passes;
  if (grid < 1) grid = 1;
  uint32_t magic = 0;
  int shift = 0;
  kdiv_params(kslots, &magic, &shift);
  auto kern = fp8 ? sparse_attn_kernel<G, true> : sparse_attn_kernel<G, false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream, q, k, v,
                     N, H_kv, kslots, magic, shift, scale_log2, out_scale, blk_offsets,
                     blk_entries, sched, sv, q_begin, q_count, o_part, lse_part);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const void* q, const void* k, const void* v, bool fp8, int batch,
                              int64_t N, int H_kv, int G, int kslots, float scale_log2,
                              float out_scale, const int32_t* blk_offsets,
                              const int32_t* blk_entries, const int32_t* sched, int64_t q_begin,
                              int64_t q_count, uint16_t* o_part, float* lse_part,
                              hipStream_t stream) {
#define MSA_ATTN_CASE(GG)                                                                      \
  case GG:                                                                                     \
    return launch_g<GG>(q, k, v, fp8, batch, N, H_kv, kslots, scale_log2, out_scale,           \
                        blk_offsets, blk_entries, sched, q_begin, q_count, o_part, lse_part,   \
                        stream);
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
