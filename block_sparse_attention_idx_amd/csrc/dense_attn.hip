// Dense causal GQA attention forward: the baseline that the sparse path is
// measured against.
//
// What is computed ("MiniMax Sparse Attention", sec. 2.1: causal scaled
// dot-product attention in which G adjacent query heads share one K/V head;
// the pages quote MSA's prefill speed against this dense form):
//     O[i, h]   = sum_{j <= i} softmax_j(s_j) V[j, r],
//     lse[i, h] = ln sum_{j <= i} exp(s_j),
//     s_j = scale * Q[i, h] . K[j, r],   r = h / G.
//
// gfx950 design (query-outer, online softmax):
//  * One workgroup = 8 waves = 256 (token, head) rows: 256 / G consecutive
//    tokens times the G heads of one group (a token's G heads are contiguous
//    in Q and O), one 32-row MFMA column tile per wave.  Q stays in VGPRs.
//  * The group's key blocks 0 .. (last token) / 128 stream through two LDS
//    buffers (the shared tile layout: K row-major, V transposed, rows padded
//    to 272 B), loaded into registers one step ahead.
//  * Per block and wave: S^T = K_b Q^T (32 v_mfma_f32_32x32x16_bf16, keys on
//    the row dimension, so each lane holds 64 keys of its own row), the
//    running max and sum update in base 2, and O^T += V^T P^T (32 MFMAs) with
//    P^T straight from the score registers.  Every output element a lane
//    accumulates belongs to the lane's own row, so the rescale by
//    exp2(m_old - m_new) is a per-lane multiply, and the reference max only
//    moves when a block exceeds it by more than 2^8 (probabilities stay
//    below 256), so almost every block skips the rescale.  The lanes keep
//    their partial row sums; the two half-waves add them once, at the end.
//  * A wave skips the blocks that lie wholly after its last token, and masks
//    only the blocks that reach past its first token.
//  * Workgroups are issued heaviest (latest tokens) first; consecutive
//    workgroups take the same token tile of consecutive groups, so the
//    workgroups of one XCD (dealt round-robin) share a K/V head in its L2.
//  * The output leaves through an LDS tile, row-contiguous, 1 KB per store
//    instruction.
#include "attn_tile.h"
#include "msa_internal.h"

namespace msa {
namespace {

using namespace tile;

constexpr int kDWaves = 8;
constexpr int kDThreads = 64 * kDWaves;
constexpr int kDRows = 32 * kDWaves;             // (token, head) rows per workgroup
constexpr float kLazy = 8.f;                     // log2 of the largest unnormalised probability
template <int G>
__global__ __launch_bounds__(kDThreads, 1) void dense_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t N, int H_kv, int nseq, int64_t q_begin, int64_t q_count, int64_t ntile,
    float scale_log2, uint16_t* __restrict__ o, float* __restrict__ lse) {
  constexpr int T = kDRows / G;  // tokens per workgroup
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBufBytes];

  const int64_t wg = blockIdx.x;
  const int seq = static_cast<int>(wg % nseq);
  const int64_t tile = ntile - 1 - wg / nseq;
  const int bat = seq / H_kv, r = seq - bat * H_kv;
  const int H_q = H_kv * G;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;

  const int64_t q_end = q_begin + q_count;
  const int64_t t0 = q_begin + tile * T;
  const int64_t t_last = min(t0 + T, q_end) - 1;
  const int nb = static_cast<int>(t_last / kBk) + 1;

  // This lane's row (rows past the range repeat the last token; not stored).
  const int rho = 32 * wave + n;
  const int64_t t_raw = t0 + rho / G;
  const int64_t t_row = min(t_raw, t_last);
  const int g = rho % G;
  const int64_t orow = (static_cast<int64_t>(bat) * N + t_row) * H_q + r * G + g;
  // The wave's first token.
  const int64_t tw_lo = min(t0 + (32 * wave) / G, t_last);

  u32x4 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qf[ks] = *reinterpret_cast<const u32x4*>(q + orow * kDh + 16 * ks + 8 * h);

  const int64_t rstride = static_cast<int64_t>(H_kv) * kDh * 2;
  const uint8_t* kseq = reinterpret_cast<const uint8_t*>(k) + (static_cast<int64_t>(bat) * N * H_kv + r) * kDh * 2;
  const uint8_t* vseq = reinterpret_cast<const uint8_t*>(v) + (static_cast<int64_t>(bat) * N * H_kv + r) * kDh * 2;
  auto nvalid_of = [&](int b) { return static_cast<int>(min<int64_t>(kBk, N - static_cast<int64_t>(b) * kBk)); };

  const int dsel = 64 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
  float m_run = -__builtin_huge_valf(), l_run = 0.f;

  // ---- software pipeline over half blocks (64 keys).  Step (b, hb) runs the
  // scores of the next half on the matrix cores while the VALU turns the
  // scores of half (b, hb) into probabilities, then that half's P V.  The loop
  // body holds the two steps of block b, so the score registers alternate by
  // name.  LDS: block b in slot b & 1; block b + 1 is written into the other
  // slot at the top of iteration b (its previous block was last read before
  // the barrier that ended iteration b - 1) and published by the barrier
  // between the two steps, in time for the second step's look-ahead scores.
  //
  // Scores of one half: s[mt2] holds keys 64 hb + 32 mt2 + 8 (e / 4) + 4 h +
  // (e % 4) of this lane's row.
  auto scores_half = [&](const uint8_t* kbuf, int hb, f32x16(&s)[2]) {
    const uint8_t* kfr = kbuf + (64 * hb + n) * kStr + h * 16;
#pragma unroll
    for (int mt2 = 0; mt2 < 2; ++mt2) {
      s[mt2] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s[mt2] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(kfr + 32 * mt2 * kStr + 32 * ks)),
                              as_bf16x8(qf[ks]), s[mt2]);
    }
  };

  const uint8_t* vlane = lds + kVtOff + dvt_row(dsel) * kStr + h * 16;  // slot 0
  auto step = [&](f32x16(&s)[2], f32x16(&sn)[2], int slot, int b, int hb, const uint8_t* kbuf_next,
                  int hb_next) {
    const int64_t key0 = static_cast<int64_t>(b) * kBk + 64 * hb;
    if (key0 + 63 > tw_lo) {  // wave-uniform: some key of the half lies past some row's token
      asm volatile("" ::: "memory");
      const int lim = static_cast<int>(t_row - key0) - 4 * h;
#pragma unroll
      for (int mt2 = 0; mt2 < 2; ++mt2) {
#pragma unroll
        for (int el = 0; el < 16; ++el) {
          const uint32_t hide = static_cast<uint32_t>((lim - (32 * mt2 + 8 * (el >> 2) + (el & 3))) >> 31);
          s[mt2][el] = __uint_as_float((__float_as_uint(s[mt2][el]) & ~hide) | (0xFF800000u & hide));
        }
      }
    }
    // Reference max in base-2 units (scale_log2 > 0).  It moves only when
    // the half's max exceeds it by more than kLazy, so every probability
    // stays below 2^kLazy and almost no step rescales O; the final O / l and
    // m + log2 l are exact for any reference.  Every row sees key 0, so m_run
    // is finite from the first half on, and a fully hidden row of a later
    // half keeps alpha = 1 and gets p = 0.
    float m0 = -__builtin_huge_valf(), m1 = -__builtin_huge_valf();
#pragma unroll
    for (int mt2 = 0; mt2 < 2; ++mt2) {
#pragma unroll
      for (int el = 0; el < 16; el += 4) {
        m0 = max3f(m0, s[mt2][el], s[mt2][el + 1]);
        m1 = max3f(m1, s[mt2][el + 2], s[mt2][el + 3]);
      }
    }
    const float m_blk = halves_max(fmaxf(m0, m1)) * scale_log2;
    const bool raise = m_blk > m_run + kLazy;
    const float m_new = raise ? m_blk : m_run;
    if (__any(raise)) {  // wave-uniform, rare
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
      l_run *= alpha;
    }
    m_run = m_new;

    // ---- the next half's scores || this half's probabilities, interleaved by
    // hand (fenced slots): slot i issues look-ahead MFMA i (key tile i / 8,
    // reduction step i % 8), reads the K fragment of MFMA i + 2, and turns
    // score pair i (tile i / 8, elements 2 (i % 8), + 1) into probabilities.
    const uint8_t* kfr = kbuf_next + (64 * hb_next + n) * kStr + h * 16;
    auto kread = [&](int i) {
      return *reinterpret_cast<const u32x4*>(kfr + 32 * (i >> 3) * kStr + 32 * (i & 7));
    };
    u32x4 kq[3];
    kq[0] = kread(0);
    kq[1] = kread(1);
    uint32_t w[16];
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) kq[(i + 2) % 3] = kread(i + 2);
      const int mt2 = i >> 3, ks = i & 7;
      sn[mt2] = mfma32x32x16(as_bf16x8(kq[i % 3]), as_bf16x8(qf[ks]), ks == 0 ? f32x16{} : sn[mt2]);
      const float pa = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt2][2 * ks], scale_log2, -m_new));
      const float pb = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt2][2 * ks + 1], scale_log2, -m_new));
      w[i] = pack_bf16x2(pa, pb);
      s0 += pa;
      s1 += pb;
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += s0 + s1;
    // P^T fragment f = 2 mt2 + e2 holds elements 8 e2 .. 8 e2 + 7 of tile
    // mt2, i.e. pairs 8 mt2 + 4 e2 .. + 3.
    bf16x8 pf[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
      pf[f] = as_bf16x8(u32x4{w[4 * f + 0], w[4 * f + 1], w[4 * f + 2], w[4 * f + 3]});

    // ---- O^T += V^T P^T over this half: P^T steps 4 hb .. 4 hb + 3 of the
    // block; lane (n, h) holds dims 64 h + 16 dt + e of its row (V^T operand
    // row dsel + 16 dt, stored at dvt_row(dsel) + 32 dt).  Fragment reads run
    // two MFMAs ahead.
    const uint8_t* vfr = vlane + slot * kBufBytes + 32 * 4 * hb;
    auto vread = [&](int i) {
      return *reinterpret_cast<const u32x4*>(vfr + 32 * (i >> 2) * kStr + 32 * (i & 3));
    };
    u32x4 vq[3];
    vq[0] = vread(0);
    vq[1] = vread(1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) vq[(i + 2) % 3] = vread(i + 2);
      const int dt = i >> 2, st = i & 3;
      oacc[dt] = mfma32x32x16(as_bf16x8(vq[i % 3]), pf[st], oacc[dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16 sA[2], sB[2];
  KVRegs R;
  kv_load(R, kseq, vseq, rstride, nvalid_of(0), tid);
  kv_store(R, lds, nvalid_of(0), tid);
  {
    const int b1 = min(1, nb - 1);
    kv_load(R, kseq + static_cast<int64_t>(b1) * kBk * rstride, vseq + static_cast<int64_t>(b1) * kBk * rstride,
            rstride, nvalid_of(b1), tid);
  }
  __syncthreads();
  scores_half(lds, 0, sA);

  for (int b = 0; b < nb; ++b) {
    // Past the last block the copies repeat block nb - 1: the loads stay in
    // bounds and the look-ahead scores from it are never used.
    const int slot = b & 1;
    uint8_t* cur = lds + slot * kBufBytes;
    uint8_t* nxt = lds + (slot ^ 1) * kBufBytes;
    const int b1 = min(b + 1, nb - 1), b2 = min(b + 2, nb - 1);
    kv_store(R, nxt, nvalid_of(b1), tid);
    step(sA, sB, slot, b, 0, cur, 1);
    kv_load(R, kseq + static_cast<int64_t>(b2) * kBk * rstride, vseq + static_cast<int64_t>(b2) * kBk * rstride,
            rstride, nvalid_of(b2), tid);
    __syncthreads();
    step(sB, sA, slot, b, 1, nxt, 0);
    __syncthreads();
  }

  // ---- normalise and write out (the buffers are free after the last barrier)
  const float l = halves_sum(l_run);
  const float inv = __builtin_amdgcn_rcpf(l);
  if (h == 0 && t_raw < q_end && lse != nullptr)
    lse[orow] = (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
  uint8_t* o_tile = lds + wave * 32 * kStr;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    uint8_t* dst = o_tile + n * kStr + 128 * h + 32 * dt;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int b8 = 8 * hf;
      *reinterpret_cast<u32x4*>(dst + 16 * hf) =
          u32x4{pack_bf16x2(oacc[dt][b8 + 0] * inv, oacc[dt][b8 + 1] * inv),
                pack_bf16x2(oacc[dt][b8 + 2] * inv, oacc[dt][b8 + 3] * inv),
                pack_bf16x2(oacc[dt][b8 + 4] * inv, oacc[dt][b8 + 5] * inv),
                pack_bf16x2(oacc[dt][b8 + 6] * inv, oacc[dt][b8 + 7] * inv)};
    }
  }
  // LDS operations of a wave complete in order: the tile is read back after it
  // was written.  Instruction j stores rows 4 j .. 4 j + 3, lane L the 16-byte
  // chunk L % 16 of row 4 j + L / 16.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 4 * j + (lane >> 4), chunk = lane & 15;
    const int rr = 32 * wave + row;
    const int64_t t = t0 + rr / G;
    const u32x4 val = *reinterpret_cast<const u32x4*>(o_tile + row * kStr + chunk * 16);
    if (t < q_end) {
      const int64_t orr = (static_cast<int64_t>(bat) * N + t) * H_q + r * G + rr % G;
      *reinterpret_cast<u32x4*>(o + orr * kDh + chunk * 8) = val;
    }
  }
}

template <int G>
hipError_t launch_dense_g(const uint16_t* q, const uint16_t* k, const uint16_t* v, int batch, int64_t N,
                          int H_kv, int64_t q_begin, int64_t q_count, float scale_log2, uint16_t* o,
                          float* lse, hipStream_t stream) {
  constexpr int T = kDRows / G;
  const int nseq = batch * H_kv;
  const int64_t ntile = (q_count + T - 1) / T;
  const int64_t grid = ntile * nseq;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dense_attn_kernel<G>, dim3(static_cast<unsigned>(grid)), dim3(kDThreads), 0,
                     stream, q, k, v, N, H_kv, nseq, q_begin, q_count, ntile, scale_log2, o, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int batch,
                             int64_t N, int H_kv, int G, int64_t q_begin, int64_t q_count,
                             float scale_log2, uint16_t* o, float* lse, hipStream_t stream) {
  switch (G) {
    case 1: return launch_dense_g<1>(q, k, v, batch, N, H_kv, q_begin, q_count, scale_log2, o, lse, stream);
    case 2: return launch_dense_g<2>(q, k, v, batch, N, H_kv, q_begin, q_count, scale_log2, o, lse, stream);
    case 4: return launch_dense_g<4>(q, k, v, batch, N, H_kv, q_begin, q_count, scale_log2, o, lse, stream);
    case 8: return launch_dense_g<8>(q, k, v, batch, N, H_kv, q_begin, q_count, scale_log2, o, lse, stream);
    case 16: return launch_dense_g<16>(q, k, v, batch, N, H_kv, q_begin, q_count, scale_log2, o, lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace msa
