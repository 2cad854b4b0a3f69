// Index branch of MSA: block scores, causal block max-pool and a streaming
// top-k with the forced local block, fused in one kernel.
//
// What is computed ("MiniMax Sparse Attention (MSA)", Deep Dive > Index Branch
// Architecture; "Flash-MSA", Forward > Proxy attention): for query i and group
// r, every earlier key block b < L = floor(i / B_k) scores
//     M[i, r, b] = max_{j in block b} Q^idx[i, r] . K^idx[j]
// and the k - 1 best blocks are kept next to the local block L.  Softmax is
// order preserving, so selection works on raw scores with no exponentials
// ("MiniMax Sparse Attention (MSA)", Exp-Free TopK Kernel); the 1/sqrt(d_idx)
// factor is a positive constant and is left out.  Every token of an earlier
// block is visible to the query, so the causal mask never has to be applied:
// the only partially visible block is the local one, which is forced.
//
// gfx950 design:
//  * One workgroup = 8 waves = 512 (query, group) rows; rows are consecutive
//    in Q^idx memory ([N][H_kv][d_idx]), so all groups of a query tile share
//    each staged K^idx block (there is a single index key head).
//  * Scores are computed transposed, S^T = K^idx_b * Q^idx^T, with
//    v_mfma_f32_32x32x16_bf16: keys on the MFMA row dimension, queries on the
//    column dimension.  Each lane then holds 16 keys of one query column per
//    32-key tile, so the block max-pool is an in-lane max plus one exchange
//    between the two half-waves.  No score ever leaves the VGPRs.
//  * Q^idx fragments stay in VGPRs for the whole scan; K^idx blocks stream
//    through a 4-buffer, row-padded LDS ring filled by direct global->LDS
//    loads, with one barrier per two blocks.  K^idx fragments roll: the
//    register that fed a step is refilled with the next tile's fragment.
//  * After the exchange, each lane owns exactly one row and keeps that row's
//    top-(k-1) (score, block) list sorted in VGPRs; blocks arrive in
//    ascending id order, so "ties keep the earlier block" is a strict
//    compare.
//  * A tile's MFMAs are interleaved with VALU work that does not depend on
//    them, so the vector ALU runs beside the matrix cores within each wave:
//    the previous tile's max-pool, and a block's whole epilogue (its last
//    tile's max-pool, the exchange, the threshold test and the branch-free
//    insertion) under the next block's first two key tiles.
//  * Workgroups are issued heaviest (latest queries, most blocks) first.
#include <limits.h>

#include <type_traits>

#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kIdxThreads = 512;
constexpr int kIdxWaves = kIdxThreads / 64;
constexpr int kIdxRows = 512;  // rows per workgroup, 64 per wave

// K^idx rows in LDS are padded by 16 bytes (272 B for d_idx = 128, 144 B for
// 64): a 16-lane phase of 16-byte reads of rows n .. n + 15 starts at distinct
// 4-bank groups, and every fragment read of a lane is one base address plus a
// compile-time offset.
template <int DIDX>
constexpr int kidx_stride() { return DIDX * 2 + 16; }

template <int DIDX>
__device__ __forceinline__ int kidx_lds_off(int key, int c) {
  return key * kidx_stride<DIDX>() + c * 16;
}

// 16 bytes per lane from global memory straight into LDS: the wave writes
// 1 KB at lds_base (wave-uniform), lane i at lds_base + 16 i, reading
// byte offset voff of the buffer r.  The buffer form (MUBUF) of the LDS load
// is used rather than the global one: with a global load to LDS in flight,
// the compiler cannot count LDS reads in order and makes every wait for an
// LDS fragment wait for all of them; with the buffer form it waits for the
// one fragment an MFMA needs.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, 0, 0, 0);
}
// Raw buffer resource over bytes [p, p + bytes) (gfx9 data-format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Ascending compare-exchange network (bitonic) over KP (power of two) ints.
template <int KP>
__device__ __forceinline__ void sort_ascending(int (&v)[KP]) {
#pragma unroll
  for (int size = 2; size <= KP; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const int a = v[i], b = v[j];
          const int lo = min(a, b), hi = max(a, b);
          v[i] = up ? lo : hi;
          v[j] = up ? hi : lo;
        }
      }
    }
  }
}

// KP = capacity rounded up to a power of two; the list holds KP - 1 entries of
// which the first KP - k are +inf sentinels, so the last entry is always the
// row's (k-1)-th best score.
//
// FORCED (the early-training variant, "MiniMax Sparse Attention", ablation of
// forced sink and local blocks): block 0 (force_first) and the window - 1
// blocks before the local one score +inf, so they always take slots; among
// equal scores the smaller id still wins.
//
// KT: 32-key MFMA tiles per key block, so blocks of BK = 32 KT tokens (the
// block-size variants 32 and 64 of the paper's block-size ablation; 128 is
// the default).
template <int DIDX, int KP, bool FORCED, int KT>
__global__ __launch_bounds__(kIdxThreads, 1) void index_topk_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, int64_t N, int H_kv,
    int k, int64_t q_begin, int64_t q_count, int force_first, int window,
    int32_t* __restrict__ block_idx) {
  constexpr int KM = KP - 1;
  constexpr int NCH = DIDX / 8;
  constexpr int STEPS = DIDX / 16;
  constexpr int KSTR = kidx_stride<DIDX>();
  constexpr int BK = 32 * KT;
  // Ring buffer stride: a whole number of the 1 KB a wave's DMA instruction
  // writes.  The last instruction of a block covers slots past the tile's end
  // (their sources are clamped to the last slot, the LDS destination is not),
  // so with 32-key blocks (4.5 or 8.5 KB of slots) the stride is padded and
  // those lanes land in the buffer's own padding instead of the next buffer.
  constexpr int TILE = (BK * KSTR + 1023) / 1024 * 1024;
  constexpr int NBUF = 4;  // LDS ring: two blocks scored, two in flight
  __shared__ __attribute__((aligned(16))) uint8_t lds[KM > 0 ? NBUF * TILE : 16];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int64_t rows_total = q_count * H_kv;
  const int64_t nwg = (rows_total + kIdxRows - 1) / kIdxRows;
  const int64_t wg = nwg - 1 - static_cast<int64_t>(blockIdx.x);
  const int64_t bat = blockIdx.y;
  const int64_t f0 = wg * kIdxRows;

  // The row whose top-k this lane keeps: column tile h of this wave, column n.
  const int64_t f_mine = f0 + wave * 64 + h * 32 + n;
  const bool mine_ok = f_mine < rows_total;
  const int64_t il_mine = mine_ok ? f_mine / H_kv : 0;
  const int r_mine = mine_ok ? static_cast<int>(f_mine % H_kv) : 0;
  const int L_mine = static_cast<int>((q_begin + il_mine) / BK);
  const int64_t f_last = min(f0 + kIdxRows, rows_total) - 1;
  const int Lmax = static_cast<int>((q_begin + f_last / H_kv) / BK);

  int ids[KM > 0 ? KM : 1];
  if constexpr (KM > 0) {
    float ts[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const bool sentinel = j < KP - k;
      ts[j] = sentinel ? __builtin_huge_valf() : -__builtin_huge_valf();
      ids[j] = sentinel ? INT_MAX : -1;
    }

    // Q^idx fragments of the wave's two 32-row column tiles (B operand).
    bf16x8 qf[2][STEPS];
    const uint16_t* qbase = q_idx + (bat * N + q_begin) * H_kv * DIDX;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      int64_t f = f0 + wave * 64 + nt * 32 + n;
      f = f < rows_total ? f : rows_total - 1;
      const uint16_t* qrow = qbase + f * DIDX;
#pragma unroll
      for (int ks = 0; ks < STEPS; ++ks)
        qf[nt][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * h));
    }

    // K^idx blocks go straight from global memory into a 4-buffer LDS ring
    // (buffer_load ... lds, no registers): while blocks b and b + 1 are scored,
    // blocks b + 2 and b + 3 are in flight into the other two buffers, and one
    // barrier per two blocks makes them visible.  The padded tile is
    // NSLOT = 128 x (NCH + 1) 16-byte slots; wave instruction j fills slots
    // 64 j .. 64 j + 63, lane i slot 64 j + i = (key row) (NCH + 1) + chunk,
    // where the padding chunk NCH loads the row's last chunk again.  A block
    // index past the last is clamped to it (its data is never used).
    const uint16_t* kbase = k_idx + bat * N * DIDX;
    constexpr int NSLOT = BK * (NCH + 1);
    constexpr int NJ = (NSLOT + 63) / 64;          // wave instructions per block
    constexpr int JW = (NJ + kIdxWaves - 1) / kIdxWaves;  // per wave (some do one less)
    int src_off[JW];  // element offset of this lane's slot within a block
#pragma unroll
    for (int q = 0; q < JW; ++q) {
      const int j = wave + kIdxWaves * q;
      const int sl = min(64 * j + lane, NSLOT - 1);
      const int key = sl / (NCH + 1), c = min(sl % (NCH + 1), NCH - 1);
      src_off[q] = key * DIDX + c * 8;
    }
    auto stage_block = [&](int blk, int buf) {
      blk = min(blk, Lmax - 1);
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(kbase + static_cast<int64_t>(blk) * BK * DIDX, BK * DIDX * 2);
#pragma unroll
      for (int q = 0; q < JW; ++q) {
        const int j = wave + kIdxWaves * q;
        if (j < NJ)  // wave-uniform
          lds_dma16(rs, static_cast<uint32_t>(src_off[q]) * 2, lds + buf * TILE + 1024 * j);
      }
    };

    // Insertion of a candidate (score, block) into the row's sorted list: the
    // candidate moves down the list, swapping with every smaller entry.  For
    // lists of up to 15 entries the insertion is branch-free and split over
    // the steps of a key tile, so that its VALU work sits between MFMAs
    // instead of stalling the matrix cores.  (Longer lists would not fit the
    // registers that way; they insert at once, when a lane needs it.)
    constexpr bool kDefer = KP <= 16;
    float pend_x = 0.f;
    int pend_b = 0;
    bool pend_need = false;
    // The list is sorted descending, so c_j = (x > ts[j]) holds exactly for
    // j >= the candidate's place p: entry j takes ts[j - 1] when c_{j-1}
    // (shifted down), x when c_j alone (j = p), and keeps ts[j] otherwise.
    // Walking j downwards keeps ts[j - 1] unmodified when entry j needs it,
    // and each comparison serves two entries: per entry one compare, two
    // selects for the id and one median-of-three for the score.  A candidate that is not needed enters as -inf and moves
    // nothing (the comparisons are strict).
    // The walk can be split into ranges of entries (insert_entries), so that
    // its VALU work can sit between MFMAs.
    float ins_x = 0.f;
    int ins_xi = 0;
    bool ins_c = false;
    auto insert_begin = [&]() {
      ins_x = pend_need ? pend_x : -__builtin_huge_valf();
      ins_xi = pend_b;
      ins_c = ins_x > ts[KM - 1];
    };
    auto insert_entries = [&](int jhi, int jlo) {  // entries jhi down to jlo
#pragma unroll
      for (int j = KM - 1; j >= 0; --j) {
        if (j > jhi || j < jlo) continue;
        // (values, not lvalues, in the selects: a conditional over two
        // lvalues selects an address and would put the list in scratch)
        // The new score is clamp(x, ts[j], ts[j - 1]) (ts[j - 1] >= ts[j]),
        // one v_med3_f32: ts[j - 1] when c_{j-1}, x when c_j alone, ts[j]
        // otherwise, bit for bit the selects below make for the ids.
        const float x = ins_x, tj = ts[j], tp = ts[j > 0 ? j - 1 : 0];
        const int xi = ins_xi, ij = ids[j], ip = ids[j > 0 ? j - 1 : 0];
        const bool c = ins_c, cp = j > 0 && x > tp;
        const int ni = c ? xi : ij;
        ts[j] = j > 0 ? __builtin_amdgcn_fmed3f(x, tp, tj) : fmaxf(x, tj);
        ids[j] = cp ? ip : ni;
        ins_c = cp;
      }
    };
    auto insert_pending = [&]() {
      insert_begin();
      insert_entries(KM - 1, 0);
      pend_need = false;
    };

    // Key tile mt of block b uses accumulators A[(b * KT + mt) & 1], so
    // consecutive tiles alternate also across blocks.  A block's epilogue --
    // the max-pool of its last tile, the exchange between the half-waves, the
    // threshold test and the insertion -- runs under the MFMAs of the next
    // block's first two tiles: the matrix cores go from one block to the next
    // without waiting for it.  (Lists longer than 15 entries leave no
    // registers for that; their blocks finish at once, with A[mt & 1].)
    // mx0 / mx1 collect the pooled maxima of the block whose tiles are being
    // pooled (column tile 0 / 1).
    constexpr bool kLate = kDefer;
    f32x16 A[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) A[st][0] = A[st][1] = f32x16{};
    float mx0 = -__builtin_huge_valf(), mx1 = -__builtin_huge_valf();
    bf16x8 kr[STEPS];
    auto pool = [&](const f32x16& a0, const f32x16& a1, int e0, int e1) {  // elements [e0, e1)
#pragma unroll
      for (int e = e0; e < e1; e += 2) {
        mx0 = max3f(mx0, a0[e], a0[e + 1]);
        mx1 = max3f(mx1, a1[e], a1[e + 1]);
      }
    };
    // Block pb's pooled maxima are complete: lane half 0 holds keys 4h.. of
    // every 8 for both column tiles; v_permlane32_swap hands half 0 the other
    // half's column-tile-0 maxima and half 1 the other half's column-tile-1
    // maxima, so half 0 finishes column tile 0 and half 1 column tile 1.
    auto finish = [&](int pb) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx0), __float_as_uint(mx1), false, false);
      float score = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      if constexpr (FORCED) {
        if ((force_first && pb == 0) || pb > L_mine - window) score = __builtin_huge_valf();
      }
      pend_x = score;
      pend_b = pb;
      pend_need = pb >= 0 && pb < L_mine && score > ts[KM - 1];
      mx0 = mx1 = -__builtin_huge_valf();
    };

    // Score block b (parity PAR = b & 1) from LDS buffer b % NBUF.  Fragment
    // (mt, ks) of this lane: key row 32 mt + n, 16-byte chunk 2 ks + h.  K
    // fragments roll: the register that fed step ks of tile mt is refilled
    // with tile mt + 1's fragment right after its MFMAs, and in the last tile
    // of the first block of a pair with the next block's first fragment (that
    // buffer is already visible), so the second block starts with its
    // operands in registers.  Each pair of MFMAs is followed, inside
    // scheduling fences, by VALU work that does not depend on it: in tile 0
    // the max-pool of the previous block's last tile and then its finish, in
    // tile 1 (KT >= 2) that block's insertion, and from tile 1 on the
    // max-pool of the tile before.
    constexpr int EPK = 16 / STEPS;                // max-pool elements per step
    constexpr int IPK = (KM + STEPS - 1) / STEPS;  // insertion entries per step
    auto score_block = [&](auto par, int b) {
      constexpr int PAR = decltype(par)::value;
      constexpr int SP = ((PAR ^ 1) * KT + KT - 1) & 1;  // the previous block's last tile
      const uint8_t* tile = lds + (b % NBUF) * TILE + n * KSTR + h * 16;
      const uint8_t* tnext = lds + ((b + 1) % NBUF) * TILE + n * KSTR + h * 16;
      if (PAR == 0) {
#pragma unroll
        for (int ks = 0; ks < STEPS; ++ks) kr[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(tile + 32 * ks));
      }
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
        const int st = kLate ? (PAR * KT + mt) & 1 : mt & 1;
#pragma unroll
        for (int ks = 0; ks < STEPS; ++ks) {
          A[st][0] = mfma32x32x16(kr[ks], qf[0][ks], ks ? A[st][0] : f32x16{});
          A[st][1] = mfma32x32x16(kr[ks], qf[1][ks], ks ? A[st][1] : f32x16{});
          __builtin_amdgcn_sched_barrier(0);
          if (mt + 1 < KT)
            kr[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(tile + 32 * (mt + 1) * KSTR + 32 * ks));
          else if (PAR == 0)
            kr[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(tnext + 32 * ks));
          if (mt == 0) {
            if constexpr (kLate) {
              pool(A[SP][0], A[SP][1], EPK * ks, EPK * (ks + 1));
              if (ks == STEPS - 1) {
                finish(b - 1);
                if (KT == 1) insert_pending();
                else insert_begin();
              }
            }
          } else {
            pool(A[st ^ 1][0], A[st ^ 1][1], EPK * ks, EPK * (ks + 1));
            if (kDefer && mt == 1) {
              const int jhi = KM - 1 - IPK * ks, jlo = jhi - IPK + 1;
              if (jhi >= 0) insert_entries(jhi, jlo < 0 ? 0 : jlo);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (!kLate) {
        pool(A[(KT - 1) & 1][0], A[(KT - 1) & 1][1], 0, 16);
        finish(b);
        if (__any(pend_need)) insert_pending();
      }
    };
    // The last block's epilogue, after the loop.
    auto finish_last = [&](auto par) {
      constexpr int SL = (decltype(par)::value * KT + KT - 1) & 1;
      pool(A[SL][0], A[SL][1], 0, 16);
      finish(Lmax - 1);
      insert_pending();
    };

    if (Lmax > 0) {
      stage_block(0, 0);
      stage_block(1, 1);
      __builtin_amdgcn_s_waitcnt(0);  // (all counters: only the ring loads are out)
      __syncthreads();
    }
    for (int b = 0; b < Lmax; b += 2) {
      if (b + 2 < Lmax) {
        stage_block(b + 2, (b + 2) % NBUF);
        stage_block(b + 3, (b + 3) % NBUF);
      }
      score_block(std::integral_constant<int, 0>{}, b);
      if (b + 1 < Lmax) score_block(std::integral_constant<int, 1>{}, b + 1);
      // this wave's ring loads have landed; the barrier makes every wave's
      // visible and frees the two buffers just scored
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (kLate && Lmax > 0) {
      if (KT % 2 == 0 || ((Lmax - 1) & 1)) finish_last(std::integral_constant<int, 1>{});
      else finish_last(std::integral_constant<int, 0>{});
    }
  }

  if (!mine_ok) return;
  int32_t* dst = block_idx + ((bat * H_kv + r_mine) * q_count + il_mine) * k;
  if constexpr (KM == 0) {
    dst[0] = L_mine;
  } else {
    int v[KP];
#pragma unroll
    for (int j = 0; j < KM; ++j) v[j] = ids[j] < 0 ? INT_MAX : ids[j];
    v[KM] = INT_MAX;
    sort_ascending<KP>(v);
    int nv = 0;
#pragma unroll
    for (int j = 0; j < KP; ++j) nv += v[j] != INT_MAX ? 1 : 0;
#pragma unroll
    for (int j = 0; j < KP; ++j)
      if (j < k) dst[j] = j < nv ? v[j] : (j == nv ? L_mine : -1);
  }
}

struct IdxArgs {
  const uint16_t* q_idx;
  const uint16_t* k_idx;
  int batch;
  int64_t N;
  int H_kv, k;
  int64_t q_begin, q_count;
  int force_first, window;
  int32_t* block_idx;
  hipStream_t stream;
  int bk;
};

template <int DIDX, int KP, bool FORCED, int KT>
hipError_t launch_t(const IdxArgs& a) {
  const int64_t nwg = (a.q_count * a.H_kv + kIdxRows - 1) / kIdxRows;
  hipLaunchKernelGGL((index_topk_kernel<DIDX, KP, FORCED, KT>), dim3(static_cast<unsigned>(nwg), a.batch),
                     dim3(kIdxThreads), 0, a.stream, a.q_idx, a.k_idx, a.N, a.H_kv, a.k, a.q_begin,
                     a.q_count, a.force_first, a.window, a.block_idx);
  return hipGetLastError();
}

template <int DIDX, bool FORCED, int KT>
hipError_t launch_k(const IdxArgs& a) {
  if (a.k <= 1) return launch_t<DIDX, 1, FORCED, KT>(a);
  if (a.k <= 2) return launch_t<DIDX, 2, FORCED, KT>(a);
  if (a.k <= 4) return launch_t<DIDX, 4, FORCED, KT>(a);
  if (a.k <= 8) return launch_t<DIDX, 8, FORCED, KT>(a);
  if (a.k <= 16) return launch_t<DIDX, 16, FORCED, KT>(a);
  return launch_t<DIDX, 32, FORCED, KT>(a);
}

template <int DIDX, bool FORCED>
hipError_t launch_d(const IdxArgs& a) {
  if (a.bk == 32) return launch_k<DIDX, FORCED, 1>(a);
  if (a.bk == 64) return launch_k<DIDX, FORCED, 2>(a);
  return launch_k<DIDX, FORCED, 4>(a);
}

}  // namespace

hipError_t launch_index_topk(const uint16_t* q_idx, const uint16_t* k_idx, int batch, int64_t N,
                             int H_kv, int d_idx, int k, int64_t q_begin, int64_t q_count,
                             int32_t* block_idx, hipStream_t stream, int force_first, int window, int bk) {
  const IdxArgs a{q_idx, k_idx, batch, N, H_kv, k, q_begin, q_count, force_first, window, block_idx, stream, bk};
  const bool forced = force_first != 0 || window > 1;
  if (d_idx == 64) return forced ? launch_d<64, true>(a) : launch_d<64, false>(a);
  return forced ? launch_d<128, true>(a) : launch_d<128, false>(a);
}

}  // namespace msa
