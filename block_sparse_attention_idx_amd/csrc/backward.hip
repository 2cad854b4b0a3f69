// Backward pass of MSA: gradients of the sparse main attention and the KL
// alignment gradient of the index branch.
//
// What is computed ("MiniMax Sparse Attention (MSA)", Deep Dive > KL Alignment
// Loss; "Flash-MSA", Backward and KL Divergence Loss): for query i, selection
// group r and its visible selected tokens T (the forward's block selection,
// tokens j <= i), with p_h = softmax_T(scale Q_h . K_j) for the group's heads h,
//   main branch:  dV_j += sum_h p_hj dO_h,   dP_hj = dO_h . V_j,
//                 dS_hj = p_hj (dP_hj - dO_h . O_h),
//                 dQ_h = scale sum_j dS_hj K_j,   dK_j += scale sum_h dS_hj Q_h;
//   index branch: teacher P_j = mean_h p_hj (a constant), proxy
//                 p_px = softmax_T(z_j), z_j = q_idx . k_idx_j / sqrt(d_idx),
//                 KL_i,r = sum_j P_j ln(P_j / p_px,j), and the gradient
//                 w (p_px - P) on z carried to q_idx and k_idx.
//
// Schedule ("Flash-MSA", Backward: the cached selection is inverted and the
// inverse drives the work): the forward's inversion and pass list are reused.
// Each pass is one (sequence, group, key block) bin restricted to up to
// 256 / G consecutive entries (query, slot); persistent workgroups take equal
// contiguous shares of the pass list, so every workgroup keeps one key block
// for a run of passes.  In the main branch (8 waves) wave w owns keys
// 32 (w % 4) .. + 31 of the block and rows 32 (w / 4) .. + 31 of each chunk;
// in the index branch (4 waves) wave w owns keys 32 w .. + 31.  The block's
// K and V rows are staged in LDS when the block changes (the index branch
// keeps its K^idx rows in registers), and each wave accumulates its keys'
// dK^T, dV^T (or dK^idx^T) in MFMA accumulators across the run; when the
// block changes, the accumulators are
// added to fp32 gradient buffers with global atomics (a block's passes may be
// shared by two workgroups, and with more index heads than K/V heads several
// groups share a K/V head).  dQ (and dq_idx) need a sum over the block's keys,
// i.e. over the waves: dS goes through LDS and every (query, slot) writes a
// partial, summed over the slots afterwards as in the forward's combine.
//
// Rows of a pass are processed 64 at a time (64 / G queries x G heads).  All
// products run on v_mfma_f32_32x32x16_bf16:
//   S  = Q K^T       A = Q rows (LDS),       B = K rows (LDS)
//   dP = dO V^T      A = dO rows (LDS),      B = V rows (LDS)
//   dV^T += dO^T P   A = dO^T (LDS, read transposed), B = P straight from the accumulator
//   dK^T += Q^T dS   A = Q^T (LDS, read transposed),  B = dS straight from the accumulator
//   dQ^T = K^T dS^T  A = K^T (LDS, read transposed),  B = dS rows (LDS)
// S, P and dS have the keys on the lane (column) index, so the row-reducing
// products take them as B operands without a shuffle.  Q, dO, K and V sit in
// LDS once, row-major; the transposed A operands come straight out of those
// tiles through ds_read_b64_tr_b16, in the row order the accumulator gives
// the B operand (the 8 rows a lane contributes to one 16-row step are rows
// 4 h .. 4 h + 3 and 8 + 4 h .. 8 + 4 h + 3 of the step).
//
// The main-branch kernel, which has every head's probabilities, also forms
// the teacher distribution (the mean over the group's heads) and writes one
// fp32 row of it per (query, slot); the index-branch kernel reads those rows
// and only the proxy operands.  The proxy softmax needs the proxy LSE over all
// of a query's selected tokens first: a KV-outer pass over the same work list
// (one wave per workgroup) writes one partial LSE per (query, slot), merged per
// query ("Flash-MSA", Backward: a cheap sparse proxy pass recomputes the proxy
// LSE).  Order: D, proxy LSE, main branch (with the teacher rows), index
// branch, then the per-slot sums.
#include "attn_tile.h"
#include "msa_internal.h"

namespace msa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
using tile::bf16_of;
using tile::halves_max;
using tile::halves_sum;

constexpr int kBW = 4;           // waves per index-branch workgroup
constexpr int kBT = 64 * kBW;    // threads
constexpr int kRows = 64;        // (query, head) rows per chunk
constexpr int kStr = 272;        // row-major LDS row: 128 bf16 + 16 B of padding
constexpr int kTStr = 144;       // transposed LDS row: 64 bf16 + 16 B of padding
// Main-branch row-major tiles: 128 bf16 + 48 B of padding.  At this stride
// both of their read forms run without bank conflicts on gfx950: the 16-byte
// fragment reads (32 rows, two 16-byte halves) and the transposed
// ds_read_b64_tr_b16 reads (8 rows of 64 bytes).  At 288 B the fragment
// reads conflict two ways, at 272 B the transposed ones.
constexpr int kRS = 304;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// Column of chunk row rho in a transposed tile: bits 2 and 3 swapped, so the
// rows 16 s + 4 h + (0..3) and 16 s + 8 + 4 h + (0..3) that lane half h feeds
// to 16-row step s are the 8 consecutive columns 16 s + 8 h .. + 7.
__device__ __forceinline__ int tpos(int rho) { return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1); }

// Byte offset of byte b (0 .. 127) of row d in a transposed tile.  The
// row's eight 16-byte chunks are permuted, chunk c stored at position
// c ^ ((d / 8) % 8): the 8-byte stores that fill the tile hit rows 8 apart
// at one column, which at the 144-byte row stride fell on two sets of banks
// (an 8-way conflict); swizzled they take the minimum two passes.  Eight
// consecutive rows, which the fragment reads take together, share one
// permutation, so those reads stay conflict-free.
__device__ __forceinline__ int tr_off(int d, int b) {
  return d * kTStr + ((((b >> 4) ^ (d >> 3)) & 7) << 4) + (b & 15);
}

// A operand of v_mfma_f32_32x32x16_bf16 read transposed out of a row-major
// bf16 tile T (row stride kRS): lane (n, h) receives, as k-values j = 0 .. 7,
// T[r_lo + j][c0 + n] for j < 4 and T[r_hi + j - 4][c0 + n] for j >= 4 (r_lo,
// r_hi may depend on h).  ds_read_b64_tr_b16 works on groups of 16 lanes:
// output lane i of a group receives, as its element m, element i % 4 of the
// 8-byte piece addressed by lane i / 4 + 4 m of the group.  So lane s of group
// g addresses row r + s / 4 and columns c0 + 16 (g % 2) + 4 (s % 4) .. + 3, and
// two reads (rows from r_lo, then from r_hi) give the eight k-values.  At the
// 288-byte stride the 16 pieces of a group (4 rows x 4 column quarters) fall
// on 32 distinct banks.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 lds_frag_tr(const uint8_t* tile, int r_lo, int r_hi, int c0) {
  const int l = threadIdx.x & 63, s = l & 15;
  const int off = (s >> 2) * kRS + 2 * (c0 + 16 * ((l >> 4) & 1) + 4 * (s & 3));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + r_lo * kRS + off));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + r_hi * kRS + off));
  return as_bf16x8(u32x4{__builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 0, 1)),
                         __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 2, 3))});
}

// Accumulator element e of a 32x32 tile holds row 8 (e / 4) + 4 h + (e % 4).
__device__ __forceinline__ int acc_row(int e, int h) { return 8 * (e >> 2) + 4 * h + (e & 3); }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.f) & 0xFFFFu);
}

// Elements 8 s .. 8 s + 7 of a tile accumulator (rows 16 s + 8 a + 4 h + b,
// slot 4 a + b) as the bf16 B operand of one 16-row step.
__device__ __forceinline__ bf16x8 pack_step(const f32x16& a, int s) {
  return as_bf16x8(u32x4{pack_bf16x2(a[8 * s + 0], a[8 * s + 1]), pack_bf16x2(a[8 * s + 2], a[8 * s + 3]),
                         pack_bf16x2(a[8 * s + 4], a[8 * s + 5]), pack_bf16x2(a[8 * s + 6], a[8 * s + 7])});
}

__device__ __forceinline__ bf16x8 lds_frag(const uint8_t* p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

// This workgroup's passes: the sequences in order and, in each, one
// contiguous equal share of its passes (the forward's partition).
struct PassIter {
  const int32_t* segp;
  int B_c, nseqs;
  int pair = -1, p = 0, end = 0;
  __device__ int next() {
    if (++p < end) return p;
    while (++pair < nseqs) {
      const int a = segp[pair * B_c];
      const int64_t np = segp[(pair + 1) * B_c] - a;
      const int s0 = a + static_cast<int>(np * blockIdx.x / gridDim.x);
      const int s1 = a + static_cast<int>(np * (blockIdx.x + 1) / gridDim.x);
      if (s0 < s1) {
        p = s0;
        end = s1;
        return s0;
      }
    }
    return -1;
  }
};

// Where entry word `ent` (query row * k + slot) of group seq points.
struct EntryRef {
  int i;          // query position
  int64_t slot;   // (seq, query row, slot) index
};
__device__ __forceinline__ EntryRef entry_ref(uint32_t ent, int seq, int kslots, int q_begin, int q_count) {
  const uint32_t qrow = ent / static_cast<uint32_t>(kslots);
  const uint32_t s = ent - qrow * static_cast<uint32_t>(kslots);
  EntryRef r;
  r.i = q_begin + static_cast<int>(qrow);
  r.slot = (static_cast<int64_t>(seq) * q_count + qrow) * kslots + s;
  return r;
}

// Staging of 64 rows of a [*, d_h = 128] bf16 tensor for software
// pipelining, by 1024 / RPT threads: load_rows issues this thread's
// global loads (16-byte chunk t % 16 of rows RPT (t / 16) .. + RPT - 1;
// `row_ptr(rho)` must give a readable row), put_rows writes them row-major
// into `rm` (row stride kRS).
template <int RPT, typename RowPtr>
__device__ __forceinline__ void load_rows(RowPtr row_ptr, u32x4 (&w)[RPT]) {
  const int dg = threadIdx.x & 15, rc = threadIdx.x >> 4;
#pragma unroll
  for (int j = 0; j < RPT; ++j) w[j] = *reinterpret_cast<const u32x4*>(row_ptr(RPT * rc + j) + 8 * dg);
}

template <int RPT>
__device__ __forceinline__ void put_rows(const u32x4 (&w)[RPT], uint8_t* rm) {
  const int dg = threadIdx.x & 15, rc = threadIdx.x >> 4;
#pragma unroll
  for (int j = 0; j < RPT; ++j) *reinterpret_cast<u32x4*>(rm + (RPT * rc + j) * kRS + 16 * dg) = w[j];
}

// The chunks of a workgroup's passes in order: pass descriptor and first
// entry.  `next_chunk` advances the pass iterator, so it is called once per chunk,
// in sequence.
struct Chunk {
  PassDesc D;
  int cb;
  bool ok;
};

//
// MERGE: a chunk may also span several passes.  The passes of one (seq, key
// block) segment hold consecutive runs of its entries, so when a pass holds
// fewer than EC entries, the passes that follow it in the workgroup's share
// and continue the same run join its chunk while the total fits in EC.
template <int EC, bool MERGE>
__device__ __forceinline__ PassDesc take_pass(int pi, PassIter& it, const PassDesc* __restrict__ passes) {
  PassDesc D = passes[pi];
  if constexpr (MERGE) {
    while (D.cnt < EC && it.p + 1 < it.end) {
      const PassDesc E = passes[it.p + 1];
      if (E.seq != D.seq || E.blk != D.blk || E.start != D.start + D.cnt || D.cnt + E.cnt > EC) break;
      ++it.p;
      D.cnt += E.cnt;
    }
  }
  return D;
}

template <int EC, bool MERGE = false>
__device__ __forceinline__ Chunk first_chunk(PassIter& it, const PassDesc* __restrict__ passes) {
  Chunk c{};
  const int pi = it.next();
  c.ok = pi >= 0;
  if (c.ok) c.D = take_pass<EC, MERGE>(pi, it, passes);
  c.cb = 0;
  return c;
}

template <int EC, bool MERGE = false>
__device__ __forceinline__ Chunk next_chunk(const Chunk& c, PassIter& it, const PassDesc* __restrict__ passes) {
  Chunk n = c;
  n.cb += EC;
  if (n.cb >= c.D.cnt) {
    const int pi = it.next();
    n.ok = pi >= 0;
    if (n.ok) n.D = take_pass<EC, MERGE>(pi, it, passes);
    n.cb = 0;
  }
  return n;
}

// Write the 32 keys x 128 dims a wave holds in registers (lane n: key n, dims
// 16 ks + 8 h .. + 7) transposed into `kt` ([dim][key], kStr per dim row),
// columns 32 wave + n.
template <int KS>
__device__ __forceinline__ void store_keys_t(const u32x4 (&f)[KS], uint8_t* kt, int wave, int n, int h) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int dd = 0; dd < 8; ++dd)
      *reinterpret_cast<uint16_t*>(kt + (16 * ks + 8 * h + dd) * kStr + 2 * (32 * wave + n)) =
          static_cast<uint16_t>(bf16_of(f[ks], dd));
}

// ---------------------------------------------------------------- main branch
// Workgroup of 8 waves, two per SIMD.  Wave w owns keys 32 (w % 4) .. + 31
// of the block and rows 32 (w / 4) .. + 31 of each 64-row chunk: it forms S,
// P, dP and dS of that 32 x 32 tile and adds its rows' share of dV^T and dK^T
// of its keys to accumulators of its own (waves w and w + 4 both add theirs
// into the fp32 buffers when the block changes).  No product is formed twice
// and each wave keeps one 32-key x 128-dim dV^T, dK^T pair, so a wave fits
// the 256 registers of two waves per SIMD.  Then all 8 waves share
// dQ^T = K^T dS^T.
// IDX: the index branch runs, so the teacher T of every entry (the mean over
// the G heads of the probabilities of each key of the block) is written to
// `tch_out` ([slot][key] fp32) for the index-branch kernel.
constexpr int kMW = 8;           // waves per main-branch workgroup
constexpr int kMT = 64 * kMW;    // threads
constexpr int kMRows = 1024 / kMT;  // staged rows per thread (64 rows x 16 chunks)

template <int G, bool IDX>
__global__ __launch_bounds__(kMT, 1) void bwd_main_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dlt,
    int64_t N, int H_sel, int kv_shift, int kslots, float scale, float scale_log2,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ segp,
    const PassDesc* __restrict__ passes, int B_c, int nseqs, int q_begin, int q_count, int64_t dummy_slot,
    uint16_t* __restrict__ dq_part, float* __restrict__ dk_acc, float* __restrict__ dv_acc,
    float* __restrict__ tch_out) {
  constexpr int EC = kRows / G;  // queries per chunk
  constexpr float kInvG = 1.f / G;
  constexpr int RPT = kMRows;
  __shared__ __attribute__((aligned(16))) uint8_t qr_lds[kRows * kRS];
  __shared__ __attribute__((aligned(16))) uint8_t dor_lds[kRows * kRS];
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kBk * kRS];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[kBk * kRS];
  __shared__ __attribute__((aligned(16))) uint8_t ds_lds[kRows * kStr];
  __shared__ __attribute__((aligned(16))) int ri_i[kRows];
  __shared__ __attribute__((aligned(16))) float ri_lse2[kRows], ri_dlt[kRows];
  __shared__ int64_t ri_orow[kRows];

  PassIter it{segp, B_c, nseqs};
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int kw = wave & 3, rt = wave >> 2;  // key tile, row tile
  const int H_q = H_sel * G, H_kv = H_sel >> kv_shift;
  const int key_l = 32 * kw + n;  // this lane's key within the block

  int cur_seq = -1, cur_blk = 0, cur_nvalid = 0;
  f32x16 dkt[4], dvt[4];  // this wave's rows' share of dK^T, dV^T of its keys

  auto flush = [&]() {
    if (cur_seq < 0 || key_l >= cur_nvalid) return;
    const int bat = cur_seq / H_sel, r = cur_seq - bat * H_sel;
    const int64_t row = (static_cast<int64_t>(bat) * N + static_cast<int64_t>(cur_blk) * kBk + key_l) * H_kv +
                        (r >> kv_shift);
    float* dkp = dk_acc + row * kDh;
    float* dvp = dv_acc + row * kDh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int d = 32 * dt + acc_row(e, h);
        unsafeAtomicAdd(dkp + d, dkt[dt][e] * scale);
        unsafeAtomicAdd(dvp + d, dvt[dt][e]);
      }
  };

  // Software pipeline over the workgroup's chunks: while chunk c computes,
  // chunk c + 1's entries are loaded (before S) and then its Q and dO rows
  // and row constants (after S), into registers that go to LDS at the top of
  // the next iteration.  Every global load and store of the loop is issued
  // unconditionally (rows past a pass's end read its last entry and store
  // their zero dQ to a spare row), so the in-order vmcnt waits never drain
  // the prefetch early.
  Chunk cur = first_chunk<EC>(it, passes);
  if (!cur.ok) return;
  u32x4 wq[RPT], wdo[RPT];  // this thread's staging chunks of the next rows
  int p_i = -1;             // the row constants of row tid (< kRows); the loaded
  float p_l = 0.f, p_dl = 0.f;  // lse and D stay raw until the next iteration
  int64_t p_orow = 0;
  const int rc = tid >> 4, crow = tid & (kRows - 1);

  // entry words of chunk c for this thread's staging rows and constant row
  auto chunk_entries = [&](const Chunk& c, uint32_t (&en)[RPT], uint32_t& enc) {
#pragma unroll
    for (int j = 0; j < RPT; ++j)
      en[j] = static_cast<uint32_t>(entries[c.D.start + min(c.cb + (RPT * rc + j) / G, c.D.cnt - 1)]);
    enc = static_cast<uint32_t>(entries[c.D.start + min(c.cb + crow / G, c.D.cnt - 1)]);
  };
  // issue the row loads of chunk c from its entry words
  auto chunk_rows = [&](const Chunk& c, const uint32_t (&en)[RPT], uint32_t enc) {
    const int cbat = c.D.seq / H_sel, cr = c.D.seq - cbat * H_sel;
    auto rowoff = [&](uint32_t ent, int rho) -> int64_t {
      const EntryRef x = entry_ref(ent, c.D.seq, kslots, q_begin, q_count);
      return (static_cast<int64_t>(cbat) * N + x.i) * H_q + cr * G + rho % G;
    };
    load_rows<RPT>([&](int rho) { return q + rowoff(en[rho % RPT], rho) * kDh; }, wq);
    load_rows<RPT>([&](int rho) { return dout + rowoff(en[rho % RPT], rho) * kDh; }, wdo);
    const EntryRef x = entry_ref(enc, c.D.seq, kslots, q_begin, q_count);
    const int64_t o = (static_cast<int64_t>(cbat) * N + x.i) * H_q + cr * G + crow % G;
    const bool ok = c.cb + crow / G < c.D.cnt;
    p_l = lse[o];
    p_dl = dlt[o];
    p_i = ok ? x.i : -1;
    p_orow = (ok ? x.slot : dummy_slot) * G + crow % G;
  };
  {
    uint32_t en[RPT], enc;
    chunk_entries(cur, en, enc);
    chunk_rows(cur, en, enc);
  }
  Chunk nx = next_chunk<EC>(cur, it, passes);

  while (true) {
    const PassDesc D = cur.D;
    const int bat = D.seq / H_sel, r = D.seq - bat * H_sel;
    // ---- this chunk's rows and constants into LDS
    put_rows<RPT>(wq, qr_lds);
    put_rows<RPT>(wdo, dor_lds);
    if (tid < kRows) {
      ri_i[tid] = p_i;
      ri_lse2[tid] = p_i >= 0 ? p_l * kLog2e : 0.f;
      ri_dlt[tid] = p_i >= 0 ? p_dl : 0.f;
      ri_orow[tid] = p_orow;
    }
    if (D.seq != cur_seq || D.blk != cur_blk) {
      flush();
      cur_seq = D.seq;
      cur_blk = D.blk;
      const int64_t key0 = static_cast<int64_t>(D.blk) * kBk;
      cur_nvalid = static_cast<int>(min<int64_t>(kBk, N - key0));
      // the block's K and V rows into LDS, row-major (keys at or past the
      // sequence end as zeros): thread t moves 16-byte chunk t % 16 of keys
      // t / 16 + 32 p.  Every wave finished the previous chunk's reads of
      // them (trailing barrier); the barrier below publishes them.
      const int64_t rstride = static_cast<int64_t>(H_kv) * kDh;
      const uint16_t* kb = k + ((static_cast<int64_t>(bat) * N + key0) * H_kv + (r >> kv_shift)) * kDh;
      const uint16_t* vb = v + ((static_cast<int64_t>(bat) * N + key0) * H_kv + (r >> kv_shift)) * kDh;
      const int ch = tid & 15;
      constexpr int KP = kBk * 16 / kMT;  // keys per thread
      u32x4 a[KP], b[KP];
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        const int key = (tid >> 4) + (kMT / 16) * p;
        const int64_t o = min(key, cur_nvalid - 1) * rstride + 8 * ch;
        a[p] = *reinterpret_cast<const u32x4*>(kb + o);
        b[p] = *reinterpret_cast<const u32x4*>(vb + o);
      }
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        const int key = (tid >> 4) + (kMT / 16) * p;
        const bool ok = key < cur_nvalid;
        *reinterpret_cast<u32x4*>(k_lds + key * kRS + 16 * ch) = ok ? a[p] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(v_lds + key * kRS + 16 * ch) = ok ? b[p] : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        dkt[dt] = f32x16{};
        dvt[dt] = f32x16{};
      }
    }
    const int key_abs = D.blk * kBk + key_l;
    // ---- the next chunk's entry words (the last chunk reloads its own)
    const Chunk& src = nx.ok ? nx : cur;
    uint32_t en[RPT], enc;
    chunk_entries(src, en, enc);
    __syncthreads();

    // ---- S, P, dP, dS of the wave's tile (lane = key, elements = rows)
    bf16x8 pb[2], db[2];  // P and dS as B operands of the tile's two 16-row steps
    {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = (32 * rt + n) * kRS + 32 * ks + 16 * h;
        const int koff = key_l * kRS + 32 * ks + 16 * h;
        s = mfma32x32x16(lds_frag(qr_lds + off), lds_frag(k_lds + koff), s);
        dp = mfma32x32x16(lds_frag(dor_lds + off), lds_frag(v_lds + koff), dp);
      }
      f32x16 p, ds;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        // elements 4 a4 .. + 3 are rows rb .. rb + 3: one 16-byte read per constant
        const int rb = 32 * rt + 8 * a4 + 4 * h;
        const i32x4 ri = *reinterpret_cast<const i32x4*>(ri_i + rb);
        const f32x4 rl = *reinterpret_cast<const f32x4*>(ri_lse2 + rb);
        const f32x4 rd = *reinterpret_cast<const f32x4*>(ri_dlt + rb);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int e = 4 * a4 + b;
          // the exponential runs for every key and a bit mask hides the keys
          // past the row (no branch per element)
          const float ev = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], scale_log2, -rl[b]));
          const float pe = __uint_as_float(__float_as_uint(ev) & (key_abs <= ri[b] ? 0xFFFFFFFFu : 0u));
          p[e] = pe;
          ds[e] = pe * (dp[e] - rd[b]);
          *reinterpret_cast<uint16_t*>(ds_lds + (rb + b) * kStr + 2 * key_l) = bf16_bits(ds[e]);
        }
      }
      pb[0] = pack_step(p, 0);
      pb[1] = pack_step(p, 1);
      db[0] = pack_step(ds, 0);
      db[1] = pack_step(ds, 1);
      if constexpr (IDX) {
        // teacher: the mean over a query's G heads of this lane's key.  The
        // lane holds rows acc_row(e, h): for G <= 4 each run of G elements
        // is one query's heads; for G = 8 elements 4a .. 4a + 3 of the two
        // lane halves are the two halves of one query's heads, for G = 16
        // elements 0-7 (8-15) of both halves.  The halves meet through
        // v_permlane32_swap (half 0 receives the total of the first
        // operand, half 1 of the second), so every (query, key) value is
        // formed in registers and stored once, straight into its entry's
        // teacher row (32 lanes write 128 contiguous bytes).
        if constexpr (G <= 4) {
#pragma unroll
          for (int e0 = 0; e0 < 16; e0 += G) {
            float t = 0.f;
#pragma unroll
            for (int e = e0; e < e0 + G; ++e) t += p[e];
            tch_out[(ri_orow[32 * rt + acc_row(e0, h)] / G) * kBk + key_l] = t * kInvG;
          }
        } else {
          constexpr int NS = 16 / (G / 2);  // per-half sums: 4 (G = 8) or 2 (G = 16)
          float hs[NS];
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            hs[j] = 0.f;
#pragma unroll
            for (int e = j * (G / 2); e < (j + 1) * (G / 2); ++e) hs[j] += p[e];
          }
#pragma unroll
          for (int j = 0; j < NS; j += 2) {
            const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(hs[j]), __float_as_uint(hs[j + 1]),
                                                             false, false);
            const float tot = __uint_as_float(x[0]) + __uint_as_float(x[1]);
            // query (32 rt + 8 j (G = 8) or 16 j (G = 16)) / G, plus the half
            tch_out[(ri_orow[((32 * rt) / G + j + h) * G] / G) * kBk + key_l] = tot * kInvG;
          }
        }
      }
    }

    // ---- the next chunk's rows go out while this chunk finishes
    chunk_rows(src, en, enc);

    // ---- dV^T += dO^T P, dK^T += Q^T dS over the tile's 32 rows
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // rows 16 st + 4 h + (0..3) and 16 st + 8 + 4 h + (0..3) (st = 2 rt + j):
        // the order in which pb[j] and db[j] hold them
        const int r_lo = 16 * (2 * rt + j) + 4 * h, r_hi = r_lo + 8;
        dvt[dt] = mfma32x32x16(lds_frag_tr(dor_lds, r_lo, r_hi, 32 * dt), pb[j], dvt[dt]);
        dkt[dt] = mfma32x32x16(lds_frag_tr(qr_lds, r_lo, r_hi, 32 * dt), db[j], dkt[dt]);
      }
    __syncthreads();

    // ---- dQ^T = K^T dS^T over the block's 128 keys: wave w takes rows
    // 32 (w / 4) .. + 31 and dims 32 (w % 4) .. + 31
    {
      const int dt = wave & 3;
      f32x16 qa = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        qa = mfma32x32x16(lds_frag_tr(k_lds, 16 * kk + 8 * h, 16 * kk + 8 * h + 4, 32 * dt),
                          lds_frag(ds_lds + (32 * rt + n) * kStr + 32 * kk + 16 * h), qa);
      const int rho = 32 * rt + n;
      uint16_t* dst = dq_part + ri_orow[rho] * kDh;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d0 = 32 * dt + 8 * e4 + 4 * h;
        *reinterpret_cast<u32x2*>(dst + d0) =
            u32x2{pack_bf16x2(qa[4 * e4] * scale, qa[4 * e4 + 1] * scale),
                  pack_bf16x2(qa[4 * e4 + 2] * scale, qa[4 * e4 + 3] * scale)};
      }
    }
    __syncthreads();
    if (!nx.ok) break;
    cur = nx;
    nx = next_chunk<EC>(cur, it, passes);
  }
  // The prefetch registers stay live on the exit path: otherwise the compiler
  // sinks their loads to the loop's back edge (where the exit path no longer
  // runs them) and the next iteration waits for them at once.
#pragma unroll
  for (int j = 0; j < RPT; ++j) asm volatile("" ::"v"(wq[j]), "v"(wdo[j]));
  asm volatile("" ::"v"(p_l), "v"(p_dl));
  flush();
}

// ---------------------------------------------------------------- index branch
// The teacher T (for each entry (query, slot) and key of the block, the mean
// over the group's heads of the main probabilities; zero for keys past the
// query) comes from the main-branch kernel as one fp32 row per entry, so this
// kernel reads only the proxy operands: z = q_idx . k_idx (scaled),
// p_px = exp(z - LSE_px), the KL terms T ln(T / p_px) and g = w (p_px - T),
// then dk_idx^T += q_idx^T g (per-block accumulators, as dK) and
// dq_idx^T = k_idx^T g^T per entry.  Chunks are EI index rows (entries) of
// one key block, from one pass or from consecutive passes of the block,
// prefetched one chunk ahead like the main branch.
template <int G, int DIDX>
__global__ __launch_bounds__(kBT, 1) void bwd_idx_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const float* __restrict__ lsei2,
    const float* __restrict__ tch_in, int64_t N, int H_sel, int kslots, float idx_scale_log2, float gscale,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ segp,
    const PassDesc* __restrict__ passes, int B_c, int nseqs, int q_begin, int q_count, int64_t dummy_slot,
    float* __restrict__ dqi_part, float* __restrict__ kl_part, float* __restrict__ dki_acc) {
  // Index rows per chunk: 64 entries of one key block, from one pass (a pass
  // holds 256 / G entries) or from consecutive passes of the block (G >= 8).
  constexpr int EI = 64;
  constexpr int ZT = (EI + 31) / 32;           // 32-row tiles of index rows
  constexpr int KE = (EI + 15) / 16;           // 16-row steps of index rows
  constexpr int KSI = DIDX / 16;               // reduction steps of the index dot product
  constexpr int TT = DIDX / 32;                // 32-dim tiles of dq_idx / dk_idx
  constexpr int NCI = DIDX / 8;                // 16-byte chunks per index row
  constexpr int NT4 = EI * (kBk / 4) / kBT;    // 16-byte pieces of T per thread
  static_assert(EI % kBW == 0 && NT4 >= 1, "chunk shape");
  __shared__ __attribute__((aligned(16))) uint8_t qi_lds[64 * kStr];
  __shared__ __attribute__((aligned(16))) uint8_t qit_lds[kDh * kTStr];
  __shared__ __attribute__((aligned(16))) uint8_t kit_lds[kDh * kStr];
  __shared__ __attribute__((aligned(16))) uint8_t g_lds[64 * kStr];
  __shared__ __attribute__((aligned(16))) float tt[EI * kBk];  // teacher, then KL terms, [index row][key]
  __shared__ int ei_i[64];
  __shared__ float ei_l2[64];
  __shared__ int64_t ei_slot[64];

  PassIter it{segp, B_c, nseqs};
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int key_l = 32 * wave + n;

  int cur_seq = -1, cur_blk = 0, cur_nvalid = 0;
  u32x4 kif[KSI];
  f32x16 dkit[TT];

  auto flush = [&]() {
    if (cur_seq < 0 || key_l >= cur_nvalid) return;
    const int bat = cur_seq / H_sel;
    float* dst = dki_acc + (static_cast<int64_t>(bat) * N + static_cast<int64_t>(cur_blk) * kBk + key_l) * DIDX;
#pragma unroll
    for (int tt2 = 0; tt2 < TT; ++tt2)
#pragma unroll
      for (int e = 0; e < 16; ++e) unsafeAtomicAdd(dst + 32 * tt2 + acc_row(e, h), dkit[tt2][e]);
  };

  Chunk cur = first_chunk<EI, true>(it, passes);
  if (!cur.ok) return;
  const int rc = tid >> 4, dg = tid & 15, crow = tid & 63;
  u32x4 wqi[4];       // this thread's 16-byte pieces of index rows 4 rc .. + 3
  f32x4 wt[NT4];      // and of T rows tid / 32 + 8 j (pieces tid % 32)
  int pe_i = -1;      // row constants of index row crow; the loaded proxy LSE
  float pe_l = 0.f;   // stays raw until the next iteration
  int64_t pe_slot = 0;

  auto chunk_entries = [&](const Chunk& c, uint32_t (&eni)[4], uint32_t (&ent)[NT4], uint32_t& enci) {
    const int last = c.D.cnt - 1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      eni[j] = static_cast<uint32_t>(entries[c.D.start + min(c.cb + min(4 * rc + j, EI - 1), last)]);
#pragma unroll
    for (int j = 0; j < NT4; ++j)
      ent[j] = static_cast<uint32_t>(entries[c.D.start + min(c.cb + (tid >> 5) + 8 * j, last)]);
    enci = static_cast<uint32_t>(entries[c.D.start + min(c.cb + min(crow, EI - 1), last)]);
  };
  auto chunk_rows = [&](const Chunk& c, const uint32_t (&eni)[4], const uint32_t (&ent)[NT4], uint32_t enci) {
    const int cbat = c.D.seq / H_sel, cr = c.D.seq - cbat * H_sel;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const EntryRef x = entry_ref(eni[j], c.D.seq, kslots, q_begin, q_count);
      wqi[j] = *reinterpret_cast<const u32x4*>(
          q_idx + ((static_cast<int64_t>(cbat) * N + x.i) * H_sel + cr) * DIDX + 8 * min(dg, NCI - 1));
    }
#pragma unroll
    for (int j = 0; j < NT4; ++j) {
      const EntryRef x = entry_ref(ent[j], c.D.seq, kslots, q_begin, q_count);
      wt[j] = *reinterpret_cast<const f32x4*>(tch_in + x.slot * kBk + 4 * (tid & 31));
    }
    const EntryRef y = entry_ref(enci, c.D.seq, kslots, q_begin, q_count);
    pe_l = lsei2[y.slot / kslots];
    const bool oke = crow < EI && c.cb + crow < c.D.cnt;
    pe_i = oke ? y.i : -1;
    pe_slot = oke ? y.slot : dummy_slot;
  };
  {
    uint32_t eni[4], ent[NT4], enci;
    chunk_entries(cur, eni, ent, enci);
    chunk_rows(cur, eni, ent, enci);
  }
  Chunk nx = next_chunk<EI, true>(cur, it, passes);

  while (true) {
    const PassDesc D = cur.D;
    const int bat = D.seq / H_sel;
    // ---- this chunk's index rows (row-major and transposed; rows past the
    // chunk are zeros), T rows (zeros for padding rows) and row constants
    if (dg < NCI) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 w = 4 * rc + j < EI ? wqi[j] : u32x4{0u, 0u, 0u, 0u};
        wqi[j] = w;
        *reinterpret_cast<u32x4*>(qi_lds + (4 * rc + j) * kStr + 16 * dg) = w;
      }
      const int col = tpos(4 * rc);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const u32x2 v = {bf16_of(wqi[0], dd) | (bf16_of(wqi[1], dd) << 16),
                         bf16_of(wqi[2], dd) | (bf16_of(wqi[3], dd) << 16)};
        *reinterpret_cast<u32x2*>(qit_lds + tr_off(8 * dg + dd, 2 * col)) = v;
      }
    }
#pragma unroll
    for (int j = 0; j < NT4; ++j) {
      const int row = (tid >> 5) + 8 * j;
      *reinterpret_cast<f32x4*>(tt + row * kBk + 4 * (tid & 31)) =
          cur.cb + row < D.cnt ? wt[j] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (tid < 64) {
      ei_i[tid] = pe_i;
      ei_l2[tid] = pe_i >= 0 ? pe_l : 0.f;
      ei_slot[tid] = pe_slot;
    }
    if (D.seq != cur_seq || D.blk != cur_blk) {
      flush();
      cur_seq = D.seq;
      cur_blk = D.blk;
      const int64_t key0 = static_cast<int64_t>(D.blk) * kBk;
      cur_nvalid = static_cast<int>(min<int64_t>(kBk, N - key0));
      const int kr = min(key_l, cur_nvalid - 1);
      const bool ok = key_l < cur_nvalid;
      const uint16_t* kib = k_idx + (static_cast<int64_t>(bat) * N + key0 + kr) * DIDX;
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kib + 16 * ks + 8 * h);
        kif[ks] = ok ? a : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int t2 = 0; t2 < TT; ++t2) dkit[t2] = f32x16{};
      store_keys_t<KSI>(kif, kit_lds, wave, n, h);
    }
    const int key_abs = D.blk * kBk + key_l;
    const Chunk& src = nx.ok ? nx : cur;
    uint32_t eni[4], ent[NT4], enci;
    chunk_entries(src, eni, ent, enci);
    __syncthreads();

    // ---- proxy probabilities, KL terms and the gradient g on z
    bf16x8 gb[2 * ZT];
#pragma unroll
    for (int zt = 0; zt < ZT; ++zt) {
      f32x16 z = {};
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks)
        z = mfma32x32x16(lds_frag(qi_lds + (32 * zt + n) * kStr + 32 * ks + 16 * h), as_bf16x8(kif[ks]), z);
      f32x16 g;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = 32 * zt + acc_row(e, h);
        float ge = 0.f;
        if (row < EI) {
          const bool vis = key_abs <= ei_i[row];
          const float zl2 = __builtin_fmaf(z[e], idx_scale_log2, -ei_l2[row]);  // log2 p_px
          const float ppx = vis ? __builtin_amdgcn_exp2f(zl2) : 0.f;
          float* tp = tt + row * kBk + key_l;
          const float T = *tp;
          *tp = (vis && T > 0.f) ? T * (__builtin_amdgcn_logf(T) - zl2) * kLn2 : 0.f;
          ge = gscale * (ppx - T);
          *reinterpret_cast<uint16_t*>(g_lds + row * kStr + 2 * key_l) = bf16_bits(ge);
        }
        g[e] = ge;
      }
      gb[2 * zt] = pack_step(g, 0);
      gb[2 * zt + 1] = pack_step(g, 1);
    }

    // ---- the next chunk's rows go out while this chunk finishes
    chunk_rows(src, eni, ent, enci);

    // ---- dk_idx^T += q_idx^T g (reduction over the chunk's index rows)
#pragma unroll
    for (int t2 = 0; t2 < TT; ++t2)
#pragma unroll
      for (int st = 0; st < KE; ++st)
        dkit[t2] = mfma32x32x16(lds_frag(qit_lds + tr_off(32 * t2 + n, 32 * st + 16 * h)), gb[st], dkit[t2]);
    __syncthreads();

    // ---- dq_idx^T = k_idx^T g^T over the block's keys (rows past the chunk
    // write the spare row), and the per-row KL sums (a wave per row); the
    // trip counts are compile-time, so the compiler can count the stores its
    // waits leave in flight
    constexpr int NXT = (TT * ZT + kBW - 1) / kBW;
#pragma unroll
    for (int j = 0; j < NXT; ++j) {
      const int x = wave + kBW * j;
      if ((TT * ZT) % kBW != 0 && x >= TT * ZT) break;
      const int t2 = x % TT, zt = x / TT;
      f32x16 a = {};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
        a = mfma32x32x16(lds_frag(kit_lds + (32 * t2 + n) * kStr + 32 * kk + 16 * h),
                         lds_frag(g_lds + (32 * zt + n) * kStr + 32 * kk + 16 * h), a);
      const int row = 32 * zt + n;
      float* dst = dqi_part + (row < EI ? ei_slot[row] : dummy_slot) * DIDX + 32 * t2 + 4 * h;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<f32x4*>(dst + 8 * e4) = f32x4{a[4 * e4], a[4 * e4 + 1], a[4 * e4 + 2], a[4 * e4 + 3]};
    }
    {
      // row tid / 4, keys 32 (tid % 4) .. + 31: eight 16-byte reads, then the
      // four threads of the row add their sums (two shuffles in a quad)
      static_assert(EI * 4 == kBT, "one thread per quarter row");
      const int row = tid >> 2, q4 = tid & 3;
      const f32x4* src = reinterpret_cast<const f32x4*>(tt + row * kBk + 32 * q4);
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 x = src[j];
        sum += (x[0] + x[1]) + (x[2] + x[3]);
      }
      sum += __shfl_xor(sum, 1);
      sum += __shfl_xor(sum, 2);
      kl_part[ei_slot[row]] = sum;  // the quad's four lanes: the same value to the same word
    }
    __syncthreads();
    if (!nx.ok) break;
    cur = nx;
    nx = next_chunk<EI, true>(cur, it, passes);
  }
  // (the prefetch registers stay live on the exit path; see the main branch)
  asm volatile("" ::"v"(wqi[0]), "v"(wqi[1]), "v"(wqi[2]), "v"(wqi[3]), "v"(pe_l));
#pragma unroll
  for (int j = 0; j < NT4; ++j) asm volatile("" ::"v"(wt[j]));
  flush();
}

// ---------------------------------------------------------------- proxy LSE
// One wave per workgroup: for every entry (query, slot) of a pass, the
// log2-sum-exp2 of its proxy scores over the block's visible keys, 32
// entries at a time (a pass of fewer entries takes the block's next passes
// along).  z^T = K^idx Q^idx^T with the keys on the row index, as in the
// forward.  Software pipeline over chunks of 32 entries: while chunk c is
// scored, the Q^idx rows of chunk c+1 are in flight and the entry words of
// chunk c+2 are read (past the end of the work the last chunk stands in, so
// every load of the loop is unconditional).
constexpr int kLseWgPerCu = 4;

template <int DIDX>
__global__ __launch_bounds__(64) void proxy_lse_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, int64_t N, int H_sel, int kslots,
    float idx_scale_log2, const int32_t* __restrict__ entries, const int32_t* __restrict__ segp,
    const PassDesc* __restrict__ passes, int B_c, int nseqs, int q_begin, int q_count,
    float* __restrict__ lsei_part) {
  constexpr int KSI = DIDX / 16;
  constexpr int KC = DIDX / 8;  // 16-byte chunks per K^idx row
  __shared__ __attribute__((aligned(16))) uint8_t ki_lds[kBk * kStr];
  PassIter it{segp, B_c, nseqs};
  const int lane = threadIdx.x, n = lane & 31, h = lane >> 5;

  auto entry_of = [&](const Chunk& c) {
    const int e = c.cb + n;
    return static_cast<uint32_t>(entries[c.D.start + (e < c.D.cnt ? e : c.cb)]);
  };
  auto q_of = [&](const Chunk& c, uint32_t ent, bf16x8(&qf)[KSI]) {
    const int bat = c.D.seq / H_sel, r = c.D.seq - bat * H_sel;
    const EntryRef er = entry_ref(ent, c.D.seq, kslots, q_begin, q_count);
    const uint16_t* qr = q_idx + ((static_cast<int64_t>(bat) * N + er.i) * H_sel + r) * DIDX;
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + 16 * ks + 8 * h));
  };

  Chunk cur = first_chunk<32, true>(it, passes);
  if (!cur.ok) return;  // uniform
  uint32_t ent_cur = entry_of(cur);
  bf16x8 q_cur[KSI];
  q_of(cur, ent_cur, q_cur);
  Chunk nx = next_chunk<32, true>(cur, it, passes);
  uint32_t ent_nx = entry_of(nx.ok ? nx : cur);
  int stg_bat = -1, stg_blk = 0;

  for (;;) {
    // K^idx of the chunk's block (shared by the groups of a sequence), all
    // loads in flight before the LDS stores; the wave is alone in its
    // workgroup and its LDS operations complete in order.
    const int bat = cur.D.seq / H_sel;
    if (bat != stg_bat || cur.D.blk != stg_blk) {
      stg_bat = bat;
      stg_blk = cur.D.blk;
      const int64_t key0 = static_cast<int64_t>(cur.D.blk) * kBk;
      const int nvalid = static_cast<int>(min<int64_t>(kBk, N - key0));
      const uint16_t* kb = k_idx + (static_cast<int64_t>(bat) * N + key0) * DIDX;
      u32x4 w[kBk * KC / 64];
#pragma unroll
      for (int j = 0; j < kBk * KC / 64; ++j) {
        const int x = lane + 64 * j, key = x / KC, c = x % KC;
        w[j] = *reinterpret_cast<const u32x4*>(kb + min(key, nvalid - 1) * DIDX + 8 * c);
      }
#pragma unroll
      for (int j = 0; j < kBk * KC / 64; ++j) {
        const int x = lane + 64 * j, key = x / KC, c = x % KC;
        *reinterpret_cast<u32x4*>(ki_lds + key * kStr + 16 * c) = key < nvalid ? w[j] : u32x4{0u, 0u, 0u, 0u};
      }
    }

    // ---- the next chunk's Q^idx rows, the entry words of the one after
    const Chunk nxv = nx.ok ? nx : cur;
    bf16x8 q_nx[KSI];
    q_of(nxv, ent_nx, q_nx);
    const Chunk nx2 = nx.ok ? next_chunk<32, true>(nx, it, passes) : nx;
    const uint32_t ent_nx2 = entry_of(nx2.ok ? nx2 : nxv);

    // ---- this chunk
    const int e = cur.cb + n;
    const EntryRef er = entry_ref(ent_cur, cur.D.seq, kslots, q_begin, q_count);
    f32x16 z[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      z[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks)
        z[mt] = mfma32x32x16(lds_frag(ki_lds + (32 * mt + n) * kStr + 32 * ks + 16 * h), q_cur[ks], z[mt]);
    }
    // keys 32 mt + acc_row(e, h) of the block; hide those past the query
    const int lim = er.i - cur.D.blk * kBk;
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int el = 0; el < 16; ++el)
        if (32 * mt + acc_row(el, h) <= lim) m = fmaxf(m, z[mt][el]);
    m = halves_max(m);
    float l = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int el = 0; el < 16; ++el)
        if (32 * mt + acc_row(el, h) <= lim) l += __builtin_amdgcn_exp2f((z[mt][el] - m) * idx_scale_log2);
    l = halves_sum(l);
    if (h == 0 && e < cur.D.cnt) lsei_part[er.slot] = m * idx_scale_log2 + __builtin_amdgcn_logf(l);

    if (!nx.ok) break;
    cur = nx;
    nx = nx2;
    ent_cur = ent_nx;
    ent_nx = ent_nx2;
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks) q_cur[ks] = q_nx[ks];
  }
}

// Merge of the partial proxy LSEs of one (group, query) over its valid slots
// (log2 units).  The slot loop is unrolled at compile time (KMAX >= k): every
// id and value is requested before the max and the sum, which then run over
// the slots in order.
template <int KMAX>
__global__ __launch_bounds__(256) void proxy_lse_merge_kernel(const int32_t* __restrict__ block_idx,
                                                              const float* __restrict__ lsei_part, int k,
                                                              int64_t q_begin, int64_t q_count, int64_t rows,
                                                              float* __restrict__ lsei2) {
  const int64_t f = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (f >= rows) return;
  const int64_t L = (q_begin + f % q_count) / kBk;
  int b[KMAX];
  float v[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) b[s] = s < k ? block_idx[f * k + s] : -1;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) v[s] = s < k ? lsei_part[f * k + s] : 0.f;
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int s = 0; s < KMAX; ++s)
    if (b[s] >= 0 && b[s] <= L) m = fmaxf(m, v[s]);
  float l = 0.f;
#pragma unroll
  for (int s = 0; s < KMAX; ++s)
    if (b[s] >= 0 && b[s] <= L) l += __builtin_amdgcn_exp2f(v[s] - m);
  lsei2[f] = m + __builtin_amdgcn_logf(l);
}

// D = rowsum(dO * O) per (query, head), fp32: 16 threads per row.  blockIdx.y
// is the batch element, whose rows of the range (q_count queries x H_q heads)
// are contiguous; each 16-lane group takes kPrepRows rows a grid width apart,
// with all of its loads in flight before the sums.
constexpr int kPrepRows = 4;

__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ dout,
                                                       const uint16_t* __restrict__ o, int64_t N, int H_q,
                                                       int64_t q_begin, int64_t rows, float* __restrict__ dlt) {
  const int64_t base = (static_cast<int64_t>(blockIdx.y) * N + q_begin) * H_q;
  const int64_t grp = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 4;
  const int64_t ngrp = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 4);
  const int c = static_cast<int>(threadIdx.x & 15);
  u32x4 a[kPrepRows], b[kPrepRows];
#pragma unroll
  for (int j = 0; j < kPrepRows; ++j) {
    const int64_t row = grp + j * ngrp;
    const int64_t off = (base + (row < rows ? row : rows - 1)) * kDh + 8 * c;
    a[j] = *reinterpret_cast<const u32x4*>(dout + off);
    b[j] = *reinterpret_cast<const u32x4*>(o + off);
  }
#pragma unroll
  for (int j = 0; j < kPrepRows; ++j) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s += __uint_as_float(a[j][e] << 16) * __uint_as_float(b[j][e] << 16);
      s += __uint_as_float(a[j][e] & 0xFFFF0000u) * __uint_as_float(b[j][e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1) s += __shfl_xor(s, w, 16);
    const int64_t row = grp + j * ngrp;
    if (row < rows && c == 0) dlt[base + row] = s;
  }
}

// Sum of the per-slot partials of one (group, query): dQ of its G heads,
// dq_idx and the KL value, over the slots with a valid block.  A pure
// streaming kernel like the forward's combine: the slot loop is unrolled at
// compile time (KMAX >= k), so a thread's loads of all valid slots are in
// flight together, and the sums still run over the slots in order.  Each XCD
// streams one contiguous share of the partial buffer.  Partials are read once
// and the outputs written once, in whole lines: loads and stores are
// non-temporal.
constexpr int kRedThreads = 320;

template <int G, int KMAX>
__global__ __launch_bounds__(kRedThreads) void bwd_reduce_kernel(
    const int32_t* __restrict__ block_idx, const uint16_t* __restrict__ dq_part,
    const float* __restrict__ dqi_part, const float* __restrict__ kl_part, int64_t N, int H_sel, int k,
    int d_idx, int64_t q_begin, int64_t q_count, int64_t rows_total, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dq_idx, float* __restrict__ kl) {
  // Workgroups are dealt round-robin to the kXcds XCDs; the grid is a
  // multiple of kXcds and XCD x takes the x-th contiguous share of the rows.
  const int64_t per = gridDim.x / kXcds;
  const int64_t f = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;  // seq * q_count + query row
  if (f >= rows_total) return;
  const int64_t seq = f / q_count, qrow = f % q_count, i = q_begin + qrow;
  const int64_t bat = seq / H_sel;
  const int r = static_cast<int>(seq % H_sel);
  const int64_t L = i / kBk;
  const int t = threadIdx.x;
  const int32_t* sel = block_idx + f * k;
  bool ok[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    const int b = s < k ? sel[s] : -1;
    ok[s] = b >= 0 && b <= L;
  }
  if (t < 16 * G) {
    const int g = t >> 4, c = t & 15;
    u32x4 w[KMAX];
#pragma unroll
    for (int s = 0; s < KMAX; ++s)
      w[s] = ok[s] ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dq_part + ((f * k + s) * G + g) * kDh + 8 * c))
                   : u32x4{0u, 0u, 0u, 0u};
    float acc[8] = {};
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      if (!ok[s]) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(w[s][j] << 16);
        acc[2 * j + 1] += __uint_as_float(w[s][j] & 0xFFFF0000u);
      }
    }
    __builtin_nontemporal_store(
        u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
              pack_bf16x2(acc[6], acc[7])},
        reinterpret_cast<u32x4*>(dq + ((bat * N + i) * (H_sel * G) + r * G + g) * kDh + 8 * c));
  } else if (dq_idx && t < 16 * G + d_idx / 4) {
    const int c = t - 16 * G;
    f32x4 w[KMAX];
#pragma unroll
    for (int s = 0; s < KMAX; ++s)
      w[s] = ok[s] ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dqi_part + (f * k + s) * d_idx + 4 * c)) : f32x4{};
    float acc[4] = {};
#pragma unroll
    for (int s = 0; s < KMAX; ++s) {
      if (!ok[s]) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += w[s][j];
    }
    __builtin_nontemporal_store(u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])},
        reinterpret_cast<u32x2*>(dq_idx + ((bat * N + i) * H_sel + r) * d_idx + 4 * c));
  } else if (kl && t == 16 * G + d_idx / 4) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (ok[j]) s += kl_part[f * k + j];
    kl[seq * N + i] = s;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; x < n;
       x += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[x] = 0.f;
}

// fp32 accumulators -> bf16 (round to nearest even), 4 values per thread.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                      int64_t n4) {
  for (int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; x < n4;
       x += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(src + 4 * x);
    *reinterpret_cast<u32x2*>(dst + 4 * x) = u32x2{pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3])};
  }
}

// Grid-stride kernels: at most 65536 workgroups.
unsigned grid_of(int64_t n, int per = 256) {
  int64_t g = (n + per - 1) / per;
  if (g > 65536) g = 65536;
  return static_cast<unsigned>(g < 1 ? 1 : g);
}

// One thread per item: every item gets a thread.
unsigned grid_exact(int64_t n, int per = 256) {
  const int64_t g = (n + per - 1) / per;
  return static_cast<unsigned>(g < 1 ? 1 : g);
}

int cus_of_device() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

}  // namespace

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_of(n)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(to_bf16_kernel, dim3(grid_of(n / 4)), dim3(256), 0, stream, src, dst, n / 4);
  return hipGetLastError();
}

hipError_t launch_backward_chunk(const BwdArgs& a, hipStream_t stream) {
  const SchedLayout s = sched_layout(a.batch, a.H_sel, a.G, a.k, a.q_begin, a.q_count, kBk);
  const int64_t seqs = static_cast<int64_t>(a.batch) * a.H_sel;
  const int H_q = a.H_sel * a.G;
  const int nseqs = static_cast<int>(seqs);
  const int32_t* segp = a.sched + s.off_segp;
  const PassDesc* passes = reinterpret_cast<const PassDesc*>(a.sched + s.off_pass);
  const int64_t min_passes = (seqs * a.q_count * a.k + s.EPP - 1) / s.EPP;
  auto clamp_grid = [&](int64_t g) { return static_cast<unsigned>(g < min_passes ? (g < 1 ? 1 : g) : min_passes); };
  const float scale_log2 = a.scale * kLog2e;
  // the spare partial row past this range's slots (rows that are padding write there)
  const int64_t dummy_slot = seqs * a.q_count * a.k;

  // D = rowsum(dO * O) of the range's rows
  {
    const int64_t rows = a.q_count * H_q;  // per batch element
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(grid_exact(rows * 16, 256 * kPrepRows), a.batch), dim3(256), 0, stream,
                       a.dout, a.o, a.N, H_q, a.q_begin, rows, a.dlt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  const float isl2 = a.idx_scale * kLog2e;
  if (a.index) {
    const unsigned lgrid = clamp_grid(static_cast<int64_t>(cus_of_device()) * kLseWgPerCu);
    auto lk = a.d_idx == 64 ? proxy_lse_kernel<64> : proxy_lse_kernel<128>;
    hipLaunchKernelGGL(lk, dim3(lgrid), dim3(64), 0, stream, a.q_idx, a.k_idx, a.N, a.H_sel, a.k, isl2,
                       a.entries, segp, passes, static_cast<int>(s.B_c), nseqs, static_cast<int>(a.q_begin),
                       static_cast<int>(a.q_count), a.lsei_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = seqs * a.q_count;
    auto mk = a.k <= 4 ? proxy_lse_merge_kernel<4>
              : a.k <= 8 ? proxy_lse_merge_kernel<8>
              : a.k <= 16 ? proxy_lse_merge_kernel<16> : proxy_lse_merge_kernel<32>;
    hipLaunchKernelGGL(mk, dim3(grid_exact(rows)), dim3(256), 0, stream, a.block_idx, a.lsei_part, a.k,
                       a.q_begin, a.q_count, rows, a.lsei2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  {
    const unsigned grid = clamp_grid(cus_of_device());
#define MSA_BWD_MAIN(GG)                                                                                        \
  case GG:                                                                                                      \
    if (a.index)                                                                                                \
      hipLaunchKernelGGL((bwd_main_kernel<GG, true>), dim3(grid), dim3(kMT), 0, stream, a.q, a.k_ptr, a.v,     \
                         a.dout, a.lse, a.dlt, a.N, a.H_sel, a.kv_shift, a.k, a.scale, scale_log2, a.entries,   \
                         segp, passes, static_cast<int>(s.B_c), nseqs, static_cast<int>(a.q_begin),            \
                         static_cast<int>(a.q_count), dummy_slot, a.dq_part, a.dk_acc, a.dv_acc, a.tch);        \
    else                                                                                                        \
      hipLaunchKernelGGL((bwd_main_kernel<GG, false>), dim3(grid), dim3(kMT), 0, stream, a.q, a.k_ptr, a.v,    \
                         a.dout, a.lse, a.dlt, a.N, a.H_sel, a.kv_shift, a.k, a.scale, scale_log2, a.entries,   \
                         segp, passes, static_cast<int>(s.B_c), nseqs, static_cast<int>(a.q_begin),            \
                         static_cast<int>(a.q_count), dummy_slot, a.dq_part, a.dk_acc, a.dv_acc, a.tch);        \
    break;
    switch (a.G) {
      MSA_BWD_MAIN(1)
      MSA_BWD_MAIN(2)
      MSA_BWD_MAIN(4)
      MSA_BWD_MAIN(8)
      MSA_BWD_MAIN(16)
      default:
        return hipErrorInvalidValue;
    }
#undef MSA_BWD_MAIN
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  if (a.index) {
    const unsigned grid = clamp_grid(cus_of_device());
#define MSA_BWD_IDX(GG, DD)                                                                                    \
  hipLaunchKernelGGL((bwd_idx_kernel<GG, DD>), dim3(grid), dim3(kBT), 0, stream, a.q_idx, a.k_idx, a.lsei2,     \
                     a.tch, a.N, a.H_sel, a.k, isl2, a.kl_weight * a.idx_scale, a.entries, segp, passes,        \
                     static_cast<int>(s.B_c), nseqs, static_cast<int>(a.q_begin), static_cast<int>(a.q_count), \
                     dummy_slot, a.dqi_part, a.kl_part, a.dki_acc)
#define MSA_BWD_IDX_G(GG)          \
  case GG:                         \
    if (a.d_idx == 64)             \
      MSA_BWD_IDX(GG, 64);         \
    else                           \
      MSA_BWD_IDX(GG, 128);        \
    break;
    switch (a.G) {
      MSA_BWD_IDX_G(1)
      MSA_BWD_IDX_G(2)
      MSA_BWD_IDX_G(4)
      MSA_BWD_IDX_G(8)
      MSA_BWD_IDX_G(16)
      default:
        return hipErrorInvalidValue;
    }
#undef MSA_BWD_IDX_G
#undef MSA_BWD_IDX
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  {
    const int64_t rows = seqs * a.q_count;
    const int64_t grid = (rows + kXcds - 1) / kXcds * kXcds;  // see the kernel
    auto launch = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kRedThreads), 0, stream, a.block_idx,
                         a.dq_part, a.dqi_part, a.kl_part, a.N, a.H_sel, a.k, a.d_idx, a.q_begin, a.q_count,
                         rows, a.dq, a.index ? a.dq_idx : nullptr, a.index ? a.kl : nullptr);
    };
#define MSA_BWD_RED(GG)                                            \
  case GG:                                                         \
    if (a.k <= 4) launch(bwd_reduce_kernel<GG, 4>);                \
    else if (a.k <= 8) launch(bwd_reduce_kernel<GG, 8>);           \
    else if (a.k <= 16) launch(bwd_reduce_kernel<GG, 16>);         \
    else launch(bwd_reduce_kernel<GG, 32>);                        \
    break;
    switch (a.G) {
      MSA_BWD_RED(1)
      MSA_BWD_RED(2)
      MSA_BWD_RED(4)
      MSA_BWD_RED(8)
      MSA_BWD_RED(16)
      default: return hipErrorInvalidValue;
    }
#undef MSA_BWD_RED
    return hipGetLastError();
  }
}

}  // namespace msa
