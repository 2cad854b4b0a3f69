// Block-index inversion and work-list construction for the KV-outer pass.
//
// The selection B[seq, query, slot] -> block (seq = batch * H_kv + group) is
// inverted into B*[seq, block] -> the queries that selected it ("Flash-MSA",
// Backward; "MiniMax Sparse Attention (MSA)", Deep Dive > KV-Outer Sparse
// Attention, step 1: reverse index).  The result is a CSR whose entries are
// ascending in query inside every bin, i.e. a stable counting sort, computed
// deterministically without global atomics:
//
//  1. count:    one workgroup per (seq, 64-row query tile) builds, in LDS, a
//               64-bit mask per block of which tile rows selected it (LDS
//               atomic OR is order independent) and writes the popcounts,
//               cnt[seq][tile][block].
//  2. colscan:  exclusive prefix of cnt down each block column (over tiles),
//               in place; column totals tot[seq][block].
//  3. binscan:  one workgroup scans the totals over all (seq, block) bins into
//               absolute CSR offsets, then the pass counts ceil(len / EPP),
//               EPP = kPassRows / G, of the bins into the first pass of every
//               bin.
//  4. scatter:  the count workgroup's masks are rebuilt and every entry lands at
//               offset[bin] + colprefix[tile][bin] + popcount(mask below row).
//  5. passes:   the work list: one descriptor per pass of EPP consecutive
//               entries of a bin (the last one partial).
//
// Pre-scheduled chunking ("MiniMax Sparse Attention (MSA)", KV-Outer Sparse
// Attention, step 5): the attention kernel takes the sequences one after
// another and splits each one's passes into one contiguous, equal share per
// workgroup, so a block that many queries picked is spread over as many
// workgroups as its share of the work asks for, a workgroup restages K/V only
// when its passes move to the next bin, and every (query, slot) keeps its own
// preassigned output slot.
#include "msa_internal.h"

namespace msa {

SchedLayout sched_layout(int batch, int H_kv, int G, int k, int64_t q_begin, int64_t q_count, int bk) {
  SchedLayout s{};
  auto al = [](int64_t w) { return (w + 63) / 64 * 64; };  // 256-byte alignment
  const int64_t nseq = static_cast<int64_t>(batch) * H_kv;
  s.B_c = (q_begin + q_count + bk - 1) / bk;
  s.T64 = (q_count + 63) / 64;
  s.nbins = nseq * s.B_c;
  s.EPP = kPassRows / (G > 0 ? G : 1);
  // sum_g ceil(t_g / EPP) <= (sum_g t_g) / EPP + (non-empty bins)
  s.max_passes = (nseq * q_count * k + s.EPP - 1) / s.EPP + s.nbins;
  int64_t w = kHdrWords;
  s.off_tot = w;
  w = al(w + s.nbins);
  s.off_bad = w;
  w = al(w + nseq * s.T64);
  s.off_segp = w;
  w = al(w + s.nbins + 1);
  s.off_pass = w;
  w = al(w + s.max_passes * 4);
  s.off_cnt = w;
  w = al(w + nseq * s.T64 * s.B_c);
  s.words = w;
  return s;
}

namespace {

constexpr int kInvThreads = 256;

// Build the LDS row masks of one (seq, tile).  Returns the number of bins used.
__device__ __forceinline__ int build_masks(const int32_t* __restrict__ rows, int k, int64_t q_begin,
                                           int64_t q0, int nrows, unsigned long long* mask,
                                           int* bad, int bk) {
  const int tmax = static_cast<int>((q_begin + q0 + nrows - 1) / bk);
  const int nb = tmax + 1;
  for (int b = threadIdx.x; b < nb; b += blockDim.x) mask[b] = 0ull;
  __syncthreads();
  int nbad = 0;
  for (int e = threadIdx.x; e < nrows * k; e += blockDim.x) {
    const int row = e / k;
    const int v = rows[e];
    const int L = static_cast<int>((q_begin + q0 + row) / bk);
    if (v >= 0 && v <= L)
      atomicOr(&mask[v], 1ull << row);
    else if (v != -1)
      ++nbad;
  }
  *bad = nbad;
  __syncthreads();
  return nb;
}

__global__ __launch_bounds__(kInvThreads) void inv_count_kernel(
    const int32_t* __restrict__ block_idx, int k, int64_t q_begin, int64_t q_count, int64_t B_c,
    int64_t T64, int32_t* __restrict__ cnt, int32_t* __restrict__ bad_out, int bk) {
  extern __shared__ unsigned long long mask[];
  __shared__ int bad_sum;
  const int64_t tq = blockIdx.x, seq = blockIdx.y;
  const int64_t q0 = tq * 64;
  const int nrows = static_cast<int>(min<int64_t>(64, q_count - q0));
  if (threadIdx.x == 0) bad_sum = 0;
  int nbad;
  const int nb = build_masks(block_idx + (seq * q_count + q0) * k, k, q_begin, q0, nrows, mask, &nbad, bk);
  if (nbad) atomicAdd(&bad_sum, nbad);
  int32_t* out = cnt + (seq * T64 + tq) * B_c;
  for (int64_t b = threadIdx.x; b < B_c; b += blockDim.x)
    out[b] = b < nb ? __popcll(mask[b]) : 0;
  __syncthreads();
  if (threadIdx.x == 0) bad_out[seq * T64 + tq] = bad_sum;
}

// 16 waves per workgroup walk the tiles of 64 block columns.
constexpr int kScanWaves = 16;

__global__ __launch_bounds__(kScanWaves * 64) void inv_colscan_kernel(
    int32_t* __restrict__ cnt, int64_t B_c, int64_t T64, int32_t* __restrict__ tot) {
  __shared__ int part[kScanWaves][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t seq = blockIdx.y;
  const int64_t col = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const int64_t per = (T64 + kScanWaves - 1) / kScanWaves;
  const int64_t t0 = min<int64_t>(T64, wave * per), t1 = min<int64_t>(T64, t0 + per);
  int32_t* base = cnt + seq * T64 * B_c + col;
  int s = 0;
  if (col < B_c)
    for (int64_t t = t0; t < t1; ++t) s += base[t * B_c];
  part[wave][lane] = s;
  __syncthreads();
  int run = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kScanWaves; ++w) {
    run += w < wave ? part[w][lane] : 0;
    all += part[w][lane];
  }
  if (col < B_c) {
    for (int64_t t = t0; t < t1; ++t) {
      const int c = base[t * B_c];
      base[t * B_c] = run;
      run += c;
    }
    if (wave == 0) tot[seq * B_c + col] = all;
  }
}

// Single workgroup.  Part 1: exclusive scan of the entry counts over all bins
// (CSR offsets) and the sum of the bad-id counts.  Part 2: exclusive scan of
// the pass counts of the bins (seq, block).  Both read only what
// earlier kernels wrote.
constexpr int kBinThreads = 1024;

__device__ __forceinline__ void block_exclusive_scan(int* se, int& e) {
  const int t = threadIdx.x;
  se[t] = e;
  __syncthreads();
  // Hillis-Steele inclusive scan over the per-thread sums.
  for (int d = 1; d < kBinThreads; d <<= 1) {
    const int a = t >= d ? se[t - d] : 0;
    __syncthreads();
    se[t] += a;
    __syncthreads();
  }
  e = se[t] - e;  // exclusive start of this thread's range
}

__global__ __launch_bounds__(kBinThreads) void inv_binscan_kernel(
    const int32_t* __restrict__ tot, int64_t nbins, int64_t B_c,
    int epp, const int32_t* __restrict__ bad,
    int64_t nbad_slots, int32_t* __restrict__ blk_offsets, int32_t* __restrict__ segp,
    int32_t* __restrict__ hdr) {
  __shared__ int se[kBinThreads];
  __shared__ int sbad;
  const int t = threadIdx.x;
  if (t == 0) sbad = 0;

  // ---- part 1: CSR offsets
  {
    const int64_t per = (nbins + kBinThreads - 1) / kBinThreads;
    const int64_t b0 = min<int64_t>(nbins, t * per), b1 = min<int64_t>(nbins, b0 + per);
    int e = 0;
    for (int64_t b = b0; b < b1; ++b) e += tot[b];
    block_exclusive_scan(se, e);
    for (int64_t b = b0; b < b1; ++b) {
      const int64_t seq = b / B_c, blk = b % B_c;
      blk_offsets[seq * (B_c + 1) + blk] = e;
      e += tot[b];
      if (blk == B_c - 1) blk_offsets[seq * (B_c + 1) + B_c] = e;
    }
    if (t == kBinThreads - 1) hdr[kHdrEntries] = e;
    int nb = 0;
    for (int64_t j = t; j < nbad_slots; j += kBinThreads) nb += bad[j];
    if (nb) atomicAdd(&sbad, nb);
  }
  __syncthreads();

  // ---- part 2: first pass of every bin
  {
    const int64_t per = (nbins + kBinThreads - 1) / kBinThreads;
    const int64_t s0 = min<int64_t>(nbins, t * per), s1 = min<int64_t>(nbins, s0 + per);
    int np = 0;
    for (int64_t g = s0; g < s1; ++g) np += (tot[g] + epp - 1) / epp;
    block_exclusive_scan(se, np);
    for (int64_t g = s0; g < s1; ++g) {
      segp[g] = np;
      np += (tot[g] + epp - 1) / epp;
    }
    if (t == kBinThreads - 1) {
      segp[nbins] = np;
      hdr[kHdrPasses] = np;
    }
  }
  if (t == 0) hdr[kHdrBad] = sbad;
}

// Pass descriptors: workgroups stride over the bins, threads over a bin's
// passes.
__global__ __launch_bounds__(kInvThreads) void inv_passes_kernel(
    const int32_t* __restrict__ tot, const int32_t* __restrict__ segp,
    const int32_t* __restrict__ blk_offsets, int64_t B_c, int64_t nbins, int epp,
    PassDesc* __restrict__ passes) {
  for (int64_t g = blockIdx.x; g < nbins; g += gridDim.x) {
    const int p0 = segp[g], np = segp[g + 1] - p0;
    if (np == 0) continue;
    const int64_t blk = g % B_c, seq = g / B_c;
    const int len = tot[g];
    const int off = blk_offsets[seq * (B_c + 1) + blk];
    for (int j = threadIdx.x; j < np; j += blockDim.x) {
      PassDesc d;
      d.start = off + j * epp;
      d.cnt = min(epp, len - j * epp);
      d.seq = static_cast<int32_t>(seq);
      d.blk = static_cast<int32_t>(blk);
      passes[p0 + j] = d;
    }
  }
}

__global__ __launch_bounds__(kInvThreads) void inv_scatter_kernel(
    const int32_t* __restrict__ block_idx, int k, int64_t q_begin, int64_t q_count, int64_t B_c,
    int64_t T64, const int32_t* __restrict__ colpre, const int32_t* __restrict__ blk_offsets,
    int32_t* __restrict__ entries, int bk) {
  extern __shared__ unsigned long long mask[];
  const int64_t tq = blockIdx.x, seq = blockIdx.y;
  const int64_t q0 = tq * 64;
  const int nrows = static_cast<int>(min<int64_t>(64, q_count - q0));
  const int32_t* rows = block_idx + (seq * q_count + q0) * k;
  int nbad;
  build_masks(rows, k, q_begin, q0, nrows, mask, &nbad, bk);
  const int32_t* pre = colpre + (seq * T64 + tq) * B_c;
  const int32_t* off = blk_offsets + seq * (B_c + 1);
  for (int e = threadIdx.x; e < nrows * k; e += blockDim.x) {
    const int row = e / k, slot = e % k;
    const int v = rows[e];
    const int L = static_cast<int>((q_begin + q0 + row) / bk);
    if (v < 0 || v > L) continue;
    const int rank = __popcll(mask[v] & ((1ull << row) - 1ull));
    entries[off[v] + pre[v] + rank] = static_cast<int32_t>((q0 + row) * k + slot);
  }
}

bool g_lds_attr_set = false;

}  // namespace

hipError_t launch_invert(const int32_t* block_idx, int batch, int H_kv, int G, int k,
                         int64_t q_begin, int64_t q_count, int32_t* blk_offsets,
                         int32_t* blk_entries, int32_t* sched, hipStream_t stream, int bk) {
  const SchedLayout s = sched_layout(batch, H_kv, G, k, q_begin, q_count, bk);
  const int64_t nseq = static_cast<int64_t>(batch) * H_kv;
  const size_t lds = static_cast<size_t>(s.B_c) * sizeof(unsigned long long);
  if (!g_lds_attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(inv_count_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(inv_scatter_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 1024);
    if (e != hipSuccess) return e;
    g_lds_attr_set = true;
  }
  int32_t* hdr = sched;
  int32_t* tot = sched + s.off_tot;
  int32_t* bad = sched + s.off_bad;
  int32_t* cnt = sched + s.off_cnt;
  int32_t* segp = sched + s.off_segp;
  const int epp = static_cast<int>(s.EPP);
  const dim3 tiles(static_cast<unsigned>(s.T64), static_cast<unsigned>(nseq));
  hipLaunchKernelGGL(inv_count_kernel, tiles, dim3(kInvThreads), lds, stream, block_idx, k, q_begin,
                     q_count, s.B_c, s.T64, cnt, bad, bk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(inv_colscan_kernel, dim3(static_cast<unsigned>((s.B_c + 63) / 64), nseq),
                     dim3(kScanWaves * 64), 0, stream, cnt, s.B_c, s.T64, tot);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(inv_binscan_kernel, dim3(1), dim3(kBinThreads), 0, stream, tot, s.nbins,
                     s.B_c, epp, bad, nseq * s.T64, blk_offsets, segp, hdr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(inv_scatter_kernel, tiles, dim3(kInvThreads), lds, stream, block_idx, k, q_begin,
                     q_count, s.B_c, s.T64, cnt, blk_offsets, blk_entries, bk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t pgrid = s.nbins < 8192 ? s.nbins : 8192;
  hipLaunchKernelGGL(inv_passes_kernel, dim3(static_cast<unsigned>(pgrid > 0 ? pgrid : 1)),
                     dim3(kInvThreads), 0, stream, tot, segp, blk_offsets, s.B_c, s.nbins, epp,
                     reinterpret_cast<PassDesc*>(sched + s.off_pass));
  return hipGetLastError();
}

}  // namespace msa
