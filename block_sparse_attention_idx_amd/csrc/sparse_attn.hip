// KV-outer block-sparse attention (main branch of MSA).
//
// What is computed ("MiniMax Sparse Attention", sec. 2.2 and 4.2;
// "MiniMax Sparse Attention (MSA)", Deep Dive > KV-Outer Sparse Attention):
// for every work item -- a (sequence, group r, key block b) bin of the
// inverted index, cut into pieces of at most queries_per_item(G) queries --
// the K and V rows of block b (head r) are staged in LDS once, and every
// (query i, head g of group r) that selected the block gets the block's
// partial softmax attention over its causally visible tokens:
//     Obar = sum_j softmax(s)_j V_j,  lse = ln sum_j exp(s_j),
//     s_j = scale * Q[i, rG+g] . K[j, r],  j in block b, j <= i.
// The causal mask only bites when b is the query's own block.  One (Obar, lse)
// pair per (query, slot, head) goes to the partial buffers, merged afterwards
// by the combine kernel.
//
// gfx950 design:
//  * 4 waves per workgroup, one 128-row MFMA tile at a time: 128 / G queries x
//    G heads (a query's G heads are contiguous in Q, 256 B each); each wave
//    owns 32 rows.  K (row-major) and V (transposed) live in XOR-swizzled LDS,
//    64 KB per workgroup, two workgroups per CU.
//  * S^T = K_b * Q^T with v_mfma_f32_32x32x16_bf16 (keys on the row dimension).
//    The accumulator layout then gives every lane 64 of the 128 keys of one
//    (query, head) row, so the row max and row sum need one half-wave exchange,
//    and the probabilities feed O^T = V^T * P^T directly as the MFMA B operand
//    with no shuffle: the reduction slots of each P^T step are exactly the keys
//    that lane already holds.  The V^T operand rows are permuted so that every
//    lane ends up with 64 contiguous output dimensions of its row, stored as
//    eight 16-byte writes.
//  * Softmax in base 2 (v_exp_f32) with the scale folded in; fp8 (OCP e4m3)
//    inputs are widened exactly to bf16 while loading and the per-tensor
//    scales are folded into the softmax scale and the output scale.
//  * Work items are mapped XCD-aware: consecutive items (same K/V block) run on
//    the same XCD, so the block is fetched into one L2 instead of eight.
#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kAttnThreads = 256;

__device__ __forceinline__ int k_lds_off(int key, int c) {  // 16-byte chunk c of key row
  return key * 256 + ((c ^ (key & 15)) << 4);
}

__device__ __forceinline__ int vt_swz(int d) {
  return (d & 7) | ((d >> 3) & 8) | ((d << 1) & 16);
}

__device__ __forceinline__ int vt_lds_off(int d, int kc) {  // 8-byte chunk kc (4 keys) of row d
  return d * 256 + ((kc ^ vt_swz(d)) << 3);
}

__device__ __forceinline__ uint32_t half_of(const u32x4& w, int dd) {
  const uint32_t x = w[dd >> 1];
  return (dd & 1) ? (x >> 16) : (x & 0xFFFFu);
}

template <int G, bool FP8>
__global__ __launch_bounds__(kAttnThreads, 2) void sparse_attn_kernel(
    const void* __restrict__ qp, const void* __restrict__ kp, const void* __restrict__ vp,
    int64_t N, int H_kv, int kslots, float scale_log2, float out_scale,
    const int32_t* __restrict__ blk_offsets, const int32_t* __restrict__ entries,
    const int32_t* __restrict__ items, const int32_t* __restrict__ hdr, int64_t nbins, int64_t B_c,
    int64_t q_begin, int64_t q_count, uint16_t* __restrict__ o_part, float* __restrict__ lse_part) {
  constexpr int QT = 128 / G;  // queries per 128-row tile
  constexpr int QPI = queries_per_item(G);
  constexpr int EB = FP8 ? 1 : 2;  // bytes per Q/K/V element
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kBk * kDh * 2];
  __shared__ __attribute__((aligned(16))) uint8_t vt_lds[kBk * kDh * 2];
  __shared__ int64_t s_item[4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int H_q = H_kv * G;

  if (tid == 0) {
    const int64_t n_items = hdr[kHdrItems];
    const int64_t per = (n_items + kXcds - 1) / kXcds;
    const int64_t x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
    const int64_t logical = x * per + j;
    int64_t ok = 0, bin = 0, e0 = 0, e1 = 0;
    if (j < per && logical < n_items) {
      int64_t lo = 0, hi = nbins - 1;  // largest bin with items[bin] <= logical
      while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        if (items[mid] <= logical) lo = mid; else hi = mid - 1;
      }
      bin = lo;
      const int64_t seq = bin / B_c, blk = bin % B_c;
      const int64_t beg = blk_offsets[seq * (B_c + 1) + blk];
      const int64_t end = blk_offsets[seq * (B_c + 1) + blk + 1];
      e0 = beg + (logical - items[bin]) * QPI;
      e1 = min(end, e0 + QPI);
      ok = e1 > e0;
    }
    s_item[0] = ok;
    s_item[1] = bin;
    s_item[2] = e0;
    s_item[3] = e1;
  }
  __syncthreads();
  if (!s_item[0]) return;
  const int64_t bin = s_item[1], e0 = s_item[2];
  const int n_ent = static_cast<int>(s_item[3] - e0);
  const int64_t seq = bin / B_c, blk = bin % B_c;
  const int64_t bat = seq / H_kv;
  const int r = static_cast<int>(seq % H_kv);
  const int64_t key0 = blk * kBk;

  // ---- stage K (row-major) and V (transposed) of block blk, head r
  {
    const uint8_t* kb = static_cast<const uint8_t*>(kp) + ((bat * N + key0) * H_kv + r) * kDh * EB;
    const uint8_t* vb = static_cast<const uint8_t*>(vp) + ((bat * N + key0) * H_kv + r) * kDh * EB;
    const int64_t rstride = static_cast<int64_t>(H_kv) * kDh * EB;  // bytes between token rows
    if constexpr (!FP8) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int cid = tid + p * kAttnThreads;
        const int key = cid >> 4, c = cid & 15;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key0 + key < N) w = *reinterpret_cast<const u32x4*>(kb + key * rstride + c * 16);
        *reinterpret_cast<u32x4*>(k_lds + k_lds_off(key, c)) = w;
      }
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int cid = tid + p * kAttnThreads;
        const int key = cid >> 3, cc = cid & 7;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (key0 + key < N) w = *reinterpret_cast<const u32x4*>(kb + key * rstride + cc * 16);
        const u32x2 a = e4m3x4_to_bf16x4(w[0]), b = e4m3x4_to_bf16x4(w[1]);
        const u32x2 c2 = e4m3x4_to_bf16x4(w[2]), d2 = e4m3x4_to_bf16x4(w[3]);
        *reinterpret_cast<u32x4*>(k_lds + k_lds_off(key, 2 * cc)) = u32x4{a[0], a[1], b[0], b[1]};
        *reinterpret_cast<u32x4*>(k_lds + k_lds_off(key, 2 * cc + 1)) = u32x4{c2[0], c2[1], d2[0], d2[1]};
      }
    }
    const int kc = tid & 31;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int dg = (tid >> 5) + 8 * p;  // 8 output dims d = 8 dg .. 8 dg + 7
      u32x4 row[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = 4 * kc + j;
        row[j] = u32x4{0u, 0u, 0u, 0u};
        if (key0 + key < N) {
          if constexpr (!FP8) {
            row[j] = *reinterpret_cast<const u32x4*>(vb + key * rstride + dg * 16);
          } else {
            const u32x2 w = *reinterpret_cast<const u32x2*>(vb + key * rstride + dg * 8);
            const u32x2 a = e4m3x4_to_bf16x4(w[0]), b = e4m3x4_to_bf16x4(w[1]);
            row[j] = u32x4{a[0], a[1], b[0], b[1]};
          }
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
  }
  __syncthreads();

  // Output dimension of V^T operand row n in d-tile nt (see the store below).
  const int dsel = 64 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);
  const int rho = 32 * wave + n;  // this lane's row in the 128-row tile
  const int qs = rho / G, g = rho % G;

  for (int t0 = 0; t0 < n_ent; t0 += QT) {
    // The LDS tiles do not change across row tiles; an opaque zero added to
    // their addresses keeps the compiler from hoisting all 96 fragment reads
    // (256 VGPRs) out of the loop.
    int salt = 0;
    asm volatile("" : "+s"(salt));
    const uint8_t* kl = k_lds + salt;
    const uint8_t* vl = vt_lds + salt;
    const int e = t0 + qs;
    const bool row_ok = e < n_ent;
    const int ent = entries[e0 + (row_ok ? e : n_ent - 1)];
    const int64_t qrow = ent / kslots;
    const int slot = ent % kslots;
    const int64_t i = q_begin + qrow;

    // ---- Q fragments (B operand of S^T): row (i, rG+g), dims 16ks + 8h .. +8
    bf16x8 qf[8];
    {
      const uint8_t* qr = static_cast<const uint8_t*>(qp) + ((bat * N + i) * H_q + r * G + g) * kDh * EB;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        if constexpr (!FP8) {
          qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qr + (16 * ks + 8 * h) * 2));
        } else {
          const u32x2 w = *reinterpret_cast<const u32x2*>(qr + 16 * ks + 8 * h);
          const u32x2 a = e4m3x4_to_bf16x4(w[0]), b = e4m3x4_to_bf16x4(w[1]);
          qf[ks] = as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
        }
      }
    }

    // ---- S^T = K_b Q^T: acc[mt] holds keys 32mt + 8(e/4) + 4h + (e%4) of row rho
    f32x16 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      acc[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(kl + k_lds_off(32 * mt + n, 2 * ks + h)));
        acc[mt] = mfma32x32x16(kf, qf[ks], acc[mt]);
      }
    }

    // ---- causal limit (only the query's own block is partially visible)
    const int limit = (blk == i / kBk) ? static_cast<int>(i - key0) : kBk - 1;
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int el = 0; el < 16; ++el) {
        const int key = 32 * mt + 8 * (el >> 2) + 4 * h + (el & 3);
        const float t = key <= limit ? acc[mt][el] * scale_log2 : -__builtin_huge_valf();
        acc[mt][el] = t;
        m = fmaxf(m, t);
      }
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    float l = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int el = 0; el < 16; ++el) {
        const float p = __builtin_amdgcn_exp2f(acc[mt][el] - m);
        acc[mt][el] = p;
        l += p;
      }
    }
    l += __shfl_xor(l, 32);

    // ---- P^T fragments (B operand of O^T = V^T P^T): step (mt, e2) covers
    // keys 32mt + 16e2 + 8(j/4) + 4h + (j%4), exactly accumulator elements
    // 8e2 .. 8e2 + 7 of acc[mt].
    bf16x8 pf[8];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        pf[2 * mt + e2] = as_bf16x8(u32x4{
            pack_bf16x2(acc[mt][8 * e2 + 0], acc[mt][8 * e2 + 1]),
            pack_bf16x2(acc[mt][8 * e2 + 2], acc[mt][8 * e2 + 3]),
            pack_bf16x2(acc[mt][8 * e2 + 4], acc[mt][8 * e2 + 5]),
            pack_bf16x2(acc[mt][8 * e2 + 6], acc[mt][8 * e2 + 7])});
      }
    }
    const float inv = out_scale / l;
    const int64_t orow = ((seq * q_count + qrow) * kslots + slot) * G + g;
    uint16_t* dst = o_part + orow * kDh + 64 * h;

    // ---- O^T = V^T P^T, one 32-dim tile at a time; lane (n, h) receives dims
    // 64h + 16nt + el of its row and stores them straight away.
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int d = dsel + 16 * nt;
      f32x16 oacc = {};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int c1 = 4 * st + h;  // = 8 mt + 4 e2 + h
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vl + vt_lds_off(d, c1));
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vl + vt_lds_off(d, c1 + 2));
        oacc = mfma32x32x16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pf[st], oacc);
      }
      if (row_ok) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int b8 = 8 * hf;
          *reinterpret_cast<u32x4*>(dst + 16 * nt + b8) = u32x4{
              pack_bf16x2(oacc[b8 + 0] * inv, oacc[b8 + 1] * inv),
              pack_bf16x2(oacc[b8 + 2] * inv, oacc[b8 + 3] * inv),
              pack_bf16x2(oacc[b8 + 4] * inv, oacc[b8 + 5] * inv),
              pack_bf16x2(oacc[b8 + 6] * inv, oacc[b8 + 7] * inv)};
        }
      }
    }
    if (row_ok && h == 0) lse_part[orow] = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
  }
}

template <int G>
hipError_t launch_g(const void* q, const void* k, const void* v, bool fp8, int batch, int64_t N,
                    int H_kv, int kslots, float scale_log2, float out_scale,
                    const int32_t* blk_offsets, const int32_t* blk_entries, const int32_t* sched,
                    int64_t q_begin, int64_t q_count, uint16_t* o_part, float* lse_part,
                    hipStream_t stream) {
  const SchedLayout s = sched_layout(batch, H_kv, G, q_begin, q_count);
  int64_t grid = attn_max_items(batch, H_kv, G, kslots, q_begin, q_count) + kXcds;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  auto kern = fp8 ? sparse_attn_kernel<G, true> : sparse_attn_kernel<G, false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kAttnThreads), 0, stream, q, k,
                     v, N, H_kv, kslots, scale_log2, out_scale, blk_offsets, blk_entries,
                     sched + s.off_items, sched, s.nbins, s.B_c, q_begin, q_count, o_part,
                     lse_part);
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
