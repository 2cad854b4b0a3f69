// Host side of the C ABI declared in include/msa.h: argument validation,
// scratch/workspace sizing, the chunk loop of the whole forward pass and the
// kernel launches.  Validation makes no HIP call, so every error path returns
// before anything is enqueued.
#include <math.h>
#include <string.h>

#include <mutex>

#include "msa.h"
#include "msa_internal.h"

// Device-resident scratch of msa_decode_static, for callers that cannot
// allocate.  In host code `scratch` names a host-side stand-in, never the
// device copy: only the address hipGetSymbolAddress returns is passed on.
static __device__ __align__(256) uint8_t scratch[MSA_STATIC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

// Per-device address of `scratch`, looked up once per device (with that
// device current) on the first msa_decode_static call there.
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return MSA_ERR_HIP;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Selection groups: one per index (proxy) head, each the adjacent
// H_q / H_sel query heads; H_idx = 0 makes them the GQA groups.
int HS(const msa_dims* d) { return d->H_idx > 0 ? d->H_idx : d->H_kv; }
int GS(const msa_dims* d) { return d->H_q / HS(d); }
// log2 of H_sel / H_kv (= G / G_sel, a ratio of powers of two)
int KVS(const msa_dims* d) {
  int s = 0;
  while ((d->H_kv << s) < HS(d)) ++s;
  return s;
}

int check_dims(const msa_dims* d) {
  if (!d) return MSA_ERR_NULL;
  if (d->batch < 1 || d->N < 1 || d->H_kv < 1 || d->G < 1 || d->H_q < 1 || d->k < 1 ||
      d->d_h < 1 || d->d_idx < 1 || d->B_k < 1)
    return MSA_ERR_SHAPE;
  if (static_cast<int64_t>(d->G) * d->H_kv != d->H_q) return MSA_ERR_SHAPE;
  if (d->d_h != msa::kDh) return MSA_ERR_UNSUPPORTED;
  if (d->B_k != 32 && d->B_k != 64 && d->B_k != msa::kBk) return MSA_ERR_UNSUPPORTED;
  if (d->d_idx != 64 && d->d_idx != 128) return MSA_ERR_UNSUPPORTED;
  if (d->G != 1 && d->G != 2 && d->G != 4 && d->G != 8 && d->G != 16) return MSA_ERR_UNSUPPORTED;
  if (d->k > 32) return MSA_ERR_UNSUPPORTED;
  if (d->H_idx < 0) return MSA_ERR_SHAPE;
  if (d->H_idx > 0) {
    if (d->H_idx % d->H_kv != 0 || d->H_q % d->H_idx != 0) return MSA_ERR_SHAPE;
    const int gs = d->H_q / d->H_idx;
    if (gs != 1 && gs != 2 && gs != 4 && gs != 8 && gs != 16) return MSA_ERR_UNSUPPORTED;
  }
  if ((d->N + d->B_k - 1) / d->B_k > 16384) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

int check_range(const msa_dims* d, int64_t q_begin, int64_t q_count) {
  if (q_begin < 0 || q_count < 1 || q_begin > d->N || q_count > d->N - q_begin) return MSA_ERR_SHAPE;
  if (q_begin % d->B_k != 0) return MSA_ERR_SHAPE;
  const int64_t slots = static_cast<int64_t>(d->batch) * HS(d) * q_count * d->k;
  if (slots >= (int64_t(1) << 31)) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

int check_opts(const msa_dims* d, const msa_opts* o) {
  if (!o) return MSA_ERR_NULL;
  if (o->qkv_dtype != MSA_DTYPE_BF16 && o->qkv_dtype != MSA_DTYPE_FP8_E4M3) return MSA_ERR_UNSUPPORTED;
  if (o->reserved != 0) return MSA_ERR_SHAPE;
  if (!isfinite(o->softmax_scale)) return MSA_ERR_SHAPE;
  if (o->qkv_dtype == MSA_DTYPE_FP8_E4M3) {
    if (!(o->q_scale > 0.f) || !(o->k_scale > 0.f) || !(o->v_scale > 0.f) ||
        !isfinite(o->q_scale) || !isfinite(o->k_scale) || !isfinite(o->v_scale))
      return MSA_ERR_SHAPE;
  }
  if (o->q_chunk < 0 || (o->q_chunk > 0 && o->q_chunk % d->B_k != 0)) return MSA_ERR_SHAPE;
  // fp8 Q/K/V run with 128-token blocks only
  if (o->qkv_dtype == MSA_DTYPE_FP8_E4M3 && d->B_k != msa::kBk) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

// Softmax multiplier in log2 units and the output multiplier of the attention
// kernel.  fp8 operands are widened as value * 2^-8 each, which the scales undo.
void attn_scales(const msa_dims* d, const msa_opts* o, float* scale_log2, float* out_scale) {
  double s = o->softmax_scale > 0.f ? o->softmax_scale : 1.0 / sqrt(static_cast<double>(d->d_h));
  double out = 1.0;
  if (o->qkv_dtype == MSA_DTYPE_FP8_E4M3) {
    s *= static_cast<double>(o->q_scale) * o->k_scale * 65536.0;
    out = static_cast<double>(o->v_scale) * 256.0;
  }
  *scale_log2 = static_cast<float>(s * 1.4426950408889634);
  *out_scale = static_cast<float>(out);
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

struct ForwardLayout {
  int64_t qc;  // rows per chunk
  size_t off_bi, off_off, off_ent, off_sched, off_opart, off_lpart, off_biall, total;
};

ForwardLayout forward_layout(const msa_dims* d, const msa_opts* o) {
  ForwardLayout L{};
  const int64_t want = o->q_chunk > 0 ? o->q_chunk : MSA_DEFAULT_Q_CHUNK;
  L.qc = want < d->N ? want : d->N;
  const int64_t seqs = static_cast<int64_t>(d->batch) * HS(d);
  const int64_t B = (d->N + d->B_k - 1) / d->B_k;
  const size_t slots = static_cast<size_t>(seqs) * L.qc * d->k;
  // the largest scratch is needed by the last (or the only) full-size chunk
  int64_t words = 0;
  const int64_t nchunks = (d->N + L.qc - 1) / L.qc;
  for (int64_t c = (nchunks > 2 ? nchunks - 2 : 0); c < nchunks; ++c) {
    const int64_t qb = c * L.qc, qn = (d->N - qb) < L.qc ? (d->N - qb) : L.qc;
    const msa::SchedLayout s = msa::sched_layout(d->batch, HS(d), GS(d), d->k, qb, qn, d->B_k);
    words = s.words > words ? s.words : words;
  }
  size_t off = 0;
  L.off_bi = off;
  off += align256(slots * 4);
  L.off_off = off;
  off += align256(static_cast<size_t>(seqs) * (B + 1) * 4);
  L.off_ent = off;
  off += align256(slots * 4);
  L.off_sched = off;
  off += align256(static_cast<size_t>(words) * 4);
  L.off_opart = off;
  off += align256(slots * GS(d) * d->d_h * 2);
  L.off_lpart = off;
  off += align256(slots * GS(d) * 4);
  // chunked: the whole selection (one index launch over all rows)
  L.off_biall = off;
  if (L.qc < d->N) off += align256(static_cast<size_t>(seqs) * d->N * d->k * 4);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

int msa_abi_version(void) { return MSA_ABI_VERSION; }

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_NULL: return "a required pointer is NULL";
    case MSA_ERR_SHAPE: return "inconsistent sizes or range";
    case MSA_ERR_UNSUPPORTED: return "shape outside the supported set";
    case MSA_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP runtime error";
    case MSA_ERR_SCRATCH: return "problem needs more than the static scratch (MSA_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int msa_last_hip_error(void) { return g_last_hip_error; }

int msa_index_topk(const msa_dims* dims, const void* q_idx, const void* k_idx, int64_t q_begin,
                   int64_t q_count, int32_t* block_idx, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_range(dims, q_begin, q_count))) return st;
  if (!q_idx || !k_idx || !block_idx) return MSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(k_idx) || misaligned(block_idx)) return MSA_ERR_ALIGN;
  hipError_t e = msa::launch_index_topk(static_cast<const uint16_t*>(q_idx),
                                        static_cast<const uint16_t*>(k_idx), dims->batch, dims->N,
                                        HS(dims), dims->d_idx, dims->k, q_begin, q_count,
                                        block_idx, static_cast<hipStream_t>(stream), 0, 1, dims->B_k);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_index_topk_forced(const msa_dims* dims, const void* q_idx, const void* k_idx,
                          int64_t q_begin, int64_t q_count, int force_first, int local_window,
                          int32_t* block_idx, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_range(dims, q_begin, q_count))) return st;
  if (force_first != 0 && force_first != 1) return MSA_ERR_SHAPE;
  if (local_window < 1 || (force_first ? 1 : 0) + (local_window - 1) > dims->k - 1) return MSA_ERR_SHAPE;
  if (!q_idx || !k_idx || !block_idx) return MSA_ERR_NULL;
  if (misaligned(q_idx) || misaligned(k_idx) || misaligned(block_idx)) return MSA_ERR_ALIGN;
  hipError_t e = msa::launch_index_topk(static_cast<const uint16_t*>(q_idx),
                                        static_cast<const uint16_t*>(k_idx), dims->batch, dims->N,
                                        HS(dims), dims->d_idx, dims->k, q_begin, q_count,
                                        block_idx, static_cast<hipStream_t>(stream), force_first,
                                        local_window, dims->B_k);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_window_select(const msa_dims* dims, int64_t q_begin, int64_t q_count, int32_t* block_idx,
                      void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_range(dims, q_begin, q_count))) return st;
  if (!block_idx) return MSA_ERR_NULL;
  if (misaligned(block_idx)) return MSA_ERR_ALIGN;
  hipError_t e = msa::launch_window_select(dims->batch, HS(dims), dims->k, q_begin, q_count, block_idx,
                                           static_cast<hipStream_t>(stream), dims->B_k);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_invert_workspace_size(const msa_dims* dims, int64_t q_begin, int64_t q_count,
                              size_t* bytes) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_range(dims, q_begin, q_count))) return st;
  if (!bytes) return MSA_ERR_NULL;
  const msa::SchedLayout s = msa::sched_layout(dims->batch, HS(dims), GS(dims), dims->k, q_begin, q_count,
                                               dims->B_k);
  *bytes = static_cast<size_t>(s.words) * 4;
  return MSA_OK;
}

int msa_invert_blocks(const msa_dims* dims, const int32_t* block_idx, int64_t q_begin,
                      int64_t q_count, int32_t* blk_offsets, int32_t* blk_entries, void* sched,
                      size_t sched_bytes, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_range(dims, q_begin, q_count))) return st;
  if (!block_idx || !blk_offsets || !blk_entries || !sched) return MSA_ERR_NULL;
  if (misaligned(block_idx) || misaligned(blk_offsets) || misaligned(blk_entries) ||
      misaligned(sched))
    return MSA_ERR_ALIGN;
  const msa::SchedLayout s = msa::sched_layout(dims->batch, HS(dims), GS(dims), dims->k, q_begin, q_count,
                                               dims->B_k);
  if (sched_bytes < static_cast<size_t>(s.words) * 4) return MSA_ERR_WORKSPACE;
  hipError_t e = msa::launch_invert(block_idx, dims->batch, HS(dims), GS(dims), dims->k, q_begin,
                                    q_count, blk_offsets, blk_entries, static_cast<int32_t*>(sched),
                                    static_cast<hipStream_t>(stream), dims->B_k);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_invert_status(const void* sched, int32_t* bad_ids, void* stream) {
  if (!sched || !bad_ids) return MSA_ERR_NULL;
  if (misaligned(sched)) return MSA_ERR_ALIGN;
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e);
  e = hipMemcpy(bad_ids, static_cast<const int32_t*>(sched) + msa::kHdrBad, sizeof(int32_t),
                hipMemcpyDeviceToHost);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_sparse_attn_fwd(const msa_dims* dims, const msa_opts* opts, const void* q, const void* k,
                        const void* v, const int32_t* blk_offsets, const int32_t* blk_entries,
                        const void* sched, int64_t q_begin, int64_t q_count, void* o_part,
                        float* lse_part, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_range(dims, q_begin, q_count))) return st;
  if ((st = check_opts(dims, opts))) return st;
  if (!q || !k || !v || !blk_offsets || !blk_entries || !sched || !o_part || !lse_part)
    return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(blk_offsets) ||
      misaligned(blk_entries) || misaligned(sched) || misaligned(o_part) || misaligned(lse_part))
    return MSA_ERR_ALIGN;
  float sl2, osc;
  attn_scales(dims, opts, &sl2, &osc);
  hipError_t e = msa::launch_sparse_attn(
      q, k, v, opts->qkv_dtype == MSA_DTYPE_FP8_E4M3, dims->batch, dims->N, HS(dims), GS(dims),
      KVS(dims), dims->k, sl2, osc, blk_offsets, blk_entries, static_cast<const int32_t*>(sched), q_begin,
      q_count, static_cast<uint16_t*>(o_part), lse_part, static_cast<hipStream_t>(stream), dims->B_k);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_combine(const msa_dims* dims, const int32_t* block_idx, const void* o_part,
                const float* lse_part, int64_t q_begin, int64_t q_count, void* o, float* lse,
                void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_range(dims, q_begin, q_count))) return st;
  if (!block_idx || !o_part || !lse_part || !o) return MSA_ERR_NULL;
  if (misaligned(block_idx) || misaligned(o_part) || misaligned(lse_part) || misaligned(o) ||
      (lse && misaligned(lse)))
    return MSA_ERR_ALIGN;
  hipError_t e = msa::launch_combine(block_idx, static_cast<const uint16_t*>(o_part), lse_part,
                                     dims->batch, dims->N, HS(dims), GS(dims), dims->k, q_begin,
                                     q_count, static_cast<uint16_t*>(o), lse,
                                     static_cast<hipStream_t>(stream), dims->B_k);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_dense_attn_fwd(const msa_dims* dims, const msa_opts* opts, const void* q, const void* k,
                       const void* v, int64_t q_begin, int64_t q_count, void* o, float* lse,
                       void* stream) {
  if (!dims || !opts) return MSA_ERR_NULL;
  if (dims->batch < 1 || dims->N < 1 || dims->H_kv < 1 || dims->G < 1 || dims->H_q < 1 ||
      dims->d_h < 1)
    return MSA_ERR_SHAPE;
  if (static_cast<int64_t>(dims->G) * dims->H_kv != dims->H_q) return MSA_ERR_SHAPE;
  if (dims->d_h != msa::kDh) return MSA_ERR_UNSUPPORTED;
  if (dims->G != 1 && dims->G != 2 && dims->G != 4 && dims->G != 8 && dims->G != 16)
    return MSA_ERR_UNSUPPORTED;
  if (q_begin < 0 || q_count < 1 || q_begin > dims->N || q_count > dims->N - q_begin)
    return MSA_ERR_SHAPE;
  if (static_cast<int64_t>(dims->batch) * dims->H_kv > (int64_t(1) << 20)) return MSA_ERR_UNSUPPORTED;
  if (opts->reserved != 0 || !isfinite(opts->softmax_scale)) return MSA_ERR_SHAPE;
  if (opts->qkv_dtype != MSA_DTYPE_BF16) return MSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || (lse && misaligned(lse)))
    return MSA_ERR_ALIGN;
  float sl2, osc;
  attn_scales(dims, opts, &sl2, &osc);
  hipError_t e = msa::launch_dense_attn(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                        static_cast<const uint16_t*>(v), dims->batch, dims->N,
                                        dims->H_kv, dims->G, q_begin, q_count, sl2,
                                        static_cast<uint16_t*>(o), lse, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

namespace {

struct DecodeLayout {
  size_t off_scores, off_bi, off_opart, off_lpart, total;
};

DecodeLayout decode_layout(const msa_dims* d) {
  DecodeLayout L{};
  const size_t seqs = static_cast<size_t>(d->batch) * HS(d);
  const size_t B = static_cast<size_t>((d->N + d->B_k - 1) / d->B_k);
  size_t off = 0;
  L.off_scores = off;
  off += align256(seqs * B * 4);
  L.off_bi = off;
  off += align256(seqs * d->k * 4);
  L.off_opart = off;
  off += align256(seqs * d->k * GS(d) * d->d_h * 2);
  L.off_lpart = off;
  off += align256(seqs * d->k * GS(d) * 4);
  L.total = off;
  return L;
}

int check_decode(const msa_dims* d, const msa_opts* o) {
  int st = check_dims(d);
  if (st) return st;
  if (!o) return MSA_ERR_NULL;
  if (o->reserved != 0 || !isfinite(o->softmax_scale)) return MSA_ERR_SHAPE;
  if (o->qkv_dtype != MSA_DTYPE_BF16) return MSA_ERR_UNSUPPORTED;
  if (HS(d) > 32 || d->batch > 65535) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

}  // namespace

int msa_decode_workspace_size(const msa_dims* dims, const msa_opts* opts, size_t* bytes) {
  int st = check_decode(dims, opts);
  if (st) return st;
  if (!bytes) return MSA_ERR_NULL;
  *bytes = decode_layout(dims).total;
  return MSA_OK;
}

int msa_decode(const msa_dims* dims, const msa_opts* opts, const void* q, const void* q_idx,
               const void* k, const void* v, const void* k_idx, const int32_t* seq_lens, void* o,
               float* lse, int32_t* block_idx_out, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_decode(dims, opts);
  if (st) return st;
  if (!q || !q_idx || !k || !v || !k_idx || !o || !workspace) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(q_idx) || misaligned(k) || misaligned(v) || misaligned(k_idx) ||
      misaligned(o) || (lse && misaligned(lse)) || (block_idx_out && misaligned(block_idx_out)) ||
      (seq_lens && (reinterpret_cast<uintptr_t>(seq_lens) & 3u)) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return MSA_ERR_ALIGN;
  const DecodeLayout L = decode_layout(dims);
  if (ws_bytes < L.total) return MSA_ERR_WORKSPACE;
  float sl2, osc;
  attn_scales(dims, opts, &sl2, &osc);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* bi = block_idx_out ? block_idx_out : reinterpret_cast<int32_t*>(ws + L.off_bi);
  hipError_t e = msa::launch_decode(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(k_idx), dims->batch, dims->N, HS(dims),
      GS(dims), KVS(dims), dims->d_idx, dims->k, sl2, reinterpret_cast<float*>(ws + L.off_scores), bi,
      reinterpret_cast<uint16_t*>(ws + L.off_opart), reinterpret_cast<float*>(ws + L.off_lpart),
      static_cast<uint16_t*>(o), lse, static_cast<hipStream_t>(stream), dims->B_k, seq_lens);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_decode_static(const msa_dims* dims, const msa_opts* opts, const void* q, const void* q_idx,
                      const void* k, const void* v, const void* k_idx, const int32_t* seq_lens,
                      void* o, float* lse, int32_t* block_idx_out, void* stream) {
  int st = check_decode(dims, opts);
  if (st) return st;
  if (decode_layout(dims).total > static_cast<size_t>(MSA_STATIC_SCRATCH_BYTES)) return MSA_ERR_SCRATCH;
  // (msa_decode checks pointers and alignment before it enqueues anything;
  // these are the same checks, made before the scratch lookup touches the
  // device)
  if (!q || !q_idx || !k || !v || !k_idx || !o) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(q_idx) || misaligned(k) || misaligned(v) || misaligned(k_idx) ||
      misaligned(o) || (lse && misaligned(lse)) || (block_idx_out && misaligned(block_idx_out)) ||
      (seq_lens && (reinterpret_cast<uintptr_t>(seq_lens) & 3u)))
    return MSA_ERR_ALIGN;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e);
  // Every kernel of the step writes the scratch regions it later reads
  // (scores of the blocks before each sequence's local block, the selection,
  // the partials of the valid slots), so nothing needs clearing between calls.
  return msa_decode(dims, opts, q, q_idx, k, v, k_idx, seq_lens, o, lse, block_idx_out, ws,
                    static_cast<size_t>(MSA_STATIC_SCRATCH_BYTES), stream);
}

namespace {

struct BackwardLayout {
  int64_t qc;  // rows per chunk
  size_t off_dk, off_dv, off_dki, off_dlt, off_bi, off_off, off_ent, off_sched, off_dqp, off_lsp, off_lsi,
      off_dqip, off_klp, off_tch, total;
};

BackwardLayout backward_layout(const msa_dims* d, const msa_opts* o) {
  BackwardLayout L{};
  L.qc = o->q_chunk > 0 ? (o->q_chunk < d->N ? o->q_chunk : d->N) : d->N;
  const int64_t seqs = static_cast<int64_t>(d->batch) * HS(d);
  const int64_t B = (d->N + d->B_k - 1) / d->B_k;
  const size_t slots = static_cast<size_t>(seqs) * L.qc * d->k;
  int64_t words = 0;
  const int64_t nchunks = (d->N + L.qc - 1) / L.qc;
  for (int64_t c = (nchunks > 2 ? nchunks - 2 : 0); c < nchunks; ++c) {
    const int64_t qb = c * L.qc, qn = (d->N - qb) < L.qc ? (d->N - qb) : L.qc;
    const msa::SchedLayout s = msa::sched_layout(d->batch, HS(d), GS(d), d->k, qb, qn, d->B_k);
    words = s.words > words ? s.words : words;
  }
  const size_t kv = static_cast<size_t>(d->batch) * d->N * d->H_kv * d->d_h * 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.off_dk = take(kv);
  L.off_dv = take(kv);
  L.off_dki = take(static_cast<size_t>(d->batch) * d->N * d->d_idx * 4);
  L.off_dlt = take(static_cast<size_t>(d->batch) * d->N * d->H_q * 4);
  L.off_bi = take(slots * 4);
  L.off_off = take(static_cast<size_t>(seqs) * (B + 1) * 4);
  L.off_ent = take(slots * 4);
  L.off_sched = take(static_cast<size_t>(words) * 4);
  L.off_dqp = take((slots + 1) * GS(d) * d->d_h * 2);  // + a spare row for padding rows
  L.off_lsp = take(slots * 4);
  L.off_lsi = take(static_cast<size_t>(seqs) * L.qc * 4);
  L.off_dqip = take((slots + 1) * d->d_idx * 4);
  L.off_klp = take((slots + 1) * 4);
  L.off_tch = take((slots + 1) * static_cast<size_t>(d->B_k) * 4);
  L.total = off;
  return L;
}

int check_backward(const msa_dims* d, const msa_opts* o) {
  int st = check_dims(d);
  if (st) return st;
  if ((st = check_opts(d, o))) return st;
  if (o->qkv_dtype != MSA_DTYPE_BF16 || d->B_k != msa::kBk) return MSA_ERR_UNSUPPORTED;
  const BackwardLayout L = backward_layout(d, o);
  return check_range(d, 0, L.qc);
}

}  // namespace

int msa_backward_workspace_size(const msa_dims* dims, const msa_opts* opts, size_t* bytes) {
  int st = check_backward(dims, opts);
  if (st) return st;
  if (!bytes) return MSA_ERR_NULL;
  *bytes = backward_layout(dims, opts).total;
  return MSA_OK;
}

int msa_backward(const msa_dims* dims, const msa_opts* opts, float kl_weight, const void* q, const void* k,
                 const void* v, const void* q_idx, const void* k_idx, const void* o, const float* lse,
                 const void* d_o, const int32_t* block_idx, void* dq, void* dk, void* dv, void* dq_idx,
                 void* dk_idx, float* kl, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_backward(dims, opts);
  if (st) return st;
  if (!isfinite(kl_weight)) return MSA_ERR_SHAPE;
  const bool index = dq_idx != nullptr || dk_idx != nullptr || kl != nullptr;
  if (!q || !k || !v || !o || !lse || !d_o || !block_idx || !dq || !dk || !dv || !workspace) return MSA_ERR_NULL;
  if (index && (!q_idx || !k_idx || !dq_idx || !dk_idx)) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse) || misaligned(d_o) ||
      misaligned(block_idx) || misaligned(dq) || misaligned(dk) || misaligned(dv) ||
      (index && (misaligned(q_idx) || misaligned(k_idx) || misaligned(dq_idx) || misaligned(dk_idx))) ||
      (kl && misaligned(kl)) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return MSA_ERR_ALIGN;
  const BackwardLayout L = backward_layout(dims, opts);
  if (ws_bytes < L.total) return MSA_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* dk_acc = reinterpret_cast<float*>(ws + L.off_dk);
  float* dv_acc = reinterpret_cast<float*>(ws + L.off_dv);
  float* dki_acc = reinterpret_cast<float*>(ws + L.off_dki);
  const int64_t nkv = static_cast<int64_t>(dims->batch) * dims->N * dims->H_kv * dims->d_h;
  const int64_t nki = static_cast<int64_t>(dims->batch) * dims->N * dims->d_idx;
  hipError_t e = msa::launch_fill_zero(dk_acc, nkv, s);
  if (e == hipSuccess) e = msa::launch_fill_zero(dv_acc, nkv, s);
  if (e == hipSuccess && index) e = msa::launch_fill_zero(dki_acc, nki, s);
  if (e != hipSuccess) return hip_fail(e);

  msa::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_ptr = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.dout = static_cast<const uint16_t*>(d_o);
  a.o = static_cast<const uint16_t*>(o);
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.k_idx = static_cast<const uint16_t*>(k_idx);
  a.lse = lse;
  a.batch = dims->batch;
  a.N = dims->N;
  a.H_sel = HS(dims);
  a.G = GS(dims);
  a.kv_shift = KVS(dims);
  a.k = dims->k;
  a.d_idx = dims->d_idx;
  a.scale = opts->softmax_scale > 0.f ? opts->softmax_scale : static_cast<float>(1.0 / sqrt(static_cast<double>(dims->d_h)));
  a.idx_scale = static_cast<float>(1.0 / sqrt(static_cast<double>(dims->d_idx)));
  a.kl_weight = kl_weight;
  a.index = index;
  a.dlt = reinterpret_cast<float*>(ws + L.off_dlt);
  a.lsei_part = reinterpret_cast<float*>(ws + L.off_lsp);
  a.lsei2 = reinterpret_cast<float*>(ws + L.off_lsi);
  a.dqi_part = reinterpret_cast<float*>(ws + L.off_dqip);
  a.kl_part = reinterpret_cast<float*>(ws + L.off_klp);
  a.tch = reinterpret_cast<float*>(ws + L.off_tch);
  a.dk_acc = dk_acc;
  a.dv_acc = dv_acc;
  a.dki_acc = dki_acc;
  a.kl = kl;
  a.dq_part = reinterpret_cast<uint16_t*>(ws + L.off_dqp);
  a.dq = static_cast<uint16_t*>(dq);
  a.dq_idx = static_cast<uint16_t*>(dq_idx);
  int32_t* offs = reinterpret_cast<int32_t*>(ws + L.off_off);
  int32_t* ents = reinterpret_cast<int32_t*>(ws + L.off_ent);
  int32_t* sched = reinterpret_cast<int32_t*>(ws + L.off_sched);
  int32_t* bi_chunk = reinterpret_cast<int32_t*>(ws + L.off_bi);
  const bool one_chunk = L.qc >= dims->N;
  const int64_t seqs = static_cast<int64_t>(dims->batch) * HS(dims);

  for (int64_t qb = 0; qb < dims->N; qb += L.qc) {
    const int64_t qn = (dims->N - qb) < L.qc ? (dims->N - qb) : L.qc;
    const int32_t* bi = block_idx;
    if (!one_chunk) {
      const size_t w = static_cast<size_t>(qn) * dims->k * sizeof(int32_t);
      e = hipMemcpy2DAsync(bi_chunk, w, block_idx + qb * dims->k, static_cast<size_t>(dims->N) * dims->k * 4, w,
                           static_cast<size_t>(seqs), hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e);
      bi = bi_chunk;
    }
    e = msa::launch_invert(bi, dims->batch, HS(dims), GS(dims), dims->k, qb, qn, offs, ents, sched, s, dims->B_k);
    if (e != hipSuccess) return hip_fail(e);
    a.block_idx = bi;
    a.entries = ents;
    a.sched = sched;
    a.q_begin = qb;
    a.q_count = qn;
    e = msa::launch_backward_chunk(a, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  e = msa::launch_to_bf16(dk_acc, static_cast<uint16_t*>(dk), nkv, s);
  if (e == hipSuccess) e = msa::launch_to_bf16(dv_acc, static_cast<uint16_t*>(dv), nkv, s);
  if (e == hipSuccess && index) e = msa::launch_to_bf16(dki_acc, static_cast<uint16_t*>(dk_idx), nki, s);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_workspace_size(const msa_dims* dims, const msa_opts* opts, size_t* bytes) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_opts(dims, opts))) return st;
  if (!bytes) return MSA_ERR_NULL;
  const ForwardLayout L = forward_layout(dims, opts);
  if ((st = check_range(dims, 0, L.qc))) return st;
  *bytes = L.total;
  return MSA_OK;
}

int msa_forward(const msa_dims* dims, const msa_opts* opts, const void* q, const void* k,
                const void* v, const void* q_idx, const void* k_idx, void* o, float* lse,
                int32_t* block_idx_out, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_opts(dims, opts))) return st;
  if (!q || !k || !v || !q_idx || !k_idx || !o || !workspace) return MSA_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(q_idx) || misaligned(k_idx) ||
      misaligned(o) || (lse && misaligned(lse)) || (block_idx_out && misaligned(block_idx_out)) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return MSA_ERR_ALIGN;
  const ForwardLayout L = forward_layout(dims, opts);
  if ((st = check_range(dims, 0, L.qc))) return st;
  if (ws_bytes < L.total) return MSA_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* bi_chunk = reinterpret_cast<int32_t*>(ws + L.off_bi);
  int32_t* offs = reinterpret_cast<int32_t*>(ws + L.off_off);
  int32_t* ents = reinterpret_cast<int32_t*>(ws + L.off_ent);
  int32_t* sched = reinterpret_cast<int32_t*>(ws + L.off_sched);
  uint16_t* opart = reinterpret_cast<uint16_t*>(ws + L.off_opart);
  float* lpart = reinterpret_cast<float*>(ws + L.off_lpart);
  float sl2, osc;
  attn_scales(dims, opts, &sl2, &osc);
  const bool fp8 = opts->qkv_dtype == MSA_DTYPE_FP8_E4M3;
  const bool one_chunk = L.qc >= dims->N;
  const int64_t seqs = static_cast<int64_t>(dims->batch) * HS(dims);

  // With several chunks the index branch runs once over all rows (its
  // workgroups heaviest first across the whole sequence, instead of one
  // launch per chunk that waits for its heaviest tile); each chunk's rows of
  // every sequence are then copied out contiguous for the inversion and the
  // combine.
  int32_t* bi_all = nullptr;
  if (!one_chunk) {
    bi_all = block_idx_out ? block_idx_out : reinterpret_cast<int32_t*>(ws + L.off_biall);
    const hipError_t e = msa::launch_index_topk(static_cast<const uint16_t*>(q_idx),
                                                static_cast<const uint16_t*>(k_idx), dims->batch, dims->N,
                                                HS(dims), dims->d_idx, dims->k, 0, dims->N, bi_all, s, 0, 1,
                                                dims->B_k);
    if (e != hipSuccess) return hip_fail(e);
  }

  for (int64_t qb = 0; qb < dims->N; qb += L.qc) {
    const int64_t qn = (dims->N - qb) < L.qc ? (dims->N - qb) : L.qc;
    int32_t* bi = (one_chunk && block_idx_out) ? block_idx_out : bi_chunk;
    hipError_t e;
    if (one_chunk) {
      e = msa::launch_index_topk(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                                 dims->batch, dims->N, HS(dims), dims->d_idx, dims->k, qb, qn, bi, s, 0, 1,
                                 dims->B_k);
    } else {
      const size_t w = static_cast<size_t>(qn) * dims->k * sizeof(int32_t);
      e = hipMemcpy2DAsync(bi, w, bi_all + qb * dims->k, static_cast<size_t>(dims->N) * dims->k * 4, w,
                           static_cast<size_t>(seqs), hipMemcpyDeviceToDevice, s);
    }
    if (e != hipSuccess) return hip_fail(e);
    e = msa::launch_invert(bi, dims->batch, HS(dims), GS(dims), dims->k, qb, qn, offs, ents, sched, s,
                           dims->B_k);
    if (e != hipSuccess) return hip_fail(e);
    e = msa::launch_sparse_attn(q, k, v, fp8, dims->batch, dims->N, HS(dims), GS(dims),
                                KVS(dims), dims->k,
                                sl2, osc, offs, ents, sched, qb, qn, opart, lpart, s, dims->B_k);
    if (e != hipSuccess) return hip_fail(e);
    e = msa::launch_combine(bi, opart, lpart, dims->batch, dims->N, HS(dims), GS(dims), dims->k,
                            qb, qn, static_cast<uint16_t*>(o), lse, s, dims->B_k);
    if (e != hipSuccess) return hip_fail(e);
  }
  return MSA_OK;
}

}  // extern "C"
