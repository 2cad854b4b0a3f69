// Seeded input fill kernel (test and benchmark input generation only; not part
// of the MSA library).  Writes, for element e of a tensor, table[hash(e) >> 48]
// where hash is SplitMix64 output number e of the stream seeded with `key`
// (Steele, Lea, Flood, OOPSLA 2014).  Optionally adds an fp32 vector to bf16
// rows before rounding back to bf16 (round-to-nearest-even), all in integer and
// IEEE fp32 operations so the host generator reproduces the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t splitmix_at(uint64_t key, uint64_t e) {
  uint64_t z = key + (e + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint16_t add_round_bf16(uint16_t x, float v) {
  float f = __uint_as_float(static_cast<uint32_t>(x) << 16);
  float y = __fadd_rn(f, v);
  uint32_t u = __float_as_uint(y);
  u = u + 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// mode 0: plain; 1: add vec[col] to every row; 2: add vec[col] to rows whose
// block within their sequence ((e mod seq_elems) / block_elems) is flagged in
// block_mask.
__global__ void fill_kernel(void* out, int elem_bytes, int64_t n, uint64_t key, int64_t offset,
                            const void* table, const float* vec, int dim,
                            const uint8_t* block_mask, int64_t block_elems, int64_t seq_elems,
                            int mode) {
  int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) {
    uint64_t h = splitmix_at(key, static_cast<uint64_t>(e + offset));
    uint32_t u = static_cast<uint32_t>(h >> 48);
    if (elem_bytes == 1) {
      static_cast<uint8_t*>(out)[e] = static_cast<const uint8_t*>(table)[u];
    } else {
      uint16_t x = static_cast<const uint16_t*>(table)[u];
      if (mode == 1 || (mode == 2 && block_mask[((e + offset) % seq_elems) / block_elems]))
        x = add_round_bf16(x, vec[(e + offset) % dim]);
      static_cast<uint16_t*>(out)[e] = x;
    }
  }
}

}  // namespace

// seq_elems: elements of one sequence (N rows); block_mask holds
// ceil(seq_elems / block_elems) flags.
extern "C" int synth_fill(void* out, int elem_bytes, int64_t n, uint64_t key, int64_t offset,
                          const void* table, const float* vec, int dim, const uint8_t* block_mask,
                          int64_t block_elems, int64_t seq_elems, int mode, hipStream_t stream) {
  if (n <= 0) return 0;
  if (!out || !table || (elem_bytes != 1 && elem_bytes != 2)) return -1;
  if (mode != 0 && (!vec || dim <= 0 || elem_bytes != 2)) return -1;
  if (mode == 2 && (!block_mask || block_elems <= 0 || seq_elems <= 0)) return -1;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, out,
                     elem_bytes, n, key, offset, table, vec, dim, block_mask, block_elems, seq_elems,
                     mode);
  return static_cast<int>(hipGetLastError());
}
