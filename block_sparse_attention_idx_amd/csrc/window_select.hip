// FLOP-matched sliding-window selection ("MiniMax Sparse Attention", the
// comparison of dynamic selection with a fixed sparse pattern): no index
// branch; query i attends to the first key block and to a local window of the
// same token budget ending at the query, i.e. block 0 and blocks
// L - k + 2 .. L with L = floor(i / B_k), k blocks in all -- the budget of the
// top-k selection.  When L < k every block 0 .. L is taken.  The rows use the
// selection layout [batch][H_kv][q_count][k] (ascending ids, -1 padded), so
// the inversion, the KV-outer attention and the combine run on them unchanged.
#include "msa_internal.h"

namespace msa {
namespace {

__global__ __launch_bounds__(256) void window_select_kernel(int64_t rows, int k, int64_t q_begin,
                                                            int64_t q_count, int bk,
                                                            int32_t* __restrict__ block_idx) {
  const int64_t f = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;  // (seq, row)
  if (f >= rows) return;
  const int64_t i = q_begin + f % q_count;
  const int L = static_cast<int>(i / bk);
  int32_t* dst = block_idx + f * k;
  if (L < k) {
    for (int s = 0; s < k; ++s) dst[s] = s <= L ? s : -1;
  } else {
    dst[0] = 0;
    for (int s = 1; s < k; ++s) dst[s] = L - k + 1 + s;
  }
}

}  // namespace

hipError_t launch_window_select(int batch, int H_kv, int k, int64_t q_begin, int64_t q_count,
                                int32_t* block_idx, hipStream_t stream, int bk) {
  const int64_t rows = static_cast<int64_t>(batch) * H_kv * q_count;
  const int64_t grid = (rows + 255) / 256;
  hipLaunchKernelGGL(window_select_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, rows, k,
                     q_begin, q_count, bk, block_idx);
  return hipGetLastError();
}

}  // namespace msa
