// Row copies between a sequence and its copy padded to whole chunks: a prefill whose length is
// not a multiple of the chunk runs on the padded copy (the padded rows are zero, lie after every
// real row and are therefore never visible to one), and its real rows are copied back.
#include "hils_launch.h"

namespace hils {

// dst[s][r] = r < rows_src ? src[s][r] : 0 for r < rows_dst, rows of row_words 32-bit words.
__global__ __launch_bounds__(256) void copy_rows_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                        int nseq, int rows_src, int rows_dst, int row_words) {
  const size_t per_seq = (size_t)rows_dst * row_words;
  const size_t n = (size_t)nseq * per_seq;
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (size_t)gridDim.x * 256) {
    const size_t s = x / per_seq, rem = x % per_seq;
    const int r = (int)(rem / row_words), c = (int)(rem % row_words);
    dst[x] = r < rows_src ? src[(s * rows_src + r) * row_words + c] : 0u;
  }
}

hipError_t launch_copy_rows(const void* src, void* dst, int nseq, int rows_src, int rows_dst, size_t row_bytes,
                            hipStream_t st) {
  const size_t n = (size_t)nseq * rows_dst * (row_bytes / 4);
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(copy_rows_kernel, dim3(grid), dim3(256), 0, st, static_cast<const uint32_t*>(src),
                     static_cast<uint32_t*>(dst), nseq, rows_src, rows_dst, (int)(row_bytes / 4));
  return hipGetLastError();
}

}  // namespace hils
