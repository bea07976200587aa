// Measurement probe (not part of the library's interface): a plain row copy with the
// access pattern of the library's row movers -- one wavefront per row, 16-byte
// non-temporal loads and stores -- in identity order or in a given row order.  Its rate
// on the same byte count is the achievable ceiling the benchmark reports beside each
// workload.  Built into its own shared library.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// dst row i <- src row (order ? order[i] : i); rows are row16 16-byte units long.
__global__ __launch_bounds__(256) void probe_copy_rows_kernel(const v4u* __restrict__ src, v4u* __restrict__ dst,
                                                              int64_t row16, int64_t nrows,
                                                              const int32_t* __restrict__ order) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (i >= nrows) return;
  const int64_t s = order != nullptr ? order[i] : i;
  const int lane = threadIdx.x % 64;
  const v4u* sp = src + s * row16;
  v4u* dp = dst + i * row16;
  for (int64_t b = 0; b < row16; b += 64 * 16) {
    v4u v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t j = b + u * 64 + lane;
      if (j < row16) v[u] = __builtin_nontemporal_load(sp + j);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t j = b + u * 64 + lane;
      if (j < row16) __builtin_nontemporal_store(v[u], dp + j);
    }
  }
}

}  // namespace

// Copies nrows rows of row_bytes bytes (a multiple of 16; both buffers 16-byte aligned)
// on `stream`.  order (device, nrows entries in [0, nrows)) or NULL.  Returns 0, or 1
// when the arguments are rejected, 2 when the launch fails.
extern "C" int ffnwb_probe_copy_rows(const void* src, void* dst, int64_t row_bytes, int64_t nrows,
                                     const int32_t* order, void* stream) {
  if (src == nullptr || dst == nullptr || row_bytes <= 0 || row_bytes % 16 != 0 || nrows < 0) return 1;
  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) != 0) return 1;
  if (nrows == 0) return 0;
  const unsigned blocks = static_cast<unsigned>((nrows + 3) / 4);
  hipLaunchKernelGGL(probe_copy_rows_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v4u*>(src), static_cast<v4u*>(dst), row_bytes / 16, nrows, order);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
