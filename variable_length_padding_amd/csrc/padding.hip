// transpose_padding_remove / transpose_padding_rebuild (Energon-AI
// announcement article, "Runtime" section), read as a gather/scatter of whole
// rows between the padded [B, P, H] layout and the packed [T, H] layout.
//
// Both kernels are HBM-bound copies: one workgroup per row (grid-strided),
// 16-byte vector loads and stores, four loads in flight per thread before the
// stores.  The bytes are copied as they are, so the kernels serve every dtype.
#include "device_common.h"
#include "internal.h"

namespace ee {
namespace {

constexpr int kCopyThreads = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes

__device__ __forceinline__ void copy_row(const u32x4* __restrict__ s, u32x4* __restrict__ d, int vpr) {
  int c = threadIdx.x;
  for (; c + 3 * kCopyThreads < vpr; c += 4 * kCopyThreads) {
    const u32x4 a0 = __builtin_nontemporal_load(s + c);
    const u32x4 a1 = __builtin_nontemporal_load(s + c + kCopyThreads);
    const u32x4 a2 = __builtin_nontemporal_load(s + c + 2 * kCopyThreads);
    const u32x4 a3 = __builtin_nontemporal_load(s + c + 3 * kCopyThreads);
    d[c] = a0;
    d[c + kCopyThreads] = a1;
    d[c + 2 * kCopyThreads] = a2;
    d[c + 3 * kCopyThreads] = a3;
  }
  for (; c < vpr; c += kCopyThreads) d[c] = __builtin_nontemporal_load(s + c);
}

// packed[t] = padded[token_src[t]]
__global__ __launch_bounds__(kCopyThreads) void remove_kernel(const u32x4* __restrict__ padded,
                                                              const int32_t* __restrict__ token_src, int64_t T,
                                                              int vpr, u32x4* __restrict__ packed) {
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int64_t src = token_src[t];
    copy_row(padded + src * vpr, packed + t * vpr, vpr);
  }
}

// padded[r] = packed[pad2pack[r]], or zeros where pad2pack[r] < 0
__global__ __launch_bounds__(kCopyThreads) void rebuild_kernel(const u32x4* __restrict__ packed,
                                                               const int32_t* __restrict__ pad2pack, int64_t rows,
                                                               int vpr, u32x4* __restrict__ padded) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const int32_t idx = pad2pack[r];
    u32x4* d = padded + r * vpr;
    if (idx >= 0) {
      copy_row(packed + (int64_t)idx * vpr, d, vpr);
    } else {
      const u32x4 z = {0u, 0u, 0u, 0u};
      for (int c = threadIdx.x; c < vpr; c += kCopyThreads) d[c] = z;
    }
  }
}

unsigned grid_for_rows(int64_t rows) {
  const int64_t cap = 1 << 16;
  return (unsigned)(rows < 1 ? 1 : (rows > cap ? cap : rows));
}

}  // namespace

hipError_t launch_remove(const void* padded, const int32_t* token_src, int64_t T, int64_t row_bytes, void* packed,
                         hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(remove_kernel, dim3(grid_for_rows(T)), dim3(kCopyThreads), 0, s,
                     static_cast<const u32x4*>(padded), token_src, T, (int)(row_bytes / 16),
                     static_cast<u32x4*>(packed));
  return hipGetLastError();
}

hipError_t launch_rebuild(const void* packed, const int32_t* pad2pack, int64_t rows, int64_t row_bytes, void* padded,
                          hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rebuild_kernel, dim3(grid_for_rows(rows)), dim3(kCopyThreads), 0, s,
                     static_cast<const u32x4*>(packed), pad2pack, rows, (int)(row_bytes / 16),
                     static_cast<u32x4*>(padded));
  return hipGetLastError();
}

}  // namespace ee
