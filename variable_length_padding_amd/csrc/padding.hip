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

// Transposing rebuild: packed q|k|v rows [T, n*nh*hd] -> head-major padded
// tensors [n, B, nh, P, hd], pads zero.  One workgroup per (matrix, sequence,
// head) slab of P x hd elements, 16-byte vectors (vph per head row).
__global__ __launch_bounds__(kCopyThreads) void rebuild_heads_kernel(const u32x4* __restrict__ packed,
                                                                     const int32_t* __restrict__ cu, int B, int nh,
                                                                     int P, int vph, int64_t ld_vec, int n_mats,
                                                                     u32x4* __restrict__ out) {
  const int64_t slabs = (int64_t)n_mats * B * nh;
  for (int64_t slab = blockIdx.x; slab < slabs; slab += gridDim.x) {
    const int h = (int)(slab % nh);
    const int b = (int)((slab / nh) % B);
    const int m = (int)(slab / ((int64_t)nh * B));
    const int s0 = cu[b], L = cu[b + 1] - s0;
    const u32x4* src = packed + (int64_t)s0 * ld_vec + (int64_t)(m * nh + h) * vph;
    u32x4* dst = out + slab * (int64_t)P * vph;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int i = threadIdx.x; i < P * vph; i += kCopyThreads) {
      const int p = i / vph, c = i - p * vph;
      dst[i] = p < L ? src[(int64_t)p * ld_vec + c] : z;
    }
  }
}

// Transposing remove: head-major padded [B, nh, P, hd] -> packed [T, nh*hd];
// only the valid rows are read.
__global__ __launch_bounds__(kCopyThreads) void remove_heads_kernel(const u32x4* __restrict__ heads,
                                                                    const int32_t* __restrict__ cu, int B, int nh,
                                                                    int P, int vph, u32x4* __restrict__ packed) {
  const int64_t ld_vec = (int64_t)nh * vph;
  for (int64_t slab = blockIdx.x; slab < (int64_t)B * nh; slab += gridDim.x) {
    const int h = (int)(slab % nh), b = (int)(slab / nh);
    const int s0 = cu[b], L = cu[b + 1] - s0;
    const u32x4* src = heads + slab * (int64_t)P * vph;
    u32x4* dst = packed + (int64_t)s0 * ld_vec + (int64_t)h * vph;
    for (int i = threadIdx.x; i < L * vph; i += kCopyThreads) {
      const int p = i / vph, c = i - p * vph;
      dst[(int64_t)p * ld_vec + c] = src[i];
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

hipError_t launch_rebuild_heads(const void* packed, const int32_t* cu, int B, int nh, int P, int head_bytes,
                                int n_mats, void* out, hipStream_t s) {
  const int vph = head_bytes / 16;
  const int64_t slabs = (int64_t)n_mats * B * nh;
  if (slabs <= 0) return hipSuccess;
  hipLaunchKernelGGL(rebuild_heads_kernel, dim3(grid_for_rows(slabs)), dim3(kCopyThreads), 0, s,
                     static_cast<const u32x4*>(packed), cu, B, nh, P, vph, (int64_t)n_mats * nh * vph, n_mats,
                     static_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t launch_remove_heads(const void* heads, const int32_t* cu, int B, int nh, int P, int head_bytes, void* packed,
                               hipStream_t s) {
  const int64_t slabs = (int64_t)B * nh;
  if (slabs <= 0) return hipSuccess;
  hipLaunchKernelGGL(remove_heads_kernel, dim3(grid_for_rows(slabs)), dim3(kCopyThreads), 0, s,
                     static_cast<const u32x4*>(heads), cu, B, nh, P, head_bytes / 16, static_cast<u32x4*>(packed));
  return hipGetLastError();
}

}  // namespace ee
