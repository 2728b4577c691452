// Direct-to-LDS loading helpers shared by the fp16 GEMM kernels (gfx950).
#pragma once

#include "device_common.h"

namespace ee {

// Word 3 of a raw (unformatted, stride 0) buffer descriptor on gfx9-family GPUs.
constexpr int kBufferFlags = 0x00020000;

// 16-byte direct-to-LDS buffer load (buffer_load_dwordx4 ... lds): lane l of
// the wave writes its 16 bytes at lds + 16 * l.  A device-only function: the
// builtin needs a device target feature, and calling it from a lambda (which
// HIP compiles for both sides) makes the host pass drop the kernel's stub.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds, int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset, 0,
                                           0);
}

// LDS rows of 128 bytes (8 chunks of 16 B): chunk c of row r is stored at
// chunk c ^ lds_swizzle(r), so the 16 rows a quarter-wave reads land on
// distinct banks whether the LDS serves 8 or 16 lanes of a 128-bit read per
// cycle.  Depends on r & 15 only.
__device__ __forceinline__ int lds_swizzle(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// Waits until this wave's direct-to-LDS loads have written LDS.  Needed before
// the barrier that publishes them: the workgroup-scope fence of __syncthreads
// only waits for LDS instructions (lgkmcnt), and the compiler does not count
// a direct-to-LDS load as an LDS write.  The memory clobber keeps LDS reads below it.
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier that lets this wave's newest N vector memory operations
// stay in flight: it waits for this wave's LDS reads (their stage may be
// refilled right after) and all older loads, then s_barrier.  Direct-to-LDS
// loads retire in issue order among themselves, so with the newest N allowed
// to fly every older one has written LDS.  __syncthreads cannot be used here:
// its fence makes the compiler wait for every load.
template <int N>
__device__ __forceinline__ void barrier_after_loads() {
  static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace ee
