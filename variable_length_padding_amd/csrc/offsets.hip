// Offsets: per-sequence lengths (or the attention mask) prefix-summed into the
// packed token offsets that transpose_padding_remove / _rebuild use
// (Energon-AI announcement article, "Runtime" section).
//
//   cu[b]            exclusive prefix sum of the lengths, cu[B] = T
//   pad2pack[b*P+p]  cu[b] + p for a valid position, -1 for a pad
//   token_src[t]     the padded row of packed token t (inverse of pad2pack)
#include "device_common.h"
#include "internal.h"

namespace ee {
namespace {

constexpr int kScanThreads = 256;  // 4 waves; 2 lengths per thread covers EE_MAX_BATCH = 512

// Exclusive scan of the batch's lengths into s_cu[0..B] with wave64 shuffles;
// every workgroup repeats it (B <= 512 values, a few hundred cycles) so the
// fill below needs no grid-wide dependency.
__device__ void scan_lengths(const int32_t* s_len, int B, int32_t* s_cu) {
  __shared__ int32_t s_wave[kScanThreads / kWave];
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int a = 2 * t < B ? s_len[2 * t] : 0;
  const int b = 2 * t + 1 < B ? s_len[2 * t + 1] : 0;
  const int own = a + b;
  int x = own;  // inclusive scan within the wave
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  const int excl = before + x - own;
  if (2 * t < B) s_cu[2 * t] = excl;
  if (2 * t + 1 < B) s_cu[2 * t + 1] = excl + a;
  if (t == kScanThreads - 1) s_cu[B] = before + x;  // slots past B hold zeros: this is T
  __syncthreads();
}

__global__ __launch_bounds__(kScanThreads) void offsets_kernel(LensArg lens, int B, int P, int32_t* __restrict__ cu,
                                                               int32_t* __restrict__ token_src,
                                                               int32_t* __restrict__ pad2pack) {
  __shared__ int32_t s_len[EE_MAX_BATCH];
  __shared__ int32_t s_cu[EE_MAX_BATCH + 1];
  for (int i = threadIdx.x; i < B; i += kScanThreads) s_len[i] = lens.v[i];
  __syncthreads();
  scan_lengths(s_len, B, s_cu);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= B; i += kScanThreads) cu[i] = s_cu[i];
  const int64_t rows = (int64_t)B * P;
  for (int64_t r = (int64_t)blockIdx.x * kScanThreads + threadIdx.x; r < rows;
       r += (int64_t)gridDim.x * kScanThreads) {
    const int b = (int)(r / P);
    const int p = (int)(r - (int64_t)b * P);
    if (p < s_len[b]) {
      const int32_t tk = s_cu[b] + p;
      pad2pack[r] = tk;
      token_src[tk] = (int32_t)r;
    } else {
      pad2pack[r] = -1;
    }
  }
}

// Mask form: one workgroup walks the flattened mask in chunks of
// kMaskThreads * kItems bytes, scanning each chunk with wave64 shuffles and
// carrying the running count across chunks.
constexpr int kMaskThreads = 1024;
constexpr int kItems = 8;

__global__ __launch_bounds__(kMaskThreads) void offsets_mask_kernel(const uint8_t* __restrict__ mask, int B, int P,
                                                                    int32_t* __restrict__ cu,
                                                                    int32_t* __restrict__ token_src,
                                                                    int32_t* __restrict__ pad2pack,
                                                                    int32_t* __restrict__ total) {
  __shared__ int32_t s_wave[kMaskThreads / kWave];
  __shared__ int32_t s_carry;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int64_t n = (int64_t)B * P;
  if (t == 0) s_carry = 0;
  __syncthreads();
  for (int64_t base = 0; base < n; base += (int64_t)kMaskThreads * kItems) {
    const int64_t r0 = base + (int64_t)t * kItems;
    int v[kItems];
    int own = 0;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      v[i] = (r0 + i < n && mask[r0 + i] != 0) ? 1 : 0;
      own += v[i];
    }
    int x = own;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(x, d, kWave);
      if (lane >= d) x += y;
    }
    if (lane == kWave - 1) s_wave[wave] = x;
    const int carry = s_carry;
    __syncthreads();
    int before = carry, chunk_total = 0;
    for (int w = 0; w < kMaskThreads / kWave; ++w) {
      if (w < wave) before += s_wave[w];
      chunk_total += s_wave[w];
    }
    int e = before + x - own;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int64_t r = r0 + i;
      if (r < n) {
        if (r % P == 0) cu[r / P] = e;
        if (v[i]) {
          pad2pack[r] = e;
          token_src[e] = (int32_t)r;
        } else {
          pad2pack[r] = -1;
        }
        e += v[i];
      }
    }
    __syncthreads();
    if (t == 0) s_carry = carry + chunk_total;
    __syncthreads();
  }
  if (t == 0) {
    cu[B] = s_carry;
    *total = s_carry;
  }
}

}  // namespace

hipError_t launch_offsets(const LensArg& lens, int B, int P, int32_t* cu, int32_t* token_src, int32_t* pad2pack,
                          hipStream_t s) {
  const int64_t rows = (int64_t)B * P;
  int64_t blocks = (rows + kScanThreads - 1) / kScanThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(offsets_kernel, dim3((unsigned)blocks), dim3(kScanThreads), 0, s, lens, B, P, cu, token_src,
                     pad2pack);
  return hipGetLastError();
}

hipError_t launch_offsets_mask(const uint8_t* mask, int B, int P, int32_t* cu, int32_t* token_src,
                               int32_t* pad2pack, int32_t* total, hipStream_t s) {
  hipLaunchKernelGGL(offsets_mask_kernel, dim3(1), dim3(kMaskThreads), 0, s, mask, B, P, cu, token_src, pad2pack,
                     total);
  return hipGetLastError();
}

}  // namespace ee
