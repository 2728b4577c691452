// Incremental decoding with a packed KV cache: the kernels of an "extend"
// step, in which sequence b brings new_len[b] new tokens at positions
// ctx_len[b] .. ctx_len[b] + new_len[b] - 1 after ctx_len[b] cached ones
// (a prefill is an extend from ctx_len = 0, a decode step one new token).
// The README's "Latency" section measures a GPT-3 text-generation service
// and the EET page reports decoder-layer speedups; both are generation
// workloads, in which each new token attends to every earlier token of its
// sequence through the cached keys and values.
//
// Cache layout (caller-owned, per layer): [2 (k | v)][n_heads][capacity][head_dim].
// Sequence b owns the slots slot_base[b] .. slot_base[b] + ctx + new - 1, so
// the cache is packed by sequence (no padding to a batch maximum) and the keys
// of one (sequence, head) are one contiguous block.
#include "device_common.h"
#include "internal.h"

namespace ee {
namespace {

constexpr int kExtendThreads = 256;

// cu[b] = sum of new_len before b (one wave, B <= EE_MAX_EXTEND_BATCH)
__global__ __launch_bounds__(64) void extend_cu_kernel(ExtendArg arg, int B, int32_t* __restrict__ cu) {
  if (threadIdx.x != 0) return;
  int32_t run = 0;
  for (int b = 0; b < B; ++b) {
    cu[b] = run;
    run += arg.new_len[b];
  }
  cu[B] = run;
}

// sequence of packed new-token row t: the b with cu[b] <= t < cu[b + 1]
__device__ __forceinline__ int seq_of(const int32_t* __restrict__ cu, int B, int64_t t) {
  int lo = 0, hi = B;  // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Copies the k and v parts of each new token's qkv row into its cache slot.
// One workgroup per token (grid-strided); 16-byte vectors; vph vectors per head.
__global__ __launch_bounds__(kExtendThreads) void append_kv_kernel(const u32x4* __restrict__ qkv, ExtendArg arg,
                                                                 const int32_t* __restrict__ cu, int B, int64_t T,
                                                                 int nh, int vph, int64_t capacity,
                                                                 u32x4* __restrict__ cache) {
  const int64_t row_vec = (int64_t)3 * nh * vph;  // vectors per qkv row
  const int per_tok = 2 * nh * vph;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int b = seq_of(cu, B, t);
    const int64_t slot = (int64_t)arg.slot_base[b] + arg.ctx_len[b] + (t - cu[b]);
    const u32x4* src = qkv + t * row_vec + (int64_t)nh * vph;  // k | v of this token
    for (int i = threadIdx.x; i < per_tok; i += kExtendThreads) {
      const int kv = i / (nh * vph), r = i - kv * nh * vph;
      const int h = r / vph, c = r - h * vph;
      cache[(((int64_t)kv * nh + h) * capacity + slot) * vph + c] = src[i];
    }
  }
}

template <typename T>
struct Vec8;  // 8 consecutive elements as one or two 16-byte loads
template <>
struct Vec8<f16> {
  __device__ static void load(const f16* p, float (&o)[8]) {
    const half8 v = *reinterpret_cast<const half8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
  }
};
template <>
struct Vec8<float> {
  __device__ static void load(const float* p, float (&o)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x, o[1] = a.y, o[2] = a.z, o[3] = a.w, o[4] = b.x, o[5] = b.y, o[6] = b.z, o[7] = b.w;
  }
};

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float o = __shfl_xor(v, d, kWave);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();  // red may still be read from the previous reduction
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kExtendThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// Attention of the new tokens over the cache.  One workgroup per (head,
// sequence); the new queries of the sequence one after another, query i at
// position p = ctx + i seeing keys 0..p (causal).
//   scores: a key is read by LPK lanes at 8 elements each (a whole row per
//           lane group, coalesced), partial dot products summed by shuffles;
//           scores go to LDS (dynamic, >= p + 1 floats);
//   softmax: block max and sum; exp(s - max) in place;
//   P.V:    the same key partition: a lane group reads a key's V row in
//           16-byte chunks and accumulates its 8 dims; shuffles sum the key
//           groups of a wave, LDS the four waves.
template <typename T, int HD>
__global__ __launch_bounds__(kExtendThreads) void cache_attention_kernel(const T* __restrict__ qkv, ExtendArg arg,
                                                                       const int32_t* __restrict__ cu, int nh,
                                                                       int64_t capacity, const T* __restrict__ kc,
                                                                       const T* __restrict__ vc, T* __restrict__ o) {
  constexpr int LPK = HD / 8;            // lanes per key row
  constexpr int KPW = 64 / LPK;          // keys per wave per pass
  constexpr int NW = kExtendThreads / 64;
  static_assert(64 % LPK == 0, "a key row must be split over a power-of-two lane group");
  extern __shared__ float smem[];
  float* red = smem;                       // NW floats
  float* part = smem + NW;                 // NW * HD floats
  float* scores = part + NW * HD;          // >= max position + 1 floats
  const int h = blockIdx.x, b = blockIdx.y;
  const int n_new = arg.new_len[b];
  if (n_new == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Hp = nh * HD;
  const int64_t row_len = 3 * (int64_t)Hp;
  const T* K = kc + ((int64_t)h * capacity + arg.slot_base[b]) * HD;
  const T* V = vc + ((int64_t)h * capacity + arg.slot_base[b]) * HD;
  const float scale = 1.0f / sqrtf((float)HD);
  const int g = lane / LPK, c = lane % LPK;  // key within the wave's pass, chunk of the row

  for (int i = 0; i < n_new; ++i) {
    const int64_t row = cu[b] + i;
    const int nk = arg.ctx_len[b] + i + 1;
    float q[8];
    Vec8<T>::load(qkv + row * row_len + h * HD + c * 8, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] *= scale;
    float m = -INFINITY;
    for (int j0 = wave * KPW; j0 < nk; j0 += NW * KPW) {
      const int j = j0 + g;
      float s = 0.f;
      if (j < nk) {
        float k[8];
        Vec8<T>::load(K + (int64_t)j * HD + c * 8, k);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += q[e] * k[e];
      }
#pragma unroll
      for (int d = LPK / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d, kWave);
      if (j < nk) {
        if (c == 0) scores[j] = s;
        m = fmaxf(m, s);
      }
    }
    m = block_reduce(m, true, red);
    float l = 0.f;
    for (int j = threadIdx.x; j < nk; j += kExtendThreads) {
      const float e = __builtin_amdgcn_exp2f((scores[j] - m) * kLog2e);
      scores[j] = e;
      l += e;
    }
    l = block_reduce(l, false, red);  // its barriers also publish the exponentials
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int j0 = wave * KPW; j0 < nk; j0 += NW * KPW) {
      const int j = j0 + g;
      if (j < nk) {
        const float pj = scores[j];
        float v[8];
        Vec8<T>::load(V + (int64_t)j * HD + c * 8, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += pj * v[e];
      }
    }
#pragma unroll
    for (int d = LPK; d < 64; d <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], d, kWave);
    if (g == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) part[wave * HD + c * 8 + e] = acc[e];
    __syncthreads();
    for (int d = threadIdx.x; d < HD; d += kExtendThreads) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += part[w * HD + d];
      o[row * Hp + h * HD + d] = (T)(s / l);
    }
    __syncthreads();  // scores and part are rewritten by the next query
  }
}

template <typename T, int HD>
hipError_t launch_cache_attn_t(const void* qkv, const ExtendArg& arg, const int32_t* cu, int B, int nh,
                               int max_pos, int64_t capacity, const void* kc, const void* vc, void* o, hipStream_t s) {
  const size_t lds = sizeof(float) * ((size_t)(kExtendThreads / 64) * (HD + 1) + (size_t)max_pos);
  hipLaunchKernelGGL((cache_attention_kernel<T, HD>), dim3(nh, B), dim3(kExtendThreads), lds, s,
                     static_cast<const T*>(qkv), arg, cu, nh, capacity, static_cast<const T*>(kc),
                     static_cast<const T*>(vc), static_cast<T*>(o));
  return hipGetLastError();
}

}  // namespace

bool cache_attention_ok(int head_dim) {
  return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128;
}

// scores of one query (4 bytes per position) plus the partial sums stay
// within 64 KiB of dynamic LDS
int cache_attention_max_positions() { return 15360; }

hipError_t launch_extend_cu(const ExtendArg& arg, int B, int32_t* cu, hipStream_t s) {
  hipLaunchKernelGGL(extend_cu_kernel, dim3(1), dim3(64), 0, s, arg, B, cu);
  return hipGetLastError();
}

hipError_t launch_append_kv(const void* qkv, const ExtendArg& arg, const int32_t* cu, int B, int64_t T, int nh,
                            int head_bytes, int64_t capacity, void* cache, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(T < 65536 ? T : 65536);
  hipLaunchKernelGGL(append_kv_kernel, dim3(grid), dim3(kExtendThreads), 0, s, static_cast<const u32x4*>(qkv), arg,
                     cu, B, T, nh, head_bytes / 16, capacity, static_cast<u32x4*>(cache));
  return hipGetLastError();
}

hipError_t launch_cache_attention(ee_dtype dt, const void* qkv, const ExtendArg& arg, const int32_t* cu, int B,
                                  int nh, int hd, int max_pos, int64_t capacity, const void* kc, const void* vc,
                                  void* o, hipStream_t s) {
#define EE_CACHE_ATTN(HDV)                                                                                     \
  if (hd == HDV)                                                                                               \
    return dt == EE_F16 ? launch_cache_attn_t<f16, HDV>(qkv, arg, cu, B, nh, max_pos, capacity, kc, vc, o, s) \
                        : launch_cache_attn_t<float, HDV>(qkv, arg, cu, B, nh, max_pos, capacity, kc, vc, o, s);
  EE_CACHE_ATTN(16)
  EE_CACHE_ATTN(32)
  EE_CACHE_ATTN(64)
  EE_CACHE_ATTN(128)
#undef EE_CACHE_ATTN
  return hipErrorInvalidValue;
}

}  // namespace ee
