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
#include <algorithm>
#include <climits>

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

// Running softmax state of one query over a set of keys, in the exp2
// domain (scores pre-multiplied by log2(e) / sqrt(head_dim)): m = the largest
// score, l = sum of 2^(s - m), acc = sum of 2^(s - m) v.  An empty set is
// (-inf, 0, 0).  Merging rescales both sides to the larger maximum.
__device__ __forceinline__ float rescale(float m, float to) { return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - to); }

// Attention of the new tokens over the cache, split over key chunks.  One
// workgroup per (chunk, head, new token): query t of sequence b at position
// p = ctx + i sees keys 0..p; the chunk is keys [c*chunk, (c+1)*chunk) of
// those.  A lane group of LPK = HD/8 lanes reads a key row (8 elements per
// lane, coalesced) and owns 8 dims of the output; the groups step through the
// chunk KB keys at a time with an online softmax (one rescale per block of
// KB keys), so no score buffer is kept and the context is not limited by LDS.
// The groups' states are merged by shuffles, the four waves' in LDS.  With
// one chunk (FINAL) the normalised output is stored directly; otherwise the
// chunk's (m, l, acc[HD]) go to `part`, and cache_attn_merge_kernel combines
// the chunks.
template <typename T, int HD, bool FINAL>
__global__ __launch_bounds__(kExtendThreads) void cache_attn_chunk_kernel(
    const T* __restrict__ qkv, ExtendArg arg, const int32_t* __restrict__ cu, int B, int64_t T_new, int nh,
    int64_t capacity, const T* __restrict__ kc, const T* __restrict__ vc, int chunk, int n_chunks,
    float* __restrict__ part, T* __restrict__ o) {
  constexpr int LPK = HD / 8;            // lanes per key row
  constexpr int GPW = 64 / LPK;          // lane groups per wave
  constexpr int NW = kExtendThreads / 64;
  constexpr int G = NW * GPW;            // lane groups per workgroup
  constexpr int KB = 4;                  // keys per lane group per step
  static_assert(64 % LPK == 0, "a key row must be split over a power-of-two lane group");
  __shared__ float red[NW][HD + 2];
  const int c = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gl = lane / LPK, ch = lane % LPK;
  const int grp = wave * GPW + gl;
  const int Hp = nh * HD;
  const float qscale = kLog2e / sqrtf((float)HD);
  for (int64_t t = blockIdx.z; t < T_new; t += gridDim.z) {
    const int b = seq_of(cu, B, t);
    const int nk = arg.ctx_len[b] + (int)(t - cu[b]) + 1;
    const int k0 = c * chunk;
    const int k1 = min(nk, k0 + chunk);
    const T* K = kc + ((int64_t)h * capacity + arg.slot_base[b]) * HD + ch * 8;
    const T* V = vc + ((int64_t)h * capacity + arg.slot_base[b]) * HD + ch * 8;
    float q[8];
    Vec8<T>::load(qkv + t * 3 * (int64_t)Hp + h * HD + ch * 8, q);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] *= qscale;
    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    // every lane of a group runs the same trip count, so the shuffles below
    // never straddle a branch
    for (int j0 = k0 + grp * KB; j0 < k1; j0 += G * KB) {
      float s[KB];
      float mb = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int j = j0 + kk;
        float d = 0.f;
        if (j < k1) {
          float k[8];
          Vec8<T>::load(K + (int64_t)j * HD, k);
#pragma unroll
          for (int e = 0; e < 8; ++e) d += q[e] * k[e];
        }
#pragma unroll
        for (int x = LPK / 2; x >= 1; x >>= 1) d += __shfl_xor(d, x, kWave);
        s[kk] = j < k1 ? d : -INFINITY;
        mb = fmaxf(mb, s[kk]);
      }
      const float mn = fmaxf(m, mb);  // finite: key j0 < k1 is in the block
      const float r = rescale(m, mn);
      l *= r;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= r;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int j = j0 + kk;
        if (j < k1) {
          const float pj = __builtin_amdgcn_exp2f(s[kk] - mn);
          float v[8];
          Vec8<T>::load(V + (int64_t)j * HD, v);
          l += pj;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += pj * v[e];
        }
      }
      m = mn;
    }
    // the lane groups of a wave
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) {
      const float mo = __shfl_xor(m, x, kWave), lo = __shfl_xor(l, x, kWave);
      float ao[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ao[e] = __shfl_xor(acc[e], x, kWave);
      const float mn = fmaxf(m, mo);
      const float ra = rescale(m, mn), rb = rescale(mo, mn);
      l = l * ra + lo * rb;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] * ra + ao[e] * rb;
      m = mn;
    }
    if (gl == 0) {
      if (ch == 0) {
        red[wave][0] = m;
        red[wave][1] = l;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][2 + ch * 8 + e] = acc[e];
    }
    __syncthreads();
    for (int d = threadIdx.x; d < HD; d += kExtendThreads) {
      float M = red[0][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, red[w][0]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = rescale(red[w][0], M);
        L += red[w][1] * f;
        A += red[w][2 + d] * f;
      }
      if constexpr (FINAL) {
        o[t * Hp + h * HD + d] = from_f32<T>(A / L);
      } else {
        float* pp = part + ((t * nh + h) * (int64_t)n_chunks + c) * (HD + 2);
        if (d == 0) {
          pp[0] = M;
          pp[1] = L;
        }
        pp[2 + d] = A;
      }
    }
    __syncthreads();  // red is rewritten for the next token
  }
}

// o = the chunks' states of one (token, head) merged: rescaled to the
// largest maximum, summed in chunk order, normalised.
template <typename T, int HD>
__global__ __launch_bounds__(HD) void cache_attn_merge_kernel(const float* __restrict__ part, int64_t T_new, int nh,
                                                              int n_chunks, T* __restrict__ o) {
  const int h = blockIdx.x, d = threadIdx.x;
  for (int64_t t = blockIdx.y; t < T_new; t += gridDim.y) {
    const float* pp = part + (t * nh + h) * (int64_t)n_chunks * (HD + 2);
    float M = -INFINITY;
    for (int c = 0; c < n_chunks; ++c) M = fmaxf(M, pp[(int64_t)c * (HD + 2)]);
    float L = 0.f, A = 0.f;
    for (int c = 0; c < n_chunks; ++c) {
      const float* q = pp + (int64_t)c * (HD + 2);
      const float f = rescale(q[0], M);
      L += q[1] * f;
      A += q[2 + d] * f;
    }
    o[t * (int64_t)nh * HD + h * HD + d] = from_f32<T>(A / L);
  }
}

template <typename T, int HD>
hipError_t launch_cache_attn_t(const void* qkv, const ExtendArg& arg, const int32_t* cu, int B, int64_t T_new, int nh,
                               int max_pos, int64_t capacity, const void* kc, const void* vc, void* o, void* scratch,
                               size_t scratch_bytes, hipStream_t s) {
  const CacheAttnPlan p = cache_attention_plan(T_new, nh, HD, max_pos, scratch_bytes);
  if (p.n_chunks < 1) return hipErrorInvalidValue;
  const unsigned gz = (unsigned)(T_new < 65535 ? T_new : 65535);
  const T* q = static_cast<const T*>(qkv);
  const T* k = static_cast<const T*>(kc);
  const T* v = static_cast<const T*>(vc);
  T* out = static_cast<T*>(o);
  float* part = static_cast<float*>(scratch);
  if (p.n_chunks == 1) {
    hipLaunchKernelGGL((cache_attn_chunk_kernel<T, HD, true>), dim3(1, nh, gz), dim3(kExtendThreads), 0, s, q, arg, cu,
                       B, T_new, nh, capacity, k, v, p.chunk, 1, nullptr, out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((cache_attn_chunk_kernel<T, HD, false>), dim3(p.n_chunks, nh, gz), dim3(kExtendThreads), 0, s, q,
                     arg, cu, B, T_new, nh, capacity, k, v, p.chunk, p.n_chunks, part, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((cache_attn_merge_kernel<T, HD>), dim3(nh, gz), dim3(HD), 0, s, part, T_new, nh, p.n_chunks,
                     out);
  return hipGetLastError();
}

}  // namespace

bool cache_attention_ok(int head_dim) {
  return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128;
}

// The cache attention keeps no per-position buffer, so the context is bounded
// only by the cache's 32-bit slot range.
int cache_attention_max_positions() { return INT32_MAX; }

CacheAttnPlan cache_attention_plan(int64_t T_new, int nh, int hd, int max_pos, size_t scratch_bytes) {
  CacheAttnPlan p{0, 0};
  if (T_new < 1 || nh < 1 || max_pos < 1) return p;
  const double per_chunk = (double)T_new * nh * (hd + 2) * 4.0;  // partial-state bytes per chunk
  int64_t chunk = kCacheAttnChunk;
  int64_t n = (max_pos + chunk - 1) / chunk;
  while (n > 1 && (double)n * per_chunk > (double)scratch_bytes) {
    chunk *= 2;
    n = (max_pos + chunk - 1) / chunk;
  }
  if (n > 1 && (double)n * per_chunk > (double)scratch_bytes) return p;
  p.chunk = (int)std::min<int64_t>(chunk, INT32_MAX);
  p.n_chunks = (int)n;
  return p;
}

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
                                  int64_t T_new, int nh, int hd, int max_pos, int64_t capacity, const void* kc,
                                  const void* vc, void* o, void* scratch, size_t scratch_bytes, hipStream_t s) {
#define EE_CACHE_ATTN(HDV)                                                                                         \
  if (hd == HDV)                                                                                                   \
    return dt == EE_F16 ? launch_cache_attn_t<f16, HDV>(qkv, arg, cu, B, T_new, nh, max_pos, capacity, kc, vc, o,  \
                                                        scratch, scratch_bytes, s)                                 \
                        : launch_cache_attn_t<float, HDV>(qkv, arg, cu, B, T_new, nh, max_pos, capacity, kc, vc, o, \
                                                          scratch, scratch_bytes, s);
  EE_CACHE_ATTN(16)
  EE_CACHE_ATTN(32)
  EE_CACHE_ATTN(64)
  EE_CACHE_ATTN(128)
#undef EE_CACHE_ATTN
  return hipErrorInvalidValue;
}

}  // namespace ee
