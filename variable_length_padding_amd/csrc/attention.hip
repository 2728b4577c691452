// Causal self-attention run per sequence over the packed token offsets: query i
// of sequence b attends to keys cu[b] .. cu[b]+i with weights
// softmax(q.k / sqrt(head_dim)).  Packing means no query or key of padding
// exists at all; sequences never see each other.  (The pages give no
// attention kernel; the packed layout follows from removing the padding for
// the whole layer, the announcement article's "Runtime" section.)
//
// fp16, head_dim in {32, 64, 128}: the MFMA kernel.  A workgroup owns 128
// queries of one (sequence, head); each of its 4 waves owns 32 queries and
// keeps an online softmax per query.  Keys and values are staged through LDS
// 32 at a time: K row-major (chunk-swizzled), V transposed to [d][key].
//   S^T = K . Q^T   (v_mfma_f32_32x32x16_f16, A = K tile, B = Q^T from registers)
// puts one query per lane column, so the softmax max/sum of a query is an
// in-lane reduction plus one exchange with lane l^32, and the rescale of the
// output accumulator is per lane.  The probabilities are rounded to fp16 and
// used in place as the B operand of
//   O^T += V^T . P^T
// whose A operand is read from the transposed V tile in the key order the S^T
// accumulator layout produced.
//
// Any other case (fp32, head_dim 16): a vector-ALU kernel, one query per lane.
#include "device_common.h"
#include "internal.h"

namespace ee {
namespace {

constexpr int kQB = 128;  // queries per workgroup (MFMA kernel)
constexpr int kKB = 32;   // keys per LDS tile
constexpr int kVtPitch = kKB + 4;  // halves per transposed-V row: 72 B, 8-byte aligned, conflict-free b64 reads

template <int HD>
__device__ __forceinline__ int k_swizzle(int r) {
  constexpr int KCH = HD / 8;  // 16-byte chunks per key row
  if (KCH >= 16) return r & 15;
  if (KCH == 8) return ((r >> 1) & 7) ^ ((r & 1) << 2);
  return r & (KCH - 1);
}

template <int HD>
__global__ __launch_bounds__(256) void attn_mfma_kernel(const f16* __restrict__ qkv, const int32_t* __restrict__ cu,
                                                        int nh, float scale_log2, f16* __restrict__ o) {
  constexpr int KCH = HD / 8;
  constexpr int NKK = HD / 16;  // MFMA K steps for S
  constexpr int NDB = HD / 32;  // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) f16 sK[kKB * HD];
  __shared__ __attribute__((aligned(16))) f16 sVt[HD * kVtPitch];

  const int b = blockIdx.y, head = blockIdx.z;
  const int s0 = cu[b];
  const int L = cu[b + 1] - s0;
  const int q_start = blockIdx.x * kQB;
  if (q_start >= L) return;  // uniform over the workgroup
  const int Hp = nh * HD, ld = 3 * Hp;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, hk = lane >> 5;
  const int q0 = q_start + wave * 32;
  const int qi = q0 + (lane & 31);
  const int qc = min(qi, L - 1);

  half8 qf[NKK];
  {
    const f16* qrow = qkv + (int64_t)(s0 + qc) * ld + head * HD + hk * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const half8*>(qrow + kk * 16);
  }
  floatx16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = min(L, q_start + kQB);
  const int wave_last_q = min(q0 + 31, L - 1);
  const int kswz = k_swizzle<HD>(lane & 31);

  for (int k0 = 0; k0 < kend; k0 += kKB) {
    for (int c = t; c < kKB * KCH; c += 256) {
      const int r = c / KCH, ch = c % KCH;
      const int key = min(k0 + r, L - 1);
      const f16* base = qkv + (int64_t)(s0 + key) * ld + head * HD + ch * 8;
      const half8 kv = *reinterpret_cast<const half8*>(base + Hp);
      const half8 vv = *reinterpret_cast<const half8*>(base + 2 * Hp);
      *reinterpret_cast<half8*>(sK + r * HD + ((ch ^ k_swizzle<HD>(r)) * 8)) = kv;
#pragma unroll
      for (int i = 0; i < 8; ++i) sVt[(ch * 8 + i) * kVtPitch + r] = vv[i];
    }
    __syncthreads();
    if (k0 <= wave_last_q) {
      floatx16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const half8 kf =
            *reinterpret_cast<const half8*>(sK + (lane & 31) * HD + (((kk * 2 + hk) ^ kswz) * 8));
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[kk], s, 0, 0, 0);
      }
      // element e: key k0 + (e/4)*8 + hk*4 + e%4, query qi
      float mloc = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + (e >> 2) * 8 + hk * 4 + (e & 3);
        const float v = key <= qi ? s[e] * scale_log2 : -INFINITY;
        s[e] = v;
        mloc = fmaxf(mloc, v);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
      const float m_new = fmaxf(m_run, mloc);  // finite: the first tile holds key 0 <= qi
      const float alpha = exp2f(m_run - m_new);
      half8 p0, p1;
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p0[e] = (f16)exp2f(s[e] - m_new);
        p1[e] = (f16)exp2f(s[8 + e] - m_new);
        rs += (float)p0[e] + (float)p1[e];
      }
      rs += __shfl_xor(rs, 32, kWave);
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
        const f16* vrow = sVt + (d * 32 + (lane & 31)) * kVtPitch + hk * 4;
        const half4 a0 = *reinterpret_cast<const half4*>(vrow);
        const half4 a1 = *reinterpret_cast<const half4*>(vrow + 8);
        const half4 a2 = *reinterpret_cast<const half4*>(vrow + 16);
        const half4 a3 = *reinterpret_cast<const half4*>(vrow + 24);
        const half8 va = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const half8 vb = {a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, p0, oacc[d], 0, 0, 0);
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb, p1, oacc[d], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (qi < L) {
    const float inv = 1.0f / l_run;
    f16* orow = o + (int64_t)(s0 + qi) * Hp + head * HD + hk * 4;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        half4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (f16)(oacc[d][g * 4 + e] * inv);
        *reinterpret_cast<half4*>(orow + d * 32 + g * 8) = w;
      }
  }
}

// ---- vector-ALU fallback: one query per lane, 64 queries per workgroup ----
constexpr int kVQ = 64;

template <typename T, int HD>
__global__ __launch_bounds__(kVQ) void attn_valu_kernel(const T* __restrict__ qkv, const int32_t* __restrict__ cu,
                                                        int nh, float scale, T* __restrict__ o) {
  __shared__ float sK[kVQ][HD + 1];
  __shared__ float sV[kVQ][HD + 1];
  const int b = blockIdx.y, head = blockIdx.z;
  const int s0 = cu[b];
  const int L = cu[b + 1] - s0;
  const int q_start = blockIdx.x * kVQ;
  if (q_start >= L) return;
  const int Hp = nh * HD, ld = 3 * Hp;
  const int qi = q_start + (int)threadIdx.x;
  float q[HD], acc[HD];
  const T* qrow = qkv + (int64_t)(s0 + min(qi, L - 1)) * ld + head * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    q[d] = to_f32(qrow[d]);
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kend = min(L, q_start + kVQ);
  for (int k0 = 0; k0 < kend; k0 += kVQ) {
    for (int idx = threadIdx.x; idx < kVQ * HD; idx += kVQ) {
      const int r = idx / HD, d = idx % HD;
      const T* base = qkv + (int64_t)(s0 + min(k0 + r, L - 1)) * ld + head * HD + d;
      sK[r][d] = to_f32(base[Hp]);
      sV[r][d] = to_f32(base[2 * Hp]);
    }
    __syncthreads();
    const int jn = min(kVQ, qi - k0 + 1);
    for (int j = 0; j < jn; ++j) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < HD; ++d) s = fmaf(q[d], sK[j][d], s);
      s *= scale;
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn);
      const float p = expf(s - mn);
      l = l * a + p;
#pragma unroll
      for (int d = 0; d < HD; ++d) acc[d] = acc[d] * a + p * sV[j][d];
      m = mn;
    }
    __syncthreads();
  }
  if (qi < L) {
    T* orow = o + (int64_t)(s0 + qi) * Hp + head * HD;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < HD; ++d) orow[d] = from_f32<T>(acc[d] * inv);
  }
}

template <typename T>
hipError_t launch_valu(const void* qkv, const int32_t* cu, int B, int max_len, int nh, int hd, void* o,
                       hipStream_t s) {
  const dim3 grid((unsigned)((max_len + kVQ - 1) / kVQ), (unsigned)B, (unsigned)nh), block(kVQ);
  const float scale = 1.0f / sqrtf((float)hd);
  const T* q = static_cast<const T*>(qkv);
  T* out = static_cast<T*>(o);
  switch (hd) {
    case 16: hipLaunchKernelGGL((attn_valu_kernel<T, 16>), grid, block, 0, s, q, cu, nh, scale, out); break;
    case 32: hipLaunchKernelGGL((attn_valu_kernel<T, 32>), grid, block, 0, s, q, cu, nh, scale, out); break;
    case 64: hipLaunchKernelGGL((attn_valu_kernel<T, 64>), grid, block, 0, s, q, cu, nh, scale, out); break;
    default: hipLaunchKernelGGL((attn_valu_kernel<T, 128>), grid, block, 0, s, q, cu, nh, scale, out); break;
  }
  return hipGetLastError();
}

}  // namespace

bool attention_mfma_ok(ee_dtype dt, int hd) { return dt == EE_F16 && (hd == 32 || hd == 64 || hd == 128); }

hipError_t launch_attention(ee_dtype dt, const void* qkv, const int32_t* cu, int B, int max_len, int nh, int hd,
                            void* o, hipStream_t s) {
  if (B <= 0 || max_len <= 0) return hipSuccess;
  if (attention_mfma_ok(dt, hd)) {
    const dim3 grid((unsigned)((max_len + kQB - 1) / kQB), (unsigned)B, (unsigned)nh), block(256);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)hd);  // log2(e) / sqrt(hd)
    const f16* q = static_cast<const f16*>(qkv);
    f16* out = static_cast<f16*>(o);
    switch (hd) {
      case 32: hipLaunchKernelGGL((attn_mfma_kernel<32>), grid, block, 0, s, q, cu, nh, scale_log2, out); break;
      case 64: hipLaunchKernelGGL((attn_mfma_kernel<64>), grid, block, 0, s, q, cu, nh, scale_log2, out); break;
      default: hipLaunchKernelGGL((attn_mfma_kernel<128>), grid, block, 0, s, q, cu, nh, scale_log2, out); break;
    }
    return hipGetLastError();
  }
  return dt == EE_F16 ? launch_valu<f16>(qkv, cu, B, max_len, nh, hd, o, s)
                      : launch_valu<float>(qkv, cu, B, max_len, nh, hd, o, s);
}

}  // namespace ee
