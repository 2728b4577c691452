// Self-attention run per sequence: query i of sequence b attends, with weights
// softmax(q.k / sqrt(head_dim)), to keys 0..i of its sequence (causal, the GPT
// decoder) or to all of its sequence's keys (bidirectional, the BERT-style
// encoder).  Rows are read either from the packed q|k|v buffer over the token
// offsets cu, or from padded head-major [B, nh, P, hd] tensors (the
// page-literal form, with lengths still from cu).  Packing means no query or key of padding
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
#include <type_traits>

#include "device_common.h"
#include "attention_limits.h"
#include "internal.h"
#include "lds_dma.h"

namespace ee {
namespace {

constexpr int kQB = 128;  // queries per workgroup (MFMA kernel)
constexpr int kKB = kAttnKeyTile;   // keys per LDS tile
constexpr int kVtPitch = kKB + 4;  // halves per transposed-V row: 72 B, 8-byte aligned, conflict-free b64 reads

// Where the rows of q, k, v and o live.  Row `row` of (sequence b, head h) of
// tensor X sits at X + (seq ? cu[b] : 0) * row_stride + b * batch_stride
// + h * head_stride + row * row_stride (elements).  Packed q|k|v rows:
// seq = 1, batch_stride = 0, head_stride = hd, row_stride = 3H' (o: H').
// Padded head-major [B, nh, P, hd]: seq = 0, batch_stride = nh*P*hd,
// head_stride = P*hd, row_stride = hd.  Lengths always come from cu.
struct AttnAddr {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t in_batch_stride, in_head_stride, in_row_stride;
  int64_t out_batch_stride, out_head_stride, out_row_stride;
  int seq;
};

template <int HD>
__device__ __forceinline__ int k_swizzle(int r) {
  constexpr int KCH = HD / 8;  // 16-byte chunks per key row
  if (KCH >= 16) return r & 15;
  if (KCH == 8) return ((r >> 1) & 7) ^ ((r & 1) << 2);
  return r & (KCH - 1);
}

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_mfma_kernel(AttnAddr ad, const int32_t* __restrict__ cu,
                                                        float scale_log2) {
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
  const int64_t in_base = (ad.seq ? (int64_t)s0 * ad.in_row_stride : 0) + b * ad.in_batch_stride + head * ad.in_head_stride;
  const int64_t ld = ad.in_row_stride;
  const f16* qb = static_cast<const f16*>(ad.q) + in_base;
  const f16* kb = static_cast<const f16*>(ad.k) + in_base;
  const f16* vb = static_cast<const f16*>(ad.v) + in_base;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, hk = lane >> 5;
  const int q0 = q_start + wave * 32;
  const int qi = q0 + (lane & 31);
  const int qc = min(qi, L - 1);

  half8 qf[NKK];
  {
    const f16* qrow = qb + qc * ld + hk * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const half8*>(qrow + kk * 16);
  }
  floatx16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // keys this workgroup needs: up to its last query (causal) or all of them
  const int kend = CAUSAL ? min(L, q_start + kQB) : L;
  const int wave_last_key = CAUSAL ? min(q0 + 31, L - 1) : L - 1;
  const bool wave_active = q0 < L;
  const int kswz = k_swizzle<HD>(lane & 31);

  for (int k0 = 0; k0 < kend; k0 += kKB) {
    for (int c = t; c < kKB * KCH; c += 256) {
      const int r = c / KCH, ch = c % KCH;
      const int64_t key_off = (int64_t)min(k0 + r, L - 1) * ld + ch * 8;
      const half8 kv = *reinterpret_cast<const half8*>(kb + key_off);
      const half8 vv = *reinterpret_cast<const half8*>(vb + key_off);
      *reinterpret_cast<half8*>(sK + r * HD + ((ch ^ k_swizzle<HD>(r)) * 8)) = kv;
#pragma unroll
      for (int i = 0; i < 8; ++i) sVt[(ch * 8 + i) * kVtPitch + r] = vv[i];
    }
    __syncthreads();
    if (wave_active && k0 <= wave_last_key) {
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
        const bool keep = CAUSAL ? key <= qi : key < L;
        const float v = keep ? s[e] * scale_log2 : -INFINITY;
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
        const half8 v_lo = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const half8 v_hi = {a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v_lo, p0, oacc[d], 0, 0, 0);
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v_hi, p1, oacc[d], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (qi < L) {
    const float inv = 1.0f / l_run;
    f16* orow = static_cast<f16*>(ad.o) + (ad.seq ? (int64_t)s0 * ad.out_row_stride : 0) + b * ad.out_batch_stride +
                head * ad.out_head_stride + (int64_t)qi * ad.out_row_stride + hk * 4;
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

// ---- head_dim 64 / 128: the same algorithm, K and V double-buffered ----
// Tile t+1 of K and V is fetched into registers (16-byte buffer loads) while
// tile t is multiplied, then written to the other LDS stage; both are stored
// row-major with the chunk swizzle k_swizzle, so the writes are 16-byte and
// conflict-free.  The A operand of O^T += V^T . P^T (row d of V^T, 8 keys)
// comes from two transposing LDS reads (ds_read_b64_tr_b16): within each
// 16-lane group, element j of lane i is element i % 4 of the 8 bytes that
// lane 4j + i / 4 of the group addresses.  Each lane therefore addresses key
// (lane % 16) / 4 of its 4-key slice at d = 4 * (lane % 4) of its 16-wide d
// slice and receives 4 keys of one d: no transposing LDS writes.  (Direct-to-
// LDS loads are not used here: the compiler waits for every one in flight
// before a transposing read.)  Key rows past the sequence are left to the
// buffer descriptor, which ends at its last row: the row offset travels in the
// lane offset (the range check does not cover the scalar offset), so those
// rows load as zeros and their scores are masked.
template <int HD>
__device__ __forceinline__ half4 tr_read(const f16* p) {
  typedef short short4_t __attribute__((ext_vector_type(4)));
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
  return __builtin_bit_cast(half4, v);
}

// Growth of a row's maximum (exp2 units) that the softmax of attn_tr_kernel
// absorbs before it rescales: probabilities stay below 2^8.
constexpr float kAttnSlack = 8.0f;

// Waves per SIMD the register budget is sized for.  Three (166 VGPRs at
// head_dim 128) ran at the same speed as two on the GPT-3 shapes; four spills.
#ifndef EE_ATTN_WAVES_PER_SIMD
#define EE_ATTN_WAVES_PER_SIMD 2
#endif

// The keys and values of an extend step (new tokens after cached ones) come
// from the packed KV cache: sequence b's keys 0 .. ctx_len[b] + new_len[b] - 1
// sit at slots slot_base[b] + j of each head's [capacity, hd] block, the new
// tokens' own keys already appended; its new queries are the packed q rows
// cu[b] .. cu[b+1] - 1, query i at position ctx_len[b] + i.
struct NoCache {};
struct CacheKV {
  ExtendArg arg;
  const f16* kc;
  const f16* vc;
  int64_t capacity;
};

template <int HD, bool CAUSAL, class KV = NoCache>
__global__ __launch_bounds__(256, EE_ATTN_WAVES_PER_SIMD) void attn_tr_kernel(AttnAddr ad, const int32_t* __restrict__ cu,
                                                       float scale_log2, KV kv = KV{}) {
  constexpr bool EXT = !std::is_same<KV, NoCache>::value;
  constexpr int KCH = HD / 8;          // 16-byte chunks per key row
  constexpr int RPL = 64 / KCH;        // rows one wave covers per 16-byte access
  constexpr int NLQ = kKB / 4 / RPL;   // accesses per wave per matrix per tile (8 rows per wave)
  constexpr int NKK = HD / 16;         // MFMA K steps for S
  constexpr int NDB = HD / 32;         // 32-row blocks of O^T
  constexpr int TILE = kKB * HD;       // halves per matrix per stage
  static_assert(HD == 64 || HD == 128, "head_dim 64 or 128");
  __shared__ __attribute__((aligned(16))) f16 smem[2 * 2 * TILE];  // [stage][K | V]

  // grid (query tiles, heads, sequences): the workgroups of one sequence's
  // heads run together, so each packed row is read in one stretch of time
  const int b = blockIdx.z, head = blockIdx.y;
  const int s0 = cu[b];
  const int L = cu[b + 1] - s0;  // queries (all the sequence's rows, or its new tokens)
  const int q_start = blockIdx.x * kQB;
  if (q_start >= L) return;  // uniform over the workgroup
  const int64_t in_base = (ad.seq ? (int64_t)s0 * ad.in_row_stride : 0) + b * ad.in_batch_stride + head * ad.in_head_stride;
  const int ldq = (int)ad.in_row_stride;
  const f16* qb = static_cast<const f16*>(ad.q) + in_base;
  // keys: the same rows as the queries, or the cached context and then the new tokens
  int ctx = 0, Lk = L, ld = ldq;
  const f16* kbase = static_cast<const f16*>(ad.k) + in_base;
  const f16* vbase = static_cast<const f16*>(ad.v) + in_base;
  if constexpr (EXT) {
    ctx = kv.arg.ctx_len[b];
    Lk = ctx + L;
    ld = HD;
    const int64_t kv_off = ((int64_t)head * kv.capacity + kv.arg.slot_base[b]) * HD;
    kbase = kv.kc + kv_off;
    vbase = kv.vc + kv_off;
  }
  const int t = threadIdx.x, lane = t & 63, hk = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q0 = q_start + wave * 32;
  const int qi = q0 + (lane & 31);
  const int qc = min(qi, L - 1);
  const int qpos = ctx + qi;  // the query's position: it sees keys 0 .. qpos

  // descriptors over this sequence's rows of k and v (head slice), ending at row Lk
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, Lk * ld * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, Lk * ld * 2, kBufferFlags);
  // this lane's 16 bytes of each access: tile row r, physical chunk lp, which
  // holds the row's logical chunk lp ^ k_swizzle(r)
  const int lr = lane / KCH, lp = lane % KCH;
  int roff[NLQ], lds_off[NLQ];
#pragma unroll
  for (int q = 0; q < NLQ; ++q) {
    const int r = wave * (kKB / 4) + q * RPL + lr;
    roff[q] = r * ld * 2 + ((lp ^ k_swizzle<HD>(r)) * 16);
    lds_off[q] = r * HD + lp * 8;
  }
  u32x4 kn[NLQ], vn[NLQ];
  auto fetch = [&](int k0) {
    const int koff = k0 * ld * 2;
#pragma unroll
    for (int q = 0; q < NLQ; ++q) {
      kn[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, roff[q] + koff, 0, 0));
      vn[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, roff[q] + koff, 0, 0));
    }
  };
  auto stash = [&](int stage) {
    f16* sk = smem + stage * 2 * TILE;
#pragma unroll
    for (int q = 0; q < NLQ; ++q) {
      *reinterpret_cast<u32x4*>(sk + lds_off[q]) = kn[q];
      *reinterpret_cast<u32x4*>(sk + TILE + lds_off[q]) = vn[q];
    }
  };

  half8 qf[NKK];
  {
    const f16* qrow = qb + (int64_t)qc * ldq + hk * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const half8*>(qrow + kk * 16);
  }
  floatx16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[d][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = CAUSAL ? min(Lk, ctx + q_start + kQB) : Lk;
  const int wave_last_key = CAUSAL ? min(ctx + q0 + 31, Lk - 1) : Lk - 1;
  const bool wave_active = q0 < L;
  const int kswz = k_swizzle<HD>(lane & 31);
  // transposing-read address of this lane within a V tile, for key slice
  // base 0 and d block 0: key (lane % 16) / 4 + 4 * hk, d 16 * ((lane / 16) % 2) + 4 * (lane % 4)
  const int tr_key = ((lane & 15) >> 2) + 4 * hk;
  const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  fetch(0);
  stash(0);
  // q's fragments and tile 0 have arrived.  Said as an s_waitcnt the compiler
  // reads: otherwise it keeps counting q's loads as pending inside the loop
  // and waits for the next tile's fetch before the first MFMAs.
  __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
  int stage = 0;
  for (int k0 = 0; k0 < kend; k0 += kKB) {
    // every wave's writes of this tile are visible and every wave is done
    // with the other stage
    __syncthreads();
    const bool more = k0 + kKB < kend;
    if (more) fetch(k0 + kKB);
    const f16* sk = smem + stage * 2 * TILE;
    const f16* sv = sk + TILE;
    if (wave_active && k0 <= wave_last_key) {
      floatx16 sacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const half8 kf = *reinterpret_cast<const half8*>(sk + (lane & 31) * HD + (((kk * 2 + hk) ^ kswz) * 8));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[kk], sacc, 0, 0, 0);
      }
      // element e: key k0 + (e/4)*8 + hk*4 + e%4, query qi
      // Masking only where the tile reaches past the wave's first query
      // (causal) or past the sequence; the scale goes into the exponent's fma.
      // The running maximum m_run (in exp2 units) is raised only when some row
      // of the wave exceeds it by more than kAttnSlack: until then the rows'
      // p = 2^(s - m_run) stay below 2^kAttnSlack (fine in fp16) and the
      // output accumulator is not rescaled.  The final division by l_run
      // cancels whichever maximum was used.
      const bool edge = CAUSAL ? k0 + kKB - 1 > ctx + q0 : k0 + kKB > Lk;
      if (edge) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + (e >> 2) * 8 + hk * 4 + (e & 3);
          if (!(CAUSAL ? key <= qpos : key < Lk)) sacc[e] = -INFINITY;
        }
      }
      float mloc = sacc[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mloc = fmaxf(mloc, sacc[e]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave)) * scale_log2;
      float alpha = 1.f;
      const bool rescale = __any(mloc > m_run + kAttnSlack);
      if (rescale) {
        const float m_new = fmaxf(m_run, mloc);  // finite: the first tile holds key 0 <= qi
        alpha = exp2f(m_run - m_new);
        m_run = m_new;
      }
      half8 p0, p1;
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pa = exp2f(__builtin_fmaf(sacc[e], scale_log2, -m_run));
        const float pb = exp2f(__builtin_fmaf(sacc[8 + e], scale_log2, -m_run));
        p0[e] = (f16)pa;
        p1[e] = (f16)pb;
        rs += pa + pb;
      }
      rs += __shfl_xor(rs, 32, kWave);
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        if (rescale) {
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[d][e] *= alpha;
        }
        // keys 0..15 of the tile (slots: 8h + 4hk + j), then 16..31
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          half4 lo, hi;
          {
            const int key = 16 * m + tr_key, dd = d * 32 + tr_d;
            lo = tr_read<HD>(sv + key * HD + (((dd >> 3) ^ k_swizzle<HD>(key)) * 8) + (dd & 7));
          }
          {
            const int key = 16 * m + 8 + tr_key, dd = d * 32 + tr_d;
            hi = tr_read<HD>(sv + key * HD + (((dd >> 3) ^ k_swizzle<HD>(key)) * 8) + (dd & 7));
          }
          const half8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, m ? p1 : p0, oacc[d], 0, 0, 0);
        }
      }
    }
    if (more) stash(stage ^ 1);
    stage ^= 1;
  }
  if (qi < L) {
    const float inv = 1.0f / l_run;
    f16* orow = static_cast<f16*>(ad.o) + (ad.seq ? (int64_t)s0 * ad.out_row_stride : 0) + b * ad.out_batch_stride +
                head * ad.out_head_stride + (int64_t)qi * ad.out_row_stride + hk * 4;
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

template <typename T, int HD, bool CAUSAL>
__global__ __launch_bounds__(kVQ) void attn_valu_kernel(AttnAddr ad, const int32_t* __restrict__ cu, float scale) {
  __shared__ float sK[kVQ][HD + 1];
  __shared__ float sV[kVQ][HD + 1];
  const int b = blockIdx.y, head = blockIdx.z;
  const int s0 = cu[b];
  const int L = cu[b + 1] - s0;
  const int q_start = blockIdx.x * kVQ;
  if (q_start >= L) return;
  const int64_t in_base = (ad.seq ? (int64_t)s0 * ad.in_row_stride : 0) + b * ad.in_batch_stride + head * ad.in_head_stride;
  const int64_t ld = ad.in_row_stride;
  const T* qb = static_cast<const T*>(ad.q) + in_base;
  const T* kb = static_cast<const T*>(ad.k) + in_base;
  const T* vb = static_cast<const T*>(ad.v) + in_base;
  const int qi = q_start + (int)threadIdx.x;
  float q[HD], acc[HD];
  const T* qrow = qb + min(qi, L - 1) * ld;
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    q[d] = to_f32(qrow[d]);
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kend = CAUSAL ? min(L, q_start + kVQ) : L;
  for (int k0 = 0; k0 < kend; k0 += kVQ) {
    for (int idx = threadIdx.x; idx < kVQ * HD; idx += kVQ) {
      const int r = idx / HD, d = idx % HD;
      const int64_t off = (int64_t)min(k0 + r, L - 1) * ld + d;
      sK[r][d] = to_f32(kb[off]);
      sV[r][d] = to_f32(vb[off]);
    }
    __syncthreads();
    const int jn = CAUSAL ? min(kVQ, qi - k0 + 1) : min(kVQ, L - k0);
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
    T* orow = static_cast<T*>(ad.o) + (ad.seq ? (int64_t)s0 * ad.out_row_stride : 0) + b * ad.out_batch_stride +
              head * ad.out_head_stride + (int64_t)qi * ad.out_row_stride;
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < HD; ++d) orow[d] = from_f32<T>(acc[d] * inv);
  }
}

template <typename T, bool CAUSAL>
void launch_valu(const AttnAddr& ad, const int32_t* cu, int B, int max_len, int nh, int hd, hipStream_t s) {
  const dim3 grid((unsigned)((max_len + kVQ - 1) / kVQ), (unsigned)B, (unsigned)nh), block(kVQ);
  const float scale = 1.0f / sqrtf((float)hd);
  switch (hd) {
    case 16: hipLaunchKernelGGL((attn_valu_kernel<T, 16, CAUSAL>), grid, block, 0, s, ad, cu, scale); break;
    case 32: hipLaunchKernelGGL((attn_valu_kernel<T, 32, CAUSAL>), grid, block, 0, s, ad, cu, scale); break;
    case 64: hipLaunchKernelGGL((attn_valu_kernel<T, 64, CAUSAL>), grid, block, 0, s, ad, cu, scale); break;
    default: hipLaunchKernelGGL((attn_valu_kernel<T, 128, CAUSAL>), grid, block, 0, s, ad, cu, scale); break;
  }
}

template <bool CAUSAL>
void launch_mfma(const AttnAddr& ad, const int32_t* cu, int B, int max_len, int nh, int hd, hipStream_t s) {
  const dim3 grid((unsigned)((max_len + kQB - 1) / kQB), (unsigned)B, (unsigned)nh), block(256);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)hd);  // log2(e) / sqrt(hd)
  // the transposing-read kernel addresses a sequence's rows with 32-bit byte
  // offsets, up to row k0 + kKB - 1 of the last key tile (past the sequence's
  // end: those loads fall outside the descriptor's range and read zeros)
  if ((hd == 64 || hd == 128) && attn_tr_offsets_fit(max_len, ad.in_row_stride)) {
    const dim3 tgrid(grid.x, grid.z, grid.y);  // (query tiles, heads, sequences)
    if (hd == 64) hipLaunchKernelGGL((attn_tr_kernel<64, CAUSAL>), tgrid, block, 0, s, ad, cu, scale_log2);
    else hipLaunchKernelGGL((attn_tr_kernel<128, CAUSAL>), tgrid, block, 0, s, ad, cu, scale_log2);
    return;
  }
  switch (hd) {
    case 32: hipLaunchKernelGGL((attn_mfma_kernel<32, CAUSAL>), grid, block, 0, s, ad, cu, scale_log2); break;
    case 64: hipLaunchKernelGGL((attn_mfma_kernel<64, CAUSAL>), grid, block, 0, s, ad, cu, scale_log2); break;
    default: hipLaunchKernelGGL((attn_mfma_kernel<128, CAUSAL>), grid, block, 0, s, ad, cu, scale_log2); break;
  }
}

hipError_t launch_attn(ee_dtype dt, const AttnAddr& ad, const int32_t* cu, int B, int max_len, int nh, int hd,
                       bool causal, hipStream_t s) {
  if (B <= 0 || max_len <= 0) return hipSuccess;
  if (dt == EE_F16 && (hd == 32 || hd == 64 || hd == 128)) {
    if (causal) launch_mfma<true>(ad, cu, B, max_len, nh, hd, s);
    else launch_mfma<false>(ad, cu, B, max_len, nh, hd, s);
  } else if (dt == EE_F16) {
    if (causal) launch_valu<f16, true>(ad, cu, B, max_len, nh, hd, s);
    else launch_valu<f16, false>(ad, cu, B, max_len, nh, hd, s);
  } else {
    if (causal) launch_valu<float, true>(ad, cu, B, max_len, nh, hd, s);
    else launch_valu<float, false>(ad, cu, B, max_len, nh, hd, s);
  }
  return hipGetLastError();
}

}  // namespace

bool attention_mfma_ok(ee_dtype dt, int hd) { return dt == EE_F16 && (hd == 32 || hd == 64 || hd == 128); }

hipError_t launch_attention(ee_dtype dt, const void* qkv, const int32_t* cu, int B, int max_len, int nh, int hd,
                            bool causal, void* o, hipStream_t s) {
  const int64_t Hp = (int64_t)nh * hd, es = dt == EE_F16 ? 2 : 4;
  const char* base = static_cast<const char*>(qkv);
  const AttnAddr ad{base, base + Hp * es, base + 2 * Hp * es, o, 0, hd, 3 * Hp, 0, hd, Hp, 1};
  return launch_attn(dt, ad, cu, B, max_len, nh, hd, causal, s);
}

bool cache_attention_mfma_ok(ee_dtype dt, int hd, int64_t max_pos) {
  // the kernel addresses a sequence's cached rows with 32-bit byte offsets
  return dt == EE_F16 && (hd == 64 || hd == 128) && attn_tr_offsets_fit(max_pos, hd);
}

hipError_t launch_cache_attention_mfma(ee_dtype dt, const void* qkv, const ExtendArg& arg, const int32_t* cu, int B,
                                       int max_new, int nh, int hd, int64_t max_pos, int64_t capacity,
                                       const void* kc, const void* vc, void* o, hipStream_t s) {
  if (!cache_attention_mfma_ok(dt, hd, max_pos)) return hipErrorInvalidValue;
  if (B <= 0 || max_new <= 0) return hipSuccess;
  const int64_t Hp = (int64_t)nh * hd;
  const AttnAddr ad{qkv, nullptr, nullptr, o, 0, hd, 3 * Hp, 0, hd, Hp, 1};
  const CacheKV kv{arg, static_cast<const f16*>(kc), static_cast<const f16*>(vc), capacity};
  const dim3 grid((unsigned)((max_new + kQB - 1) / kQB), (unsigned)nh, (unsigned)B), block(256);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)hd);
  if (hd == 64)
    hipLaunchKernelGGL((attn_tr_kernel<64, true, CacheKV>), grid, block, 0, s, ad, cu, scale_log2, kv);
  else
    hipLaunchKernelGGL((attn_tr_kernel<128, true, CacheKV>), grid, block, 0, s, ad, cu, scale_log2, kv);
  return hipGetLastError();
}

hipError_t launch_attention_padded(ee_dtype dt, const void* q, const void* k, const void* v, const int32_t* cu,
                                   int B, int P, int nh, int hd, bool causal, void* o, hipStream_t s) {
  const int64_t hs = (int64_t)P * hd, bs = (int64_t)nh * hs;
  const AttnAddr ad{q, k, v, o, bs, hs, hd, bs, hs, hd, 0};
  return launch_attn(dt, ad, cu, B, P, nh, hd, causal, s);
}

}  // namespace ee
