// LayerNorm over packed rows: y = (x - mean) / sqrt(var + eps) * gamma + beta,
// biased variance, fp32 statistics.  (LayerNorm is part of the add bias +
// input + LayerNorm step in the announcement article's "Ease of use" listing;
// the pre-LN placement inside the decoder block is this library's reading.)
//
// HBM-bound.  Rows of up to 8 x 64 16-byte vectors (H <= 4096 in fp16, 2048
// in fp32) go one wave per row; wider rows one workgroup (4 waves) per row,
// which measured faster there (a wave holding a 12288-wide row needs all 256
// VGPRs and leaves too few rows in flight).  Either way the row is read once into registers with 16-byte loads,
// reduced twice (mean, then the centred sum of squares, so no cancellation)
// and written once.  The workgroup kernel keeps gamma/beta in registers across
// its rows (the wave kernel re-reads them from L2 by every row).
#include "device_common.h"
#include "internal.h"

namespace ee {
namespace {

constexpr int kLnThreads = 256;


__device__ __forceinline__ float block_sum(float v, float* s_red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < kLnThreads / kWave; ++w) r += s_red[w];
  __syncthreads();  // s_red is reused by the next reduction
  return r;
}

template <typename T>
struct Vec16;  // one 16-byte vector of T
template <>
struct Vec16<f16> {
  typedef half8 type;
  static constexpr int n = 8;
};
template <>
struct Vec16<float> {
  typedef floatx4 type;
  static constexpr int n = 4;
};

// VPT: 16-byte vectors per thread (compile-time upper bound; nvec <= VPT*256).
// A workgroup walks rows blockIdx.x, +gridDim.x, ...; the next row's vectors
// are requested before the current row's two reductions and store, so the
// loads of one row overlap the barriers and stores of the previous one.
// ADD: the row is x + r, rounded to the storage type and written to `sum`
// (which may be x itself: each element is read, then written, by one thread)
// before it is normalised; NORM = false stops there (a plain residual add).
template <typename T, int VPT, bool ADD, bool NORM>
__global__ __launch_bounds__(kLnThreads) void layernorm_kernel(const T* x, const T* __restrict__ r, T* sum,
                                                               const T* __restrict__ gamma,
                                                               const T* __restrict__ beta, int64_t rows, int H,
                                                               float eps, T* __restrict__ y) {
  typedef typename Vec16<T>::type V;
  constexpr int E = Vec16<T>::n;
  __shared__ float s_red[kLnThreads / kWave];
  const int nvec = H / E;
  const float inv_h = 1.0f / (float)H;
  V cur[VPT], nxt[VPT], rcur[ADD ? VPT : 1], rnxt[ADD ? VPT : 1];
  auto load = [&](V (&dst)[VPT], V (&rdst)[ADD ? VPT : 1], int64_t row) {
    const V* xr = reinterpret_cast<const V*>(x + row * H);
    const V* rr = reinterpret_cast<const V*>(r + row * H);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * kLnThreads;
      if (c < nvec) {
        dst[i] = __builtin_nontemporal_load(xr + c);
        if constexpr (ADD) rdst[i] = __builtin_nontemporal_load(rr + c);
      }
    }
  };
  // gamma and beta: the same columns for every row of this thread, so they
  // are read once into registers (the plain LayerNorm at up to 2048 vectors
  // per row; the residual-add forms and wider rows have no register room)
  constexpr bool GB = NORM && !ADD && VPT <= 8;
  V gam[GB ? VPT : 1], bet[GB ? VPT : 1];
  if constexpr (GB) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * kLnThreads;
      if (c < nvec) {
        gam[i] = reinterpret_cast<const V*>(gamma)[c];
        bet[i] = reinterpret_cast<const V*>(beta)[c];
      }
    }
  }
  int64_t row = blockIdx.x;
  if (row < rows) load(cur, rcur, row);
  for (; row < rows; row += gridDim.x) {
    const int64_t next = row + gridDim.x;
    if (next < rows) load(nxt, rnxt, next);
    if constexpr (ADD) {
      V* sr = reinterpret_cast<V*>(sum + row * H);
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * kLnThreads;
        if (c < nvec) {
#pragma unroll
          for (int e = 0; e < E; ++e) cur[i][e] = from_f32<T>(to_f32(cur[i][e]) + to_f32(rcur[i][e]));
          sr[c] = cur[i];
        }
      }
    }
    if constexpr (NORM) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (threadIdx.x + i * kLnThreads < nvec)
#pragma unroll
          for (int e = 0; e < E; ++e) s += to_f32(cur[i][e]);
      const float mean = block_sum(s, s_red) * inv_h;
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (threadIdx.x + i * kLnThreads < nvec)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float d = to_f32(cur[i][e]) - mean;
            q += d * d;
          }
      const float rstd = 1.0f / sqrtf(block_sum(q, s_red) * inv_h + eps);
      V* yr = reinterpret_cast<V*>(y + row * H);
      const V* gv = reinterpret_cast<const V*>(gamma);
      const V* bv = reinterpret_cast<const V*>(beta);
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * kLnThreads;
        if (c < nvec) {
          V g, b;
          if constexpr (GB) {
            g = gam[i];
            b = bet[i];
          } else {
            g = gv[c];
            b = bv[c];
          }
          V o;
#pragma unroll
          for (int e = 0; e < E; ++e)
            o[e] = from_f32<T>((to_f32(cur[i][e]) - mean) * rstd * to_f32(g[e]) + to_f32(b[e]));
          yr[c] = o;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      cur[i] = nxt[i];
      if constexpr (ADD) rcur[i] = rnxt[i];
    }
  }
}

// One wave per row (4 rows per workgroup): the row is held in registers in
// its storage type (VPL 16-byte vectors per lane), the two reductions are wave
// shuffles, so rows never wait on each other at a barrier.  ADD and NORM as in
// layernorm_kernel.
template <typename T, int VPL, bool ADD, bool NORM>
__global__ __launch_bounds__(kLnThreads) void layernorm_wave_kernel(const T* x, const T* __restrict__ r, T* sum,
                                                                    const T* __restrict__ gamma,
                                                                    const T* __restrict__ beta, int64_t rows,
                                                                    int H, float eps, T* __restrict__ y) {
  typedef typename Vec16<T>::type V;
  constexpr int E = Vec16<T>::n;
  const int lane = threadIdx.x & (kWave - 1);
  const int nvec = H / E;
  const float inv_h = 1.0f / (float)H;
  const int64_t row0 = (int64_t)blockIdx.x * (kLnThreads / kWave) + (threadIdx.x / kWave);
  const int64_t stride = (int64_t)gridDim.x * (kLnThreads / kWave);
  for (int64_t row = row0; row < rows; row += stride) {
    const V* xr = reinterpret_cast<const V*>(x + row * H);
    V v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int c = lane + i * kWave;
      if (c < nvec) v[i] = __builtin_nontemporal_load(xr + c);
    }
    if constexpr (ADD) {
      const V* rr = reinterpret_cast<const V*>(r + row * H);
      V* sr = reinterpret_cast<V*>(sum + row * H);
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int c = lane + i * kWave;
        if (c < nvec) {
          const V rv = __builtin_nontemporal_load(rr + c);
#pragma unroll
          for (int e = 0; e < E; ++e) v[i][e] = from_f32<T>(to_f32(v[i][e]) + to_f32(rv[e]));
          sr[c] = v[i];
        }
      }
    }
    if constexpr (NORM) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + i * kWave < nvec)
#pragma unroll
          for (int e = 0; e < E; ++e) s += to_f32(v[i][e]);
      const float mean = wave_sum(s) * inv_h;
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + i * kWave < nvec)
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float d = to_f32(v[i][e]) - mean;
            q += d * d;
          }
      const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_h + eps);
      V* yr = reinterpret_cast<V*>(y + row * H);
      const V* gv = reinterpret_cast<const V*>(gamma);
      const V* bv = reinterpret_cast<const V*>(beta);
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int c = lane + i * kWave;
        if (c < nvec) {
          const V g = gv[c], b = bv[c];
          V o;
#pragma unroll
          for (int e = 0; e < E; ++e)
            o[e] = from_f32<T>((to_f32(v[i][e]) - mean) * rstd * to_f32(g[e]) + to_f32(b[e]));
          yr[c] = o;
        }
      }
    }
  }
}

// Post-LN residual step (the add bias + input + LayerNorm launcher of the
// announcement article's "Ease of use" listing): y = LN(u + bias + residual),
// the sum formed in fp32 and never stored.  One workgroup per row.
template <typename T, int VPT>
__global__ __launch_bounds__(kLnThreads) void add_bias_residual_ln_kernel(
    const T* __restrict__ u, const T* __restrict__ bias, const T* __restrict__ res, const T* __restrict__ gamma,
    const T* __restrict__ beta, int64_t rows, int H, float eps, T* __restrict__ y) {
  typedef typename Vec16<T>::type V;
  constexpr int E = Vec16<T>::n;
  __shared__ float s_red[kLnThreads / kWave];
  const int nvec = H / E;
  const float inv_h = 1.0f / (float)H;
  const V* bv = reinterpret_cast<const V*>(bias);
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const V* ur = reinterpret_cast<const V*>(u + row * H);
    const V* rr = reinterpret_cast<const V*>(res + row * H);
    float v[VPT][E];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * kLnThreads;
      if (c < nvec) {
        const V a = ur[c], r = rr[c], bb = bv[c];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          v[i][e] = to_f32(a[e]) + to_f32(bb[e]) + to_f32(r[e]);
          s += v[i][e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) v[i][e] = 0.f;
      }
    }
    const float mean = block_sum(s, s_red) * inv_h;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (threadIdx.x + i * kLnThreads < nvec)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float d = v[i][e] - mean;
          q += d * d;
        }
    const float rstd = 1.0f / sqrtf(block_sum(q, s_red) * inv_h + eps);
    V* yr = reinterpret_cast<V*>(y + row * H);
    const V* gv = reinterpret_cast<const V*>(gamma);
    const V* btv = reinterpret_cast<const V*>(beta);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = threadIdx.x + i * kLnThreads;
      if (c < nvec) {
        const V g = gv[c], bt = btv[c];
        V o;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = from_f32<T>((v[i][e] - mean) * rstd * to_f32(g[e]) + to_f32(bt[e]));
        yr[c] = o;
      }
    }
  }
}

template <typename T>
hipError_t launch_abrln_t(const void* u, const void* bias, const void* res, const void* g, const void* b,
                          int64_t rows, int H, float eps, void* y, hipStream_t s) {
  const int nvec = H / Vec16<T>::n;
  const unsigned grid = (unsigned)(rows > (1 << 20) ? (1 << 20) : rows);
  const T *up = static_cast<const T*>(u), *bp = static_cast<const T*>(bias), *rp = static_cast<const T*>(res);
  const T *gp = static_cast<const T*>(g), *btp = static_cast<const T*>(b);
  T* yp = static_cast<T*>(y);
  if (nvec <= 256)
    hipLaunchKernelGGL((add_bias_residual_ln_kernel<T, 1>), dim3(grid), dim3(kLnThreads), 0, s, up, bp, rp, gp, btp, rows, H, eps, yp);
  else if (nvec <= 1024)
    hipLaunchKernelGGL((add_bias_residual_ln_kernel<T, 4>), dim3(grid), dim3(kLnThreads), 0, s, up, bp, rp, gp, btp, rows, H, eps, yp);
  else if (nvec <= 2048)
    hipLaunchKernelGGL((add_bias_residual_ln_kernel<T, 8>), dim3(grid), dim3(kLnThreads), 0, s, up, bp, rp, gp, btp, rows, H, eps, yp);
  else
    hipLaunchKernelGGL((add_bias_residual_ln_kernel<T, 16>), dim3(grid), dim3(kLnThreads), 0, s, up, bp, rp, gp, btp, rows, H, eps, yp);
  return hipGetLastError();
}

// y = LN(x) (r == nullptr), or sum = x + r then y = LN(sum) (gamma != nullptr)
// or only sum = x + r (gamma == nullptr).
// Workgroups of kernel KERN resident on a device at once (computed on the
// first launch of each kernel form, on the device current then; every device
// this library targets has the same CU count), capped by the row count.
template <auto KERN>
unsigned ln_grid(int64_t rows) {
  static const int resident = [] {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, KERN, kLnThreads, 0) != hipSuccess || per_cu < 1)
      per_cu = 2;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    return per_cu * cus;
  }();
  return (unsigned)(rows < resident ? rows : resident);
}

template <typename T, bool ADD, bool NORM>
hipError_t launch_ln_mode(const T* xp, const T* rp, T* sp, const T* gp, const T* bp, int64_t rows, int H, float eps,
                          T* yp, hipStream_t s) {
  const int nvec = H / Vec16<T>::n;
  if (nvec <= 8 * kWave) {  // narrow rows: one wave per row
    const int64_t wgs = (rows + 3) / 4;
    const dim3 wg((unsigned)(wgs > (1 << 20) ? (1 << 20) : wgs)), blk(kLnThreads);
    const int vpl = (nvec + kWave - 1) / kWave;
#define EE_LN_WAVE(V) \
  hipLaunchKernelGGL((layernorm_wave_kernel<T, V, ADD, NORM>), wg, blk, 0, s, xp, rp, sp, gp, bp, rows, H, eps, yp)
    if (vpl <= 1)
      EE_LN_WAVE(1);
    else if (vpl <= 2)
      EE_LN_WAVE(2);
    else if (vpl <= 4)
      EE_LN_WAVE(4);
    else
      EE_LN_WAVE(8);
#undef EE_LN_WAVE
    return hipGetLastError();
  }
  // block kernel: as many workgroups as the device holds at once (one wave
  // of workgroups, none waiting for a slot), each walking several rows.  At
  // 12288 fp16 columns (two workgroups per CU) 512 workgroups ran 8-12%
  // faster than 2048 on 4096 rows and the same on 8125.
  const dim3 blk(kLnThreads);
#define EE_LN_BLOCK(V)                                                                                   \
  hipLaunchKernelGGL((layernorm_kernel<T, V, ADD, NORM>), dim3(ln_grid<layernorm_kernel<T, V, ADD, NORM>>(rows)), \
                     blk, 0, s, xp, rp, sp, gp, bp, rows, H, eps, yp)
  if (nvec <= 256)
    EE_LN_BLOCK(1);
  else if (nvec <= 512)
    EE_LN_BLOCK(2);
  else if (nvec <= 1024)
    EE_LN_BLOCK(4);
  else if (nvec <= 2048)
    EE_LN_BLOCK(8);
  else
    EE_LN_BLOCK(16);
#undef EE_LN_BLOCK
  return hipGetLastError();
}

template <typename T>
hipError_t launch_ln_t(const void* x, const void* r, void* sum, const void* g, const void* b, int64_t rows, int H,
                       float eps, void* y, hipStream_t s) {
  const T* xp = static_cast<const T*>(x);
  const T* rp = static_cast<const T*>(r);
  T* sp = static_cast<T*>(sum);
  const T* gp = static_cast<const T*>(g);
  const T* bp = static_cast<const T*>(b);
  T* yp = static_cast<T*>(y);
  if (!r) return launch_ln_mode<T, false, true>(xp, rp, sp, gp, bp, rows, H, eps, yp, s);
  if (g) return launch_ln_mode<T, true, true>(xp, rp, sp, gp, bp, rows, H, eps, yp, s);
  return launch_ln_mode<T, true, false>(xp, rp, sp, gp, bp, rows, H, eps, yp, s);
}

}  // namespace

int layernorm_max_hidden(ee_dtype dt) { return 16 * kLnThreads * (dt == EE_F16 ? 8 : 4); }

hipError_t launch_layernorm(ee_dtype dt, const void* x, const void* g, const void* b, int64_t rows, int H, float eps,
                            void* y, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return dt == EE_F16 ? launch_ln_t<f16>(x, nullptr, nullptr, g, b, rows, H, eps, y, s)
                      : launch_ln_t<float>(x, nullptr, nullptr, g, b, rows, H, eps, y, s);
}

hipError_t launch_residual_add_layernorm(ee_dtype dt, const void* x, const void* r, void* sum, const void* g,
                                         const void* b, int64_t rows, int H, float eps, void* y, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return dt == EE_F16 ? launch_ln_t<f16>(x, r, sum, g, b, rows, H, eps, y, s)
                      : launch_ln_t<float>(x, r, sum, g, b, rows, H, eps, y, s);
}

hipError_t launch_add_bias_residual_layernorm(ee_dtype dt, const void* u, const void* bias, const void* res,
                                              const void* g, const void* b, int64_t rows, int H, float eps, void* y,
                                              hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return dt == EE_F16 ? launch_abrln_t<f16>(u, bias, res, g, b, rows, H, eps, y, s)
                      : launch_abrln_t<float>(u, bias, res, g, b, rows, H, eps, y, s);
}

}  // namespace ee
