// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
// Not installed; every symbol lives in namespace ee and is hidden from the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ee.h"
#include "gemm_plan.h"

namespace ee {

// Host lengths travel to the device as a by-value kernel argument: no
// host-to-device copy, so the caller's array is free once the call returns.
struct LensArg {
  int32_t v[EE_MAX_BATCH];
};

// Records `msg` as the calling thread's last error (ee_last_error) and returns s.
ee_status set_error(ee_status s, const char* msg);

// ee_stack_extend with an explicit workspace (api.cpp); the no-allocation
// entry point passes its static scratch buffer.
ee_status stack_extend_into(ee_layer* const* layers, int32_t n_layers, const void* d_x, const int32_t* new_len,
                            const int32_t* ctx_len, const int32_t* slot_base, int32_t batch, void* d_cache,
                            int64_t capacity, void* d_y, void* ws, size_t ws_bytes, void* stream);

// ---- offsets.hip ----
hipError_t launch_offsets(const LensArg& lens, int B, int P, int32_t* cu, int32_t* token_src,
                          int32_t* pad2pack, hipStream_t s);
hipError_t launch_offsets_mask(const uint8_t* mask, int B, int P, int32_t* cu, int32_t* token_src,
                               int32_t* pad2pack, int32_t* total, hipStream_t s);

// ---- padding.hip ----  (row_bytes % 16 == 0, pointers 16-byte aligned)
hipError_t launch_remove(const void* padded, const int32_t* token_src, int64_t T, int64_t row_bytes,
                         void* packed, hipStream_t s);
hipError_t launch_rebuild(const void* packed, const int32_t* pad2pack, int64_t rows, int64_t row_bytes,
                          void* padded, hipStream_t s);
// transposing forms: packed [T, n*nh*hd] <-> head-major padded [n, B, nh, P, hd]
// (head_bytes = hd * element size, a multiple of 16)
hipError_t launch_rebuild_heads(const void* packed, const int32_t* cu, int B, int nh, int P, int head_bytes,
                                int n_mats, void* out, hipStream_t s);
hipError_t launch_remove_heads(const void* heads, const int32_t* cu, int B, int nh, int P, int head_bytes,
                               void* packed, hipStream_t s);

// ---- decode.hip ----  (extend step: new tokens after cached ones; B <= EE_MAX_EXTEND_BATCH)
struct ExtendArg {
  int32_t new_len[EE_MAX_EXTEND_BATCH];
  int32_t ctx_len[EE_MAX_EXTEND_BATCH];
  int32_t slot_base[EE_MAX_EXTEND_BATCH];
};
bool cache_attention_ok(int head_dim);
// Extend steps with many new tokens per sequence: the MFMA attention kernel
// (attention.hip) over the cached keys, one workgroup per 128 new queries of a
// (sequence, head).  fp16, head_dim 64 or 128, positions below the 32-bit
// offset limit.
bool cache_attention_mfma_ok(ee_dtype dt, int hd, int64_t max_pos);
hipError_t launch_cache_attention_mfma(ee_dtype dt, const void* qkv, const ExtendArg& arg, const int32_t* cu, int B,
                                       int max_new, int nh, int hd, int64_t max_pos, int64_t capacity,
                                       const void* kc, const void* vc, void* o, hipStream_t s);
int cache_attention_max_positions();
hipError_t launch_extend_cu(const ExtendArg& arg, int B, int32_t* cu, hipStream_t s);
hipError_t launch_append_kv(const void* qkv, const ExtendArg& arg, const int32_t* cu, int B, int64_t T, int nh,
                            int head_bytes, int64_t capacity, void* cache, hipStream_t s);
// Cache attention over key chunks of `chunk` positions (n_chunks per query):
// each chunk's softmax state is a partial in scratch, merged by a second
// kernel (none when n_chunks == 1).  The chunk length starts at
// kCacheAttnChunk and doubles until the partials fit scratch_bytes;
// n_chunks == 0: they never fit.
constexpr int kCacheAttnChunk = 512;
struct CacheAttnPlan {
  int chunk, n_chunks;
};
CacheAttnPlan cache_attention_plan(int64_t T_new, int nh, int hd, int max_pos, size_t scratch_bytes);
hipError_t launch_cache_attention(ee_dtype dt, const void* qkv, const ExtendArg& arg, const int32_t* cu, int B,
                                  int64_t T_new, int nh, int hd, int max_pos, int64_t capacity, const void* kc,
                                  const void* vc, void* o, void* scratch, size_t scratch_bytes, hipStream_t s);

// ---- layernorm.hip ----
int layernorm_max_hidden(ee_dtype dt);
hipError_t launch_layernorm(ee_dtype dt, const void* x, const void* g, const void* b, int64_t rows, int H,
                            float eps, void* y, hipStream_t s);
// sum = x + r (rounded to the storage type; sum may be x), then y = LN(sum)
// when g and b are given, else only the sum.
hipError_t launch_residual_add_layernorm(ee_dtype dt, const void* x, const void* r, void* sum, const void* g,
                                         const void* b, int64_t rows, int H, float eps, void* y, hipStream_t s);
hipError_t launch_add_bias_residual_layernorm(ee_dtype dt, const void* u, const void* bias, const void* res,
                                              const void* g, const void* b, int64_t rows, int H, float eps, void* y,
                                              hipStream_t s);

// ---- bias_gelu.hip ----
// u and g are [rows, ld] (ld >= cols, a multiple of 16 bytes)
hipError_t launch_bias_gelu(ee_dtype dt, const void* u, const void* bias, int64_t rows, int cols, int ld,
                            ee_gelu form, void* g, hipStream_t s);

// Compute units of the current device, cached per device (gemm_f16.hip).
int device_cu_count();

// ---- gemm_f16.hip / gemm_valu.hip ----
// Row pitches, in elements, of a GEMM's operands: A [M, a], W [N, w], and
// C and the residual R [M, c].
struct GemmPitch {
  int a, w, c;
};
// Whether the MFMA kernel takes this problem: K % 64 == 0, pitches of A and W
// that are multiples of 8 (16-byte rows) and 16-byte aligned A and W.
bool gemm_f16_mfma_ok(int64_t M, int N, int K, const GemmPitch& ld, const void* A, const void* W);
hipError_t launch_gemm_f16_mfma(const void* A, const void* W, const void* bias, const void* R, int64_t M,
                                int N, int K, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C,
                                hipStream_t s);
// The launches launch_gemm_f16_mfma makes, for callers that time them one by
// one: rows [row0, row0 + rows) of the problem on one kernel configuration.
// A large problem whose 256 x 256 tile count is just past a multiple of the
// CU count runs its partial last round as in-order stream-K pieces of the one
// persistent launch when given `ordered` scratch of gemm_f16_ordered_bytes()
// (bit-identical to whole tiles); without it, whole rounds of 256-row tiles
// and the remaining rows as a second part on smaller tiles.
// (The parts, GemmPart and the plan itself: gemm_plan.h.)
size_t gemm_f16_ordered_bytes();
// Number of parts (0 for M <= 0).  vec_stores: N and C's pitch are multiples
// of 8 and C and the residual 16-byte aligned (the ordered form needs it).
int gemm_f16_parts(int64_t M, int N, int K, GemmPart (&parts)[kGemmMaxParts], size_t ordered_bytes, bool vec_stores);
hipError_t launch_gemm_f16_part(const GemmPart& p, const void* A, const void* W, const void* bias, const void* R,
                                int N, int K, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C,
                                hipStream_t s, void* ordered, size_t ordered_bytes);
// The kernel template a part runs, as
// gemm_f16_mfma_kernel<MF, BM, BN, WGM, WGN, EPI, WDEPTH, ORD>.
const char* gemm_f16_kernel_label(int cfg, ee_epilogue epi, bool ordered);
// Split-K for small M: `splits` equal K ranges (K % (64 * splits) == 0) summed
// into fp32 partials in scratch (gemm_f16_splitk_bytes), then reduced with the
// epilogue.  gemm_f16_splitk_choice picks the split count (1 = do not split)
// for a problem gemm_f16_mfma_ok accepts.
int gemm_f16_splitk_choice(int64_t M, int N, int K, size_t scratch_bytes);
size_t gemm_f16_splitk_bytes(int64_t M, int N, int splits);
hipError_t launch_gemm_f16_splitk(const void* A, const void* W, const void* bias, const void* R, int64_t M, int N,
                                  int K, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C, int splits,
                                  void* scratch, hipStream_t s);
// Stream-K for M <= kStreamKMaxRows (gemm_streamk.hip): every workgroup
// streams an equal share of W's (N tile, K tile) space into fp32 partial sums
// in scratch (plan.scratch_bytes), then a reduce adds each tile's pieces in K
// order and applies the epilogue.  workgroups == 0: the kernel does not take
// the problem.
constexpr int64_t kStreamKMaxRows = 128;
struct StreamKPlan {
  int tile_rows, kt, tiles_n, per_wg, workgroups;
  size_t scratch_bytes;
};
StreamKPlan gemm_f16_streamk_plan(int64_t M, int N, int K, const GemmPitch& ld);
hipError_t launch_gemm_f16_streamk(const StreamKPlan& p, const void* A, const void* W, const void* bias, const void* R,
                                   int64_t M, int N, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C,
                                   void* scratch, hipStream_t s);
hipError_t launch_gemm_valu(ee_dtype dt, const void* A, const void* W, const void* bias, const void* R,
                            int64_t M, int N, int K, const GemmPitch& ld, ee_epilogue epi, ee_gelu form, void* C,
                            hipStream_t s);

// ---- attention.hip ----
bool attention_mfma_ok(ee_dtype dt, int head_dim);
hipError_t launch_attention(ee_dtype dt, const void* qkv, const int32_t* cu, int B, int max_len, int nh,
                            int hd, bool causal, void* o, hipStream_t s);
hipError_t launch_attention_padded(ee_dtype dt, const void* q, const void* k, const void* v, const int32_t* cu,
                                   int B, int P, int nh, int hd, bool causal, void* o, hipStream_t s);

}  // namespace ee
