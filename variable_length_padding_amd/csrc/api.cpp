// C ABI of libee (declared in include/ee.h): host-side validation, workspace
// planning, kernel sequencing and per-launch event timing.  Every check runs
// before the first HIP call of an entry point, so a rejected call enqueues
// nothing.  The forward path allocates nothing and never synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <type_traits>
#include <utility>
#include <vector>

#include "ee.h"
#include "internal.h"

using namespace ee;

struct ee_layer {
  ee_layer_desc desc;
  ee_layer_weights w;  // ld_* resolved: the row pitch of each matrix, never 0
  int ld_big;          // row pitch of the FC1 output in the workspace
};

namespace {

thread_local std::string g_err;

ee_status fail(ee_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

}  // namespace

ee_status ee::set_error(ee_status s, const char* msg) {
  g_err = msg;
  return s;
}

namespace {

ee_status hip_fail(hipError_t e, const char* what) {
  return fail(EE_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// The int a caller passed for an enum argument or field.  The ABI's enums are
// C enums, so any int can arrive; in C++ loading an enum object whose value
// lies outside its enumerators' range is undefined, so validation reads the
// object representation instead.
template <class E>
int ev(const E& e) {
  static_assert(std::is_enum<E>::value && sizeof(E) == sizeof(int), "an int-sized enum");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

size_t dtype_size(ee_dtype d) { return d == EE_F16 ? 2 : 4; }
bool dtype_ok(int d) { return d == EE_F32 || d == EE_F16; }
bool gelu_ok(int g) { return g == EE_GELU_TANH || g == EE_GELU_ERF; }
bool epilogue_ok(int e) { return e >= EE_EPI_NONE && e <= EE_EPI_BIAS_GELU; }
size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ee_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(EE_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(EE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return EE_OK;
}

// Bytes spanned by `rows` rows of `cols` elements at a pitch of ld elements.
size_t span(int64_t rows, int64_t cols, int64_t ld, size_t s) {
  return rows <= 0 ? 0 : ((size_t)(rows - 1) * (size_t)ld + (size_t)cols) * s;
}

// cols, plus 128 bytes when a row is a multiple of 32 KiB (see ee.h).
int64_t preferred_pitch(int64_t cols, size_t s) {
  return (size_t)cols * s % 32768 == 0 ? cols + (int64_t)(128 / s) : cols;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

#define EE_TRY(expr)                 \
  do {                               \
    const ee_status s_ = (expr);     \
    if (s_ != EE_OK) return s_;      \
  } while (0)

// ---------------------------------------------------------------- profiling
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::string only;  // the one site timed, or empty for every site
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  size_t used = 0;
  struct Rec {
    std::string site;
    size_t event;        // pool index
    double flops;        // algorithmic flops of the launch (GEMMs; 0 elsewhere)
    const char* kernel;  // static label of the kernel launched, or nullptr
  };
  std::vector<Rec> recs;
};
Profiler& prof() {
  static Profiler* p = new Profiler();  // never destroyed: events may outlive static teardown order
  return *p;
}

// Debug mode (ee_debug_sync, or EE_DEBUG_SYNC=1 in the environment when the
// library loads): every launch is followed by a synchronisation of its
// stream, so an asynchronous failure surfaces at the launch site that caused
// it instead of at some later call.
std::atomic<bool> g_debug_sync{[] {
  const char* v = std::getenv("EE_DEBUG_SYNC");
  return v && v[0] && v[0] != '0';
}()};

// Runs `launch` (which returns the launch's hipError_t); while profiling is on,
// brackets it with two events recorded on `s`.  `flops` and `kernel` are
// recorded with the launch.
template <class F>
hipError_t timed_launch(const char* site, hipStream_t s, F&& launch, double flops, const char* kernel) {
  Profiler& p = prof();
  if (!p.on) return launch();
  std::lock_guard<std::mutex> lk(p.mu);
  if (!p.only.empty() && p.only != site) return launch();
  if (p.used == p.pool.size()) {
    // timing-only events: no system-scope fence (a cache writeback) when they
    // are recorded, which would stall the stream between the timed launches
    std::pair<hipEvent_t, hipEvent_t> e{};
    hipError_t r = hipEventCreateWithFlags(&e.first, hipEventDisableSystemFence);
    if (r == hipSuccess) r = hipEventCreateWithFlags(&e.second, hipEventDisableSystemFence);
    if (r != hipSuccess) return r;
    p.pool.push_back(e);
  }
  const size_t i = p.used++;
  hipError_t r = hipEventRecord(p.pool[i].first, s);
  if (r != hipSuccess) return r;
  r = launch();
  if (r != hipSuccess) return r;
  r = hipEventRecord(p.pool[i].second, s);
  if (r != hipSuccess) return r;
  p.recs.push_back(Profiler::Rec{site, i, flops, kernel});
  return hipSuccess;
}

template <class F>
hipError_t timed(const char* site, hipStream_t s, F&& launch, double flops = 0.0, const char* kernel = nullptr) {
  hipError_t r = timed_launch(site, s, launch, flops, kernel);
  if (r == hipSuccess && g_debug_sync.load(std::memory_order_relaxed)) r = hipStreamSynchronize(s);
  return r;
}

#define EE_LAUNCH(site, stream, call)                                        \
  do {                                                                       \
    const hipError_t e_ = timed(site, stream, [&]() { return (call); });    \
    if (e_ != hipSuccess) return hip_fail(e_, site);                         \
  } while (0)

// ---------------------------------------------------------------- validation
ee_status check_lengths(const int32_t* lens, int32_t B, int32_t P, int64_t* total, int32_t* max_len) {
  if (!lens) return fail(EE_ERR_INVALID_ARG, "seq_lens is NULL");
  if (B < 1 || B > EE_MAX_BATCH) return fail(EE_ERR_INVALID_ARG, "batch %d outside [1, %d]", B, EE_MAX_BATCH);
  if (P < 1) return fail(EE_ERR_INVALID_ARG, "pad_len %d < 1", P);
  if ((int64_t)B * P > INT32_MAX) return fail(EE_ERR_INVALID_ARG, "batch*pad_len exceeds 2^31-1");
  int64_t T = 0;
  int32_t mx = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (lens[b] < 0 || lens[b] > P)
      return fail(EE_ERR_INVALID_ARG, "seq_lens[%d] = %d outside [0, pad_len=%d]", b, lens[b], P);
    T += lens[b];
    mx = std::max(mx, lens[b]);
  }
  *total = T;
  if (max_len) *max_len = mx;
  return EE_OK;
}

ee_status check_desc(const ee_layer_desc* d) {
  if (!d) return fail(EE_ERR_INVALID_ARG, "desc is NULL");
  if (!dtype_ok(ev(d->dtype))) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", ev(d->dtype));
  if (!gelu_ok(ev(d->gelu))) return fail(EE_ERR_INVALID_ARG, "unknown gelu %d", ev(d->gelu));
  if (d->fuse_gelu != 0 && d->fuse_gelu != 1) return fail(EE_ERR_INVALID_ARG, "fuse_gelu must be 0 or 1");
  const int block = ev(d->block), attention = ev(d->attention), residual = ev(d->residual);
  if (block != EE_BLOCK_GPT_PRELN && block != EE_BLOCK_BERT_POSTLN)
    return fail(EE_ERR_INVALID_ARG, "unknown block %d", block);
  if (attention != EE_ATTN_VARLEN && attention != EE_ATTN_PADDED)
    return fail(EE_ERR_INVALID_ARG, "unknown attention form %d", attention);
  if (residual != EE_RESIDUAL_AUTO && residual != EE_RESIDUAL_EPILOGUE && residual != EE_RESIDUAL_PASS)
    return fail(EE_ERR_INVALID_ARG, "unknown residual mode %d", residual);
  if (d->hidden < 1 || d->n_heads < 1 || d->ffn < 1)
    return fail(EE_ERR_INVALID_ARG, "hidden, n_heads and ffn must be >= 1");
  if (!(d->ln_eps > 0.f) || !std::isfinite(d->ln_eps)) return fail(EE_ERR_INVALID_ARG, "ln_eps must be finite and > 0");
  const int hd = d->head_dim;
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return fail(EE_ERR_UNSUPPORTED, "head_dim %d not in {16, 32, 64, 128}", hd);
  if (d->n_heads > 65535) return fail(EE_ERR_UNSUPPORTED, "n_heads %d > 65535", d->n_heads);
  const size_t s = dtype_size(d->dtype);
  if ((size_t)d->hidden * s % 16 || (size_t)d->ffn * s % 16)
    return fail(EE_ERR_UNSUPPORTED, "hidden and ffn rows must be multiples of 16 bytes");
  if (d->hidden > layernorm_max_hidden(d->dtype))
    return fail(EE_ERR_UNSUPPORTED, "hidden %d above the LayerNorm kernel's %d", d->hidden,
                layernorm_max_hidden(d->dtype));
  if ((int64_t)d->n_heads * hd > (1 << 24) || d->ffn > (1 << 24) || d->hidden > (1 << 24))
    return fail(EE_ERR_UNSUPPORTED, "layer dimension too large");
  return EE_OK;
}

bool desc_equal(const ee_layer_desc& a, const ee_layer_desc& b) {
  return a.hidden == b.hidden && a.n_heads == b.n_heads && a.head_dim == b.head_dim && a.ffn == b.ffn &&
         a.ln_eps == b.ln_eps && a.dtype == b.dtype && a.gelu == b.gelu && a.fuse_gelu == b.fuse_gelu &&
         a.block == b.block && a.attention == b.attention && a.residual == b.residual;
}

// ---------------------------------------------------------------- workspace
struct Plan {
  size_t cu, token_src, pad2pack, x, ln, big, o, h, heads, o_heads, splitk, splitk_bytes, ordered, ordered_bytes,
      total;
};

// Whether the pre-LN residuals are added in a separate pass (EE_RESIDUAL_AUTO: in the epilogue).
bool residual_pass(const ee_layer_desc& d) { return d.residual == EE_RESIDUAL_PASS; }

// split-K partial sums of the small-M GEMMs of an extend step
constexpr size_t kSplitkScratch = size_t(64) << 20;
constexpr int64_t kSplitkMaxRows = 128;

Plan plan_offsets_only(int32_t B, int32_t P) {
  Plan p{};
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += align256(n);
    return o;
  };
  p.cu = take(4 * (size_t)(B + 1));
  p.token_src = take(4 * (size_t)B * P);
  p.pad2pack = take(4 * (size_t)B * P);
  p.total = off;
  return p;
}

Plan plan_layer(const ee_layer_desc& d, int32_t B, int32_t P, int64_t T) {
  Plan p = plan_offsets_only(B, P);
  size_t off = p.total;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += align256(n);
    return o;
  };
  const size_t s = dtype_size(d.dtype), t = (size_t)T;
  const size_t H = d.hidden, Hp = (size_t)d.n_heads * d.head_dim, F = d.ffn;
  p.x = take(t * H * s);
  p.ln = take(t * H * s);
  p.big = take(t * std::max<size_t>(3 * Hp, preferred_pitch((int64_t)F, s)) * s);
  p.o = take(t * Hp * s);
  p.h = take(t * H * s);
  if (d.attention == EE_ATTN_PADDED) {  // head-major padded q|k|v and output
    const size_t pad_rows = (size_t)B * P;
    p.heads = take(3 * pad_rows * Hp * s);
    p.o_heads = take(pad_rows * Hp * s);
  }
  if (d.dtype == EE_F16) {  // the large GEMMs' in-order stream-K pieces
    p.ordered_bytes = gemm_f16_ordered_bytes();
    p.ordered = take(p.ordered_bytes);
  }
  p.total = off;
  return p;
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// ---------------------------------------------------------------- launch helpers
// One GEMM launch site.  With a scratch buffer (extend steps), small-M
// problems run stream-K or split-K (two kernels, timed as one launch of
// `site`).  The dense fp16 path runs as one or two parts (gemm_f16_parts):
// the first is timed as `site`, a remainder of rows as `rest_site`; with
// `ordered` scratch a large problem is one part whose partial last round
// runs as in-order stream-K pieces (the same bits).  Each launch records its
// algorithmic flops, 2*rows*N*K.
ee_status gemm_site(const char* site, const char* rest_site, ee_dtype dt, const void* A, const void* W,
                    const void* bias, const void* R, int64_t M, int N, int K, const GemmPitch& ld, ee_epilogue epi,
                    ee_gelu g, void* C, hipStream_t s, void* scratch = nullptr, size_t scratch_bytes = 0,
                    void* ordered = nullptr, size_t ordered_bytes = 0) {
  const double flops = 2.0 * (double)M * N * K;
  if (dt == EE_F16 && gemm_f16_mfma_ok(M, N, K, ld, A, W)) {
    if (scratch) {
      const StreamKPlan sk = gemm_f16_streamk_plan(M, N, K, ld);
      if (sk.workgroups > 0 && sk.scratch_bytes <= scratch_bytes) {
        const hipError_t e = timed(
            site, s, [&]() { return launch_gemm_f16_streamk(sk, A, W, bias, R, M, N, ld, epi, g, C, scratch, s); },
            flops, "gemm_streamk_kernel + streamk_reduce_kernel");
        return e == hipSuccess ? EE_OK : hip_fail(e, site);
      }
    }
    const int splits = scratch && M <= kSplitkMaxRows ? gemm_f16_splitk_choice(M, N, K, scratch_bytes) : 1;
    if (splits > 1) {
      const hipError_t e = timed(
          site, s, [&]() { return launch_gemm_f16_splitk(A, W, bias, R, M, N, K, ld, epi, g, C, splits, scratch, s); },
          flops, "gemm_f16_mfma_kernel<32, 128, 128, 2, 2, 4, 2, false> + splitk_reduce_kernel");
      return e == hipSuccess ? EE_OK : hip_fail(e, site);
    }
    GemmPart parts[kGemmMaxParts];
    const bool vec_stores = N % 8 == 0 && ld.c % 8 == 0 && aligned16(C) && (!R || aligned16(R));
    const int n = gemm_f16_parts(M, N, K, parts, ordered ? ordered_bytes : 0, vec_stores);
    for (int i = 0; i < n; ++i) {
      const char* at_site = i == 0 ? site : rest_site;
      const hipError_t e = timed(
          at_site, s,
          [&]() { return launch_gemm_f16_part(parts[i], A, W, bias, R, N, K, ld, epi, g, C, s, ordered, ordered_bytes); },
          2.0 * (double)parts[i].rows * N * K,
          gemm_f16_kernel_label(parts[i].cfg, epi, parts[i].ordered));
      if (e != hipSuccess) return hip_fail(e, at_site);
    }
    return EE_OK;
  }
  const hipError_t e = timed(
      site, s, [&]() { return launch_gemm_valu(dt, A, W, bias, R, M, N, K, ld, epi, g, C, s); }, flops,
      "gemm_valu_kernel");
  return e == hipSuccess ? EE_OK : hip_fail(e, site);
}

// A GEMM launch site `site`; a second part of its rows is timed as site "_rest".
#define EE_GEMM(site, ...) EE_TRY(gemm_site(site, site "_rest", __VA_ARGS__))

GemmPitch dense(int N, int K) { return GemmPitch{K, K, N}; }

ee_status offsets_from_host(const int32_t* lens, int32_t B, int32_t P, int32_t* cu, int32_t* token_src,
                            int32_t* pad2pack, hipStream_t s) {
  LensArg la;
  std::memset(&la, 0, sizeof la);
  std::memcpy(la.v, lens, sizeof(int32_t) * (size_t)B);
  EE_LAUNCH("offsets", s, launch_offsets(la, B, P, cu, token_src, pad2pack, s));
  return EE_OK;
}

// Attention of the layer on packed qkv -> o, in the descriptor's form.
ee_status attend(const ee_layer_desc& d, void* ws, const Plan& p, const void* qkv, void* o, int32_t B, int32_t P,
                 int32_t max_len, bool causal, hipStream_t s) {
  const int32_t* cu = reinterpret_cast<const int32_t*>(at(ws, p.cu));
  if (d.attention == EE_ATTN_VARLEN) {
    EE_LAUNCH("attention", s, launch_attention(d.dtype, qkv, cu, B, max_len, d.n_heads, d.head_dim, causal, o, s));
    return EE_OK;
  }
  const int head_bytes = d.head_dim * (int)dtype_size(d.dtype);
  char* heads = at(ws, p.heads);
  const size_t mat = (size_t)B * P * d.n_heads * d.head_dim * dtype_size(d.dtype);
  EE_LAUNCH("rebuild_heads", s, launch_rebuild_heads(qkv, cu, B, d.n_heads, P, head_bytes, 3, heads, s));
  EE_LAUNCH("attention", s, launch_attention_padded(d.dtype, heads, heads + mat, heads + 2 * mat, cu, B, P, d.n_heads,
                                                    d.head_dim, causal, at(ws, p.o_heads), s));
  EE_LAUNCH("remove_heads", s, launch_remove_heads(at(ws, p.o_heads), cu, B, d.n_heads, P, head_bytes, o, s));
  return EE_OK;
}

// The packed layer on T rows held in ws.x; the output replaces ws.x.
// attn(qkv, o, causal) runs the attention step from the packed qkv rows.
template <class Attn>
ee_status packed_layer(const ee_layer* L, void* ws, const Plan& p, int64_t T, hipStream_t s, Attn&& attn) {
  const ee_layer_desc& d = L->desc;
  const ee_layer_weights& w = L->w;
  const int H = d.hidden, Hp = d.n_heads * d.head_dim, F = d.ffn;
  void* x = at(ws, p.x);
  void* ln = at(ws, p.ln);
  void* big = at(ws, p.big);
  void* o = at(ws, p.o);
  void* h = at(ws, p.h);
  void* sk = p.splitk_bytes ? at(ws, p.splitk) : nullptr;
  const size_t skb = p.splitk_bytes;
  // in-order stream-K scratch: its own region in a forward, the (sequentially
  // reused) partial-sum region in an extend step
  void* ord = p.ordered_bytes ? at(ws, p.ordered) : sk;
  const size_t ordb = p.ordered_bytes ? p.ordered_bytes : skb;
  // A [T, .] . W^T: activations dense except the FC1 output (pitch ld_big)
  const GemmPitch ld_qkv{H, (int)w.ld_qkv, 3 * Hp}, ld_out{Hp, (int)w.ld_out, H};
  const GemmPitch ld_fc1{H, (int)w.ld_fc1, L->ld_big}, ld_fc2{L->ld_big, (int)w.ld_fc2, H};
  auto fc1 = [&](const void* in) -> ee_status {
    if (d.fuse_gelu) {
      EE_GEMM("gemm_fc1", d.dtype, in, w.w_fc1, w.b_fc1, nullptr, T, F, H, ld_fc1, EE_EPI_BIAS_GELU, d.gelu, big, s, sk, skb, ord, ordb);
    } else {
      EE_GEMM("gemm_fc1", d.dtype, in, w.w_fc1, nullptr, nullptr, T, F, H, ld_fc1, EE_EPI_NONE, d.gelu, big, s, sk, skb, ord, ordb);
      EE_LAUNCH("bias_gelu", s, launch_bias_gelu(d.dtype, big, w.b_fc1, T, F, L->ld_big, d.gelu, big, s));
    }
    return EE_OK;
  };
  if (d.block == EE_BLOCK_GPT_PRELN) {
    EE_LAUNCH("ln1", s, launch_layernorm(d.dtype, x, w.ln1_g, w.ln1_b, T, H, d.ln_eps, ln, s));
    EE_GEMM("gemm_qkv", d.dtype, ln, w.w_qkv, w.b_qkv, nullptr, T, 3 * Hp, H, ld_qkv, EE_EPI_BIAS, d.gelu, big, s, sk, skb, ord, ordb);
    EE_TRY(attn(big, o, true));
    if (residual_pass(d)) {
      // h = (o W_out^T + b_out) + x and ln = LN2(h); x = (g W_fc2^T + b_fc2) + h
      EE_GEMM("gemm_out", d.dtype, o, w.w_out, w.b_out, nullptr, T, H, Hp, ld_out, EE_EPI_BIAS, d.gelu, h, s, sk, skb, ord, ordb);
      EE_LAUNCH("res_ln2", s, launch_residual_add_layernorm(d.dtype, h, x, h, w.ln2_g, w.ln2_b, T, H, d.ln_eps, ln, s));
      EE_TRY(fc1(ln));
      EE_GEMM("gemm_fc2", d.dtype, big, w.w_fc2, w.b_fc2, nullptr, T, H, F, ld_fc2, EE_EPI_BIAS, d.gelu, x, s, sk, skb, ord, ordb);
      EE_LAUNCH("res_add", s, launch_residual_add_layernorm(d.dtype, x, h, x, nullptr, nullptr, T, H, 0.f, nullptr, s));
      return EE_OK;
    }
    EE_GEMM("gemm_out", d.dtype, o, w.w_out, w.b_out, x, T, H, Hp, ld_out, EE_EPI_BIAS_RESIDUAL, d.gelu, h, s, sk, skb, ord, ordb);
    EE_LAUNCH("ln2", s, launch_layernorm(d.dtype, h, w.ln2_g, w.ln2_b, T, H, d.ln_eps, ln, s));
    EE_TRY(fc1(ln));
    EE_GEMM("gemm_fc2", d.dtype, big, w.w_fc2, w.b_fc2, h, T, H, F, ld_fc2, EE_EPI_BIAS_RESIDUAL, d.gelu, x, s, sk, skb, ord, ordb);
    return EE_OK;
  }
  // post-LN encoder: GEMM, then bias + residual + LayerNorm in one pass
  EE_GEMM("gemm_qkv", d.dtype, x, w.w_qkv, w.b_qkv, nullptr, T, 3 * Hp, H, ld_qkv, EE_EPI_BIAS, d.gelu, big, s, sk, skb, ord, ordb);
  EE_TRY(attn(big, o, false));
  EE_GEMM("gemm_out", d.dtype, o, w.w_out, nullptr, nullptr, T, H, Hp, ld_out, EE_EPI_NONE, d.gelu, ln, s, sk, skb, ord, ordb);
  EE_LAUNCH("add_ln1", s,
            launch_add_bias_residual_layernorm(d.dtype, ln, w.b_out, x, w.ln1_g, w.ln1_b, T, H, d.ln_eps, h, s));
  EE_TRY(fc1(h));
  EE_GEMM("gemm_fc2", d.dtype, big, w.w_fc2, nullptr, nullptr, T, H, F, ld_fc2, EE_EPI_NONE, d.gelu, ln, s, sk, skb, ord, ordb);
  EE_LAUNCH("add_ln2", s,
            launch_add_bias_residual_layernorm(d.dtype, ln, w.b_fc2, h, w.ln2_g, w.ln2_b, T, H, d.ln_eps, x, s));
  return EE_OK;
}

ee_status stack_impl(ee_layer* const* layers, int32_t n_layers, const void* x_padded, const int32_t* seq_lens,
                     int32_t B, int32_t P, void* y_padded, void* ws, size_t ws_bytes, void* stream) {
  if (!layers || n_layers < 1) return fail(EE_ERR_INVALID_ARG, "need at least one layer");
  for (int32_t i = 0; i < n_layers; ++i) {
    if (!layers[i]) return fail(EE_ERR_INVALID_ARG, "layers[%d] is NULL", i);
    if (!desc_equal(layers[i]->desc, layers[0]->desc))
      return fail(EE_ERR_INVALID_ARG, "layers[%d] has a different descriptor from layers[0]", i);
  }
  const ee_layer_desc& d = layers[0]->desc;
  int64_t T = 0;
  int32_t max_len = 0;
  EE_TRY(check_lengths(seq_lens, B, P, &T, &max_len));
  EE_TRY(check_ptr(x_padded, "x_padded"));
  EE_TRY(check_ptr(y_padded, "y_padded"));
  EE_TRY(check_ptr(ws, "workspace"));
  const Plan p = plan_layer(d, B, P, T);
  if (ws_bytes < p.total)
    return fail(EE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu for T=%lld", ws_bytes, p.total, (long long)T);
  const size_t io = (size_t)B * P * d.hidden * dtype_size(d.dtype);
  if (overlap(x_padded, io, y_padded, io)) return fail(EE_ERR_INVALID_ARG, "x_padded and y_padded overlap");
  if (overlap(ws, p.total, x_padded, io) || overlap(ws, p.total, y_padded, io))
    return fail(EE_ERR_INVALID_ARG, "workspace overlaps x_padded or y_padded");

  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* cu = reinterpret_cast<int32_t*>(at(ws, p.cu));
  int32_t* tsrc = reinterpret_cast<int32_t*>(at(ws, p.token_src));
  int32_t* p2p = reinterpret_cast<int32_t*>(at(ws, p.pad2pack));
  const int64_t row_bytes = (int64_t)d.hidden * (int64_t)dtype_size(d.dtype);
  EE_TRY(offsets_from_host(seq_lens, B, P, cu, tsrc, p2p, s));
  if (T > 0) {
    EE_LAUNCH("remove", s, launch_remove(x_padded, tsrc, T, row_bytes, at(ws, p.x), s));
    for (int32_t i = 0; i < n_layers; ++i)
      EE_TRY(packed_layer(layers[i], ws, p, T, s, [&](const void* qkv, void* o, bool causal) {
        return attend(d, ws, p, qkv, o, B, P, max_len, causal, s);
      }));
  }
  EE_LAUNCH("rebuild", s, launch_rebuild(at(ws, p.x), p2p, (int64_t)B * P, row_bytes, y_padded, s));
  return EE_OK;
}

// ---------------------------------------------------------------- extend (incremental decoding)
// The attention of an extend step runs on the MFMA kernel (a workgroup per
// 128 new queries of a sequence and head, each key tile read once for all of
// them) from this many new tokens in some sequence on, and from 2 when the
// sequences with new tokens times the heads give every CU a workgroup.
// Otherwise it runs on the cache-attention kernel (a workgroup per query,
// head and key chunk), which splits long contexts over many workgroups and
// reads the keys once per query.  GPT-3 width, 32 sequences after 2048 cached
// positions: equal at 1 new token each (0.56 ms), 0.55 against 0.83 ms at 2,
// 0.61 against 9.2 ms at 16, 1.48 against 101 ms at 256.
constexpr int32_t kExtendMfmaMinNew = 16;
Plan plan_extend(const ee_layer_desc& d, int32_t B, int64_t T) {
  Plan p{};
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += align256(n);
    return o;
  };
  const size_t s = dtype_size(d.dtype), t = (size_t)T;
  const size_t H = d.hidden, Hp = (size_t)d.n_heads * d.head_dim, F = d.ffn;
  p.cu = take(4 * (size_t)(B + 1));
  p.x = take(t * H * s);
  p.ln = take(t * H * s);
  p.big = take(t * std::max<size_t>(3 * Hp, preferred_pitch((int64_t)F, s)) * s);
  p.o = take(t * Hp * s);
  p.h = take(t * H * s);
  // partial sums (the small-M GEMMs' split-K / stream-K pieces, then the cache
  // attention's per-chunk softmax states), reserved at every T, so a size
  // taken for T covers any smaller step
  p.splitk = take(kSplitkScratch);
  p.splitk_bytes = kSplitkScratch;
  p.total = off;
  return p;
}

size_t cache_layer_bytes(const ee_layer_desc& d, int64_t capacity) {
  return 2 * (size_t)d.n_heads * (size_t)capacity * (size_t)d.head_dim * dtype_size(d.dtype);
}

ee_status extend_impl(ee_layer* const* layers, int32_t n_layers, const void* d_x, const int32_t* new_len,
                      const int32_t* ctx_len, const int32_t* slot_base, int32_t B, void* d_cache, int64_t capacity,
                      void* d_y, void* ws, size_t ws_bytes, void* stream) {
  if (!layers || n_layers < 1) return fail(EE_ERR_INVALID_ARG, "need at least one layer");
  for (int32_t i = 0; i < n_layers; ++i) {
    if (!layers[i]) return fail(EE_ERR_INVALID_ARG, "layers[%d] is NULL", i);
    if (!desc_equal(layers[i]->desc, layers[0]->desc))
      return fail(EE_ERR_INVALID_ARG, "layers[%d] has a different descriptor from layers[0]", i);
  }
  const ee_layer_desc& d = layers[0]->desc;
  if (d.block != EE_BLOCK_GPT_PRELN)
    return fail(EE_ERR_INVALID_ARG, "incremental decoding needs the causal (GPT pre-LN) block");
  if (!cache_attention_ok(d.head_dim)) return fail(EE_ERR_UNSUPPORTED, "head_dim %d unsupported", d.head_dim);
  if (B < 1 || B > EE_MAX_EXTEND_BATCH) return fail(EE_ERR_INVALID_ARG, "batch %d not in [1, %d]", B, EE_MAX_EXTEND_BATCH);
  if (!new_len || !ctx_len || !slot_base) return fail(EE_ERR_INVALID_ARG, "new_len, ctx_len, slot_base are required");
  if (capacity < 1 || capacity > INT32_MAX) return fail(EE_ERR_INVALID_ARG, "capacity must be in [1, 2^31)");
  // every slot written or read lies in [0, capacity), and sequences with
  // tokens own disjoint slot ranges
  int64_t T = 0;
  int32_t max_pos = 0;
  std::vector<std::pair<int64_t, int64_t>> ranges;
  for (int32_t b = 0; b < B; ++b) {
    if (new_len[b] < 0 || ctx_len[b] < 0 || slot_base[b] < 0)
      return fail(EE_ERR_INVALID_ARG, "negative new_len, ctx_len or slot_base at %d", b);
    const int64_t used = (int64_t)ctx_len[b] + new_len[b];
    if ((int64_t)slot_base[b] + used > capacity)
      return fail(EE_ERR_INVALID_ARG, "sequence %d needs slots up to %lld, capacity %lld", b,
                  (long long)(slot_base[b] + used), (long long)capacity);
    if (new_len[b] > 0) {
      if (used > ee_extend_max_positions())
        return fail(EE_ERR_UNSUPPORTED, "sequence %d reaches %lld positions, above %d", b, (long long)used,
                    ee_extend_max_positions());
      max_pos = std::max<int32_t>(max_pos, (int32_t)used);
    }
    if (used > 0) ranges.emplace_back(slot_base[b], slot_base[b] + used);
    T += new_len[b];
  }
  std::sort(ranges.begin(), ranges.end());
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].first < ranges[i - 1].second) return fail(EE_ERR_INVALID_ARG, "sequences share cache slots");
  if (T == 0) return EE_OK;
  EE_TRY(check_ptr(d_x, "d_x"));
  EE_TRY(check_ptr(d_y, "d_y"));
  EE_TRY(check_ptr(d_cache, "d_cache"));
  EE_TRY(check_ptr(ws, "workspace"));
  const Plan p = plan_extend(d, B, T);
  if (ws_bytes < p.total)
    return fail(EE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu for %lld new tokens", ws_bytes, p.total,
                (long long)T);
  const size_t s_el = dtype_size(d.dtype);
  const size_t io = (size_t)T * d.hidden * s_el, cl = cache_layer_bytes(d, capacity);
  const size_t cache_bytes = cl * (size_t)n_layers;
  if (overlap(d_x, io, d_y, io)) return fail(EE_ERR_INVALID_ARG, "d_x and d_y overlap");
  if (overlap(ws, p.total, d_x, io) || overlap(ws, p.total, d_y, io) || overlap(ws, p.total, d_cache, cache_bytes))
    return fail(EE_ERR_INVALID_ARG, "workspace overlaps d_x, d_y or the cache");
  if (overlap(d_cache, cache_bytes, d_x, io) || overlap(d_cache, cache_bytes, d_y, io))
    return fail(EE_ERR_INVALID_ARG, "the cache overlaps d_x or d_y");

  ExtendArg arg;
  std::memset(&arg, 0, sizeof arg);
  bool prefill = true;  // no sequence with new tokens has cached ones
  int32_t max_new = 0;
  for (int32_t b = 0; b < B; ++b) {
    arg.new_len[b] = new_len[b];
    arg.ctx_len[b] = ctx_len[b];
    arg.slot_base[b] = slot_base[b];
    if (new_len[b] > 0 && ctx_len[b] > 0) prefill = false;
    max_new = std::max(max_new, new_len[b]);
  }
  int64_t active = 0;  // sequences with new tokens
  for (int32_t b = 0; b < B; ++b) active += new_len[b] > 0;
  const bool mfma_attention =
      cache_attention_mfma_ok(d.dtype, d.head_dim, max_pos) &&
      (max_new >= kExtendMfmaMinNew || (max_new >= 2 && active * d.n_heads >= device_cu_count()));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* cu = reinterpret_cast<int32_t*>(at(ws, p.cu));
  EE_LAUNCH("extend_cu", s, launch_extend_cu(arg, B, cu, s));
  const hipError_t e_in = hipMemcpyAsync(at(ws, p.x), d_x, io, hipMemcpyDeviceToDevice, s);
  if (e_in != hipSuccess) return hip_fail(e_in, "copy in");
  const int nh = d.n_heads, hd = d.head_dim;
  const size_t kv_half = (size_t)nh * (size_t)capacity * hd * s_el;  // the k part of a layer's cache
  for (int32_t l = 0; l < n_layers; ++l) {
    char* layer_cache = static_cast<char*>(d_cache) + cl * (size_t)l;
    EE_TRY(packed_layer(layers[l], ws, p, T, s, [&](const void* qkv, void* o, bool) -> ee_status {
      EE_LAUNCH("append_kv", s,
                launch_append_kv(qkv, arg, cu, B, T, nh, hd * (int)s_el, capacity, layer_cache, s));
      if (prefill) {  // attention among the new tokens only: the packed varlen kernel
        EE_LAUNCH("attention", s, launch_attention(d.dtype, qkv, cu, B, max_new, nh, hd, true, o, s));
      } else if (mfma_attention) {
        // many new tokens per sequence: 128 of them share each key tile (MFMA)
        EE_LAUNCH("cache_attention", s,
                  launch_cache_attention_mfma(d.dtype, qkv, arg, cu, B, max_new, nh, hd, max_pos, capacity,
                                              layer_cache, layer_cache + kv_half, o, s));
      } else {
        // the chunks' softmax partials use the GEMMs' partial-sum region, idle
        // between the QKV GEMM's reduce and the out GEMM
        EE_LAUNCH("cache_attention", s,
                  launch_cache_attention(d.dtype, qkv, arg, cu, B, T, nh, hd, max_pos, capacity, layer_cache,
                                         layer_cache + kv_half, o, at(ws, p.splitk), p.splitk_bytes, s));
      }
      return EE_OK;
    }));
  }
  const hipError_t e_out = hipMemcpyAsync(d_y, at(ws, p.x), io, hipMemcpyDeviceToDevice, s);
  if (e_out != hipSuccess) return hip_fail(e_out, "copy out");
  return EE_OK;
}

}  // namespace

ee_status ee::stack_extend_into(ee_layer* const* layers, int32_t n_layers, const void* d_x, const int32_t* new_len,
                                const int32_t* ctx_len, const int32_t* slot_base, int32_t batch, void* d_cache,
                                int64_t capacity, void* d_y, void* ws, size_t ws_bytes, void* stream) {
  return extend_impl(layers, n_layers, d_x, new_len, ctx_len, slot_base, batch, d_cache, capacity, d_y, ws, ws_bytes,
                     stream);
}

// ======================================================================= ABI
extern "C" {

const char* ee_status_string(ee_status s) {
  switch (ev(s)) {
    case EE_OK: return "EE_OK";
    case EE_ERR_INVALID_ARG: return "EE_ERR_INVALID_ARG";
    case EE_ERR_UNSUPPORTED: return "EE_ERR_UNSUPPORTED";
    case EE_ERR_WORKSPACE: return "EE_ERR_WORKSPACE";
    case EE_ERR_OOM: return "EE_ERR_OOM";
    case EE_ERR_HIP: return "EE_ERR_HIP";
  }
  return "EE_UNKNOWN_STATUS";
}

const char* ee_last_error(void) { return g_err.c_str(); }

const char* ee_version(void) { return "ee 0.1 (gfx950)"; }

ee_status ee_layer_create(const ee_layer_desc* desc, const ee_layer_weights* weights, ee_layer** out) {
  if (!out) return fail(EE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  EE_TRY(check_desc(desc));
  if (!weights) return fail(EE_ERR_INVALID_ARG, "weights is NULL");
  const void* const ptrs[] = {weights->ln1_g, weights->ln1_b, weights->w_qkv, weights->b_qkv,
                              weights->w_out, weights->b_out, weights->ln2_g, weights->ln2_b,
                              weights->w_fc1, weights->b_fc1, weights->w_fc2, weights->b_fc2};
  static const char* const names[] = {"ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_out", "b_out",
                                      "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2"};
  for (int i = 0; i < 12; ++i) EE_TRY(check_ptr(ptrs[i], names[i]));
  const int64_t H = desc->hidden, Hp = (int64_t)desc->n_heads * desc->head_dim, F = desc->ffn;
  const size_t s = dtype_size(desc->dtype);
  ee_layer_weights w = *weights;
  int64_t* const lds[] = {&w.ld_qkv, &w.ld_out, &w.ld_fc1, &w.ld_fc2};
  const int64_t rowlen[] = {H, Hp, H, F};
  static const char* const ldnames[] = {"ld_qkv", "ld_out", "ld_fc1", "ld_fc2"};
  for (int i = 0; i < 4; ++i) {
    if (*lds[i] == 0) *lds[i] = rowlen[i];
    if (*lds[i] < rowlen[i] || *lds[i] > INT32_MAX || (size_t)*lds[i] * s % 16)
      return fail(EE_ERR_INVALID_ARG, "%s = %lld: need a pitch >= %lld elements, below 2^31, of 16-byte rows",
                  ldnames[i], (long long)*lds[i], (long long)rowlen[i]);
  }
  ee_layer* L = new (std::nothrow) ee_layer;
  if (!L) return fail(EE_ERR_OOM, "host allocation of the layer handle failed");
  L->desc = *desc;
  L->w = w;
  L->ld_big = (int)preferred_pitch(F, s);
  *out = L;
  return EE_OK;
}

ee_status ee_layer_destroy(ee_layer* layer) {
  delete layer;
  return EE_OK;
}

ee_status ee_layer_workspace_size(const ee_layer* layer, int32_t batch, int32_t pad_len, int64_t max_tokens,
                                  size_t* bytes) {
  if (!layer || !bytes) return fail(EE_ERR_INVALID_ARG, "layer and bytes must be non-NULL");
  if (batch < 1 || batch > EE_MAX_BATCH || pad_len < 1 || (int64_t)batch * pad_len > INT32_MAX)
    return fail(EE_ERR_INVALID_ARG, "bad batch %d / pad_len %d", batch, pad_len);
  const int64_t cap = (int64_t)batch * pad_len;
  if (max_tokens < 0 || max_tokens > cap) max_tokens = cap;
  *bytes = plan_layer(layer->desc, batch, pad_len, max_tokens).total;
  return EE_OK;
}

ee_status ee_layer_forward(ee_layer* layer, const void* x_padded, const int32_t* seq_lens, int32_t batch,
                           int32_t pad_len, void* y_padded, void* workspace, size_t ws_bytes, void* stream) {
  if (!layer) return fail(EE_ERR_INVALID_ARG, "layer is NULL");
  ee_layer* const one[1] = {layer};
  return stack_impl(one, 1, x_padded, seq_lens, batch, pad_len, y_padded, workspace, ws_bytes, stream);
}

ee_status ee_stack_forward(ee_layer* const* layers, int32_t n_layers, const void* x_padded, const int32_t* seq_lens,
                           int32_t batch, int32_t pad_len, void* y_padded, void* workspace, size_t ws_bytes,
                           void* stream) {
  return stack_impl(layers, n_layers, x_padded, seq_lens, batch, pad_len, y_padded, workspace, ws_bytes, stream);
}

ee_status ee_kv_cache_bytes(const ee_layer* layer, int32_t n_layers, int64_t capacity, size_t* bytes) {
  if (!layer || !bytes || n_layers < 1 || capacity < 1 || capacity > INT32_MAX)
    return fail(EE_ERR_INVALID_ARG, "need a layer, n_layers >= 1, capacity in [1, 2^31) and an output");
  *bytes = cache_layer_bytes(layer->desc, capacity) * (size_t)n_layers;
  return EE_OK;
}

ee_status ee_extend_workspace_size(const ee_layer* layer, int32_t batch, int64_t max_new_tokens, size_t* bytes) {
  if (!layer || !bytes || batch < 1 || batch > EE_MAX_EXTEND_BATCH || max_new_tokens < 0)
    return fail(EE_ERR_INVALID_ARG, "need a layer, batch in [1, %d], max_new_tokens >= 0 and an output",
                EE_MAX_EXTEND_BATCH);
  *bytes = plan_extend(layer->desc, batch, max_new_tokens).total;
  return EE_OK;
}

int32_t ee_extend_max_positions(void) { return cache_attention_max_positions(); }

ee_status ee_stack_extend(ee_layer* const* layers, int32_t n_layers, const void* d_x, const int32_t* new_len,
                          const int32_t* ctx_len, const int32_t* slot_base, int32_t batch, void* d_cache,
                          int64_t capacity, void* d_y, void* ws, size_t ws_bytes, void* stream) {
  return extend_impl(layers, n_layers, d_x, new_len, ctx_len, slot_base, batch, d_cache, capacity, d_y, ws, ws_bytes,
                     stream);
}

ee_status ee_compute_offsets(const int32_t* seq_lens, int32_t batch, int32_t pad_len, int32_t* d_cu,
                             int32_t* d_token_src, int32_t* d_pad2pack, int32_t* total_tokens, void* stream) {
  int64_t T = 0;
  EE_TRY(check_lengths(seq_lens, batch, pad_len, &T, nullptr));
  if (!d_cu || !d_token_src || !d_pad2pack || !total_tokens)
    return fail(EE_ERR_INVALID_ARG, "output pointers must be non-NULL");
  const size_t n = 4 * (size_t)batch * pad_len;
  if (overlap(d_cu, 4 * (size_t)(batch + 1), d_token_src, n) || overlap(d_cu, 4 * (size_t)(batch + 1), d_pad2pack, n) ||
      overlap(d_token_src, n, d_pad2pack, n))
    return fail(EE_ERR_INVALID_ARG, "offset output arrays overlap");
  *total_tokens = (int32_t)T;
  return offsets_from_host(seq_lens, batch, pad_len, d_cu, d_token_src, d_pad2pack, static_cast<hipStream_t>(stream));
}

ee_status ee_compute_offsets_mask(const uint8_t* d_mask, int32_t batch, int32_t pad_len, int32_t* d_cu,
                                  int32_t* d_token_src, int32_t* d_pad2pack, int32_t* d_total, void* stream) {
  if (!d_mask || !d_cu || !d_token_src || !d_pad2pack || !d_total)
    return fail(EE_ERR_INVALID_ARG, "pointers must be non-NULL");
  if (batch < 1 || pad_len < 1 || (int64_t)batch * pad_len > INT32_MAX)
    return fail(EE_ERR_INVALID_ARG, "bad batch %d / pad_len %d", batch, pad_len);
  hipStream_t s = static_cast<hipStream_t>(stream);
  EE_LAUNCH("offsets_mask", s, launch_offsets_mask(d_mask, batch, pad_len, d_cu, d_token_src, d_pad2pack, d_total, s));
  return EE_OK;
}

ee_status ee_padding_workspace_size(int32_t batch, int32_t pad_len, size_t* bytes) {
  if (!bytes) return fail(EE_ERR_INVALID_ARG, "bytes is NULL");
  if (batch < 1 || batch > EE_MAX_BATCH || pad_len < 1 || (int64_t)batch * pad_len > INT32_MAX)
    return fail(EE_ERR_INVALID_ARG, "bad batch %d / pad_len %d", batch, pad_len);
  *bytes = plan_offsets_only(batch, pad_len).total;
  return EE_OK;
}

static ee_status padding_common(const void* src, const int32_t* seq_lens, int32_t batch, int32_t pad_len,
                                int32_t hidden, int dtype_i, void* dst, void* ws, size_t ws_bytes, int64_t* T,
                                Plan* p) {
  EE_TRY(check_lengths(seq_lens, batch, pad_len, T, nullptr));
  if (!dtype_ok(dtype_i)) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", dtype_i);
  const ee_dtype dtype = static_cast<ee_dtype>(dtype_i);
  if (hidden < 1 || (size_t)hidden * dtype_size(dtype) % 16)
    return fail(EE_ERR_UNSUPPORTED, "hidden*sizeof(dtype) must be a positive multiple of 16 bytes");
  EE_TRY(check_ptr(src, "source"));
  EE_TRY(check_ptr(dst, "destination"));
  EE_TRY(check_ptr(ws, "workspace"));
  *p = plan_offsets_only(batch, pad_len);
  if (ws_bytes < p->total) return fail(EE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, p->total);
  return EE_OK;
}

// The padded buffer spans batch*pad_len rows, the packed one T rows.
static ee_status check_padding_overlaps(const void* padded, const void* packed, const void* ws, size_t ws_total,
                                        int32_t batch, int32_t pad_len, int64_t T, int32_t hidden, ee_dtype dtype) {
  const size_t row = (size_t)hidden * dtype_size(dtype);
  const size_t np = (size_t)batch * pad_len * row, nk = (size_t)T * row;
  if (overlap(padded, np, packed, nk)) return fail(EE_ERR_INVALID_ARG, "padded and packed buffers overlap");
  if (overlap(ws, ws_total, padded, np) || overlap(ws, ws_total, packed, nk))
    return fail(EE_ERR_INVALID_ARG, "workspace overlaps the padded or packed buffer");
  return EE_OK;
}

ee_status ee_remove_padding(const void* d_padded, const int32_t* seq_lens, int32_t batch, int32_t pad_len,
                            int32_t hidden, ee_dtype dtype, void* d_packed, void* workspace, size_t ws_bytes,
                            void* stream) {
  int64_t T = 0;
  Plan p{};
  EE_TRY(padding_common(d_padded, seq_lens, batch, pad_len, hidden, ev(dtype), d_packed, workspace, ws_bytes, &T, &p));
  EE_TRY(check_padding_overlaps(d_padded, d_packed, workspace, p.total, batch, pad_len, T, hidden, dtype));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* cu = reinterpret_cast<int32_t*>(at(workspace, p.cu));
  int32_t* tsrc = reinterpret_cast<int32_t*>(at(workspace, p.token_src));
  int32_t* p2p = reinterpret_cast<int32_t*>(at(workspace, p.pad2pack));
  EE_TRY(offsets_from_host(seq_lens, batch, pad_len, cu, tsrc, p2p, s));
  EE_LAUNCH("remove", s, launch_remove(d_padded, tsrc, T, (int64_t)hidden * dtype_size(dtype), d_packed, s));
  return EE_OK;
}

ee_status ee_rebuild_padding(const void* d_packed, const int32_t* seq_lens, int32_t batch, int32_t pad_len,
                             int32_t hidden, ee_dtype dtype, void* d_padded, void* workspace, size_t ws_bytes,
                             void* stream) {
  int64_t T = 0;
  Plan p{};
  EE_TRY(padding_common(d_packed, seq_lens, batch, pad_len, hidden, ev(dtype), d_padded, workspace, ws_bytes, &T, &p));
  EE_TRY(check_padding_overlaps(d_padded, d_packed, workspace, p.total, batch, pad_len, T, hidden, dtype));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* cu = reinterpret_cast<int32_t*>(at(workspace, p.cu));
  int32_t* tsrc = reinterpret_cast<int32_t*>(at(workspace, p.token_src));
  int32_t* p2p = reinterpret_cast<int32_t*>(at(workspace, p.pad2pack));
  EE_TRY(offsets_from_host(seq_lens, batch, pad_len, cu, tsrc, p2p, s));
  EE_LAUNCH("rebuild", s,
            launch_rebuild(d_packed, p2p, (int64_t)batch * pad_len, (int64_t)hidden * dtype_size(dtype), d_padded, s));
  return EE_OK;
}

ee_status ee_layernorm(const void* x, const void* gamma, const void* beta, int64_t rows, int32_t hidden, float eps,
                       ee_dtype dtype, void* y, void* stream) {
  if (!dtype_ok(ev(dtype))) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", ev(dtype));
  if (rows < 0) return fail(EE_ERR_INVALID_ARG, "rows < 0");
  if (hidden < 1 || (size_t)hidden * dtype_size(dtype) % 16)
    return fail(EE_ERR_UNSUPPORTED, "hidden*sizeof(dtype) must be a positive multiple of 16 bytes");
  if (hidden > layernorm_max_hidden(dtype)) return fail(EE_ERR_UNSUPPORTED, "hidden %d too large", hidden);
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(EE_ERR_INVALID_ARG, "eps must be finite and > 0");
  EE_TRY(check_ptr(gamma, "gamma"));
  EE_TRY(check_ptr(beta, "beta"));
  if (rows == 0) return EE_OK;
  EE_TRY(check_ptr(x, "x"));
  EE_TRY(check_ptr(y, "y"));
  const size_t n = (size_t)rows * hidden * dtype_size(dtype);
  if (overlap(x, n, y, n)) return fail(EE_ERR_INVALID_ARG, "x and y overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  EE_LAUNCH("layernorm", s, launch_layernorm(dtype, x, gamma, beta, rows, hidden, eps, y, s));
  return EE_OK;
}

// ee_linear_strided with the enum arguments as the ints the caller passed
static ee_status linear_strided(const void* A, int64_t lda, const void* W, int64_t ldw, const void* bias,
                                const void* residual, int64_t M, int32_t N, int32_t K, int dtype_i, int epi_i,
                                int gelu_i, void* C, int64_t ldc, void* stream, void* ws = nullptr,
                                size_t ws_bytes = 0) {
  if (!dtype_ok(dtype_i)) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", dtype_i);
  if (!epilogue_ok(epi_i)) return fail(EE_ERR_INVALID_ARG, "unknown epilogue %d", epi_i);
  if (!gelu_ok(gelu_i)) return fail(EE_ERR_INVALID_ARG, "unknown gelu %d", gelu_i);
  const ee_dtype dtype = static_cast<ee_dtype>(dtype_i);
  const ee_epilogue epi = static_cast<ee_epilogue>(epi_i);
  const ee_gelu gelu = static_cast<ee_gelu>(gelu_i);
  if (M < 0 || N < 1 || K < 1) return fail(EE_ERR_INVALID_ARG, "need M >= 0, N >= 1, K >= 1");
  if (lda < K || ldw < K || ldc < N || lda > INT32_MAX || ldw > INT32_MAX || ldc > INT32_MAX)
    return fail(EE_ERR_INVALID_ARG, "pitches lda %lld, ldw %lld, ldc %lld: need >= K, K, N and < 2^31",
                (long long)lda, (long long)ldw, (long long)ldc);
  if (M > 4000000) return fail(EE_ERR_UNSUPPORTED, "M = %lld above 4,000,000", (long long)M);
  EE_TRY(check_ptr(W, "W"));
  if (epi != EE_EPI_NONE) EE_TRY(check_ptr(bias, "bias"));
  if (M == 0) return EE_OK;
  EE_TRY(check_ptr(A, "A"));
  EE_TRY(check_ptr(C, "C"));
  if (epi == EE_EPI_BIAS_RESIDUAL) EE_TRY(check_ptr(residual, "residual"));
  const size_t s = dtype_size(dtype);
  const size_t nc = span(M, N, ldc, s);
  if (overlap(C, nc, A, span(M, K, lda, s)) || overlap(C, nc, W, span(N, K, ldw, s)) ||
      (epi != EE_EPI_NONE && overlap(C, nc, bias, (size_t)N * s)) ||
      (epi == EE_EPI_BIAS_RESIDUAL && overlap(C, nc, residual, nc)))
    return fail(EE_ERR_INVALID_ARG, "C overlaps an input");
  if (ws) {
    const size_t na = span(M, K, lda, s), nw = span(N, K, ldw, s);
    if (overlap(ws, ws_bytes, A, na) || overlap(ws, ws_bytes, W, nw) || overlap(ws, ws_bytes, C, nc) ||
        (epi != EE_EPI_NONE && overlap(ws, ws_bytes, bias, (size_t)N * s)) ||
        (epi == EE_EPI_BIAS_RESIDUAL && overlap(ws, ws_bytes, residual, nc)))
      return fail(EE_ERR_INVALID_ARG, "the workspace overlaps an operand");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const GemmPitch ld{(int)lda, (int)ldw, (int)ldc};
  EE_TRY(gemm_site("linear", "linear_rest", dtype, A, W, bias, residual, M, N, K, ld, epi, gelu, C, st, nullptr, 0,
                   ws, ws_bytes));
  return EE_OK;
}

size_t ee_linear_ws_workspace_size(void) { return gemm_f16_ordered_bytes(); }

ee_status ee_linear_ws(const void* A, int64_t lda, const void* W, int64_t ldw, const void* bias,
                       const void* residual, int64_t M, int32_t N, int32_t K, ee_dtype dtype, ee_epilogue epi,
                       ee_gelu gelu, void* C, int64_t ldc, void* ws, size_t ws_bytes, void* stream) {
  EE_TRY(check_ptr(ws, "workspace"));
  if (ws_bytes < gemm_f16_ordered_bytes())
    return fail(EE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, gemm_f16_ordered_bytes());
  return linear_strided(A, lda, W, ldw, bias, residual, M, N, K, ev(dtype), ev(epi), ev(gelu), C, ldc, stream, ws,
                        ws_bytes);
}

ee_status ee_linear_strided(const void* A, int64_t lda, const void* W, int64_t ldw, const void* bias,
                            const void* residual, int64_t M, int32_t N, int32_t K, ee_dtype dtype, ee_epilogue epi,
                            ee_gelu gelu, void* C, int64_t ldc, void* stream) {
  return linear_strided(A, lda, W, ldw, bias, residual, M, N, K, ev(dtype), ev(epi), ev(gelu), C, ldc, stream);
}

ee_status ee_linear(const void* A, const void* W, const void* bias, const void* residual, int64_t M, int32_t N,
                    int32_t K, ee_dtype dtype, ee_epilogue epi, ee_gelu gelu, void* C, void* stream) {
  return linear_strided(A, K, W, K, bias, residual, M, N, K, ev(dtype), ev(epi), ev(gelu), C, N, stream);
}

int64_t ee_preferred_row_pitch(int64_t cols, ee_dtype dtype) {
  if (cols < 1 || !dtype_ok(ev(dtype))) return 0;
  return preferred_pitch(cols, dtype_size(dtype));
}

ee_status ee_linear_splitk_workspace_size(int64_t M, int32_t N, int32_t splits, size_t* bytes) {
  if (M < 0 || N < 1 || splits < 1 || splits > 64 || !bytes)
    return fail(EE_ERR_INVALID_ARG, "need M >= 0, N >= 1, 1 <= splits <= 64 and an output");
  *bytes = gemm_f16_splitk_bytes(M, N, splits);
  return EE_OK;
}

ee_status ee_linear_splitk(const void* A, const void* W, const void* bias, const void* residual, int64_t M,
                           int32_t N, int32_t K, ee_dtype dtype, ee_epilogue epi, ee_gelu gelu, int32_t splits,
                           void* C, void* ws, size_t ws_bytes, void* stream) {
  if (ev(dtype) != EE_F16) return fail(EE_ERR_UNSUPPORTED, "split-K is fp16 only");
  if (!epilogue_ok(ev(epi))) return fail(EE_ERR_INVALID_ARG, "unknown epilogue %d", ev(epi));
  if (!gelu_ok(ev(gelu))) return fail(EE_ERR_INVALID_ARG, "unknown gelu %d", ev(gelu));
  if (M < 0 || N < 1 || K < 1 || splits < 1 || splits > 64)
    return fail(EE_ERR_INVALID_ARG, "need M >= 0, N >= 1, K >= 1, 1 <= splits <= 64");
  if (M == 0) return EE_OK;
  if (!gemm_f16_mfma_ok(M, N, K, dense(N, K), A, W) || K % (64 * splits) != 0)
    return fail(EE_ERR_UNSUPPORTED, "shape M=%lld N=%d K=%d splits=%d not supported", (long long)M, N, K, splits);
  EE_TRY(check_ptr(A, "A"));
  EE_TRY(check_ptr(W, "W"));
  EE_TRY(check_ptr(C, "C"));
  EE_TRY(check_ptr(ws, "workspace"));
  if (epi != EE_EPI_NONE) EE_TRY(check_ptr(bias, "bias"));
  if (epi == EE_EPI_BIAS_RESIDUAL) EE_TRY(check_ptr(residual, "residual"));
  const size_t need = gemm_f16_splitk_bytes(M, N, splits);
  if (ws_bytes < need) return fail(EE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
  const size_t nc = (size_t)M * N * 2;
  if (overlap(C, nc, A, (size_t)M * K * 2) || overlap(C, nc, W, (size_t)N * K * 2) ||
      (epi != EE_EPI_NONE && overlap(C, nc, bias, (size_t)N * 2)) ||
      (epi == EE_EPI_BIAS_RESIDUAL && overlap(C, nc, residual, nc)) || overlap(ws, need, C, nc) ||
      overlap(ws, need, A, (size_t)M * K * 2) || overlap(ws, need, W, (size_t)N * K * 2))
    return fail(EE_ERR_INVALID_ARG, "C or the workspace overlaps an input");
  hipStream_t st = static_cast<hipStream_t>(stream);
  EE_LAUNCH("linear", st,
            launch_gemm_f16_splitk(A, W, bias, residual, M, N, K, dense(N, K), epi, gelu, C, splits, ws, st));
  return EE_OK;
}

ee_status ee_linear_streamk_workspace_size(int64_t M, int32_t N, int32_t K, size_t* bytes) {
  if (M < 0 || N < 1 || K < 1 || !bytes) return fail(EE_ERR_INVALID_ARG, "need M >= 0, N >= 1, K >= 1 and an output");
  if (M == 0) {
    *bytes = 0;
    return EE_OK;
  }
  const StreamKPlan p = gemm_f16_streamk_plan(M, N, K, dense(N, K));
  if (p.workgroups < 1)
    return fail(EE_ERR_UNSUPPORTED, "stream-K does not take M=%lld N=%d K=%d", (long long)M, N, K);
  *bytes = p.scratch_bytes;
  return EE_OK;
}

ee_status ee_linear_streamk(const void* A, const void* W, const void* bias, const void* residual, int64_t M,
                            int32_t N, int32_t K, ee_dtype dtype, ee_epilogue epi, ee_gelu gelu, void* C, void* ws,
                            size_t ws_bytes, void* stream) {
  if (ev(dtype) != EE_F16) return fail(EE_ERR_UNSUPPORTED, "stream-K is fp16 only");
  if (!epilogue_ok(ev(epi))) return fail(EE_ERR_INVALID_ARG, "unknown epilogue %d", ev(epi));
  if (!gelu_ok(ev(gelu))) return fail(EE_ERR_INVALID_ARG, "unknown gelu %d", ev(gelu));
  if (M < 0 || N < 1 || K < 1) return fail(EE_ERR_INVALID_ARG, "need M >= 0, N >= 1, K >= 1");
  if (M == 0) return EE_OK;
  const StreamKPlan p = gemm_f16_streamk_plan(M, N, K, dense(N, K));
  if (p.workgroups < 1 || !gemm_f16_mfma_ok(M, N, K, dense(N, K), A, W))
    return fail(EE_ERR_UNSUPPORTED, "stream-K does not take M=%lld N=%d K=%d", (long long)M, N, K);
  EE_TRY(check_ptr(A, "A"));
  EE_TRY(check_ptr(W, "W"));
  EE_TRY(check_ptr(C, "C"));
  EE_TRY(check_ptr(ws, "workspace"));
  if (epi != EE_EPI_NONE) EE_TRY(check_ptr(bias, "bias"));
  if (epi == EE_EPI_BIAS_RESIDUAL) EE_TRY(check_ptr(residual, "residual"));
  if (ws_bytes < p.scratch_bytes)
    return fail(EE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, p.scratch_bytes);
  const size_t nc = (size_t)M * N * 2, need = p.scratch_bytes;
  if (overlap(C, nc, A, (size_t)M * K * 2) || overlap(C, nc, W, (size_t)N * K * 2) ||
      (epi != EE_EPI_NONE && overlap(C, nc, bias, (size_t)N * 2)) ||
      (epi == EE_EPI_BIAS_RESIDUAL && overlap(C, nc, residual, nc)) || overlap(ws, need, C, nc) ||
      overlap(ws, need, A, (size_t)M * K * 2) || overlap(ws, need, W, (size_t)N * K * 2) ||
      (epi != EE_EPI_NONE && overlap(ws, need, bias, (size_t)N * 2)) ||
      (epi == EE_EPI_BIAS_RESIDUAL && overlap(ws, need, residual, nc)))
    return fail(EE_ERR_INVALID_ARG, "C or the workspace overlaps an input");
  hipStream_t st = static_cast<hipStream_t>(stream);
  EE_LAUNCH("linear", st,
            launch_gemm_f16_streamk(p, A, W, bias, residual, M, N, dense(N, K), epi, gelu, C, ws, st));
  return EE_OK;
}

ee_status ee_bias_gelu(const void* u, const void* bias, int64_t rows, int32_t cols, ee_dtype dtype, ee_gelu gelu,
                       void* g, void* stream) {
  if (!dtype_ok(ev(dtype))) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", ev(dtype));
  if (!gelu_ok(ev(gelu))) return fail(EE_ERR_INVALID_ARG, "unknown gelu %d", ev(gelu));
  if (rows < 0 || cols < 1) return fail(EE_ERR_INVALID_ARG, "need rows >= 0, cols >= 1");
  if ((size_t)cols * dtype_size(dtype) % 16) return fail(EE_ERR_UNSUPPORTED, "cols*sizeof(dtype) % 16 != 0");
  EE_TRY(check_ptr(bias, "bias"));
  if (rows == 0) return EE_OK;
  EE_TRY(check_ptr(u, "u"));
  EE_TRY(check_ptr(g, "g"));
  const size_t n = (size_t)rows * cols * dtype_size(dtype);
  if (overlap(u, n, g, n)) return fail(EE_ERR_INVALID_ARG, "u and g overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  EE_LAUNCH("bias_gelu", s, launch_bias_gelu(dtype, u, bias, rows, cols, cols, gelu, g, s));
  return EE_OK;
}

ee_status ee_attention_varlen(const void* qkv, const int32_t* d_cu, int32_t batch, int32_t max_len, int32_t n_heads,
                              int32_t head_dim, int64_t total_tokens, int32_t causal, ee_dtype dtype, void* o,
                              void* stream) {
  if (!dtype_ok(ev(dtype))) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", ev(dtype));
  if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(EE_ERR_UNSUPPORTED, "head_dim %d not in {16, 32, 64, 128}", head_dim);
  if (batch < 1 || batch > 65535 || n_heads < 1 || n_heads > 65535 || max_len < 0 || total_tokens < 0)
    return fail(EE_ERR_INVALID_ARG, "bad batch/n_heads/max_len/total_tokens");
  if (!d_cu) return fail(EE_ERR_INVALID_ARG, "d_cu is NULL");
  if (total_tokens == 0 || max_len == 0) return EE_OK;
  EE_TRY(check_ptr(qkv, "qkv"));
  EE_TRY(check_ptr(o, "o"));
  const size_t s = dtype_size(dtype), Hp = (size_t)n_heads * head_dim;
  if (overlap(qkv, (size_t)total_tokens * 3 * Hp * s, o, (size_t)total_tokens * Hp * s))
    return fail(EE_ERR_INVALID_ARG, "qkv and o overlap");
  hipStream_t st = static_cast<hipStream_t>(stream);
  EE_LAUNCH("attention", st, launch_attention(dtype, qkv, d_cu, batch, max_len, n_heads, head_dim, causal != 0, o, st));
  return EE_OK;
}

ee_status ee_attention_padded(const void* q, const void* k, const void* v, const int32_t* d_cu, int32_t batch,
                              int32_t pad_len, int32_t n_heads, int32_t head_dim, int32_t causal, ee_dtype dtype,
                              void* o, void* stream) {
  if (!dtype_ok(ev(dtype))) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", ev(dtype));
  if (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(EE_ERR_UNSUPPORTED, "head_dim %d not in {16, 32, 64, 128}", head_dim);
  if (batch < 1 || batch > 65535 || n_heads < 1 || n_heads > 65535 || pad_len < 1)
    return fail(EE_ERR_INVALID_ARG, "bad batch/n_heads/pad_len");
  if (!d_cu) return fail(EE_ERR_INVALID_ARG, "d_cu is NULL");
  EE_TRY(check_ptr(q, "q"));
  EE_TRY(check_ptr(k, "k"));
  EE_TRY(check_ptr(v, "v"));
  EE_TRY(check_ptr(o, "o"));
  const size_t n = (size_t)batch * n_heads * pad_len * head_dim * dtype_size(dtype);
  if (overlap(o, n, q, n) || overlap(o, n, k, n) || overlap(o, n, v, n))
    return fail(EE_ERR_INVALID_ARG, "o overlaps q, k or v");
  hipStream_t st = static_cast<hipStream_t>(stream);
  EE_LAUNCH("attention", st,
            launch_attention_padded(dtype, q, k, v, d_cu, batch, pad_len, n_heads, head_dim, causal != 0, o, st));
  return EE_OK;
}

ee_status ee_transpose_padding_rebuild_heads(const void* d_packed, const int32_t* seq_lens, int32_t batch,
                                             int32_t pad_len, int32_t n_mats, int32_t n_heads, int32_t head_dim,
                                             ee_dtype dtype, void* d_heads, void* workspace, size_t ws_bytes,
                                             void* stream) {
  if (n_mats < 1 || n_heads < 1 || head_dim < 1) return fail(EE_ERR_INVALID_ARG, "n_mats, n_heads, head_dim >= 1");
  if (!dtype_ok(ev(dtype))) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", ev(dtype));
  if ((size_t)head_dim * dtype_size(dtype) % 16) return fail(EE_ERR_UNSUPPORTED, "head_dim*sizeof(dtype) % 16 != 0");
  int64_t T = 0;
  Plan p{};
  const int32_t width = n_mats * n_heads * head_dim;
  EE_TRY(padding_common(d_packed, seq_lens, batch, pad_len, width, ev(dtype), d_heads, workspace, ws_bytes, &T, &p));
  const size_t es = dtype_size(dtype);
  if (overlap(d_packed, (size_t)T * width * es, d_heads, (size_t)batch * pad_len * width * es) ||
      overlap(workspace, p.total, d_heads, (size_t)batch * pad_len * width * es) ||
      overlap(workspace, p.total, d_packed, (size_t)T * width * es))
    return fail(EE_ERR_INVALID_ARG, "buffers overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* cu = reinterpret_cast<int32_t*>(at(workspace, p.cu));
  EE_TRY(offsets_from_host(seq_lens, batch, pad_len, cu, reinterpret_cast<int32_t*>(at(workspace, p.token_src)),
                           reinterpret_cast<int32_t*>(at(workspace, p.pad2pack)), s));
  EE_LAUNCH("rebuild_heads", s,
            launch_rebuild_heads(d_packed, cu, batch, n_heads, pad_len, head_dim * (int)es, n_mats, d_heads, s));
  return EE_OK;
}

ee_status ee_transpose_padding_remove_heads(const void* d_heads, const int32_t* seq_lens, int32_t batch,
                                            int32_t pad_len, int32_t n_heads, int32_t head_dim, ee_dtype dtype,
                                            void* d_packed, void* workspace, size_t ws_bytes, void* stream) {
  if (n_heads < 1 || head_dim < 1) return fail(EE_ERR_INVALID_ARG, "n_heads, head_dim >= 1");
  if (!dtype_ok(ev(dtype))) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", ev(dtype));
  if ((size_t)head_dim * dtype_size(dtype) % 16) return fail(EE_ERR_UNSUPPORTED, "head_dim*sizeof(dtype) % 16 != 0");
  int64_t T = 0;
  Plan p{};
  const int32_t width = n_heads * head_dim;
  EE_TRY(padding_common(d_heads, seq_lens, batch, pad_len, width, ev(dtype), d_packed, workspace, ws_bytes, &T, &p));
  const size_t es = dtype_size(dtype);
  if (overlap(d_packed, (size_t)T * width * es, d_heads, (size_t)batch * pad_len * width * es) ||
      overlap(workspace, p.total, d_heads, (size_t)batch * pad_len * width * es) ||
      overlap(workspace, p.total, d_packed, (size_t)T * width * es))
    return fail(EE_ERR_INVALID_ARG, "buffers overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* cu = reinterpret_cast<int32_t*>(at(workspace, p.cu));
  EE_TRY(offsets_from_host(seq_lens, batch, pad_len, cu, reinterpret_cast<int32_t*>(at(workspace, p.token_src)),
                           reinterpret_cast<int32_t*>(at(workspace, p.pad2pack)), s));
  EE_LAUNCH("remove_heads", s, launch_remove_heads(d_heads, cu, batch, n_heads, pad_len, head_dim * (int)es, d_packed, s));
  return EE_OK;
}

ee_status ee_add_bias_residual_layernorm(const void* u, const void* bias, const void* residual, const void* gamma,
                                         const void* beta, int64_t rows, int32_t hidden, float eps, ee_dtype dtype,
                                         void* y, void* stream) {
  if (!dtype_ok(ev(dtype))) return fail(EE_ERR_INVALID_ARG, "unknown dtype %d", ev(dtype));
  if (rows < 0) return fail(EE_ERR_INVALID_ARG, "rows < 0");
  if (hidden < 1 || (size_t)hidden * dtype_size(dtype) % 16)
    return fail(EE_ERR_UNSUPPORTED, "hidden*sizeof(dtype) must be a positive multiple of 16 bytes");
  if (hidden > layernorm_max_hidden(dtype)) return fail(EE_ERR_UNSUPPORTED, "hidden %d too large", hidden);
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(EE_ERR_INVALID_ARG, "eps must be finite and > 0");
  EE_TRY(check_ptr(bias, "bias"));
  EE_TRY(check_ptr(gamma, "gamma"));
  EE_TRY(check_ptr(beta, "beta"));
  if (rows == 0) return EE_OK;
  EE_TRY(check_ptr(u, "u"));
  EE_TRY(check_ptr(residual, "residual"));
  EE_TRY(check_ptr(y, "y"));
  const size_t n = (size_t)rows * hidden * dtype_size(dtype);
  if (overlap(y, n, u, n) || overlap(y, n, residual, n)) return fail(EE_ERR_INVALID_ARG, "y overlaps an input");
  hipStream_t s = static_cast<hipStream_t>(stream);
  EE_LAUNCH("add_bias_residual_ln", s,
            launch_add_bias_residual_layernorm(dtype, u, bias, residual, gamma, beta, rows, hidden, eps, y, s));
  return EE_OK;
}

ee_status ee_debug_sync(int32_t on) {
  g_debug_sync.store(on != 0);
  return EE_OK;
}

ee_status ee_profile_enable(int32_t on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.on = on != 0;
  return EE_OK;
}

ee_status ee_profile_filter(const char* site) {
  const size_t n = site ? std::strlen(site) : 0;
  if (n >= sizeof(ee_kernel_stat{}.name)) return fail(EE_ERR_INVALID_ARG, "site name of %zu characters", n);
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.only.assign(site ? site : "", n);
  return EE_OK;
}

ee_status ee_profile_collect(ee_kernel_stat* out, int32_t capacity, int32_t* count) {
  if (!count || (capacity > 0 && !out)) return fail(EE_ERR_INVALID_ARG, "out/count must be non-NULL");
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  // one row per (site, kernel) pair, in the order first seen
  struct Agg {
    std::string site;
    const char* kernel = nullptr;
    int64_t launches = 0;
    double ms = 0.0, flops = 0.0;
  };
  std::vector<Agg> rows;
  std::map<std::pair<std::string, std::string>, size_t> index;
  for (const auto& r : p.recs) {
    const auto& ev = p.pool[r.event];
    hipError_t e = hipEventSynchronize(ev.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev.first, ev.second);
    if (e != hipSuccess) {
      p.recs.clear();
      p.used = 0;
      return hip_fail(e, "profile event");
    }
    const auto key = std::make_pair(r.site, std::string(r.kernel ? r.kernel : ""));
    auto it = index.find(key);
    if (it == index.end()) {
      it = index.emplace(key, rows.size()).first;
      rows.push_back(Agg{r.site, r.kernel});
    }
    Agg& a = rows[it->second];
    a.launches += 1;
    a.ms += ms;
    a.flops += r.flops;
  }
  int32_t n = 0;
  for (const Agg& a : rows) {
    if (n < capacity) {
      ee_kernel_stat& k = out[n];
      std::memset(&k, 0, sizeof k);
      std::strncpy(k.name, a.site.c_str(), sizeof k.name - 1);
      k.launches = a.launches;
      k.total_ms = a.ms;
      k.flops = a.flops;
      if (a.kernel) std::strncpy(k.kernel, a.kernel, sizeof k.kernel - 1);
    }
    ++n;
  }
  *count = std::min(n, capacity);
  p.recs.clear();
  p.used = 0;
  return EE_OK;
}

}  // extern "C"
