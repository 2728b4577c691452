/*
 * ee.h -- C ABI of libee: the forward pass of a pre-LN GPT decoder layer with
 * redundant-computation elimination (RCE) on one AMD Instinct MI355X (gfx950).
 *
 * The method: the Energon-AI announcement article (Colossal-AI team), "Runtime"
 * section, adds two ops, transpose_padding_remove and transpose_padding_rebuild,
 * so that the layers of encoder and decoder models do no work on the padding of
 * variable-length inputs; the EnergonAI README ("Scaling Ability", "Latency")
 * runs GPT-3 layers in FP16 with that method, with sequence length half the
 * padding length.  This library computes, on one GPU:
 *
 *   offsets:  per-sequence lengths (or the attention mask) prefix-summed into
 *             packed token offsets;
 *   remove:   padded [batch, pad_len, hidden] -> packed [T, hidden], T = sum(len);
 *   layer:    LayerNorm, the QKV / out-projection / MLP GEMMs and GeLU on the T
 *             valid rows only; attention causally per sequence over the offsets;
 *   rebuild:  packed [T, hidden] -> padded [batch, pad_len, hidden], pads +0.0.
 *
 * Conventions (all entry points):
 *   - Every device pointer is caller-owned device memory (hipMalloc or any
 *     allocator), 16-byte aligned, row-major and dense.  Host pointers are
 *     marked "host".  The library never frees caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on `stream`: no device synchronisation,
 *     no device-to-host copy, no allocation in the forward path.
 *   - Arguments are validated on the host BEFORE any device work; a failed
 *     check returns EE_ERR_INVALID_ARG / EE_ERR_UNSUPPORTED / EE_ERR_WORKSPACE
 *     and enqueues nothing.  A HIP launch error returns EE_ERR_HIP; an
 *     asynchronous fault of earlier work may surface as EE_ERR_HIP on a later
 *     call.  ee_last_error() gives a thread-local message for the last failure.
 *   - No call works in place: outputs must not overlap inputs.
 *   - Per-sequence lengths are host int32 values in [0, pad_len] (the batcher
 *     that built the batch knows them); they reach the device as kernel
 *     arguments, so the caller's array may be reused as soon as the call
 *     returns.  batch <= EE_MAX_BATCH.
 *   - Weights use the nn.Linear [out, in] layout.  The fused QKV weight is
 *     [3*n_heads*head_dim, hidden]: rows q | k | v, each block head-major.
 *   - Thread safety: distinct layer handles may be used from distinct threads;
 *     one handle's calls must not run concurrently.
 */
#ifndef EE_H_
#define EE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define EE_API __attribute__((visibility("default")))
#else
#define EE_API
#endif

#define EE_MAX_BATCH 512
#define EE_MAX_EXTEND_BATCH 256

typedef enum {
  EE_OK = 0,
  EE_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, overlapping buffers */
  EE_ERR_UNSUPPORTED = 2, /* valid request the kernels do not cover (head_dim, sizes) */
  EE_ERR_WORKSPACE = 3,   /* workspace smaller than the ..._workspace_size result */
  EE_ERR_OOM = 4,         /* host allocation failed (handles only) */
  EE_ERR_HIP = 5          /* a HIP runtime call failed */
} ee_status;

/* Storage type of activations and weights.  Arithmetic is fp32 in both cases
 * (fp16 storage with fp32 accumulation is the pages' `half = True` setting,
 * announcement article, "Ease of use" config). */
typedef enum { EE_F32 = 0, EE_F16 = 1 } ee_dtype;

/* GeLU form: tanh approximation (GPT-2/3 default) or the erf definition. */
typedef enum { EE_GELU_TANH = 0, EE_GELU_ERF = 1 } ee_gelu;

/* Epilogue of ee_linear: C = A W^T (+ bias) (+ residual) or gelu(A W^T + bias). */
typedef enum {
  EE_EPI_NONE = 0,
  EE_EPI_BIAS = 1,
  EE_EPI_BIAS_RESIDUAL = 2,
  EE_EPI_BIAS_GELU = 3
} ee_epilogue;

/* Block form.  GPT_PRELN: the pre-LN causal decoder block,
 *   a = LN1(x); h = x + Out(Attn(QKV(a))); y = h + FC2(gelu(FC1(LN2(h)))).
 * BERT_POSTLN: the post-LN bidirectional encoder block (the EnergonAI README
 * lists BERT among its models), with the add bias + input + LayerNorm step of
 * the announcement article's "Ease of use" listing after each sublayer:
 *   h = LN1(x + Out(Attn(QKV(x)))); y = LN2(h + FC2(gelu(FC1(h)))). */
typedef enum { EE_BLOCK_GPT_PRELN = 0, EE_BLOCK_BERT_POSTLN = 1 } ee_block;

/* Attention form.  VARLEN: per sequence directly over the packed rows.
 * PADDED: the page-literal form of the announcement article's "Runtime"
 * section (remove/rebuild around the MLP layers): a transposing rebuild scatters
 * the packed q|k|v into head-major padded [B, nh, P, hd] tensors, attention runs
 * on them with the key mask, a transposing remove gathers the output back.
 * Valid rows are the same either way. */
typedef enum { EE_ATTN_VARLEN = 0, EE_ATTN_PADDED = 1 } ee_attention;

/* Where the pre-LN block adds its two residuals (out projection + x, FC2 +
 * h).  EPILOGUE: inside the GEMM's store, one rounding of acc + bias + residual.
 * PASS: the GEMM stores acc + bias (rounded); a separate pass forms the rounded
 * sum and, after the out projection, the second LayerNorm of it in the same
 * pass.  At GPT-3 width and 4096 rows the two run at the same speed (the out
 * GEMM gains what the passes' extra 200 MB per layer cost), so AUTO is
 * EPILOGUE: one rounding, less traffic.  Post-LN blocks always add in their
 * bias + residual + LayerNorm pass. */
typedef enum { EE_RESIDUAL_AUTO = 0, EE_RESIDUAL_EPILOGUE = 1, EE_RESIDUAL_PASS = 2 } ee_residual;

typedef struct {
  int32_t hidden;    /* H */
  int32_t n_heads;   /* nh */
  int32_t head_dim;  /* hd in {16, 32, 64, 128}; H' = nh*hd */
  int32_t ffn;       /* F */
  float ln_eps;      /* LayerNorm epsilon (inside the square root), e.g. 1e-5 */
  ee_dtype dtype;
  ee_gelu gelu;
  int32_t fuse_gelu; /* 1: bias+GeLU in the FC1 GEMM epilogue; 0: separate bias+GeLU kernel */
  ee_block block;
  ee_attention attention;
  ee_residual residual;  /* where a pre-LN layer adds its residuals (EE_RESIDUAL_AUTO if unsure) */
} ee_layer_desc;

/* Device pointers, all of the descriptor's dtype, borrowed (not copied) by
 * ee_layer_create for the handle's lifetime.  Each weight matrix is
 * [out, in], row-major.  Its rows may sit ld_* elements apart: 0 means dense
 * (ld = in); a nonzero ld must be >= in and keep rows 16-byte aligned
 * (ld * element size % 16 == 0).  ee_preferred_row_pitch gives a pitch that
 * spreads the rows over the HBM channels. */
typedef struct {
  const void *ln1_g, *ln1_b;   /* [H] */
  const void *w_qkv, *b_qkv;   /* [3H', H], [3H'] */
  const void *w_out, *b_out;   /* [H, H'],  [H] */
  const void *ln2_g, *ln2_b;   /* [H] */
  const void *w_fc1, *b_fc1;   /* [F, H],   [F] */
  const void *w_fc2, *b_fc2;   /* [H, F],   [H] */
  int64_t ld_qkv, ld_out, ld_fc1, ld_fc2;  /* row pitches of the four matrices (0: dense) */
} ee_layer_weights;

typedef struct ee_layer ee_layer;

/* ---- status ------------------------------------------------------------ */
EE_API const char* ee_status_string(ee_status s);
/* Thread-local detail of the last non-OK status returned on this thread. */
EE_API const char* ee_last_error(void);
/* Library version string. */
EE_API const char* ee_version(void);

/* ---- layer handle (announcement article, "Runtime": the RCE layer forward) -- */
/* Validates the descriptor and borrows the weight pointers.  No device work. */
EE_API ee_status ee_layer_create(const ee_layer_desc* desc, const ee_layer_weights* weights, ee_layer** out);
EE_API ee_status ee_layer_destroy(ee_layer* layer);

/* Device workspace bytes that ee_layer_forward / ee_stack_forward need for
 * `batch` sequences padded to `pad_len` holding at most `max_tokens` valid
 * tokens (max_tokens < 0 means batch*pad_len).  Holds the offsets, the packed
 * activations and every intermediate of one layer, 256-byte aligned. */
EE_API ee_status ee_layer_workspace_size(const ee_layer* layer, int32_t batch, int32_t pad_len,
                                  int64_t max_tokens, size_t* bytes);

/* One layer: offsets, remove, the packed layer, rebuild.
 *   x_padded  [batch, pad_len, H] device, layer dtype (pads may hold anything,
 *             NaN included: no pad value reaches a valid row)
 *   seq_lens  [batch] host int32 in [0, pad_len] (right padding)
 *   y_padded  [batch, pad_len, H] device; valid rows = layer output,
 *             pads = +0.0 (all zeros when every length is 0) */
EE_API ee_status ee_layer_forward(ee_layer* layer, const void* x_padded, const int32_t* seq_lens,
                           int32_t batch, int32_t pad_len, void* y_padded,
                           void* workspace, size_t ws_bytes, void* stream);

/* A stack (the EnergonAI README, "Scaling Ability" and "Latency": GPT-3
 * stacks of 12, 24 and 48 layers with redundant-computation elimination):
 * n_layers layers with one offsets/remove before and one rebuild after; the
 * packed output of layer l is the input of layer l+1, so the padding is
 * removed once per stack.  All layers must share one descriptor.  Arguments
 * and errors as ee_layer_forward, plus EE_ERR_INVALID_ARG for n_layers < 1, a
 * NULL layer or layers with different descriptors.  The workspace is that of
 * one layer (ee_layer_workspace_size): layers reuse it in turn. */
EE_API ee_status ee_stack_forward(ee_layer* const* layers, int32_t n_layers, const void* x_padded,
                           const int32_t* seq_lens, int32_t batch, int32_t pad_len,
                           void* y_padded, void* workspace, size_t ws_bytes, void* stream);

/* ---- offsets (the attention mask prefix-summed into token offsets) ------- */
/* The packed position of every valid token, which the announcement article's
 * "Runtime" ops need to move rows between the padded and the packed layout
 * (the README's "Scaling Ability" and "Latency" runs give each sequence a
 * length below the padding length).
 * From host lengths.  Writes, on `stream`:
 *   d_cu        [batch+1]        cu[0]=0, cu[b+1]=cu[b]+len[b]
 *   d_token_src [batch*pad_len]  token_src[t] = b*pad_len + t - cu[b] for t < T
 *                                (entries >= T are left untouched)
 *   d_pad2pack  [batch*pad_len]  cu[b]+p for p < len[b], else -1
 * and T = sum(len) into *total_tokens (host, computed before any device work). */
EE_API ee_status ee_compute_offsets(const int32_t* seq_lens, int32_t batch, int32_t pad_len,
                             int32_t* d_cu, int32_t* d_token_src, int32_t* d_pad2pack,
                             int32_t* total_tokens, void* stream);

/* From a device mask [batch, pad_len] (nonzero byte = valid token): its
 * flattened exclusive prefix sum gives each valid position its packed index.
 * Same outputs as above (any mask, not only right-padded ones); T goes to the
 * device int32 *d_total.  batch*pad_len <= 2^31 - 1. */
EE_API ee_status ee_compute_offsets_mask(const uint8_t* d_mask, int32_t batch, int32_t pad_len,
                                  int32_t* d_cu, int32_t* d_token_src, int32_t* d_pad2pack,
                                  int32_t* d_total, void* stream);

/* ---- transpose_padding_remove / transpose_padding_rebuild --------------- */
/* Bytes of workspace the two calls below need (the offsets arrays). */
EE_API ee_status ee_padding_workspace_size(int32_t batch, int32_t pad_len, size_t* bytes);

/* transpose_padding_remove (announcement article, "Runtime"), read as a row
 * gather: packed[t, :] = padded[token_src[t], :], the valid rows in sequence
 * order.  d_padded [batch, pad_len, hidden], d_packed [T, hidden] (T =
 * sum(len), caller-owned, at least T rows); hidden*sizeof(dtype) % 16 == 0.
 * seq_lens host.  workspace: ee_padding_workspace_size(batch, pad_len) bytes of
 * device memory (the offsets arrays, rewritten by the call).  Errors:
 * EE_ERR_INVALID_ARG for lengths outside [0, pad_len], batch outside
 * [1, EE_MAX_BATCH], NULL or misaligned pointers, overlapping buffers;
 * EE_ERR_UNSUPPORTED for a row that is not a multiple of 16 bytes;
 * EE_ERR_WORKSPACE for a small workspace. */
EE_API ee_status ee_remove_padding(const void* d_padded, const int32_t* seq_lens, int32_t batch,
                            int32_t pad_len, int32_t hidden, ee_dtype dtype, void* d_packed,
                            void* workspace, size_t ws_bytes, void* stream);

/* transpose_padding_rebuild (announcement article, "Runtime"; spelt
 * "rebulid" there), read as a row scatter: padded[r, :] = packed[pad2pack[r], :],
 * or +0.0 (bit pattern 0) where pad2pack[r] = -1, i.e. on every pad row, so the
 * whole [batch, pad_len, hidden] output is written.  Arguments, workspace and
 * errors as ee_remove_padding. */
EE_API ee_status ee_rebuild_padding(const void* d_packed, const int32_t* seq_lens, int32_t batch,
                             int32_t pad_len, int32_t hidden, ee_dtype dtype, void* d_padded,
                             void* workspace, size_t ws_bytes, void* stream);

/* ---- the layer's operations on packed rows (each a step of the forward) ---- */
/* y[r] = (x[r] - mean) / sqrt(var + eps) * gamma + beta per row, biased
 * variance, fp32 statistics.  x, y [rows, hidden]; gamma, beta [hidden]. */
EE_API ee_status ee_layernorm(const void* x, const void* gamma, const void* beta, int64_t rows,
                       int32_t hidden, float eps, ee_dtype dtype, void* y, void* stream);

/* C[M, N] = epilogue(A[M, K] . W[N, K]^T): bias [N], residual [M, N] (may not
 * alias C).  fp16: MFMA kernels, fp32 accumulation, one rounding to fp16 at
 * the end; row r of C depends only on row r of A (and of the residual).  Every
 * kernel adds an element's K tiles in the same order, so the bits do not
 * depend on M either, and a sequence gives the same result alone or in any
 * batch -- provided the two MFMA shapes the kernels use (16x16x32 for large
 * problems, 32x32x16 for small ones and for the rows past whole rounds of
 * large tiles) sum a K step in the same way.  That is measured on gfx950, not
 * derived from a specification: random-data tests compare large GEMMs with
 * GEMMs over each 256-row block alone (test_gemm_row_split_bit_identical) and
 * sequences of 48-layer batches run alone (test_stream_sequence_alone_equals_batch).
 * fp32: fp32 FMA kernels.  M may be 0 (no work).  All matrices dense;
 * ee_linear_strided is the general form. */
EE_API ee_status ee_linear(const void* A, const void* W, const void* bias, const void* residual,
                    int64_t M, int32_t N, int32_t K, ee_dtype dtype, ee_epilogue epi,
                    ee_gelu gelu, void* C, void* stream);

/* ee_linear with row pitches, in elements: A [M, lda], W [N, ldw], C and the
 * residual [M, ldc], with lda >= K, ldw >= K, ldc >= N (the columns past
 * K or N are neither read nor written).  The fp16 MFMA kernels take K % 64
 * == 0 with lda, ldw multiples of 8 and 16-byte aligned A and W; other fp16
 * shapes run on the fp32 FMA kernels.  Errors as ee_linear, plus
 * EE_ERR_INVALID_ARG for a pitch below its row length or above 2^31 - 1. */
EE_API ee_status ee_linear_strided(const void* A, int64_t lda, const void* W, int64_t ldw, const void* bias,
                                   const void* residual, int64_t M, int32_t N, int32_t K, ee_dtype dtype,
                                   ee_epilogue epi, ee_gelu gelu, void* C, int64_t ldc, void* stream);

/* ee_linear_strided with a workspace of at least ee_linear_ws_workspace_size()
 * bytes (device memory, not read before it is written; the caller keeps it).
 * A large fp16 problem runs as one persistent launch of one workgroup per CU
 * over 256 x 256 tiles, or 256 x 384 where N is a multiple of 384 and that
 * is estimated to end sooner.  When the tiles leave that launch's last round
 * partial, its tiles are shared out as stream-K pieces (Osama et al., PPoPP
 * 2023): equal contiguous ranges of (tile, K tile) steps, one per workgroup.
 * A piece that starts inside a tile continues, in the same fp32 accumulators,
 * from the sums its predecessor left in the workspace, so each element still
 * adds its K tiles in one chain, in order: the result is bit for bit that of
 * ee_linear_strided, which runs the remaining rows as a second launch on
 * other tiles instead (every tile shape adds an element's K tiles in the
 * same order; the MFMA shapes' equal sums are measured on gfx950, see
 * ee_linear).  The workspace holds 4 KiB of flags and one 256 x 384 fp32
 * tile per CU (96 MiB + 4 KiB).  Calls that share a workspace must not overlap in
 * time (one stream).  fp32 and small problems run as ee_linear_strided.
 * Errors as ee_linear_strided, plus EE_ERR_WORKSPACE for a small workspace
 * and EE_ERR_INVALID_ARG for a workspace overlapping an operand. */
EE_API size_t ee_linear_ws_workspace_size(void);
EE_API ee_status ee_linear_ws(const void* A, int64_t lda, const void* W, int64_t ldw, const void* bias,
                              const void* residual, int64_t M, int32_t N, int32_t K, ee_dtype dtype,
                              ee_epilogue epi, ee_gelu gelu, void* C, int64_t ldc, void* ws, size_t ws_bytes,
                              void* stream);

/* The row pitch, in elements, that the library gives a matrix of `cols`
 * columns it stores itself (the FC1 output in the layer workspace), and the
 * one it suggests for weights: cols, plus 128 bytes when a row is a multiple
 * of 32 KiB.  Such strides put every row of a GEMM panel on the same few HBM
 * channels (K = 49152 fp16: 7% slower without the padding).  Returns 0 for
 * cols < 1 or an unknown dtype. */
EE_API int64_t ee_preferred_row_pitch(int64_t cols, ee_dtype dtype);

/* ee_linear for fp16 with the K dimension split: `splits` workgroup rows each
 * sum an equal K range (K % (64 * splits) == 0) into fp32 partials in the
 * workspace (ee_linear_splitk_workspace_size bytes), and a second kernel adds
 * the partials in split order and applies the epilogue.  For small M (e.g. a
 * decode step, M = batch), where the unsplit grid has too few workgroups to
 * stream W at full bandwidth; the layer calls choose the split themselves.
 * Errors: EE_ERR_UNSUPPORTED for fp32 or shapes the fp16 kernels do not take;
 * EE_ERR_WORKSPACE for a small workspace. */
EE_API ee_status ee_linear_splitk_workspace_size(int64_t M, int32_t N, int32_t splits, size_t* bytes);
EE_API ee_status ee_linear_splitk(const void* A, const void* W, const void* bias, const void* residual,
                                  int64_t M, int32_t N, int32_t K, ee_dtype dtype, ee_epilogue epi, ee_gelu gelu,
                                  int32_t splits, void* C, void* ws, size_t ws_bytes, void* stream);

/* ee_linear for fp16 with at most 128 rows of A (a decode step of up to 128
 * sequences), decomposed stream-K (Osama et al., "Stream-K: Work-centric
 * Parallel Decomposition for Dense Matrix-Matrix Multiplication", PPoPP 2023):
 * the (256-row N tile, 64-wide K tile) space of W is cut into equal
 * contiguous ranges, one per workgroup, whose fp32 partial sums go to the
 * workspace (ee_linear_streamk_workspace_size bytes, M x 1 KiB per slot,
 * depends on M, N, K and the device's CU count); a second kernel adds each
 * tile's pieces in K order and applies the epilogue.  The layer's extend step
 * uses it whenever it takes the shape and its partials fit the extend
 * workspace's 64 MiB.  Arguments as ee_linear; A, W, C and the residual dense.
 * Errors: EE_ERR_UNSUPPORTED for fp32, M > 128, K % 64 != 0 or a problem too
 * small to give each workgroup 8 K tiles; EE_ERR_WORKSPACE for a small
 * workspace; EE_ERR_INVALID_ARG for overlapping buffers. */
EE_API ee_status ee_linear_streamk_workspace_size(int64_t M, int32_t N, int32_t K, size_t* bytes);
EE_API ee_status ee_linear_streamk(const void* A, const void* W, const void* bias, const void* residual,
                                   int64_t M, int32_t N, int32_t K, ee_dtype dtype, ee_epilogue epi, ee_gelu gelu,
                                   void* C, void* ws, size_t ws_bytes, void* stream);

/* g[r, c] = gelu(u[r, c] + bias[c]): the standalone form of the FC1 epilogue
 * (announcement article, "Ease of use" listing: add bias + activation). */
EE_API ee_status ee_bias_gelu(const void* u, const void* bias, int64_t rows, int32_t cols, ee_dtype dtype,
                       ee_gelu gelu, void* g, void* stream);

/* Attention per sequence over packed offsets.  qkv [T, 3H'] (q | k | v,
 * head-major), d_cu [batch+1] device int32 (e.g. from ee_compute_offsets),
 * o [T, H'].  Query i of sequence b attends with weights
 * softmax(q.k / sqrt(head_dim)) to keys cu[b] .. cu[b]+i (causal != 0) or to
 * all keys of its sequence (causal == 0); max_len >= every sequence length. */
EE_API ee_status ee_attention_varlen(const void* qkv, const int32_t* d_cu, int32_t batch, int32_t max_len,
                              int32_t n_heads, int32_t head_dim, int64_t total_tokens, int32_t causal,
                              ee_dtype dtype, void* o, void* stream);

/* The same attention on padded head-major tensors q, k, v, o [batch, n_heads,
 * pad_len, head_dim], lengths from d_cu [batch+1]: keys j < len[b] (and j <= i
 * when causal) of the same (sequence, head); rows p >= len[b] of o are not
 * written. */
EE_API ee_status ee_attention_padded(const void* q, const void* k, const void* v, const int32_t* d_cu,
                                     int32_t batch, int32_t pad_len, int32_t n_heads, int32_t head_dim,
                                     int32_t causal, ee_dtype dtype, void* o, void* stream);

/* Transposing rebuild (announcement article, "Runtime"): packed [T, n_mats *
 * n_heads * head_dim] (n_mats column blocks, each head-major) -> d_heads
 * [n_mats, batch, n_heads, pad_len, head_dim], pads +0.0.  seq_lens host;
 * workspace: ee_padding_workspace_size bytes.  head_dim*sizeof(dtype) % 16 == 0. */
EE_API ee_status ee_transpose_padding_rebuild_heads(const void* d_packed, const int32_t* seq_lens, int32_t batch,
                                                    int32_t pad_len, int32_t n_mats, int32_t n_heads,
                                                    int32_t head_dim, ee_dtype dtype, void* d_heads,
                                                    void* workspace, size_t ws_bytes, void* stream);

/* Transposing remove: d_heads [batch, n_heads, pad_len, head_dim] -> packed
 * [T, n_heads * head_dim] (valid rows only). */
EE_API ee_status ee_transpose_padding_remove_heads(const void* d_heads, const int32_t* seq_lens, int32_t batch,
                                                   int32_t pad_len, int32_t n_heads, int32_t head_dim,
                                                   ee_dtype dtype, void* d_packed, void* workspace,
                                                   size_t ws_bytes, void* stream);

/* y = LN(u + bias + residual) per row (the add bias + input + LayerNorm step
 * of the announcement article's "Ease of use" listing); the sum is formed in
 * fp32 and not stored.  u, residual, y [rows, hidden]; bias, gamma, beta [hidden]. */
EE_API ee_status ee_add_bias_residual_layernorm(const void* u, const void* bias, const void* residual,
                                                const void* gamma, const void* beta, int64_t rows, int32_t hidden,
                                                float eps, ee_dtype dtype, void* y, void* stream);

/* ---- per-kernel timing ----------------------------------------------------- */
/* While enabled, every kernel that the calls above launch from this process is
 * bracketed by a pair of hipEvents recorded on its launch stream.  A GEMM site
 * whose rows run as two launches (whole rounds of 256-row tiles, then the
 * remaining rows on smaller tiles) records the second as site "<site>_rest",
 * e.g. "gemm_fc1_rest". */
typedef struct {
  char name[32];      /* launch site, e.g. "gemm_fc1", "attention", "remove" */
  int64_t launches;
  double total_ms;    /* sum of event-measured durations */
  double flops;       /* sum of the launches' algorithmic flops (GEMM sites: 2*rows*N*K; else 0) */
  char kernel[96];    /* the kernel these launches ran, e.g. "gemm_f16_mfma_kernel<16, 256, 256, 2, 2, 3, 2, false>"
                         (template arguments in declaration order), or "" if not recorded */
} ee_kernel_stat;

EE_API ee_status ee_profile_enable(int32_t on);
/* Debug mode: while on, every kernel launch of the calls above is followed by
 * hipStreamSynchronize of its stream, so an asynchronous failure (a memory
 * fault, an illegal instruction) is returned as EE_ERR_HIP by the call that
 * launched the failing kernel, with that launch site in ee_last_error()
 * (e.g. "gemm_fc1: ..."), instead of surfacing at a later call.  It also
 * makes every call synchronous: for debugging, never under graph capture.
 * Setting EE_DEBUG_SYNC=1 in the environment before the library loads turns
 * it on from the start.  Always EE_OK. */
EE_API ee_status ee_debug_sync(int32_t on);
/* Restricts the timing to one launch site (e.g. "gemm_fc1"); NULL or "" times
 * every site again.  Each recorded event pair leaves a bubble of a few us in
 * its stream, so timing only the kernel of interest keeps the rest of the work
 * at full speed.  The name is copied.  EE_ERR_INVALID_ARG for a name of 32 or
 * more characters. */
EE_API ee_status ee_profile_filter(const char* site);
/* Waits for the recorded events, writes up to `capacity` totals into `out`
 * (host), one per (site, kernel) pair in the order first seen -- a site whose
 * launches ran different kernels (a GEMM with and without an in-order split)
 * has one row per kernel -- sets *count, and clears the record. */
EE_API ee_status ee_profile_collect(ee_kernel_stat* out, int32_t capacity, int32_t* count);

/* ---- Incremental decoding with a packed KV cache ----
 *
 * Generation (the README's "Latency" section times a GPT-3 generation
 * service; the EET page reports decoder-layer speedups): each new token of a
 * sequence attends to all earlier tokens of that sequence through their
 * cached keys and values.  One call runs an "extend" step of a layer stack:
 * sequence b brings new_len[b] >= 0 new tokens at positions
 * ctx_len[b] .. ctx_len[b] + new_len[b] - 1, after ctx_len[b] tokens whose
 * keys and values are already cached.  A prefill is an extend from
 * ctx_len = 0; a decode step brings one token per sequence.  Only the new
 * tokens are computed (the padding-free layout of the forward above).
 *
 * KV cache (caller-owned device memory, ee_kv_cache_bytes): for each layer
 * l, [2 (k | v)][n_heads][capacity][head_dim] elements of the layer dtype,
 * layers one after another.  Sequence b owns the slots
 * slot_base[b] .. slot_base[b] + ctx_len[b] + new_len[b] - 1, so sequences
 * take only the slots they use.  The call writes the new tokens' keys and
 * values of every layer into their slots and reads the cached ones; the
 * caller advances ctx_len by new_len afterwards.
 *
 * Arguments: layers as for ee_stack_forward (all GPT pre-LN, same
 * descriptor; the descriptor's attention form does not apply here).
 * d_x: device [T_new, hidden], the new tokens packed sequence by sequence
 * (T_new = sum new_len); d_y: device [T_new, hidden] output; new_len,
 * ctx_len, slot_base: host [batch], batch <= EE_MAX_EXTEND_BATCH, not kept
 * after the call.  Errors: EE_ERR_INVALID_ARG for negative counts, a slot
 * range outside [0, capacity), overlapping slot ranges of sequences with
 * tokens, overlapping buffers, or a post-LN descriptor; EE_ERR_UNSUPPORTED
 * for head_dim outside {16, 32, 64, 128} or more than
 * ee_extend_max_positions() (2^31 - 1) positions in one sequence;
 * EE_ERR_WORKSPACE when ws_bytes < ee_extend_workspace_size(layer, batch,
 * T_new).  A size taken for some T_new covers every step with fewer new
 * tokens; every size includes 64 MiB for partial sums: the small-M GEMMs'
 * split-K / stream-K pieces, and the attention's per-key-chunk softmax
 * states.  The attention over the cache splits each new token's keys into
 * chunks (512 positions, doubled until the chunks' states fit the 64 MiB)
 * and merges the chunks' softmax states in a second kernel, so no buffer
 * grows with the context. */
EE_API ee_status ee_kv_cache_bytes(const ee_layer* layer, int32_t n_layers, int64_t capacity, size_t* bytes);
EE_API ee_status ee_extend_workspace_size(const ee_layer* layer, int32_t batch, int64_t max_new_tokens,
                                          size_t* bytes);
EE_API int32_t ee_extend_max_positions(void);
EE_API ee_status ee_stack_extend(ee_layer* const* layers, int32_t n_layers, const void* d_x,
                                 const int32_t* new_len, const int32_t* ctx_len, const int32_t* slot_base,
                                 int32_t batch, void* d_cache, int64_t capacity, void* d_y, void* ws,
                                 size_t ws_bytes, void* stream);

/* ---- Extend step that allocates nothing ----
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc.  The same step
 * as ee_stack_extend (same arguments, kernels and results), with the
 * workspace in a static device buffer of EE_NOALLOC_SCRATCH_BYTES that the
 * library owns; the caller passes inputs, outputs and the cache only.  Each
 * GPU the call runs on holds its own copy of the buffer until the process
 * ends.  Every call on a GPU shares that GPU's buffer, so calls that overlap
 * in time on one GPU (from two streams or threads) race; serialise them.
 * A step whose workspace (ee_extend_workspace_size(layers[0], batch, T_new))
 * exceeds the buffer returns EE_ERR_WORKSPACE before any device work: at
 * GPT-3 width (H 12288, F 49152, 96 x 128 heads, fp16) that is about 340 new
 * tokens; decode steps of up to EE_MAX_EXTEND_BATCH sequences fit.  Other
 * errors as ee_stack_extend, plus EE_ERR_HIP if the buffer's device address
 * cannot be obtained.  No hipMalloc, hipFree or allocating library routine is
 * called; the step copies its new-token rows in and out with two
 * device-to-device copies on `stream`, as ee_stack_extend does. */
#define EE_NOALLOC_SCRATCH_BYTES (128u << 20)
EE_API ee_status ee_stack_extend_noalloc(ee_layer* const* layers, int32_t n_layers, const void* d_x,
                                         const int32_t* new_len, const int32_t* ctx_len, const int32_t* slot_base,
                                         int32_t batch, void* d_cache, int64_t capacity, void* d_y, void* stream);

/* ---- Batch planning over a request queue (host only; no device work) ----
 *
 * The announcement article's "Serving" section and the README's "Batching"
 * section: queued variable-length requests are packed into batches according
 * to how fast the machine runs them, then the batch with the highest priority
 * is run first (waiting time, batch size, how much the batch could still grow
 * at its padded length); the packing follows TurboTransformers' dynamic
 * programming scheduler.  The baseline is FIFO packing, each batch padded to
 * its longest request (the "Performance tests" section).
 *
 * Cost of running one batch of B requests with lengths len_1..len_B, padded
 * to P = max len_i:
 *   t_batch + S(tokens) + t_row * B * P + t_pair * pairs
 * tokens = sum len_i rounded up to a multiple of token_quantum (1 = no
 * rounding), pairs = sum len_i (len_i + 1) / 2 (causal attention);
 * padded_compute != 0 models a forward that keeps the padding: tokens = B * P
 * and pairs = B * P (P + 1) / 2.
 * S(tokens) = t_token * tokens, or, when token_table is given (host,
 * token_table_len >= 1 entries), the measured seconds of a batch of
 * tokens = (k + 1) * token_quantum at entry k, extended past the last entry
 * along the line through the last two (or through the origin and the only
 * one).  The coefficients and the table come from batch times measured on
 * the machine. */
typedef struct {
  double t_batch;
  double t_token;
  double t_row;
  double t_pair;
  int32_t token_quantum;
  int32_t padded_compute;
  const double* token_table;
  int32_t token_table_len;
} ee_batch_cost;

/* Cost of one batch under `cost` (as above).  lens: host, n >= 1 values >= 1. */
EE_API ee_status ee_batch_cost_eval(const int32_t* lens, int32_t n, const ee_batch_cost* cost, double* out);

/* FIFO: request i (arrival order) goes to batch i / max_batch.
 * batch_of: host [n] output; *n_batches set.  lens only checked (>= 1). */
EE_API ee_status ee_plan_fifo(const int32_t* lens, int32_t n, int32_t max_batch, int32_t* batch_of,
                              int32_t* n_batches);

/* Dynamic batching.  The requests are ordered by length (arrival order breaks
 * ties) and split into contiguous runs of that order by dynamic programming
 * over prefixes, minimising the summed batch cost subject to at most
 * max_batch requests and at most max_tokens rows per batch (rows = sum len,
 * or B * P with padded_compute; max_tokens <= 0: no limit).  Ties between
 * equal-cost splits go to the longer last batch.  The batches are then
 * numbered in priority order: longest waiting request first (wait: host [n]
 * seconds each request has waited, or NULL for all zero), then more
 * requests, then earliest arrival.
 * batch_of: host [n] output, the run position of each request's batch;
 * *n_batches set; *total_cost (may be NULL) the summed cost.
 * Errors: EE_ERR_INVALID_ARG for n < 0, max_batch < 1, a length < 1, a
 * request longer than max_tokens, or NULL outputs.  Allocates host memory. */
EE_API ee_status ee_plan_dynamic(const int32_t* lens, const double* wait, int32_t n, int32_t max_batch,
                                 int64_t max_tokens, const ee_batch_cost* cost, int32_t* batch_of,
                                 int32_t* n_batches, double* total_cost);

#ifdef __cplusplus
}
#endif
#endif /* EE_H_ */
