/*
 * libturboquant — TurboQuant KV-cache quantization and compressed-cache
 * attention for AMD Instinct MI355X (gfx950). C ABI.
 *
 * What is computed (sources are web pages, cited by title and section):
 *
 *  [ZB] zubnet.ai news, "Google's TurboQuant quantizes LLM KV cache 3.5 bits
 *       per channel, near ..." (es/pt/fr editions), paragraph 2: stage one
 *       rotates each vector at random, which gives every coordinate a Beta
 *       law, and applies an optimal scalar quantizer per coordinate; stage two
 *       applies an MSE quantizer and then a 1-bit quantized Johnson-
 *       Lindenstrauss transform of the residual; a token is stored as its
 *       quantization indices, its sign bits and an L2 norm; 3.5 and 2.5 bits
 *       per channel are named.
 *  [WD] winningdata.io blog, "TurboQuant: Google comprime KV cache para 3
 *       bits sem perder acuracia ...": section "Como o TurboQuant funciona",
 *       sub-sections "1. PolarQuant" (a product with a random orthogonal
 *       matrix, then a standard quantizer) and "2. QJL Residual" (one extra
 *       bit per value, built on Johnson-Lindenstrauss, removes the
 *       inner-product bias); the article's introduction and the table in
 *       "Os numeros que importam" put the speed-up in the attention logits
 *       computed from the compressed cache.
 *
 * The readings this library takes where the pages are silent:
 *  - Pi is a dense d_g x d_g orthogonal matrix and the quantizer acts on the
 *    unit vector y = Pi x_g / ||x_g||; its per-coordinate law has density
 *    proportional to (1 - y^2)^((d_g - 3)/2) on [-1, 1].
 *  - The scalar quantizer is Lloyd-Max (minimum MSE) for that density, with
 *    2^m levels; a coordinate's code is the number of decision boundaries
 *    (midpoints of neighbouring centroids) strictly below it.
 *  - b bits per channel = m = b - 1 Lloyd-Max bits + 1 sign bit of a
 *    d_g x d_g Gaussian sketch S of the residual r = x_g - n Pi^T c[idx].
 *  - Two norms per group are stored: n = ||x_g|| and gamma = ||r||.
 *  - Dequantization: x~_g = n Pi^T c[idx] + alpha gamma S^T z with
 *    z = +-1 (bit 1 -> +1) and alpha = sqrt(pi/2) / d_g, which is unbiased.
 *  - Fractional widths are two independent instances on a channel split:
 *    channels are permuted, cut into two consecutive groups, and each group
 *    has its own rotation, sketch, codebook and norms.
 *  - Queries are not quantized; logit = scale * <q, k~>; a decode step
 *    attends over every cached token; query head h reads KV head
 *    floor(h / (n_q_heads / n_kv_heads)).
 *
 * Conventions for every entry point:
 *  - Every function returns a tq_status. Arguments are validated on the host
 *    before any HIP call; on an error nothing is launched and no output is
 *    written.
 *  - Device pointers are plain device addresses (e.g. from hipMalloc or a
 *    torch tensor) and must be 16-byte aligned. The caller owns every
 *    buffer, including the decode workspace; the library allocates nothing,
 *    keeps no mutable global state (apart from the static workspace of
 *    tq_attn_decode_scratch) and never synchronizes: kernels are
 *    enqueued on `stream` (a hipStream_t passed as void*, NULL = the null
 *    stream) and results are visible after the caller's own sync.
 *  - Inputs and outputs must not alias.
 *  - A kernel launch failure returns TQ_ERR_DEVICE; faults during execution
 *    surface at the caller's next synchronization.
 */
#ifndef TURBOQUANT_H
#define TURBOQUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 5

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID = -1,     /* an argument is malformed (null, negative, inconsistent) */
  TQ_ERR_UNSUPPORTED = -2, /* valid, but this build has no kernel for that shape */
  TQ_ERR_NOCONVERGE = -3,  /* Lloyd-Max did not meet its tolerance within max_iter */
  TQ_ERR_WORKSPACE = -4,   /* decode workspace smaller than required */
  TQ_ERR_DEVICE = -5       /* a HIP call or kernel launch failed */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

/* Record formats of a compressed cache (see the bit layouts below). */
typedef enum {
  TQ_TOKEN_MAJOR = 0, /* one contiguous record per row; used for K */
  TQ_BLOCK32 = 1      /* rows packed by aligned blocks of 32; used for V */
} tq_format;

/* Shape of one quantizer instance. Groups are consecutive ranges of the
 * permuted (grouped) channel order; n_groups = 1 uses one instance on all
 * channels, n_groups = 2 gives fractional widths ([ZB] paragraph 2). */
typedef struct {
  int32_t d;            /* vector length, 3 <= d <= 256 */
  int32_t n_groups;     /* 1 or 2 */
  int32_t group_dim[2]; /* d_g >= 3, sum over groups == d */
  int32_t mse_bits[2];  /* m_g in [1, 4]; bits per channel of group g = m_g + 1 */
  int32_t mse_only;     /* 0: stage two as above (sign bits of the residual sketch);
                           1: stage one alone (the MSE quantizer): records carry no
                           sign words, bits per channel = m_g, gamma is stored but
                           not used, and dequantization is n Pi^T c[idx]. Decode
                           takes it for V only. */
  int32_t norm_f16;     /* 0: the norms (n_g, gamma_g) are stored as float32;
                           1: as float16 (rounded to nearest even from float32;
                           32 bits per group instead of 64). fp16 norms need
                           every n_g below 65504 and lose relative precision
                           below 6.1e-5 (subnormals). Every entry point takes
                           either form, for K and V independently. */
} tq_layout;

/* One quantizer instance (one for K, one for V). All pointers are device
 * memory, fp32, read-only, owned by the caller.
 *   rot        d x d row-major: rows [o_g, o_g + d_g) hold Pi_g applied to the
 *              channels of group g, i.e. rot = blockdiag(Pi_g) * P where P is
 *              the channel permutation; the rotated vector is y = rot x.
 *   sketch     d x d row-major, blockdiag(S_g) * P (used on queries and for
 *              the back-transform of the attention output).
 *   sketch_rot d x d row-major, sketch * rot^T (= blockdiag(S_g Pi_g^T)),
 *              as produced by tq_fold_sketch; applied to the rotated
 *              residual during quantization.
 *   centroids  concatenation over groups of the 2^m_g Lloyd-Max centroids
 *              (increasing), each the float32 rounding of the double value.
 *   boundaries concatenation over groups of the 2^m_g - 1 decision
 *              boundaries, each the float32 rounding of the double midpoint
 *              of neighbouring double centroids. */
typedef struct {
  tq_layout layout;
  const float* rot;
  const float* sketch;
  const float* sketch_rot;
  const float* centroids;
  const float* boundaries;
} tq_quantizer;

/* A compressed cache in device memory (caller-owned). For TQ_TOKEN_MAJOR,
 * row r's record is codes[r * code_words ...], signs[r * sign_words ...],
 * norms[r * norm_floats ...]. For TQ_BLOCK32, block b = r / 32 holds
 * codes[b * block_code_words ...] and signs[b * block_sign_words ...];
 * norms stay one row per token. n_rows is the number of rows allocated (a
 * multiple of 32 for TQ_BLOCK32). */
typedef struct {
  uint32_t* codes;
  uint32_t* signs;
  float* norms;
  int64_t n_rows;
} tq_cache;

/* Sizes of one record, in 32-bit words / floats (see tq_record_layout). */
typedef struct {
  int32_t code_words;       /* TQ_TOKEN_MAJOR code words per row */
  int32_t sign_words;       /* TQ_TOKEN_MAJOR sign words per row */
  int32_t norm_floats;      /* norm values per row, both formats: 2 * n_groups
                               (float32, or float16 when norm_f16) */
  int32_t block_code_words; /* TQ_BLOCK32 code words per 32-row block */
  int32_t block_sign_words; /* TQ_BLOCK32 sign words per 32-row block */
  int32_t record_bits;      /* algorithmic bits per row: sum_g (m_g + 1) d_g + 64 n_groups
                               (MSE-only: m_g in place of m_g + 1; fp16 norms:
                               32 n_groups in place of 64 n_groups) */
} tq_record_info;

/*
 * Bit layouts (this library's own choice; the pages fix only the contents).
 * "Stream bit b" of a sequence of 32-bit words is bit (b mod 32) of word
 * floor(b / 32). Codes are unsigned m_g-bit integers, least significant bit
 * first. Pad bits are zero.
 *
 * TQ_TOKEN_MAJOR, per row:
 *   codes: for each group g in order, ceil(m_g d_g / 32) words; the code of
 *          channel j (0-based within the group) is stream bits
 *          [m_g j, m_g j + m_g) of the group's words.
 *   signs: for each group, ceil(d_g / 32) words; bit j = sign bit of channel j.
 *   norms: (n_g, gamma_g) as float32 (float16 when norm_f16) for each group;
 *          tq_cache.norms then points to float16 values.
 * TQ_BLOCK32, per block of 32 rows (row r = 32 b + t, t = 8 o + s with octet
 * o in 0..3 and position s in 0..7):
 *   codes: for each group g, m_g d_g words; the code of slot t at channel j is
 *          stream bits [8 m_g (o d_g + j) + m_g s, ... + m_g) of the group's
 *          words (each octet keeps the 8 codes of a channel in m_g bytes).
 *   signs: for each group, d_g words; the sign bit of slot t at channel j is
 *          stream bit 8 (o d_g + j) + s.
 *   norms: as TQ_TOKEN_MAJOR (one row per token).
 * A sign bit is 1 exactly when the sketch coordinate is >= 0.
 * MSE-only layouts have no sign words (sign_words = block_sign_words = 0);
 * their norms keep the (n_g, gamma_g) pair, gamma_g being the norm of the
 * stage-one residual.
 */

/* Rows written by tq_quantize. Vector i goes to row dst_rows[i] when
 * dst_rows (device int64 [n_vec]) is non-NULL, otherwise to row
 * (i / seg_len) * seg_stride + seg_offset + (i % seg_len). Every row must be
 * in [0, cache.n_rows); with dst_rows the kernel skips rows outside that
 * range (it cannot report them). Two vectors of one call must not share a
 * row. */
typedef struct {
  const int64_t* dst_rows;
  int64_t seg_len;
  int64_t seg_stride;
  int64_t seg_offset;
} tq_rows;

/* One decode step over a compressed K/V cache. K and V of (batch b, KV head
 * h) occupy rows (b * n_kv_heads + h) * cache_capacity + t for tokens
 * t in [0, n_ctx). With n_q_tokens = T > 1 the step attends T query tokens
 * per head at once (a chunk of a prefill): query token i sits at position
 * n_ctx - T + i of the context (its own K/V already cached) and attends
 * causally to tokens [0, n_ctx - T + i]. */
typedef struct {
  int32_t batch;
  int32_t n_q_heads;      /* multiple of n_kv_heads */
  int32_t n_kv_heads;
  int32_t n_split;        /* token splits per KV head, 0 = chosen by the library */
  int64_t n_ctx;          /* >= 1, <= cache_capacity */
  int64_t cache_capacity; /* rows per (b, h); a multiple of 32 */
  float scale;            /* logit = scale * <q, k~> */
  int32_t n_q_tokens;     /* T, 1 <= T <= n_ctx (0 is read as 1) */
} tq_decode_shape;

/* ABI version of the loaded library (TQ_ABI_VERSION). */
int tq_abi_version(void);

/* Static English text for a status code. */
const char* tq_status_string(int status);

/* Lloyd-Max codebook for one rotated coordinate ([ZB] paragraph 2: the
 * rotation gives each coordinate a Beta law, and an optimal scalar
 * quantizer is fitted to it). Host-only, double precision.
 *   d              dimension of the rotated vector (d_g), d >= 3.
 *   mse_bits       m in [1, 4]; 2^m levels.
 *   max_iter       iteration cap, 0 = 200000.
 *   tol            stop when no centroid moves more than tol; 0 = 1e-13/sqrt(d).
 *   centroids      host out [2^m], increasing and exactly antisymmetric.
 *   boundaries     host out [2^m - 1], midpoints of neighbouring centroids.
 *   mse_per_coord  host out (may be NULL): E[(y - Q(y))^2] for one coordinate.
 * Errors: TQ_ERR_INVALID (domain, NULL outputs), TQ_ERR_NOCONVERGE. */
tq_status tq_build_codebook(int32_t d, int32_t mse_bits, int32_t max_iter, double tol,
                            double* centroids, double* boundaries, double* mse_per_coord);

/* Record sizes for a layout (host-only): the words of one token's stored
 * form, which [ZB] paragraph 2 names as the quantization indices, the sign
 * bits of the residual sketch and the norm (two norms per group here, n_g
 * and gamma_g, as read above). Per group g: d_g m_g code bits and d_g sign
 * bits (none for MSE-only records), each group's fields starting on a 32-bit
 * word; TQ_BLOCK32 sizes are those of 32 tokens. Errors: TQ_ERR_INVALID. */
tq_status tq_record_layout(const tq_layout* layout, tq_record_info* info);

/* sketch_rot = sketch * rot^T for d x d row-major host matrices, accumulated
 * in double and rounded once to float. Host-only. The sketch of [WD] "2. QJL
 * Residual" acts on the residual r = x_g - n Pi^T c[idx]; with the residual
 * kept in the rotated domain (Pi r = y n - n c[idx]) the sketch it needs is
 * S Pi^T, which this folds once per quantizer. Errors: TQ_ERR_INVALID. */
tq_status tq_fold_sketch(int32_t d, const float* rot, const float* sketch, float* sketch_rot);

/* Quantize-on-append ([ZB] paragraph 2; [WD] "1. PolarQuant" and "2. QJL
 * Residual"): for each of n_vec input vectors compute the group norms, the
 * Lloyd-Max codes of the rotated unit vector, the residual norms and the
 * sign bits of the sketched residual, and write the packed record to its
 * row of `cache` in format `fmt`.
 *   x            device [n_vec rows, row stride x_row_stride elements], f32 or bf16.
 *   rows         destination rows (see tq_rows).
 * Other rows of the cache are not modified (TQ_BLOCK32 updates the bits of
 * a partially written block in place with device atomics).
 * Errors: TQ_ERR_INVALID (NULL pointers, n_vec < 0, x_row_stride < d, rows
 * out of range, TQ_BLOCK32 with n_rows % 32 != 0), TQ_ERR_UNSUPPORTED
 * (n_groups == 2 with a group boundary not a multiple of 16; TQ_BLOCK32 with
 * a group dimension not a multiple of 8), TQ_ERR_DEVICE. n_vec == 0 is a
 * no-op. */
tq_status tq_quantize(const tq_quantizer* qz, tq_format fmt, const void* x, tq_dtype x_dtype,
                      int64_t n_vec, int64_t x_row_stride, const tq_rows* rows,
                      const tq_cache* cache, void* stream);

/* Bytes of decode workspace needed for a shape (host-only).
 *   vq  V quantizer, or NULL for a logits-only call. */
tq_status tq_attn_decode_workspace_bytes(const tq_quantizer* kq, const tq_quantizer* vq,
                                         const tq_decode_shape* shape, size_t* bytes);

/* One decode step over the compressed cache ([WD] introduction and "Os
 * numeros que importam": attention logits from the compressed keys; then
 * softmax times the dequantized values). For each batch b and query head h:
 *   logits[b, h, t] = scale * <q[b, h], k~[b, h_kv, t]>  for t < n_ctx,
 *   out[b, h]       = sum_t softmax(logits[b, h])_t v~[b, h_kv, t].
 * With T = n_q_tokens > 1 (causal chunk): q is [batch, T, n_q_heads, d],
 * out [batch, T, n_q_heads, d], logits [batch, n_q_heads, T, n_ctx] with
 * -inf past each query token's causal limit, and query token i attends to
 * tokens [0, n_ctx - T + i].
 * The estimate is evaluated in factored form: scale * sum_g (n_g <rot q,
 * c[idx]>_g + alpha_g gamma_g <sketch q, z>_g); V is accumulated in the
 * rotated and sketch domains and mapped back once per head with rot^T and
 * sketch^T. Operand precision: fp16 products, fp32 accumulation (the
 * rotated and the sketched query each as an fp16 hi/lo pair; K centroids tabulated as fp16(s c) with a scale
 * s in [1, 2) chosen per codebook so that the rounding is far below fp16's
 * own, and 1/s applied with the norm); stored norms must be below 65504,
 * and scale * |rot q| below about 4.5e4.
 *   q        device [batch, n_q_heads, d], f32 or bf16.
 *   k_cache  K records, TQ_TOKEN_MAJOR. v_cache: V records, TQ_BLOCK32
 *            (ignored when vq is NULL).
 *   logits   device fp32 [batch, n_q_heads, n_ctx], or NULL; required when
 *            vq is NULL.
 *   out      device fp32 [batch, n_q_heads, d]; must be NULL when vq is NULL.
 *   workspace device scratch of at least tq_attn_decode_workspace_bytes().
 * Supported: kq and vq with the same group dimensions and bits, every group
 * dimension a multiple of 32, d <= 256 (this build: d = 128), kq with sign
 * bits (mse_only = 0), otherwise TQ_ERR_UNSUPPORTED. vq may be MSE-only
 * (mse_only = 1): then v_cache->signs is not read (it may be NULL) and each
 * value is dequantized as n Pi^T c[idx], the biased stage-one estimate. Errors: TQ_ERR_INVALID, TQ_ERR_WORKSPACE,
 * TQ_ERR_DEVICE. */
tq_status tq_attn_decode(const tq_quantizer* kq, const tq_quantizer* vq,
                         const tq_decode_shape* shape, const void* q, tq_dtype q_dtype,
                         const tq_cache* k_cache, const tq_cache* v_cache, float* logits,
                         float* out, void* workspace, size_t workspace_bytes, void* stream);

/* The three stages of tq_attn_decode, for callers that schedule or time them
 * separately (e.g. to bracket the split-K kernel with events):
 *   TQ_PHASE_PREP    q_rot = rot q, q_sk = sketch q and the K codebook
 *                    scales into the workspace,
 *   TQ_PHASE_SPLIT   the split-K pass over the cache (logits; partial softmax
 *                    sums and accumulators into the workspace),
 *   TQ_PHASE_COMBINE merge of the splits and back-transform into `out`.
 * A stage reads what the earlier stages left in the same workspace, so
 * stages must run in this order on one stream with identical arguments. */
enum { TQ_PHASE_PREP = 1, TQ_PHASE_SPLIT = 2, TQ_PHASE_COMBINE = 4, TQ_PHASE_ALL = 7 };

/* tq_attn_decode restricted to the stages in `phases` (a non-zero subset of
 * TQ_PHASE_ALL); arguments, validation and errors as tq_attn_decode, plus
 * TQ_ERR_INVALID for an empty or unknown phase mask. */
tq_status tq_attn_decode_phases(unsigned phases, const tq_quantizer* kq, const tq_quantizer* vq,
                                const tq_decode_shape* shape, const void* q, tq_dtype q_dtype,
                                const tq_cache* k_cache, const tq_cache* v_cache, float* logits,
                                float* out, void* workspace, size_t workspace_bytes, void* stream);

/* A paged cache (a block table with per-sequence lengths). Physical block p
 * holds 32 consecutive tokens of every KV head: the K and V records of KV
 * head h at token offset i of block p are row (p * n_kv_heads + h) * 32 + i
 * of the caches (for TQ_BLOCK32 V caches that is block p * n_kv_heads + h).
 * Logical block j (tokens [32 j, 32 j + 32)) of batch b lives in physical
 * block block_table[b * max_blocks + j]. */
typedef struct {
  const int32_t* block_table; /* device [batch, max_blocks] physical block ids */
  const int32_t* seq_lens;    /* device [batch] cached tokens per sequence, clamped
                                 to [1, n_ctx]; NULL: n_ctx for every sequence */
  int32_t max_blocks;         /* row length of block_table; 32 * max_blocks must
                                 equal the shape's cache_capacity */
} tq_paging;

/* tq_attn_decode over a paged cache (the paged layout is this library's
 * extension of the decode step for serving with per-sequence lengths; the
 * arithmetic is that of tq_attn_decode). shape->n_ctx is the longest
 * sequence: logits rows keep that length and entries past a sequence's own
 * length are not written; n_q_tokens chunks take their causal limits from
 * each sequence's length (a query token of a chunk that sees no cached token,
 * when a sequence is shorter than the chunk, gets a zero output row and -inf
 * logits). Block ids outside the caches are clamped into them
 * (the caller keeps the table valid; nothing is read outside the caches).
 * Workspace: tq_attn_decode_workspace_bytes(shape). Errors as
 * tq_attn_decode, plus TQ_ERR_INVALID for a missing or misaligned table or
 * a capacity other than 32 * max_blocks. */
tq_status tq_attn_decode_paged(const tq_quantizer* kq, const tq_quantizer* vq, const tq_decode_shape* shape,
                               const tq_paging* paging, const void* q, tq_dtype q_dtype,
                               const tq_cache* k_cache, const tq_cache* v_cache, float* logits, float* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Vectors to append to a cache within a decode step (see
 * tq_attn_decode_append): x, dtype, n_vec, x_row_stride and rows as for
 * tq_quantize. */
typedef struct {
  const void* x;
  tq_dtype dtype;
  int64_t n_vec;
  int64_t x_row_stride;
  tq_rows rows;
} tq_append;

/* One decode step with its appends ([ZB] paragraph 2: each new token is
 * quantized as it enters the cache; [WD] introduction: attention logits from
 * the compressed cache; R14: the new tokens are attended to). Equivalent to
 *   tq_quantize(kq, TQ_TOKEN_MAJOR, k_new..., k_cache);
 *   tq_quantize(vq, TQ_BLOCK32, v_new..., v_cache);
 *   tq_attn_decode(kq, vq, shape, q, ...);
 * on the same stream, but the two appends and the query preparation run as
 * one launch (they are independent), followed by the split-K pass and the
 * combine. k_new / v_new may be NULL (nothing appended; v_new requires vq).
 * Same arguments, validation and errors as those calls; everything is
 * validated before anything is launched. Supported for d = 128 (as
 * tq_attn_decode), otherwise TQ_ERR_UNSUPPORTED. */
tq_status tq_attn_decode_append(const tq_quantizer* kq, const tq_quantizer* vq,
                                const tq_decode_shape* shape, const tq_append* k_new,
                                const tq_append* v_new, const void* q, tq_dtype q_dtype,
                                const tq_cache* k_cache, const tq_cache* v_cache, float* logits,
                                float* out, void* workspace, size_t workspace_bytes, void* stream);

/* tq_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a static device array
 * of the library (16 MiB on each GPU the library runs on, held until the
 * process ends); its per-device address is looked up on the first call on
 * each device. Arguments, results and errors as tq_attn_decode, plus
 * TQ_ERR_WORKSPACE when the shape needs more than 16 MiB of workspace
 * (tq_attn_decode_workspace_bytes) and TQ_ERR_DEVICE when the array's
 * address cannot be obtained. Nothing in the array needs to start at zero.
 * Every call on one GPU uses the same array: calls that overlap in time on
 * one GPU (on different streams, or from different threads) race and give
 * undefined results; calls in order on one stream are safe. */
tq_status tq_attn_decode_scratch(const tq_quantizer* kq, const tq_quantizer* vq,
                                 const tq_decode_shape* shape, const void* q, tq_dtype q_dtype,
                                 const tq_cache* k_cache, const tq_cache* v_cache, float* logits,
                                 float* out, void* stream);

/* Uncompressed decode baseline: the same decode step over bf16 K/V caches,
 * for comparison with tq_attn_decode ([WD] "Os numeros que importam": the
 * reported speed-ups are against unquantized keys). For each batch b and
 * query head h over KV head h_kv:
 *   logits[b, h, t] = scale * <q[b, h], k[b, h_kv, t]>  for t < n_ctx,
 *   out[b, h]       = sum_t softmax(logits[b, h])_t v[b, h_kv, t],
 * with fp32 accumulation (the scaled query and the softmax weights enter the
 * bf16 products as hi + lo bf16 pairs).
 *   shape    as tq_attn_decode (n_split 0 = automatic); d = 128.
 *   q        device [batch, n_q_heads, d], f32 or bf16, 16-byte aligned.
 *   k        device bf16 [batch * n_kv_heads * cache_capacity, d], token-major
 *            (KV head bh owns rows [bh * cache_capacity, (bh + 1) * cache_capacity)).
 *   v        device bf16 [batch * n_kv_heads * cache_capacity / 32, d, 32]: the
 *            rows in blocks of 32, channel-major inside a block.
 *   logits   device fp32 [batch, n_q_heads, n_ctx], or NULL.
 *   out      device fp32 [batch, n_q_heads, d].
 *   workspace device scratch of at least tq_attn_decode_bf16_workspace_bytes().
 * Rows past n_ctx inside the last 32-row block are ignored, whatever they
 * hold. Errors: TQ_ERR_INVALID (shape, null or misaligned pointers, dtype),
 * TQ_ERR_UNSUPPORTED (d != 128, n_q_tokens > 1), TQ_ERR_WORKSPACE,
 * TQ_ERR_DEVICE. */
tq_status tq_attn_decode_bf16_workspace_bytes(const tq_decode_shape* shape, int d, size_t* bytes);
tq_status tq_attn_decode_bf16(const tq_decode_shape* shape, int d, const void* q, tq_dtype q_dtype,
                              const void* k, const void* v, float* logits, float* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Nearest-neighbour search with the compressed codes ([WD] "Os numeros que
 * importam": the method also serves vector search). Every query is scored
 * against database rows [0, n_db) of a token-major cache with the
 * inner-product estimator of tq_attn_decode at scale 1,
 *   score(q, i) = n_i <Pi q, c[idx_i]> + alpha gamma_i <S q, z_i>,
 * and its k best rows are returned in decreasing score order; equal scores
 * go to the lower row index.
 *   qz         the database's quantizer: one group, d = 128 or 200, m <= 3.
 *   db         token-major cache holding the database records (n_rows >= n_db).
 *   q          [n_q, d] fp32 or bf16, row-major, 16-byte aligned rows.
 *   k          1 <= k <= 10.
 *   out_idx    [n_q, k] int64 (8-byte aligned); -1 where fewer than k rows exist.
 *   out_score  [n_q, k] fp32 (-inf where out_idx is -1).
 *   workspace  device scratch of at least tq_search_workspace_bytes() bytes.
 * Limits: 1 <= n_db < 2^31 - 1, 1 <= n_q <= 2^30.
 * Errors: TQ_ERR_INVALID (sizes, k, null or misaligned pointers, dtype),
 * TQ_ERR_UNSUPPORTED (layout outside the limits above, or MSE-only records),
 * TQ_ERR_WORKSPACE, TQ_ERR_DEVICE. */
tq_status tq_search_workspace_bytes(const tq_quantizer* qz, int64_t n_db, int64_t n_q, int k, size_t* bytes);
tq_status tq_search(const tq_quantizer* qz, const tq_cache* db, int64_t n_db, const void* q, tq_dtype q_dtype,
                    int64_t n_q, int k, int64_t* out_idx, float* out_score, void* workspace,
                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TURBOQUANT_H */
