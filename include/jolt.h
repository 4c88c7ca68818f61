/*
 * jolt.h -- C ABI of the MI355X (gfx950) JoLT compressed-cache decode library.
 *
 * What the library computes.  "A JoLT for the KV cache: Near-Lossless KV Cache
 * Compression via Joint Rank-bit Allocation" (arXiv 2607.12550v4 summary),
 * Abstract, §1 and §4.5: decode attention evaluated directly over the stored
 * factors and packed residuals of a JoLT-compressed KV cache, without
 * materialising dense K/V.  The cache of each (layer group, K or V) cell is a
 * partial Tucker decomposition (§3: token factor A and feature factor B shared
 * by the group's layers and heads, a core G per layer and head) plus a
 * residual rotated along the feature axis by a seeded orthogonal matrix that
 * is shared by all cells and regenerated at decode, quantised to
 * b in {0, 2, 4, 8} bits (b = 0: no residual stored).
 *
 * For KV head h of layer l (index l' inside its group) the decoded cache is
 *     K^_t = A_K[t] G_K[l', h] B_K^T + [b_K > 0] deq_K[l', h, t] Pi^T   (V^ alike)
 *     deq[i] = (code[i] - (2^b - 1)/2) * scale[l', h, t]
 * and query head j (KV head h = j / (n_q / n_kv)) at position q_pos gets
 *     o_j = sum_t softmax_t(scale_s * rope(q_j, q_pos) . rope(K^_t, t)) V^_t
 * with rotate-half RoPE at the float32 angle fl32(t * inv_freq[i]) (the
 * sarnas.ru JoLT post, section on building cos/sin in-kernel from the model's
 * inv_freq and int32 positions).  Keys are rebuilt tile by tile because RoPE
 * does not commute with the factorisation (§4.5, §5); values never are:
 *     o_j = ((sum_t p_t A_V[t]) G_V[l', h]) B_V^T + (sum_t p_t deq_V[t]) Pi^T.
 *
 * Conventions for every call:
 *  - Return value: JOLT_OK (0) or a negative jolt_status.  All arguments are
 *    validated before anything is launched; on error nothing is launched or
 *    written and jolt_last_error() (thread-local) says why.  HIP runtime
 *    failures return JOLT_E_HIP with HIP's error string in the message.
 *  - "HOST" pointers are read during the call only.  "DEVICE" pointers must
 *    stay valid until the work queued on the stream has finished.
 *  - Work is queued asynchronously on the given stream (NULL = default).
 *  - Caches are read-only after load; any number of decodes may use a cache
 *    concurrently.  Synchronise before jolt_free_cache.
 */
#ifndef JOLT_H
#define JOLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *jolt_stream; /* a hipStream_t */

typedef enum {
  JOLT_OK = 0,
  JOLT_E_INVALID = -1,     /* bad argument or descriptor                    */
  JOLT_E_UNSUPPORTED = -2, /* valid but not implemented (e.g. d not 64/128) */
  JOLT_E_OOM = -3,         /* device or host allocation failed              */
  JOLT_E_HIP = -4,         /* HIP runtime error                             */
  JOLT_E_WORKSPACE = -5    /* workspace NULL or smaller than required       */
} jolt_status;

typedef enum { JOLT_F32 = 0, JOLT_BF16 = 1 } jolt_dtype;

/* Opaque handle to one sequence's compressed cache in device memory. */
typedef struct jolt_cache jolt_cache;

/*
 * One stored cell = (layer group, K or V).  All pointers are HOST memory,
 * row-major, in the element type named by jolt_cache_desc.factor_dtype
 * (A, B, G) or as stated.  Shapes use |g| = layers in the group,
 * H = n_kv_heads, d = head_dim, T = cached tokens.
 *   0 <= r_T <= min(T, |g| H d), 0 <= r_F <= d, r_T == 0 iff r_F == 0.
 *   bits in {0, 2, 4, 8}.
 */
typedef struct {
  int32_t r_T, r_F, bits;
  const void *A;          /* [T][r_T]                                         */
  const void *B;          /* [d][r_F]                                         */
  const void *G;          /* [|g|][H][r_T][r_F]                               */
  const uint8_t *codes;   /* [|g|][H][T][d*bits/8], codes packed least        */
                          /* significant bits first (b=2: c0|c1<<2|c2<<4|c3<<6,*/
                          /* b=4: c0|c1<<4, b=8: one code per byte);          */
                          /* NULL iff bits == 0                               */
  const float *scales;    /* [|g|][H][T] quantiser step per row; NULL iff bits == 0 */
} jolt_cell;

typedef struct {
  int32_t n_layers, n_groups, n_kv_heads, n_q_heads, head_dim, T;
  const int32_t *group_start; /* HOST [n_groups+1]: 0 = g_0 < g_1 < ... = n_layers */
  jolt_dtype factor_dtype;    /* JOLT_BF16 or JOLT_F32                             */
  uint64_t rotation_seed;     /* Pi is regenerated from this seed                  */
  const jolt_cell *cells;     /* HOST [n_groups][2]: [g][0] = K cell, [g][1] = V   */
} jolt_cache_desc;

/* Kernel selection and split size; pass NULL for the library's choice.     */
typedef enum { JOLT_KERNEL_AUTO = 0, JOLT_KERNEL_GENERIC = 1, JOLT_KERNEL_MFMA = 2 } jolt_kernel;
typedef struct {
  int32_t kernel;        /* jolt_kernel                                           */
  int32_t split_tokens;  /* tokens per split-T work item (0 = auto); rounded up   */
                         /* to the kernel's tile                                  */
  void *ev_begin;        /* optional hipEvent_t (NULL = none), set to the GPU     */
  void *ev_end;          /* start time of the first split-T kernel launch of the  */
                         /* call / the end time of its last one (kernel           */
                         /* timestamps, not stream markers), so a caller can time */
                         /* the split-T kernels alone; where the call has a       */
                         /* second value pass (one query per KV head, value ranks */
                         /* above 128) the end is that pass's last kernel's       */
  int32_t deterministic; /* 1: fixed assignment of token blocks to waves, so two  */
                         /* calls with the same inputs and settings give the same */
                         /* output bits (the Reproducibility Statement of the     */
                         /* JoLT summary asks for repeatable results); 0: blocks  */
                         /* handed out on demand (faster, last-bit differences    */
                         /* between runs)                                         */
} jolt_launch;

/*
 * Copy one sequence's compressed cache to the device (off the per-step clock).
 * Regenerates the rotation Pi from rotation_seed (the summary's §3: seeded,
 * shared by all cells, regenerated at decode), re-lays the factors and codes
 * out for the decode kernels and uploads everything on `stream`.  Returns
 * after the host buffers are no longer needed (the call synchronises
 * `stream`).  *out receives a handle owned by the caller (jolt_free_cache).
 * Errors: JOLT_E_INVALID (shape/rank/bits/NULL rules above, group_start not
 * strictly increasing from 0 to n_layers, n_q_heads not a multiple of
 * n_kv_heads, odd head_dim, T < 1), JOLT_E_UNSUPPORTED (head_dim not 64 or
 * 128, n_q_heads/n_kv_heads > 16, T > 2^20), JOLT_E_OOM, JOLT_E_HIP.
 */
jolt_status jolt_load_cache(const jolt_cache_desc *desc, jolt_stream stream, jolt_cache **out);

/* Free a cache (NULL is a no-op).  The caller must have synchronised every
 * stream that used it. */
jolt_status jolt_free_cache(jolt_cache *cache);

/* Shape of a loaded cache (any output pointer may be NULL). */
jolt_status jolt_cache_info(const jolt_cache *cache, int32_t *n_layers, int32_t *n_kv_heads,
                            int32_t *n_q_heads, int32_t *head_dim, int32_t *T,
                            size_t *device_bytes);

/* Workspace bytes jolt_decode_attention needs for these caches, layer and
 * launch settings (launch may be NULL): the split partials (each a partial
 * softmax state of the fused kernel that "A JoLT for the KV cache" §4.5
 * describes: running max, weight sum and weighted value sum of one token
 * range) and, where a class of the call takes the second value pass, every
 * token's logit, the softmax statistics and the partial value-factor sums.
 * Errors: JOLT_E_INVALID (NULL pointers, batch < 0, layer out of range,
 * handles with different shapes, launch fields out of range),
 * JOLT_E_UNSUPPORTED (kernel forced to MFMA for a cache it cannot run). */
jolt_status jolt_decode_workspace_size(const jolt_cache *const *caches, int32_t batch,
                                       int32_t layer, const jolt_launch *launch, size_t *bytes);

/*
 * Decode attention of one layer for a batch of sequences, each with its own
 * cache handle (handles in one call share n_layers, groups, heads and d; T
 * and the per-cell ranks and bits may differ).  This is the operation of
 * "A JoLT for the KV cache" §4.5 (and the Abstract): attention for one new
 * query per head evaluated over the stored factors and packed residuals,
 * with key tiles rebuilt and rotated at their positions (RoPE does not
 * commute with the factorisation, §5) and values taken in factor space; the
 * result is the formula in this file's header.
 *   q         DEVICE [batch][n_q_heads][d], pre-RoPE, q_dtype (F32 or BF16)
 *   q_pos     HOST   [batch] query positions (normally the cache's T), in
 *             [0, 2^20]
 *   inv_freq  HOST   [d/2] float32 RoPE inverse frequencies in [0, 1] (any
 *             rope scaling already applied)
 *   softmax_scale    multiplies q.k (normally 1/sqrt(d) x attention scaling)
 *   out       DEVICE [batch][n_q_heads][d] float32
 *   workspace DEVICE, >= jolt_decode_workspace_size bytes, caller-owned;
 *             needs no initialisation; one workspace serves one call at a
 *             time (stream order).
 * Errors: JOLT_E_INVALID (NULL pointers, batch < 0, layer out of range,
 * handles with different shapes, q_pos or inv_freq out of range),
 * JOLT_E_WORKSPACE,
 * JOLT_E_UNSUPPORTED (kernel forced to MFMA for a cache it cannot run),
 * JOLT_E_HIP.  batch == 0 is a no-op.
 */
jolt_status jolt_decode_attention(const jolt_cache *const *caches, int32_t batch, int32_t layer,
                                  const void *q, jolt_dtype q_dtype, const int32_t *q_pos,
                                  const float *inv_freq, float softmax_scale, float *out,
                                  void *workspace, size_t ws_bytes, const jolt_launch *launch,
                                  jolt_stream stream);

/*
 * Decode attention over a compressed cache followed by an uncompressed tail
 * (the tokens generated since the cache was compressed).  The JoLT summary
 * compresses the prefill cache in one global pass and notes (§5) that this
 * does not by itself support streaming generation; a decode loop therefore
 * keeps its newest tokens dense until the next compression.  The query
 * attends, under one softmax, to the T compressed tokens of its sequence
 * (keys rotated to positions 0..T-1) and then to the first tail_len[b] rows
 * of the tail:
 *   k_tail, v_tail  DEVICE [batch][n_kv_heads][tail_cap][d] in tail_dtype
 *                   (F32 or BF16); keys already rotated to their own
 *                   positions (normally T, T+1, ...)
 *   tail_cap        rows per (sequence, head) of k_tail / v_tail, >= 0
 *   tail_len        HOST [batch], 0 <= tail_len[b] <= tail_cap
 * The other arguments are as for jolt_decode_attention; the workspace must
 * hold jolt_decode_tail_workspace_size bytes for the same tail_cap.  The
 * tail's partial softmax states join the compressed splits' in the same
 * merge.  Errors: those of jolt_decode_attention, and JOLT_E_INVALID for a
 * negative or too large tail_cap, a tail_len outside [0, tail_cap], NULL tail
 * pointers with tail_cap > 0 or another tail dtype.
 */
jolt_status jolt_decode_tail_workspace_size(const jolt_cache *const *caches, int32_t batch,
                                            int32_t layer, int32_t tail_cap,
                                            const jolt_launch *launch, size_t *bytes);
jolt_status jolt_decode_attention_tail(const jolt_cache *const *caches, int32_t batch,
                                       int32_t layer, const void *q, jolt_dtype q_dtype,
                                       const int32_t *q_pos, const float *inv_freq,
                                       float softmax_scale, const void *k_tail,
                                       const void *v_tail, jolt_dtype tail_dtype,
                                       int32_t tail_cap, const int32_t *tail_len, float *out,
                                       void *workspace, size_t ws_bytes,
                                       const jolt_launch *launch, jolt_stream stream);

/*
 * jolt_decode_attention without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid allocation.  The split partials go to
 * a device array inside the library of jolt_noalloc_scratch_bytes() bytes
 * (16 MiB), one per GPU, held until the process ends; the call makes no
 * allocation of any kind.  Every call on a GPU shares that GPU's array:
 * calls that overlap in time on one GPU (different streams, or a graph
 * replayed while another call runs) race and may return wrong results --
 * order them on one stream.  The array needs no clearing between calls.
 * Errors: those of jolt_decode_attention, and JOLT_E_WORKSPACE when the call
 * would need more partials than the array holds (fewer splits, a smaller
 * batch or the workspace entry point then).
 */
size_t jolt_noalloc_scratch_bytes(void);
jolt_status jolt_decode_attention_noalloc(const jolt_cache *const *caches, int32_t batch,
                                          int32_t layer, const void *q, jolt_dtype q_dtype,
                                          const int32_t *q_pos, const float *inv_freq,
                                          float softmax_scale, float *out,
                                          const jolt_launch *launch, jolt_stream stream);

/* Workspace bytes jolt_dense_attention needs. */
jolt_status jolt_dense_workspace_size(int32_t batch, int32_t n_kv, int32_t n_q, int32_t d,
                                      int32_t T, const jolt_launch *launch, size_t *bytes);

/*
 * Dense decode attention over an uncompressed post-RoPE cache -- the
 * comparator the JoLT summary's §4.5 measures its fused kernel against.
 *   k_rope, v  DEVICE [batch][n_kv][T][d] in kv_dtype (F32 or BF16); keys
 *              already rotated to their positions 0..T-1
 *   q, q_pos, inv_freq, softmax_scale, out, workspace: as jolt_decode_attention
 * Errors: JOLT_E_INVALID, JOLT_E_UNSUPPORTED (d not 64/128, n_q/n_kv > 16,
 * T > 2^20), JOLT_E_WORKSPACE, JOLT_E_HIP.
 */
jolt_status jolt_dense_attention(const void *k_rope, const void *v, jolt_dtype kv_dtype,
                                 int32_t batch, int32_t n_kv, int32_t n_q, int32_t d, int32_t T,
                                 const void *q, jolt_dtype q_dtype, const int32_t *q_pos,
                                 const float *inv_freq, float softmax_scale, float *out,
                                 void *workspace, size_t ws_bytes, const jolt_launch *launch,
                                 jolt_stream stream);

/*
 * GPU compressor (FlashJoLT).  "A JoLT for the KV cache" (arXiv 2607.12550v4
 * summary), §3 and §3.1 "Fast variant: FlashJoLT": ST-HOSVD of one cell whose
 * token-mode SVD is a randomized SVD of the leading q_cap directions
 * (randomized subspace iteration with a seeded Gaussian test matrix of
 * q_cap + oversample columns and power_iters iterations), exact feature-mode
 * SVD, residual against the stored factors rotated by the seeded Pi and
 * quantised to b bits.  X is one cell's grouped cache, DEVICE
 * [group_size][n_kv_heads][T][head_dim] in x_dtype (F32 or BF16); all
 * arithmetic is float64.  Synchronous on `stream`; allocates its own device
 * scratch (a prefill-time operation, not for capture).
 */
typedef struct {
  int32_t q_cap;        /* token-mode directions computed; also the largest r_T  */
  int32_t oversample;   /* extra sketch columns (>= 0)                          */
  int32_t power_iters;  /* subspace iterations (0..16)                          */
  uint64_t sketch_seed; /* seed of the Gaussian test matrix (SplitMix64 stream, */
                        /* Box-Muller, row by row as for the rotation)          */
} jolt_flash_params;

/* Allocator inputs of one cell: HOST sT2[q_cap + 1] (the q_cap leading squared
 * token-mode singular values, descending, then the synthetic tail entry
 * max(||X||^2 - their sum, 0)), HOST sF2[head_dim] (squared feature-mode
 * singular values of the unprojected tensor, descending), HOST *norm2.
 * Errors: JOLT_E_INVALID (shape, params, NULL), JOLT_E_HIP. */
jolt_status jolt_flash_spectra(const void *X, jolt_dtype x_dtype, int32_t group_size,
                               int32_t n_kv_heads, int32_t T, int32_t head_dim,
                               const jolt_flash_params *params, double *sT2, double *sF2,
                               double *norm2, jolt_stream stream);

/* Compress one cell at (r_T <= q_cap, r_F, bits) into HOST buffers in the
 * layout of jolt_cell: A [T][r_T], B [head_dim][r_F], G [group_size][H][r_T][r_F]
 * in factor_dtype (F32, or BF16 as its 16-bit patterns), codes
 * [group_size][H][T][head_dim*bits/8] packed least significant bits first
 * and scales [group_size][H][T] (unused when bits == 0; A, B, G unused when
 * r_T == 0).  Errors: JOLT_E_INVALID (ranks, bits, dtype, NULL), JOLT_E_HIP. */
jolt_status jolt_flash_compress_cell(const void *X, jolt_dtype x_dtype, int32_t group_size,
                                     int32_t n_kv_heads, int32_t T, int32_t head_dim,
                                     const jolt_flash_params *params, int32_t r_T, int32_t r_F,
                                     int32_t bits, uint64_t rotation_seed,
                                     jolt_dtype factor_dtype, void *A, void *B, void *G,
                                     uint8_t *codes, float *scales, jolt_stream stream);

/* Alignment-based layer grouping (the summary's §3: consecutive layers whose
 * token-mode singular vectors align share a group, computed from the cache
 * itself).  k_layers[l], v_layers[l]: DEVICE [n_kv_heads][T][head_dim] of
 * layer l in x_dtype.  Each layer's basis is the leading q_cap left singular
 * vectors of its keys and values side by side (params as above); the
 * alignment of neighbours is ||U_l^T U_(l+1)||_F^2 / q_cap; groups are the
 * maximal runs of neighbours aligned at least tau, split to at most
 * max_group layers (0: no limit).  HOST group_start[n_layers + 1] receives
 * 0 = g_0 < ... < g_n = n_layers, *n_groups = n, HOST align[n_layers - 1]
 * (may be NULL) the alignments.  Synchronous.  Errors: JOLT_E_INVALID,
 * JOLT_E_HIP. */
jolt_status jolt_flash_layer_groups(const void *const *k_layers, const void *const *v_layers,
                                    jolt_dtype x_dtype, int32_t n_layers, int32_t n_kv_heads,
                                    int32_t T, int32_t head_dim, const jolt_flash_params *params,
                                    double tau, int32_t max_group, int32_t *group_start,
                                    int32_t *n_groups, double *align, jolt_stream stream);

/* The quantiser and packer alone, on rotated residual rows: DEVICE rows
 * [n_rows][d] float64 -> DEVICE codes [n_rows][d*bits/8] and scales [n_rows]:
 * delta = fl32(2 max|r| / (2^b - 1)), c = clip(rint(r / delta + (2^b - 1)/2))
 * with ties to even (delta = 0: c = floor((2^b - 1)/2)), packed least
 * significant bits first.  Asynchronous on `stream`.  Errors: JOLT_E_INVALID
 * (d not in 2..128, bits not 2/4/8, NULL), JOLT_E_HIP. */
jolt_status jolt_quantize_rows(const double *rows, int64_t n_rows, int32_t d, int32_t bits,
                               uint8_t *codes, float *scales, jolt_stream stream);

/*
 * Rank/bit allocation (host only, no GPU): "A JoLT for the KV cache" §3 --
 * one Lagrange multiplier prices bytes for all cells; each cell takes the
 * (r_T, r_F, bits) minimising estimated error + lambda * bytes, and lambda
 * is bisected (in log space) to the smallest value whose total bytes fit the
 * budget.  A cell's error estimate is min(||X||^2, tail_T(r_T) + tail_F(r_F))
 * times phi(bits) = 1 (b = 0) or m2(d) / (3 (2^b - 1)^2), m2(d) = E[max_i
 * z_i^2] for z ~ N(0, I_d); ranks on a grid of 16 (r_T = 0 iff r_F = 0),
 * r_T up to min(T, group_size H d, cap); bits in {0, 2, 4, 8}.  Cells take
 * their spectra from jolt_flash_spectra (cap = q_cap) or an exact SVD.
 * HOST cells[n_cells]; HOST choice[n_cells][3] receives (r_T, r_F, bits);
 * *lambda (may be NULL) the multiplier.  Errors: JOLT_E_INVALID (bad cell,
 * budget below what rank 0 and no residual would need).
 */
typedef struct {
  int32_t T, d, group_size, n_kv_heads, factor_bytes; /* factor bytes: 2 or 4 */
  int32_t n_sT2;
  const double *sT2; /* squared token-mode singular values, descending        */
  int32_t n_sF2;
  const double *sF2; /* squared feature-mode singular values, descending      */
  double norm2;      /* ||X||^2                                               */
  int32_t cap;       /* largest token rank (0: none)                          */
} jolt_alloc_cell;
jolt_status jolt_allocate(const jolt_alloc_cell *cells, int32_t n_cells, double budget_bytes,
                          int32_t *choice, double *lambda);

/* Thread-local description of the last error of this thread ("" if none). */
const char *jolt_last_error(void);

/*
 * Test helpers (not on the decode path).
 * jolt_make_rotation: the rotation the library regenerates from `seed`
 *   (SplitMix64 -> Box-Muller Gaussian d x d, row-major -> Householder QR ->
 *   Q with columns scaled by sign(diag R)), written to HOST out[d*d]
 *   (row-major float64).  Host-only; needs no GPU.
 * jolt_debug_unpack: the residual codes of (layer, tau: 0 = K, 1 = V) read
 *   back from the device layout by a device kernel, in canonical order,
 *   one code per byte, HOST [n_kv][T][d].  Synchronises `stream`.
 *   JOLT_E_INVALID if that cell has bits == 0.
 */
jolt_status jolt_make_rotation(uint64_t seed, int32_t d, double *out);
/* jolt_debug_sincos: the kernels' float32 sine and cosine of HOST angles[n]
 *   (evaluated on the current device; synchronous), written to HOST outputs.
 *   variant 0: the polynomial evaluation of the float32 paths and of query
 *   RoPE; variant 1: the hardware-unit evaluation of the MFMA key path;
 *   variant 2: the key path's small-angle blocks -- angles[2i] is a position
 *   t and angles[2i + 1] an inverse frequency f (2n floats in), evaluated as
 *   the hardware units of t * fl32(f / 2 pi) revolutions.
 *   JOLT_E_INVALID for |angle| or |t| >= 2^20, f outside [0, 1] or another
 *   variant. */
jolt_status jolt_debug_sincos(const float *angles, int32_t n, float *sin_out, float *cos_out,
                              int32_t variant);
jolt_status jolt_debug_unpack(const jolt_cache *cache, int32_t layer, int32_t tau,
                              uint8_t *codes_out, jolt_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* JOLT_H */
