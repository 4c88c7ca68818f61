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
                         /* the split-T kernels alone                             */
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
 * launch settings (launch may be NULL). */
jolt_status jolt_decode_workspace_size(const jolt_cache *const *caches, int32_t batch,
                                       int32_t layer, const jolt_launch *launch, size_t *bytes);

/*
 * Decode attention of one layer for a batch of sequences, each with its own
 * cache handle (handles in one call share n_layers, groups, heads and d; T
 * and the per-cell ranks and bits may differ).
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
 *   RoPE; variant 1: the hardware-unit evaluation of the MFMA key path.
 *   JOLT_E_INVALID for |angle| >= 2^20 or another variant. */
jolt_status jolt_debug_sincos(const float *angles, int32_t n, float *sin_out, float *cos_out,
                              int32_t variant);
jolt_status jolt_debug_unpack(const jolt_cache *cache, int32_t layer, int32_t tau,
                              uint8_t *codes_out, jolt_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* JOLT_H */
