/*
 * attn.h -- C ABI of exact tiled attention (forward and backward) for AMD
 * MI355X (gfx950).
 *
 * What is computed.  For every batch b, query head h and query row i:
 *
 *     out[b,i,h,:] = sum_j P[i,j] * v[b,j,g,:],
 *     P[i,:]       = softmax_j( scale * <q[b,i,h,:], k[b,j,g,:]> )  over visible j,
 *     lse[b,h,i]   = log( sum_j exp(scale * <q[b,i,h,:], k[b,j,g,:]>) )  (natural log)
 *
 * with g = floor(h / (Hq / Hkv)).  This is scaled dot-product attention as the
 * interface section of the page "FlashAttention: exakte Attention-Kernel fuer
 * CUDA und ROCm" (hysenlabs.com, section "Die Schnittstellen von
 * flash_attn_func bis KV-Cache") states it: softmax(Q @ K^T * softmax_scale) @ V,
 * with a causal flag and fewer KV heads than query heads when the query head
 * count is divisible (MQA/GQA).  It is exact attention (tokenwerk.de,
 * "FlashAttention", section "Was FlashAttention veraendert"): the result
 * differs from a reference only by floating-point rounding.  The N x N score
 * matrix is never written to device memory; the kernel streams K/V tiles
 * through on-chip memory (tokenwerk.de, section "Warum Kacheln beim
 * Speicherzugriff helfen"; unite.ai, "Was ist FlashAttention?", section
 * "Eine fuenfstufige Betriebsuebersicht").
 *
 * Causal masking: key j is visible to query i iff j <= i + (Nk - Nq), i.e. the
 * mask is aligned to the bottom-right corner when Nq != Nk (hysenlabs.com page,
 * section "Von 2.0 bis 2.7", version 2.1).  A query row with no visible key gets
 * out = 0 and lse = -inf.
 *
 * Layouts (all contiguous, row-major, element = 2 bytes):
 *     q, out : [B, Nq, Hq, d]     k, v : [B, Nk, Hkv, d]     lse : [B, Hq, Nq] fp32
 * out has the element type of q, k and v; outputs are rounded to nearest-even.
 *
 * Ownership: every pointer is a DEVICE pointer owned by the caller, who keeps
 * the buffers alive until the enqueued work has finished.  The library
 * allocates no device memory and keeps no state besides a per-device cached
 * architecture check.
 *
 * Synchronisation: attn_fwd enqueues one kernel on `stream` (a hipStream_t;
 * NULL = the default stream) and returns without waiting.  Faults during
 * execution surface at the caller's next synchronisation.  Calls are
 * re-entrant and thread-safe.
 *
 * Errors: arguments are validated before any HIP call, in this order, and the
 * first failing check is returned; nothing is enqueued on error:
 *     shape -> empty (B == 0 or Nq == 0: returns ATTN_OK, pointers may be NULL)
 *     -> null pointers -> GQA ratio -> head dim -> dtype -> scale
 *     -> 16-byte alignment -> aliasing -> device -> launch.
 */
#ifndef EXACT_TILED_ATTENTION_ATTN_H
#define EXACT_TILED_ATTENTION_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v and out (the page's FlashAttention-2 envelope:
 * fp16 and bf16, hysenlabs.com, section "GPU-Abdeckung"). */
typedef enum { ATTN_DTYPE_F16 = 0, ATTN_DTYPE_BF16 = 1 } attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL_POINTER = -1,      /* q, k, v, out or lse is NULL                        */
  ATTN_ERR_BAD_SHAPE = -2,         /* B<0, Nq<0, Hq<1, Hkv<1, Nk<1, d<1, or too large    */
  ATTN_ERR_GQA_RATIO = -3,         /* Hq is not a multiple of Hkv                         */
  ATTN_ERR_UNSUPPORTED_HDIM = -4,  /* d not in {64, 128, 256}                             */
  ATTN_ERR_UNSUPPORTED_DTYPE = -5, /* dtype is not ATTN_DTYPE_F16 or ATTN_DTYPE_BF16      */
  ATTN_ERR_BAD_SCALE = -6,         /* scale is NaN or +-inf                               */
  ATTN_ERR_MISALIGNED = -7,        /* a base pointer is not 16-byte aligned              */
  ATTN_ERR_ALIASING = -8,          /* out or lse overlaps an input, or each other        */
  ATTN_ERR_NO_DEVICE = -9,         /* no HIP device, or the current device is not gfx950 */
  ATTN_ERR_LAUNCH = -10,           /* the kernel launch failed                            */
  ATTN_ERR_WORKSPACE = -11,        /* attn_decode: workspace smaller than required       */
  ATTN_ERR_BAD_ARGUMENT = -12,     /* window bound < -1, bad softcap; mask_heads not 1/Hq */
  ATTN_ERR_SCRATCH_LIMIT = -13     /* attn_decode_noalloc: partials exceed its scratch   */
} attn_status;

/*
 * Exact attention forward.
 *   q      [B, Nq, Hq, d]  element type `dtype`            (read)
 *   k, v   [B, Nk, Hkv, d] element type `dtype`            (read)
 *   out    [B, Nq, Hq, d]  element type `dtype`            (written)
 *   lse    [B, Hq, Nq]     fp32, natural-log logsumexp     (written)
 *   scale  the softmax scale (any finite value; 1/sqrt(d) is the usual one)
 *   causal nonzero: bottom-right aligned causal mask
 *   dtype  an attn_dtype value
 *   stream hipStream_t to enqueue on, or NULL
 * Returns an attn_status value.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d,
             float scale, int causal, int dtype, void* stream);

/*
 * attn_fwd with score variants: the sliding window, ALiBi and softcapping
 * that the hysenlabs.com page lists among the interface parameters
 * (window_size, alibi_slopes; section "Die Schnittstellen von
 * flash_attn_func bis KV-Cache") and dates in its version history (2.3,
 * 2.4, 2.6; section "Von 2.0 bis 2.7").  With diag = Nk - Nq and
 * t = scale * <q_i, k_j>:
 *   window       key j kept for row i iff i + diag - window_left <= j and
 *                j <= i + diag + window_right (-1 = no bound on that side;
 *                combined with the causal mask when causal != 0)
 *   softcap      > 0: t = softcap * tanh(t / softcap); 0 = off
 *   alibi_slopes NULL, or Hq fp32 device values: t -= slopes[h] * |i + diag - j|
 * then softmax over the kept keys as in attn_fwd (rows with no kept key:
 * out = 0, lse = -inf).  With every variant off this is attn_fwd.
 * Additional errors: ATTN_ERR_BAD_ARGUMENT (window bound < -1, softcap
 * negative or not finite), ATTN_ERR_MISALIGNED (slopes not 4-byte aligned),
 * ATTN_ERR_ALIASING (out or lse overlapping the slopes).
 */
int attn_fwd_ext(const void* q, const void* k, const void* v, void* out, float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 int window_left, int window_right, const float* alibi_slopes, float softcap,
                 int dtype, void* stream);

/*
 * attn_fwd over variable-length sequences packed along the row axis (the
 * unpadded layout the hysenlabs.com page's version history refers to,
 * section "Von 2.0 bis 2.7"): sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]); each sequence is attended on its
 * own exactly as attn_fwd does for one batch entry (causal: bottom-right
 * aligned per sequence; a sequence without keys gets out = 0, lse = -inf).
 *   q, out  [total_q, Hq, d]   k, v [total_k, Hkv, d]   lse [Hq, total_q] fp32
 *   cu_seqlens_q, cu_seqlens_k  [B + 1] int32, device, nondecreasing from 0
 *           to total_q / total_k (values outside [0, total] are clamped)
 *   max_seqlen_q  at least the longest query sequence (sizes the grid)
 * k and v may be NULL when total_k == 0.  Validation as attn_fwd; B == 0,
 * total_q == 0 or max_seqlen_q == 0 is a no-op.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                    int total_q, int total_k, int max_seqlen_q, int d, float scale, int causal,
                    int dtype, void* stream);

/*
 * attn_fwd restricted by a block mask (block sparsity, which the liora.io
 * item on FlexAttention's new backend lists among its features in its
 * section on limitations; the same item gives 128 x 128 as the Hopper
 * kernel's block size).  Query row i and key j interact only if
 *     block_mask[b, hm, i / 128, j / 128] != 0
 * with hm = 0 when mask_heads == 1 (one mask for all query heads) and hm = h
 * when mask_heads == Hq, and, when causal != 0, j <= i + (Nk - Nq) as in
 * attn_fwd.  Everything else is attn_fwd's definition; a row that keeps no
 * key gets out = 0 and lse = -inf.  Key blocks whose flag is 0 are never
 * read.
 *   block_mask  [B, mask_heads, ceil(Nq / 128), ceil(Nk / 128)] bytes,
 *               device, read; any nonzero byte keeps its block
 * The other arguments, layouts and the validation order are attn_fwd's, with
 * ATTN_ERR_NULL_POINTER also for a NULL block_mask, ATTN_ERR_BAD_ARGUMENT
 * when mask_heads is neither 1 nor Hq (checked after the scale), and
 * ATTN_ERR_ALIASING also when out or lse overlaps the mask.  The mask needs
 * no alignment.
 */
#define ATTN_BLOCK_MASK_SIZE 128
int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* out, float* lse,
                         const unsigned char* block_mask, int mask_heads, int B, int Hq, int Hkv,
                         int Nq, int Nk, int d, float scale, int causal, int dtype, void* stream);

/*
 * Exact attention backward: gradients of L = sum(dout * out) with respect to
 * q, k and v, for out = attn_fwd(q, k, v, scale, causal).  The pages state
 * that the library's backward pass computes these gradients, that it is
 * deterministic since version 2.4 (hysenlabs.com page, section "Von 2.0 bis
 * 2.7"), and that the tests compare gradients with a reference (section
 * "Tests, BSD-3-Clause und Zitierpraxis"); the formulas are the chain rule of
 * the forward definition above, with P the probabilities of attn_fwd:
 *
 *     delta[b,h,i] = sum_c dout[b,i,h,c] * out[b,i,h,c]
 *     dS[i,j]      = P[i,j] * ( sum_c dout[b,i,h,c] v[b,j,g,c] - delta[b,h,i] )
 *     dq[b,i,h,:]  = scale * sum_j dS[i,j] k[b,j,g,:]
 *     dk[b,j,g,:]  = scale * sum_{h in group g} sum_i dS[i,j] q[b,i,h,:]
 *     dv[b,j,g,:]  =         sum_{h in group g} sum_i P[i,j] dout[b,i,h,:]
 *
 * P is recomputed from q, k and the forward's lse; no N x N matrix is
 * stored.  Masked pairs and rows without a visible key contribute nothing.
 *   q, dout, out [B, Nq, Hq, d]  element type `dtype` (read); out and lse must
 *                                be attn_fwd's outputs for these arguments
 *   k, v         [B, Nk, Hkv, d] element type `dtype` (read)
 *   lse          [B, Hq, Nq]     fp32                 (read)
 *   dq           [B, Nq, Hq, d]  element type `dtype` (written)
 *   dk, dv       [B, Nk, Hkv, d] element type `dtype` (written; KV heads
 *                                shared by a GQA group get the group's sum)
 *   delta        [B, Hq, Nq]     fp32                 (written)
 * Two kernels are enqueued on `stream`; no atomics, so results are bitwise
 * reproducible.  The library allocates nothing.
 * Validation order as attn_fwd, with these differences: B == 0 is a no-op;
 * Nq == 0 (B > 0) writes zeros to dk and dv, and then q, out, dout, lse, dq
 * and delta may be NULL; ATTN_ERR_NULL_POINTER names any required pointer;
 * ATTN_ERR_ALIASING means an output (dq, dk, dv, delta) overlaps an input
 * or another output.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             int B, int Hq, int Hkv, int Nq, int Nk, int d,
             float scale, int causal, int dtype, void* stream);

/*
 * attn_bwd for attn_fwd_ext: gradients of L = sum(dout * out) for
 * out = attn_fwd_ext(q, k, v, ..., window_left, window_right, alibi_slopes,
 * softcap).  P is that function's probability matrix; the window and the
 * ALiBi bias enter through P only, and with a softcap the derivative of
 * cap * tanh(s / cap) multiplies dS before the products with K and Q:
 *     dS[i,j] = P[i,j] (dP[i,j] - delta[i]) (1 - tanh(s[i,j] / cap)^2)
 * with s = scale * <q_i, k_j>.  The arguments are attn_bwd's followed by
 * attn_fwd_ext's variant arguments (same meanings and checks:
 * ATTN_ERR_BAD_ARGUMENT after the scale, slopes 4-byte aligned and not
 * overlapped by an output).  No atomics: bitwise reproducible.
 */
int attn_bwd_ext(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* delta,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 int window_left, int window_right, const float* alibi_slopes, float softcap,
                 int dtype, void* stream);

/*
 * attn_bwd for attn_fwd_blocksparse: gradients of L = sum(dout * out) for
 * out = attn_fwd_blocksparse(q, k, v, block_mask, mask_heads, scale, causal)
 * (P is that function's probability matrix: zero outside the kept blocks).
 * The pages' FlexAttention item notes that its backward is not deterministic
 * with block sparsity enabled; this one, like attn_bwd, uses no atomics and
 * is bitwise reproducible.  Blocks whose flag is 0 are never read.
 *   block_mask, mask_heads  as for attn_fwd_blocksparse (may be NULL when
 *                           Nq == 0)
 * The other arguments, layouts and the validation order are attn_bwd's, with
 * ATTN_ERR_NULL_POINTER also for a NULL block_mask (Nq > 0),
 * ATTN_ERR_BAD_ARGUMENT when mask_heads is neither 1 nor Hq (checked after
 * the scale), and ATTN_ERR_ALIASING also when an output overlaps the mask.
 */
int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* delta, const unsigned char* block_mask, int mask_heads,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d,
                         float scale, int causal, int dtype, void* stream);

/*
 * attn_bwd for attn_fwd_varlen: gradients over sequences packed along the
 * row axis (sequence b: query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]), key
 * rows [cu_seqlens_k[b], cu_seqlens_k[b+1])), each sequence exactly as
 * attn_bwd computes it for one batch entry; sequences share no gradients.
 *   q, out, dout, dq  [total_q, Hq, d]      k, v, dk, dv  [total_k, Hkv, d]
 *   lse, delta        [Hq, total_q] fp32 (lse as attn_fwd_varlen returned it)
 *   cu_seqlens_q/k    [B + 1] int32, device (clamped to [0, total] as in
 *                     attn_fwd_varlen)
 *   max_seqlen_q/k    at least the longest query / key sequence (they size
 *                     the two grids; rows past them are not written)
 * Key rows of a sequence without query rows get dk = dv = 0; query rows of a
 * sequence without keys get dq = 0.  No atomics: bitwise reproducible.
 * Validation order as attn_bwd; B == 0 or total_q == total_k == 0 is a
 * no-op; the buffers of a side without rows (total_q == 0 or total_k == 0)
 * may be NULL.
 */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    float* delta, const int* cu_seqlens_q, const int* cu_seqlens_k,
                    int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                    int max_seqlen_k, int d, float scale, int causal, int dtype, void* stream);

/*
 * KV-cache decode forward: new query rows against a key/value cache that is
 * updated in place, as the interface section of the hysenlabs.com page
 * describes the inference function ("Die Schnittstellen von flash_attn_func
 * bis KV-Cache": it writes the new keys and values into k_cache and v_cache
 * directly and has no backward pass).
 *
 * For each batch b, with L = cache_seqlens[b] (device memory, read by the
 * kernels) and n_b = L + Nnew:
 *   1. k_cache[b, L + t] = k_new[b, t] and v_cache[b, L + t] = v_new[b, t]
 *      for t < Nnew (rows at or past Ncap are not written; the caller keeps
 *      L + Nnew <= Ncap);
 *   2. out[b, i, h] and lse[b, h, i] as attn_fwd computes them for query
 *      rows i < Nq against the keys and values [0, n_b) of the updated
 *      cache (causal: key j visible to row i iff j <= i + n_b - Nq).
 * cache_seqlens is not modified.
 *   q             [B, Nq, Hq, d]    element type `dtype` (read)
 *   k_cache, v_cache [B, Ncap, Hkv, d] element type `dtype` (read, rows
 *                                   [L, L + Nnew) written)
 *   cache_seqlens [B] int32, device (read)
 *   k_new, v_new  [B, Nnew, Hkv, d] element type `dtype` (read; may be NULL
 *                                   when Nnew == 0)
 *   out, lse      as attn_fwd (written)
 *   workspace     device scratch owned by the caller, at least
 *                 attn_decode_workspace_size(B, Hq, Nq, d, splits) bytes,
 *                 16-byte aligned (may be NULL when that size is 0); its
 *                 contents are undefined afterwards.  Calls sharing one
 *                 workspace must not overlap in time.
 *   num_splits    key ranges per (batch, KV head) computed by separate
 *                 workgroups and merged by logsumexp; 0 = the library's choice
 *                 (attn_decode_num_splits), otherwise 1..128.
 * The query heads of a GQA group share one pass over their KV head's cache.
 * Validation as attn_fwd; B == 0, or Nq == 0 with Nnew == 0, is a no-op;
 * ATTN_ERR_WORKSPACE when workspace_bytes is too small; ATTN_ERR_ALIASING
 * when a written buffer (caches, out, lse, workspace) overlaps another
 * buffer.  One or two kernels are enqueued on `stream` (the split attention,
 * which also appends the new rows, and with several splits their merge;
 * with Nq == 0 one append kernel).
 */
int attn_decode(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens,
                const void* k_new, const void* v_new, void* out, float* lse,
                void* workspace, size_t workspace_bytes,
                int B, int Hq, int Hkv, int Nq, int Ncap, int Nnew, int d,
                float scale, int causal, int dtype, int num_splits, void* stream);

/*
 * attn_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and validation as
 * attn_decode, minus workspace and workspace_bytes.  The split partials live
 * in a device array of ATTN_DECODE_SCRATCH_BYTES inside the library, one per
 * GPU it runs on, held until the process ends; no call allocates anything.
 *   num_splits == 0  attn_decode_num_splits' choice, lowered to the largest
 *                    count whose partials fit the array (1 split needs none);
 *   num_splits >= 2  ATTN_ERR_SCRATCH_LIMIT when
 *                    attn_decode_workspace_size(B, Hq, Nq, d, num_splits) >
 *                    ATTN_DECODE_SCRATCH_BYTES (checked before any HIP call).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero: each partial is written
 * before it is read).  Calls that overlap in time on one GPU race: issue them
 * on one stream, or order them.  The first call on a device looks up the
 * array's address on that device (hipGetSymbolAddress); ATTN_ERR_LAUNCH when
 * that fails.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
int attn_decode_noalloc(const void* q, void* k_cache, void* v_cache, const int* cache_seqlens,
                        const void* k_new, const void* v_new, void* out, float* lse,
                        int B, int Hq, int Hkv, int Nq, int Ncap, int Nnew, int d,
                        float scale, int causal, int dtype, int num_splits, void* stream);

/* The split count attn_decode uses for num_splits == 0 (always >= 1). */
int attn_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Ncap, int d);

/* Workspace bytes attn_decode needs for `num_splits` splits (0 for one split). */
size_t attn_decode_workspace_size(int B, int Hq, int Nq, int d, int num_splits);

/* A fixed, static message for a status code (never NULL; unknown codes get a
 * message of their own).  tokenwerk.de's "FlashAttention" page (section
 * "Fehler und Leistungsversprechen richtig einordnen") asks that a failing
 * call's exact message be recorded: each code maps to one unchanging string,
 * so a caller can log it verbatim and compare it across runs.  The pointer
 * refers to static storage; the caller does not free it. */
const char* attn_status_string(int status);

/* Library version and build description, e.g. "0.2.0 gfx950 ...".  The same
 * page asks that a performance claim name what was measured; the version
 * string identifies the library build behind a measurement.  Static storage,
 * never NULL. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TILED_ATTENTION_ATTN_H */
