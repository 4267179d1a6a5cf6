/*
 * inkling_rel_attn.h - C ABI of the MI355X (gfx950) relative-bias paged
 * attention library (libinkling_rel_attn.so).
 *
 * The operation (TensorRT-LLM Inkling page, section "Architecture"): the
 * model uses no rotary embedding.  Position enters only through a learned
 * bias, one value per (query token, query head, relative distance), added to
 * the scaled QK^T logit before the softmax.  Local layers attend over a
 * sliding window (512 keys, 16 KV heads); global layers attend over the full
 * causal prefix (8 KV heads); query heads share grouped KV heads.  Keys and
 * values always come from a paged cache (vLLM page, section "Purpose").  The
 * TensorRT-LLM page (section "Implementation") describes a paged prefill and
 * a decode kernel with a static-shape bias, so decode can be captured in a
 * graph; the vLLM page (section "Changes") describes a split-KV decode with
 * a separate query for the split count.
 *
 * For sequence b with n_b new query tokens and L_b keys (including the new
 * ones), query token t sits at logical position p = L_b - n_b + t.  With
 * d = p - j the distance to key j, key j is visible when d >= 0 and, for a
 * sliding window W > 0, d < W.  For query row i (packed), head h, and
 * G = Hq / Hkv, KV head g = h / G:
 *
 *   s_j = scale * <q[i,h,:], K_j[g,:]> + rel_logits[i, h, min(d, R-1)]
 *   out[i,h,:] = sum_j softmax_j(s) * V_j[g,:]     (visible j only)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensors are dense, row-major, caller-owned device memory.  The
 *    library never allocates, frees, copies between host and device or
 *    synchronises; all work is enqueued on `stream` (graph-capturable).
 *  - q, k_cache, v_cache, rel_logits and out share one dtype (dims->dtype).
 *    Every tensor pointer (and the decode workspace) is 16-byte aligned;
 *    a misaligned one is INKLING_ERR_INVALID_ARGUMENT.
 *  - k_cache / v_cache: [num_blocks, block_size, Hkv, head_dim]; logical key
 *    j of sequence b lives in page block_table[b * max_blocks_per_seq + j /
 *    block_size], slot j % block_size.
 *  - Host-visible arguments are validated before any launch; an invalid
 *    argument returns a status and launches nothing.  num_seqs == 0 returns
 *    INKLING_OK without a launch.
 *  - Device-resident metadata is a precondition, not checked (checking it
 *    would need a host sync): 0 <= n_b <= max_q_len, n_b <= L_b <=
 *    max_seq_len, cu_q_lens non-decreasing with cu_q_lens[0] = 0 and
 *    cu_q_lens[B] = total_q, block ids of the first ceil(L_b / block_size)
 *    entries in [0, num_blocks).  The kernels clamp what they read so that a
 *    violated precondition cannot make them access memory outside the
 *    arguments, but the result is then unspecified.
 *  - K/V rows that no query of the call can see (keys older than every
 *    query's window, slots at or past L_b, pages the block table does not
 *    reference) and rel_logits entries no visible (query, key) pair indexes
 *    may hold anything, NaN included: they never reach an output.  A
 *    non-finite K/V row of a key that some query of a sequence sees may make
 *    other rows of that sequence non-finite as well (their weight for it is
 *    0, and 0 * NaN is NaN).
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef INKLING_REL_ATTN_H
#define INKLING_REL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  INKLING_OK = 0,
  INKLING_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, Hq % Hkv   */
  INKLING_ERR_UNSUPPORTED = 2,        /* head_dim, block_size, dtype, R     */
  INKLING_ERR_UNSUPPORTED_DEVICE = 3, /* device is not gfx950               */
  INKLING_ERR_NO_DEVICE = 4,          /* no HIP device visible              */
  INKLING_ERR_WORKSPACE_TOO_SMALL = 5,
  INKLING_ERR_LAUNCH = 6              /* the runtime rejected a launch      */
} inkling_status_t;

typedef enum { INKLING_DTYPE_BF16 = 0, INKLING_DTYPE_FP32 = 1 } inkling_dtype_t;

/* Shapes of one call.  Read during the call only, never retained. */
typedef struct {
  int32_t num_seqs;           /* B (at most 65535)                           */
  int32_t num_q_heads;        /* Hq                                          */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0 and Hq / Hkv <= 16        */
  int32_t head_dim;           /* 64 or 128                                   */
  int32_t block_size;         /* tokens per page: 16                         */
  int32_t num_blocks;         /* pages in the pool                           */
  int32_t max_blocks_per_seq; /* row stride of block_table                   */
  int32_t rel_len;            /* R, last dim of rel_logits; R * sizeof(dtype)
                                 must be a multiple of 16 bytes             */
  int32_t total_q;            /* rows of q / out / rel_logits                */
  int32_t max_q_len;          /* host-known bound on n_b (sizes the grid)    */
  int32_t max_seq_len;        /* host-known bound on L_b                     */
  int32_t dtype;              /* inkling_dtype_t                             */
} inkling_rel_attn_dims_t;

/*
 * Varlen prefill (any n_b >= 0, so a chunked batch mixing decode rows and
 * prompt chunks is one call).  The caller has already written the new
 * tokens' K/V into their pages.
 *   q          [total_q, Hq, head_dim]
 *   block_table int32 [num_seqs, max_blocks_per_seq]
 *   seq_lens   int32 [num_seqs]   L_b
 *   cu_q_lens  int32 [num_seqs+1] packed row offsets
 *   rel_logits [total_q, Hq, R]
 *   window     > 0: sliding window of `window` keys (query included);
 *              <= 0: full causal attention
 *   scale      multiplies q.k only (the bias is not scaled); finite
 *   out        [total_q, Hq, head_dim], written for every row
 */
inkling_status_t inkling_rel_attn_prefill(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens,
    const int32_t* cu_q_lens, const void* rel_logits, int32_t window,
    float scale, void* out, const inkling_rel_attn_dims_t* dims,
    void* stream /* hipStream_t; NULL = default stream */);

/*
 * Prefill that also appends the new tokens' K/V rows to the cache, in the
 * same launch (the attention-side KV write of the TensorRT-LLM Inkling
 * page's pull request, commit list: the attention op's arguments include
 * a switch to skip its own KV write).  Same inputs, outputs and errors as
 * inkling_rel_attn_prefill, plus:
 *   k_new, v_new  [total_q, Hkv, head_dim] in the cache dtype, rows aligned
 *                 with q: row cu_q_lens[b] + t holds the K / V of token t
 *                 of sequence b, at position L_b - n_b + t.  Each row is
 *                 stored into its cache slot (page block_table[b][pos / 16],
 *                 slot pos % 16), and the attention reads every new key
 *                 from these rows, whatever the slots held before.
 *   k_cache, v_cache  read and written; slots of new tokens must be
 *                 distinct across the batch; k_new / v_new must not
 *                 overlap the caches.
 * Null k_new or v_new (with total_q > 0) is INKLING_ERR_INVALID_ARGUMENT.
 * Later work on the stream sees the stored rows.
 */
inkling_status_t inkling_rel_attn_prefill_append(
    const void* q, const void* k_new, const void* v_new, void* k_cache,
    void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
    const int32_t* cu_q_lens, const void* rel_logits, int32_t window,
    float scale, void* out, const inkling_rel_attn_dims_t* dims,
    void* stream);

/*
 * Single-token decode with split-KV (vLLM page, section "Changes": the keys
 * of each sequence are split into num_splits parts, each part produces a
 * partial output and its log-sum-exp, and a merge pass combines them).
 * Row b of q / rel_logits / out is the one new token of sequence b, at
 * position L_b - 1 (total_q must equal num_seqs).
 *   num_splits 0 = library choice (inkling_rel_attn_num_splits); 1 = one
 *              pass, no merge; at most 128.
 *   workspace  device memory of at least
 *              inkling_rel_attn_decode_workspace_bytes(dims, window,
 *              num_splits) bytes,
 *              16-byte aligned; may be NULL only when that size is 0.
 *              Contents on entry are ignored; on exit they are unspecified.
 */
inkling_status_t inkling_rel_attn_decode(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens,
    const void* rel_logits, int32_t window, float scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes, void* out,
    const inkling_rel_attn_dims_t* dims, void* stream);

/*
 * The same decode as inkling_rel_attn_decode, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation): it takes no workspace and calls no
 * allocating routine.  The split partials go to a buffer the library holds
 * on each GPU it runs on (a 32 MiB device array, kept until the process
 * ends), whose address is looked up on the first call on that GPU.
 *   - A call whose split workspace, inkling_rel_attn_decode_workspace_bytes(
 *     dims, window, num_splits), exceeds 32 MiB returns
 *     INKLING_ERR_WORKSPACE_TOO_SMALL and launches nothing (use
 *     inkling_rel_attn_decode with a caller workspace, or fewer splits).
 *   - Every call on one GPU shares that buffer: calls that overlap in time
 *     on one GPU (on different streams, or from several threads without
 *     ordering) race and give unspecified results.  Calls ordered on one
 *     stream are safe; nothing in it needs to start at zero.
 *   - No device is current: INKLING_ERR_NO_DEVICE.  Other arguments, outputs
 *     and errors as inkling_rel_attn_decode.
 */
inkling_status_t inkling_rel_attn_decode_noalloc(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens,
    const void* rel_logits, int32_t window, float scale, int32_t num_splits,
    void* out, const inkling_rel_attn_dims_t* dims, void* stream);

/*
 * Decode that also appends this step's K/V rows to the cache, in the same
 * launch.  The TensorRT-LLM Inkling page's pull request (commit list, the
 * clean-up of the attention op's arguments) shows an attention op that
 * writes the new K/V itself unless told to skip it.  Same inputs, outputs
 * and errors as inkling_rel_attn_decode, plus:
 *   k_new, v_new  [num_seqs, Hkv, head_dim] in the cache dtype: the K and V
 *                 rows of each sequence's new token (position L_b - 1).
 *                 Row b is stored into page block_table[b][(L_b - 1) / 16],
 *                 slot (L_b - 1) % 16, and the attention uses it as key
 *                 L_b - 1 whatever that slot held before.  Sequences with
 *                 L_b = 0 store nothing.
 *   k_cache, v_cache  read and written.  No two sequences may map key
 *                 L_b - 1 to the same slot; k_new / v_new must not overlap
 *                 the caches.
 * Null k_new or v_new (with num_seqs > 0) is INKLING_ERR_INVALID_ARGUMENT.
 * Later work on the stream sees the stored rows.
 */
inkling_status_t inkling_rel_attn_decode_append(
    const void* q, const void* k_new, const void* v_new, void* k_cache,
    void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
    const void* rel_logits, int32_t window, float scale, int32_t num_splits,
    void* workspace, size_t workspace_bytes, void* out,
    const inkling_rel_attn_dims_t* dims, void* stream);

/*
 * Split count the library would use for a decode call with these shapes
 * (1..128).  Chosen from the device's compute-unit count, B * Hkv and the
 * keys per sequence (window on local layers, max_seq_len on global ones).
 * device < 0 or no device: assumes 256 compute units.  Never fails; a null
 * dims gives 1.
 */
int32_t inkling_rel_attn_num_splits(const inkling_rel_attn_dims_t* dims,
                                    int32_t window, int32_t device);

/* Workspace bytes a decode call with `num_splits` needs (0 when it is 1;
 * num_splits 0 means the library's choice for device 0, which depends on
 * the window as well as the shapes, hence the window argument). */
size_t inkling_rel_attn_decode_workspace_bytes(
    const inkling_rel_attn_dims_t* dims, int32_t window, int32_t num_splits);

/*
 * Checks that `device` exists and is a gfx950 GPU.  On failure writes a
 * NUL-terminated message naming the device and its architecture into msg
 * (when msg != NULL and msg_len > 0).  This is the up-front support check
 * of the vLLM page (sections "Purpose" and "Changes"): a device the kernels
 * were not built for is rejected before any work, with an error that names
 * it, instead of failing later inside a kernel.  Returns INKLING_OK,
 * INKLING_ERR_NO_DEVICE, INKLING_ERR_INVALID_ARGUMENT (no such device) or
 * INKLING_ERR_UNSUPPORTED_DEVICE.
 */
inkling_status_t inkling_rel_attn_check_device(int32_t device, char* msg,
                                               size_t msg_len);

/* Static string describing a status code. */
const char* inkling_rel_attn_status_string(inkling_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* INKLING_REL_ATTN_H */
