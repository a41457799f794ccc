/*
 * kvc.h -- attention against a KV cache on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over four operations and two helpers.  Every pointer named
 * "device" must point to memory on the current HIP device; the library never
 * allocates, never frees and keeps no caller pointer after a call returns.
 * Its state is per device: a cached read-only device property (the CU count)
 * and one static scratch array that only kvc_attn_decode_noalloc uses, so
 * calls on different streams are independent except for that one call.
 * Every call is asynchronous on the given stream (a hipStream_t passed as
 * void*, NULL for the default stream) and never synchronises the device.
 *
 * Cache layout (nanochat post, "What the KV cache looks like on disk"): K and
 * V are each one contiguous array of shape
 *     (n_layers, batch, max_seq, n_kv_heads, head_dim)
 * in row-major order, and seqlens is an int32 array of shape (batch,) giving
 * how many positions of each row are filled.  Under GQA the cache holds only
 * the n_kv_heads key/value heads; query head h reads KV head
 * h / (n_q_heads / n_kv_heads).  The library's kernels read seqlens and never
 * change it (the clone excepted, which sets the destination's): as on that
 * page, the caller advances it once per step, after every layer has run.
 *
 * Data types: q, out, k_new, v_new and the cache share one element type,
 * KVC_F32 or KVC_BF16 (bfloat16, round to nearest even).  All accumulation
 * is in float32.  head_dim must be 64 or 128.
 *
 * Rolling window (rolling = 1).  Tiny-GPT post, "The Cache, in Code" and "Does
 * the Cache Change the Output?": the cache keeps the last max_seq positions,
 * each rotated at its absolute position; under RoPE a score is a function of
 * how far apart the two positions are, not of where they sit, so the window
 * can slide without rotating any cached key again.  seqlens[b] then counts
 * every token row b has seen, and absolute position p lives in slot
 * p mod max_seq.  kvc_rope_append writes
 * token t at slot (P + t) mod max_seq (T <= max_seq, else KVC_E_ARG), rotated
 * at P + t; a one-token decode (kvc_attn_decode, kvc_decode_step) attends the
 * min(P + 1, max_seq) filled slots -- positions max(0, P + 1 - max_seq) .. P,
 * order being irrelevant to softmax.  kvc_attn_prefill keeps the linear rule
 * P + T <= max_seq for every T, so a prompt is prefilled before the window
 * first wraps; the clone copies slots [0, src_len) as in a linear cache.
 *
 * 8-bit cache (KVC_I8).  Cake paper, Section 5.1 ("Compression methods") and
 * Section 5.5 (Table 6): the KV cache can be kept in 8 bits, which halves the
 * bytes decode must stream.  K and V then hold int8 codes, and k_scale /
 * v_scale hold one float32 scale per cached vector, shape
 *     (n_layers, batch, n_kv_heads, max_seq),
 * head-major, so that one KV head's scales are contiguous over positions and
 * a decode tile's scales are one dense run.
 * A vector x (the head_dim values of one position and KV head, as a bfloat16
 * cache would hold them: the rotated key rounded to bfloat16, the value
 * rounded to bfloat16) is stored as s = amax|x| / 127 and codes
 * c_i = round_half_even(x_i / s) in [-127, 127] (float32 quotient; s = 0 and
 * all codes 0 for an all-zero vector); it reads back as c_i * s.  q, out,
 * k_new and v_new are bfloat16.  kvc_rope_append quantizes as it appends,
 * kvc_attn_decode decodes from the codes, and kvc_prefill_clone copies codes
 * and scales.  kvc_attn_prefill and kvc_decode_step do not take an 8-bit
 * cache (KVC_E_DTYPE).
 *
 * Errors.  A call first validates its arguments on the host; if that fails
 * it returns a negative KVC_E_* code and launches nothing, so nothing is
 * written.  Conditions that depend on device data (seqlens) are checked by
 * the kernels: the offending batch row is skipped -- nothing is written for
 * it -- and the matching KVC_DEV_* bit is OR-ed into *dev_err, a device int32
 * the caller owns and reads after it next synchronises.  dev_err may be NULL,
 * in which case those rows are still skipped but not reported.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of the cache (and of q, out, k_new, v_new: bfloat16 for KVC_I8). */
enum { KVC_F32 = 0, KVC_BF16 = 1, KVC_I8 = 2 };

/* Host-side status codes (return values). */
enum {
  KVC_OK = 0,
  KVC_E_ARG = -1,       /* null pointer, T < 1, layer out of range, bad scale or split size */
  KVC_E_SHAPE = -2,     /* n_q_heads % n_kv_heads != 0, unsupported head_dim, descriptor mismatch */
  KVC_E_CAPACITY = -3,  /* clone: dst.max_seq < src.max_seq, or src_len outside [0, src.max_seq] */
  KVC_E_DTYPE = -4,     /* unknown element type, or source and destination types differ */
  KVC_E_WORKSPACE = -5, /* decode workspace missing or smaller than kvc_decode_workspace_bytes */
  KVC_E_LAUNCH = -6,    /* a HIP launch failed */
  KVC_E_SCRATCH = -7    /* kvc_attn_decode_noalloc: the call needs more than KVC_DECODE_SCRATCH_MAX_BYTES */
};

/* Bytes of the static device scratch behind kvc_attn_decode_noalloc (16 MiB). */
#define KVC_DECODE_SCRATCH_MAX_BYTES ((size_t)16 << 20)

/* Device-side error bits OR-ed into *dev_err. */
enum {
  KVC_DEV_CAPACITY = 1,  /* seqlens[b] < 0, or seqlens[b] + T > max_seq: row b skipped */
  KVC_DEV_NOT_EMPTY = 2, /* clone: destination row b had seqlens[b] != 0: row b skipped */
  KVC_DEV_SRC_LEN = 4,   /* clone: source seqlens[0] != src_len: nothing copied */
  KVC_DEV_TOKENS = 8     /* ragged calls: row b's token range in cu_tokens is malformed: row b skipped */
};

/* Describes caller-owned device buffers; the library only reads the struct. */
typedef struct kvc_cache {
  void* k;          /* device, (n_layers, batch, max_seq, n_kv_heads, head_dim) */
  void* v;          /* device, same shape as k */
  int32_t* seqlens; /* device, (batch,) */
  int32_t n_layers;
  int32_t batch;
  int32_t max_seq;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;    /* KVC_F32, KVC_BF16 or KVC_I8 */
  float* k_scale;   /* KVC_I8 only: device, (n_layers, batch, n_kv_heads, max_seq); else ignored */
  float* v_scale;   /* KVC_I8 only: device, same shape */
  int32_t rolling;  /* 0: linear cache; 1: rolling window of max_seq positions (see above) */
} kvc_cache;

/*
 * kvc_rope_append -- rotate new q and k at each row's own position offset
 * and write the new k and v in place into layer `layer` of the cache.
 *
 * Tiny-GPT post, "Two Gotchas That Break It Quietly", Gotcha 1: a cached
 * step rotates its tokens at positions start .. start+T-1, where start is the
 * row's offset, with angles f32(f32(p) * inv_freq[i]), inv_freq[i] =
 * rope_base^(-2i/head_dim) (rounded once to float32), dimension i paired
 * with i + head_dim/2.  "The Cache, in Code": the rotated q and k are cast to
 * the value type and the rotated k is what the cache keeps.  nanochat post,
 * "What the KV cache looks like on disk": the new K/V slices are written in
 * place at each row's cache_seqlens offset.
 *
 *   q      device, (batch, T, n_q_heads, head_dim), raw (unrotated) queries.
 *   q_out  device, same shape; receives the rotated queries.  May equal q.
 *   k_new  device, (batch, T, n_kv_heads, head_dim), raw keys.
 *   v_new  device, (batch, T, n_kv_heads, head_dim), values (copied bit for bit).
 *
 * For row b with P = seqlens[b], token t goes to position P + t:
 *   K[layer, b, P+t] = round(rotate(k_new[b, t], P+t)),  V[layer, b, P+t] = v_new[b, t],
 *   q_out[b, t] = round(rotate(q[b, t], P+t)).
 * Nothing else in the cache is written and seqlens is not changed.  A row with
 * P < 0 or P + T > max_seq is skipped entirely (KVC_DEV_CAPACITY), q_out included.
 */
int kvc_rope_append(const kvc_cache* cache, int32_t layer, const void* q, void* q_out,
                    const void* k_new, const void* v_new, int32_t T, int32_t n_q_heads,
                    float rope_base, int32_t* dev_err, void* stream);

/*
 * kvc_decode_workspace_bytes -- size of the float32 scratch kvc_attn_decode
 * needs for its partial results with this cache, query-head count and worker
 * count (n_workers 0 = the library default).  A host function: it may query
 * the current HIP device's properties, and launches nothing.  Returns 0 for an
 * invalid descriptor or when no scratch is needed.
 */
size_t kvc_decode_workspace_bytes(const kvc_cache* cache, int32_t n_q_heads, int32_t n_workers);

/*
 * kvc_attn_decode -- one query token per row against the whole cached
 * prefix of layer `layer`, after its k/v were appended.
 *
 * Tiny-GPT post, Gotcha 2: a single decode query sees every cached key
 * (no causal mask).  nanochat post: attention runs against the full cache,
 * with GQA head sharing.  Cake paper, Section 3: softmax(q K^T * scale) V,
 * scale = 1/sqrt(head_dim) (the default of the post's attention call).
 *
 *   q_rot  device, (batch, 1, n_q_heads, head_dim), rotated queries (q_out of
 *          kvc_rope_append).
 *   out    device, same shape as q_rot.
 *   scale  softmax scale; <= 0 selects 1/sqrt(head_dim).
 *   n_workers  bfloat16 and int8 caches: the number of workgroups the cached
 *          keys of all rows are split evenly over (split-KV); 0 = one per
 *          compute unit of the current device.  Float32 caches use fixed
 *          512-key splits and ignore it.  A result depends on the lengths of
 *          all rows and on
 *          n_workers only through the order of float32 additions; it is
 *          bit-identical run to run for the same inputs and n_workers.
 *   workspace   device scratch of at least kvc_decode_workspace_bytes bytes,
 *          owned by the caller, clobbered by the call.
 *
 * For row b with P = seqlens[b], keys 0..P (P+1 of them, the new token's
 * included) are attended.  Rows with P < 0 or P + 1 > max_seq are skipped
 * (KVC_DEV_CAPACITY) and their out is not written.  bfloat16 caches whose one
 * head row (max_seq * n_kv_heads * head_dim elements) reaches 2^30 are
 * rejected with KVC_E_SHAPE.
 */
int kvc_attn_decode(const kvc_cache* cache, int32_t layer, const void* q_rot, void* out,
                    int32_t n_q_heads, float scale, int32_t n_workers, void* workspace,
                    size_t workspace_bytes, int32_t* dev_err, void* stream);

/*
 * kvc_attn_decode_noalloc -- kvc_attn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels, with the partial results in a
 * static device array of KVC_DECODE_SCRATCH_MAX_BYTES that the library owns
 * (one copy per device, held until the process ends) instead of a caller
 * workspace.  It calls no allocating routine.
 *
 * Arguments, results and errors are kvc_attn_decode's (output bit-identical
 * to it for the same inputs and n_workers), except: a call whose
 * kvc_decode_workspace_bytes(cache, n_q_heads, n_workers) exceeds
 * KVC_DECODE_SCRATCH_MAX_BYTES returns KVC_E_SCRATCH and launches nothing.
 * With the default worker count every bfloat16 and int8 cache fits (at most
 * 8.5 MB at 256 workgroups); a float32 cache needs
 * batch * n_q_heads * ceil(max_seq / 512) * (head_dim + 2) * 4 bytes once
 * max_seq exceeds 512.  The array's address on a device is looked up on the
 * first call made with that device current.
 *
 * Every call on one device shares that device's array, and each call
 * overwrites what the last one left there (no part of it needs to start at
 * zero).  Calls that overlap in time on one device -- on different streams,
 * or from different host threads without stream ordering -- race on it and
 * may return wrong results; calls ordered on one stream are safe.
 */
int kvc_attn_decode_noalloc(const kvc_cache* cache, int32_t layer, const void* q_rot, void* out,
                            int32_t n_q_heads, float scale, int32_t n_workers, int32_t* dev_err, void* stream);

/*
 * kvc_attn_prefill -- T new query tokens per row, causal by absolute position,
 * against layer `layer` of the cache after their k/v were appended.
 *
 * Tiny-GPT post, Gotcha 2 (causal mask for a multi-token prompt) and Cake
 * paper, Section 3 "Chunk Prefill" (each chunk attends to every earlier
 * token): query t of row b sits at position P + t, P = seqlens[b], and sees
 * keys 0..P+t.  P = 0 is a one-shot prefill; P > 0 a later chunk.  bfloat16
 * runs on MFMA matrix cores (float32 accumulation, probabilities rounded to
 * bfloat16 for the P*V product); float32 runs on vector ALUs.
 *
 *   q_rot  device, (batch, T, n_q_heads, head_dim), rotated queries.
 *   out    device, same shape.
 *   scale  softmax scale; <= 0 selects 1/sqrt(head_dim).
 *
 * Rows with P < 0 or P + T > max_seq are skipped (KVC_DEV_CAPACITY).  bfloat16
 * caches whose one head row (max_seq * n_kv_heads * head_dim elements) reaches
 * 2^30 are rejected with KVC_E_SHAPE.
 */
int kvc_attn_prefill(const kvc_cache* cache, int32_t layer, const void* q_rot, void* out,
                     int32_t T, int32_t n_q_heads, float scale, int32_t* dev_err, void* stream);

/*
 * Ragged batches.  Cake paper, Section 3: serving systems run chunked prefill
 * beside decoding in one batch (the chunk of one request next to the single
 * new tokens of others).  The two calls below take such a batch: row b brings
 * T_b >= 0 new tokens, packed one after another,
 *
 *   cu_tokens   device int32, (batch + 1,): row b's tokens are packed rows
 *               [cu_tokens[b], cu_tokens[b+1]) of q, q_out, k_new, v_new and
 *               out; T_b = cu_tokens[b+1] - cu_tokens[b].  Read, never written.
 *   n_tokens    packed rows in those tensors (their leading dimension), >= 0.
 *   max_tokens  host-known bound on every T_b, >= 1; it sizes the grid.
 *
 * and the tensors are (n_tokens, heads, head_dim).  A row whose range is
 * malformed (cu_tokens[b] < 0, a decreasing pair, an end past n_tokens, or
 * T_b > max_tokens) is skipped and KVC_DEV_TOKENS is set; nothing outside the
 * packed rows is ever read or written.  A row with T_b = 0 is left alone, and
 * a call with n_tokens = 0 returns KVC_OK without launching anything (its
 * tensor pointers may then be null).
 * Otherwise each row follows the rules of the uniform calls with T = T_b.
 */

/*
 * kvc_rope_append_ragged -- kvc_rope_append for a ragged batch: row b's T_b
 * tokens go to positions P .. P + T_b - 1 (P = seqlens[b]), its rotated
 * queries to the same packed rows of q_out.  Rows with P < 0 or
 * P + T_b > max_seq are skipped (KVC_DEV_CAPACITY); on a rolling cache
 * max_tokens must not exceed max_seq.
 */
int kvc_rope_append_ragged(const kvc_cache* cache, int32_t layer, const void* q, void* q_out,
                           const void* k_new, const void* v_new, const int32_t* cu_tokens,
                           int32_t n_tokens, int32_t max_tokens, int32_t n_q_heads, float rope_base,
                           int32_t* dev_err, void* stream);

/*
 * kvc_attn_mixed -- attention for a ragged batch in one call, after its k/v
 * were appended: rows with one new token decode (keys 0..P, as
 * kvc_attn_decode, the rolling rule included), rows with more prefill
 * causally (query t sees keys 0..P+t, as kvc_attn_prefill, linear rule),
 * rows with none are left alone.
 *
 *   q_rot, out  device, (n_tokens, n_q_heads, head_dim), packed.
 *   scale, n_workers, workspace, workspace_bytes  as kvc_attn_decode: the
 *               workspace needs kvc_decode_workspace_bytes(cache, n_q_heads,
 *               n_workers) bytes (none for float32 caches).
 *
 * bfloat16: the prefill rows run the matrix-core prefill kernel and the
 * decode rows the split-KV decode (two launches and the fold, in stream
 * order; each kernel skips the other's rows).  float32: one launch, one
 * direct split per query row.  int8 caches are rejected (KVC_E_DTYPE), as by
 * kvc_attn_prefill.  The outputs of a prefill row are bit-identical to
 * kvc_attn_prefill on that row alone; a decode row's differ from
 * kvc_attn_decode only in the order of float32 additions.
 */
int kvc_attn_mixed(const kvc_cache* cache, int32_t layer, const void* q_rot, void* out,
                   const int32_t* cu_tokens, int32_t n_tokens, int32_t max_tokens, int32_t n_q_heads,
                   float scale, int32_t n_workers, void* workspace, size_t workspace_bytes,
                   int32_t* dev_err, void* stream);

/*
 * kvc_decode_step -- one decode token per row in a single launch: RoPE of the
 * new q and k at the row's position, in-place append of k and v, and
 * attention of the rotated queries over keys 0..P (P = seqlens[b], the new
 * key included).  No workspace.
 *
 * For small shapes, where a decode step is bound by kernel launches rather
 * than arithmetic (Tiny-GPT post, "Why the GPU Shrugs"), and after the
 * nanochat post ("What the KV cache looks like on disk"): the new K/V slices
 * are written in place and attention runs against the full cache in one
 * kernel launch.  The result equals kvc_rope_append (T = 1, same rope_base)
 * followed by kvc_attn_decode, up to the order of float32 additions; the K/V
 * bytes written into slot P are identical to kvc_rope_append's.  One
 * workgroup handles one (row, KV head) and walks the row's keys itself, so
 * this call suits short rows and small batches; long rows decode faster with
 * kvc_rope_append + kvc_attn_decode, which spread a row over the whole GPU.
 *
 *   q        device, (batch, 1, n_q_heads, head_dim), raw (unrotated) queries.
 *   k_new    device, (batch, 1, n_kv_heads, head_dim), raw key.
 *   v_new    device, same shape, value.
 *   out      device, (batch, 1, n_q_heads, head_dim).  May alias q: each
 *            workgroup reads its query heads before it writes them.
 *   scale    softmax scale; <= 0 selects 1/sqrt(head_dim).
 *   rope_base  RoPE base (10000 in the pages' workloads); must be > 1.
 *
 * n_q_heads / n_kv_heads must not exceed 16 (KVC_E_SHAPE).  seqlens is read,
 * never written: the caller advances it after every layer of the step.  Rows
 * with P < 0 or P + 1 > max_seq are skipped (KVC_DEV_CAPACITY): nothing is
 * written for them.
 */
int kvc_decode_step(const kvc_cache* cache, int32_t layer, const void* q, const void* k_new,
                    const void* v_new, void* out, int32_t n_q_heads, float scale, float rope_base,
                    int32_t* dev_err, void* stream);

/*
 * kvc_prefill_clone -- copy a batch-1 prefill into every row of an empty
 * batch-N cache (nanochat post, "The prefill trick, 12 lines").
 *
 * Preconditions, from the post's asserts: the destination is empty, both
 * caches have the same n_layers, n_kv_heads and head_dim (the post's n_heads
 * read as the cache's KV-head axis) and element type, and dst->max_seq >=
 * src->max_seq; src->batch must be 1.  src_len is the host-known number of
 * filled source positions (the post's other.get_pos()); it must equal
 * src->seqlens[0] on the device.
 *
 * For every layer and every destination row b with dst seqlens[b] == 0:
 *   dst K/V[layer, b, 0:src_len] = src K/V[layer, 0, 0:src_len], then dst seqlens[b] = src_len.
 * Destination positions >= src_len are not touched.  A row with
 * seqlens[b] != 0 is skipped (KVC_DEV_NOT_EMPTY); if src seqlens[0] !=
 * src_len nothing at all is written (KVC_DEV_SRC_LEN).
 */
int kvc_prefill_clone(const kvc_cache* src, int32_t src_len, const kvc_cache* dst,
                      int32_t* dev_err, void* stream);

/* A static, human-readable string for a KVC_OK / KVC_E_* status. */
const char* kvc_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
