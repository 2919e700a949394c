/*
 * pkv.h -- C ABI of libpkv: paged KV-cache decode attention for MI355X (gfx950).
 *
 * The operation: for each sequence b and query head h, the newest query
 * q[b,h,:] is scored against every cached key of KV head h / (Hq/Hkv),
 * scores are scaled (normally by 1/sqrt(head_dim)), passed through a softmax,
 * and the output is the weighted sum of the cached values:
 *
 *   out[b,h,:] = sum_t softmax_t(scale * q[b,h,:] . K_b[t,:]) V_b[t,:],
 *   t = 0 .. context_lens[b]-1,
 *
 * which is the attention formula of §1.1 of the page "The KV Cache Problem
 * of Traditional Attention" (pyllm.pages.dev) and §1.2 of "Understanding KV
 * Cache: Attention, P/D Disaggregation and vLLM's Paged Memory Management"
 * (steinslab.io), evaluated for the last row of the causal mask (§2.2,
 * "Decode"). K_b and V_b are gathered through a per-sequence block table that
 * maps logical 16-token blocks to physical blocks of a shared pool (page "KV
 * Cache and Inference Optimization", note.yj-dis.top, section "PagedAttention:
 * manage the KV cache like virtual memory"; slot rule of "Understanding KV
 * Cache" §3.3).
 *
 * Conventions shared by every call:
 *  - Pointers named "device" are GPU memory owned by the caller; the library
 *    never allocates, frees or keeps device memory (the allocator below is a
 *    host-side bookkeeping object that hands out block ids, not memory).
 *  - Cache layout (HND, "Understanding KV Cache" §3.2): k_cache and v_cache
 *    are each [num_blocks, num_kv_heads, block_size, head_dim], contiguous,
 *    in the element type `dtype`.
 *  - q and out: [num_seqs, num_heads, head_dim]; new k and v:
 *    [num_tokens, num_kv_heads, head_dim]; contiguous, element type `dtype`.
 *  - Query head h uses KV head h / (num_heads / num_kv_heads): consecutive
 *    query heads share a KV head (GQA diagram of "KV Cache and Inference
 *    Optimization", section "Three attention layouts").
 *  - Supported: dtype f32/f16/bf16, head_dim 64 or 128, block_size 16.
 *  - `stream` is a hipStream_t (NULL = the default stream). Device calls are
 *    asynchronous: a PKV_OK return means the work was enqueued; kernel faults
 *    surface at the next synchronising HIP call.
 *  - No call throws; each returns a pkv_status.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_EINVAL = 1,       /* null pointer, bad shape, Hq % Hkv != 0, bad dtype     */
  PKV_ERANGE = 2,       /* length beyond table capacity, id out of range          */
  PKV_ENOMEM = 3,       /* block pool exhausted                                    */
  PKV_EBUSY = 4,        /* write into a shared block, or two writes to one slot   */
  PKV_EUNSUPPORTED = 5, /* head_dim / block_size the kernels do not implement       */
  PKV_EHIP = 6,         /* the HIP runtime reported an error at launch             */
  PKV_ESMALL = 7        /* caller-provided workspace or output buffer too small    */
} pkv_status;

typedef enum pkv_dtype { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/*
 * Cache block layouts ("Understanding KV Cache" §3.2). One layer's K (and,
 * separately, V) cache of num_blocks blocks of block_size tokens:
 *   PKV_HND  [num_blocks, num_kv_heads, block_size, head_dim] (head-major:
 *            one head's tokens of a block are contiguous)
 *   PKV_NHD  [num_blocks, block_size, num_kv_heads, head_dim] (token-major)
 * FP8 scale tensors follow the same order without the head_dim axis.
 * Attention calls take block sizes that are multiples of 16 up to 2048
 * (the kernels walk 16-token tiles); the append takes any block size.
 */
typedef enum pkv_layout { PKV_HND = 0, PKV_NHD = 1 } pkv_layout;

/* Human-readable name of a status code (static string, never NULL). */
const char* pkv_status_string(pkv_status s);

/* Library ABI version (major * 100 + minor): 200. */
int32_t pkv_version(void);

/* ------------------------------------------------------------------------ */
/* Device calls                                                              */
/* ------------------------------------------------------------------------ */

/*
 * pkv_kv_append -- write each new token's K and V into its cache slot.
 *
 * The cache is an append-only log ("Understanding KV Cache" §1.3); token i's
 * slot s = slot_mapping[i] is offset s % block_size of physical block
 * s / block_size (§3.3). For every KV head j:
 *   k_cache[s / bs, j, s % bs, :] = k[i, j, :]   (HND; likewise v)
 *   k_cache[s / bs, s % bs, j, :] = k[i, j, :]   (NHD)
 * The copy is bit-exact. slot_mapping[i] < 0 marks a padding token: skipped.
 *
 *   k, v          device, [num_tokens, num_kv_heads, head_dim]
 *   slot_mapping  device int64 [num_tokens]
 *   k_cache, v_cache  device, written in place
 *   num_blocks    pool size (bounds every slot)
 *
 * Slots must be distinct and must not lie in a block shared by several
 * sequences (the host builder guarantees both). A slot >= num_blocks *
 * block_size is skipped on the device rather than written out of bounds.
 * Errors: EINVAL (null/shape/dtype), EUNSUPPORTED, EHIP. num_tokens == 0 is a
 * no-op returning PKV_OK.
 */
pkv_status pkv_kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                         void* k_cache, void* v_cache, int32_t num_blocks, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, pkv_layout layout, pkv_dtype dtype, void* stream);

/*
 * pkv_decode_partition_blocks -- cache blocks per context partition the
 * library picks for a launch of this shape (the split-context work unit).
 * Each partition covers this many blocks of one sequence and one KV head;
 * partial results are merged exactly with a log-sum-exp combine. Returns 0
 * for an unsupported block_size. A partition may span at most 2048 tokens
 * (partition_blocks * block_size <= 2048) in every call below, except the
 * prefill calls' workgroup kernel (see pkv_prefill_attention): 16384.
 */
int32_t pkv_decode_partition_blocks(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t max_blocks_per_seq, int32_t block_size);

/*
 * pkv_decode_workspace_bytes -- device scratch that pkv_paged_decode_attention
 * needs for this shape with `partition_blocks` (0 = the library's choice):
 * num_seqs * num_heads * P * (head_dim + 1) * 4 bytes rounded up, where
 * P = ceil(max_blocks_per_seq / partition_blocks). Returns 0 when every
 * sequence fits one partition (no merge needed).
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                  int32_t partition_blocks);

/*
 * pkv_paged_decode_attention -- one decode step of attention over the paged
 * cache, for all sequences and query heads.
 *
 *   q             device [num_seqs, num_heads, head_dim]
 *   k_cache, v_cache  device, in `layout` (see pkv_layout)
 *   block_tables  device int32 [num_seqs, max_blocks_per_seq]: entry [b][i]
 *                 is the physical block of logical block i of sequence b.
 *                 Each partition reads every entry of its slice of the row
 *                 (up to max_blocks_per_seq); entries past
 *                 ceil(context_lens[b] / block_size) may hold any value:
 *                 they are read and then ignored, and no K/V is fetched
 *                 through them
 *   context_lens  device int32 [num_seqs]: tokens attended, the newest one
 *                 included; 0 gives an all-zero output row
 *   scale         multiplies q . k (1/sqrt(head_dim) for standard attention)
 *   out           device [num_seqs, num_heads, head_dim], same dtype as q;
 *                 rounded from fp32 to the output type to nearest-even
 *   workspace     device scratch of >= pkv_decode_workspace_bytes(...) bytes
 *                 (may be NULL when that is 0); contents on entry ignored
 *   partition_blocks  blocks per partition (partition_blocks * block_size
 *                 <= 2048), 0 = the library's choice
 *
 * Accumulation is fp32. Preconditions the device does not check at full
 * cost: context_lens[b] <= max_blocks_per_seq * block_size and table entries
 * in [0, num_blocks); the kernel clamps lengths to the table capacity and
 * skips out-of-range block ids instead of reading outside the pool, so a bad
 * table gives a wrong result, never a fault (pkv_validate_tables checks them
 * on the host).
 * Errors: EINVAL (null/shape/dtype/Hq % Hkv, layout, partition size),
 * EUNSUPPORTED (head_dim not 64/128, block_size not a multiple of 16 up to
 * 2048, num_blocks * num_kv_heads * block_size >= 2^31), ESMALL (workspace),
 * EHIP. num_seqs == 0 is a no-op.
 */
pkv_status pkv_paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      pkv_layout layout, int32_t num_blocks, float scale, void* out,
                                      pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                      int32_t partition_blocks, void* stream);

/*
 * The two phases of pkv_paged_decode_attention, for callers that schedule or
 * time them separately (pkv_paged_decode_attention == partitions, then merge,
 * on one stream).
 *
 * pkv_decode_partitions -- same arguments and errors as
 * pkv_paged_decode_attention. Each (sequence, KV head, context partition)
 * work unit attends over its partition; a sequence that fits one partition
 * gets its final output row written to `out`, the others leave per-partition
 * results o_p (normalised, fp32) and lse_p (log2 of the partition's softmax
 * denominator plus its running maximum, in log2 units of scale * q.k) in the
 * workspace.
 *
 * pkv_decode_merge -- exact log-sum-exp combine of those partials:
 * out = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M), M = max_p lse_p, for
 * every sequence with more than one partition; rows of single-partition
 * sequences are left as written. Arguments must match the preceding
 * pkv_decode_partitions call. Errors: EINVAL, ESMALL, EHIP.
 */
pkv_status pkv_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                                 int32_t num_blocks, float scale, void* out, pkv_dtype dtype, void* workspace,
                                 size_t workspace_bytes, int32_t partition_blocks, void* stream);
pkv_status pkv_decode_merge(const void* workspace, size_t workspace_bytes, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_blocks, void* out,
                            pkv_dtype dtype, void* stream);

/*
 * pkv_decode_step -- one whole decode step for one layer in a single launch:
 * append the newest token of every sequence, then attend over the cache.
 * Equivalent to pkv_kv_append with slot_mapping[b] = the slot of position
 * context_lens[b] - 1 (block_tables[b][(n-1)/bs] * bs + (n-1) % bs, the rule
 * of "Understanding KV Cache" §3.3) followed by pkv_paged_decode_attention.
 * The kernel writes the new K/V into its slot and uses them from registers;
 * a sequence split into several partitions is merged by whichever of its
 * partitions finishes last (device-scope arrival counter), so no second
 * launch is needed.
 *
 *   k_new, v_new  device [num_seqs, num_heads_kv, head_dim]: token at
 *                 position context_lens[b] - 1 (sequences with length 0
 *                 append nothing)
 *   workspace     >= pkv_decode_step_workspace_bytes(...) bytes. It holds
 *                 partition results and arrival counters: it must be
 *                 zero-filled before its first use, and every completed call
 *                 leaves the counters at zero again. Calls that share one
 *                 workspace must not run concurrently.
 * Every other argument as pkv_paged_decode_attention. The newest token's
 * block must be private to its sequence (the host pool's slot builder checks
 * this; here it is a precondition). A sequence whose context_lens[b] exceeds
 * max_blocks_per_seq * block_size (a precondition violation) appends nothing:
 * its length is clamped for reading, as in pkv_paged_decode_attention, and
 * no cached token is overwritten.
 */
size_t pkv_decode_step_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t max_blocks_per_seq, int32_t block_size,
                                       int32_t partition_blocks);
pkv_status pkv_decode_step(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, pkv_layout layout, int32_t num_blocks, float scale, void* out,
                           pkv_dtype dtype, void* workspace, size_t workspace_bytes, int32_t partition_blocks,
                           void* stream);

/*
 * pkv_decode_step_noalloc -- pkv_decode_step without a caller workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. The partition
 * results and arrival counters live in a library-owned device array of
 * 64 MiB per GPU (held until the process ends; its first 64 KiB are the
 * counters). The call allocates and frees nothing.
 *   - Limits: at most 16384 work units (num_seqs * num_kv_heads *
 *     ceil((num_heads / num_kv_heads) / 16)) and
 *     pkv_decode_step_workspace_bytes(...) <= 64 MiB - 64 KiB for this shape
 *     and partition_blocks; larger shapes return PKV_ESMALL before any GPU
 *     work (pick longer partitions, or use pkv_decode_step).
 *   - Every call on one GPU shares that GPU's array: calls that overlap on
 *     one GPU (two streams, two threads) race and give wrong results. Each
 *     completed call leaves the counters at zero for the next; the first call
 *     on a device also enqueues a small fill kernel that clears them.
 * Every other argument, the result and the errors as pkv_decode_step.
 */
pkv_status pkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new, void* k_cache,
                                   void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                                   int32_t num_blocks, float scale, void* out, pkv_dtype dtype,
                                   int32_t partition_blocks, void* stream);

/*
 * FP8 KV cache. The pages name low-precision KV storage (INT8/FP8) with
 * higher-precision arithmetic ("KV Cache and Inference Optimization", section
 * "KV quantization") without fixing a format; these calls use:
 *   - codes: OCP 8-bit float E4M3 (1 sign, 4 exponent bits with bias 7, 3
 *     mantissa bits; no infinities; S.1111.111 is NaN; largest value 448),
 *     caches [num_blocks, num_kv_heads, block_size, head_dim] of uint8 (HND;
 *     [num_blocks, block_size, num_kv_heads, head_dim] for NHD);
 *   - scales: one fp32 per token row of one KV head, arrays
 *     [num_blocks, num_kv_heads, block_size] (NHD: [num_blocks, block_size,
 *     num_kv_heads]);
 *   - value attended over = code * scale;
 *   - quantization of a new row x (head_dim values, computed in fp32):
 *     amax = max |x|, scale = amax / 448, inv = 448 / amax (1 and 1 when
 *     amax == 0), code = E4M3 nearest to x * inv (ties to even, clamped to
 *     +-448, sign kept);
 *   - a row holding a NaN or an infinity gets scale NaN and every code 0x7F
 *     (E4M3 NaN), so each of its values reads back as NaN.
 * Queries and outputs stay bf16 or fp16 (dtype); codes are converted exactly
 * to that type in registers, scores and weights are scaled in fp32.
 *
 * pkv_kv_append_fp8 -- quantize each new token's K and V rows (k, v of type
 *   `dtype`: f32, f16 or bf16) and write codes and scales into slot
 *   slot_mapping[i]; slot < 0 skipped; otherwise as pkv_kv_append.
 * pkv_paged_decode_attention_fp8 -- as pkv_paged_decode_attention over FP8
 *   caches (dtype = q/out type: f16 or bf16; f32 is EUNSUPPORTED); the
 *   workspace is sized by pkv_decode_workspace_bytes.
 * pkv_decode_step_fp8 -- as pkv_decode_step over FP8 caches: the new rows
 *   are quantized in the kernel with the rule above (bit-identical to
 *   pkv_kv_append_fp8) and attended over as code * scale; workspace sized by
 *   pkv_decode_step_workspace_bytes, zero-filled before first use.
 */
pkv_status pkv_kv_append_fp8(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                             void* k_cache, void* v_cache, float* k_scales, float* v_scales, int32_t num_blocks,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                             pkv_dtype dtype, void* stream);
pkv_status pkv_paged_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                                          const float* k_scales, const float* v_scales,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                          pkv_layout layout, int32_t num_blocks, float scale, void* out,
                                          pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                          int32_t partition_blocks, void* stream);
pkv_status pkv_decode_step_fp8(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               float* k_scales, float* v_scales, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               pkv_layout layout, int32_t num_blocks, float scale, void* out, pkv_dtype dtype,
                               void* workspace, size_t workspace_bytes, int32_t partition_blocks, void* stream);

/*
 * INT8 KV cache: the same calls over signed 8-bit integer codes. The pages
 * name INT8 beside FP8 for KV storage ("KV Cache and Inference Optimization",
 * section "KV quantization"); the scaling rule is the FP8 one with 127 as the
 * largest code:
 *   - codes: int8 in the cache layout, scales fp32 as for FP8;
 *   - value attended over = code * scale;
 *   - quantization of a new row x (fp32): amax = max |x|, scale = amax / 127,
 *     inv = 127 / amax (1 and 1 when amax == 0), code = x * inv rounded to the
 *     nearest integer (ties to even), clamped to +-127 (-128 is never produced
 *     for a finite row);
 *   - a row holding a NaN or an infinity gets scale NaN and every code -128
 *     (0x80), so each of its values reads back as NaN.
 * Queries and outputs are bf16 or fp16 (f32 is EUNSUPPORTED); codes convert
 * exactly to those types. Arguments, layouts and errors as the _fp8 calls.
 */
pkv_status pkv_kv_append_int8(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                              void* k_cache, void* v_cache, float* k_scales, float* v_scales, int32_t num_blocks,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                              pkv_dtype dtype, void* stream);
pkv_status pkv_paged_decode_attention_int8(const void* q, const void* k_cache, const void* v_cache,
                                           const float* k_scales, const float* v_scales,
                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                           pkv_layout layout, int32_t num_blocks, float scale, void* out,
                                           pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                           int32_t partition_blocks, void* stream);
pkv_status pkv_decode_step_int8(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                float* k_scales, float* v_scales, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                pkv_layout layout, int32_t num_blocks, float scale, void* out, pkv_dtype dtype,
                                void* workspace, size_t workspace_bytes, int32_t partition_blocks, void* stream);
pkv_status pkv_prefill_attention_int8(const void* q, const void* k_cache, const void* v_cache, const float* k_scales,
                                      const float* v_scales, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* q_start, int32_t max_q_len, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, pkv_layout layout, int32_t num_blocks, float scale,
                                      void* out, pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                      int32_t partition_blocks, void* stream);

/*
 * pkv_prefill_attention -- chunked prefill: causal attention of a chunk of
 * new query tokens per sequence over the paged cache. Prefill processes many
 * query positions at once as matrix products ("KV Cache and Inference
 * Optimization", the prefill / decode comparison; "Understanding KV Cache"
 * §2.1); split into chunks, each chunk's K/V is appended first
 * (pkv_kv_append) and the chunk then attends to everything cached before it
 * plus itself, causally (§1.2: position i sees positions <= i).
 *
 *   q             device [total_q, num_heads, head_dim]: the chunks of all
 *                 sequences, packed; sequence b owns rows q_start[b] ..
 *                 q_start[b+1]-1 (q_len_b = q_start[b+1] - q_start[b])
 *   q_start       device int32 [num_seqs + 1], non-decreasing
 *   max_q_len     host bound on every q_len_b (sizes the launch); longer
 *                 chunks are truncated to it
 *   context_lens  device int32 [num_seqs]: the sequence's cached tokens, the
 *                 chunk's own included; chunk token i is at position
 *                 context_lens[b] - q_len_b + i and attends to positions
 *                 0 .. context_lens[b] - q_len_b + i (q_len_b is clamped to
 *                 context_lens[b])
 *   out           device [total_q, num_heads, head_dim], dtype of q; rows
 *                 beyond a truncated chunk are not written
 *   workspace     >= pkv_prefill_workspace_bytes(...) bytes, zero-filled before
 *                 its first use; each completed call leaves its counters at
 *                 zero (calls sharing a workspace must not overlap)
 *   partition_blocks  blocks per partition: partition_blocks * block_size
 *                 <= 16384 for the workgroup kernel, <= 2048 for the
 *                 one-wave kernel (see below); 0 = the library's choice,
 *                 16384 or 1024 tokens, halved while the launch would have
 *                 fewer than 512 work units
 * Every other argument as pkv_paged_decode_attention. Work unit: a group of
 * (query token, query head) rows of one KV head and one context partition --
 * 128 rows in a four-wave workgroup that shares each K/V tile through LDS for
 * 16-bit caches (8-bit caches: head size 128) and scale > 0, 64 (16-bit
 * queries) or 32 (fp32) rows in one wave otherwise; split contexts are merged
 * in the kernel by the partition that finishes last. The workspace size
 * covers every variant. A workgroup reads the table entries of its partition
 * up to the last key its rows see.
 * Errors as pkv_paged_decode_attention.
 */
size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_q_len, int32_t max_blocks_per_seq, int32_t block_size,
                                   int32_t partition_blocks);
pkv_status pkv_prefill_attention(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* q_start,
                                 int32_t max_q_len, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size, pkv_layout layout,
                                 int32_t num_blocks, float scale, void* out, pkv_dtype dtype, void* workspace,
                                 size_t workspace_bytes, int32_t partition_blocks, void* stream);
/* As pkv_prefill_attention over FP8 caches (codes + per-row scales, see the
 * FP8 section above; dtype = q/out type, f16 or bf16). */
pkv_status pkv_prefill_attention_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scales,
                                     const float* v_scales, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* q_start, int32_t max_q_len, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t block_size, pkv_layout layout, int32_t num_blocks, float scale,
                                     void* out, pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                                     int32_t partition_blocks, void* stream);

/*
 * pkv_copy_blocks -- copy-on-write of whole physical blocks ("KV Cache and
 * Inference Optimization", section "PagedAttention": shared blocks are copied
 * when a sequence diverges). For each pair k (pairs[2k] = source id,
 * pairs[2k+1] = destination id; DEVICE int32 array) and each of the n_caches
 * tensors c, copies block_bytes[c] bytes from caches[c] + src * block_bytes[c]
 * to caches[c] + dst * block_bytes[c]. `caches` and `block_bytes` are HOST
 * arrays of n_caches (1..4) entries: e.g. K and V caches with
 * Hkv * block_size * head_dim * elt bytes per block, plus for FP8 caches the
 * two scale tensors with Hkv * block_size * 4 bytes per block. Pairs with an
 * id outside [0, num_blocks) or src == dst are skipped. Precondition (what
 * pkv_seq_append_slots produces): no destination appears twice or is also a
 * source; otherwise the result depends on scheduling. Asynchronous on
 * `stream`; run it before the append that writes the destinations.
 * Errors: EINVAL (n_caches outside 1..4, a block_bytes not a positive
 * multiple of 16, a null or unaligned pointer, n_pairs < 0), EHIP.
 */
pkv_status pkv_copy_blocks(void* const* caches, const int64_t* block_bytes, int32_t n_caches, int32_t num_blocks,
                           const int32_t* pairs, int32_t n_pairs, void* stream);

/*
 * pkv_stream_tiles -- a measurement call, not part of attention: the read
 * ceiling of the decode access pattern. It launches one wave per (sequence,
 * KV head, context partition) over the decode call's partitions, in the
 * workgroups and XCD order of the split decode launch (consecutive KV heads of
 * one partition per workgroup), looks up
 * each tile through block_tables and loads the K and V tiles (plus the row
 * scales when given) with the same bounded nontemporal loads, and computes
 * nothing but an XOR of the loaded words, written to sink. The time it takes
 * is what the memory system gives for exactly the bytes decode attention must
 * read (decode is bound by those reads: "Understanding KV Cache" §2.2).
 *
 *   k_cache, v_cache  device caches in `layout`, rows of row_bytes bytes per
 *                 head (head_dim * element size: 64, 128, 256 or 512)
 *   k_scales, v_scales  device fp32 row scales of 8-bit caches, or both NULL
 *   block_tables, context_lens, max_blocks_per_seq, num_blocks, block_size
 *                 as pkv_paged_decode_attention
 *   partition_blocks  blocks per partition (> 0; pass the decode call's
 *                 pkv_decode_partition_blocks to mirror it)
 *   sink          device uint32, >= num_seqs * num_kv_heads * P * 64 words,
 *                 P = ceil(max_blocks_per_seq / partition_blocks); overwritten
 * Errors: EINVAL (null pointers, one scale pointer without the other, sizes,
 * partition_blocks), EUNSUPPORTED (row_bytes, block_size), ESMALL (sink), EHIP.
 */
pkv_status pkv_stream_tiles(const void* k_cache, const void* v_cache, const float* k_scales, const float* v_scales,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_kv_heads, int32_t row_bytes, int32_t block_size,
                            pkv_layout layout, int32_t num_blocks, int32_t partition_blocks, uint32_t* sink,
                            size_t sink_words, void* stream);

/* ------------------------------------------------------------------------ */
/* Host block pool, block tables and slot mapping                            */
/* ------------------------------------------------------------------------ */
/*
 * A pool of num_blocks equal physical blocks and per-sequence block lists
 * (block lifecycle of "Understanding KV Cache" §3.5: allocate from the free
 * pool, use through the block table, return on finish). Host memory only; not
 * thread-safe (one owner, like a scheduler). Sequence ids are dense integers
 * in [0, max_seqs).
 */
typedef struct pkv_pool pkv_pool;

typedef struct pkv_pool_stats {
  int64_t num_blocks;       /* pool size                                          */
  int64_t free_blocks;      /* blocks no sequence holds (incl. evictable cached)  */
  int64_t used_blocks;      /* distinct blocks held by at least one sequence      */
  int64_t shared_blocks;    /* blocks held by more than one sequence              */
  int64_t live_seqs;        /* sequences with at least one token                  */
  int64_t payload_tokens;   /* sum of sequence lengths (logical tokens)           */
  int64_t capacity_tokens;  /* sum over sequences of blocks x block_size          */
} pkv_pool_stats;

/* Create a pool. seed != 0 shuffles the free list with a seeded Fisher-Yates
 * permutation (xorshift64* generator); seed == 0 keeps ids in ascending order.
 * Errors: EINVAL (sizes <= 0, null out). */
pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, int32_t max_seqs, uint64_t seed,
                           pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);

/* Grow sequence `seq` to new_len tokens, taking ceil(new_len / block_size)
 * minus its current block count from the free list. Shrinking is ERANGE.
 * ENOMEM if the pool runs dry; EBUSY if the new positions would start inside
 * a partial last block that another sequence or the prefix cache also holds
 * (use pkv_seq_append_slots, which copies such a block first). On any error
 * the sequence is left unchanged. */
pkv_status pkv_seq_grow(pkv_pool* pool, int32_t seq, int32_t new_len);

/* Make empty sequence `dst` share the first floor(n_tokens / block_size) FULL
 * blocks of `src` (reference counts + 1); dst's length becomes that many
 * blocks' worth of tokens. Only full blocks are shared, matching block-
 * granular prefix reuse ("KV Cache and Inference Optimization", sections
 * "PagedAttention" and "APC"). EINVAL if dst is not empty, ERANGE if n_tokens
 * exceeds src's length. */
pkv_status pkv_seq_share_prefix(pkv_pool* pool, int32_t dst, int32_t src, int32_t n_tokens);

/* Make empty sequence `dst` share ALL blocks of `src`, the partial last block
 * included (reference counts + 1), and take src's length: parallel samples or
 * beams that store their common prefix once and copy only where they branch
 * ("KV Cache and Inference Optimization", the beam-search / multi-sample item
 * of its list of pitfalls, and "PagedAttention": shared blocks, copied on
 * divergence). The first append of either sequence into the shared
 * partial block goes through pkv_seq_append_slots, which copies it.
 * EINVAL if dst is not empty or dst == src. */
pkv_status pkv_seq_fork(pkv_pool* pool, int32_t dst, int32_t src);

/* Release all blocks of `seq` (a block nobody holds any more returns to the
 * free list, or, if it is in the prefix cache, becomes evictable).
 * EINVAL if `seq` holds nothing (double free). */
pkv_status pkv_seq_free(pkv_pool* pool, int32_t seq);

/* One decode step's append for sequences seqs[0..n) (distinct): each grows by
 * one token at position = its current length, and slots[i] receives that
 * token's slot. A position at a block boundary takes a fresh block; a
 * position inside a block that other sequences also hold makes the block
 * private first (copy-on-write, "KV Cache and Inference Optimization",
 * "PagedAttention"): a fresh block replaces it in this sequence and the pair
 * (shared id, fresh id) is written to copy_pairs[2k], copy_pairs[2k+1];
 * *n_copies receives k. copy_pairs must hold 2n ints. The caller copies those
 * blocks on the device (pkv_copy_blocks) before the append writes the slots.
 * Errors (nothing is changed): EINVAL (bad or repeated sequence, null
 * pointers), ENOMEM (fewer free blocks than needed), EBUSY (the target block
 * is in the prefix cache: cannot happen through this API, since only full
 * blocks are cached). */
pkv_status pkv_seq_append_slots(pkv_pool* pool, const int32_t* seqs, int32_t n, int64_t* slots,
                                int32_t* copy_pairs, int32_t* n_copies);

/* ---- Prefix cache ("KV Cache and Inference Optimization", section "APC") ----
 * Full blocks are cached under a key chained over the token prefix that ends
 * with them (block i's key covers tokens [0, 16(i+1))) and the caller's
 * namespace `ns` (e.g. a model / adapter identity: reused state must match the
 * model and the exact token sequence and positions, "Why does a request use
 * more memory the longer it generates?", section "Paging changes allocation,
 * not a token's representation"). A lookup walks a request's full blocks from the first one
 * and stops at the first miss; a hit is accepted only after comparing the
 * block's tokens and its predecessor exactly, so a hash collision can only
 * cause a miss. Partial blocks are never cached. */
typedef struct pkv_prefix_stats {
  int64_t cached_blocks;     /* blocks in the prefix cache                          */
  int64_t evictable_blocks;  /* cached blocks no sequence holds                      */
  int64_t lookups;           /* pkv_seq_adopt_prefix calls                           */
  int64_t lookup_blocks;     /* full blocks those requests had                       */
  int64_t hit_blocks;        /* of which reused from the cache                       */
  int64_t evictions;         /* cached blocks reclaimed for new data                 */
  int64_t cow_copies;        /* blocks copied by pkv_seq_append_slots                */
} pkv_prefix_stats;

/* Cache the full blocks of `seq` covering tokens[0..n_tokens) (the caller has
 * written their K/V). Registration stops early where the same content is
 * already cached in another block. *n_cached (may be NULL) receives how many
 * leading blocks of `seq` are now in the cache. Errors: EINVAL (bad sequence,
 * or a block of `seq` already cached with other tokens), ERANGE (n_tokens
 * beyond the sequence's length), ENOMEM. */
pkv_status pkv_prefix_register(pkv_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                               uint64_t ns, int32_t* n_cached);

/* Leading cached blocks for tokens[0..n_tokens): *n_hit receives their count
 * and block_ids (may be NULL) the first min(count, capacity) ids. Changes
 * nothing. */
pkv_status pkv_prefix_match(const pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, uint64_t ns,
                            int32_t* block_ids, int32_t capacity, int32_t* n_hit);

/* Start empty sequence `seq` from the cache: it holds the leading hit blocks
 * of tokens[0..n_tokens) (reference counts + 1) and its length becomes
 * 16 x hits tokens, returned in *hit_tokens (may be NULL); the caller computes
 * K/V only for the rest. EINVAL if `seq` is not empty. */
pkv_status pkv_seq_adopt_prefix(pkv_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens, uint64_t ns,
                                int32_t* hit_tokens);

pkv_status pkv_pool_get_prefix_stats(const pkv_pool* pool, pkv_prefix_stats* out);

/* Current length and block list of one sequence. `blocks` may be NULL to
 * query only the count; otherwise capacity must hold the count (ESMALL). */
pkv_status pkv_seq_info(const pkv_pool* pool, int32_t seq, int32_t* length, int32_t* num_blocks,
                        int32_t* blocks, int32_t capacity);

/* Dense block table [n, max_blocks] (row-major int32) for sequences seqs[0..n),
 * padded with `pad`. ERANGE if a sequence has more than max_blocks blocks. */
pkv_status pkv_build_block_tables(const pkv_pool* pool, const int32_t* seqs, int32_t n,
                                  int32_t max_blocks, int32_t pad, int32_t* out);

/* Slot of token positions[i] of sequence seqs[i]: physical block x block_size
 * + offset ("Understanding KV Cache" §3.3). positions[i] < 0 gives -1 (a
 * padding token). ERANGE if a position is at or beyond the sequence's length;
 * EBUSY if the slot's block is shared (its writer would change another
 * sequence) or if two entries name the same slot. */
pkv_status pkv_build_slot_mapping(const pkv_pool* pool, const int32_t* seqs, const int32_t* positions,
                                  int32_t n, int64_t* out);

/* Stateless variant for callers that keep their own tables: slot of token
 * positions[i] of row i of a dense int32 table [n, max_blocks] (row-major).
 * positions[i] < 0 gives -1. ERANGE if positions[i] / block_size >=
 * max_blocks or the table entry is negative; EBUSY if two entries name the
 * same slot. */
pkv_status pkv_slot_mapping_from_tables(const int32_t* block_tables, int32_t max_blocks, const int32_t* positions,
                                        int32_t n, int32_t block_size, int64_t* out);

/* Accounting snapshot (payload vs capacity, as in the block-accounting
 * example of "Why does a request use more memory the longer it generates?",
 * section "Paging changes allocation, not a token's representation"). */
pkv_status pkv_pool_get_stats(const pkv_pool* pool, pkv_pool_stats* out);

/* ceil(n / block_size) and the empty slots left in the last block. */
int64_t pkv_blocks_for(int64_t n, int32_t block_size);
int64_t pkv_empty_slots(int64_t n, int32_t block_size);

/* Host-side check of decode inputs: every context length within the table
 * capacity and every table entry a sequence actually reads in [0, num_blocks).
 * ERANGE on the first violation, with its sequence index in *bad_seq (may be
 * NULL). Inputs are HOST arrays. */
pkv_status pkv_validate_tables(const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                               int32_t num_blocks, int32_t* bad_seq);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
