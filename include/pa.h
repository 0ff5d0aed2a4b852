/*
 * pa.h - C ABI of the gfx950 paged decode-attention library (libpa.so).
 *
 * Two operations, both from the paged KV-cache design, plus the two fused
 * into one decode step (pa_decode_append, below):
 *
 *   pa_kv_append  writes each new token's K and V into the pool slot the
 *                 block manager reserved for it.  The block manager takes a
 *                 fresh block only when the sequence's last block is full and
 *                 then writes the token into that last block ("49 vLLM /
 *                 PagedAttention", listing "Таблица блоков (идея пейджинга)";
 *                 "PagedAttention：KV cache 即虚拟内存（block manager & 碎片）",
 *                 section "深入原理", lifecycle bullet).
 *
 *   pa_decode     single-token decode attention over K/V that live in
 *                 fixed 16-token blocks scattered through a shared pool, each
 *                 sequence's block table mapping logical block t/16 to a
 *                 physical block ("49 vLLM / PagedAttention", section "Идея и
 *                 механизм"; "PagedAttention：KV cache 即虚拟内存", section
 *                 "直接答案").  The result equals dense attention over the
 *                 contiguous context (same page, sections "直接答案" and
 *                 "面试官追问"):
 *                     out[b,h,:] = sum_t softmax_t(scale * <q[b,h,:], K_t>) V_t
 *                 over t < seq_lens[b], with query head h reading KV head
 *                 h / (num_q_heads / num_kv_heads).
 *
 * Storage layouts (row-major, element counts):
 *   q, out        [num_seqs][num_q_heads][head_size]
 *   k_pool        [num_blocks][num_kv_heads][16][head_size]   (token rows)
 *   v_pool        [num_blocks][num_kv_heads][head_size][16]   (tokens inner)
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens      int32 [num_seqs]
 *   k_new, v_new  [num_tokens][num_kv_heads][head_size]
 *   slot_mapping  int32 [num_tokens]; slot = physical_block * 16 + offset
 * The byte count of one block is 2 * 16 * num_kv_heads * head_size * the
 * element size ("vLLM innenfra", KV-cache-manager paragraph); the order of
 * the axes inside a block is this library's choice: each (block, KV head)
 * K tile and V tile is one contiguous 16*head_size run, and V is stored with
 * the 16 tokens innermost so that the matrix-core contraction over tokens
 * reads contiguous bytes.
 *
 * Ownership: every array argument is device memory owned by the caller; the
 * library keeps no pointer after a call returns and allocates nothing.
 * Calls are asynchronous on `stream` and never synchronise the host.
 * `stream` is a hipStream_t passed as void* (NULL = the default stream), so
 * that this header needs no HIP header and plain C programs can include it.
 *
 * Errors: functions return PA_OK (0) or a negative pa_status from host-side
 * checks (null pointers, unsupported shapes or dtypes, misaligned pointers,
 * workspace too small) or from the launch itself.  Nothing is launched when a
 * check fails.  Data-dependent contract violations are not reported but are
 * contained: a slot outside [0, num_blocks*16) is skipped, a block-table
 * entry outside [0, num_blocks) contributes nothing, a sequence length is
 * clamped to [0, max_blocks_per_seq*16]; no access ever leaves the buffers.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_F32 = 0,         /* IEEE binary32 */
  PA_BF16 = 1,        /* bfloat16 */
  PA_FP8_E4M3FN = 2   /* OCP fp8 e4m3fn (bias 7, max 448, no inf) */
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,         /* a required pointer is NULL */
  PA_ERR_DTYPE = -2,        /* unsupported dtype combination */
  PA_ERR_SHAPE = -3,        /* unsupported or inconsistent size */
  PA_ERR_ALIGN = -4,        /* a pointer is not 16-byte aligned */
  PA_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required */
  PA_ERR_LAUNCH = -6,       /* the HIP runtime rejected a launch */
  PA_ERR_DEVICE = -7,       /* no usable HIP device */
  PA_ERR_SCRATCH = -8       /* pa_decode_append_noalloc: the call needs more
                               than the static scratch buffer holds */
} pa_status;

/*
 * Shapes and options of one decode call.
 *   num_seqs            B >= 0 (at most 65536)
 *   num_q_heads         Hq, a multiple of num_kv_heads
 *   num_kv_heads        Hkv >= 1
 *   head_size           D in {64, 128, 256}
 *   block_size          must be 16
 *   num_blocks          NB >= 1, NB*16 <= INT32_MAX
 *   max_blocks_per_seq  row length of block_tables (>= 1)
 *   max_seq_len         upper bound of seq_lens (scheduling hint; >= 0)
 *   q_dtype / kv_dtype  (F32, F32) or (BF16, BF16) or (BF16, FP8_E4M3FN);
 *                       out has q_dtype.  G = Hq/Hkv must be <= 8 for F32 and
 *                       <= 16 otherwise.
 *   k_scale / v_scale   per-tensor dequantisation scales of an FP8 pool
 *                       (stored value * scale = real value); ignored (use 1)
 *                       for F32/BF16 pools.
 *   total_blocks_hint   sum over b of ceil(seq_lens[b]/16) if the caller
 *                       knows it, else 0; only sizes the work split (fewer
 *                       ranges for small batches), never changes a result.
 *   num_waves           0 = automatic (the recommended setting: one
 *                       workgroup per range, four per compute unit, in one
 *                       round); else the number of 64-lane workgroups of the
 *                       main kernel (rounded down to a multiple of
 *                       num_kv_heads).  This replaces a per-sequence
 *                       partition size: the main kernel cuts the flattened
 *                       work of all sequences into num_waves equal ranges,
 *                       so no partition length is chosen per sequence.
 *   reserved            set to 0 (keeps profile_events 8-byte aligned).
 *   profile_events      a measurement hook, not needed for computing:
 *                       NULL, or two hipEvent_t that the main kernel's
 *                       dispatch records at its own start and end (for
 *                       pa_decode_append_shared with groups: recorded on
 *                       `stream` before its first and after its last
 *                       launch), so that a benchmark can time the dominant
 *                       kernel on the stream it runs on.  Timed dispatches
 *                       are serialised; leave both NULL in production
 *                       calls.
 */
typedef struct {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_size;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_seq_len;
  pa_dtype q_dtype;
  pa_dtype kv_dtype;
  float k_scale;
  float v_scale;
  int64_t total_blocks_hint;
  int32_t num_waves;
  int32_t reserved;
  void* profile_events[2];
} pa_decode_desc;

/*
 * Bytes of device workspace pa_decode needs for `desc` on the current
 * device (0 on an invalid descriptor).  The workspace holds the per-sequence
 * block prefix sums and the split-context partial results; its contents
 * need no initialisation and are scratch between calls.
 */
size_t pa_decode_workspace_size(const pa_decode_desc* desc);

/*
 * Decode attention (see the top of this file).
 *   q             [B][Hq][D] of q_dtype, 16-byte aligned
 *   k_pool        [NB][Hkv][16][D] of kv_dtype, 16-byte aligned
 *   v_pool        [NB][Hkv][D][16] of kv_dtype, 16-byte aligned
 *   block_tables  int32 [B][max_blocks_per_seq]; entries past
 *                 ceil(seq_lens[b]/16) are never read (pad freely, e.g. -1)
 *   seq_lens      int32 [B]: tokens attended, including any token appended
 *                 for this step; 0 gives an all-zero output row
 *   scale         multiplier of q.K (usually 1/sqrt(D))
 *   out           [B][Hq][D] of q_dtype, 16-byte aligned, written entirely
 *   workspace     device buffer of at least pa_decode_workspace_size(desc)
 *                 bytes, 256-byte aligned; may be NULL when that size is 0
 * Two kernels run on `stream`: the main pass (which writes the rows of
 * sequences handled by a single workgroup) and a merge pass for sequences
 * whose context was split across workgroups.  Calls that share a workspace
 * must be ordered on one stream.
 */
int pa_decode(const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, const int32_t* seq_lens,
              float scale, void* out, const pa_decode_desc* desc,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace pa_decode_append needs for `desc` on the current
 * device (0 on an invalid descriptor): that of pa_decode plus one fp32
 * partial of head_size + 2 values per (sequence, query head).
 */
size_t pa_decode_append_workspace_size(const pa_decode_desc* desc);

/*
 * One decode step in two launches: the append of each sequence's newest
 * token followed by decode attention that includes it.  The result equals
 *     pa_kv_append(k_new, v_new, slot_mapping, k_pool, v_pool)  with N = B
 *     pa_decode(q, k_pool, v_pool, block_tables, seq_lens, scale, out)
 * (the append step of the block manager: take a block only when the last
 * one is full, then write the token into the last block - "49 vLLM /
 * PagedAttention", listing "Таблица блоков"; the attention over the grown
 * context equals dense attention - "PagedAttention：KV cache 即虚拟内存",
 * section "直接答案"), up to floating-point rounding order, provided that
 * slot_mapping[b] is the slot of token seq_lens[b] - 1 of sequence b in
 * block_tables, in a block no other sequence of the batch reads (the block
 * manager's allocate-on-growth slot for an unshared last block; writing
 * into a shared block would need copy-on-write).  A negative slot skips
 * only the write: the token is still attended from k_new / v_new.
 *
 *   q, block_tables, seq_lens, scale, out, desc: as for pa_decode;
 *     seq_lens[b] counts the new token.
 *   k_pool, v_pool  written: token b's K row and V column go to
 *                   slot_mapping[b] (a byte copy; negative or out-of-pool
 *                   slots are skipped, as in pa_kv_append).
 *   k_new, v_new    [B][Hkv][D] of kv_dtype, 16-byte aligned: sequence b's
 *                   newest token (attended from here, not from the pool).
 *   slot_mapping    int32 [B].
 *   workspace       at least pa_decode_append_workspace_size(desc) bytes,
 *                   256-byte aligned.
 * The main pass attends the first seq_lens[b] - 1 tokens from the pool; the
 * merge pass writes the new token's K/V, scores it and folds it into the
 * main pass's partials as one more term of the online softmax.  With
 * seq_lens[b] <= 0 the row is zero (the slot is still written).
 * Errors as for pa_decode, plus PA_ERR_NULL for missing k_new / v_new /
 * slot_mapping and PA_ERR_ALIGN for misaligned ones.
 */
int pa_decode_append(const void* q, void* k_pool, void* v_pool,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     float scale, void* out, const void* k_new,
                     const void* v_new, const int32_t* slot_mapping,
                     const pa_decode_desc* desc, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * pa_decode_append for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, arguments and results, without a workspace
 * argument.  Its scratch (the contents pa_decode_append keeps in its
 * workspace) is a static buffer of 32 MiB in the library's device code,
 * one per device, held from the library's first use on that device until
 * the process ends.  The call itself allocates nothing.
 *   Size limit: the call fits when pa_decode_append_workspace_size(desc)
 *   is at most 32 MiB (33554432 bytes); otherwise it returns
 *   PA_ERR_SCRATCH and launches nothing.  (About 5 MiB for 64 sequences
 *   with 32 query heads of size 128, 17 MiB for 256 sequences with 64.)
 *   Concurrency: every call on one device shares that device's buffer and
 *   its contents are scratch between calls: calls that overlap on one
 *   device (unordered streams, or several host threads with different
 *   streams) race and give undefined results.  Calls ordered on one
 *   stream are safe.
 * Errors: as for pa_decode_append (without PA_ERR_WORKSPACE), plus
 * PA_ERR_SCRATCH, and PA_ERR_DEVICE when the buffer's device address
 * cannot be resolved.
 */
int pa_decode_append_noalloc(const void* q, void* k_pool, void* v_pool,
                             const int32_t* block_tables,
                             const int32_t* seq_lens, float scale, void* out,
                             const void* k_new, const void* v_new,
                             const int32_t* slot_mapping,
                             const pa_decode_desc* desc, void* stream);

/*
 * Bytes of workspace that pa_decode_append_shared needs (0 on an invalid
 * descriptor): that of pa_decode_append plus a suffix block table
 * (num_seqs x max_blocks_per_seq int32), num_seqs suffix lengths, and one
 * fp32 partial of head_size + 2 values per (sequence, query head).
 */
size_t pa_decode_append_shared_workspace_size(const pa_decode_desc* desc);

/*
 * Cascade form of pa_decode_append for batches whose sequences share a
 * prompt prefix.  Sequences that share full prefix blocks hold the same
 * physical blocks at the head of their tables ("PagedAttention：KV cache
 * 即虚拟内存（block manager & 碎片）", section "深入原理", sharing bullet),
 * and paged attention over such a table equals dense attention over the
 * contiguous context (same page, section "直接答案"), so the softmax splits
 * exactly into the shared part and each sequence's own part.  This call
 * reads each shared prefix once per group: a matrix-core pass attends every
 * member's query to its group's prefix blocks (one fp32 partial per
 * sequence and query head), the ordinary main pass attends each sequence's
 * remaining blocks, and the merge pass folds both with the appended token.
 *   group_start          int32 [num_groups + 1], device, non-decreasing:
 *                        group j is sequences group_start[j] ..
 *                        group_start[j+1] - 1; sequences outside every
 *                        group have no shared part.
 *   group_prefix_blocks  int32 [num_groups], device: P_j, the number of
 *                        leading table entries that every member of group
 *                        j shares (read through the first member's row).
 *   num_groups           0 .. num_seqs; 0 is pa_decode_append (the group
 *                        arrays may then be NULL).
 *   workspace            at least
 *                        pa_decode_append_shared_workspace_size(desc)
 *                        bytes, 256-byte aligned.
 * Other arguments as for pa_decode_append; only bf16 q with bf16 or fp8
 * e4m3fn pools, head_size 64 or 128, and scale > 0 are supported.  total_blocks_hint, if
 * given, should count the suffix blocks.  The caller guarantees that the
 * members' first P_j entries are equal; if they are not, the prefix of the
 * first member is used for all (memory-safe, numerically the first
 * member's prefix).  The shared part ends where the first member's tokens
 * before its newest end, if that is earlier than 16 P_j; a member shorter
 * than the shared part attends only its own tokens before its newest.
 * Errors: as pa_decode_append; PA_ERR_DTYPE for other dtypes; PA_ERR_SHAPE
 * for head_size, num_groups or scale out of range; PA_ERR_NULL /
 * PA_ERR_ALIGN for missing or misaligned group arrays.
 */
int pa_decode_append_shared(const void* q, void* k_pool, void* v_pool,
                            const int32_t* block_tables,
                            const int32_t* seq_lens, float scale, void* out,
                            const void* k_new, const void* v_new,
                            const int32_t* slot_mapping,
                            const int32_t* group_start,
                            const int32_t* group_prefix_blocks,
                            int32_t num_groups, const pa_decode_desc* desc,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Shapes of one append call.
 *   num_tokens    N >= 0
 *   num_kv_heads  Hkv >= 1
 *   head_size     D in {64, 128, 256}
 *   block_size    must be 16
 *   num_blocks    NB >= 1, NB*16 <= INT32_MAX
 *   kv_dtype      element type of the pools and of k_new / v_new
 */
typedef struct {
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t head_size;
  int32_t block_size;
  int32_t num_blocks;
  pa_dtype kv_dtype;
} pa_append_desc;

/*
 * KV append: for every i < N with s = slot_mapping[i] in [0, NB*16):
 *   k_pool[s/16][g][s%16][d] = k_new[i][g][d]
 *   v_pool[s/16][g][d][s%16] = v_new[i][g][d]     for all g < Hkv, d < D.
 * A pure byte copy (bit-exact for every dtype).  Negative slots are
 * skipped.  Slots must be distinct; with duplicates one of the writes wins.
 * k_new, v_new, k_pool and v_pool must be 16-byte aligned.
 */
int pa_kv_append(const void* k_new, const void* v_new,
                 const int32_t* slot_mapping, void* k_pool, void* v_pool,
                 const pa_append_desc* desc, void* stream);

/*
 * Quantising append into an fp8 pool: like pa_kv_append, but k_new / v_new
 * are bfloat16 [N][Hkv][D] and each value is stored as the e4m3fn code of
 * value / scale, with k_scale for K and v_scale for V (the pool's
 * per-tensor scales: stored value * scale = real value).  FP8 storage
 * halves a block's bytes ("PagedAttention：KV cache 即虚拟内存", section
 * "面试官追问").  The code is the nearest e4m3fn value of the IEEE float32
 * quotient, ties to the even code, magnitudes above 448 saturated to 448,
 * NaN stored as 0x7F, the sign of zero kept.
 *   desc->kv_dtype must be PA_FP8_E4M3FN (the pool's type); scales must be
 *   finite and > 0 (else PA_ERR_SHAPE).  Pointers, slots and errors as for
 *   pa_kv_append.
 */
int pa_kv_append_quant(const void* k_new, const void* v_new,
                       const int32_t* slot_mapping, void* k_pool,
                       void* v_pool, const pa_append_desc* desc,
                       float k_scale, float v_scale, void* stream);

/*
 * Shapes of one block copy.
 *   num_pairs     P >= 0
 *   num_kv_heads, head_size, block_size (16), num_blocks, kv_dtype: the
 *                 pools' shape and element type, as for pa_kv_append
 */
typedef struct {
  int32_t num_pairs;
  int32_t num_kv_heads;
  int32_t head_size;
  int32_t block_size;
  int32_t num_blocks;
  pa_dtype kv_dtype;
} pa_copy_desc;

/*
 * Copy-on-write of shared blocks: for every i < P, K block src_blocks[i]
 * and V block src_blocks[i] (all KV heads, all 16 slots) are copied byte
 * for byte to block dst_blocks[i] of the same pools.  The block manager
 * issues these when a sequence appends into a block another sequence still
 * references: sharing is copy-on-write, and a diverging sequence gets its
 * own copy of the block first ("49 vLLM / PagedAttention", section "Почему
 * это важно"; "PagedAttention：KV cache 即虚拟内存", section "深入原理",
 * sharing bullet).
 *   k_pool, v_pool          16-byte aligned pools (layouts as above).
 *   src_blocks, dst_blocks  int32 [P], device memory.  Destinations must be
 *                           distinct and must not appear as sources of the
 *                           same call (else the result is unspecified);
 *                           pairs with an id outside [0, num_blocks) are
 *                           skipped.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_DTYPE, PA_ERR_ALIGN,
 * PA_ERR_LAUNCH, as for pa_kv_append.
 */
int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_blocks,
                   const int32_t* dst_blocks, const pa_copy_desc* desc,
                   void* stream);

/*
 * Shapes of one chunked-prefill call.
 *   num_seqs            B >= 0 (at most 65536)
 *   num_q_heads         Hq, a multiple of num_kv_heads, Hq/Hkv <= 16
 *   num_kv_heads        Hkv >= 1
 *   head_size           D in {64, 128}
 *   block_size          must be 16
 *   num_blocks          NB >= 1
 *   max_blocks_per_seq  row length of block_tables
 *   num_query_tokens    T = q_start[B], the packed query rows of q / out
 *   q_dtype, kv_dtype   (BF16, BF16) or (BF16, FP8_E4M3FN)
 *   k_scale, v_scale    per-tensor dequantisation scales of an FP8 pool
 *                       (finite, > 0); ignored for BF16 pools.
 */
typedef struct {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_size;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_query_tokens;
  pa_dtype q_dtype;
  pa_dtype kv_dtype;
  float k_scale;
  float v_scale;
} pa_prefill_desc;

/*
 * Chunked-prefill attention over the paged pool.  A prompt may be cut into
 * chunks that the scheduler mixes with decode work ("vLLM innenfra",
 * step() and continuous-batching paragraphs); the chunk's own K/V are in
 * the pool already (pa_kv_append), and each of its query tokens attends to
 * every cached token before it and to the chunk up to itself.  For
 * sequence b with L = seq_lens[b] cached tokens and chunk rows
 * q_start[b] .. q_start[b+1] (C rows), query row i sits at position
 * p = L - C + i and
 *     out[q_start[b] + i][h][:] = sum_{t <= p} softmax_t(scale <q, K_t>) V_t
 * with K_t, V_t of KV head h / (Hq / Hkv) found through the block table.
 * The result equals dense causal attention over the contiguous context
 * ("PagedAttention：KV cache 即虚拟内存", section "直接答案").
 *   q, out          [T][Hq][D] bf16, 16-byte aligned
 *   k_pool, v_pool  as for pa_decode: bf16, or fp8 e4m3fn codes whose
 *                   values are code * k_scale (K) and code * v_scale (V)
 *   block_tables    int32 [B][max_blocks_per_seq]
 *   seq_lens        int32 [B], the chunk included
 *   q_start         int32 [B+1], non-decreasing, q_start[B] = T
 * Containment: q_start values are clamped to [0, T] (rows outside are not
 * read or written), seq_lens to [0, max_blocks_per_seq * 16]; a chunk
 * longer than its sequence gives zero rows for tokens before position 0;
 * block ids outside [0, NB) contribute nothing.
 * scale must be finite and positive (the kernel takes each step's row
 * maximum on the unscaled scores).
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (also for scale <= 0 and for FP8 scales
 * that are not finite and positive), PA_ERR_DTYPE,
 * PA_ERR_ALIGN, PA_ERR_LAUNCH.  Asynchronous on `stream`; no workspace.
 */
int pa_prefill(const void* q, const void* k_pool, const void* v_pool,
               const int32_t* block_tables, const int32_t* seq_lens,
               const int32_t* q_start, float scale, void* out,
               const pa_prefill_desc* desc, void* stream);

/* Static English text of a pa_status value. */
const char* pa_status_string(int status);

/* ABI version of this header (bumped on any incompatible change). */
int pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
