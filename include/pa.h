/*
 * pa.h -- C ABI of libpa.so, MI355X (gfx950) paged attention.
 *
 * Paged attention keeps each sequence's keys and values in fixed-size blocks
 * of a shared pool; a per-sequence block table maps the sequence's logical
 * blocks to physical ones, so the storage need not be contiguous.
 *   - "Inside vLLM: Anatomy of a High-Throughput LLM Inference System",
 *     section "LLM Engine & Engine Core": the KV-cache manager keeps a
 *     free_block_queue, and blocks are the index from a sequence's tokens to
 *     their KV-cache blocks.  Section "LLM Engine constructor": block bytes
 *     = 2 * block_size * num_kv_heads * head_size * dtype_num_bytes; the
 *     CPU-side input batch holds the block tables; the cache is allocated
 *     once, reshaped and bound to the attention layers; attention metadata
 *     is prepared on the host and consumed by the kernels.
 *   - "Im Inneren von vLLM: Anatomie eines Hochdurchsatz-LLM-Inferenzsystems",
 *     sections "Paged Attention & KV-Cache" and "Fortgeschrittene Funktionen"
 *     (chunked prefill, prefix caching).
 *   - "vLLM: Ein tiefer Einblick ... auf Basis von PagedAttention", section
 *     "Tiefenanalyse": non-contiguous KV storage modelled on OS paging.
 *
 * Conventions used by every entry point
 *   Status: every int-returning call returns a pa_status; on failure
 *   pa_last_error() returns a message (thread-local, valid until the next
 *   failing call on that thread).  Arguments are validated on the host
 *   before anything is enqueued, so a failed call has no device effect.
 *
 *   Pool layout (the pages give only the byte count; this is the reading):
 *     kv_cache[num_blocks][2][num_kv_heads][block_size][head_size]
 *   index 0 of the second axis holds keys, 1 holds values; one block is
 *   exactly pa_kv_block_bytes() contiguous bytes.  Element type is fp32 or
 *   bf16 (pa_dtype); queries and outputs use the same element type.
 *
 *   Token position p of a sequence lives at slot
 *     block_tables[b][p / block_size] * block_size + p % block_size.
 *   Query head h reads KV head h / (H_q / H_kv).
 *
 *   Device pointers are device memory owned by the caller (e.g. allocated by
 *   torch).  The library never allocates or frees device memory and never
 *   synchronises: device work is enqueued on `stream` (a hipStream_t; NULL
 *   is the default stream) and returns immediately.  Device-side contents
 *   (block ids, slots, seq_lens) are the caller's contract: block ids must be
 *   in [0, num_blocks), seq_lens[b] <= max_seq_len, slots unique.  Out-of-
 *   range block ids are clamped to block 0 (wrong result, no fault).
 *   Nothing here is thread-safe per allocator handle.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_EINVAL = 1,     /* bad argument (shape, pointer, refcount, ...) */
  PA_ENOBLOCKS = 2,  /* allocator: not enough free blocks; state unchanged */
  PA_ENOTSUP = 3,    /* valid but unsupported (head size, block size, dtype) */
  PA_EHIP = 4        /* the HIP runtime reported an error at launch */
} pa_status;

/* PA_FP8: an FP8 (OCP E4M3) KV cache with per-tensor key/value scales; the
 * queries and outputs around it are bf16 (pa_reshape_and_cache_fp8,
 * pa_decode_fp8).  Passed as the dtype of an entry point without scales
 * (pa_reshape_and_cache, pa_decode, pa_decode_append, pa_decode_multi,
 * pa_prefill_chunk, pa_attention_varlen) it is PA_EINVAL: the *_fp8 entry
 * points carry the scales. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8 = 2 } pa_dtype;

/* Message of the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int pa_version(void);

/* ---------------------------------------------------------------------------
 * Closed forms ("Inside vLLM", section "LLM Engine constructor")
 * ------------------------------------------------------------------------- */

/* Bytes of one block: 2 (key and value) * block_size * num_kv_heads *
 * head_size * dtype_bytes.  Returns 0 if any argument is <= 0. */
size_t pa_kv_block_bytes(int32_t block_size, int32_t num_kv_heads,
                         int32_t head_size, int32_t dtype_bytes);

/* Blocks that fit in budget_bytes when each of num_layers layers needs one
 * block per block id: floor(budget / (block_bytes * num_layers)).
 * Returns -1 if block_bytes or num_layers is 0 / negative. */
int64_t pa_num_blocks_for_budget(uint64_t budget_bytes, size_t block_bytes,
                                 int32_t num_layers);

/* ---------------------------------------------------------------------------
 * Host block allocator: the free_block_queue ("Inside vLLM", section
 * "LLM Engine & Engine Core").  The pages name the queue but not its policy;
 * this one is FIFO: allocate pops from the head, a block goes back to the
 * tail when its reference count drops to zero (in the order the ids are
 * given).  Prefix caching ("Im Inneren von vLLM", "Fortgeschrittene
 * Funktionen") shares blocks by reference count.  Host memory only; every
 * pointer argument is host memory owned by the caller.
 * ------------------------------------------------------------------------- */
typedef struct pa_allocator pa_allocator;

/* Creates an allocator over block ids 0..num_blocks-1.  initial_order
 * (nullable: 0..N-1) gives the initial queue order and must be a
 * permutation.  *out receives an opaque handle owned by the library. */
int pa_allocator_create(int32_t num_blocks, const int32_t* initial_order,
                        pa_allocator** out);
void pa_allocator_destroy(pa_allocator* a);

/* Pops n ids from the head into out_ids[0..n) and sets their reference
 * counts to 1.  All-or-nothing: PA_ENOBLOCKS if fewer than n are free, with
 * no state change.  n == 0 is a no-op; n < 0 is PA_EINVAL. */
int pa_allocator_allocate(pa_allocator* a, int32_t n, int32_t* out_ids);

/* Block tables of a batch in one call ("Inside vLLM", "LLM Engine
 * constructor": the CPU side holds the block tables for KV-cache
 * indexing): sequences 0..B-1 in order each take ceil(seq_lens[b] /
 * block_size) blocks from the head of the queue, exactly as that many
 * pa_allocator_allocate calls would, and row b of block_tables ([B][width]
 * int32, host) receives their ids followed by -1 padding.  All-or-nothing:
 * PA_ENOBLOCKS if the batch needs more blocks than are free, PA_EINVAL if
 * a sequence needs more than width blocks; either leaves the allocator and
 * the table untouched. */
int pa_allocator_build_tables(pa_allocator* a, const int32_t* seq_lens, int32_t B,
                              int32_t block_size, int32_t width, int32_t* block_tables);

/* Adds one reference to each listed (allocated) block.  PA_EINVAL, with no
 * state change, if any id is out of range or free. */
int pa_allocator_share(pa_allocator* a, const int32_t* ids, int32_t n);

/* Drops one reference per listed id (an id may repeat); a block whose count
 * reaches zero is pushed to the tail, in list order.  PA_EINVAL, with no
 * state change, if any id is out of range or would drop below zero. */
int pa_allocator_free(pa_allocator* a, const int32_t* ids, int32_t n);

int32_t pa_allocator_num_free(const pa_allocator* a);
int32_t pa_allocator_num_blocks(const pa_allocator* a);

/* Whole state: queue_out[0..num_free) = queue head..tail (nullable),
 * refcount_out[0..num_blocks) (nullable). */
int pa_allocator_export(const pa_allocator* a, int32_t* queue_out,
                        int32_t* refcount_out);

/* Fragmentation stats: *used_blocks = blocks with a live reference;
 * *tail_waste_tokens = sum over the B sequences of ceil(L/bs)*bs - L (the
 * unused slots of each last block). */
int pa_allocator_stats(const pa_allocator* a, const int32_t* seq_lens,
                       int32_t B, int32_t block_size, int64_t* used_blocks,
                       int64_t* tail_waste_tokens);

/* ---------------------------------------------------------------------------
 * Prefix cache on the allocator ("Im Inneren von vLLM", section
 * "Fortgeschrittene Funktionen"; "vLLM: Ein tiefer Einblick ...", section
 * "Tiefenanalyse": the KV cache of common prompt prefixes is kept and reused).
 * The pages give no mechanism; the reading implemented here:
 *   - only full blocks are cached; a block's keys and values depend on every
 *     token up to its end, so a cached block is identified by that whole
 *     token prefix (exact comparison, no hash collisions);
 *   - a freed block (reference count 0) goes back to the free queue as
 *     before but keeps its cached contents ("cached free") until
 *     pa_allocator_allocate pops it, which evicts it from the cache;
 *   - a lookup that hits a cached free block takes it out of the queue;
 *   - the queue order decides eviction, so a sequence should free its
 *     blocks last-to-first: a deeper block is only reachable through its
 *     predecessors and is the one to go first.
 * Host memory only; tokens are int32 token ids.
 * ------------------------------------------------------------------------- */

/* Turns the prefix cache on for blocks of block_size tokens.  Calling it
 * again with the same block_size is a no-op; another value is PA_EINVAL. */
int pa_prefix_cache_enable(pa_allocator* a, int32_t block_size);

/* Longest cached prefix of tokens[0..num_tokens): walks the full blocks
 * j = 0, 1, ... of the token list and stops at the first whose prefix is not
 * cached.  Each hit block gains one reference (a cached free block leaves
 * the free queue) and its id goes to out_ids[j]; *num_hit receives the
 * count.  out_ids must hold num_tokens / block_size entries.  A caller that
 * must compute at least one token passes num_tokens - 1. */
int pa_prefix_cache_acquire(pa_allocator* a, const int32_t* tokens,
                            int32_t num_tokens, int32_t* out_ids,
                            int32_t* num_hit);

/* Registers the full blocks of a sequence whose keys and values are now
 * written: block_ids[j] (allocated, num_blocks >= num_tokens / block_size)
 * holds tokens [j*bs, (j+1)*bs).  A prefix that is cached already keeps its
 * block (block_ids[j] then stays uncached).  PA_EINVAL, with no state change,
 * if an id is out of range, free, listed twice, or already caches another
 * prefix. */
int pa_prefix_cache_insert(pa_allocator* a, const int32_t* tokens,
                           int32_t num_tokens, const int32_t* block_ids,
                           int32_t num_blocks);

/* cached_out[0..num_blocks) (nullable): 1 if the block caches a prefix.
 * stats_out[3] (nullable): cached blocks, total hit blocks, total evictions. */
int pa_prefix_cache_export(const pa_allocator* a, int32_t* cached_out,
                           int64_t* stats_out);

/* ---------------------------------------------------------------------------
 * Token -> slot ("Inside vLLM", section "LLM Engine & Engine Core": blocks
 * map tokens to their KV-cache blocks).  Host memory.
 * For each sequence b (in order) and i in [0, num_tokens[b]):
 *   p = start_pos[b] + i
 *   out[k++] = block_tables[b*max_blocks_per_seq + p/bs] * bs + p % bs
 * Returns PA_EINVAL if a needed table entry is negative or p/bs is beyond
 * max_blocks_per_seq.  *total (nullable) receives the number of slots.
 * ------------------------------------------------------------------------- */
int pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* start_pos, const int32_t* num_tokens,
                    int32_t B, int32_t block_size, int64_t* out,
                    int64_t* total);

/* ---------------------------------------------------------------------------
 * Device operations
 * ------------------------------------------------------------------------- */

/* Writes new keys/values into the cache ("Inside vLLM", section "LLM Engine
 * constructor": KV tensors bound to the layers; section "LLM Engine & Engine
 * Core": tokens map to their blocks).
 *   key, value   [num_tokens][num_kv_heads][head_size], dtype, device
 *   slot_mapping [num_tokens] int64, device; slot < 0 skips the token;
 *                slots must be unique and < num_blocks*block_size
 *   kv_cache     pool layout above, device
 * Values are copied bit for bit.  block_size must be 16; head_size 64 or
 * 128 (PA_ENOTSUP otherwise).  num_tokens == 0 enqueues nothing. */
int pa_reshape_and_cache(const void* key, const void* value,
                         const int64_t* slot_mapping, int32_t num_tokens,
                         void* kv_cache, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads,
                         int32_t head_size, int32_t dtype, void* stream);

/* FP8 cache write: keys/values arrive in bf16 and are stored as FP8 (OCP
 * E4M3) codes, one byte per element, in the same pool layout ("Inside
 * vLLM", "LLM Engine constructor", for the cache; "vLLM: Ein tiefer
 * Einblick ...", "Tiefenanalyse", lists FP8 among the engine's quantisation
 * formats but fixes no format or scale: E4M3 and per-tensor scales are this
 * library's reading).  Element x of
 * the keys becomes the E4M3 code of x / k_scale, computed in fp32 with IEEE
 * division, saturated at +-448 and rounded to nearest even, sign kept; the
 * values likewise with v_scale.  The cache then represents code * scale.
 *   key, value   [num_tokens][num_kv_heads][head_size] bf16, device,
 *                16-byte aligned
 *   slot_mapping as pa_reshape_and_cache
 *   kv_cache     [num_blocks][2][num_kv_heads][16][head_size] uint8, device,
 *                16-byte aligned
 *   k_scale, v_scale  positive and finite (PA_EINVAL otherwise)
 * block_size 16, head_size 64 or 128. */
int pa_reshape_and_cache_fp8(const void* key, const void* value,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             void* kv_cache, int32_t num_blocks,
                             int32_t block_size, int32_t num_kv_heads,
                             int32_t head_size, float k_scale, float v_scale,
                             void* stream);

/* Device workspace pa_decode needs for split-K, in bytes: a fixed region of
 * 65536 arrival counters (one per (sequence, KV head), so B * H_kv <= 65536
 * with split-K) followed by one fp32 record per (sequence, KV head,
 * partition): the G heads' normalised outputs, maxima and denominators,
 * padded to 128-byte lines.  0 when partition_size == 0 or one partition
 * covers max_seq_len.  A workspace sized for the largest shape serves calls
 * of any smaller shape. */
size_t pa_decode_workspace_bytes(int32_t B, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_size,
                                 int32_t max_seq_len, int32_t partition_size);

/* Zero-fills a decode workspace on `stream` (a fill kernel, no memset).  A
 * workspace must be zero before its first pa_decode; every completed
 * pa_decode leaves it reusable (its counters return to zero), so one
 * initialisation serves any number of calls, including graph replays.
 * workspace: device, 256-byte aligned; bytes a multiple of 4. */
int pa_decode_workspace_init(void* workspace, size_t workspace_bytes,
                             void* stream);

/* Decode work plan (host).  The attention metadata of a step is prepared on
 * the CPU and consumed by the kernels ("Inside vLLM", section "LLM Engine
 * constructor"); this builds the decode kernel's work list from host-side
 * sequence lengths: one entry per non-empty (sequence, partition) pair,
 * encoded as (partition << 16) | sequence, longest partitions first.
 *   seq_lens     [B] int32, host, each in [0, max_seq_len]
 *   plan         [capacity] int32, host (nullable when capacity is 0)
 *   num_entries  receives the number of entries (also when capacity is too
 *                small, in which case PA_EINVAL is returned)
 * At most B * ceil(max_seq_len / partition_size) entries (B when
 * partition_size is 0).  B <= 65535 and <= 65535 partitions. */
int pa_decode_plan(const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                   int32_t partition_size, int32_t* plan, int32_t capacity,
                   int32_t* num_entries);

/* The host half of one decode step in one call ("Inside vLLM", section
 * "LLM Engine & Engine Core": the KV-cache manager allocates blocks from
 * the free_block_queue as sequences grow; section "LLM Engine constructor":
 * the CPU side prepares the step's attention metadata).  Every sequence b
 * gains one token at position p = seq_lens[b]: if p % block_size == 0 the
 * token opens a block, which is taken from the head of the allocator's
 * queue (sequences in order, exactly as one pa_allocator_allocate of that
 * many blocks) into block_tables[b][p / block_size]; slots[b] receives
 * block_tables[b][p / block_size] * block_size + p % block_size, and
 * seq_lens[b] becomes p + 1.  With plan non-NULL, plan receives
 * pa_decode_plan of the new lengths (max_seq_len, partition_size) and
 * *num_entries (nullable) its length.
 *   block_tables [B][max_blocks_per_seq] int32, host, updated in place
 *   seq_lens     [B] int32, host, updated in place
 *   slots        [B] int64, host (written)
 *   plan         [plan_capacity] int32, host, nullable
 * All-or-nothing: nothing changes when a call fails.  PA_EINVAL if a new
 * token reaches max_seq_len or beyond the table, if the entry a new block
 * goes to already holds one (>= 0), if a token that does not open a block
 * finds none, or if the plan needs more than plan_capacity entries;
 * PA_ENOBLOCKS if fewer blocks are free than the step opens.  Host memory
 * only. */
int pa_decode_step_prepare(pa_allocator* allocator, int32_t* block_tables,
                           int32_t max_blocks_per_seq, int32_t* seq_lens, int32_t B,
                           int32_t block_size, int32_t max_seq_len,
                           int32_t partition_size, int64_t* slots, int32_t* plan,
                           int32_t plan_capacity, int32_t* num_entries);

/* Decode attention: one query token per sequence, the last of its seq_len
 * cached tokens (already written), attends to all of them through its block
 * table; grouped-query heads share KV heads.  The attention itself is the
 * standard transformer's ("Inside vLLM", "LLM Engine & Engine Core"):
 *   o = softmax(scale * q K^T) V,  lse = ln sum exp(scale * q K^T).
 *   out          [B][H_q][D] dtype, device (written)
 *   lse_out      [B][H_q] fp32, device, nullable (natural log; -inf and
 *                out = 0 for seq_len 0)
 *   query        [B][H_q][D] dtype, device
 *   block_tables [B][max_blocks_per_seq] int32, device
 *   seq_lens     [B] int32, device, each in [0, max_seq_len]
 *   partition_size  0: one pass per (sequence, KV head); otherwise a
 *                multiple of block_size: the context is split into
 *                partitions of that many tokens, each processed by its own
 *                workgroup, and the partials are combined with a
 *                log-sum-exp weighted sum (split-K): by the last workgroup
 *                of each (sequence, KV head) to finish, or, for partitions
 *                of 1024 tokens or more, by a second launch on the same
 *                stream.
 *   plan, plan_entries  device copy of pa_decode_plan's output for these
 *                seq_lens and partition_size, or NULL / 0: then every
 *                (sequence, partition up to max_seq_len) pair is visited and
 *                the empty ones are skipped on the device.
 *   workspace    device, >= pa_decode_workspace_bytes(...) bytes (nullable
 *                when that is 0), owned by the caller, zeroed once by
 *                pa_decode_workspace_init (or any zero fill) before first
 *                use.  Two pa_decode calls sharing a workspace must not run
 *                concurrently.
 * With a plan the launch has one workgroup per work item; without one, a
 * grid of a few times the resident workgroups walks the items.
 * Supported: block_size 16; head_size 64 or 128; H_q % H_kv == 0 with
 * G = H_q/H_kv in {1, 2, 4, 8} (and 16 for head_size 64). */
int pa_decode(void* out, float* lse_out, const void* query,
              const void* kv_cache, int32_t num_blocks,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
              int32_t block_size, float scale, int32_t partition_size,
              const int32_t* plan, int32_t plan_entries, void* workspace,
              size_t workspace_bytes, int32_t dtype, void* stream);

/* The device half of a decode step in one launch: the new token of every
 * sequence is written into the cache and attended to with the others.  The
 * result, the cache and the errors equal pa_reshape_and_cache of the new
 * tokens (each at its position seq_len - 1, in the slot the block table
 * gives: block_tables[b][(seq_len - 1) / 16] * 16 + (seq_len - 1) % 16)
 * followed by pa_decode with the same arguments ("Inside vLLM", "LLM
 * Engine constructor": the new K/V are bound into the paged cache before
 * attention reads it).
 *   new_key, new_value  [B][H_kv][D] dtype, device, 16-byte aligned: the K
 *                and V of token seq_len[b] - 1 of each sequence (unused
 *                for seq_len 0).
 *   kv_cache     written at those slots only; a block id out of range is
 *                read as block 0 (as in pa_decode) and not written.
 * All other arguments as pa_decode. */
int pa_decode_append(void* out, float* lse_out, const void* query,
                     const void* new_key, const void* new_value, void* kv_cache,
                     int32_t num_blocks, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                     int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_size, int32_t block_size, float scale,
                     int32_t partition_size, const int32_t* plan, int32_t plan_entries,
                     void* workspace, size_t workspace_bytes, int32_t dtype, void* stream);

/* pa_decode over an FP8 cache written by pa_reshape_and_cache_fp8: keys and
 * values are their codes times k_scale / v_scale, and the result is
 * pa_decode's on those values (scores scale * q . (code * k_scale)).
 * query and out are bf16; lse_out, the workspace, plan and every other
 * argument as pa_decode.  E4M3 codes are exact in bf16, so the products run
 * on the same bf16 matrix-core path; k_scale folds into the score scale and
 * v_scale into the outputs.  Same shapes as pa_decode's bf16 path. */
int pa_decode_fp8(void* out, float* lse_out, const void* query,
                  const void* kv_cache, int32_t num_blocks,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* seq_lens, int32_t B, int32_t max_seq_len,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_size,
                  int32_t block_size, float scale, float k_scale, float v_scale,
                  int32_t partition_size, const int32_t* plan,
                  int32_t plan_entries, void* workspace, size_t workspace_bytes,
                  void* stream);

/* pa_decode_append without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Its split-K counters and
 * partial records live in a static device array of
 * PA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per device the
 * library runs on, held until the process ends; the call allocates
 * nothing.  Inputs, outputs and errors as pa_decode_append; additionally
 * PA_EINVAL when the split-K layout (pa_decode_workspace_bytes of the same
 * sizes) exceeds PA_NOALLOC_SCRATCH_BYTES, and PA_EHIP when the runtime
 * cannot resolve the array's device address.  The first call on a device
 * clears the array's counters on `stream` (a fill kernel); every completed
 * call leaves them at zero.  All calls on one device share the array:
 * calls that overlap on one GPU (two streams, two threads) race and give
 * wrong results. */
#define PA_NOALLOC_SCRATCH_BYTES (128u << 20)
int pa_decode_append_noalloc(void* out, float* lse_out, const void* query,
                             const void* new_key, const void* new_value, void* kv_cache,
                             int32_t num_blocks, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                             int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size, float scale,
                             int32_t partition_size, const int32_t* plan, int32_t plan_entries,
                             int32_t dtype, void* stream);

/* pa_decode_append for an FP8 cache: the new token of every sequence is
 * quantised exactly as pa_reshape_and_cache_fp8 does (new_key/new_value
 * bf16 [B][H_kv][D], 16-byte aligned; k_scale/v_scale), written to its slot
 * and attended to, in one launch.  Equals pa_reshape_and_cache_fp8 of the
 * new tokens followed by pa_decode_fp8 (pool bit for bit, outputs as
 * pa_decode_fp8).  Other arguments as pa_decode_fp8. */
int pa_decode_append_fp8(void* out, float* lse_out, const void* query,
                         const void* new_key, const void* new_value, void* kv_cache,
                         int32_t num_blocks, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                         int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size, float scale,
                         float k_scale, float v_scale, int32_t partition_size,
                         const int32_t* plan, int32_t plan_entries, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Several query rows per sequence on the decode path: sequence b's last
 * `rows` tokens (already written to the cache) each attend causally to the
 * tokens up to themselves, as in a chunk of pa_prefill_chunk.  This is the
 * verification step of speculative decoding, which proposes several tokens
 * and checks them in one pass ("vLLM: Ein tiefer Einblick ...", section
 * "Tiefenanalyse", and "Im Inneren von vLLM", "Fortgeschrittene
 * Funktionen": speculative decoding; "Inside vLLM", "LLM Engine & Engine
 * Core": the attention is the standard transformer's).  Query row i of
 * sequence b (0 <= i < rows) sits at position seq_lens[b] - rows + i:
 *   o = softmax(scale * q K[0..pos]^T) V[0..pos]; a row before position 0
 *   (seq_lens[b] < rows) gets o = 0 and lse = -inf.
 *   out, query   [B * rows][H_q][D], bf16, device; row b * rows + i
 *   lse_out      [B * rows][H_q] fp32, device, nullable
 *   other arguments as pa_decode (plan: pa_decode_plan of the same seq_lens
 *   and partition_size); workspace >= pa_decode_multi_workspace_bytes(...).
 * A work item covers floor(16 / G) rows with their G heads (one matrix tile
 * of 16 columns; at head size 64, when the rows need more than one tile,
 * two tiles: floor(32 / G) rows) over one partition; longer row sets take
 * several items.  rows in [1, 64]; rows > 1 needs a bf16 cache (an FP8
 * cache goes through pa_decode_multi_fp8: dtype PA_FP8 here is PA_EINVAL)
 * and G <= 16; rows == 1 is pa_decode.  Split-K needs
 * B * H_kv * (items per (sequence, KV head)) <= 65536. */
size_t pa_decode_multi_workspace_bytes(int32_t B, int32_t rows, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_size,
                                       int32_t max_seq_len, int32_t partition_size);
int pa_decode_multi(void* out, float* lse_out, const void* query, const void* kv_cache,
                    int32_t num_blocks, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                    int32_t max_seq_len, int32_t rows, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                    float scale, int32_t partition_size, const int32_t* plan,
                    int32_t plan_entries, void* workspace, size_t workspace_bytes,
                    int32_t dtype, void* stream);

/* pa_decode_multi over an FP8 (E4M3) cache with per-tensor key/value scales
 * (as pa_decode_fp8): queries and outputs bf16, the cache uint8 codes whose
 * values are code * k_scale / code * v_scale.  Other arguments, the
 * workspace and the limits as pa_decode_multi; rows == 1 is pa_decode_fp8.
 * k_scale, v_scale positive and finite (PA_EINVAL otherwise). */
int pa_decode_multi_fp8(void* out, float* lse_out, const void* query, const void* kv_cache,
                        int32_t num_blocks, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t B,
                        int32_t max_seq_len, int32_t rows, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                        float scale, float k_scale, float v_scale, int32_t partition_size,
                        const int32_t* plan, int32_t plan_entries, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Chunked prefill ("Im Inneren von vLLM", "Fortgeschrittene Funktionen":
 * long prompts are split into chunks; "Inside vLLM", "Generate function":
 * the batch is flattened into one sequence of tokens).  Sequence b owns the
 * packed query rows [query_start_loc[b], query_start_loc[b+1]); its C_b
 * queries are its last C_b tokens (keys/values already written), and query
 * i at position seq_lens[b] - C_b + i attends causally to tokens
 * 0..position, reading the cached prefix (possibly blocks shared with other
 * sequences) and its own keys through its block table.
 *   out, query      [total_query_tokens][H_q][D] bf16, device
 *   lse_out         [total_query_tokens][H_q] fp32, device, nullable
 *   query_start_loc [B+1] int32, device, non-decreasing, [0] = 0,
 *                   [B] = total_query_tokens, every C_b <= max_query_len
 *   seq_lens        [B] int32, device, C_b <= seq_lens[b] <= max_seq_len
 * Supported: bf16 only; block_size 16; head_size 128 or 64; G in
 * {1, 2, 4, 8}. */
int pa_prefill_chunk(void* out, float* lse_out, const void* query,
                     const int32_t* query_start_loc, int32_t max_query_len,
                     int32_t total_query_tokens, const void* kv_cache,
                     int32_t num_blocks, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* seq_lens,
                     int32_t B, int32_t max_seq_len, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_size,
                     int32_t block_size, float scale, int32_t dtype,
                     void* stream);

/* Work plan of a flattened batch (host).  A step's query rows come from
 * every scheduled sequence at once: one row for a sequence in decode, a
 * chunk of its prompt for one in prefill ("Inside vLLM", "Generate
 * function" and "LLM Engine & Engine Core": continuous batching over a
 * batch flattened into one sequence).  Sequences with C_b = 1 query row
 * become decode items (split into partitions of partition_size tokens
 * when that is non-zero and max_seq_len needs more than one); a short
 * chunk, C_b >= 2 rows that fit 4 groups of 16 / G rows (e.g. the tokens a
 * speculative step checks), becomes one multi-row decode item per group,
 * each a single pass over the sequence's tokens (pa_decode_multi's tile);
 * longer chunks become query tiles of 128 / G rows; C_b = 0 nothing.
 * Entries are (1 << 31) | (tile << 16) | b for a query tile,
 * (partition << 16) | b for a decode item (partition < 2^14) and
 * (1 << 30) | (group << 16) | b for a short chunk's group.
 *   query_start_loc [B+1] int32, host, [0] = 0, non-decreasing
 *   seq_lens        [B] int32, host, C_b <= seq_lens[b] <= max_seq_len
 *   plan            [capacity] int32, host (nullable when capacity is 0)
 *   num_entries, num_prefill_entries  receive the entry counts (also when
 *                   capacity is too small: then PA_EINVAL)
 * G = num_q_heads / num_kv_heads in {1, 2, 4, 8}; B <= 65535; at most 16383
 * partitions. */
int pa_varlen_plan(const int32_t* query_start_loc, const int32_t* seq_lens,
                   int32_t B, int32_t max_seq_len, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t partition_size, int32_t* plan,
                   int32_t capacity, int32_t* num_entries,
                   int32_t* num_prefill_entries);

/* Attention over a flattened batch in one launch: decode rows and prefill
 * chunks together.  Every query row computes what pa_prefill_chunk defines
 * for it (query i of sequence b, at position seq_lens[b] - C_b + i, attends
 * causally to tokens 0..position through the block table; keys/values
 * already written); a sequence with one row gets exactly pa_decode's
 * result for it.  Chunks run on the prefill path (matrix-core tiles),
 * single rows on the decode path (optionally split-K), short chunks on the
 * decode path's multi-row tiles, in one grid.
 *   out, query      [total_query_tokens][H_q][D] bf16, device
 *   lse_out         [total_query_tokens][H_q] fp32, device, nullable
 *   query_start_loc [B+1] int32, device: the same values the plan was
 *                   built from (the kernel reads rows from it)
 *   seq_lens        [B] int32, device, likewise
 *   partition_size  as given to pa_varlen_plan
 *   plan, plan_entries  device copy of pa_varlen_plan's output and its
 *                   entry count
 *   workspace       as pa_decode's, sized by pa_decode_workspace_bytes(B,
 *                   H_q, H_kv, D, max_seq_len, partition_size); calls
 *                   sharing a workspace must not run concurrently
 * Rows of sequences with C_b = 0 are not touched.  Supported: bf16;
 * block_size 16; head_size 64 or 128; G in {1, 2, 4, 8}. */
int pa_attention_varlen(void* out, float* lse_out, const void* query,
                        const int32_t* query_start_loc,
                        int32_t total_query_tokens, const void* kv_cache,
                        int32_t num_blocks, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* seq_lens,
                        int32_t B, int32_t max_seq_len, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_size,
                        int32_t block_size, float scale, int32_t partition_size,
                        const int32_t* plan, int32_t plan_entries,
                        void* workspace, size_t workspace_bytes,
                        int32_t dtype, void* stream);

/* ---------------------------------------------------------------------------
 * Decode-step graphs for warm-up batch sizes ("Inside vLLM", section "LLM
 * Engine constructor": the engine captures a graph of the forward pass for
 * each of a list of warm-up batch sizes and replays it during decoding).
 * ------------------------------------------------------------------------- */
typedef struct pa_decode_graphs pa_decode_graphs;

/* Captures, once per size Bc in batch_sizes (num_sizes entries, each in
 * [1, 65535]; duplicates ignored), the attention of a decode step over
 * num_layers layers: pa_decode_append for layer 0, 1, ... in order, each with
 * B = Bc on the first Bc rows of that layer's buffers and no plan (its
 * fixed grid walks every (sequence, partition up to max_seq_len) pair and
 * skips the empty ones on the device, so one graph serves any lengths up to
 * max_seq_len).  Capture runs on `stream`, which must not be the null
 * stream; the graphs are instantiated at once.  The buffers are the
 * caller's, static, device memory, sized for the largest size Bmax and
 * layer-major:
 *   out, query        [num_layers][Bmax][H_q][D] dtype
 *   lse_out           [num_layers][Bmax][H_q] fp32, nullable
 *   new_key, new_value [num_layers][Bmax][H_kv][D] dtype
 *   kv_caches         host array of num_layers device pointers, each a
 *                     cache of num_blocks blocks as pa_decode_append's
 *   block_tables      [Bmax][max_blocks_per_seq] int32, shared by the layers
 *   seq_lens          [Bmax] int32, shared by the layers
 *   workspace         as pa_decode_append's for Bmax sequences (shared by
 *                     the layers, which run one after another), zeroed by
 *                     pa_decode_workspace_init before the first replay.
 * dtype is PA_BF16 or PA_F32.  The addresses are recorded: the buffers must
 * stay allocated, and their contents at replay time are what a replay
 * reads.  Argument errors are PA_EINVAL here or pa_decode_append's (checked
 * at capture); PA_EHIP if capture or instantiation fails.  *handle receives
 * an object owned by the library (pa_decode_graphs_destroy); nothing is
 * launched. */
int pa_decode_graphs_create(void* out, float* lse_out, const void* query,
                            const void* new_key, const void* new_value,
                            void* const* kv_caches, int32_t num_layers, int32_t num_blocks,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            int32_t* seq_lens, int32_t max_seq_len, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                            float scale, int32_t partition_size, void* workspace,
                            size_t workspace_bytes, int32_t dtype,
                            const int32_t* batch_sizes, int32_t num_sizes, void* stream,
                            pa_decode_graphs** handle);

/* One decode step of B sequences (0 <= B <= Bmax) whose rows 0..B-1 the
 * caller has written into the static buffers (every layer's): on `stream`
 * (any stream of the capturing device), writes seq_lens[B..Bc) = 0 with a
 * fill kernel, where Bc is the smallest captured size >= B, then launches
 * graph Bc.  Padding rows B..Bc-1 get a zero output row and lse -inf in
 * every layer and write nothing into the caches; rows from Bc on are not
 * touched.  *graph_batch
 * (nullable) receives Bc (0 for B = 0, which launches nothing).
 * PA_EINVAL for B outside [0, Bmax] or another current device.  Replays of
 * one handle share its buffers and workspace: they must not overlap. */
int pa_decode_graphs_replay(pa_decode_graphs* handle, int32_t B, void* stream,
                            int32_t* graph_batch);

/* Number of captured sizes (-1 for a NULL handle); the first `capacity` of
 * them, ascending, into batch_sizes (nullable). */
int32_t pa_decode_graphs_count(const pa_decode_graphs* handle, int32_t* batch_sizes,
                               int32_t capacity);

/* Releases the graphs (the caller's buffers are untouched).  NULL is a
 * no-op. */
void pa_decode_graphs_destroy(pa_decode_graphs* handle);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
