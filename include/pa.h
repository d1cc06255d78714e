/*
 * pa.h — paged KV-cache attention (decode and prefill) for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * Plain C ABI: raw pointers and sizes, no HIP or PyTorch types. Streams are hipStream_t
 * handles passed as void* (NULL = the default stream). All device buffers are owned by the
 * caller; the library allocates no device memory and keeps no per-call state (the one exception
 * is pa_decode_static's fixed partition-state array, which the library holds on each device
 * from its loading on). Every call is asynchronous on its stream.
 *
 * Sources, cited by page title and section:
 *   [wiki] "PagedAttention" (newikis.com/ko/PagedAttention), "수학적 공식" (mathematical
 *          formulation): dense causal attention of query token i, and the same computation
 *          over key/value blocks K_j, V_j of B tokens, summed over the first ceil(i/B) blocks.
 *   [anal] "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리" (ryotta.opik.net): §2 fixed-size
 *          KV blocks in scattered physical memory addressed through a block table; §3 the
 *          block-wise attention kernel and its block-table lookup pseudocode; §4 copy-on-write.
 *   [blog] "PagedAttention 논문 쉽게 읽기" (iplexlaw.co.kr): §2 a new token is written into the
 *          free slot of its sequence's last block; ② copy-on-write of a shared block.
 *   [dev]  "추론 엔진에서의 메모리 가상화: PagedAttention과 메모리 단편화의 제거" (molayo1419.me):
 *          two large preallocated pools, key_cache and value_cache; block_tables handed to the
 *          attention kernel as a 2-D integer array; the copy in copy-on-write.
 *
 * ---------------------------------------------------------------------------------------------
 * Physical pool layout (chosen for gfx950; the pages' own permuted key layout targets 32-thread
 * warps and is not used)
 * ---------------------------------------------------------------------------------------------
 * Each pool holds num_blocks * num_kv_heads tiles of T = block_size * head_dim elements. Tile
 * (physical block b, KV head h) is contiguous and starts at element (b * num_kv_heads + h) * T,
 * so one physical block is num_kv_heads consecutive tiles. Inside a tile, for slot t in
 * [0, block_size) and head-dimension index i in [0, head_dim):
 *
 *   value pool:  element (t, i) at   t * head_dim + i                      (token rows)
 *   key pool:    with W = 64 / sizeof(element) (elements per 64-byte chunk),
 *                element (t, i) at   (i / W) * (block_size * W) + t * W + (i % W)
 *
 * i.e. the key tile is cut into head_dim / W chunk rows; chunk row c holds the W elements
 * [c*W, c*W + W) of slot 0, then of slot 1, ... of slot block_size-1 (64 bytes per slot). Any
 * 16 consecutive slots of a chunk row are 1 KiB, so one 64-lane wavefront loading 16 bytes per
 * lane reads them in one fully coalesced instruction, each group of four lanes holding 64
 * contiguous bytes of one token: a chunk row is that 1 KiB at block_size 16, two of them at 32,
 * and half of one at 8 (the two halves of a wave load then come from two blocks). A tile is
 * block_size * 256 bytes in every configuration with 256-byte token rows (head_dim 128 at
 * 16-bit, head_dim 64 at 32-bit).
 *
 * Supported: dtype PA_F32 / PA_F16 / PA_BF16 (query, new keys/values, pools and output share
 * it), head_dim 64 or 128, block_size 8, 16 or 32 ([anal] §6 and [dev]: 16 is the default; the
 * block size trades table lookups against the up to B-1 slots a sequence's last block wastes).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library exports these functions and nothing else. */
#if defined(__GNUC__) || defined(__clang__)
#define PA_API __attribute__((visibility("default")))
#else
#define PA_API
#endif

#define PA_ABI_VERSION 7
#define PA_MAX_PARTITION_TOKENS 2048 /* largest partition_size pa_decode accepts */

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent (this includes
                             sizes whose launch would exceed 2^32 - 1 work-items) */
  PA_ERR_UNSUPPORTED = 3, /* dtype, head_dim, block_size or flag the kernels do not support, or
                             memory the device cannot address (pa_swap_blocks) */
  PA_ERR_ALIGN = 4,       /* a data pointer is not 16-byte aligned (int arrays: 4-byte) */
  PA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than pa_decode_workspace_bytes() */
  PA_ERR_LAUNCH = 6,      /* the HIP runtime reported an error when launching */
} pa_status;

/*
 * pa_cache_desc.flags bits.
 *
 * PA_CACHE_SHARED_BLOCKS: some physical blocks are referenced by several sequences of one
 *   pa_decode call (shared prompt prefixes, parallel samples; [anal] §4, [dev] copy-on-write).
 *   pa_decode then reads key/value tiles through the caches so that the sharers reuse them.
 *   Without it every tile is read as a stream (non-temporal loads that do not allocate in the
 *   caches), which is faster when each tile is read once. With 16-bit pools, head_dim 128 and
 *   more than one partition, it also has pa_decode compute a partition that consecutive
 *   sequences share (the whole partition inside every sharer's context, the same physical block
 *   ids in their tables) once for up to 8 of them: one workgroup scores all their queries
 *   against each shared tile. The workspace then also holds a map of those groups
 *   (pa_decode_workspace_bytes counts it when the descriptor carries the flag). Results agree
 *   with the unshared computation within the stated tolerance; they are not bit-identical.
 */
#define PA_CACHE_SHARED_BLOCKS 1u

/* Shape of both pools. */
typedef struct {
  int32_t dtype;        /* pa_dtype of every element in both pools */
  int32_t num_blocks;   /* NB: physical blocks per pool */
  int32_t num_kv_heads; /* Hkv */
  int32_t head_dim;     /* d */
  int32_t block_size;   /* B: token slots per block */
  uint32_t flags;       /* PA_CACHE_* bits; any other bit gives PA_ERR_UNSUPPORTED */
} pa_cache_desc;

/*
 * pa_reshape_and_cache — write new tokens' keys and values into their cache slots.
 * ([blog] §2: a token goes into the free slot of its sequence's last block; [anal] §2 and
 *  "핵심 개념": blocks are attached on demand through the block table.)
 *
 * For token n in [0, num_tokens): sequence s = token_seq[n], position p = token_pos[n].
 * p < 0 skips the token. Otherwise its slot is
 *     block_tables[s * max_blocks_per_seq + p / B] * B + p % B
 * and key[n][h][:] / value[n][h][:] are copied bit for bit into the key / value pool at
 * (slot / B, h, slot % B) for every KV head h.
 *
 *   key_cache, value_cache  device, pools in the layout above (written in place)
 *   key, value              device, [num_tokens][Hkv][d], c->dtype, contiguous
 *   block_tables            device int32 [num_seqs][max_blocks_per_seq], row-major
 *   token_seq, token_pos    device int32 [num_tokens]
 *   num_tokens = 0          returns PA_OK without launching
 * Caller contract (not checked on the device beyond clamping; pa_validate_writes counts
 * violations): distinct tokens map to distinct slots; block ids in [0, NB). A token whose
 * sequence is outside [0, num_seqs) or whose position is at or past max_blocks_per_seq * B is
 * skipped; a block id outside [0, NB) is clamped into range (no fault, but the write lands in the
 * wrong block).
 */
PA_API pa_status pa_reshape_and_cache(const pa_cache_desc* c, void* key_cache, void* value_cache,
                               const void* key, const void* value, const int32_t* block_tables,
                               int32_t num_seqs, int32_t max_blocks_per_seq,
                               const int32_t* token_seq, const int32_t* token_pos,
                               int32_t num_tokens, void* stream);

/*
 * pa_decode_workspace_bytes — bytes of device workspace pa_decode needs for these sizes.
 * partition_size 0 means the library's choice (the same one pa_decode makes: 512 tokens for
 * workgroups of one query head, 1024 when an even group size lets a workgroup serve 2 or 4
 * query heads). Returns 0 when
 * no workspace is needed (every context fits one partition) and (size_t)-1 for invalid sizes.
 * The size depends on c->flags: with PA_CACHE_SHARED_BLOCKS, 16-bit pools, head_dim 128 and more
 * than one partition, the share plan follows the partition states (16-byte aligned):
 * 3 * num_seqs * partitions + 4 int32s (the share map, two work lists and their counts).
 */
PA_API size_t pa_decode_workspace_bytes(const pa_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode — single-query (decode) attention of every sequence over its paged KV cache.
 * ([wiki] dense and block forms; [anal] §3 block-wise kernel and lookup pseudocode.)
 *
 * For sequence s with n = context_lens[s] tokens and query head h (KV head g = h / G with
 * G = num_q_heads / Hkv): token t in [0, n) is at physical block block_tables[s][t / B],
 * slot t % B;
 *     z_t = scale * dot(query[s][h], K_t),   out[s][h] = sum_t softmax(z)_t * V_t.
 * Slots at or past n in the last block and table entries past ceil(n / B) are never read.
 * n = 0 writes zeros. Accumulation is fp32; out is rounded to c->dtype (nearest even).
 *
 * Contexts longer than one partition are split into partitions of partition_size tokens
 * (a multiple of 16 and of B, at most PA_MAX_PARTITION_TOKENS; 0 = library choice). Each partition keeps
 * its softmax state (running max m, sum l, unnormalised output) in the workspace, and a second
 * kernel merges the states of each (sequence, head) with the usual max-rescaling.
 *
 *   key_cache, value_cache  device pools (layout above), read only
 *   out                     device [num_seqs][num_q_heads][d], c->dtype
 *   query                   device [num_seqs][num_q_heads][d], c->dtype
 *   block_tables            device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens            device int32 [num_seqs]
 *   scale                   softmax scale (1/sqrt(d) in the usual case)
 *   max_context_len         host-side upper bound of context_lens (sizes the grid; no
 *                           device-to-host copy is made); must be <= max_blocks_per_seq * B.
 *                           A context above it is truncated to it.
 *   workspace               device, >= pa_decode_workspace_bytes(...) bytes, 16-byte aligned
 *                           (may be NULL when that is 0); contents need no initialisation.
 * Errors: checked on the host before any HIP call (PA_ERR_NULL / SHAPE / UNSUPPORTED / ALIGN /
 * WORKSPACE); a failed launch gives PA_ERR_LAUNCH. num_seqs = 0 returns PA_OK. A block id
 * outside [0, NB) is clamped into range (no fault, but the result is then meaningless).
 */
PA_API pa_status pa_decode(const pa_cache_desc* c, const void* key_cache, const void* value_cache,
                    void* out, const void* query, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_q_heads, float scale, int32_t max_context_len,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * pa_decode_static — pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The partition states
 * live in a fixed device array of PA_STATIC_WORKSPACE_BYTES that the library itself holds on
 * every GPU it runs on (from the library's loading until the process ends) instead of in a
 * caller's workspace; the call allocates nothing.
 *
 * Arguments, results, checks and kernels are pa_decode's, without workspace / workspace_bytes.
 * Sizes for which pa_decode_workspace_bytes(...) exceeds PA_STATIC_WORKSPACE_BYTES give
 * PA_ERR_WORKSPACE, checked on the host before any HIP call. The call uses the array of the
 * calling thread's current device, and `stream` must belong to that device. Every call on one
 * device shares that device's array, which keeps the last call's partition states: calls that
 * overlap on one device (on two streams, or from two threads, at once) race, and the caller
 * must order them. The contents need no clearing (every partition state is written before it
 * is read). The array's device address is looked up once per device, on the first call that
 * needs it (hipGetSymbolAddress); a failed lookup gives PA_ERR_LAUNCH.
 */
#define PA_STATIC_WORKSPACE_BYTES (32u * 1024u * 1024u)
PA_API pa_status pa_decode_static(const pa_cache_desc* c, const void* key_cache,
                                  const void* value_cache, void* out, const void* query,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, float scale, int32_t max_context_len,
                                  int32_t partition_size, void* stream);

/*
 * The two stages pa_decode launches, exported separately (same arguments, same checks) so a
 * caller can time or interleave them: pa_decode_attention runs the per-partition attention
 * kernel (writing out directly for sequences that fit one partition, partition states
 * otherwise); pa_decode_reduce merges the partition states into out. pa_decode_reduce launches
 * nothing when every context fits one partition.
 */
PA_API pa_status pa_decode_attention(const pa_cache_desc* c, const void* key_cache,
                              const void* value_cache, void* out, const void* query,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                              float scale, int32_t max_context_len, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, void* stream);
PA_API pa_status pa_decode_reduce(const pa_cache_desc* c, const void* key_cache,
                           const void* value_cache, void* out, const void* query,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                           float scale, int32_t max_context_len, int32_t partition_size,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_contiguous — the same decode attention over a KV cache that is not paged: the
 * contiguous twin, kept to measure what paging costs. ([anal] §3 compares the paged kernel with
 * an ordinary one over contiguous keys and values and puts it about 20-26% slower.)
 *
 * There is no block table: logical block j of sequence s is physical block
 * s * max_blocks_per_seq + j of the pools (same layout, same partitions and merge as pa_decode),
 * so the result equals pa_decode's with block_tables[s][j] = s * max_blocks_per_seq + j.
 * Arguments as pa_decode without block_tables. Contiguous sequences never share blocks, so the
 * key/value tiles are always streamed; PA_CACHE_SHARED_BLOCKS gives PA_ERR_UNSUPPORTED.
 * num_seqs * max_blocks_per_seq > num_blocks gives PA_ERR_SHAPE.
 */
PA_API pa_status pa_decode_contiguous(const pa_cache_desc* c, const void* key_cache,
                               const void* value_cache, void* out, const void* query,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, float scale,
                               int32_t max_context_len, int32_t partition_size, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * pa_prefill — causal attention of many new query tokens per sequence over its paged KV cache
 * (a prompt, or a chunk of one, whose keys and values pa_reshape_and_cache has already written).
 * ([wiki] the dense causal form for a general query token i and its blocked form over the first
 *  ceil(i/B) blocks; pa_decode is the case of one query per sequence.)
 *
 * Sequence s owns query rows query_start[s] .. query_start[s+1]-1: its newest
 * q_len = query_start[s+1] - query_start[s] tokens, so with n = context_lens[s] cached tokens
 * (those q_len included) its query j sits at position p = n - q_len + j. For query head h (KV
 * head g = h / G):
 *     z_t = scale * dot(query[row][h], K_t) for t in [0, p],   out[row][h] = sum_t softmax(z)_t V_t
 * with token t at physical block block_tables[s][t / B], slot t % B. Nothing past position p is
 * read into the result; slots past n and table entries past ceil(n / B) are never read. Products
 * are formed on the matrix cores from the 16-bit inputs and summed in fp32; the softmax weights
 * are rounded to c->dtype before they multiply the values (as in the usual flash-attention
 * form); out is rounded to c->dtype (nearest even).
 *
 *   key_cache, value_cache  device pools (layout above), read only
 *   out, query              device [T][num_q_heads][d], c->dtype, T = query_start[num_seqs]
 *   block_tables            device int32 [num_seqs][max_blocks_per_seq]
 *   query_start             device int32 [num_seqs + 1], non-decreasing, query_start[0] = 0
 *   context_lens            device int32 [num_seqs]
 *   scale                   softmax scale, finite and > 0 (1/sqrt(d) in the usual case)
 *   max_query_len           host-side upper bound of every q_len (sizes the grid: one workgroup
 *                           per 128 queries of each (sequence, query head)); queries past it
 *                           are not computed and their rows of out are left as they were
 *   max_context_len         host-side upper bound of context_lens, <= max_blocks_per_seq * B;
 *                           a context above it is truncated to it
 * Supported: PA_F16 and PA_BF16 (PA_F32 gives PA_ERR_UNSUPPORTED), head_dim 64 or 128, block
 * sizes 8, 16, 32; PA_CACHE_SHARED_BLOCKS is accepted and changes nothing (tiles are always read
 * through the caches: every query tile of a sequence reads its blocks).
 * Errors: checked on the host before the launch (PA_ERR_NULL / SHAPE / UNSUPPORTED / ALIGN); a
 * failed launch gives PA_ERR_LAUNCH. num_seqs = 0 or max_query_len = 0 returns PA_OK.
 * Caller contract (not checked on the device beyond clamping): q_len <= n; a query whose
 * position would be negative (q_len > n) gets a zero row. A block id outside [0, NB) is clamped
 * into range (no fault, but the result is then meaningless). NaN in a query or in a key/value
 * inside a context gives an unspecified output row (the kernel does not propagate NaN); slots
 * past a context are never used, whatever they hold.
 */
PA_API pa_status pa_prefill(const pa_cache_desc* c, const void* key_cache, const void* value_cache,
                            void* out, const void* query, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* query_start,
                            const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                            float scale, int32_t max_query_len, int32_t max_context_len,
                            void* stream);

/*
 * pa_copy_blocks — duplicate whole physical blocks (copy-on-write).
 * ([anal] §4 and [dev]: a sharer about to write into a block whose reference count exceeds one
 *  gets a fresh block holding a copy of the old contents; [blog] ②.)
 *
 * For each pair k: block src_dst[2k] is copied to block src_dst[2k+1] in both pools: every KV
 * head and every slot, bit for bit.
 *   src_dst   device int32 [num_pairs][2]
 *   num_pairs = 0 returns PA_OK without launching
 * Caller contract (pa_validate_writes counts violations): destination ids are distinct and none
 * is also a source in the same call (otherwise the copies race). A pair with an id outside
 * [0, NB) is skipped.
 */
PA_API pa_status pa_copy_blocks(const pa_cache_desc* c, void* key_cache, void* value_cache,
                         const int32_t* src_dst, int32_t num_pairs, void* stream);

/*
 * pa_swap_blocks — copy whole blocks between two pools of the same shape, one of which may live
 * in host memory: the swap of a preempted sequence's blocks out to CPU memory and back
 * ([anal] §6: the evicted blocks move to a CPU block pool, bounded by the GPU's block count).
 *
 * For each pair k: block src_dst[2k] of the source pools (src_key, src_value) is copied to block
 * src_dst[2k+1] of the destination pools (dst_key, dst_value): every KV head and every slot, bit
 * for bit, by one kernel that reads or writes the host pool across the host link.
 *
 *   dst, src        descriptors of the two pool pairs: same dtype, num_kv_heads, head_dim and
 *                   block_size (else PA_ERR_SHAPE); num_blocks may differ
 *   dst_*, src_*    device memory or pinned host memory (hipHostMalloc), in the layout above;
 *                   each pointer is resolved on the host (hipPointerGetAttributes) to the
 *                   address the device uses, and memory the device cannot address (pageable
 *                   host memory) gives PA_ERR_UNSUPPORTED before anything is launched
 *   src_dst         int32 [num_pairs][2], device or pinned host memory; a pair with an id
 *                   outside its pool is skipped
 *   num_pairs = 0   returns PA_OK without launching
 * Caller contract: destination ids distinct, and a swap within one pool pair must not overlap a
 * source with a destination (the copies would race).
 */
PA_API pa_status pa_swap_blocks(const pa_cache_desc* dst, void* dst_key, void* dst_value,
                         const pa_cache_desc* src, const void* src_key, const void* src_value,
                         const int32_t* src_dst, int32_t num_pairs, void* stream);

/*
 * pa_validate_tables — count violations of the device-side caller contract of pa_decode,
 * pa_decode_contiguous, pa_prefill and pa_reshape_and_cache, without reading the pools.
 * ([anal] §2 and the lookup pseudocode: a logical block is resolved through the sequence's block
 *  table to a physical block of the pool; the kernels clamp a block id outside the pool instead of
 *  faulting, so a corrupt table would otherwise go unnoticed.)
 *
 * For each sequence s with n = context_lens[s], one violation is counted for each of:
 *   n < 0 or n > max_context_len (the attention calls would truncate it);
 *   each table entry block_tables[s][j], j < ceil(min(max(n, 0), max_context_len) / B) (the
 *     entries the attention calls read), outside [0, c->num_blocks);
 *   with query_start given: query_start[0] != 0 (counted once, for s = 0),
 *     query_start[s+1] < query_start[s], or q_len = query_start[s+1] - query_start[s] > n.
 * The count is written to *violations (device int32, 4-byte aligned); the library clears it
 * first with a kernel of its own, so the call can be captured in a graph. Entries past a
 * sequence's used range are not read. num_seqs * (max_blocks_per_seq + 3) must stay below 2^31
 * so that the count cannot overflow.
 *
 *   block_tables            device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens            device int32 [num_seqs]
 *   query_start             device int32 [num_seqs + 1], or NULL (decode: no query ranges)
 *   max_context_len         as passed to the attention call, <= max_blocks_per_seq * B
 *   violations              device int32 [1], written
 * Only c->block_size and c->num_blocks matter (the rest of *c is checked as everywhere).
 * Errors: checked on the host before any launch (PA_ERR_NULL / SHAPE / UNSUPPORTED / ALIGN); a
 * failed launch gives PA_ERR_LAUNCH. num_seqs = 0 writes 0.
 */
PA_API pa_status pa_validate_tables(const pa_cache_desc* c, const int32_t* block_tables,
                                    int32_t num_seqs, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, const int32_t* query_start,
                                    int32_t max_context_len, int32_t* violations, void* stream);

/*
 * pa_validate_writes — count violations of the write-race contract of pa_reshape_and_cache and
 * pa_copy_blocks on the device, without touching the pools.
 * ([blog] ② and the copy-on-write section of [dev]: a shared block is copied before a sharer
 *  writes into it precisely so that no two writers ever share a slot; [blog] §2: each new token
 *  owns one free slot of its sequence's last block.)
 *
 * Arguments as pa_reshape_and_cache (block_tables, num_seqs, max_blocks_per_seq, token_seq,
 * token_pos, num_tokens) and pa_copy_blocks (src_dst, num_pairs) of one step. Counted:
 *   for each token pa_reshape_and_cache writes (position >= 0, sequence in [0, num_seqs),
 *   position < max_blocks_per_seq * B):
 *     one if its table entry block_tables[s][p / B] lies outside [0, c->num_blocks);
 *     one if its slot (after the clamping that call applies) is also written by an earlier such
 *     token (k tokens on one slot count k - 1);
 *   for each pair pa_copy_blocks copies (both ids in [0, c->num_blocks)):
 *     one if its destination is also the destination of an earlier such pair;
 *     one if its destination is the source of any such pair, itself included.
 * The count is written to *violations (device int32, 4-byte aligned), which the library clears
 * first with a kernel of its own (no memset), so the call can be captured in a graph. The work
 * is quadratic (num_tokens^2 / 2 + num_pairs^2 comparisons on the device): a checker for tests and
 * debugging. block_tables / token_seq / token_pos may be NULL when num_tokens = 0, src_dst when
 * num_pairs = 0; num_tokens + num_pairs must stay below 2^30.
 * Errors: checked on the host before any launch (PA_ERR_NULL / SHAPE / UNSUPPORTED / ALIGN); a
 * failed launch gives PA_ERR_LAUNCH.
 */
PA_API pa_status pa_validate_writes(const pa_cache_desc* c, const int32_t* block_tables,
                                    int32_t num_seqs, int32_t max_blocks_per_seq,
                                    const int32_t* token_seq, const int32_t* token_pos,
                                    int32_t num_tokens, const int32_t* src_dst, int32_t num_pairs,
                                    int32_t* violations, void* stream);

/*
 * pa_measure_tile_read — measurement only: the bandwidth reference of the decode access pattern.
 * ([anal] §2 and §5: blocks sit wherever the pool had room, and decode attention is bound by
 *  reading them.)
 *
 * Reads tiles tiles[0..num_tiles) — tile t is bytes [t * tile_bytes, (t + 1) * tile_bytes) — of
 * both pool_a and pool_b, with the attention kernel's loads (non-temporal 16-byte wave loads,
 * 1 KiB contiguous per instruction), kMeasureTilesPerWave = 32 consecutive entries of `tiles`
 * per wavefront, and writes to sink[w] the XOR of every 32-bit word wavefront w read (so the
 * reads cannot be dropped, and a test can check them). Timing it over as many bytes as a decode
 * step reads, in a random tile order, gives what plain reads of that pattern and size reach.
 *   pool_a, pool_b  device, at least (max tile index + 1) * tile_bytes bytes each
 *   tiles           device int32 [num_tiles], tile indices (not checked against the pools)
 *   tile_bytes      a multiple of 1024, at most 65536
 *   sink            device uint32 [ceil(num_tiles / 32)]
 * Errors: checked on the host before the launch (PA_ERR_NULL / SHAPE / ALIGN); a failed launch
 * gives PA_ERR_LAUNCH. num_tiles = 0 returns PA_OK.
 */
PA_API pa_status pa_measure_tile_read(const void* pool_a, const void* pool_b,
                                      const int32_t* tiles, int32_t num_tiles,
                                      int32_t tile_bytes, uint32_t* sink, void* stream);

/* Static description of a status code (never NULL; "unknown status" for a value that is not a
 * pa_status). The code is taken as a plain int so that any value a caller passes is defined. */
PA_API const char* pa_status_string(int status);

/* PA_ABI_VERSION of the built library. */
PA_API int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
