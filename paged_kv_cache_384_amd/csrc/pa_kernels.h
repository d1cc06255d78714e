// Internal interface between the C ABI (pa_api.cpp) and the HIP kernels. Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum class DType : int { F32 = 0, F16 = 1, BF16 = 2 };

constexpr int kGroupTokens = 16;       // tokens one wave-wide key load covers (a 16-token group)
constexpr int kMaxPartitionTokens = 2048;
constexpr int kDecodeThreads = 256;    // four 64-lane wavefronts per attention workgroup
constexpr int kReduceThreads = 256;    // threads of a partition-merge workgroup
constexpr int kValidateThreads = 256;  // threads of a pa_validate_writes workgroup

struct CacheWriteArgs {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const uint8_t* key;
  const uint8_t* value;
  const int32_t* block_tables;
  const int32_t* token_seq;
  const int32_t* token_pos;
  int32_t num_tokens;
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t num_kv_heads;
};

// Whole-block copies from (src_k, src_v) to (dst_k, dst_v): the same pools for copy-on-write
// copies, a device pool and a pinned host pool (by its device address) for swaps.
struct CopyArgs {
  const uint8_t* src_k;
  const uint8_t* src_v;
  uint8_t* dst_k;
  uint8_t* dst_v;
  const int32_t* pairs;  // [num_pairs][2] (source block, destination block)
  int32_t num_pairs;
  int32_t src_num_blocks;
  int32_t dst_num_blocks;
  int64_t block_bytes;  // bytes of one physical block in one pool (all KV heads)
};

// Table and length checks of pa_validate_tables: one workgroup per sequence.
struct ValidateArgs {
  const int32_t* block_tables;  // [num_seqs][max_blocks]
  const int32_t* context_lens;  // [num_seqs]
  const int32_t* query_start;   // [num_seqs + 1] or null
  int32_t* violations;          // [1]
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t block_size;
  int32_t max_ctx;
};

// Write-race checks of pa_validate_writes: cache-write tokens (as CacheWriteArgs resolves them)
// and copy pairs, each compared with the others.
struct ValidateWritesArgs {
  const int32_t* block_tables;  // [num_seqs][max_blocks]
  const int32_t* token_seq;     // [num_tokens]
  const int32_t* token_pos;     // [num_tokens]
  const int32_t* pairs;         // [num_pairs][2]
  int32_t* violations;          // [1]
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t num_tokens;
  int32_t num_pairs;
  int32_t num_blocks;
  int32_t block_size;
};

// pa_measure_tile_read: tiles of two pools read in a given order.
constexpr int kMeasureTilesPerWave = 32;
struct MeasureArgs {
  const uint8_t* pool_a;
  const uint8_t* pool_b;
  const int32_t* tiles;  // [num_tiles] tile indices into both pools
  uint32_t* sink;        // [ceil(num_tiles / kMeasureTilesPerWave)] XOR of the words read
  int64_t num_tiles;
  int32_t tile_bytes;
};

// One launch of the attention stage covers every (KV head, sequence, head group, partition).
struct DecodeArgs {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  uint8_t* out;
  const uint8_t* query;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_m;    // [S][Hq][NP] running max (log2 domain)
  float* ws_l;    // [S][Hq][NP] sum of exp2(z - m)
  float* ws_acc;  // [S][Hq][NP][D] unnormalised output
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t group;        // query heads per KV head
  int32_t heads_per_wg; // query heads one workgroup handles (1, 2 or 4)
  int32_t head_groups;  // group / heads_per_wg
  int32_t part_tokens;  // partition size in tokens (multiple of 16)
  int32_t num_parts;    // partitions of the longest context
  int32_t max_ctx;
  float scale_log2;     // scale * log2(e): scores are kept in the base-2 domain
  bool stream_kv;       // read key/value tiles with non-temporal (streaming) loads
  bool paged;           // false: no table, sequence s's block j is physical block
                        // s * max_blocks + j (the contiguous twin)
  // The share plan (all nullptr: no sharing). share_map [S][NP], entry (s, p): 1 when sequence
  // s computes partition p itself, n >= 2 when s leads a group of n sequences s .. s+n-1 whose
  // partition p is full and made of the same physical blocks (computed once for all of them),
  // 0 when s is in such a group led by an earlier sequence. share_list: the items s * NP + p
  // sequences compute themselves (partitions inside their contexts, and partition 0 of an
  // empty context), then from offset S * NP the items of group leaders; share_counts: their
  // numbers (own, shared), counted up by the plan kernel from zero.
  int32_t* share_map;
  int32_t* share_list;
  int32_t* share_counts;
};

// Sequences one shared-partition workgroup serves; groups are cut at multiples of this index.
constexpr int kShareMax = 8;

constexpr int kPrefillThreads = 256;       // four wavefronts per prefill workgroup
constexpr int kPrefillTileQueries = 128;  // queries one prefill workgroup owns
constexpr int kPrefillTileTokens = 64;    // tokens per key/value tile of the prefill loop

// One launch covers every (query tile of kPrefillTileQueries, sequence, query head).
struct PrefillArgs {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  uint8_t* out;
  const uint8_t* query;  // [T][Hq][D], rows query_start[s] .. query_start[s+1]-1 of sequence s
  const int32_t* block_tables;
  const int32_t* query_start;  // [num_seqs + 1]
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t max_query_len;
  int32_t max_ctx;
  int32_t group;        // query heads per KV head
  int32_t q_tiles;      // ceil(max_query_len / kPrefillTileQueries)
  int32_t seq_major;    // 1: units are (sequence, KV head); 0: (query tile, sequence, KV head)
  int32_t num_units;    // units of workgroups that read the same key/value tiles
  int32_t unit_wgs;     // workgroups per unit: group, times q_tiles when seq_major
  int32_t num_wgs;      // num_units rounded up to a multiple of 8 (the XCDs), times unit_wgs
  float scale_log2;     // scale * log2(e)
};

// Units are sequence-major when every sequence has at most this many query tiles.
constexpr int kPrefillSeqMajorTiles = 4;

// Each launcher returns the hipError_t of its launch (hipSuccess when nothing was launched).
hipError_t launch_reshape_and_cache(DType dt, int head_dim, int block_size,
                                    const CacheWriteArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);
hipError_t launch_validate(const ValidateArgs& a, hipStream_t stream);
hipError_t launch_validate_writes(const ValidateWritesArgs& a, hipStream_t stream);
hipError_t launch_tile_read(const MeasureArgs& a, hipStream_t stream);
hipError_t launch_decode_attention_b8(DType dt, int head_dim, const DecodeArgs& a,
                                      hipStream_t stream);
hipError_t launch_decode_attention_b16(DType dt, int head_dim, const DecodeArgs& a,
                                       hipStream_t stream);
hipError_t launch_decode_attention_b32(DType dt, int head_dim, const DecodeArgs& a,
                                       hipStream_t stream);
hipError_t launch_decode_reduce(DType dt, int head_dim, const DecodeArgs& a, hipStream_t stream);
// the share plan (see DecodeArgs), then the attention over its two lists (16-bit pools with
// head_dim 128 only), which replaces the grid launch of launch_decode_attention_b*
hipError_t launch_share_plan(const DecodeArgs& a, int block_size, hipStream_t stream);
hipError_t launch_decode_attention_shared_b8(DType dt, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_attention_shared_b16(DType dt, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_attention_shared_b32(DType dt, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(DType dt, int head_dim, int block_size, const PrefillArgs& a,
                          hipStream_t stream);

}  // namespace pa
