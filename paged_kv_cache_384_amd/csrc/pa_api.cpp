// C ABI of the paged attention library: argument checks on the host, partition choice, dispatch.
// Every check runs before any launch; besides the launches and hipGetLastError the only HIP calls
// are pa_swap_blocks' pointer query (hipPointerGetAttributes) and pa_decode_static's one-time
// lookup of its device array (hipGetDevice, hipGetSymbolAddress). No device memory is allocated.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/pa.h"
#include "pa_kernels.h"

// pa_decode_static's partition-state array. Each GPU the library runs on holds its own copy
// (at its own address) until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the address scratch_address() looked up for the current device.
static __device__ __align__(256) uint8_t scratch[PA_STATIC_WORKSPACE_BYTES];

namespace {

using pa::DType;

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the calling thread's current device, looked up once per
// device (with that device current); nullptr if the lookup fails.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

constexpr int kStageAttention = 1;
constexpr int kStageReduce = 2;

// A dispatch's grid is at most 2^32 - 1 work-items; every kernel here runs 256-thread
// workgroups, so a launch may have at most this many of them.
constexpr int64_t kMaxWorkgroups = ((int64_t{1} << 32) - 1) / 256;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elem_size(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }

pa_status check_desc(const pa_cache_desc* c) {
  if (c == nullptr) return PA_ERR_NULL;
  if (c->dtype != PA_F32 && c->dtype != PA_F16 && c->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32) return PA_ERR_UNSUPPORTED;
  if ((c->flags & ~PA_CACHE_SHARED_BLOCKS) != 0) return PA_ERR_UNSUPPORTED;
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return PA_ERR_SHAPE;
  return PA_OK;
}

int64_t tile_bytes(const pa_cache_desc* c) {
  return static_cast<int64_t>(c->block_size) * c->head_dim * elem_size(c->dtype);
}

// Partitions are whole 16-token groups and whole blocks: multiples of max(16, B).
int32_t partition_quantum(const pa_cache_desc* c) {
  return c->block_size > pa::kGroupTokens ? c->block_size : pa::kGroupTokens;
}

// Partition size when the caller passes 0. One partition when the longest context fits in one
// default partition; otherwise default partitions: 512 tokens (32 groups: eight per wavefront)
// for single-head workgroups, which keeps every workgroup's key/value stream long enough to
// amortise its setup while giving the launch enough independent workgroups for 256 CUs, and
// 1024 for workgroups that serve several query heads of one KV head, whose setup (query loads,
// cross-wavefront merge and partition state per head) is several times larger. Measured on
// MI355X, attention kernel alone: OPT-13B-shape MHA 512 / 1024 / 2048 -> 0.79 / 0.76 / 0.72 of
// HBM peak; GQA (4 heads per workgroup) 0.70 / 0.73 / 0.72.
int32_t choose_partition(const pa_cache_desc* c, int32_t max_context_len, int32_t heads_per_wg,
                         int32_t requested) {
  if (requested > 0) return requested;
  const int32_t def = heads_per_wg > 1 ? 1024 : 512;
  const int32_t q = partition_quantum(c);
  if (max_context_len <= def) {
    const int32_t p = (max_context_len + q - 1) / q * q;
    return p < q ? q : p;
  }
  return def;
}

struct DecodePlan {
  int32_t part_tokens;
  int32_t num_parts;
  int32_t heads_per_wg;
  bool share;             // partitions shared by consecutive sequences get one workgroup
  size_t share_offset;    // byte offset of the share map in the workspace
  size_t workspace_bytes;
};

pa_status plan_decode(const pa_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_context_len, int32_t partition_size, DecodePlan* plan) {
  pa_status st = check_desc(c);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (max_context_len < 0) return PA_ERR_SHAPE;
  if (partition_size < 0 || partition_size % partition_quantum(c) != 0 ||
      partition_size > pa::kMaxPartitionTokens)
    return PA_ERR_SHAPE;
  const int32_t group = num_q_heads / c->num_kv_heads;
  const int32_t nh = group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
  const int32_t part = choose_partition(c, max_context_len, nh, partition_size);
  const int32_t np = max_context_len <= part ? 1 : (max_context_len + part - 1) / part;
  const int64_t wgs = static_cast<int64_t>(c->num_kv_heads) * num_seqs * (group / nh) * np;
  if (wgs > kMaxWorkgroups) return PA_ERR_SHAPE;
  // the merge runs one workgroup (or one wavefront) per (sequence, query head)
  if (np > 1 && static_cast<int64_t>(num_seqs) * num_q_heads > kMaxWorkgroups) return PA_ERR_SHAPE;
  plan->part_tokens = part;
  plan->num_parts = np;
  plan->heads_per_wg = nh;
  plan->workspace_bytes =
      np > 1 ? static_cast<size_t>(num_seqs) * num_q_heads * np * (c->head_dim + 2) * sizeof(float)
             : 0;
  // Shared blocks declared, several partitions, and the matrix-core score path (16-bit pools,
  // head_dim 128): the share plan after the partition states, 16-byte aligned: the map
  // ([S][NP] int32), the two work lists (2 * S * NP int32) and their two counts
  plan->share = (c->flags & PA_CACHE_SHARED_BLOCKS) != 0 && np > 1 && c->head_dim == 128 &&
                (c->dtype == PA_F16 || c->dtype == PA_BF16);
  plan->share_offset = (plan->workspace_bytes + 15) / 16 * 16;
  if (plan->share) {
    // the lists' unit counts (items x KV heads x head groups) are int64 in the kernels; the
    // items themselves (s * NP + p) must fit int32
    if (static_cast<int64_t>(num_seqs) * np > INT32_MAX / 4) return PA_ERR_SHAPE;
    plan->workspace_bytes =
        plan->share_offset + (3 * static_cast<size_t>(num_seqs) * np + 4) * sizeof(int32_t);
  }
  return PA_OK;
}

// paged = false: the contiguous twin (no table; sequence s's block j is physical block
// s * max_blocks_per_seq + j), block_tables unused.
// use_static: the partition states go to the library's own device array (pa_decode_static)
// instead of the caller's workspace.
pa_status decode_impl(int stages, bool paged, const pa_cache_desc* c, const void* key_cache,
                      const void* value_cache, void* out, const void* query,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                      float scale, int32_t max_context_len, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, void* stream,
                      bool use_static = false) {
  DecodePlan plan;
  pa_status st = plan_decode(c, num_seqs, num_q_heads, max_context_len, partition_size, &plan);
  if (st != PA_OK) return st;
  if (max_blocks_per_seq <= 0 ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * c->block_size)
    return PA_ERR_SHAPE;
  if (!paged) {
    // contiguous sequences cannot share blocks, and every sequence's span must fit the pool
    if (c->flags & PA_CACHE_SHARED_BLOCKS) return PA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(num_seqs) * max_blocks_per_seq > c->num_blocks) return PA_ERR_SHAPE;
  }
  if (num_seqs == 0) return PA_OK;
  if (!key_cache || !value_cache || !out || !query || (paged && !block_tables) || !context_lens)
    return PA_ERR_NULL;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(out, 16) ||
      !aligned(query, 16) || (paged && !aligned(block_tables, 4)) || !aligned(context_lens, 4))
    return PA_ERR_ALIGN;
  if (use_static && plan.workspace_bytes > PA_STATIC_WORKSPACE_BYTES) return PA_ERR_WORKSPACE;
  if (plan.workspace_bytes > 0 && !use_static) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
  }
  if (plan.workspace_bytes > 0 && use_static) {
    workspace = scratch_address();
    if (workspace == nullptr) return PA_ERR_LAUNCH;
    workspace_bytes = PA_STATIC_WORKSPACE_BYTES;
  }

  pa::DecodeArgs a;
  a.k_pool = static_cast<const uint8_t*>(key_cache);
  a.v_pool = static_cast<const uint8_t*>(value_cache);
  a.out = static_cast<uint8_t*>(out);
  a.query = static_cast<const uint8_t*>(query);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const int64_t states = static_cast<int64_t>(num_seqs) * num_q_heads * plan.num_parts;
  float* ws = static_cast<float*>(workspace);
  a.ws_acc = plan.workspace_bytes ? ws : nullptr;
  a.ws_m = plan.workspace_bytes ? ws + states * c->head_dim : nullptr;
  a.ws_l = plan.workspace_bytes ? ws + states * (c->head_dim + 1) : nullptr;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = c->num_kv_heads;
  a.num_blocks = c->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.group = num_q_heads / c->num_kv_heads;
  a.heads_per_wg = plan.heads_per_wg;
  a.head_groups = a.group / plan.heads_per_wg;
  a.part_tokens = plan.part_tokens;
  a.num_parts = plan.num_parts;
  a.max_ctx = max_context_len;
  a.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  a.stream_kv = (c->flags & PA_CACHE_SHARED_BLOCKS) == 0;
  a.paged = paged;
  a.share_map = nullptr;
  a.share_list = nullptr;
  a.share_counts = nullptr;
  if (plan.share && paged) {
    const int64_t items = static_cast<int64_t>(num_seqs) * plan.num_parts;
    a.share_map =
        reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + plan.share_offset);
    a.share_list = a.share_map + items;
    a.share_counts = a.share_list + 2 * items;
  }

  const DType dt = static_cast<DType>(c->dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (stages & kStageAttention) {
    hipError_t e;
    if (a.share_map != nullptr) {
      // the share plan, then the attention over its two lists
      e = pa::launch_share_plan(a, c->block_size, s);
      if (e == hipSuccess) {
        switch (c->block_size) {
          case 8: e = pa::launch_decode_attention_shared_b8(dt, a, s); break;
          case 32: e = pa::launch_decode_attention_shared_b32(dt, a, s); break;
          default: e = pa::launch_decode_attention_shared_b16(dt, a, s); break;
        }
      }
    } else {
      switch (c->block_size) {
        case 8: e = pa::launch_decode_attention_b8(dt, c->head_dim, a, s); break;
        case 32: e = pa::launch_decode_attention_b32(dt, c->head_dim, a, s); break;
        default: e = pa::launch_decode_attention_b16(dt, c->head_dim, a, s); break;
      }
    }
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  if (stages & kStageReduce) {
    if (pa::launch_decode_reduce(dt, c->head_dim, a, s) != hipSuccess) return PA_ERR_LAUNCH;
  }
  return PA_OK;
}

// The address a kernel uses for `p`: device memory as it is, pinned host memory through its
// device mapping; nullptr for memory the device cannot address (ordinary pageable host memory).
void* device_address(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the error the query left for pageable memory
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) return const_cast<void*>(p);
  // pinned host memory: the query reports the address itself as the host address and a device
  // mapping; anything else is refused rather than guessed
  if (attr.type != hipMemoryTypeHost || attr.hostPointer != p) return nullptr;
  return attr.devicePointer;
}

}  // namespace

extern "C" {

pa_status pa_reshape_and_cache(const pa_cache_desc* c, void* key_cache, void* value_cache,
                               const void* key, const void* value, const int32_t* block_tables,
                               int32_t num_seqs, int32_t max_blocks_per_seq,
                               const int32_t* token_seq, const int32_t* token_pos,
                               int32_t num_tokens, void* stream) {
  pa_status st = check_desc(c);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (num_seqs <= 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (static_cast<int64_t>(max_blocks_per_seq) * c->block_size > INT32_MAX) return PA_ERR_SHAPE;
  if (!key_cache || !value_cache || !key || !value || !block_tables || !token_seq || !token_pos)
    return PA_ERR_NULL;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(key, 16) ||
      !aligned(value, 16) || !aligned(block_tables, 4) || !aligned(token_seq, 4) ||
      !aligned(token_pos, 4))
    return PA_ERR_ALIGN;
  // one thread per 16-byte piece of every token's heads, 256 per workgroup
  const int64_t pieces = static_cast<int64_t>(num_tokens) * c->num_kv_heads * c->head_dim *
                         elem_size(c->dtype) / 16;
  if ((pieces + 255) / 256 > kMaxWorkgroups) return PA_ERR_SHAPE;
  pa::CacheWriteArgs a;
  a.k_pool = static_cast<uint8_t*>(key_cache);
  a.v_pool = static_cast<uint8_t*>(value_cache);
  a.key = static_cast<const uint8_t*>(key);
  a.value = static_cast<const uint8_t*>(value);
  a.block_tables = block_tables;
  a.token_seq = token_seq;
  a.token_pos = token_pos;
  a.num_tokens = num_tokens;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = c->num_blocks;
  a.num_kv_heads = c->num_kv_heads;
  if (pa::launch_reshape_and_cache(static_cast<DType>(c->dtype), c->head_dim, c->block_size, a,
                                   static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

size_t pa_decode_workspace_bytes(const pa_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context_len, int32_t partition_size) {
  DecodePlan plan;
  if (plan_decode(c, num_seqs, num_q_heads, max_context_len, partition_size, &plan) != PA_OK)
    return static_cast<size_t>(-1);
  return plan.workspace_bytes;
}

pa_status pa_decode(const pa_cache_desc* c, const void* key_cache, const void* value_cache,
                    void* out, const void* query, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_q_heads, float scale, int32_t max_context_len,
                    int32_t partition_size, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_impl(kStageAttention | kStageReduce, true, c, key_cache, value_cache, out, query,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale,
                     max_context_len, partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_static(const pa_cache_desc* c, const void* key_cache,
                           const void* value_cache, void* out, const void* query,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                           float scale, int32_t max_context_len, int32_t partition_size,
                           void* stream) {
  return decode_impl(kStageAttention | kStageReduce, true, c, key_cache, value_cache, out, query,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale,
                     max_context_len, partition_size, nullptr, 0, stream, true);
}

pa_status pa_decode_attention(const pa_cache_desc* c, const void* key_cache,
                              const void* value_cache, void* out, const void* query,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                              float scale, int32_t max_context_len, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kStageAttention, true, c, key_cache, value_cache, out, query, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale,
                     max_context_len, partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_reduce(const pa_cache_desc* c, const void* key_cache,
                           const void* value_cache, void* out, const void* query,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                           float scale, int32_t max_context_len, int32_t partition_size,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kStageReduce, true, c, key_cache, value_cache, out, query, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale,
                     max_context_len, partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_decode_contiguous(const pa_cache_desc* c, const void* key_cache,
                               const void* value_cache, void* out, const void* query,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, float scale,
                               int32_t max_context_len, int32_t partition_size, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return decode_impl(kStageAttention | kStageReduce, false, c, key_cache, value_cache, out, query,
                     nullptr, max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale,
                     max_context_len, partition_size, workspace, workspace_bytes, stream);
}

pa_status pa_prefill(const pa_cache_desc* c, const void* key_cache, const void* value_cache,
                     void* out, const void* query, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* query_start,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                     float scale, int32_t max_query_len, int32_t max_context_len, void* stream) {
  pa_status st = check_desc(c);
  if (st != PA_OK) return st;
  if (c->dtype == PA_F32) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!(scale > 0.0f) || scale == INFINITY) return PA_ERR_SHAPE;  // also rejects NaN
  if (max_query_len < 0 || max_context_len < 0 || max_blocks_per_seq <= 0 ||
      static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * c->block_size)
    return PA_ERR_SHAPE;
  const int64_t tiles = (static_cast<int64_t>(max_query_len) + pa::kPrefillTileQueries - 1) /
                        pa::kPrefillTileQueries;
  const int64_t group = num_q_heads / c->num_kv_heads;
  const bool seq_major = tiles <= pa::kPrefillSeqMajorTiles;
  const int64_t units = (seq_major ? 1 : tiles) * num_seqs * c->num_kv_heads;
  const int64_t unit_wgs = (seq_major ? tiles : 1) * group;
  const int64_t wgs = (units + 7) / 8 * 8 * unit_wgs;
  if (wgs > kMaxWorkgroups) return PA_ERR_SHAPE;
  if (wgs == 0) return PA_OK;
  if (!key_cache || !value_cache || !out || !query || !block_tables || !query_start ||
      !context_lens)
    return PA_ERR_NULL;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(out, 16) ||
      !aligned(query, 16) || !aligned(block_tables, 4) || !aligned(query_start, 4) ||
      !aligned(context_lens, 4))
    return PA_ERR_ALIGN;
  pa::PrefillArgs a;
  a.k_pool = static_cast<const uint8_t*>(key_cache);
  a.v_pool = static_cast<const uint8_t*>(value_cache);
  a.out = static_cast<uint8_t*>(out);
  a.query = static_cast<const uint8_t*>(query);
  a.block_tables = block_tables;
  a.query_start = query_start;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = c->num_kv_heads;
  a.num_blocks = c->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.max_query_len = max_query_len;
  a.max_ctx = max_context_len;
  a.group = static_cast<int32_t>(group);
  a.q_tiles = static_cast<int32_t>(tiles);
  a.seq_major = seq_major ? 1 : 0;
  a.num_units = static_cast<int32_t>(units);
  a.unit_wgs = static_cast<int32_t>(unit_wgs);
  a.num_wgs = static_cast<int32_t>(wgs);
  a.scale_log2 = scale * 1.4426950408889634f;  // log2(e)
  if (pa::launch_prefill(static_cast<DType>(c->dtype), c->head_dim, c->block_size, a,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_copy_blocks(const pa_cache_desc* c, void* key_cache, void* value_cache,
                         const int32_t* src_dst, int32_t num_pairs, void* stream) {
  pa_status st = check_desc(c);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !src_dst) return PA_ERR_NULL;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(src_dst, 4))
    return PA_ERR_ALIGN;
  pa::CopyArgs a;
  a.src_k = a.dst_k = static_cast<uint8_t*>(key_cache);
  a.src_v = a.dst_v = static_cast<uint8_t*>(value_cache);
  a.pairs = src_dst;
  a.num_pairs = num_pairs;
  a.src_num_blocks = a.dst_num_blocks = c->num_blocks;
  a.block_bytes = tile_bytes(c) * c->num_kv_heads;
  const int64_t chunks = (a.block_bytes / 16 + 2047) / 2048;
  if (chunks * num_pairs > kMaxWorkgroups) return PA_ERR_SHAPE;
  if (pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_validate_tables(const pa_cache_desc* c, const int32_t* block_tables,
                             int32_t num_seqs, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, const int32_t* query_start,
                             int32_t max_context_len, int32_t* violations, void* stream) {
  pa_status st = check_desc(c);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_context_len < 0) return PA_ERR_SHAPE;
  if (static_cast<int64_t>(max_context_len) >
      static_cast<int64_t>(max_blocks_per_seq) * c->block_size)
    return PA_ERR_SHAPE;
  if (static_cast<int64_t>(num_seqs) * (static_cast<int64_t>(max_blocks_per_seq) + 3) >=
      (int64_t{1} << 31) || num_seqs > kMaxWorkgroups)
    return PA_ERR_SHAPE;
  if (!violations) return PA_ERR_NULL;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PA_ERR_NULL;
  if (!aligned(violations, 4) || !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      !aligned(query_start, 4))
    return PA_ERR_ALIGN;
  pa::ValidateArgs a;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.violations = violations;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = c->num_blocks;
  a.block_size = c->block_size;
  a.max_ctx = max_context_len;
  if (pa::launch_validate(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_validate_writes(const pa_cache_desc* c, const int32_t* block_tables,
                             int32_t num_seqs, int32_t max_blocks_per_seq,
                             const int32_t* token_seq, const int32_t* token_pos,
                             int32_t num_tokens, const int32_t* src_dst, int32_t num_pairs,
                             int32_t* violations, void* stream) {
  pa_status st = check_desc(c);
  if (st != PA_OK) return st;
  if (num_tokens < 0 || num_pairs < 0) return PA_ERR_SHAPE;
  // each token counts at most 2, each pair at most 2: the count stays below 2^31
  if (static_cast<int64_t>(num_tokens) + num_pairs >= (int64_t{1} << 30)) return PA_ERR_SHAPE;
  if (num_tokens > 0 &&
      (num_seqs <= 0 || max_blocks_per_seq <= 0 ||
       static_cast<int64_t>(max_blocks_per_seq) * c->block_size > INT32_MAX))
    return PA_ERR_SHAPE;
  if (!violations) return PA_ERR_NULL;
  if (num_tokens > 0 && (!block_tables || !token_seq || !token_pos)) return PA_ERR_NULL;
  if (num_pairs > 0 && !src_dst) return PA_ERR_NULL;
  if (!aligned(violations, 4) || !aligned(block_tables, 4) || !aligned(token_seq, 4) ||
      !aligned(token_pos, 4) || !aligned(src_dst, 4))
    return PA_ERR_ALIGN;
  pa::ValidateWritesArgs a;
  a.block_tables = block_tables;
  a.token_seq = token_seq;
  a.token_pos = token_pos;
  a.pairs = src_dst;
  a.violations = violations;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.num_tokens = num_tokens;
  a.num_pairs = num_pairs;
  a.num_blocks = c->num_blocks;
  a.block_size = c->block_size;
  if (pa::launch_validate_writes(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_swap_blocks(const pa_cache_desc* dst, void* dst_key, void* dst_value,
                         const pa_cache_desc* src, const void* src_key, const void* src_value,
                         const int32_t* src_dst, int32_t num_pairs, void* stream) {
  pa_status st = check_desc(dst);
  if (st != PA_OK) return st;
  if ((st = check_desc(src)) != PA_OK) return st;
  if (dst->dtype != src->dtype || dst->num_kv_heads != src->num_kv_heads ||
      dst->head_dim != src->head_dim || dst->block_size != src->block_size)
    return PA_ERR_SHAPE;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!dst_key || !dst_value || !src_key || !src_value || !src_dst) return PA_ERR_NULL;
  if (!aligned(dst_key, 16) || !aligned(dst_value, 16) || !aligned(src_key, 16) ||
      !aligned(src_value, 16) || !aligned(src_dst, 4))
    return PA_ERR_ALIGN;
  pa::CopyArgs a;
  a.dst_k = static_cast<uint8_t*>(device_address(dst_key));
  a.dst_v = static_cast<uint8_t*>(device_address(dst_value));
  a.src_k = static_cast<const uint8_t*>(device_address(src_key));
  a.src_v = static_cast<const uint8_t*>(device_address(src_value));
  a.pairs = static_cast<const int32_t*>(device_address(src_dst));
  if (!a.dst_k || !a.dst_v || !a.src_k || !a.src_v || !a.pairs) return PA_ERR_UNSUPPORTED;
  a.num_pairs = num_pairs;
  a.src_num_blocks = src->num_blocks;
  a.dst_num_blocks = dst->num_blocks;
  a.block_bytes = tile_bytes(src) * src->num_kv_heads;
  const int64_t chunks = (a.block_bytes / 16 + 2047) / 2048;
  if (chunks * num_pairs > kMaxWorkgroups) return PA_ERR_SHAPE;
  if (pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_measure_tile_read(const void* pool_a, const void* pool_b, const int32_t* tiles,
                               int32_t num_tiles, int32_t tile_bytes, uint32_t* sink,
                               void* stream) {
  if (num_tiles < 0 || tile_bytes <= 0 || tile_bytes % 1024 != 0 || tile_bytes > 65536)
    return PA_ERR_SHAPE;
  if (num_tiles == 0) return PA_OK;
  if (!pool_a || !pool_b || !tiles || !sink) return PA_ERR_NULL;
  if (!aligned(pool_a, 16) || !aligned(pool_b, 16) || !aligned(tiles, 4) || !aligned(sink, 4))
    return PA_ERR_ALIGN;
  const int64_t waves = (static_cast<int64_t>(num_tiles) + pa::kMeasureTilesPerWave - 1) /
                        pa::kMeasureTilesPerWave;
  if ((waves + 3) / 4 > kMaxWorkgroups) return PA_ERR_SHAPE;
  pa::MeasureArgs a;
  a.pool_a = static_cast<const uint8_t*>(pool_a);
  a.pool_b = static_cast<const uint8_t*>(pool_b);
  a.tiles = tiles;
  a.sink = sink;
  a.num_tiles = num_tiles;
  a.tile_bytes = tile_bytes;
  if (pa::launch_tile_read(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "a size is out of range or sizes are inconsistent";
    case PA_ERR_UNSUPPORTED:
      return "unsupported configuration (dtype, head_dim, block_size, flags) or memory the device "
             "cannot address";
    case PA_ERR_ALIGN: return "a pointer is not aligned (16 bytes for data, 4 for int32 arrays)";
    case PA_ERR_WORKSPACE: return "workspace missing or smaller than pa_decode_workspace_bytes()";
    case PA_ERR_LAUNCH: return "the HIP runtime reported a launch error";
  }
  return "unknown status";
}

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
