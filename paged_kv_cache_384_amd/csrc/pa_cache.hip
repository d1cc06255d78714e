// Cache-side kernels: writing new tokens into their slots and copying whole blocks.
//
// Sources (page title, section):
//   "PagedAttention 논문 쉽게 읽기" (iplexlaw.co.kr), §2: a new token's key/value goes into the free
//   slot of its sequence's last block, found through the block table; ②: a shared block about
//   to be written is copied first.
//   "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리" (ryotta.opik.net), §4 copy-on-write;
//   "추론 엔진에서의 메모리 가상화" (molayo1419.me), copy-on-write: fresh block, copy, remap.
#include "pa_device.h"

namespace pa {

// One thread per 16-byte piece of a new token's key (and the same piece of its value): the
// pieces of all tokens are numbered token-major, so a workgroup of 256 threads covers whole
// tokens or parts of one, whatever the head count. Piece q of KV head h holds elements
// [q*Epp, q*Epp + Epp) of that head's vector. In the value tile it goes to row `slot`, byte
// q*16; in the key tile to chunk row q/4 (64-byte chunks = 4 pieces), slot `slot`, byte (q%4)*16
// of that slot's 64-byte segment. The payload is loaded before the slot is looked up, so the
// table read and the payload load are in flight together.
template <DType dt, int D, int B>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(CacheWriteArgs a) {
  using G = TileGeom<dt, D, B>;
  constexpr int kPieces = G::kPiecesPerRow;
  const int per_token = a.num_kv_heads * kPieces;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(a.num_tokens) * per_token) return;
  const int n = static_cast<int>(i / per_token);
  const int r = static_cast<int>(i % per_token);
  const int h = r / kPieces;
  const int q = r % kPieces;
  const int64_t src = i * 16;  // token n, head h, piece q of the [T][Hkv][D] inputs
  const u32x4 kv = load16(a.key + src);
  const u32x4 vv = load16(a.value + src);
  const int s = a.token_seq[n];
  const int pos = a.token_pos[n];
  if (pos < 0 || pos >= a.max_blocks * B || s < 0 || s >= a.num_seqs) return;
  int blk = a.block_tables[static_cast<int64_t>(s) * a.max_blocks + pos / B];
  blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
  const int slot = pos % B;
  const int64_t tile = (static_cast<int64_t>(blk) * a.num_kv_heads + h) * G::kTileBytes;
  store16(a.k_pool + tile + (q >> 2) * G::kChunkRowBytes + slot * 64 + (q & 3) * 16, kv);
  store16(a.v_pool + tile + slot * G::kRowBytes + q * 16, vv);
}

// Grid: num_pairs * chunks workgroups; each copies its chunk of one block in both pools. A
// pair with an id outside its pool is skipped. One of the pools may be pinned host memory (a
// swap): the loads or stores then cross the host link, 16 bytes per lane, a whole wave's 1 KiB
// contiguous.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a, int chunks,
                                                          int64_t chunk_pieces) {
  const int pair = blockIdx.x / chunks;
  const int chunk = blockIdx.x % chunks;
  const int src = a.pairs[2 * pair];
  const int dst = a.pairs[2 * pair + 1];
  if (src < 0 || src >= a.src_num_blocks || dst < 0 || dst >= a.dst_num_blocks) return;
  const int64_t pieces = a.block_bytes / 16;
  const int64_t p0 = chunk * chunk_pieces;
  const int64_t p1 = p0 + chunk_pieces < pieces ? p0 + chunk_pieces : pieces;
  const int64_t so = static_cast<int64_t>(src) * a.block_bytes;
  const int64_t d0 = static_cast<int64_t>(dst) * a.block_bytes;
  for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    store16(a.dst_k + d0 + p * 16, load16(a.src_k + so + p * 16));
    store16(a.dst_v + d0 + p * 16, load16(a.src_v + so + p * 16));
  }
}

template <DType dt, int D, int B>
static hipError_t launch_rc(const CacheWriteArgs& a, hipStream_t stream) {
  const int64_t pieces =
      static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * TileGeom<dt, D, B>::kPiecesPerRow;
  hipLaunchKernelGGL((reshape_and_cache_kernel<dt, D, B>),
                     dim3(static_cast<unsigned>((pieces + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <DType dt, int D>
static hipError_t launch_rc_b(int block_size, const CacheWriteArgs& a, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_rc<dt, D, 8>(a, stream);
    case 32: return launch_rc<dt, D, 32>(a, stream);
    default: return launch_rc<dt, D, 16>(a, stream);
  }
}

hipError_t launch_reshape_and_cache(DType dt, int head_dim, int block_size,
                                    const CacheWriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  switch (dt) {
    case DType::F32: return head_dim == 64 ? launch_rc_b<DType::F32, 64>(block_size, a, stream)
                                           : launch_rc_b<DType::F32, 128>(block_size, a, stream);
    case DType::F16: return head_dim == 64 ? launch_rc_b<DType::F16, 64>(block_size, a, stream)
                                           : launch_rc_b<DType::F16, 128>(block_size, a, stream);
    case DType::BF16: return head_dim == 64 ? launch_rc_b<DType::BF16, 64>(block_size, a, stream)
                                            : launch_rc_b<DType::BF16, 128>(block_size, a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0) return hipSuccess;
  // 256 threads x 8 pieces of 16 B = 32 KiB of each pool per workgroup
  const int64_t chunk_pieces = 256 * 8;
  const int64_t pieces = a.block_bytes / 16;
  const int chunks = static_cast<int>((pieces + chunk_pieces - 1) / chunk_pieces);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<unsigned>(a.num_pairs) * chunks),
                     dim3(256), 0, stream, a, chunks, chunk_pieces);
  return hipGetLastError();
}

// pa_validate_tables. The count is cleared by its own one-thread kernel (no memset node in a
// captured graph), then each workgroup checks one sequence: thread 0 its length and query range,
// all threads the table entries the attention calls would read; each wavefront adds its count
// with one atomic.
__global__ void clear_count_kernel(int32_t* count) {
  if (threadIdx.x == 0) count[0] = 0;
}

__global__ __launch_bounds__(256) void validate_kernel(ValidateArgs a) {
  const int s = static_cast<int>(blockIdx.x);
  const int n = a.context_lens[s];
  int bad = 0;
  if (threadIdx.x == 0) {
    bad += (n < 0 || n > a.max_ctx) ? 1 : 0;
    if (a.query_start != nullptr) {
      const int q0 = a.query_start[s];
      const int q1 = a.query_start[s + 1];
      bad += (s == 0 && q0 != 0) ? 1 : 0;
      bad += (q1 < q0 || q1 - q0 > (n < 0 ? 0 : n)) ? 1 : 0;
    }
  }
  const int used = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  const int nb = (used + a.block_size - 1) / a.block_size;
  const int32_t* row = a.block_tables + static_cast<int64_t>(s) * a.max_blocks;
  for (int j = static_cast<int>(threadIdx.x); j < nb; j += 256) {
    const int id = row[j];
    bad += (id < 0 || id >= a.num_blocks) ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
  if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(a.violations, bad);
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(64), 0, stream, a.violations);
  if (a.num_seqs > 0)
    hipLaunchKernelGGL(validate_kernel, dim3(static_cast<unsigned>(a.num_seqs)), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

// pa_validate_writes. Every comparison is one against all: workgroup w holds items
// [w*256, w*256 + 256) in registers and streams the items it compares them with through LDS, 256
// at a time, each thread scanning the whole LDS tile (same address in every lane: a broadcast).

// The slot pa_reshape_and_cache writes for token n (the clamped block id times B plus p % B), or
// -1 when it skips the token; *bad_id is set when the table entry lies outside the pool.
__device__ int64_t write_slot(const ValidateWritesArgs& a, int n, int* bad_id) {
  const int s = a.token_seq[n];
  const int pos = a.token_pos[n];
  *bad_id = 0;
  if (pos < 0 || pos >= a.max_blocks * a.block_size || s < 0 || s >= a.num_seqs) return -1;
  int blk = a.block_tables[static_cast<int64_t>(s) * a.max_blocks + pos / a.block_size];
  if (blk < 0 || blk >= a.num_blocks) {
    *bad_id = 1;
    blk = blk < 0 ? 0 : a.num_blocks - 1;
  }
  return static_cast<int64_t>(blk) * a.block_size + pos % a.block_size;
}

__device__ void add_count(int32_t* count, int bad) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
  if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(count, bad);
}

// One thread per written token: a table entry outside the pool, and a slot that an earlier token
// (lower index) also writes, count one each.
__global__ __launch_bounds__(kValidateThreads) void validate_slots_kernel(ValidateWritesArgs a) {
  __shared__ int64_t tile[kValidateThreads];
  const int i = static_cast<int>(blockIdx.x) * kValidateThreads + static_cast<int>(threadIdx.x);
  int bad = 0;
  int64_t mine = -1;
  if (i < a.num_tokens) mine = write_slot(a, i, &bad);
  int dup = 0;
  for (int t = 0; t <= static_cast<int>(blockIdx.x); ++t) {
    const int j = t * kValidateThreads + static_cast<int>(threadIdx.x);
    int unused;
    tile[threadIdx.x] = j < a.num_tokens ? write_slot(a, j, &unused) : -1;
    __syncthreads();
    const int earlier = t < static_cast<int>(blockIdx.x) ? kValidateThreads
                                                         : static_cast<int>(threadIdx.x);
    if (mine >= 0)
      for (int k = 0; k < earlier; ++k) dup |= tile[k] == mine ? 1 : 0;
    __syncthreads();
  }
  add_count(a.violations, bad + dup);
}

// One thread per copy pair with both ids in the pool: a destination that an earlier such pair
// also writes, and a destination that any such pair (itself included) reads, count one each.
__global__ __launch_bounds__(kValidateThreads) void validate_pairs_kernel(ValidateWritesArgs a) {
  __shared__ int2 tile[kValidateThreads];
  const int i = static_cast<int>(blockIdx.x) * kValidateThreads + static_cast<int>(threadIdx.x);
  int src = -1, dst = -1;
  if (i < a.num_pairs) {
    src = a.pairs[2 * i];
    dst = a.pairs[2 * i + 1];
    if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) src = dst = -1;
  }
  int dup = 0, reads = 0;
  const int tiles = (a.num_pairs + kValidateThreads - 1) / kValidateThreads;
  for (int t = 0; t < tiles; ++t) {
    const int j = t * kValidateThreads + static_cast<int>(threadIdx.x);
    int2 p = make_int2(-1, -1);
    if (j < a.num_pairs) {
      p = make_int2(a.pairs[2 * j], a.pairs[2 * j + 1]);
      if (p.x < 0 || p.x >= a.num_blocks || p.y < 0 || p.y >= a.num_blocks) p = make_int2(-1, -1);
    }
    tile[threadIdx.x] = p;
    __syncthreads();
    if (dst >= 0) {
      const int base = t * kValidateThreads;
      for (int k = 0; k < kValidateThreads; ++k) {
        const int2 q = tile[k];
        dup |= (base + k < i && q.y == dst) ? 1 : 0;
        reads |= q.x == dst ? 1 : 0;
      }
    }
    __syncthreads();
  }
  add_count(a.violations, dup + reads);
}

hipError_t launch_validate_writes(const ValidateWritesArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(clear_count_kernel, dim3(1), dim3(64), 0, stream, a.violations);
  if (a.num_tokens > 0)
    hipLaunchKernelGGL(validate_slots_kernel,
                       dim3(static_cast<unsigned>((a.num_tokens + kValidateThreads - 1) /
                                                  kValidateThreads)),
                       dim3(kValidateThreads), 0, stream, a);
  if (a.num_pairs > 0)
    hipLaunchKernelGGL(validate_pairs_kernel,
                       dim3(static_cast<unsigned>((a.num_pairs + kValidateThreads - 1) /
                                                  kValidateThreads)),
                       dim3(kValidateThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
