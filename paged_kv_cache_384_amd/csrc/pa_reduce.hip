// Merge of the partition states the attention kernel leaves when a context is split into
// several partitions (split-K over the context).
//
// Source (page title, section): "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리"
// (ryotta.opik.net), §3: the block-wise kernel only groups the partial sums of ordinary
// attention differently, so partial softmax states can be combined in any grouping. Each
// partition p of a (sequence, head) holds its maximum m_p (base-2 domain), its sum
// l_p = sum 2^(z - m_p) and its unnormalised output acc_p = sum 2^(z - m_p) v; with M = max m_p,
//     out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
#include "pa_device.h"

namespace pa {

// The merge for long splits: one 256-thread workgroup per (sequence, query head) merges that
// pair's partition states:
// thread t owns column t % D of partition group t / D (partitions p = group, group + G, ...),
// so every thread streams its partitions' values with independent loads; the G groups are
// summed through LDS.
template <DType dt, int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_kernel(DecodeArgs a) {
  using G = TileGeom<dt, D>;
  constexpr int kGroups = kReduceThreads / D;
  __shared__ float red_s[kReduceThreads];
  __shared__ float lred_s[kGroups];
  __shared__ float wmax_s[kReduceThreads / 64];

  const int sh = blockIdx.x;
  const int s = sh / a.num_q_heads;
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int np = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;  // written directly by the attention kernel
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const float* m = a.ws_m + static_cast<int64_t>(sh) * a.num_parts;
  const float* l = a.ws_l + static_cast<int64_t>(sh) * a.num_parts;
  const float* acc = a.ws_acc + static_cast<int64_t>(sh) * a.num_parts * D;

  float M = -INFINITY;
  for (int p = tid; p < np; p += kReduceThreads) M = fmaxf(M, m[p]);
  M = wave_max(M);
  if (lane == 0) wmax_s[tid >> 6] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kReduceThreads / 64; ++w) M = fmaxf(M, wmax_s[w]);

  const int col = tid % D;
  const int grp = tid / D;
  float o = 0.0f, L = 0.0f;
#pragma unroll 8
  for (int p = grp; p < np; p += kGroups) {
    const float w = exp2_fast(m[p] - M);
    o = __builtin_fmaf(w, acc[static_cast<int64_t>(p) * D + col], o);
    L = __builtin_fmaf(w, l[p], L);
  }
  red_s[tid] = o;
  if (col == 0) lred_s[grp] = L;
  __syncthreads();
  if (tid < D) {
    float ot = 0.0f, lt = 0.0f;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      ot += red_s[g * D + tid];
      lt += lred_s[g];
    }
    Narrow<dt>::store(a.out + (static_cast<int64_t>(sh) * D + tid) * G::kEsz, ot / lt);
  }
}

// The merge for short splits (at most kWaveMergeMaxParts partitions): one wavefront per
// (sequence, query head), four per workgroup. Lane p holds partition p's max and sum; every lane
// owns D/64 output columns, loads them for all partitions at once, and weighs them with
// 2^(m_p - M) read back from lane p as a wave-uniform value.
constexpr int kWaveMergeMaxParts = 16;

template <DType dt, int D>
__global__ __launch_bounds__(kReduceThreads) void decode_reduce_wave_kernel(DecodeArgs a) {
  using G = TileGeom<dt, D>;
  constexpr int kCols = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t sh = static_cast<int64_t>(blockIdx.x) * (kReduceThreads / 64) + (threadIdx.x >> 6);
  if (sh >= static_cast<int64_t>(a.num_seqs) * a.num_q_heads) return;
  const int s = static_cast<int>(sh / a.num_q_heads);
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int np = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;  // written directly by the attention kernel
  const float* m = a.ws_m + sh * a.num_parts;
  const float* l = a.ws_l + sh * a.num_parts;
  const float* acc = a.ws_acc + sh * a.num_parts * D + lane * kCols;

  const float mp = lane < np ? m[lane] : -INFINITY;
  const float M = wave_max(mp);
  const float w = exp2_fast(mp - M);  // 0 for lanes >= np
  const float L = wave_sum(lane < np ? w * l[lane] : 0.0f);
  // every partition's values are requested before the first is used
  float r[kWaveMergeMaxParts][kCols];
#pragma unroll
  for (int p = 0; p < kWaveMergeMaxParts; ++p)
#pragma unroll
    for (int e = 0; e < kCols; ++e) r[p][e] = p < np ? acc[p * D + e] : 0.0f;
  float o[kCols];
#pragma unroll
  for (int e = 0; e < kCols; ++e) o[e] = 0.0f;
#pragma unroll
  for (int p = 0; p < kWaveMergeMaxParts; ++p) {
    const float wp = bits_f32(__builtin_amdgcn_readlane(f32_bits(w), p));  // 0 for p >= np
#pragma unroll
    for (int e = 0; e < kCols; ++e) o[e] = __builtin_fmaf(wp, r[p][e], o[e]);
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int e = 0; e < kCols; ++e)
    Narrow<dt>::store(a.out + (sh * D + lane * kCols + e) * G::kEsz, o[e] * inv);
}

// ------------------------------------------------------------------------------------------
// launcher
// ------------------------------------------------------------------------------------------
template <DType dt, int D>
static hipError_t launch_red(const DecodeArgs& a, hipStream_t stream) {
  const int64_t pairs = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  if (a.num_parts <= kWaveMergeMaxParts) {
    constexpr int kPerWg = kReduceThreads / 64;
    hipLaunchKernelGGL((decode_reduce_wave_kernel<dt, D>),
                       dim3(static_cast<unsigned>((pairs + kPerWg - 1) / kPerWg)),
                       dim3(kReduceThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_reduce_kernel<dt, D>), dim3(static_cast<unsigned>(pairs)),
                       dim3(kReduceThreads), 0, stream, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// The share plan: which partitions consecutive sequences share, and the work lists.
//
// Source: "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리" (ryotta.opik.net), §4: sequences
// of one request (parallel samples, a common prompt) point their tables at the same physical
// blocks. A partition whose blocks are the same in two sequences holds the same keys and values
// for both, so one workgroup can score both sequences' queries against it and leave each its
// own partition state (the merge combines states in any grouping, as above).
//
// Sequence t joins the group of t - 1 on partition p when both contexts cover the whole
// partition, their table entries for it are equal, and t is not a multiple of kShareMax; groups
// are therefore cut at multiples of kShareMax, so each window of kShareMax sequences is planned
// on its own: one workgroup per (window, partition), wavefront k comparing the table entries of
// sequence 8w + k with those of its predecessor (lanes over the entries), then one thread
// writing the window's map entries and appending its items to the lists.
// ------------------------------------------------------------------------------------------
constexpr int kPlanThreads = kShareMax * 64;

__global__ void share_clear_kernel(int32_t* counts) {
  if (threadIdx.x < 2) counts[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kPlanThreads) void share_plan_kernel(DecodeArgs a, int block_size) {
  __shared__ int full_s[kShareMax];
  __shared__ int join_s[kShareMax];
  __shared__ int ctx_s[kShareMax];
  const int windows = (a.num_seqs + kShareMax - 1) / kShareMax;
  const int w = static_cast<int>(blockIdx.x % windows);
  const int p = static_cast<int>(blockIdx.x / windows);
  const int k = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int t = w * kShareMax + k;
  const int end = (p + 1) * a.part_tokens;
  const int per_part = a.part_tokens / block_size;  // table entries of one partition
  auto ctx_of = [&](int q) {
    const int c = a.context_lens[q];
    return c < 0 ? 0 : (c > a.max_ctx ? a.max_ctx : c);
  };
  const int ct = t < a.num_seqs ? ctx_of(t) : 0;
  const bool full = ct >= end;  // then end <= max_ctx <= max_blocks * block_size
  bool join = false;
  if (k != 0 && full && ctx_of(t - 1) >= end) {
    const int32_t* x = a.block_tables + static_cast<int64_t>(t - 1) * a.max_blocks +
                       static_cast<int64_t>(p) * per_part;
    const int32_t* y = x + a.max_blocks;
    bool differ = false;
    for (int j = lane; j < per_part; j += 64) differ |= x[j] != y[j];
    join = __builtin_amdgcn_ballot_w64(differ) == 0;
  }
  if (lane == 0) {
    full_s[k] = full;
    join_s[k] = join;
    ctx_s[k] = ct;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int own[kShareMax], lead[kShareMax];
  int n_own = 0, n_lead = 0;
  for (int q = 0; q < kShareMax && w * kShareMax + q < a.num_seqs; ++q) {
    const int item = (w * kShareMax + q) * a.num_parts + p;
    int n = 1;
    if (full_s[q]) {
      if (join_s[q]) {
        n = 0;
      } else {
        while (q + n < kShareMax && join_s[q + n]) ++n;
      }
    }
    a.share_map[item] = n;
    if (n >= 2) lead[n_lead++] = item;
    // a sequence computes the partitions inside its context itself (and partition 0 of an
    // empty context, which writes zeros)
    if (n == 1 && (p * a.part_tokens < ctx_s[q] || p == 0)) own[n_own++] = item;
  }
  const int64_t lead_base = static_cast<int64_t>(a.num_seqs) * a.num_parts;
  if (n_own > 0) {
    const int at = atomicAdd(&a.share_counts[0], n_own);
    for (int q = 0; q < n_own; ++q) a.share_list[at + q] = own[q];
  }
  if (n_lead > 0) {
    const int at = atomicAdd(&a.share_counts[1], n_lead);
    for (int q = 0; q < n_lead; ++q) a.share_list[lead_base + at + q] = lead[q];
  }
}

hipError_t launch_share_plan(const DecodeArgs& a, int block_size, hipStream_t stream) {
  hipLaunchKernelGGL(share_clear_kernel, dim3(1), dim3(64), 0, stream, a.share_counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>((a.num_seqs + kShareMax - 1) / kShareMax) * a.num_parts;
  hipLaunchKernelGGL(share_plan_kernel, dim3(static_cast<unsigned>(n)), dim3(kPlanThreads), 0,
                     stream, a, block_size);
  return hipGetLastError();
}

hipError_t launch_decode_reduce(DType dt, int head_dim, const DecodeArgs& a, hipStream_t stream) {
  if (a.num_parts <= 1) return hipSuccess;
  switch (dt) {
    case DType::F32: return head_dim == 64 ? launch_red<DType::F32, 64>(a, stream)
                                           : launch_red<DType::F32, 128>(a, stream);
    case DType::F16: return head_dim == 64 ? launch_red<DType::F16, 64>(a, stream)
                                           : launch_red<DType::F16, 128>(a, stream);
    case DType::BF16: return head_dim == 64 ? launch_red<DType::BF16, 64>(a, stream)
                                            : launch_red<DType::BF16, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
