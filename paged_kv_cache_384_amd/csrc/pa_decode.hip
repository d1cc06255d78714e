// Decode attention over the paged KV cache, and the merge of partition states.
//
// Sources (page title, section):
//   "PagedAttention" (newikis.com), "수학적 공식": dense causal attention of the newest token
//   and the same result written block by block over K_j, V_j.
//   "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리" (ryotta.opik.net), §3 and its block-table
//   lookup pseudocode: per logical block, look up the physical block, score its keys, fold the
//   scores and values into softmax partial sums; the result equals ordinary attention.
//
// Work decomposition (gfx950): one 256-thread workgroup (four wavefronts) per
// (KV head, sequence, query-head group, context partition). Inside a workgroup:
//   1. the partition's block-table slice is staged in LDS;
//   2. keys: each wavefront takes every fourth block; per block it issues kLoads 16-byte loads
//      per lane, each reading one whole 1 KiB key chunk row, so lane l holds 64 contiguous
//      bytes of token l/4 per row; dot2 instructions against the query piece the lane keeps in
//      registers, then a two-step DPP quad sum, give every token's score (base-2 domain);
//      scores go to LDS;
//   3. the partition maximum and exp2(score - max) are formed once per token in LDS;
//   4. values: each wavefront again takes every fourth block; lane l reads 16-byte pieces of
//      token rows and accumulates weight * value for its kEpp columns in fp32;
//   5. lanes holding the same columns are summed across the wavefront, then across the four
//      wavefronts through LDS; the workgroup writes the normalised output (single partition)
//      or its partition state (max, sum, unnormalised output) for the merge kernel.
// Only the last block of a partition can hold slots past the context end; those are masked
// with a select (score -inf, value 0) so stale or NaN contents never enter the result.
#include "pa_device.h"

namespace pa {

template <DType dt, int D, int NH, int UNROLL>
__global__ __launch_bounds__(kDecodeThreads) void decode_attention_kernel(DecodeArgs a) {
  using G = TileGeom<dt, D>;
  constexpr int kLoads = G::kLoads;
  constexpr int kEpp = G::kEpp;
  constexpr int kPiecesPerRow = G::kPiecesPerRow;
  constexpr int kRowsPerLoad = G::kRowsPerLoad;
  constexpr int kWaves = kDecodeThreads / 64;

  extern __shared__ float smem[];                 // scores [NH][part_tokens], then reduction
  __shared__ int bt_s[kMaxPartitionBlocks];
  __shared__ float wmax_s[kWaves][NH];
  __shared__ float wsum_s[kWaves][NH];

  // ---- which work item -------------------------------------------------------------------
  int r = xcd_logical_index();
  const int hg = r % a.head_groups;
  r /= a.head_groups;
  const int s = r % a.num_seqs;
  r /= a.num_seqs;
  const int part = r % a.num_parts;
  const int kvh = r / a.num_parts;

  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int h0 = kvh * a.group + hg * NH;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (ctx == 0) {
    if (part == 0) {
      for (int i = tid; i < NH * D; i += kDecodeThreads) {
        const int64_t o = (static_cast<int64_t>(s) * a.num_q_heads + h0 + i / D) * D + i % D;
        Narrow<dt>::store(a.out + o * G::kEsz, 0.0f);
      }
    }
    return;
  }
  const int start = part * a.part_tokens;
  if (start >= ctx) return;
  const int len = min(a.part_tokens, ctx - start);
  const int nblk = (len + kBlockSize - 1) / kBlockSize;
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;

  // ---- stage the block-table slice and the query pieces -------------------------------------
  {
    const int32_t* row = a.block_tables + static_cast<int64_t>(s) * a.max_blocks + start / kBlockSize;
    for (int j = tid; j < nblk; j += kDecodeThreads) {
      int id = row[j];
      bt_s[j] = id < 0 ? 0 : (id >= a.num_blocks ? a.num_blocks - 1 : id);
    }
  }
  // lane l scores token l/4 of each block; it needs query elements
  // [c*ChunkElems + (l%4)*Epp, +Epp) for each key chunk row c
  u32x4 qv[NH][kLoads];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    const uint8_t* qrow =
        a.query + (static_cast<int64_t>(s) * a.num_q_heads + h0 + hh) * G::kRowBytes;
#pragma unroll
    for (int c = 0; c < kLoads; ++c) qv[hh][c] = load16(qrow + c * 64 + (lane & 3) * 16);
  }
  __syncthreads();

  float* sc = smem;                               // [NH][part_tokens]
  const int64_t head_tiles = a.num_kv_heads;
  const float scale_log2 = a.scale_log2;

  // ---- pass 1: scores --------------------------------------------------------------------
  float lmax[NH];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) lmax[hh] = -INFINITY;
  const int tok = lane >> 2;
  for (int j0 = wave; j0 < nblk; j0 += kWaves * UNROLL) {
    u32x4 kr[UNROLL][kLoads];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int j = j0 + kWaves * u;
      if (j < nblk) {
        const int phys = __builtin_amdgcn_readfirstlane(bt_s[j]);
        const uint8_t* tile = a.k_pool + (phys * head_tiles + kvh) * G::kTileBytes;
#pragma unroll
        for (int c = 0; c < kLoads; ++c) kr[u][c] = load16(tile + c * 1024 + lane * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int j = j0 + kWaves * u;
      if (j < nblk) {
        const int t = j * kBlockSize + tok;
        const bool valid = t < len;
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
          float d = 0.0f;
#pragma unroll
          for (int c = 0; c < kLoads; ++c) d = Dot16<dt>::run(kr[u][c], qv[hh][c], d);
          d = quad_sum(d);
          const float z = valid ? d * scale_log2 : -INFINITY;
          if ((lane & 3) == 0) sc[hh * a.part_tokens + t] = z;
          lmax[hh] = fmaxf(lmax[hh], z);
        }
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    const float m = wave_max(lmax[hh]);
    if (lane == 0) wmax_s[wave][hh] = m;
  }
  __syncthreads();

  // ---- pass 2: weights exp2(z - max) and their sum ----------------------------------------
  float M[NH], L[NH];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    float m = wmax_s[0][hh];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, wmax_s[w][hh]);
    M[hh] = m;
  }
  {
    float lsum[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) lsum[hh] = 0.0f;
    for (int t = tid; t < nblk * kBlockSize; t += kDecodeThreads) {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const float p = exp2_fast(sc[hh * a.part_tokens + t] - M[hh]);
        sc[hh * a.part_tokens + t] = p;
        lsum[hh] += p;
      }
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const float l = wave_sum(lsum[hh]);
      if (lane == 0) wsum_s[wave][hh] = l;
    }
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    float l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l += wsum_s[w][hh];
    L[hh] = l;
  }

  // ---- pass 3: weighted values -----------------------------------------------------------
  // load i of lane l covers value row (l / PiecesPerRow) * kLoads + i of the block, columns
  // [(l % PiecesPerRow) * Epp, +Epp): each lane's rows are consecutive, so its weights are one
  // vector LDS read per head.
  const int vrow0 = (lane / kPiecesPerRow) * kLoads;
  const int vbyte = (lane % kPiecesPerRow) * 16;
  float acc[NH][kEpp];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int e = 0; e < kEpp; ++e) acc[hh][e] = 0.0f;

  for (int j0 = wave; j0 < nblk; j0 += kWaves * UNROLL) {
    u32x4 vr[UNROLL][kLoads];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int j = j0 + kWaves * u;
      if (j < nblk) {
        const int phys = __builtin_amdgcn_readfirstlane(bt_s[j]);
        const uint8_t* tile = a.v_pool + (phys * head_tiles + kvh) * G::kTileBytes;
#pragma unroll
        for (int i = 0; i < kLoads; ++i)
          vr[u][i] = load16(tile + (vrow0 + i) * G::kRowBytes + vbyte);
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int j = j0 + kWaves * u;
      if (j < nblk) {
        const int t0 = j * kBlockSize + vrow0;
        const bool tail = (j == nblk - 1) && (len % kBlockSize) != 0;
        float pw[NH][kLoads];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
          for (int i = 0; i < kLoads; ++i) pw[hh][i] = sc[hh * a.part_tokens + t0 + i];
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
          float v[kEpp];
          Widen<dt>::run(vr[u][i], v);
          if (tail && t0 + i >= len) {
#pragma unroll
            for (int e = 0; e < kEpp; ++e) v[e] = 0.0f;
          }
#pragma unroll
          for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int e = 0; e < kEpp; ++e) acc[hh][e] = __builtin_fmaf(pw[hh][i], v[e], acc[hh][e]);
        }
      }
    }
  }

  // ---- combine lanes, then wavefronts ------------------------------------------------------
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int e = 0; e < kEpp; ++e)
#pragma unroll
      for (int o = kPiecesPerRow; o < 64; o <<= 1) acc[hh][e] += __shfl_xor(acc[hh][e], o, 64);

  float* red = smem + NH * a.part_tokens;        // [kWaves][NH][D]
  if (lane < kPiecesPerRow) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int e = 0; e < kEpp; ++e) red[(wave * NH + hh) * D + lane * kEpp + e] = acc[hh][e];
  }
  __syncthreads();

  const int64_t sh0 = static_cast<int64_t>(s) * a.num_q_heads + h0;
  for (int i = tid; i < NH * D; i += kDecodeThreads) {
    const int hh = i / D;
    const int col = i % D;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += red[(w * NH + hh) * D + col];
    float Lh = 0.0f, Mh = 0.0f;
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      if (k == hh) { Lh = L[k]; Mh = M[k]; }
    }
    if (nparts == 1) {
      Narrow<dt>::store(a.out + ((sh0 + hh) * D + col) * G::kEsz, o / Lh);
    } else {
      const int64_t st = (sh0 + hh) * a.num_parts + part;
      a.ws_acc[st * D + col] = o;
      if (col == 0) {
        a.ws_m[st] = Mh;
        a.ws_l[st] = Lh;
      }
    }
  }
}

// One 64-lane workgroup per (sequence, query head): merge that pair's partition states.
template <DType dt, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeArgs a) {
  using G = TileGeom<dt, D>;
  constexpr int kCols = D / 64;
  const int sh = blockIdx.x;
  const int s = sh / a.num_q_heads;
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int np = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;  // written directly by the attention kernel
  const int lane = threadIdx.x;
  const float* m = a.ws_m + static_cast<int64_t>(sh) * a.num_parts;
  const float* l = a.ws_l + static_cast<int64_t>(sh) * a.num_parts;
  const float* acc = a.ws_acc + static_cast<int64_t>(sh) * a.num_parts * D;
  float M = -INFINITY;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, m[p]);
  M = wave_max(M);
  float L = 0.0f;
  for (int p = lane; p < np; p += 64) L += l[p] * exp2_fast(m[p] - M);
  L = wave_sum(L);
  float o[kCols];
#pragma unroll
  for (int e = 0; e < kCols; ++e) o[e] = 0.0f;
  for (int p = 0; p < np; ++p) {
    const float w = exp2_fast(m[p] - M);
#pragma unroll
    for (int e = 0; e < kCols; ++e) o[e] = __builtin_fmaf(w, acc[p * D + lane * kCols + e], o[e]);
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int e = 0; e < kCols; ++e)
    Narrow<dt>::store(a.out + (static_cast<int64_t>(sh) * D + lane * kCols + e) * G::kEsz,
                      o[e] * inv);
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
constexpr int kUnroll = 2;

template <DType dt, int D, int NH>
static hipError_t launch_attn(const DecodeArgs& a, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(a.num_kv_heads) * a.num_seqs * a.head_groups * a.num_parts;
  const size_t lds = (static_cast<size_t>(NH) * a.part_tokens + 4 * NH * D) * sizeof(float);
  hipLaunchKernelGGL((decode_attention_kernel<dt, D, NH, kUnroll>), dim3(static_cast<unsigned>(n)),
                     dim3(kDecodeThreads), lds, stream, a);
  return hipGetLastError();
}

template <DType dt, int D>
static hipError_t launch_attn_nh(const DecodeArgs& a, hipStream_t stream) {
  switch (a.heads_per_wg) {
    case 4: return launch_attn<dt, D, 4>(a, stream);
    case 2: return launch_attn<dt, D, 2>(a, stream);
    default: return launch_attn<dt, D, 1>(a, stream);
  }
}

hipError_t launch_decode_attention(DType dt, int head_dim, const DecodeArgs& a,
                                   hipStream_t stream) {
  switch (dt) {
    case DType::F32: return head_dim == 64 ? launch_attn_nh<DType::F32, 64>(a, stream)
                                           : launch_attn_nh<DType::F32, 128>(a, stream);
    case DType::F16: return head_dim == 64 ? launch_attn_nh<DType::F16, 64>(a, stream)
                                           : launch_attn_nh<DType::F16, 128>(a, stream);
    case DType::BF16: return head_dim == 64 ? launch_attn_nh<DType::BF16, 64>(a, stream)
                                            : launch_attn_nh<DType::BF16, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <DType dt, int D>
static hipError_t launch_red(const DecodeArgs& a, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  hipLaunchKernelGGL((decode_reduce_kernel<dt, D>), dim3(static_cast<unsigned>(n)), dim3(64), 0,
                     stream, a);
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
