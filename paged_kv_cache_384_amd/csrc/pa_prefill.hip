// Causal attention of a chunk of new query tokens per sequence over the paged KV cache (the
// prefill form: many queries per sequence instead of one).
//
// Sources (page title, section):
//   "PagedAttention" (newikis.com/ko/PagedAttention), "수학적 공식": the dense causal attention of
//   a general query token i (weights over tokens 1..i) and its blocked form, which sums over the
//   first ceil(i/B) blocks of the sequence; the decode kernel is the case of one query.
//   "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리" (ryotta.opik.net), §2 and the lookup
//   pseudocode: blocks are found through the block table and may sit anywhere in the pool.
//
// With many queries per sequence the work is two dense contractions per key/value tile
// (S = Q K^T and O += P V), so both run on the matrix cores (v_mfma_f32_16x16x32_{f16,bf16}).
//
// Workgroup: 256 threads (four wavefronts) own 128 consecutive queries of one (sequence, query
// head); each wavefront owns 32 of them as two 16-query MFMA columns. The workgroup walks the
// sequence's tokens in tiles of 64, from token 0 to the last position its queries can see:
//   * the tile's key rows and value rows are gathered through the block table into LDS (double
//     buffered, the next tile's global loads in flight while the current one is computed). Key
//     rows keep their order (a padded row per token); value rows are transposed into dim rows
//     (a padded row per head dimension), in the token order the P operand needs (below);
//   * each wavefront forms S^T = K Q^T: A = 16 tokens x 32 dims read from LDS, B = its queries
//     held in registers since the start. Lane l gets query l%16 and tokens 4(l/16)..4(l/16)+3 of
//     each 16-token block;
//   * online softmax per query (column), in the base-2 domain: causal mask on tiles that reach
//     past a query's position, running maximum shared by the four lanes of a column, rescaling of
//     the output only when the maximum grows by more than a slack of 2^8 (the final division by
//     the running sum makes the result exact either way). The running sum is one more matrix
//     product (all-ones A times the packed weights), so it sums exactly the 16-bit weights that
//     multiply the values;
//   * O^T += V^T P^T: A = 16 dims x 32 tokens from the transposed value rows, B = the
//     probabilities, packed to 16 bits straight from the S^T registers. Lane l's eight k values
//     are tokens {4(l/16)+i, 16+4(l/16)+i} (i < 4) of a 32-token step; the value rows are stored
//     in that order, so P never moves between lanes.
// Tokens at or past the context length are zero in LDS (their table entries are never read), so
// slots past the end of the last block do not matter, whatever they hold.
#include <type_traits>

#include "pa_device.h"

namespace pa {

namespace {

constexpr int kTileT = kPrefillTileTokens;   // tokens per key/value tile
constexpr int kTileQ = kPrefillTileQueries;  // queries per workgroup
constexpr int kWaveQ = 32;                   // queries per wavefront (two MFMA columns)
constexpr float kRescaleSlackPf = 8.0f;      // log2 of the largest weight before a rescale
typedef float float2_t __attribute__((ext_vector_type(2)));
// s_waitcnt immediate for gfx9-family: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kWaitVmcnt0 = 0x0F70;
static_assert(kPrefillThreads / 64 * kWaveQ == kTileQ, "four wavefronts of 32 queries");
static_assert(kTileT == 64, "the token permutation below covers two 32-token MFMA steps");

// Two fp32 values rounded (nearest even) to the 16-bit type and packed, low half first: one
// v_cvt_pk_{f16,bf16}_f32 on gfx950.
template <DType dt> struct Pack2;
template <> struct Pack2<DType::F16> {
  __device__ static __forceinline__ uint32_t run(float a, float b) {
    const float2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
};
template <> struct Pack2<DType::BF16> {
  __device__ static __forceinline__ uint32_t run(float a, float b) {
    const float2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  }
};

// Position of token t (0..63) of a tile in a transposed value row: the 32-token MFMA step
// ks = t/32 takes, in lane group r = (t%16)/4, tokens 4r..4r+3 of the step's first 16 and then
// 16+4r..16+4r+3, so a lane's 16-byte operand is eight adjacent 16-bit slots.
__device__ __forceinline__ int vt_slot(int t) {
  const int ks = t >> 5;
  const int u = t & 31;
  return ks * 32 + ((u & 15) >> 2) * 8 + (u >> 4) * 4 + (u & 3);
}

}  // namespace

// Two workgroups per CU (eight wavefronts, two per SIMD): registers are capped at 256 per lane
// so one wavefront's softmax overlaps the other's matrix-core work.
template <DType dt, int D, int B>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
  using G = TileGeom<dt, D, B>;
  static_assert(G::kEsz == 2, "matrix-core prefill takes 16-bit elements");
  constexpr int kChunks = D / 32;          // 64-byte chunks (32 dims) per key row
  constexpr int kDBlocks = D / 16;         // 16-dim output blocks
  constexpr int kKRow = D * 2 + 16;        // LDS key row: one token, padded by 16 bytes
  constexpr int kVtRow = kTileT * 2 + 16;  // LDS value row: one dim of 64 tokens, padded
  constexpr int kVTasks = D / 64;          // (token pair, 16-byte piece) tasks per thread
  __shared__ __align__(16) uint8_t k_s[2][kTileT * kKRow];
  __shared__ __align__(16) uint8_t v_s[2][D * kVtRow];

  // ---- which queries ---------------------------------------------------------------------
  // A unit is (query tile qt, sequence, KV head); its G query heads read the same key/value
  // tiles. The hardware deals workgroups round-robin over the 8 XCDs (blockIdx % 8), each with
  // its own L2: unit u goes to XCD u % 8, where its G heads run as consecutive workgroups and
  // share that L2. Units are numbered from the highest query tile down, so the longest-running
  // workgroups (the latest queries of a prompt see the most tokens) start first on every XCD.
  const int group = a.group;
  const int k8 = static_cast<int>(blockIdx.x >> 3);
  const int u = (k8 / group) * 8 + static_cast<int>(blockIdx.x & 7);
  if (u >= a.num_units) return;
  const int h_in = k8 % group;
  const int g_kv = u % a.num_kv_heads;
  const int s = (u / a.num_kv_heads) % a.num_seqs;
  const int qt = a.q_tiles - 1 - u / (a.num_kv_heads * a.num_seqs);
  const int h = g_kv * group + h_in;
  const int q0 = a.query_start[s];
  int n_q = a.query_start[s + 1] - q0;
  n_q = n_q < 0 ? 0 : n_q;
  // queries past max_query_len are not computed; positions still count every query
  const int q_len = n_q > a.max_query_len ? a.max_query_len : n_q;
  if (qt * kTileQ >= q_len) return;
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int j0 = qt * kTileQ;
  const int base_p = ctx - n_q;  // position of query 0 (its context holds tokens 0..base_p)
  const int j_last = (j0 + kTileQ < q_len ? j0 + kTileQ : q_len) - 1;
  const int p_last_raw = base_p + j_last;
  const int p_last = p_last_raw < ctx - 1 ? p_last_raw : ctx - 1;
  const int n_steps = p_last < 0 ? 0 : p_last / kTileT + 1;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;  // MFMA column (query) / row (token, dim) within a 16-block
  const int grp = lane >> 4;  // MFMA lane group: k values 8*grp .. 8*grp+7
  const int kvh = g_kv;

  // ---- this wavefront's queries, held as B operands of S^T = K Q^T ------------------------
  const int wj0 = j0 + wave * kWaveQ;
  const int wj1 = (wj0 + kWaveQ - 1 < q_len - 1 ? wj0 + kWaveQ - 1 : q_len - 1);
  const bool w_active = wj0 <= wj1;
  u32x4 qf[2][kChunks];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int jq = wj0 + qb * 16 + col;
    jq = jq < q_len ? jq : q_len - 1;
    const uint8_t* row =
        a.query + (static_cast<int64_t>(q0 + jq) * a.num_q_heads + h) * G::kRowBytes + grp * 16;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) qf[qb][c] = load16(row + c * 64);
  }

  // ---- gathering a tile: the loads each thread issues --------------------------------------
  // keys: token 16*wave + col of the tile, 16-byte piece grp of each 64-byte chunk
  const int ktok = wave * 16 + col;
  // values: tokens vtok and vtok + 1 (same block: B is even), 16-byte pieces vpc + 8*it
  const int vtok = 2 * (tid & 31);
  const int vpc = tid >> 5;
  const int64_t table_row = static_cast<int64_t>(s) * a.max_blocks;
  // the table entry of token t (clamped to the context, so entries past it are never read), and
  // the byte offset of (block b, this KV head) with b clamped into the pool
  auto table_block = [&](int t) -> int {
    t = t < ctx ? t : ctx - 1;
    return a.block_tables[table_row + t / B];
  };
  auto tile_of = [&](int b) -> int64_t {
    b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
    return (static_cast<int64_t>(b) * a.num_kv_heads + kvh) * G::kTileBytes;
  };
  u32x4 kr[kChunks];
  u32x4 vr[kVTasks][2];
  auto load_tile = [&](int64_t kt, int64_t vt) {
    const uint8_t* kp = a.k_pool + kt + (ktok % B) * 64 + grp * 16;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) kr[c] = load16(kp + c * G::kChunkRowBytes);
    const uint8_t* vp = a.v_pool + vt + (vtok % B) * G::kRowBytes + vpc * 16;
#pragma unroll
    for (int it = 0; it < kVTasks; ++it) {
      vr[it][0] = load16(vp + it * 128);
      vr[it][1] = load16(vp + G::kRowBytes + it * 128);
    }
  };
  auto store_tile = [&](int buf, int T0) {
    if (T0 + kTileT > ctx) {  // the tile that holds the context's end (workgroup-uniform)
      const u32x4 zero = {0u, 0u, 0u, 0u};
      const bool kin = T0 + ktok < ctx;
      const bool v0 = T0 + vtok < ctx;
      const bool v1 = T0 + vtok + 1 < ctx;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) kr[c] = kin ? kr[c] : zero;
#pragma unroll
      for (int it = 0; it < kVTasks; ++it) {
        vr[it][0] = v0 ? vr[it][0] : zero;
        vr[it][1] = v1 ? vr[it][1] : zero;
      }
    }
    uint8_t* kd = k_s[buf] + ktok * kKRow + grp * 16;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) store16(kd + c * 64, kr[c]);
    uint8_t* vd = v_s[buf] + vt_slot(vtok) * 2;
#pragma unroll
    for (int it = 0; it < kVTasks; ++it) {
      const u32x4 x = vr[it][0];
      const u32x4 y = vr[it][1];
      const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
      const uint32_t yw[4] = {y.x, y.y, y.z, y.w};
      const int d0 = (vpc + 8 * it) * 8;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // dims d0+2k and d0+2k+1 of the two tokens, as (token vtok, token vtok+1) pairs
        *reinterpret_cast<uint32_t*>(vd + (d0 + 2 * k) * kVtRow) =
            (xw[k] & 0xffffu) | (yw[k] << 16);
        *reinterpret_cast<uint32_t*>(vd + (d0 + 2 * k + 1) * kVtRow) =
            (xw[k] >> 16) | (yw[k] & 0xffff0000u);
      }
    }
  };

  // ---- running softmax state and output (O^T blocks: dims 16*db + 4*grp + i, query col) ---
  f32x4 o[2][kDBlocks];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) o[qb][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float m[2] = {-INFINITY, -INFINITY};
  // Running sums of the weights, formed on the matrix cores from the same 16-bit weights that
  // multiply the values (A = all ones), so numerator and denominator use identical weights; every
  // element of lacc[qb] holds the sum for the lane's column.
  f32x4 lacc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
  const uint32_t one2 = Pack2<dt>::run(1.0f, 1.0f);
  const u32x4 ones = {one2, one2, one2, one2};
  const float thresh = kRescaleSlackPf;

  // One key/value tile. Scores stay raw (unscaled) until the exponent, where one fma applies the
  // scale and subtracts the running maximum; the maximum of scaled scores is the scale times the
  // raw maximum because the scale is positive. kMasked: the tile reaches past some column's
  // position, so tokens after it get -inf.
  auto compute = [&](int buf, int T0, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    // S^T blocks: st[qb][tb][i] = score of query 16qb+col, token T0 + 16tb + 4grp + i
    f32x4 st[2][4];
    const uint8_t* kb = k_s[buf] + col * kKRow + grp * 16;
    // matrix-core sections run at raised wave priority, so a wavefront that has its operands
    // keeps the matrix pipe fed while the SIMD's other wavefront does its softmax arithmetic
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      st[0][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      st[1][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const u32x4 kf = load16(kb + tb * 16 * kKRow + c * 64);
        st[0][tb] = Mfma16x16x32<dt>::run(kf, qf[0][c], st[0][tb]);
        st[1][tb] = Mfma16x16x32<dt>::run(kf, qf[1][c], st[1][tb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    float mx[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if constexpr (kMasked) {
        const int lim = base_p + wj0 + qb * 16 + col - T0 - grp * 4;  // last visible offset
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            st[qb][tb][i] = tb * 16 + i <= lim ? st[qb][tb][i] : -INFINITY;
      }
      float mq = fmaxf(fmaxf(st[qb][0][0], st[qb][0][1]), fmaxf(st[qb][0][2], st[qb][0][3]));
#pragma unroll
      for (int tb = 1; tb < 4; ++tb)
        mq = fmaxf(mq, fmaxf(fmaxf(st[qb][tb][0], st[qb][tb][1]),
                             fmaxf(st[qb][tb][2], st[qb][tb][3])));
      mq = fmaxf(mq, __shfl_xor(mq, 16, 64));
      mq = fmaxf(mq, __shfl_xor(mq, 32, 64));
      mx[qb] = mq * a.scale_log2;
    }
    if (__builtin_amdgcn_ballot_w64(mx[0] > m[0] + thresh || mx[1] > m[1] + thresh) != 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float mn = fmaxf(m[qb], mx[qb]);
        // a column with nothing visible yet keeps m = -inf and a factor of 1
        const float corr = mn == -INFINITY ? 1.0f : exp2_fast(m[qb] - mn);
        m[qb] = mn;
        lacc[qb] *= corr;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) o[qb][db] *= corr;
      }
    }
    // probabilities, packed as the B operands of the two 32-token steps
    u32x4 pb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float neg_m = m[qb] == -INFINITY ? 0.0f : -m[qb];
      float pr[4][4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pr[tb][i] = exp2_fast(__builtin_fmaf(st[qb][tb][i], a.scale_log2, neg_m));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pb[qb][ks].x = Pack2<dt>::run(pr[2 * ks][0], pr[2 * ks][1]);
        pb[qb][ks].y = Pack2<dt>::run(pr[2 * ks][2], pr[2 * ks][3]);
        pb[qb][ks].z = Pack2<dt>::run(pr[2 * ks + 1][0], pr[2 * ks + 1][1]);
        pb[qb][ks].w = Pack2<dt>::run(pr[2 * ks + 1][2], pr[2 * ks + 1][3]);
      }
    }
    const uint8_t* vb = v_s[buf] + col * kVtRow + grp * 16;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      lacc[0] = Mfma16x16x32<dt>::run(ones, pb[0][ks], lacc[0]);
      lacc[1] = Mfma16x16x32<dt>::run(ones, pb[1][ks], lacc[1]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
        const u32x4 vf = load16(vb + db * 16 * kVtRow + ks * 64);
        o[0][db] = Mfma16x16x32<dt>::run(vf, pb[0][ks], o[0][db]);
        o[1][db] = Mfma16x16x32<dt>::run(vf, pb[1][ks], o[1][db]);
      }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- walk the tiles ----------------------------------------------------------------------
  // The block ids of tile i+2 are loaded while tile i is computed and turned into addresses only
  // at step i+1, when the tile's own loads are issued, so no step waits on a table read.
  if (n_steps > 0) {
    load_tile(tile_of(table_block(ktok)), tile_of(table_block(vtok)));
    // Every load so far (the queries and tile 0) completes here. Without this explicit wait the
    // compiler's wait-count analysis, which cannot see that the query registers are complete
    // once the first tile is, waits for every in-flight tile load before each step's first
    // matrix instruction.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    store_tile(0, 0);
    int kb_next = table_block(kTileT + ktok);
    int vb_next = table_block(kTileT + vtok);
    __syncthreads();
    const int wp_lo = base_p + wj0;  // every column of the wave sees tokens 0..wp_lo
    const int wp_hi = base_p + wj1;  // no column sees a token past wp_hi
    for (int step = 0; step < n_steps; ++step) {
      const int T0 = step * kTileT;
      const bool more = step + 1 < n_steps;
      if (more) {
        load_tile(tile_of(kb_next), tile_of(vb_next));
        kb_next = table_block(T0 + 2 * kTileT + ktok);
        vb_next = table_block(T0 + 2 * kTileT + vtok);
      }
      if (w_active && T0 <= wp_hi) {
        if (T0 + kTileT - 1 > wp_lo) compute(step & 1, T0, std::true_type{});
        else compute(step & 1, T0, std::false_type{});
      }
      if (more) store_tile((step + 1) & 1, T0 + kTileT);
      __syncthreads();
    }
  }

  // ---- normalise and store: lane holds dims 16db + 4grp .. +3 of query 16qb + col ---------
  if (!w_active) return;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = lacc[qb][0];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int j = wj0 + qb * 16 + col;
    if (j >= q_len) continue;
    uint8_t* row = a.out + (static_cast<int64_t>(q0 + j) * a.num_q_heads + h) * G::kRowBytes +
                   grp * 8;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) {
      uint2 w;
      w.x = Pack2<dt>::run(o[qb][db][0] * inv, o[qb][db][1] * inv);
      w.y = Pack2<dt>::run(o[qb][db][2] * inv, o[qb][db][3] * inv);
      *reinterpret_cast<uint2*>(row + db * 32) = w;
    }
  }
}

template <DType dt, int D, int B>
static hipError_t launch_pf(const PrefillArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<dt, D, B>), dim3(a.num_wgs), dim3(kPrefillThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <DType dt, int D>
static hipError_t launch_pf_b(int block_size, const PrefillArgs& a, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_pf<dt, D, 8>(a, stream);
    case 32: return launch_pf<dt, D, 32>(a, stream);
    default: return launch_pf<dt, D, 16>(a, stream);
  }
}

hipError_t launch_prefill(DType dt, int head_dim, int block_size, const PrefillArgs& a,
                          hipStream_t stream) {
  if (a.num_wgs == 0) return hipSuccess;
  switch (dt) {
    case DType::F16: return head_dim == 64 ? launch_pf_b<DType::F16, 64>(block_size, a, stream)
                                           : launch_pf_b<DType::F16, 128>(block_size, a, stream);
    case DType::BF16: return head_dim == 64 ? launch_pf_b<DType::BF16, 64>(block_size, a, stream)
                                            : launch_pf_b<DType::BF16, 128>(block_size, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
