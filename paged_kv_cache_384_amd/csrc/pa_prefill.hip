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
//   * the tile's keys and values are gathered through the block table straight into LDS by
//     buffer_load_dwordx4 ... lds (no trip through registers; double buffered, the next tile's
//     loads in flight while the current one is computed). Keys land in the order the matrix-core
//     operand reads want them; values in token rows whose 16-byte pieces are rotated by the
//     token, so the transposing reads below meet every bank once;
//   * each wavefront forms S^T = K Q^T: A = 16 tokens x 32 dims read from LDS, B = its queries
//     held in registers since the start. Lane l gets query l%16 and tokens 4(l/16)..4(l/16)+3 of
//     each 16-token block;
//   * online softmax per query (column), in the base-2 domain: causal mask on tiles that reach
//     past a query's position, running maximum shared by the four lanes of a column (permlane
//     swaps), rescaling of the output only when the maximum grows by more than a slack of 2^8
//     (the final division by the running sum makes the result exact either way). The running
//     sum is one more matrix product (all-ones A times the packed weights), so it sums exactly
//     the 16-bit weights that multiply the values;
//   * O^T += V^T P^T: B = the probabilities, packed to 16 bits straight from the S^T registers;
//     lane l's eight k values are tokens {4(l/16)+i, 16+4(l/16)+i} (i < 4) of a 32-token step.
//     A = 16 dims x those 32 tokens, read from the token-major value rows by the transposing
//     LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane 4a+b receives element b of
//     the 4-element chunk that lane 4k+a addresses, for k = 0..3, so lanes addressing (token k,
//     dims 4a..4a+3) hand every lane 4 tokens of its own dim.
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
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
static_assert(kPrefillThreads / 64 * kWaveQ == kTileQ, "four wavefronts of 32 queries");
static_assert(kTileT == 64, "the token permutation below covers two 32-token MFMA steps");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 from an LDS address: 4 16-bit elements, transposed across each group of 16
// lanes (see the file comment).
__device__ __forceinline__ u32x2 read_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// buffer_load_dwordx4 ... lds: 16 bytes at byte offset voff of buffer r straight into LDS, lane
// i's bytes landing at lds + 16 * i (the LDS base is taken from the first lane); counted by
// vmcnt. The buffer form rather than global_load_lds: the compiler's wait-count model takes a
// pending global (FLAT-encoded) LDS load as touching both memory counters and then makes every
// LDS read wait for all earlier ones, which would serialise the operand reads with the matrix
// products; the buffer form is tracked by vmcnt alone.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, int voff, uint8_t* lds) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds), 16, voff, 0, 0, 0);
}

// Raw buffer resource over n bytes at p (dword 3: the gfx9 data-format field set to 32 bits;
// offsets at or past n read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), static_cast<short>(0), n,
                                           0x00020000);
}

// Maximum over lanes l, l^16, l^32, l^48 (the four rows of 16 lanes), in every lane: a
// v_permlane16_swap and a v_permlane32_swap of the value with itself give each lane its partner
// in the other half of the row pair / wave half.
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(f32_bits(x), f32_bits(x), false, false);
  x = fmaxf(bits_f32(a[0]), bits_f32(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(f32_bits(x), f32_bits(x), false, false);
  return fmaxf(bits_f32(b[0]), bits_f32(b[1]));
}

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

}  // namespace

// Workgroups per CU: two at head_dim 128 (eight wavefronts, two per SIMD, registers capped at
// 256 per lane, 64 KiB of LDS each), three at head_dim 64 (registers capped at 168, 32 KiB of
// LDS each), so one wavefront's softmax overlaps another's matrix-core work.
template <int D> constexpr int prefill_waves_per_simd() { return D == 64 ? 3 : 2; }

template <DType dt, int D, int B>
__global__ __launch_bounds__(kPrefillThreads) __attribute__((amdgpu_waves_per_eu(
    prefill_waves_per_simd<D>(), prefill_waves_per_simd<D>())))
void prefill_kernel(PrefillArgs a) {
  using G = TileGeom<dt, D, B>;
  static_assert(G::kEsz == 2, "matrix-core prefill takes 16-bit elements");
  constexpr int kChunks = D / 32;          // 64-byte chunks (32 dims) per key row
  constexpr int kDBlocks = D / 16;         // 16-dim output blocks
  constexpr int kVRow = D * 2;             // LDS value row of one token (unpadded)
  constexpr int kPPR = kVRow / 16;         // 16-byte pieces per value row
  constexpr int kRPI = 1024 / kVRow;       // value rows one wave load fills
  constexpr int kVLoads = 16 / kRPI;       // wave loads per wavefront per tile (its 16 tokens)
  constexpr int kKLoads = kChunks;         // key wave loads per wavefront per tile
  constexpr int kTileBytesLds = kTileT * D * 2;  // one tile of keys (or of values) in LDS
  static_assert(kRPI * kVLoads == 16 && kRPI <= B, "a value wave load stays inside one block");
  // two buffers of each, as separate arrays: every access below names its buffer at compile time
  // (the step loop is unrolled by two), so the compiler can tell that a tile's operand reads and
  // the next tile's loads into the other buffer never overlap, and does not make the reads wait
  // for those loads
  __shared__ __align__(1024) uint8_t k_s0[kTileBytesLds];
  __shared__ __align__(1024) uint8_t k_s1[kTileBytesLds];
  __shared__ __align__(1024) uint8_t v_s0[kTileBytesLds];
  __shared__ __align__(1024) uint8_t v_s1[kTileBytesLds];

  // ---- which queries ---------------------------------------------------------------------
  // Workgroups come in units whose members read the same key/value tiles and run as
  // consecutive workgroups on one XCD, sharing its L2: the hardware deals workgroups
  // round-robin over the 8 XCDs (blockIdx % 8), so unit u goes to XCD u % 8.
  //   tile-major (many query tiles per sequence: prompts): a unit is (query tile, sequence, KV
  //     head) and holds the G query heads; units are numbered from the highest query tile down,
  //     so the longest-running workgroups (the latest queries of a prompt see the most tokens)
  //     start first on every XCD;
  //   sequence-major (a few query tiles per sequence: chunks on top of a long context, whose
  //     tiles cost about the same): a unit is (sequence, KV head) and holds all its query tiles
  //     and query heads, which then read the sequence's key/value tiles from the L2 together
  //     instead of from HBM once per tile.
  const int group = a.group;
  const int k8 = static_cast<int>(blockIdx.x >> 3);
  const int u = (k8 / a.unit_wgs) * 8 + static_cast<int>(blockIdx.x & 7);
  if (u >= a.num_units) return;
  const int within = k8 % a.unit_wgs;
  const int h_in = within % group;
  int g_kv, s, qt;
  if (a.seq_major) {
    g_kv = u % a.num_kv_heads;
    s = u / a.num_kv_heads;
    qt = a.q_tiles - 1 - within / group;
  } else {
    g_kv = u % a.num_kv_heads;
    s = (u / a.num_kv_heads) % a.num_seqs;
    qt = a.q_tiles - 1 - u / (a.num_kv_heads * a.num_seqs);
  }
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;  // MFMA column (query) / row (token, dim) within a 16-block
  const int grp = lane >> 4;  // MFMA lane group: k values 8*grp .. 8*grp+7
  const int kvh = g_kv;
  // The two workgroups on a CU put one wavefront on each SIMD. Raising both to the same
  // priority in their matrix sections changes nothing (measured); raising them to different
  // levels does: when both are in a matrix section the higher one issues first, the other falls
  // a phase behind, and from then on one does its softmax while the other keeps the matrix
  // pipe busy. The level comes from the parity of the workgroup's slot on its CU (TG_ID, bits
  // 19:16 of HW_ID), which differs between two workgroups resident together.
  const bool prio_hi = (__builtin_amdgcn_s_getreg((3 << 11) | (16 << 6) | 4) & 1) != 0;
  auto mfma_priority = [&]() {
    if (prio_hi) __builtin_amdgcn_s_setprio(2);
    else __builtin_amdgcn_s_setprio(1);
  };

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

  // ---- gathering a tile: wave loads straight into LDS ------------------------------------
  // Each lane's 16 bytes of a wave load land at (wave-uniform LDS base) + 16 * lane, so the LDS
  // layout is chosen by which global bytes each lane requests:
  //   keys, in matrix-operand order: the 1 KiB at (tb * kChunks + c) KiB holds, at 16 * lane,
  //     the A operand lane (col, grp) reads for token block tb and chunk c: token 16 tb + col,
  //     bytes [64 c + 16 grp, +16) of its key row. Wavefront w loads token block w;
  //   values, in token rows of kVRow bytes whose 16-byte pieces are rotated by the token: piece p
  //     of token t sits at piece slot p ^ vswz(t), so that the transposing operand reads below
  //     (each half-wavefront: 8 tokens, 2 adjacent pieces each) meet all 64 banks once.
  //     Wavefront w loads rows 16 w .. 16 w + 15, kRPI rows per wave load.
  // A wavefront's 16 tokens lie in one block (B >= 16) or two (B = 8; lanes col >= 8, and value
  // loads of rows 8..15, take the second), so each load is a block address plus a per-lane offset
  // that is the same for every tile.
  auto vswz = [](int t) -> int {  // piece rotation of value row t (even, below kPPR)
    return 2 * ((t / (256 / kVRow)) & (kPPR / 2 - 1));
  };
  const int ktok = wave * 16 + col;  // this lane's key token of the tile
  const int64_t table_row = static_cast<int64_t>(s) * a.max_blocks;
  // the table entry of the block holding token t (t clamped to the context, so entries past it
  // are never read); one per lane: this lane's key token, 2 tiles ahead of its use
  auto table_block = [&](int t) -> int {
    t = t < ctx ? t : ctx - 1;
    return a.block_tables[table_row + t / B];
  };
  // byte offset of (block b clamped into the pool, this KV head); b is wave-uniform
  auto tile_of = [&](int b) -> int64_t {
    b = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
    return (static_cast<int64_t>(b) * a.num_kv_heads + kvh) * G::kTileBytes;
  };
  // per-lane offsets inside a block, the same for every tile (T0 is a multiple of 64 >= B)
  const int kl_off = (ktok % B) * 64 + grp * 16;
  int vl_off[kVLoads];
#pragma unroll
  for (int i = 0; i < kVLoads; ++i) {
    const int r = wave * 16 + i * kRPI + lane / kPPR;  // value row (token) this lane fills
    vl_off[i] = (r % B) * kVRow + ((lane % kPPR) ^ vswz(r)) * 16;
  }
  // kid: this lane's table entry for its key token of the tile. A wavefront's 16 tokens lie in
  // the block of lane 0's token, and for B = 8 the second 8 (lanes col >= 8, value rows 8..15)
  // in the block of lane 8's token; each block is one buffer resource (scalar registers) over
  // that block's tile of this KV head.
  auto load_tile = [&](uint8_t* kdst, uint8_t* vdst, int kid) {
    const int64_t lo = tile_of(__builtin_amdgcn_readfirstlane(kid));
    const auto k_lo = tile_rsrc(a.k_pool + lo, G::kTileBytes);
    const auto v_lo = tile_rsrc(a.v_pool + lo, G::kTileBytes);
    if constexpr (B >= 16) {
#pragma unroll
      for (int c = 0; c < kKLoads; ++c)
        load_lds16(k_lo, kl_off + c * G::kChunkRowBytes, kdst + (wave * kChunks + c) * 1024);
#pragma unroll
      for (int i = 0; i < kVLoads; ++i)
        load_lds16(v_lo, vl_off[i], vdst + (wave * 16 + i * kRPI) * kVRow);
    } else {
      const int64_t hi = tile_of(__builtin_amdgcn_readlane(kid, 8));
      const auto k_hi = tile_rsrc(a.k_pool + hi, G::kTileBytes);
      const auto v_hi = tile_rsrc(a.v_pool + hi, G::kTileBytes);
      // keys: each half of the 16 lanes of a column group reads its own block (lanes with
      // col >= 8 under the second resource), into the same LDS slots as one wave load would
      if (col < 8) {
#pragma unroll
        for (int c = 0; c < kKLoads; ++c)
          load_lds16(k_lo, kl_off + c * G::kChunkRowBytes, kdst + (wave * kChunks + c) * 1024);
      } else {
#pragma unroll
        for (int c = 0; c < kKLoads; ++c)
          load_lds16(k_hi, kl_off + c * G::kChunkRowBytes, kdst + (wave * kChunks + c) * 1024);
      }
#pragma unroll
      for (int i = 0; i < kVLoads; ++i)
        load_lds16(i * kRPI >= 8 ? v_hi : v_lo, vl_off[i], vdst + (wave * 16 + i * kRPI) * kVRow);
    }
  };
  // after the wave's loads of tile T0 have landed: zeros over tokens at or past the context's
  // end (only the context's last tile has any), so whatever the slots past it hold never enters
  auto zero_tail = [&](uint8_t* kdst, uint8_t* vdst, int T0) {
    if (T0 + kTileT <= ctx) return;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if (T0 + ktok >= ctx) {
#pragma unroll
      for (int c = 0; c < kKLoads; ++c)
        store16(kdst + (wave * kChunks + c) * 1024 + lane * 16, zero);
    }
#pragma unroll
    for (int i = 0; i < kVLoads; ++i)
      if (T0 + wave * 16 + i * kRPI + lane / kPPR >= ctx)
        store16(vdst + (wave * 16 + i * kRPI) * kVRow + lane * 16, zero);
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
  // this lane's transposing-read offsets in a value tile, per 16-dim block db: token
  // 4grp + col/4 (adding 16 or 32 tokens keeps the piece rotation), piece 2db + (col%4)/2 rotated,
  // then the lane's 8-byte half
  // (rotation: piece slot = piece ^ vr_swz, so slot 16-byte offsets are (2db*16) ^ vr_x)
  const int vr_t = 4 * grp + (col >> 2);
  const int vr_base = vr_t * kVRow + (col & 1) * 8;
  const int vr_x = (((col & 3) >> 1) ^ vswz(vr_t)) * 16;

  // One key/value tile. Scores stay raw (unscaled) until the exponent, where one fma applies the
  // scale and subtracts the running maximum; the maximum of scaled scores is the scale times the
  // raw maximum because the scale is positive. kMasked: the tile reaches past some column's
  // position, so tokens after it get -inf.
  auto compute = [&](const uint8_t* ktile, const uint8_t* vtile, int T0, bool masked) {
    // S^T blocks: st[qb][tb][i] = score of query 16qb+col, token T0 + 16tb + 4grp + i
    f32x4 st[2][4];
    const uint8_t* kb = ktile + lane * 16;
    // matrix-core sections run at raised wave priority, so a wavefront that has its operands
    // keeps the matrix pipe fed while the SIMD's other wavefront does its softmax arithmetic
    mfma_priority();
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      st[0][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      st[1][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const u32x4 kf = load16(kb + (tb * kChunks + c) * 1024);
        st[0][tb] = Mfma16x16x32<dt>::run(kf, qf[0][c], st[0][tb]);
        st[1][tb] = Mfma16x16x32<dt>::run(kf, qf[1][c], st[1][tb]);
      }
    }
    // schedule: each operand read is issued four reads ahead of its two products, so LDS
    // latency hides behind matrix-core work instead of stalling it
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int r = 0; r < 4 * kChunks - 4; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
    __builtin_amdgcn_s_setprio(0);
    float mx[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (masked) {
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
      mq = max_over_rows(mq);
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
    // transposing reads: this lane addresses token 4grp + col/4 (+16, +32) of the tile, dims
    // 16db + 4(col%4) .. +3 (through the row's piece rotation), and receives dim 16db + col of
    // tokens 4grp .. 4grp+3 (16+...)
    const uint8_t* vb = vtile;
    mfma_priority();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      lacc[0] = Mfma16x16x32<dt>::run(ones, pb[0][ks], lacc[0]);
      lacc[1] = Mfma16x16x32<dt>::run(ones, pb[1][ks], lacc[1]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
        const int off = vr_base + ((2 * db * 16) ^ vr_x);
        const u32x2 lo = read_tr16(vb + ks * 32 * kVRow + off);
        const u32x2 hi = read_tr16(vb + (ks * 32 + 16) * kVRow + off);
        const u32x4 vf = {lo.x, lo.y, hi.x, hi.y};
        o[0][db] = Mfma16x16x32<dt>::run(vf, pb[0][ks], o[0][db]);
        o[1][db] = Mfma16x16x32<dt>::run(vf, pb[1][ks], o[1][db]);
      }
    // schedule: the value reads run four (ks, db) pairs ahead of their products
    constexpr int kPairs = 2 * kDBlocks;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
#pragma unroll
    for (int pr = 0; pr < kPairs - 4; ++pr) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- walk the tiles ----------------------------------------------------------------------
  // The block ids of tile i+2 are read (wave-uniform) while tile i is computed and used at step
  // i+1, when the tile's loads are issued, so no step waits on a table read.
  if (n_steps > 0) {
    load_tile(k_s0, v_s0, table_block(ktok));
    // Every load so far (the queries and tile 0) completes here: the tile's bytes are in LDS.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    zero_tail(k_s0, v_s0, 0);
    int kid_next = table_block(kTileT + ktok);
    __syncthreads();
    const int wp_lo = base_p + wj0;  // every column of the wave sees tokens 0..wp_lo
    const int wp_hi = base_p + wj1;  // no column sees a token past wp_hi
    // one step: compute the tile in (kc, vc) while the next one loads into (kn, vn)
    auto step_at = [&](int step, const uint8_t* kc, const uint8_t* vc, uint8_t* kn, uint8_t* vn) {
      const int T0 = step * kTileT;
      const bool more = step + 1 < n_steps;
      if (more) {
        load_tile(kn, vn, kid_next);
        kid_next = table_block(T0 + 2 * kTileT + ktok);
      }
      if (w_active && T0 <= wp_hi) compute(kc, vc, T0, T0 + kTileT - 1 > wp_lo);
      if (more) {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's part of the next tile landed
        zero_tail(kn, vn, T0 + kTileT);
      }
      __syncthreads();
    };
    for (int step = 0; step < n_steps; step += 2) {
      step_at(step, k_s0, v_s0, k_s1, v_s1);
      if (step + 1 < n_steps) step_at(step + 1, k_s1, v_s1, k_s0, v_s0);
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
