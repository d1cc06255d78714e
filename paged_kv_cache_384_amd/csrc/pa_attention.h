// Decode attention over the paged KV cache: the kernel template, instantiated per block size in
// pa_attention_b8.hip / _b16.hip / _b32.hip (the partition merge is in pa_reduce.hip).
//
// Sources (page title, section):
//   "PagedAttention" (newikis.com), "수학적 공식": dense causal attention of the newest token
//   and the same result written block by block over K_j, V_j.
//   "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리" (ryotta.opik.net), §3 and its block-table
//   lookup pseudocode: per logical block, look up the physical block, score its keys, fold the
//   scores and values into running softmax sums (running max, running denominator, running
//   output, one division at the end); the result equals ordinary attention.
//
// Work decomposition (gfx950): one 256-thread workgroup (four wavefronts) per
// (KV head, sequence, query-head group, context partition). The unit of work inside a partition
// is a group of 16 consecutive tokens, whatever the block size B: one 64-lane wave load of 16
// bytes per lane covers 16 tokens of a key chunk row (1 KiB at 64 bytes per token). At B = 16 a
// group is one block; at B = 32 a block holds two groups (its chunk rows are 2 KiB, the second
// group starts 1 KiB in); at B = 8 a group spans two blocks, lanes 0-31 and 32-63 addressing
// different physical blocks. Wavefront w streams a contiguous quarter of the partition's groups
// in a single pass over keys and values:
//   * keys: kLoads 16-byte loads per lane, each reading one whole 1 KiB key chunk row, so lane l
//     holds 64 contiguous bytes of token l/4 per row; dot2 instructions against the query piece
//     the lane keeps in registers and a two-step DPP quad sum give every token's score in the
//     base-2 domain (scale * log2 e folded in);
//   * running softmax, one state per wavefront: the maximum m is the same in every lane and is
//     raised only when some score exceeds it by more than kRescaleSlack (a ballot, so the
//     rescale of the running sums is a rare, uniform branch); weights are 2^(score - m) <=
//     2^kRescaleSlack, and the division at the end cancels the choice of m exactly;
//   * values: lane l reads 16-byte pieces of kLoads value rows and accumulates weight * value
//     for its kEpp columns in fp32; the weights of those rows are moved from the lanes that
//     scored them with DPP row broadcasts (or ds_bpermute for other tile shapes);
//   * the next block's keys are requested as soon as the scores are formed and its values as
//     soon as the weighted sum is done, so a wavefront always has a block's loads in flight.
// The four wavefront states are merged through LDS with the usual max-rescaling; the
// workgroup writes the normalised output (one partition) or its partition state (max, sum,
// unnormalised output) for the merge kernel. Only the last block of a partition can hold slots
// past the context end; those are masked with selects (score -inf, value 0) so stale or NaN
// contents never enter the result.
#pragma once

#include <utility>

#include "pa_device.h"

namespace pa {

// A wavefront's running maximum is raised only when a score exceeds it by more than this many
// powers of two; weights therefore stay <= 2^8, far from fp32 overflow.
constexpr float kRescaleSlack = 8.0f;

// Weight of value row vrow0 + I for a lane whose value rows start at vrow0: that row's score
// sits in lanes 4 * (vrow0 + I) .. +3.
template <int kPiecesPerRow, int kLoads>
struct RowWeights {
  template <int... I>
  __device__ static __forceinline__ void run(float p, int lane, float* w,
                                             std::integer_sequence<int, I...>) {
    if constexpr (kPiecesPerRow == 16 && kLoads == 4) {
      // value rows 4*(l/16) + I are scored in lanes 16*(l/16) + 4*I: lane 4*I of the lane's own
      // row of 16, which DPP row_newbcast broadcasts within each row
      ((w[I] = row_bcast<4 * I>(p)), ...);
    } else {
      const int src = ((lane / kPiecesPerRow) * kLoads) * 16;  // byte address of lane 4*vrow0
      ((w[I] = bits_f32(__builtin_amdgcn_ds_bpermute(src + 16 * I, static_cast<int>(f32_bits(p))))),
       ...);
    }
  }
};

// This lane's addresses of one 16-token group's key and value pieces: key piece c at
// k + c * (B * 64), value piece i at v + i * row bytes.
struct GroupPtrs {
  const uint8_t* k;
  const uint8_t* v;
};

// One 16-token group of one wavefront's stream: scores, running-softmax update, weighted values.
// kPrefetch: the group is full and its registers are refilled with the group at `next` as soon
// as the keys and then the values are consumed. Otherwise the group may be the partition's last,
// so slots at or past len are masked, and nothing is loaded.
template <DType dt, int D, int B, int NH, bool kStream, bool kPrefetch>
struct BlockStep {
  using G = TileGeom<dt, D, B>;
  static constexpr int kLoads = G::kLoads;
  static constexpr int kEpp = G::kEpp;
  static constexpr int kPiecesPerRow = G::kPiecesPerRow;

  const u32x4 (&qv)[NH][kLoads];
  float scale_log2;
  int lane;
  int vrow0;
  int len;

  __device__ __forceinline__ void run(int g, GroupPtrs next, u32x4 (&kb)[kLoads],
                                      u32x4 (&vb)[kLoads], float (&m)[NH], float (&lsum)[NH],
                                      float (&acc)[NH][kEpp]) const {
    float sc[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      float d = 0.0f;
#pragma unroll
      for (int c = 0; c < kLoads; ++c) d = Dot16<dt>::run(kb[c], qv[hh][c], d);
      sc[hh] = quad_sum(d) * scale_log2;
    }
    if constexpr (kPrefetch) {
#pragma unroll
      for (int c = 0; c < kLoads; ++c)
        kb[c] = load16_kv<kStream>(next.k + c * G::kChunkRowBytes);
    } else {
      const bool valid = g * kGroupTokens + (lane >> 2) < len;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) sc[hh] = valid ? sc[hh] : -INFINITY;
    }

    float pw[NH][kLoads];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      if (__builtin_amdgcn_ballot_w64(sc[hh] > m[hh] + kRescaleSlack) != 0) {
        const float mn = wave_max(sc[hh]);
        const float c = exp2_fast(m[hh] - mn);
        lsum[hh] *= c;
#pragma unroll
        for (int e = 0; e < kEpp; ++e) acc[hh][e] *= c;
        m[hh] = mn;
      }
      const float p = exp2_fast(sc[hh] - m[hh]);
      lsum[hh] += p;
      RowWeights<kPiecesPerRow, kLoads>::run(p, lane, pw[hh],
                                             std::make_integer_sequence<int, kLoads>{});
    }

    // one value row at a time: widen, products, then the refill of that row's registers
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      float v[kEpp];
      Widen<dt>::run(vb[i], v);
      if constexpr (!kPrefetch) {
        if (g * kGroupTokens + vrow0 + i >= len) {
#pragma unroll
          for (int e = 0; e < kEpp; ++e) v[e] = 0.0f;
        }
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int e = 0; e < kEpp; ++e) acc[hh][e] = __builtin_fmaf(pw[hh][i], v[e], acc[hh][e]);
      if constexpr (kPrefetch) vb[i] = load16_kv<kStream>(next.v + i * G::kRowBytes);
    }
  }
};

// Query heads of one workgroup whose scores go to the matrix cores: 16-bit tiles with
// head_dim 128 and a head group of at least this many query heads.
constexpr int kMfmaMinHeads = 2;

template <DType dt, int D, int NH>
constexpr bool use_mfma_scores() {
  return Elem<dt>::kSize == 2 && D == 128 && NH >= kMfmaMinHeads && NH <= 16;
}

// The same block step with the scores formed on the matrix cores (16-bit, head_dim 128):
// S^T (16 tokens x 16 heads) = K (16 tokens x 128 dims) * Q^T (128 dims x 16 heads, heads >= NH
// zero) as four 16x16x32 MFMAs, one per 1 KiB key chunk row. Lane l loads token l%16, dims
// [32c + 8(l/16), +8) of chunk row c (a permutation of the row: still one coalesced 1 KiB wave
// load) and holds head l%16's query slice for the same dims. It receives head l%16's scores of
// tokens 4(l/16) .. 4(l/16)+3, which are the value rows its own row of 16 lanes accumulates, so
// lane 16r + h hands head h's weights to its row with DPP row broadcasts. The running maximum m
// and sum lsum are per lane, for head l%16 (equal in the four rows once reduced).
template <DType dt, int B, int NH, bool kStream, bool kPrefetch>
struct MfmaBlockStep {
  using G = TileGeom<dt, 128, B>;
  static constexpr int kLoads = G::kLoads;
  static constexpr int kEpp = G::kEpp;
  static_assert(kLoads == 4 && G::kPiecesPerRow == 16, "256-byte rows");

  const u32x4 (&qm)[kLoads];
  float scale_log2;
  int lane;
  int vrow0;
  int len;

  template <int... H>
  __device__ static __forceinline__ void bcast_heads(float x, float (&out)[NH],
                                                     std::integer_sequence<int, H...>) {
    ((out[H] = row_bcast<H>(x)), ...);
  }

  __device__ __forceinline__ void run(int g, GroupPtrs next, u32x4 (&kb)[kLoads],
                                      u32x4 (&vb)[kLoads], float& m, float& lsum,
                                      float (&acc)[NH][kEpp]) const {
    f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < kLoads; ++c) d = Mfma16x16x32<dt>::run(kb[c], qm[c], d);
    if constexpr (kPrefetch) {
#pragma unroll
      for (int c = 0; c < kLoads; ++c)
        kb[c] = load16_kv<kStream>(next.k + c * G::kChunkRowBytes);
    }
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = d[i] * scale_log2;
    if constexpr (!kPrefetch) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = g * kGroupTokens + vrow0 + i < len ? sc[i] : -INFINITY;
    }

    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__builtin_amdgcn_ballot_w64(bm > m + kRescaleSlack) != 0) {
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float mn = fmaxf(m, bm);
      const float c = exp2_fast(m - mn);
      lsum *= c;
      m = mn;
      float ch[NH];
      bcast_heads(c, ch, std::make_integer_sequence<int, NH>{});
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int e = 0; e < kEpp; ++e) acc[hh][e] *= ch[hh];
    }
    // value row i of this lane (token 4(l/16) + i) at a time: its weight for each head, the
    // widened row, the products, then the refill of that row's registers, so that only one
    // row's temporaries are live at once
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const float pi = exp2_fast(sc[i] - m);
      lsum += pi;
      float w[NH];
      bcast_heads(pi, w, std::make_integer_sequence<int, NH>{});
      float v[kEpp];
      Widen<dt>::run(vb[i], v);
      if constexpr (!kPrefetch) {
        if (g * kGroupTokens + vrow0 + i >= len) {
#pragma unroll
          for (int e = 0; e < kEpp; ++e) v[e] = 0.0f;
        }
      }
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
#pragma unroll
        for (int e = 0; e < kEpp; ++e) acc[hh][e] = __builtin_fmaf(w[hh], v[e], acc[hh][e]);
      if constexpr (kPrefetch) vb[i] = load16_kv<kStream>(next.v + i * G::kRowBytes);
    }
  }
};

// Work item modes of the decode kernel: kGrid, one workgroup per (KV head, sequence, head group,
// partition) as the grid's blocks; kList and kListSeqRows, a persistent loop over the items of
// the share plan's lists (partitions a sequence computes itself; partitions shared by a group of
// sequences, whose NH score columns are then one query head of the group's sequences).
enum DecodeMode : int { kGrid = 0, kList = 1, kListSeqRows = 2 };

// One work item: (KV head kvh, sequence s, head group hg, partition part). kSeqRows: the NH
// score columns are head kvh * group + hg of sequences s .. s + rows - 1, which share this
// partition's blocks, instead of NH query heads of sequence s.
template <DType dt, int D, int B, int NH, bool kStream, bool kPaged, bool kSeqRows>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int kvh, int s, int hg, int part,
                                            int rows, float (&red_s)[kDecodeThreads / 64][NH][D],
                                            float (&m_s)[kDecodeThreads / 64][NH],
                                            float (&l_s)[kDecodeThreads / 64][NH]) {
  using G = TileGeom<dt, D, B>;
  constexpr int kLoads = G::kLoads;
  constexpr int kEpp = G::kEpp;
  constexpr int kPiecesPerRow = G::kPiecesPerRow;
  constexpr int kWaves = kDecodeThreads / 64;
  int ctx = a.context_lens[s];
  ctx = ctx < 0 ? 0 : (ctx > a.max_ctx ? a.max_ctx : ctx);
  const int h0 = kSeqRows ? kvh * a.group + hg : kvh * a.group + hg * NH;
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
  const int ngroups = (len + kGroupTokens - 1) / kGroupTokens;  // 16-token groups
  const int nblocks = (len + B - 1) / B;                         // table entries this partition
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;

  // ---- this wavefront's groups -------------------------------------------------------------
  // a contiguous range [jb, je) of the partition's groups. Paged: the physical ids of their
  // blocks are looked up in the table ([anal] §3: the kernel looks each logical block up in the
  // block table) once, up front, one block per lane (a wavefront covers at most 64 blocks: 32
  // groups of a 2048-token partition, two 8-token blocks each), clamped into [0, NB); each step
  // then takes its id from that register with readlane, so no table read stands between
  // consuming one block and requesting the next. The contiguous twin has no table: block j of
  // sequence s is physical block s * max_blocks + j.
  const int64_t row0 = static_cast<int64_t>(s) * a.max_blocks + start / B;
  const int per_wave = ngroups / kWaves;
  const int extra = ngroups % kWaves;
  const int jb = wave * per_wave + min(wave, extra);
  const int je = jb + per_wave + (wave < extra ? 1 : 0);
  const int num_blocks = a.num_blocks;
  const int wb0 = jb * kGroupTokens / B;  // the wavefront's first block (of the partition)
  [[maybe_unused]] int wave_ids = 0;
  if constexpr (kPaged) {
    const int jj = wb0 + lane;
    if (jj < nblocks) {
      const int id = a.block_tables[row0 + jj];
      wave_ids = id < 0 ? 0 : (id >= num_blocks ? num_blocks - 1 : id);
    }
  }
  auto block_id = [&](int j) -> int {
    if constexpr (kPaged) {
      return __builtin_amdgcn_readlane(wave_ids, j - wb0);
    } else {
      const int64_t id = row0 + j;
      return id >= num_blocks ? num_blocks - 1 : static_cast<int>(id);
    }
  };

  constexpr bool kMfma = use_mfma_scores<dt, D, NH>();
  const int64_t tile_stride = static_cast<int64_t>(a.num_kv_heads) * G::kTileBytes;
  const uint8_t* qbase = a.query + (static_cast<int64_t>(s) * a.num_q_heads + h0) * G::kRowBytes;
  // the token of the group a lane's key pieces belong to: VALU scores read byte 16*l of each
  // 16-token chunk-row segment (token l/4), matrix-core scores read byte 64*(l%16) + 16*(l/16)
  // (token l%16); its value rows are vrow0 + i, bytes [(lane % kPiecesPerRow) * 16, +16)
  const int ktok = kMfma ? (lane & 15) : (lane >> 2);
  const int kbyte = kMfma ? 64 * (lane & 15) + 16 * (lane >> 4) : 16 * lane;
  const int vrow0 = (lane / kPiecesPerRow) * kLoads;
  const int vbyte = (lane % kPiecesPerRow) * 16;
  const uint8_t* kpool = a.k_pool + static_cast<int64_t>(kvh) * G::kTileBytes;
  const uint8_t* vpool = a.v_pool + static_cast<int64_t>(kvh) * G::kTileBytes;
  // this lane's addresses for group gg
  auto group_ptrs = [&](int gg) -> GroupPtrs {
    if constexpr (B >= kGroupTokens) {
      // block gg / (B/16) holds the group; its tokens start at slot 16 * (gg % (B/16))
      constexpr int kPer = B / kGroupTokens;
      const int64_t base = block_id(gg / kPer) * tile_stride;
      const int sub = gg % kPer;
      return {kpool + base + sub * (kGroupTokens * 64) + kbyte,
              vpool + base + (sub * kGroupTokens + vrow0) * G::kRowBytes + vbyte};
    } else {
      // the group spans blocks 2gg (tokens 0-7) and 2gg + 1 (tokens 8-15); past the
      // partition's last block the second is never scored, so its id is not looked up
      static_assert(B * 2 == kGroupTokens, "block sizes 8, 16 and 32");
      const int ja = 2 * gg;
      const int ida = block_id(ja);
      const int idb = ja + 1 < nblocks ? block_id(ja + 1) : ida;
      const int kh = ktok / B;
      const int vh = vrow0 / B;
      return {kpool + (kh ? idb : ida) * tile_stride + (ktok - kh * B) * 64 + (kbyte & 63),
              vpool + (vh ? idb : ida) * tile_stride + (vrow0 - vh * B) * G::kRowBytes + vbyte};
    }
  };
  const float scale_log2 = a.scale_log2;

  float acc[NH][kEpp];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int e = 0; e < kEpp; ++e) acc[hh][e] = 0.0f;

  // the query pieces are requested first: they are older than every block load, so waiting
  // for them never waits for a block
  // matrix-core scores: head l%16's slice (zero for l%16 >= NH), dims [32c + 8(l/16), +8) of
  // chunk row c; VALU scores: lane l scores token l/4 and needs dims [c*ChunkElems +
  // (l%4)*Epp, +Epp) of every head for each chunk row c
  [[maybe_unused]] u32x4 qm[kLoads];
  [[maybe_unused]] u32x4 qv[kMfma ? 1 : NH][kLoads];
  if constexpr (kMfma) {
    const int qh = lane & 15;
    // column qh: query head h0 + qh of sequence s, or (seq rows) head h0 of sequence s + qh
    const uint8_t* qrow =
        kSeqRows ? a.query + (static_cast<int64_t>(s + qh) * a.num_q_heads + h0) * G::kRowBytes
                 : qbase + qh * G::kRowBytes;
#pragma unroll
    for (int c = 0; c < kLoads; ++c)
      qm[c] = qh < rows ? load16(qrow + c * 64 + 16 * (lane >> 4)) : u32x4{0u, 0u, 0u, 0u};
  } else {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int c = 0; c < kLoads; ++c)
        qv[hh][c] = load16(qbase + hh * G::kRowBytes + c * 64 + (lane & 3) * 16);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the scheduler from moving block loads above these

  // Key/value loads in flight per wavefront: kDepth blocks ahead of the one being computed.
  // One register set (kA, vA) per block in flight; a step consumes its set and refills it with
  // the block kDepth ahead. Inside the loops every load is issued unconditionally (a wavefront
  // with fewer than kDepth blocks loads the partition's last block in their place and never
  // uses it), so the compiler's wait counts stay exact; only the wavefront's last kDepth
  // blocks, which may include the partition's partial one, run without refilling. Two blocks
  // ahead pays off for streamed single-head workgroups with 4 KiB tiles; with more heads, 8 KiB
  // tiles or cached reads of shared blocks the extra registers cost more occupancy than the
  // deeper pipeline gains (measured on MI355X).
  constexpr int kDepth = NH == 1 && kLoads <= 4 && kStream ? 2 : 1;
  u32x4 kA[kLoads], vA[kLoads];
  [[maybe_unused]] u32x4 kB[kLoads], vB[kLoads];
  auto load_block = [&](int jj, u32x4 (&kr)[kLoads], u32x4 (&vr)[kLoads]) {
    // past the wavefront's range: its own last group again (loaded, never used)
    const GroupPtrs p = group_ptrs(jj < je ? jj : je - 1);
#pragma unroll
    for (int c = 0; c < kLoads; ++c) kr[c] = load16_kv<kStream>(p.k + c * G::kChunkRowBytes);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) vr[i] = load16_kv<kStream>(p.v + i * G::kRowBytes);
  };
  if (jb < je) {  // a wavefront without groups (partitions of fewer than 4) loads nothing
    load_block(jb, kA, vA);
    if constexpr (kDepth == 2) load_block(jb + 1, kB, vB);
  }

  // drives one step type over the wavefront's blocks [jb, je)
  auto stream_blocks = [&](auto& full, auto& tail, auto&... state) {
    int j = jb;
    if constexpr (kDepth == 1) {
      for (; j + 1 < je; ++j) full.run(j, group_ptrs(j + 1), kA, vA, state...);
      if (j < je) tail.run(j, GroupPtrs{}, kA, vA, state...);
    } else {
      // pairs of full steps while at least four blocks remain (kA holds block j, kB block
      // j + 1 at the top of each pair), then the last one to three blocks
      for (; j + 3 < je; j += 2) {
        full.run(j, group_ptrs(j + 2), kA, vA, state...);
        full.run(j + 1, group_ptrs(j + 3), kB, vB, state...);
      }
      const int left = je - j;
      if (left == 3) {
        full.run(j, group_ptrs(j + 2), kA, vA, state...);
        tail.run(j + 1, GroupPtrs{}, kB, vB, state...);
        tail.run(j + 2, GroupPtrs{}, kA, vA, state...);
      } else if (left == 2) {
        tail.run(j, GroupPtrs{}, kA, vA, state...);
        tail.run(j + 1, GroupPtrs{}, kB, vB, state...);
      } else if (left == 1) {
        tail.run(j, GroupPtrs{}, kA, vA, state...);
      }
    }
  };

  if constexpr (kMfma) {
    float m = -INFINITY, lsum = 0.0f;
    MfmaBlockStep<dt, B, NH, kStream, true> full{qm, scale_log2, lane, vrow0, len};
    MfmaBlockStep<dt, B, NH, kStream, false> tail{qm, scale_log2, lane, vrow0, len};
    stream_blocks(full, tail, m, lsum, acc);
    // lane h (< NH) of any row holds head h's maximum; its sum is spread over the four rows
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (lane < NH) {
      m_s[wave][lane] = m;
      l_s[wave][lane] = lsum;
    }
  } else {
    float m[NH], lsum[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      m[hh] = -INFINITY;
      lsum[hh] = 0.0f;
    }
    BlockStep<dt, D, B, NH, kStream, true> full{qv, scale_log2, lane, vrow0, len};
    BlockStep<dt, D, B, NH, kStream, false> tail{qv, scale_log2, lane, vrow0, len};
    stream_blocks(full, tail, m, lsum, acc);
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      // every token's weight was added in its four scoring lanes
      lsum[hh] = wave_sum(lsum[hh]) * 0.25f;
      if (lane == 0) {
        m_s[wave][hh] = m[hh];
        l_s[wave][hh] = lsum[hh];
      }
    }
  }

  // ---- combine lanes holding the same columns, then the four wavefronts -------------------
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int e = 0; e < kEpp; ++e)
#pragma unroll
      for (int o = kPiecesPerRow; o < 64; o <<= 1) acc[hh][e] += __shfl_xor(acc[hh][e], o, 64);
  if (lane < kPiecesPerRow) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int e = 0; e < kEpp; ++e) red_s[wave][hh][lane * kEpp + e] = acc[hh][e];
  }
  __syncthreads();

  const int64_t sh0 = static_cast<int64_t>(s) * a.num_q_heads + h0;
  for (int i = tid; i < NH * D; i += kDecodeThreads) {
    const int hh = i / D;
    const int col = i % D;
    // row hh: (sequence s, head h0 + hh), or (seq rows) (sequence s + hh, head h0), which has
    // its own context length and so its own partition count
    [[maybe_unused]] int row_parts = nparts;
    if constexpr (kSeqRows) {
      if (hh >= rows) break;
      int c = a.context_lens[s + hh];
      c = c < 0 ? 0 : (c > a.max_ctx ? a.max_ctx : c);
      row_parts = (c + a.part_tokens - 1) / a.part_tokens;
    }
    const int64_t row = kSeqRows ? static_cast<int64_t>(s + hh) * a.num_q_heads + h0 : sh0 + hh;
    // wave 0 always holds block 0, so the maximum is finite; idle wavefronts (m = -inf,
    // sums 0) get weight 0
    float M = m_s[0][hh];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, m_s[w][hh]);
    float o = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float c = exp2_fast(m_s[w][hh] - M);
      o = __builtin_fmaf(c, red_s[w][hh][col], o);
      L = __builtin_fmaf(c, l_s[w][hh], L);
    }
    if (row_parts == 1) {
      Narrow<dt>::store(a.out + (row * D + col) * G::kEsz, o / L);
    } else {
      const int64_t st = row * a.num_parts + part;
      a.ws_acc[st * D + col] = o;
      if (col == 0) {
        a.ws_m[st] = M;
        a.ws_l[st] = L;
      }
    }
  }
}

template <DType dt, int D, int B, int NH, bool kStream, bool kPaged, int kMode = kGrid>
__global__ __launch_bounds__(kDecodeThreads) void decode_attention_kernel(DecodeArgs a) {
  constexpr int kWaves = kDecodeThreads / 64;
  __shared__ float red_s[kWaves][NH][D];
  __shared__ float m_s[kWaves][NH];
  __shared__ float l_s[kWaves][NH];
  if constexpr (kMode == kGrid) {
    int r = xcd_logical_index();
    const int hg = r % a.head_groups;
    r /= a.head_groups;
    const int s = r % a.num_seqs;
    r /= a.num_seqs;
    const int part = r % a.num_parts;
    const int kvh = r / a.num_parts;
    decode_item<dt, D, B, NH, kStream, kPaged, false>(a, kvh, s, hg, part, NH, red_s, m_s, l_s);
  } else {
    // the share plan's list of (sequence, partition) items, each for every KV head and head
    // group; the counts were written by the plan kernel earlier on this stream
    constexpr bool kSeq = kMode == kListSeqRows;
    const int groups = kSeq ? a.group : a.head_groups;
    const int64_t per = static_cast<int64_t>(a.num_kv_heads) * groups;
    const int32_t* list = a.share_list + (kSeq ? static_cast<int64_t>(a.num_seqs) * a.num_parts : 0);
    const int64_t units = static_cast<int64_t>(a.share_counts[kSeq ? 1 : 0]) * per;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
      const int item = list[u / per];
      const int rem = static_cast<int>(u % per);
      const int s = item / a.num_parts;
      const int part = item % a.num_parts;
      const int rows = kSeq ? a.share_map[item] : NH;
      decode_item<dt, D, B, NH, kStream, kPaged, kSeq>(a, rem / groups, s, rem % groups, part,
                                                        rows, red_s, m_s, l_s);
      __syncthreads();  // the next item reuses the LDS arrays
    }
  }
}

// ------------------------------------------------------------------------------------------
// launch helpers (each pa_attention_b*.hip instantiates them for one block size)
// ------------------------------------------------------------------------------------------
template <DType dt, int D, int B, int NH>
hipError_t launch_attn(const DecodeArgs& a, hipStream_t stream) {
  const int64_t n =
      static_cast<int64_t>(a.num_kv_heads) * a.num_seqs * a.head_groups * a.num_parts;
  const dim3 grid(static_cast<unsigned>(n)), block(kDecodeThreads);
  // contiguous sequences never share blocks, so the twin always streams
  if (!a.paged)
    hipLaunchKernelGGL((decode_attention_kernel<dt, D, B, NH, true, false>), grid, block, 0,
                       stream, a);
  else if (a.stream_kv)
    hipLaunchKernelGGL((decode_attention_kernel<dt, D, B, NH, true, true>), grid, block, 0,
                       stream, a);
  else
    hipLaunchKernelGGL((decode_attention_kernel<dt, D, B, NH, false, true>), grid, block, 0,
                       stream, a);
  return hipGetLastError();
}

template <DType dt, int D, int B>
hipError_t launch_attn_nh(const DecodeArgs& a, hipStream_t stream) {
  switch (a.heads_per_wg) {
    case 4: return launch_attn<dt, D, B, 4>(a, stream);
    case 2: return launch_attn<dt, D, B, 2>(a, stream);
    default: return launch_attn<dt, D, B, 1>(a, stream);
  }
}

// With a share plan: the partitions sequences compute themselves, and those shared by groups
// of sequences, each as a persistent loop over its list (only 16-bit pools with head_dim 128
// get a plan). Grids: about what the CUs hold at once.
template <DType dt, int B, int NH>
hipError_t launch_attn_list(const DecodeArgs& a, hipStream_t stream) {
  const int64_t most = static_cast<int64_t>(a.num_seqs) * a.num_parts * a.num_kv_heads;
  const unsigned own = static_cast<unsigned>(most * a.head_groups < 2048 ? most * a.head_groups : 2048);
  const unsigned shared = static_cast<unsigned>(most * a.group < 1024 ? most * a.group : 1024);
  hipLaunchKernelGGL((decode_attention_kernel<dt, 128, B, kShareMax, false, true, kListSeqRows>),
                     dim3(shared), dim3(kDecodeThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the partitions a sequence computes itself are the ones no other sequence in the call
  // shares in full: streamed (non-temporal loads, two blocks in flight for one head)
  hipLaunchKernelGGL((decode_attention_kernel<dt, 128, B, NH, true, true, kList>), dim3(own),
                     dim3(kDecodeThreads), 0, stream, a);
  return hipGetLastError();
}

template <DType dt, int B>
hipError_t launch_attn_shared(const DecodeArgs& a, hipStream_t stream) {
  switch (a.heads_per_wg) {
    case 4: return launch_attn_list<dt, B, 4>(a, stream);
    case 2: return launch_attn_list<dt, B, 2>(a, stream);
    default: return launch_attn_list<dt, B, 1>(a, stream);
  }
}

template <int B>
hipError_t launch_attn_shared_block(DType dt, const DecodeArgs& a, hipStream_t stream) {
  switch (dt) {
    case DType::F16: return launch_attn_shared<DType::F16, B>(a, stream);
    case DType::BF16: return launch_attn_shared<DType::BF16, B>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int B>
hipError_t launch_attn_block(DType dt, int head_dim, const DecodeArgs& a, hipStream_t stream) {
  switch (dt) {
    case DType::F32: return head_dim == 64 ? launch_attn_nh<DType::F32, 64, B>(a, stream)
                                           : launch_attn_nh<DType::F32, 128, B>(a, stream);
    case DType::F16: return head_dim == 64 ? launch_attn_nh<DType::F16, 64, B>(a, stream)
                                           : launch_attn_nh<DType::F16, 128, B>(a, stream);
    case DType::BF16: return head_dim == 64 ? launch_attn_nh<DType::BF16, 64, B>(a, stream)
                                            : launch_attn_nh<DType::BF16, 128, B>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
