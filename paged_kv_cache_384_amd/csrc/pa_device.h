// Device-side helpers shared by the HIP kernels: element traits, 16-byte vector loads,
// widening to fp32, dot products over 16-byte pieces, lane reductions, output rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <DType dt> struct Elem;
template <> struct Elem<DType::F32> { static constexpr int kSize = 4; };
template <> struct Elem<DType::F16> { static constexpr int kSize = 2; };
template <> struct Elem<DType::BF16> { static constexpr int kSize = 2; };

// Geometry of a (block, head) tile for element type dt, head dimension D and block size B, and
// of the 16-token groups the kernels work in. Key tiles are cut into chunk rows of 64 bytes per
// token (B * 64 bytes per row); value tiles are token rows of D * esz bytes.
template <DType dt, int D, int B = 16>
struct TileGeom {
  static constexpr int kEsz = Elem<dt>::kSize;
  static constexpr int kRowBytes = D * kEsz;             // one token's head vector
  static constexpr int kTileBytes = B * kRowBytes;
  static constexpr int kChunkRowBytes = B * 64;          // one key chunk row
  static constexpr int kEpp = 16 / kEsz;                 // elements per 16-byte piece
  static constexpr int kLoads = kRowBytes / 64;          // 16-byte loads per lane per group
  static constexpr int kChunkElems = 64 / kEsz;          // key layout: elements per chunk
  static constexpr int kPiecesPerRow = kRowBytes / 16;   // value rows: lanes sharing a token
  static constexpr int kRowsPerLoad = 64 / kPiecesPerRow;  // value rows one load covers
  static_assert(kRowBytes % 64 == 0, "token rows must be whole 64-byte chunks");
  static_assert(kLoads * kRowsPerLoad == kGroupTokens, "value rows must cover the group");
};

__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte load of a key or value tile piece. kStream: the tile is read once per launch, so the
// load carries the non-temporal hint; it does not allocate in L2 or the Infinity Cache, which
// measurably raises random-tile read bandwidth on MI355X. Otherwise an ordinary cached load, for
// tiles that several sequences read in the same launch.
template <bool kStream>
__device__ __forceinline__ u32x4 load16_kv(const uint8_t* p) {
  if constexpr (kStream) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(uint8_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Reinterpretations take their operand by value: __builtin_bit_cast applied directly to an
// ext-vector element (v.y, v.z, ...) is miscompiled into a cast of element 0 by this compiler,
// so elements are always copied into a scalar first.
__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Widen the kEpp elements held in one 16-byte piece to fp32 (exact for every type).
template <DType dt> struct Widen;
template <> struct Widen<DType::F32> {
  __device__ static __forceinline__ void run(const u32x4& v, float* o) {
    o[0] = bits_f32(v.x); o[1] = bits_f32(v.y); o[2] = bits_f32(v.z); o[3] = bits_f32(v.w);
  }
};
template <> struct Widen<DType::F16> {
  __device__ static __forceinline__ void run(const u32x4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f16x2 h = as_f16x2(w[k]);
      o[2 * k] = static_cast<float>(h.x);
      o[2 * k + 1] = static_cast<float>(h.y);
    }
  }
};
template <> struct Widen<DType::BF16> {
  __device__ static __forceinline__ void run(const u32x4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] = bits_f32(w[k] << 16);
      o[2 * k + 1] = bits_f32(w[k] & 0xffff0000u);
    }
  }
};

// acc + dot(a, b) over one 16-byte piece of each operand, products and sums in fp32.
// 16-bit types use the packed dot2 instructions (each 16-bit product is exact in fp32).
template <DType dt> struct Dot16;
template <> struct Dot16<DType::F32> {
  __device__ static __forceinline__ float run(const u32x4& a, const u32x4& b, float acc) {
    acc = __builtin_fmaf(bits_f32(a.x), bits_f32(b.x), acc);
    acc = __builtin_fmaf(bits_f32(a.y), bits_f32(b.y), acc);
    acc = __builtin_fmaf(bits_f32(a.z), bits_f32(b.z), acc);
    acc = __builtin_fmaf(bits_f32(a.w), bits_f32(b.w), acc);
    return acc;
  }
};
template <> struct Dot16<DType::F16> {
  __device__ static __forceinline__ float run(const u32x4& a, const u32x4& b, float acc) {
    acc = __builtin_amdgcn_fdot2(as_f16x2(a.x), as_f16x2(b.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_f16x2(a.y), as_f16x2(b.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_f16x2(a.z), as_f16x2(b.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_f16x2(a.w), as_f16x2(b.w), acc, false);
    return acc;
  }
};
template <> struct Dot16<DType::BF16> {
  __device__ static __forceinline__ float run(const u32x4& a, const u32x4& b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.x), as_bf16x2(b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.y), as_bf16x2(b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.z), as_bf16x2(b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a.w), as_bf16x2(b.w), acc, false);
    return acc;
  }
};

// c + a * b on the matrix cores: a 16x16 fp32 tile, 32 deep, 16-bit operands. Each operand is
// one 16-byte piece per lane: A[i][k] in lane i + 16*(k/8), element k%8; B[k][j] in lane
// j + 16*(k/8), element k%8; the result C[i][j] in lane j + 16*(i/4), element i%4.
template <DType dt> struct Mfma16x16x32;
template <> struct Mfma16x16x32<DType::F16> {
  __device__ static __forceinline__ f32x4 run(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma16x16x32<DType::BF16> {
  __device__ static __forceinline__ f32x4 run(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// The value of lane L of the caller's own row of 16 lanes, in every lane of that row
// (DPP row_newbcast).
template <int L>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(L >= 0 && L < 16, "lane within a row of 16");
  return bits_f32(__builtin_amdgcn_update_dpp(0u, f32_bits(x), 0x150 + L, 0xF, 0xF, false));
}

// Sum over each group of four consecutive lanes, result in all four (two DPP quad swaps).
__device__ __forceinline__ float quad_sum(float x) {
  x += bits_f32(__builtin_amdgcn_update_dpp(0u, f32_bits(x), 0xB1, 0xF, 0xF, false));  // lanes 1,0,3,2
  x += bits_f32(__builtin_amdgcn_update_dpp(0u, f32_bits(x), 0x4E, 0xF, 0xF, false));  // lanes 2,3,0,1
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// 2^x with the hardware transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> stored element, round to nearest even.
template <DType dt> struct Narrow;
template <> struct Narrow<DType::F32> {
  __device__ static __forceinline__ void store(uint8_t* p, float x) {
    *reinterpret_cast<float*>(p) = x;
  }
};
template <> struct Narrow<DType::F16> {
  __device__ static __forceinline__ void store(uint8_t* p, float x) {
    *reinterpret_cast<_Float16*>(p) = static_cast<_Float16>(x);
  }
};
template <> struct Narrow<DType::BF16> {
  __device__ static __forceinline__ void store(uint8_t* p, float x) {
    uint32_t u = f32_bits(x);
    uint16_t r;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      r = static_cast<uint16_t>((u >> 16) | 0x0040u);  // NaN stays a (quiet) NaN
    } else {
      // add half an output ulp, plus one more when the kept part is odd: ties go to even
      u += 0x7fffu + ((u >> 16) & 1u);
      r = static_cast<uint16_t>(u >> 16);
    }
    *reinterpret_cast<uint16_t*>(p) = r;
  }
};

// The workgroup's position in the launch, remapped so that consecutive logical work items run
// on the same XCD: the hardware deals workgroups round-robin over the 8 XCDs, each with its own
// L2, so logical item L is placed at a blockIdx whose XCD owns the range containing L.
__device__ __forceinline__ int xcd_logical_index() {
  const int n = gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int k = b >> 3;
  const int per = n >> 3;
  const int rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + k;
}

}  // namespace pa
