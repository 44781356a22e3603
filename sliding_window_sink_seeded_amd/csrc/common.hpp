// Device helpers shared by the prefill and decode kernels (gfx950 / CDNA4, wave64).
//
// MFMA data layout used throughout (32x32 tiles):
//   * A operand (32 x 16): lane l supplies row (l % 32) and 8 contraction elements.
//   * B operand (16 x 32): lane l supplies column (l % 32) and 8 contraction elements.
//   * C/D (32 x 32, 16 fp32 per lane): lane l holds column (l % 32); register r holds row
//     8 * (r / 4) + 4 * (l / 32) + (r % 4).
// Which contraction index each of a lane's 8 elements stands for does not matter as long as the A
// and B operands of one product use the same assignment, because the product sums over it. The
// kernels therefore pick the assignment that makes their loads contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mimo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxHeads = 256;

// Storage tag types. Memory holds raw bits; fragments are what the MFMA consumes.
struct BF16 {
  using Frag = bf16x8;  // 8 contraction elements per lane, 16 bytes
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;  // elements per 16-byte chunk
};
struct F32 {
  using Frag = f32x8;  // 8 contraction elements per lane, 32 bytes
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// acc += A(32x16) * B(16x32) with 8 contraction elements per lane.
__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
// fp32: eight 32x32x2 products; product e contracts element e of both lane halves.
__device__ __forceinline__ f32x16 mma(const f32x8& a, const f32x8& b, f32x16 acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
  return acc;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Reinterprets 32 bits as a bf16 pair. Taken by value: with this toolchain,
// __builtin_bit_cast(bf16x2, v[j]) on an ext-vector element silently reads element 0.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) {
  bf16x2 r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}

// fp32 pair -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v;
  v[0] = lo;
  v[1] = hi;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint32_t bf16_bits(float x) { return pack_bf16x2(x, 0.f) & 0xFFFFu; }

template <typename E>
__device__ __forceinline__ typename E::Frag frag_from_f32(const float* x);
template <>
__device__ __forceinline__ bf16x8 frag_from_f32<BF16>(const float* x) {
  u32x4 u;
  u[0] = pack_bf16x2(x[0], x[1]);
  u[1] = pack_bf16x2(x[2], x[3]);
  u[2] = pack_bf16x2(x[4], x[5]);
  u[3] = pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, u);
}
template <>
__device__ __forceinline__ f32x8 frag_from_f32<F32>(const float* x) {
  f32x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = x[i];
  return f;
}

// Fragment from 8 consecutive accumulator registers starting at `off` (compile-time after unroll).
template <typename E>
__device__ __forceinline__ typename E::Frag frag_from_acc(const f32x16& s, int off) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = s[off + i];
  return frag_from_f32<E>(x);
}

// Reductions across the two halves of a wave: lane l and lane l ^ 32 both receive
// op(x[l % 32], x[l % 32 + 32]). permlane32_swap hands each lane the values of both halves at its
// position, so a symmetric op of its two results is the cross-half reduction in either half.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v_permlane32_swap: afterwards lanes 32-63 of `a` hold the old lanes 0-31 of `b` and lanes 0-31
// of `b` hold the old lanes 32-63 of `a`; lanes 0-31 of `a` and 32-63 of `b` are unchanged.
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Waits until every outstanding memory operation of this wave has completed.
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Checking builds (MIMO_POISON_LDS=1, libmimo_attn_poison.so): every kernel first fills its LDS
// with all-ones words (NaN as fp32 and as bf16) and waits at a barrier, so a read of LDS that the
// workgroup has not written turns its results into NaN instead of reusing what an earlier
// workgroup left there (a missing write, or a read that overtakes the write behind a missing
// barrier). Product builds compile this to nothing.
#ifndef MIMO_POISON_LDS
#define MIMO_POISON_LDS 0
#endif
__device__ __forceinline__ void poison_lds(void* lds, int bytes) {
  if constexpr (MIMO_POISON_LDS != 0) {
    const u32x4 nan = {~0u, ~0u, ~0u, ~0u};
    for (int i = (int)threadIdx.x; i < bytes / 16; i += (int)blockDim.x) st16((char*)lds + 16 * i, nan);
    __syncthreads();
  }
}
__device__ __forceinline__ u32x4 zero_chunk() {
  u32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0u;
  return z;
}

// Packs this lane's column of a 32 x (32 N) transposed accumulator block into bf16 chunks.
// acc[db][r] holds element 32 db + 8 (r / 4) + 4 half + r % 4 of the lane's row. The two wave
// halves trade register groups so that every lane owns 8 consecutive outputs: chunk i = 2 db + j
// covers outputs 32 db + 16 j + 8 half .. +7. Every lane must call it (the exchange reads the
// partner lane).
template <int N>
__device__ __forceinline__ void pack_row_bf16(const f32x16 (&acc)[N], float inv, u32x4 (&out)[2 * N]) {
#pragma unroll
  for (int db = 0; db < N; ++db) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int g0 = 8 * j, g1 = 8 * j + 4;  // register offsets of groups 2j and 2j+1
      uint32_t x0 = pack_bf16x2(acc[db][g0] * inv, acc[db][g0 + 1] * inv);
      uint32_t x1 = pack_bf16x2(acc[db][g0 + 2] * inv, acc[db][g0 + 3] * inv);
      uint32_t y0 = pack_bf16x2(acc[db][g1] * inv, acc[db][g1 + 1] * inv);
      uint32_t y1 = pack_bf16x2(acc[db][g1 + 2] * inv, acc[db][g1 + 3] * inv);
      swap_halves(x0, y0);
      swap_halves(x1, y1);
      out[2 * db + j][0] = x0;
      out[2 * db + j][1] = x1;
      out[2 * db + j][2] = y0;
      out[2 * db + j][3] = y1;
    }
  }
}
template <int M>
__device__ __forceinline__ void store_packed_row_bf16(char* orow, const u32x4 (&out)[M], int half) {
#pragma unroll
  for (int i = 0; i < M; ++i) *reinterpret_cast<u32x4*>(orow + (16 * i + 8 * half) * 2) = out[i];
}
// pack + store; lanes with !store write nothing but still take part in the exchange
template <int N>
__device__ __forceinline__ void store_row_bf16(char* orow, const f32x16 (&acc)[N], float inv,
                                               int half, bool store) {
  u32x4 out[2 * N];
  pack_row_bf16(acc, inv, out);
  if (store) store_packed_row_bf16(orow, out, half);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, output lane j element e is element
// (j % 4) of the 8 bytes read by lane 4 e + j / 4. If lanes 4e..4e+3 of a group read four
// consecutive 4-element pieces of row e of a row-major tile, every lane receives one column
// (4 consecutive rows) of it.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_ptr));
}

// A-operand fragment of V^T for O^T += V^T P^T, read from a row-major bf16 V tile
// ([key][dv], row stride `row_elems`): this lane's dv row is 32 db + lane % 32 and its 8 elements
// are keys 16 ks + 4 half + 0..3 and 16 ks + 8 + 4 half + 0..3 (the order in which the S^T
// accumulator holds P for this lane half).
__device__ __forceinline__ bf16x8 vt_frag_tr(const char* vtile, int row_elems, int db, int ks,
                                             int lane) {
  const int half = lane >> 5, i = lane & 15, dsub = (lane >> 4) & 1;
  const int key = 16 * ks + 4 * half + (i >> 2);
  const int dv = 32 * db + 16 * dsub + 4 * (i & 3);
  const char* p = vtile + (key * row_elems + dv) * 2;
  const s16x4 x = lds_read_tr16(p);
  const s16x4 y = lds_read_tr16(p + 8 * row_elems * 2);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 u;
  u[0] = x[0]; u[1] = x[1]; u[2] = x[2]; u[3] = x[3];
  u[4] = y[0]; u[5] = y[1]; u[6] = y[2]; u[7] = y[3];
  return __builtin_bit_cast(bf16x8, u);
}

// ---- rotary embedding of the leading 64 Q/K dims: pairs (i, i + 32) rotated by (cos, sin) of
// position * base^(-2i/64), read from a [position][32][2] fp32 table ----
constexpr int kRopeDims = 64;

// cs[2j], cs[2j+1] = cos, sin for element j of `lo`; lo holds dims i0.., hi the partner dims
// i0 + 32..; bf16 chunks carry 8 elements, fp32 chunks 4. Rotated values are rounded back to the
// storage type (bf16: round to nearest even). The fused multiply-adds are written out so that every
// kernel that inlines this rounds the same way (left to the compiler, contraction varied by kernel).
// One rotated pair in fp32: x' = x c - y s, y' = y c + x s, with the multiply-adds written out.
__device__ __forceinline__ float rope_x(float x, float y, float c, float s) { return __builtin_fmaf(x, c, -(y * s)); }
__device__ __forceinline__ float rope_y(float x, float y, float c, float s) { return __builtin_fmaf(y, c, x * s); }

// Two bf16 pairs packed as (x0, x1) in `lo` and (y0, y1) in `hi`, with (c0, s0, c1, s1).
__device__ __forceinline__ void rope_bf16x2(uint32_t& lo, uint32_t& hi, float c0, float s0, float c1,
                                            float s1) {
  const float x0 = __uint_as_float(lo << 16), x1 = __uint_as_float(lo & 0xFFFF0000u);
  const float y0 = __uint_as_float(hi << 16), y1 = __uint_as_float(hi & 0xFFFF0000u);
  lo = pack_bf16x2(rope_x(x0, y0, c0, s0), rope_x(x1, y1, c1, s1));
  hi = pack_bf16x2(rope_y(x0, y0, c0, s0), rope_y(x1, y1, c1, s1));
}

template <typename E>
__device__ __forceinline__ void rope_rotate_chunk(u32x4& lo, u32x4& hi, const float* cs) {
  if constexpr (E::kBytes == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t x = lo[w], y = hi[w];
      rope_bf16x2(x, y, cs[4 * w], cs[4 * w + 1], cs[4 * w + 2], cs[4 * w + 3]);
      lo[w] = x;
      hi[w] = y;
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float x = __uint_as_float(lo[w]), y = __uint_as_float(hi[w]);
      const float c = cs[2 * w], s = cs[2 * w + 1];
      lo[w] = __float_as_uint(rope_x(x, y, c, s));
      hi[w] = __float_as_uint(rope_y(x, y, c, s));
    }
  }
}

// Chunks of rotated dims per 32 dims (a pair's two elements sit in chunks j and j + kRopeH).
template <typename E>
inline constexpr int kRopeH = 32 / E::kPerChunk;

// Rotation of a 16-byte chunk whose partner chunk sits in another lane of the same wave. `ch` is
// the chunk's index within its head vector: chunks [0, H) hold dims 0..31, chunks [H, 2H) their
// partners (dims + 32), H = kRopeH<E>; other chunks are returned unchanged. The caller lays the
// chunks out so that the partner of chunk ch < H is at lane + H and that of chunk H <= ch < 2H at
// lane - H. cs holds the (cos, sin) of pairs (ch % H) * kPerChunk .. + kPerChunk - 1 at the
// vector's position (read only for rotated chunks). Every lane of the wave must call this: the
// exchange reads the partner lane. Both lanes of a pair do the arithmetic of rope_rotate_chunk.
template <typename E>
__device__ __forceinline__ u32x4 rope_chunk_xlane(u32x4 x, int ch, int lane, const float* cs) {
  constexpr int H = kRopeH<E>;
  const int src = ch < H ? lane + H : (ch < 2 * H ? lane - H : lane);
  u32x4 y;
#pragma unroll
  for (int j = 0; j < 4; ++j) y[j] = (uint32_t)__shfl((int)x[j], src, 64);
  if (ch < 2 * H) {
    u32x4 lo = ch < H ? x : y, hi = ch < H ? y : x;
    rope_rotate_chunk<E>(lo, hi, cs);
    x = ch < H ? lo : hi;
  }
  return x;
}

// Loads n (cos, sin) pairs, n a multiple of 2, for dims i0 .. i0 + n - 1 at table row `pos`.
template <int N>
__device__ __forceinline__ void rope_load(const float* table, int pos, int i0, float (&cs)[2 * N]) {
  const float* p = table + ((size_t)pos * (kRopeDims / 2) + i0) * 2;
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * j);
    cs[4 * j] = v[0]; cs[4 * j + 1] = v[1]; cs[4 * j + 2] = v[2]; cs[4 * j + 3] = v[3];
  }
}

// Rotates an MFMA fragment pair (8 elements of dims i0.. and of dims i0 + 32..) in place.
template <typename E, typename F>
__device__ __forceinline__ void rope_rotate_frag(F& lo, F& hi, const float (&cs)[16]) {
  if constexpr (E::kBytes == 2) {
    u32x4 a = __builtin_bit_cast(u32x4, lo), b = __builtin_bit_cast(u32x4, hi);
    rope_rotate_chunk<E>(a, b, cs);
    lo = __builtin_bit_cast(F, a);
    hi = __builtin_bit_cast(F, b);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = lo[e], y = hi[e], c = cs[2 * e], s = cs[2 * e + 1];
      lo[e] = rope_x(x, y, c, s);
      hi[e] = rope_y(x, y, c, s);
    }
  }
}

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Query heads grouped by KV head: heads[g * G + j] is the j-th query head served by KV head g.
// With the default map (identity set) that is g * G + j itself and the table is not read: a
// per-lane table read is a memory load whose wait would also hold back every load issued before it.
struct HeadList {
  int identity;
  int16_t heads[kMaxHeads];
  __device__ __forceinline__ int at(int i) const {
    if (identity) return i;
    return heads[i];
  }
};

}  // namespace mimo
