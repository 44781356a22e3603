// Tiles shared by the prefill and backward kernels: LDS layout of K/V blocks, the staging of a
// block from memory through registers into LDS, and the MFMA fragment readers and row writers.
#pragma once

#include "launch.hpp"

namespace mimo {

constexpr int kDQK = 192;
constexpr int kDV = 128;
constexpr int kQT = 32;  // query positions per wave

// LDS layout of one K/V block. K is row-major [key][dqk]. V is kept in one of three layouts:
// transposed [dv][key] (fp32 forward), row-major padded for the transposing LDS read (bf16
// forward), or row-major padded for plain 16-byte row reads (backward, both dtypes). Rows are
// padded so the MFMA operand reads hit distinct banks.
constexpr int kVTransposed = 0, kVRowsTr = 1, kVRows = 2;
template <typename E>
inline constexpr int kDefaultVLayout = E::kBytes == 2 ? kVRowsTr : kVTransposed;

template <typename E, int BK, int VL = kDefaultVLayout<E>>
struct PrefillTile {
  static constexpr bool kVRowMajor = VL != kVTransposed;
  static constexpr int kKStride = kDQK + 16 / E::kBytes;  // + 16 bytes: conflict-free b128 reads
  static constexpr int kVStride = VL == kVRowsTr ? kDV + 16 : (VL == kVRows ? kDV + 16 / E::kBytes : BK + 4);
  static constexpr int kKBytes = BK * kKStride * E::kBytes;
  static constexpr int kVBytes = (kVRowMajor ? BK : kDV) * kVStride * E::kBytes;
  static constexpr int kStageBytes = kKBytes + kVBytes;
  static_assert(kKBytes % 16 == 0 && kStageBytes % 16 == 0, "16-byte aligned stages");
};

// Global -> register -> LDS staging of one K block and one V block. Each thread moves a run of
// consecutive 16-byte chunks of one row (KPT of K, VPT of V), so it needs a single offset per
// tensor. For fp32 the V block is stored transposed ([dv][key]); there the chunks of thread t are
// t + i * NT with key = chunk % BK, so a wave's lanes cover consecutive keys of one dv range and
// its 4-byte transposed writes hit distinct banks.
// Rows at or past L are read from row L - 1 (finite data that the mask gives weight 0).
//
// ROPE (K arrives before the rotary embedding): thread j < H of a K row (H = chunks per 32 dims)
// then holds the partner chunks j and j + H (dims 8j.. and 8j + 32.. for bf16) plus KPT - 2 chunks
// of the unrotated dims, the other threads KPT chunks of the rest, and store() rotates the pair
// before writing LDS, with the (cos, sin) of its key position fetched by load() from the table in
// memory (kRopeMem) or read by store() from a [BK][32][2] table already in LDS (kRopeLds).
constexpr int kRopeNone = 0, kRopeMem = 1, kRopeLds = 2;

template <typename E, int NT, int BK, int ROPE = kRopeNone, int VL = kDefaultVLayout<E>>
struct KVStager {
  using Tile = PrefillTile<E, BK, VL>;
  static constexpr int kKChunksRow = kDQK / E::kPerChunk;
  static constexpr int KPT = (BK * kKChunksRow + NT - 1) / NT;  // K chunks per thread
  static_assert(kKChunksRow % KPT == 0, "a thread's K chunks stay in one row");
  static constexpr int kKTpr = kKChunksRow / KPT;  // threads per K row
  static constexpr int H = kRopeDims / 2 / E::kPerChunk;  // chunks in 32 dims
  static_assert(ROPE == kRopeNone || (KPT >= 2 && kKTpr >= H), "each rotated chunk pair fits one thread");
  // chunk (within the row) of this thread's i-th K chunk; j = thread index within the row
  __device__ static constexpr int kchunk(int j, int i) {
    if (!ROPE) return j * KPT + i;
    if (j < H) return i == 0 ? j : (i == 1 ? j + H : 2 * H + j * (KPT - 2) + (i - 2));
    return 2 * H + H * (KPT - 2) + (j - H) * KPT + i;
  }
  static constexpr int kKActive = BK * kKTpr;
  static_assert(kKActive <= NT, "one pass covers the K block");
  static constexpr int kVChunksRow = kDV / E::kPerChunk;
  static constexpr int VPT = (BK * kVChunksRow + NT - 1) / NT;  // V chunks per thread
  static_assert(!Tile::kVRowMajor || kVChunksRow % VPT == 0, "a thread's V chunks stay in one row");
  static constexpr int kVTpr = kVChunksRow / VPT;
  static constexpr int kVActive = Tile::kVRowMajor ? BK * kVTpr : NT;

  u32x4 kr[KPT];
  u32x4 vr[VPT];
  uint32_t koff, voff[Tile::kVRowMajor ? 1 : VPT];
  int krow, vrow;
  float cs[ROPE == kRopeMem ? 2 * E::kPerChunk : 1];  // (cos, sin) of this thread's rotated dims

  __device__ __forceinline__ void init(size_t kstride, size_t vstride, int tid) {
    krow = min(tid / kKTpr, BK - 1);
    koff = ROPE ? (uint32_t)(krow * kstride) : (uint32_t)(krow * kstride + (tid % kKTpr) * KPT * 16);
    if constexpr (Tile::kVRowMajor) {
      vrow = min(tid / kVTpr, BK - 1);
      voff[0] = (uint32_t)(vrow * vstride + (tid % kVTpr) * VPT * 16);
    } else {
      vrow = 0;
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = tid + i * NT;
        voff[i] = (uint32_t)((c % BK) * vstride + (c / BK) * 16);
      }
    }
  }

  // Loads the block starting at key0; only a block that reaches past L clamps its rows.
  __device__ __forceinline__ void load(const char* kbase, const char* vbase, size_t kstride,
                                       size_t vstride, int key0, int L, int tid,
                                       const float* rope = nullptr) {
    const bool tail = key0 + BK > L;
    {  // every thread loads (the spare ones re-read a chunk of the last row; only store() skips them)
      const char* p = kbase + (size_t)key0 * kstride + koff;
      if (tail) p += ((size_t)min(key0 + krow, L - 1) - (key0 + krow)) * kstride;
      if constexpr (ROPE != kRopeNone) {
        const int j = tid % kKTpr;
#pragma unroll
        for (int i = 0; i < KPT; ++i) kr[i] = ld16(p + 16 * kchunk(j, i));
        // the table row of this thread's key (spare and unrotating threads read a valid one)
        if constexpr (ROPE == kRopeMem)
          rope_load<E::kPerChunk>(rope, min(key0 + krow, L - 1), (j < H ? j : 0) * E::kPerChunk, cs);
      } else {
#pragma unroll
        for (int i = 0; i < KPT; ++i) kr[i] = ld16(p + 16 * i);
      }
    }
    if constexpr (Tile::kVRowMajor) {
      if (tid < kVActive) {
        const char* p = vbase + (size_t)key0 * vstride + voff[0];
        if (tail) p += ((size_t)min(key0 + vrow, L - 1) - (key0 + vrow)) * vstride;
#pragma unroll
        for (int i = 0; i < VPT; ++i) vr[i] = ld16(p + 16 * i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = tid + i * NT;
        if (c >= BK * kVChunksRow) continue;
        const int key = key0 + c % BK;
        const char* p = vbase + (size_t)key0 * vstride + voff[i];
        if (tail) p += ((size_t)min(key, L - 1) - key) * vstride;
        vr[i] = ld16(p);
      }
    }
  }

  __device__ __forceinline__ void store(char* stage, int tid, const char* lds_table = nullptr) {
    char* sk = stage;
    char* sv = stage + Tile::kKBytes;
    if constexpr (ROPE != kRopeNone) {
      const int j = tid % kKTpr;
      if constexpr (ROPE == kRopeLds) {
        if (j < H) {
          float c[2 * E::kPerChunk];
          const float* t = reinterpret_cast<const float*>(lds_table) + (krow * (kRopeDims / 2) + j * E::kPerChunk) * 2;
#pragma unroll
          for (int w = 0; w < E::kPerChunk / 2; ++w) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(t + 4 * w);
            c[4 * w] = v[0]; c[4 * w + 1] = v[1]; c[4 * w + 2] = v[2]; c[4 * w + 3] = v[3];
          }
          rope_rotate_chunk<E>(kr[0], kr[1], c);
        }
      } else {
        if (j < H) rope_rotate_chunk<E>(kr[0], kr[1], cs);
      }
      if (tid < kKActive) {
        char* d = sk + (krow * Tile::kKStride) * E::kBytes;
#pragma unroll
        for (int i = 0; i < KPT; ++i) st16(d + 16 * kchunk(j, i), kr[i]);
      }
    } else if (tid < kKActive) {
      char* d = sk + (krow * Tile::kKStride) * E::kBytes + (tid % kKTpr) * KPT * 16;
#pragma unroll
      for (int i = 0; i < KPT; ++i) st16(d + 16 * i, kr[i]);
    }
    if constexpr (Tile::kVRowMajor) {
      if (tid < kVActive) {
        char* d = sv + (vrow * Tile::kVStride) * E::kBytes + (tid % kVTpr) * VPT * 16;
#pragma unroll
        for (int i = 0; i < VPT; ++i) st16(d + 16 * i, vr[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = tid + i * NT;
        if (c >= BK * kVChunksRow) continue;
        uint32_t* dst = reinterpret_cast<uint32_t*>(sv) + (c / BK) * 4 * Tile::kVStride + c % BK;
#pragma unroll
        for (int d = 0; d < 4; ++d) dst[d * Tile::kVStride] = vr[i][d];
      }
    }
  }
};

// Global -> LDS staging of one bf16 K/V block without a register pass (the 16-byte
// global_load_lds of gfx950: lane i of one instruction writes LDS bytes [16 i, 16 i + 16) past the
// instruction's base; lanes that are switched off write nothing). The stage keeps PrefillTile's
// padded rows: instruction u covers LDS chunks 64 u .. 64 u + 63 of the K region (kKRow chunks per
// row, the last one padding) or of the V region; a lane whose chunk is padding re-reads a data
// chunk of its row, so every lane's address is valid, and in a region's last instruction the
// lanes past the region are switched off. The instructions are dealt round-robin to the NW waves.
// Rows at or past L are read from row L - 1. The caller waits for the loads (vmcnt) before the
// barrier that publishes the stage.
template <int NW, int BK, int VL = kVRowsTr>
struct KVStagerDMA {
  using Tile = PrefillTile<BF16, BK, VL>;
  static constexpr int kKRow = Tile::kKStride * 2 / 16, kVRow = Tile::kVStride * 2 / 16;  // chunks per row
  static constexpr int kKChunks = BK * kKRow, kVChunks = BK * kVRow;
  static constexpr int kKInst = (kKChunks + 63) / 64, kVInst = (kVChunks + 63) / 64;
  static_assert(kKChunks * 16 == Tile::kKBytes && kVChunks * 16 == Tile::kVBytes, "regions tile the stage");
  static_assert(Tile::kVRowMajor, "row-major V");
  static constexpr int kInst = kKInst + kVInst;
  static constexpr int kPer = (kInst + NW - 1) / NW;  // instruction slots per wave
  uint32_t off[kPer];  // byte offset of this lane's chunk from the block's first row (row 0 = key0)

  // row and data chunk of lane `lane` in instruction u; false for a lane past its region
  __device__ static bool row_chunk(int u, int lane, int& row, int& ch) {
    const bool is_k = u < kKInst;
    const int p = 64 * (is_k ? u : u - kKInst) + lane;
    const int n = is_k ? kKChunks : kVChunks, per = is_k ? kKRow : kVRow;
    const int pc = min(p, n - 1);
    row = pc / per;
    ch = min(pc % per, (is_k ? kDQK : kDV) / 8 - 1);
    return p < n;
  }

  __device__ __forceinline__ void init(size_t kstride, size_t vstride, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = min(wave + i * NW, kInst - 1);
      int row, ch;
      row_chunk(u, lane, row, ch);
      off[i] = (uint32_t)(row * (u < kKInst ? kstride : vstride) + ch * 16);
    }
  }

  // Issues this wave's loads of the block starting at key0 into `stage`. Only a block that reaches
  // past L needs the lane's row again (integer divisions): a uniform branch around it.
  __device__ __forceinline__ void load(char* stage, const char* kbase, const char* vbase, size_t kstride,
                                       size_t vstride, int key0, int L, int wave, int lane) const {
    const bool tail = key0 + BK > L;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = wave + i * NW;
      if (u >= kInst) break;  // uniform per wave
      const bool is_k = u < kKInst;
      const char* p = (is_k ? kbase + (size_t)key0 * kstride : vbase + (size_t)key0 * vstride) + off[i];
      if (tail) {
        int row, ch;
        row_chunk(u, lane, row, ch);
        p += ((size_t)min(key0 + row, L - 1) - (key0 + row)) * (is_k ? kstride : vstride);
      }
      char* dst = stage + (is_k ? 1024 * u : Tile::kKBytes + 1024 * (u - kKInst));
      const bool partial = is_k ? (u == kKInst - 1 && kKChunks % 64) : (u == kInst - 1 && kVChunks % 64);
      const bool active = 64 * (is_k ? u : u - kKInst) + lane < (is_k ? kKChunks : kVChunks);
      if (!partial || active)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)p,
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  }
};

// Global -> LDS staging (16-byte global_load_lds) of ROWS consecutive rows of one bf16 tensor into
// a padded LDS region of RC 16-byte chunks per row (the first DC of them data), by a group of NWG
// waves: instruction u covers region chunks 64 u .. 64 u + 63 and is issued by wave u % NWG of the
// group. A lane whose chunk is padding re-reads a data chunk of its row; in the last instruction
// the lanes past the region are switched off. Rows at or past L are read from row L - 1. The caller
// waits for the loads (vmcnt) before the barrier that publishes the region. The caller also holds
// the lane's offsets (off[i]: byte offset of its chunk in instruction i from row 0 of the block),
// so that wave groups staging different tensors can share one register array.
template <int NWG, int ROWS, int RC, int DC>
struct RowsDMA {
  static constexpr int kChunks = ROWS * RC;
  static constexpr int kInst = (kChunks + 63) / 64;
  static constexpr int kPer = (kInst + NWG - 1) / NWG;  // instructions per wave (at most)

  __device__ static int row_chunk(int u, int lane, int& ch) {
    const int p = min(64 * u + lane, kChunks - 1);
    ch = min(p % RC, DC - 1);
    return p / RC;
  }
  __device__ __forceinline__ static void init(uint32_t* off, size_t stride, int w, int lane) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int ch;
      const int row = row_chunk(min(w + i * NWG, kInst - 1), lane, ch);
      off[i] = (uint32_t)(row * stride + ch * 16);
    }
  }
  // Issues wave w's loads of rows row0 .. row0 + ROWS - 1 into `region`; only a block that reaches
  // past L needs each lane's row again (a uniform branch around it).
  __device__ __forceinline__ static void load(const uint32_t* off, char* region, const char* base, size_t stride,
                                              int row0, int L, int w, int lane) {
    const bool tail = row0 + ROWS > L;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = w + i * NWG;
      if (u >= kInst) break;  // uniform per wave
      const char* p = base + (size_t)row0 * stride + off[i];
      if (tail) {
        int ch;
        const int row = row_chunk(u, lane, ch);
        p += ((size_t)min(row0 + row, L - 1) - (row0 + row)) * stride;
      }
      if (kChunks % 64 == 0 || u < kInst - 1 || 64 * u + lane < kChunks)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)p,
                                         (__attribute__((address_space(3))) void*)(region + 1024 * u), 16, 0, 0);
    }
  }
};

// Waits for this wave's outstanding global loads, including global -> LDS loads (vmcnt 0; expcnt
// and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// MFMA fragment of a row-major LDS tile (row stride `stride` elements): row `row`, elements
// 16*kk + 8*half .. +7. Serves as the A operand (lane = row) or the B operand (lane = column).
template <typename E>
__device__ __forceinline__ typename E::Frag lds_row_frag(const char* tile, int stride, int row, int kk,
                                                        int half) {
  const char* p = tile + (row * stride + 16 * kk + 8 * half) * E::kBytes;
  if constexpr (E::kBytes == 2) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 16);
    f32x8 f;
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
  }
}

// A-operand fragment of K: key row `row`, contraction elements 16*kk + 8*half .. +7.
template <typename E, int BK>
__device__ __forceinline__ typename E::Frag lds_k_frag(const char* sk, int row, int kk, int half) {
  return lds_row_frag<E>(sk, PrefillTile<E, BK>::kKStride, row, kk, half);
}

// Fragment of the transpose of a row-major LDS tile [r][c] (row stride `stride` elements): this
// lane's row of the transpose is column c = 32 dt + lane % 32; its 8 elements are rows
// 16 ks + 4 half + 0..3 and 16 ks + 8 + 4 half + 0..3 (the order in which a 32 x 32 accumulator
// holds its rows for this lane half, so the accumulator can be the other operand).
template <typename E>
__device__ __forceinline__ typename E::Frag lds_t_frag(const char* tile, int stride, int dt, int ks,
                                                      int lane) {
  if constexpr (E::kBytes == 2) {
    return vt_frag_tr(tile, stride, dt, ks, lane);
  } else {
    const int half = lane >> 5, c = 32 * dt + (lane & 31);
    const float* t = reinterpret_cast<const float*>(tile);
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 16 * ks + 4 * half + (e & 3) + (e >> 2) * 8;
      f[e] = t[r * stride + c];
    }
    return f;
  }
}

// A-operand fragment of V^T: dv row 32 db + lane % 32; elements 0..3 are keys 16ks+4h..+3,
// 4..7 are keys 16ks+8+4h..+3 (the key order in which the S^T accumulator holds P for this lane
// half).
template <typename E, int BK, int VL = kDefaultVLayout<E>>
__device__ __forceinline__ typename E::Frag lds_vt_frag(const char* sv, int db, int ks, int lane) {
  using Tile = PrefillTile<E, BK, VL>;
  if constexpr (Tile::kVRowMajor) {
    return vt_frag_tr(sv, Tile::kVStride, db, ks, lane);
  } else {
    const int half = lane >> 5, row = 32 * db + (lane & 31);
    const char* p = sv + (row * Tile::kVStride + 16 * ks + 4 * half) * E::kBytes;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 32);
    f32x8 f;
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
  }
}

// B-operand fragment of Q^T from global memory: elements 16*kk + 8*half .. +7 of a query row.
template <typename E>
__device__ __forceinline__ typename E::Frag global_q_frag(const char* qrow, int kk, int half) {
  const char* p = qrow + (16 * kk + 8 * half) * E::kBytes;
  if constexpr (E::kBytes == 2) {
    return __builtin_bit_cast(bf16x8, ld16(p));
  } else {
    const u32x4 a = ld16(p);
    const u32x4 b = ld16(p + 16);
    f32x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(a[i]);
      f[4 + i] = __uint_as_float(b[i]);
    }
    return f;
  }
}

// Writes one output row from O^T registers; every lane calls it, lanes with !store write nothing.
// acc[t][r] holds element 32 t + 8 (r / 4) + 4 half + r % 4 of the row; N tiles of 32 elements.
template <typename E, int N>
__device__ __forceinline__ void store_out_row(char* orow, const f32x16 (&acc)[N], float inv,
                                              int half, bool store) {
  if constexpr (E::kBytes == 2) {
    store_row_bf16(orow, acc, inv, half, store);
  } else {
    if (!store) return;
#pragma unroll
    for (int db = 0; db < N; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        f32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = acc[db][4 * gq + i] * inv;
        *reinterpret_cast<f32x4*>(orow + (32 * db + 8 * gq + 4 * half) * 4) = w;
      }
    }
  }
}

}  // namespace mimo
