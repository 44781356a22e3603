// Prefill kernel: sink-seeded sliding-window / causal attention on gfx950 MFMA.
//
// Operation: MiMo-V2-Flash Technical Report review (xllm-io), §3.1 (window 128, GQA 64/8 and 64/4,
// head dims 192/128) and §3.2 (per-head sink logit in the softmax denominator); MiMo series notes
// (plmsmile), MiMo-V2-Flash > Learnable Attention Sink > mechanism (real-token weights may sum to
// less than one; the sink carries no value).
//
// Work decomposition (one workgroup = NW waves):
//   * A workgroup owns one KV head g of one sequence b, HG query heads of that group and
//     NW / HG tiles of 32 consecutive query positions. Every K/V block it stages in LDS is read
//     from HBM/L2 once and consumed by all of its waves, i.e. by every query head sharing g.
//   * Wave w owns query head (w % HG) and query tile (w / HG): 32 positions = 32 MFMA columns.
//   * The key loop covers only the union of the workgroup's windows, [P0 - W + 1, P1), in blocks
//     of BK keys, double-buffered in LDS; a block is skipped by a wave whose queries see none of it
//     and masked only when some (query, key) pair inside it is invisible.
//   * Scores are formed transposed, S^T = K Q^T, so that each lane holds one query column: row
//     max/sum need one cross-half exchange, and P^T feeds O^T += V^T P^T straight from registers.
//   * The online softmax starts from the sink: m = s_h * log2(e), l = 1, acc = 0 (no sink:
//     m = -inf, l = 0), so the sink is counted exactly once and never multiplied by the scale.
#include "launch.hpp"

namespace mimo {

constexpr int kDQK = 192;
constexpr int kDV = 128;
constexpr int kQT = 32;  // query positions per wave

template <typename E, int BK>
struct PrefillTile {
  static constexpr int kKStride = kDQK + 16 / E::kBytes;  // + 16 bytes: conflict-free b128 reads
  static constexpr int kVStride = BK + 4;                 // V^T rows, + 4 elements
  static constexpr int kKBytes = BK * kKStride * E::kBytes;
  static constexpr int kVBytes = kDV * kVStride * E::kBytes;
  static constexpr int kStageBytes = kKBytes + kVBytes;
  static_assert(kKBytes % 16 == 0 && kStageBytes % 16 == 0, "16-byte aligned stages");
};

// Global -> register -> LDS staging of one K block (row-major) and one V block (transposed).
template <typename E, int NT, int BK>
struct KVStager {
  using Tile = PrefillTile<E, BK>;
  static constexpr int kKChunksRow = kDQK / E::kPerChunk;
  static constexpr int kKChunks = BK * kKChunksRow;
  static constexpr int kKIt = (kKChunks + NT - 1) / NT;
  static constexpr int kVChunksRow = kDV / E::kPerChunk;
  static constexpr int kVUnits = (BK / 4) * kVChunksRow;  // unit = 4 keys x one 16-byte dv chunk
  static constexpr int kVIt = (kVUnits + NT - 1) / NT;

  u32x4 kr[kKIt];
  u32x4 vr[kVIt][4];

  __device__ __forceinline__ void load(const char* kbase, const char* vbase, size_t kstride,
                                       size_t vstride, int key0, int L, int tid) {
#pragma unroll
    for (int i = 0; i < kKIt; ++i) {
      const int c = tid + i * NT;
      kr[i] = zero_chunk();
      if (c < kKChunks) {
        const int key = key0 + c / kKChunksRow;
        if (key < L) kr[i] = ld16(kbase + (size_t)key * kstride + (c % kKChunksRow) * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < kVIt; ++i) {
      const int u = tid + i * NT;
#pragma unroll
      for (int r = 0; r < 4; ++r) vr[i][r] = zero_chunk();
      if (u < kVUnits) {
        const int key = key0 + 4 * (u / kVChunksRow);
        const size_t col = (size_t)(u % kVChunksRow) * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key + r < L) vr[i][r] = ld16(vbase + (size_t)(key + r) * vstride + col);
      }
    }
  }

  __device__ __forceinline__ void store(char* stage, int tid) const {
    char* sk = stage;
    char* sv = stage + Tile::kKBytes;
#pragma unroll
    for (int i = 0; i < kKIt; ++i) {
      const int c = tid + i * NT;
      if (c < kKChunks)
        st16(sk + ((c / kKChunksRow) * Tile::kKStride) * E::kBytes + (c % kKChunksRow) * 16, kr[i]);
    }
#pragma unroll
    for (int i = 0; i < kVIt; ++i) {
      const int u = tid + i * NT;
      if (u >= kVUnits) continue;
      const int kg = u / kVChunksRow;  // keys 4kg .. 4kg+3 of the block
      const int dc = u % kVChunksRow;  // dv elements dc*kPerChunk ..
      if constexpr (E::kBytes == 2) {
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const int w = d / 2;
          uint32_t e[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) e[r] = (d & 1) ? (vr[i][r][w] >> 16) : (vr[i][r][w] & 0xFFFFu);
          u32x2 out;
          out[0] = e[0] | (e[1] << 16);
          out[1] = e[2] | (e[3] << 16);
          *reinterpret_cast<u32x2*>(sv + ((dc * 8 + d) * Tile::kVStride + 4 * kg) * 2) = out;
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          u32x4 out;
#pragma unroll
          for (int r = 0; r < 4; ++r) out[r] = vr[i][r][d];
          st16(sv + ((dc * 4 + d) * Tile::kVStride + 4 * kg) * 4, out);
        }
      }
    }
  }
};

// A-operand fragment of K: key row `row`, contraction elements 16*kk + 8*half .. +7.
template <typename E, int BK>
__device__ __forceinline__ typename E::Frag lds_k_frag(const char* sk, int row, int kk, int half) {
  const char* p = sk + (row * PrefillTile<E, BK>::kKStride + 16 * kk + 8 * half) * E::kBytes;
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

// A-operand fragment of V^T: dv row `row`; elements 0..3 are keys 16ks+4h..+3, 4..7 are keys
// 16ks+8+4h..+3 (the key order in which the S^T accumulator holds P for this lane half).
template <typename E, int BK>
__device__ __forceinline__ typename E::Frag lds_vt_frag(const char* sv, int row, int ks, int half) {
  const char* p = sv + (row * PrefillTile<E, BK>::kVStride + 16 * ks + 4 * half) * E::kBytes;
  if constexpr (E::kBytes == 2) {
    const u32x2 a = *reinterpret_cast<const u32x2*>(p);
    const u32x2 b = *reinterpret_cast<const u32x2*>(p + 16);
    u32x4 u;
    u[0] = a[0]; u[1] = a[1]; u[2] = b[0]; u[3] = b[1];
    return __builtin_bit_cast(bf16x8, u);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 32);
    f32x8 f;
    f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
    f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
    return f;
  }
}

// B-operand fragment of Q^T straight from global memory: this lane's query row, elements
// 16*kk + 8*half .. +7 (zero for rows past the end of the sequence).
template <typename E>
__device__ __forceinline__ typename E::Frag global_q_frag(const char* qrow, bool valid, int kk,
                                                          int half) {
  const char* p = qrow + (16 * kk + 8 * half) * E::kBytes;
  if constexpr (E::kBytes == 2) {
    return __builtin_bit_cast(bf16x8, valid ? ld16(p) : zero_chunk());
  } else {
    const u32x4 a = valid ? ld16(p) : zero_chunk();
    const u32x4 b = valid ? ld16(p + 16) : zero_chunk();
    f32x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(a[i]);
      f[4 + i] = __uint_as_float(b[i]);
    }
    return f;
  }
}

template <typename E, int NW, int BK>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(const PrefillArgs a) {
  using Tile = PrefillTile<E, BK>;
  using Frag = typename E::Frag;
  constexpr int NT = NW * 64;
  constexpr int NSB = BK / 32;  // 32-key sub-blocks per block
  __shared__ __attribute__((aligned(16))) char smem[2 * Tile::kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = tid >> 6;

  // Heaviest query blocks (latest positions) are dispatched first.
  const int per_q = a.B * a.Hkv * a.n_hchunks;
  const int qb = a.n_qblocks - 1 - (int)(blockIdx.x / per_q);
  int rest = blockIdx.x % per_q;
  const int hc = rest % a.n_hchunks;
  rest /= a.n_hchunks;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;

  const int HG = a.heads_per_wg;
  const int qtiles = NW / HG;
  const int head = a.hl.heads[g * a.G + hc * HG + wave % HG];
  const int P0 = qb * kQT * qtiles;
  const int P1 = min(a.L, P0 + kQT * qtiles);
  const int p0 = P0 + kQT * (wave / HG);  // this wave's first query position
  const int qpos = p0 + col;              // this lane's query position

  const size_t krow_stride = (size_t)a.Hkv * kDQK * E::kBytes;
  const size_t vrow_stride = (size_t)a.Hkv * kDV * E::kBytes;
  const char* kbase = (const char*)a.k + ((size_t)b * a.L * a.Hkv + g) * kDQK * E::kBytes;
  const char* vbase = (const char*)a.v + ((size_t)b * a.L * a.Hkv + g) * kDV * E::kBytes;

  // Q^T fragments for the whole key loop.
  Frag qf[kDQK / 16];
  {
    const char* qrow = (const char*)a.q + (((size_t)b * a.L + qpos) * a.Hq + head) * kDQK * E::kBytes;
    const bool valid = qpos < a.L;
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) qf[kk] = global_q_frag<E>(qrow, valid, kk, half);
  }

  // Sink-seeded softmax state of this lane's query (identical in both lane halves).
  const float sink_l2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
  float m = sink_l2;
  float l = a.sink ? 1.f : 0.f;
  f32x16 acc[kDV / 32];
#pragma unroll
  for (int db = 0; db < kDV / 32; ++db) acc[db] = zero16();

  const int K0 = max(0, P0 - a.window + 1);
  const int kstart = (K0 / BK) * BK;
  const int nblk = (P1 - kstart + BK - 1) / BK;

  KVStager<E, NT, BK> st;
  st.load(kbase, vbase, krow_stride, vrow_stride, kstart, a.L, tid);
  st.store(smem, tid);
  __syncthreads();

  for (int ib = 0; ib < nblk; ++ib) {
    const int key0 = kstart + ib * BK;
    if (ib + 1 < nblk) st.load(kbase, vbase, krow_stride, vrow_stride, key0 + BK, a.L, tid);

    const bool skip = (key0 > p0 + kQT - 1) || (key0 + BK - 1 < p0 - a.window + 1) || (p0 >= a.L);
    if (!skip) {
      const char* sk = smem + (ib & 1) * Tile::kStageBytes;
      const char* sv = sk + Tile::kKBytes;
      const bool need_mask = !((key0 + BK - 1 <= p0) && (p0 + kQT - 1 - key0 < a.window));

      f32x16 s[NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        s[sb] = zero16();
#pragma unroll
        for (int kk = 0; kk < kDQK / 16; ++kk)
          s[sb] = mma(lds_k_frag<E, BK>(sk, 32 * sb + col, kk, half), qf[kk], s[sb]);
      }

      float bmax = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = s[sb][r] * a.scale_log2;
          if (need_mask) {
            const int key = key0 + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
            const int d = qpos - key;
            t = (d >= 0 && d < a.window) ? t : -INFINITY;
          }
          s[sb][r] = t;
          bmax = fmaxf(bmax, t);
        }
      }
      bmax = halves_max(bmax);
      const float m_new = fmaxf(m, bmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float rs = 0.f;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(s[sb][r] - m_use);
          s[sb][r] = p;
          rs += p;
        }
      }
      rs = halves_sum(rs);
      l = l * alpha + rs;
      m = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < kDV / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      }

#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const Frag pf = frag_from_acc<E>(s[ks >> 1], 8 * (ks & 1));
#pragma unroll
        for (int db = 0; db < kDV / 32; ++db)
          acc[db] = mma(lds_vt_frag<E, BK>(sv, 32 * db + col, ks, half), pf, acc[db]);
      }
    }

    if (ib + 1 < nblk) st.store(smem + ((ib + 1) & 1) * Tile::kStageBytes, tid);
    __syncthreads();
  }

  if (qpos < a.L) {
    const float inv = 1.f / l;
    char* orow = (char*)a.o + (((size_t)b * a.L + qpos) * a.Hq + head) * kDV * E::kBytes;
#pragma unroll
    for (int db = 0; db < kDV / 32; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int dv = 32 * db + 8 * gq + 4 * half;
        const float x0 = acc[db][4 * gq + 0] * inv, x1 = acc[db][4 * gq + 1] * inv;
        const float x2 = acc[db][4 * gq + 2] * inv, x3 = acc[db][4 * gq + 3] * inv;
        if constexpr (E::kBytes == 2) {
          u32x2 w;
          w[0] = pack_bf16x2(x0, x1);
          w[1] = pack_bf16x2(x2, x3);
          *reinterpret_cast<u32x2*>(orow + dv * 2) = w;
        } else {
          f32x4 w;
          w[0] = x0; w[1] = x1; w[2] = x2; w[3] = x3;
          *reinterpret_cast<f32x4*>(orow + dv * 4) = w;
        }
      }
    }
    if (a.lse && half == 0)
      a.lse[((size_t)b * a.Hq + head) * a.L + qpos] = (m + fast_log2(l)) * kLn2;
  }
}

template <typename E, int NW, int BK>
static hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  const long long n_wg = (long long)a.n_qblocks * a.B * a.Hkv * a.n_hchunks;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_kernel<E, NW, BK>), dim3((unsigned)n_wg), dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

// Picks the kernel variant; `a` arrives with everything but the tiling fields filled in.
hipError_t prefill_launch(bool bf16, PrefillArgs a, hipStream_t stream) {
  constexpr int NW = 8;
  int hg = 1;
  while (hg < NW && a.G % (hg * 2) == 0) hg *= 2;
  a.heads_per_wg = hg;
  a.n_hchunks = a.G / hg;
  const int rows_per_wg = kQT * (NW / hg);
  a.n_qblocks = (a.L + rows_per_wg - 1) / rows_per_wg;
  const bool global = a.window >= a.L;
  if (!bf16) return launch<F32, NW, 32>(a, stream);
  if (global) return launch<BF16, NW, 64>(a, stream);
  return launch<BF16, NW, 32>(a, stream);
}

}  // namespace mimo
