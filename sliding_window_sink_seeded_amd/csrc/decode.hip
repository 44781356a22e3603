// Decode / MTP-verify kernels: a few new tokens per sequence against a ring (sliding-window) or
// linear (global) KV cache, split-KV with a sink-once combine.
//
// Operation: MiMo-V2-Flash Technical Report review (xllm-io), §3.1-§3.2 (window, GQA, head dims,
// per-head sink); MiMo series notes (plmsmile), MiMo-V2-Flash > local window (the sliding-window
// cache does not grow with history) and > lightweight MTP > inference (the main model verifies the
// drafted tokens in parallel, so one step carries 1 + drafts queries per sequence).
//
// Keys of sequence b: committed positions [max(0, P - W + 1), P) read from slot (p + off) mod C,
// and the T new tokens at positions P .. P+T-1. New token t sees positions in [P + t - W + 1,
// P + t]. The committed keys are processed in 32-key MFMA blocks; the new tokens (at most 8: the
// next token plus drafts, e.g. blocks of 6 or 8) are folded in afterwards by the last split, new
// token t by wave t % 4, as one extra key per column computed on the VALU (bf16 dot2). For a
// 128-key window this keeps the committed keys at exactly four blocks, one per wave, instead of a
// fifth, nearly empty block on one wave.
//
// Work decomposition: one workgroup per (split, KV head g, column chunk, sequence b). The G*T query
// columns of (b, g) - every query head of the group times every new token - are the MFMA columns
// (32 per column block, at most two blocks per workgroup; more columns, e.g. 16 heads x 8 tokens,
// are cut into chunks of 64 that run as separate workgroups), so each K/V element read from HBM
// serves all the columns of a chunk; Q^T sits in LDS, shared by the waves. The split's keys are cut into 32-key blocks dealt round-robin to the waves. Lane
// (col, half) of a wave fetches half of the K row and half of the V row of key key0 + col: the K
// half is directly its MFMA A fragment, the V half goes to a wave-private LDS tile that the PV
// product reads back transposed.
// The next block's fetch is issued before the current block's math (register double buffer).
// A wave keeps an online softmax per column (no sink here), then the waves of the workgroup
// merge through LDS in a fixed order:
//   * single pass (one split): the sink joins the merge and O / LSE are written;
//   * several splits: the merged, unnormalised (m, l, acc) go to the workspace and
//     combine_kernel folds the splits and the sink (counted once) into O / LSE.
// Keys past the end of the split are fetched from its last key (finite data, masked to weight 0).
// The running max is refreshed lazily (see update_max).
#include "launch.hpp"

namespace mimo {

constexpr int kDDQK = 192;
constexpr int kDDV = 128;
constexpr int kDecNW = 4;  // waves per workgroup
// split partial record of one query column: acc[kDDV], m, l, two pad floats (16-byte rows)
constexpr int kRec = kDDV + 4;

template <typename E, int NCB>
struct DecodeLds {
  static constexpr int kQStride = kDDQK + 16 / E::kBytes;  // Q^T rows (one per column), padded
  static constexpr int kQBytes = NCB * 32 * kQStride * E::kBytes;
  // one 32-key V block per wave: row-major [key][dv] for bf16 (read with the transposing LDS
  // read), transposed [dv][key] for fp32; padded so operand reads hit distinct banks
  static constexpr bool kVRowMajor = E::kBytes == 2;
  static constexpr int kVStride = kVRowMajor ? kDDV + 16 : 32 + 4;
  static constexpr int kVBytes = (kVRowMajor ? 32 : kDDV) * kVStride * E::kBytes;
  static constexpr int kMergeBytes = kDecNW * 2 * 16 * 64 * 4;  // two dv blocks of one column block
  static constexpr int kWorkBytes = kDecNW * kVBytes > kMergeBytes ? kDecNW * kVBytes : kMergeBytes;
  // K and V rows of new tokens 0..3, staged with Q at kernel start (tokens 4..7 of a block draft
  // go to the work area after the key loop, which keeps the ring kernel at three workgroups per CU)
  static constexpr int kNewKBytes = 4 * kDDQK * E::kBytes;
  static constexpr int kNewBytes = kNewKBytes + 4 * kDDV * E::kBytes;
  static_assert(4 * (kDDQK + kDDV) * E::kBytes <= kDecNW * kVBytes, "tokens 4..7 fit the V tiles");
  static constexpr int kBytes = kQBytes + kNewBytes + kWorkBytes + kDecNW * 64 * 4 * 2;
};

// One lane's share of a 32-key block: half of the K row (its MFMA A fragments) and half of the V
// row (dv chunks 2i + half) of key key0 + col.
template <typename E>
struct KeyRows {
  static constexpr int kKChunks = kDDQK / E::kPerChunk / 2;  // 16-byte chunks per lane
  static constexpr int kVChunks = kDDV / E::kPerChunk / 2;
  u32x4 k[kKChunks];
  u32x4 v[kVChunks];

  __device__ __forceinline__ void load(const char* krow, const char* vrow, int half) {
    // K chunk j: elements 8*(2*(j / (8/kPerChunk... ))) - laid out so that fragment kk of this
    // half is chunk(s) of bytes [(16*kk + 8*half) * bytes, +8 elements)
#pragma unroll
    for (int j = 0; j < kKChunks; ++j) {
      const int kk = j / (8 / E::kPerChunk);
      const int sub = j % (8 / E::kPerChunk);
      k[j] = ld16(krow + (16 * kk + 8 * half) * E::kBytes + 16 * sub);
    }
#pragma unroll
    for (int i = 0; i < kVChunks; ++i) v[i] = ld16(vrow + (2 * i + half) * 16);
  }

  __device__ __forceinline__ typename E::Frag kfrag(int kk) const {
    if constexpr (E::kBytes == 2) {
      return __builtin_bit_cast(bf16x8, k[kk]);
    } else {
      f32x8 f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = __uint_as_float(k[2 * kk][i]);
        f[4 + i] = __uint_as_float(k[2 * kk + 1][i]);
      }
      return f;
    }
  }

  // This lane's V chunks (key = col, dv chunks 2i + half) -> the wave's V tile.
  __device__ __forceinline__ void store_v(char* vt, int col, int half) const {
    using L = DecodeLds<E, 1>;
    constexpr int S = L::kVStride;
#pragma unroll
    for (int i = 0; i < kVChunks; ++i) {
      const int dv0 = (2 * i + half) * E::kPerChunk;
      if constexpr (L::kVRowMajor) {
        st16(vt + (col * S + dv0) * E::kBytes, v[i]);
      } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(vt) + dv0 * S + col;
#pragma unroll
        for (int d = 0; d < 4; ++d) dst[d * S] = v[i][d];
      }
    }
  }
};

// Staging of Q^T (one row per query column: head j of the group x new token t, column c = j * T + t,
// padded columns zero) and of the K/V rows of new tokens 0..3 (tokens 4..7 of a block draft are
// staged later by the caller). load() issues every global load of the thread, store() writes them
// to LDS; a caller issues its first K/V block fetch in between. A non-default head map is read
// before any other load, so that waiting for it waits for nothing else.
template <typename E, int NCB>
struct QStage {
  using Lds = DecodeLds<E, NCB>;
  static constexpr int kChunksRow = kDDQK / E::kPerChunk;
  static constexpr int kQChunks = NCB * 32 * kChunksRow;
  static constexpr int kQPer = (kQChunks + kDecNW * 64 - 1) / (kDecNW * 64);
  static constexpr int kKCh = kDDQK / E::kPerChunk, kVCh = kDDV / E::kPerChunk;
  static constexpr int kNewPer = (4 * (kKCh + kVCh) + kDecNW * 64 - 1) / (kDecNW * 64);
  u32x4 xq[kQPer], xn[kNewPer];

  __device__ __forceinline__ void load(const DecodeArgs& a, int tid, int b, int g, int cbase, int ncols) {
    const size_t krow_bytes = (size_t)kDDQK * E::kBytes, vrow_bytes = (size_t)kDDV * E::kBytes;
    int head[kQPer];
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int c = cbase + min((tid + i * kDecNW * 64) / kChunksRow, ncols - 1);  // padding: any valid row
      head[i] = g * a.G + c / a.T;
    }
    if (!a.hl.identity) {
#pragma unroll
      for (int i = 0; i < kQPer; ++i) head[i] = a.hl.heads[head[i]];
    }
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int u = tid + i * kDecNW * 64;
      const int c = cbase + min(u / kChunksRow, ncols - 1), ch = u % kChunksRow;
      xq[i] = ld16((const char*)a.q + (((size_t)b * a.T + c % a.T) * a.Hq + head[i]) * krow_bytes + ch * 16);
    }
#pragma unroll
    for (int i = 0; i < kNewPer; ++i) {
      const int u = tid + i * kDecNW * 64;
      const int t = min(u / (kKCh + kVCh), a.T - 1), ch = u % (kKCh + kVCh);
      const char* src = ch < kKCh
                            ? (const char*)a.k_new + (((size_t)b * a.T + t) * a.Hkv + g) * krow_bytes + ch * 16
                            : (const char*)a.v_new + (((size_t)b * a.T + t) * a.Hkv + g) * vrow_bytes +
                                  (ch - kKCh) * 16;
      xn[i] = ld16(src);
    }
  }

  // Q^T rows at smem, new tokens 0..3 (K rows, then V rows) right after them; the new tokens only
  // when `last` (the split that folds them in)
  __device__ __forceinline__ void store(char* smem, int tid, int ncols, bool last, int T) const {
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int u = tid + i * kDecNW * 64;
      const int c = u / kChunksRow, ch = u % kChunksRow;
      if (u < kQChunks) st16(smem + c * Lds::kQStride * E::kBytes + ch * 16, c < ncols ? xq[i] : zero_chunk());
    }
    char* snew = smem + Lds::kQBytes;
#pragma unroll
    for (int i = 0; i < kNewPer; ++i) {
      const int u = tid + i * kDecNW * 64;
      const int t = u / (kKCh + kVCh), ch = u % (kKCh + kVCh);
      if (last && u < 4 * (kKCh + kVCh) && t < T) {
        if (ch < kKCh)
          st16(snew + t * kDDQK * E::kBytes + ch * 16, xn[i]);
        else
          st16(snew + Lds::kNewKBytes + t * kDDV * E::kBytes + (ch - kKCh) * 16, xn[i]);
      }
    }
  }
};

// q and k_new arrive before the rotary embedding: rotate the staged Q^T rows and (last split) the
// staged new-token K rows in LDS, query column c (token c % T) and new token t at positions
// P + c % T and P + t; pairs (i, i + 32), i < 32. The caller synchronises before and after.
template <typename E, int NCB>
__device__ __forceinline__ void rope_staged(const DecodeArgs& a, char* smem, int tid, int P, int cbase,
                                            int ncols, bool last) {
  using Lds = DecodeLds<E, NCB>;
  constexpr int kHalfRot = kRopeDims / 2;
  const int n_q = ncols * kHalfRot, n_k = last ? a.T * kHalfRot : 0;
  for (int u = tid; u < n_q + n_k; u += kDecNW * 64) {
    const bool is_q = u < n_q;
    const int uu = is_q ? u : u - n_q;
    const int row = uu / kHalfRot, i = uu % kHalfRot;
    const int pos = P + (is_q ? (cbase + row) % a.T : row);
    char* base = is_q ? smem + row * Lds::kQStride * E::kBytes : smem + Lds::kQBytes + row * kDDQK * E::kBytes;
    const f32x2 csn = *reinterpret_cast<const f32x2*>(a.rope + ((size_t)pos * kHalfRot + i) * 2);
    if constexpr (E::kBytes == 2) {
      uint16_t* e = reinterpret_cast<uint16_t*>(base);
      const float x = __uint_as_float((uint32_t)e[i] << 16), y = __uint_as_float((uint32_t)e[i + kHalfRot] << 16);
      e[i] = (uint16_t)bf16_bits(x * csn[0] - y * csn[1]);
      e[i + kHalfRot] = (uint16_t)bf16_bits(y * csn[0] + x * csn[1]);
    } else {
      float* e = reinterpret_cast<float*>(base);
      const float x = e[i], y = e[i + kHalfRot];
      e[i] = x * csn[0] - y * csn[1];
      e[i + kHalfRot] = y * csn[0] + x * csn[1];
    }
  }
}


// With one bf16 column block, asking for two waves per SIMD makes the compiler keep the
// accumulators in VGPRs (169 registers, no AGPR copies) instead of 137 VGPRs + 80 AGPRs; both give
// two waves per SIMD, the first runs faster (ring workload).
template <typename E, int NCB, bool PREFETCH, bool ROPE>
__global__ __launch_bounds__(kDecNW * 64)
__attribute__((amdgpu_waves_per_eu(NCB == 1 && E::kBytes == 2 ? 2 : 1))) void decode_kernel(const DecodeArgs a) {
  using Frag = typename E::Frag;
  using Lds = DecodeLds<E, NCB>;
  __shared__ __attribute__((aligned(16))) char smem[Lds::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on it

  const int split = blockIdx.x;
  const int chunk = blockIdx.y % a.n_chunks;
  const int g = blockIdx.y / a.n_chunks;
  const int b = blockIdx.z;
  // this workgroup's query columns: cbase + [0, ncols) of the G*T columns of (b, g)
  const int cbase = chunk * a.chunk_cols;
  const int ncols = min(a.chunk_cols, a.ncols - cbase);

  int P = a.cache_len[b];
  P = P < 0 ? 0 : (P > a.max_len ? a.max_len : P);
  const int off = a.cache_offset ? a.cache_offset[b] : 0;
  // committed keys [list0, P) are split into ranges of keys_per_split (a multiple of 32); the
  // T new tokens are folded in by the last split, one token per wave, on the VALU
  const int list0 = max(0, P - a.window + 1);
  const int s0 = list0 + split * a.keys_per_split;
  const int s1 = min(P, s0 + a.keys_per_split);

  const size_t krow_bytes = (size_t)kDDQK * E::kBytes;
  const size_t vrow_bytes = (size_t)kDDV * E::kBytes;
  const char* kc = (const char*)a.k_cache + (size_t)g * krow_bytes;
  const char* vc = (const char*)a.v_cache + (size_t)g * vrow_bytes;
  const size_t kstride = (size_t)a.Hkv * krow_bytes;  // between positions
  const size_t vstride = (size_t)a.Hkv * vrow_bytes;
  const size_t cache_row0 = (size_t)b * a.C;

  // K and V row addresses of this lane's key in the block starting at key0 (clamped into the split)
  auto rows = [&](int key0, const char*& krow, const char*& vrow) {
    const int pos = min(key0 + col, s1 - 1);
    int slot = (pos + off) % a.C;
    slot += slot < 0 ? a.C : 0;
    krow = kc + (cache_row0 + slot) * kstride;
    vrow = vc + (cache_row0 + slot) * vstride;
  };

  KeyRows<E> cur;
  int key0 = s0 + 32 * wave;

  // Q^T of every query column and (last split) the new tokens' K/V rows of this (b, g) go to LDS;
  // the first K/V block's fetch is issued between the loads and the LDS stores so that its
  // latency overlaps them.
  char* sq = smem;
  {
    QStage<E, NCB> st;
    st.load(a, tid, b, g, cbase, ncols);
    if (key0 < s1) {
      const char *kr, *vr;
      rows(key0, kr, vr);
      cur.load(kr, vr, half);
    }
    st.store(smem, tid, ncols, split == a.nsplit - 1, a.T);
  }

  int qpos[NCB];
  float m[NCB], l[NCB];
  f32x16 acc[NCB][kDDV / 32];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int c = cb * 32 + col;
    qpos[cb] = c < ncols ? P + (cbase + c) % a.T : -(1 << 30);  // padding columns see no key
    m[cb] = -INFINITY;
    l[cb] = 0.f;
#pragma unroll
    for (int db = 0; db < kDDV / 32; ++db) acc[cb][db] = zero16();
  }

  // Lazy running max (log2 units): rescale l and acc only when some lane's candidate max exceeds
  // its running max by more than 8; otherwise exponentiate against the stale max (exact: the same
  // max scales l and acc).
  auto update_max = [&](int cb, float mb) {
    if (__builtin_amdgcn_ballot_w64(mb > m[cb] + 8.f || (m[cb] == -INFINITY && mb > m[cb])) != 0) {
      const float m_new = fmaxf(m[cb], mb);
      const float alpha = fast_exp2(m[cb] - (m_new == -INFINITY ? 0.f : m_new));
      l[cb] *= alpha;
#pragma unroll
      for (int db = 0; db < kDDV / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][db][r] *= alpha;
      m[cb] = m_new;
    }
  };

  char* work = smem + Lds::kQBytes + Lds::kNewBytes;
  char* my_vt = work + wave * Lds::kVBytes;
  __syncthreads();  // Q^T and the new-token rows are in LDS

  if constexpr (ROPE) {
    rope_staged<E, NCB>(a, smem, tid, P, cbase, ncols, split == a.nsplit - 1);
    __syncthreads();
  }

  for (; key0 < s1; key0 += 32 * kDecNW) {
    cur.store_v(my_vt, col, half);
    KeyRows<E> nxt;
    const int key_next = key0 + 32 * kDecNW;
    if (PREFETCH && key_next < s1) {
      const char *kr, *vr;
      rows(key_next, kr, vr);
      nxt.load(kr, vr, half);
    }

    // S^T = K Q^T for every column block
    f32x16 s[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) s[cb] = zero16();
#pragma unroll
    for (int kk = 0; kk < kDDQK / 16; ++kk) {
      const Frag kf = cur.kfrag(kk);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const char* qp = sq + ((cb * 32 + col) * Lds::kQStride + 16 * kk + 8 * half) * E::kBytes;
        Frag qf;
        if constexpr (E::kBytes == 2) {
          qf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp));
        } else {
          const f32x4 x = *reinterpret_cast<const f32x4*>(qp);
          const f32x4 y = *reinterpret_cast<const f32x4*>(qp + 16);
          qf[0] = x[0]; qf[1] = x[1]; qf[2] = x[2]; qf[3] = x[3];
          qf[4] = y[0]; qf[5] = y[1]; qf[6] = y[2]; qf[7] = y[3];
        }
        s[cb] = mma(kf, qf, s[cb]);
      }
    }

    // V^T was written by other lanes of this wave: order those writes before the reads below
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const float c = a.scale_log2;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float bmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
        s[cb][r] = (qpos[cb] - pos < a.window && pos < s1) ? s[cb][r] : -INFINITY;
        bmax = fmaxf(bmax, s[cb][r]);
      }
      update_max(cb, halves_max(bmax) * c);
      const float m_use = (m[cb] == -INFINITY) ? 0.f : m[cb];
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[cb][r], c, -m_use));
        s[cb][r] = p;
        rs += p;
      }
      l[cb] += halves_sum(rs);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const Frag pf = frag_from_acc<E>(s[cb], 8 * ks);
#pragma unroll
        for (int db = 0; db < kDDV / 32; ++db) {
          Frag vf;
          if constexpr (Lds::kVRowMajor) {
            vf = vt_frag_tr(my_vt, Lds::kVStride, db, ks, lane);
          } else {
            const char* p = my_vt + ((32 * db + col) * Lds::kVStride + 16 * ks + 4 * half) * E::kBytes;
            const f32x4 x = *reinterpret_cast<const f32x4*>(p);
            const f32x4 y = *reinterpret_cast<const f32x4*>(p + 32);
            vf[0] = x[0]; vf[1] = x[1]; vf[2] = x[2]; vf[3] = x[3];
            vf[4] = y[0]; vf[5] = y[1]; vf[6] = y[2]; vf[7] = y[3];
          }
          acc[cb][db] = mma(vf, pf, acc[cb][db]);
        }
      }
    }
    // the next block rewrites this wave's V^T tile: finish every read of it first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    if (PREFETCH) {
      cur = nxt;
    } else if (key_next < s1) {
      const char *kr, *vr;
      rows(key_next, kr, vr);
      cur.load(kr, vr, half);
    }
  }

  // ---- block drafts (T > 4, last split): new tokens 4 .. T-1 are staged only now, into the V
  // tiles of the work area (idle until the merge), when the registers of the key loop are free
  // (staging them with the first four costs the whole kernel some 50 registers) ----
  char* snew_hi = work;  // K rows of tokens 4..7, then their V rows
  if (split == a.nsplit - 1 && a.T > 4) {
    constexpr int kKCh = kDDQK / E::kPerChunk, kVCh = kDDV / E::kPerChunk;
    __syncthreads();  // every wave is done with its V tile
    for (int u = tid; u < (a.T - 4) * (kKCh + kVCh); u += kDecNW * 64) {
      const int t = 4 + u / (kKCh + kVCh), ch = u % (kKCh + kVCh);
      if (ch < kKCh)
        st16(snew_hi + (t - 4) * kDDQK * E::kBytes + ch * 16,
             ld16((const char*)a.k_new + (((size_t)b * a.T + t) * a.Hkv + g) * krow_bytes + ch * 16));
      else
        st16(snew_hi + Lds::kNewKBytes + (t - 4) * kDDV * E::kBytes + (ch - kKCh) * 16,
             ld16((const char*)a.v_new + (((size_t)b * a.T + t) * a.Hkv + g) * vrow_bytes + (ch - kKCh) * 16));
    }
    __syncthreads();
  }

  // ---- new tokens wave, wave + 4 (last split only): one extra key per column, on the VALU ----
  for (int tn = wave; split == a.nsplit - 1 && tn < a.T; tn += kDecNW) {
    // staged in LDS: tokens 0..3 next to Q, tokens 4..7 in the work area
    const char* nbase = tn < 4 ? smem + Lds::kQBytes : snew_hi;
    const char* krow = nbase + (tn & 3) * kDDQK * E::kBytes;
    const char* vrow = nbase + Lds::kNewKBytes + (tn & 3) * kDDV * E::kBytes;
    const float c = a.scale_log2;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      // q . k over this lane half's 96 elements, then across halves
      const char* qrow = sq + (cb * 32 + col) * Lds::kQStride * E::kBytes;
      float dot = 0.f;
      constexpr int kHalf = kDDQK / 2;
#pragma unroll
      for (int i = 0; i < kHalf / E::kPerChunk; ++i) {
        const int e0 = kHalf * half + E::kPerChunk * i;
        const u32x4 qv = *reinterpret_cast<const u32x4*>(qrow + e0 * E::kBytes);
        const u32x4 kv = *reinterpret_cast<const u32x4*>(krow + e0 * E::kBytes);
        if constexpr (E::kBytes == 2) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            dot = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[j]), as_bf16x2(kv[j]), dot, false);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) dot = __builtin_fmaf(__uint_as_float(qv[j]), __uint_as_float(kv[j]), dot);
        }
      }
      dot = halves_sum(dot);
      const int ccol = cb * 32 + col;
      const int t = (cbase + ccol) % a.T;
      const bool vis = ccol < ncols && t >= tn && t - tn < a.window;
      const float sc = vis ? dot * c : -INFINITY;
      update_max(cb, sc);
      const float p = fast_exp2(sc - ((m[cb] == -INFINITY) ? 0.f : m[cb]));
      l[cb] += p;
#pragma unroll
      for (int db = 0; db < kDDV / 32; ++db) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int dv = 32 * db + 8 * gq + 4 * half;
          float v[4];
          if constexpr (E::kBytes == 2) {
            const u32x2 w = *reinterpret_cast<const u32x2*>(vrow + dv * 2);
            v[0] = __uint_as_float(w[0] << 16);
            v[1] = __uint_as_float(w[0] & 0xFFFF0000u);
            v[2] = __uint_as_float(w[1] << 16);
            v[3] = __uint_as_float(w[1] & 0xFFFF0000u);
          } else {
            const f32x4 w = *reinterpret_cast<const f32x4*>(vrow + dv * 4);
            v[0] = w[0]; v[1] = w[1]; v[2] = w[2]; v[3] = w[3];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[cb][db][4 * gq + i] = __builtin_fmaf(p, v[i], acc[cb][db][4 * gq + i]);
        }
      }
    }
  }

  // ---- merge the waves of this workgroup (fixed order): per column block, in two rounds of two
  // dv blocks each; in round rr wave w sums dv block 2 rr + (w & 1), registers 8 (w >> 1) .. +7 ----
  float* sm_acc = reinterpret_cast<float*>(work);  // [wave][2][r][lane]
  float* sm_m = reinterpret_cast<float*>(smem + (Lds::kBytes - kDecNW * 64 * 4 * 2));
  float* sm_l = sm_m + kDecNW * 64;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    __syncthreads();  // previous users of the work area are done
    sm_m[wave * 64 + lane] = m[cb];
    sm_l[wave * 64 + lane] = l[cb];
    __syncthreads();
    const int c = cbase + cb * 32 + col;  // column within the G*T columns of (b, g)
    const bool cvalid = cb * 32 + col < ncols;
    const int t = cvalid ? c % a.T : 0;
    const int head = cvalid ? a.hl.at(g * a.G + c / a.T) : 0;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecNW; ++w) M = fmaxf(M, sm_m[w * 64 + lane]);
    const bool fold_sink = (a.nsplit == 1) && a.sink && cvalid;
    const float s_l2 = fold_sink ? a.sink[head] * kLog2e : -INFINITY;
    M = fmaxf(M, s_l2);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float Lsum = fold_sink ? fast_exp2(s_l2 - M_use) : 0.f;
#pragma unroll
    for (int w = 0; w < kDecNW; ++w) Lsum += sm_l[w * 64 + lane] * fast_exp2(sm_m[w * 64 + lane] - M_use);
    const float scale_w = fast_exp2(m[cb] - M_use);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      if (rr) __syncthreads();  // the first pass's reads are done
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sm_acc[((wave * 2 + d2) * 16 + r) * 64 + lane] = acc[cb][2 * rr + d2][r] * scale_w;
      __syncthreads();
      const int db = 2 * rr + (wave & 1), rb = 8 * (wave >> 1);
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[i] = 0.f;
#pragma unroll
        for (int w = 0; w < kDecNW; ++w) o[i] += sm_acc[((w * 2 + (wave & 1)) * 16 + rb + i) * 64 + lane];
      }
      if (!cvalid) continue;
      if (a.nsplit == 1) {
        const float inv = 1.f / Lsum;
        char* orow = (char*)a.o + (((size_t)b * a.T + t) * a.Hq + head) * kDDV * E::kBytes;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int dv = 32 * db + 8 * ((rb >> 2) + g2) + 4 * half;
          const float x0 = o[4 * g2] * inv, x1 = o[4 * g2 + 1] * inv;
          const float x2 = o[4 * g2 + 2] * inv, x3 = o[4 * g2 + 3] * inv;
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
        if (a.lse && rr == 0 && wave == 0 && half == 0)
          a.lse[((size_t)b * a.T + t) * a.Hq + head] = (M + fast_log2(Lsum)) * kLn2;
      } else {
        // partial record for (b, g, split, column c): acc[kDDV], m, l
        const int ncols_pad = ((a.ncols + 31) / 32) * 32;
        float* rec = a.ws + ((((size_t)b * a.Hkv + g) * a.nsplit + split) * ncols_pad + c) * kRec;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          f32x4 w;
          w[0] = o[4 * g2]; w[1] = o[4 * g2 + 1]; w[2] = o[4 * g2 + 2]; w[3] = o[4 * g2 + 3];
          *reinterpret_cast<f32x4*>(rec + 32 * db + 8 * ((rb >> 2) + g2) + 4 * half) = w;
        }
        if (rr == 0 && wave == 0 && half == 0) {
          rec[kDDV] = M;
          rec[kDDV + 1] = Lsum;
        }
      }
    }
  }
}

// Sliding-window verify in one pass: at most 128 committed keys (window <= 129), at most 32 query
// columns per workgroup (a column chunk of the G*T columns of (b, g)) and at most 4 new tokens, or
// 8 with EXT (block drafts), bf16 (the ring workloads' shape). Wave w owns
// committed-key block w (keys s0 + 32 w ..), so each column's maximum over all keys is known after
// one exchange and no running max is needed:
//   1. every wave forms S^T of its block and its column maxima; wave w also scores new tokens w
//      and w + 4 on the VALU; maxima and new-token scores meet in LDS;
//   2. every wave exponentiates its block against the common maximum and leaves P (bf16 MFMA
//      fragments, over the no longer needed Q^T rows) and its column sums in LDS;
//   3. wave w forms dv rows 32 w .. 32 w + 31 of O^T from all four blocks' V tiles and P, adds
//      the new tokens and the sink, and writes them.
// Against the general kernel this replaces the per-wave (m, l, acc) merge (64 KB of LDS traffic
// and four barriers per workgroup) by two exchanges of 8 KB. A block past the committed keys
// holds zero V rows and masked scores, so the products stay finite. Tokens 4..7 (EXT): LDS is full
// during step 1, so their K rows are fetched into registers at kernel start and their V rows are
// written after the first barrier next to the P fragments.
template <bool ROPE, bool EXT>
__global__ __launch_bounds__(kDecNW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_window_kernel(const DecodeArgs a) {
  using E = BF16;
  using Lds = DecodeLds<E, 1>;
  __shared__ __attribute__((aligned(16))) char smem[Lds::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // one split. Column chunks of one (b, g) read the same K/V rows: workgroups are dealt to the
  // XCDs round-robin by linear index, so with several chunks the index is remapped to put the
  // chunks of one (b, g) eight apart (same XCD, same L2, launched together) when the (b, g) pairs
  // come in whole groups of eight.
  int chunk = blockIdx.y % a.n_chunks, g = blockIdx.y / a.n_chunks, b = blockIdx.z;
  const int pairs = a.B * a.Hkv;
  if (a.n_chunks > 1 && pairs % 8 == 0) {
    const int id = blockIdx.y + gridDim.y * blockIdx.z;
    const int q = id / 8;
    chunk = q % a.n_chunks;
    const int pair = (q / a.n_chunks) * 8 + id % 8;
    g = pair % a.Hkv;
    b = pair / a.Hkv;
  }
  const int cbase = chunk * a.chunk_cols;  // this workgroup's columns: cbase + [0, ncols)
  const int ncols = min(a.chunk_cols, a.ncols - cbase);

  int P = a.cache_len[b];
  P = P < 0 ? 0 : (P > a.max_len ? a.max_len : P);
  const int off = a.cache_offset ? a.cache_offset[b] : 0;
  const int s0 = max(0, P - a.window + 1);  // committed keys [s0, P), at most 128
  const int s1 = P;
  const int key0 = s0 + 32 * wave;
  const bool has_keys = key0 < s1;

  const size_t krow_bytes = (size_t)kDDQK * E::kBytes;
  const size_t vrow_bytes = (size_t)kDDV * E::kBytes;
  const size_t row0 = (size_t)b * a.C;

  // EXT: K row of new token wave + 4 (this lane half's 96 elements) and one 16-byte chunk of the
  // V rows of tokens 4..7 per thread, fetched now, used in steps 1 and 2
  constexpr int kHalfChunks = kDDQK / 2 / E::kPerChunk;
  u32x4 kx[EXT ? kHalfChunks : 1];
  u32x4 vx = zero_chunk();
  const int tok_hi = wave + 4;
  const int nvx = EXT ? (a.T > 4 ? (a.T - 4) * (kDDV / E::kPerChunk) : 0) : 0;  // V chunks of tokens 4..T-1
  if constexpr (EXT) {
    const int t = min(tok_hi, a.T - 1);
    const char* krow = (const char*)a.k_new + (((size_t)b * a.T + t) * a.Hkv + g) * krow_bytes + half * (kDDQK / 2) * E::kBytes;
#pragma unroll
    for (int i = 0; i < kHalfChunks; ++i) kx[i] = ld16(krow + 16 * i);
    if (tid < nvx) {
      const int tv = 4 + tid / (kDDV / E::kPerChunk), ch = tid % (kDDV / E::kPerChunk);
      vx = ld16((const char*)a.v_new + (((size_t)b * a.T + tv) * a.Hkv + g) * vrow_bytes + ch * 16);
    }
  }

  KeyRows<E> cur;
  {
    QStage<E, 1> st;
    st.load(a, tid, b, g, cbase, ncols);
    if (has_keys) {
      const int pos = min(key0 + col, s1 - 1);
      int slot = (pos + off) % a.C;
      slot += slot < 0 ? a.C : 0;
      cur.load((const char*)a.k_cache + ((row0 + slot) * a.Hkv + g) * krow_bytes,
               (const char*)a.v_cache + ((row0 + slot) * a.Hkv + g) * vrow_bytes, half);
    } else {
#pragma unroll
      for (int j = 0; j < KeyRows<E>::kKChunks; ++j) cur.k[j] = zero_chunk();
#pragma unroll
      for (int i = 0; i < KeyRows<E>::kVChunks; ++i) cur.v[i] = zero_chunk();
    }
    st.store(smem, tid, ncols, true, a.T);
  }
  char* sq = smem;
  char* snew = smem + Lds::kQBytes;
  char* work = snew + Lds::kNewBytes;
  float* xm = reinterpret_cast<float*>(smem + (Lds::kBytes - kDecNW * 64 * 4 * 2));  // [wave][col]
  float* xs = xm + kDecNW * 32;                                                      // [token][col], 8 tokens
  float* xl = xs + 2 * kDecNW * 32;                                                  // [wave][col]
  static_assert(4 * kDecNW * 32 * 4 <= kDecNW * 64 * 4 * 2, "exchange area");
  __syncthreads();  // Q^T and the new-token rows are in LDS
  if constexpr (ROPE) {
    rope_staged<E, 1>(a, smem, tid, P, cbase, ncols, true);
    __syncthreads();
  }

  const bool cvalid = col < ncols;
  const int cg = cbase + col;              // column within the G*T columns of (b, g)
  const int tq = cvalid ? cg % a.T : 0;   // new token of this column
  const float c = a.scale_log2;

  // ---- 1. S^T of this wave's block, column maxima, new token `wave` ----
  cur.store_v(work + wave * Lds::kVBytes, col, half);
  f32x16 s = zero16();
#pragma unroll
  for (int kk = 0; kk < kDDQK / 16; ++kk) {
    const bf16x8 qf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                            sq + (col * Lds::kQStride + 16 * kk + 8 * half) * E::kBytes));
    s = mma(cur.kfrag(kk), qf, s);
  }
  float bmax = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int pos = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
    s[r] = (pos < s1 && P + tq - pos < a.window) ? s[r] * c : -INFINITY;
    bmax = fmaxf(bmax, s[r]);
  }
  bmax = halves_max(bmax);
  if (half == 0) xm[wave * 32 + col] = bmax;
  // score of new token t for this lane's column: q . k over this half's 96 elements (K chunks from
  // `krow` in LDS, or from registers for tokens 4..7), then across halves
  auto new_score = [&](int t, const char* krow, bool in_regs) {
    const char* qrow = sq + col * Lds::kQStride * E::kBytes;
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kHalfChunks; ++i) {
      const int e0 = (kDDQK / 2) * half + E::kPerChunk * i;
      const u32x4 qv = *reinterpret_cast<const u32x4*>(qrow + e0 * E::kBytes);
      const u32x4 kv = in_regs ? kx[EXT ? i : 0] : *reinterpret_cast<const u32x4*>(krow + e0 * E::kBytes);
#pragma unroll
      for (int j = 0; j < 4; ++j) dot = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[j]), as_bf16x2(kv[j]), dot, false);
    }
    dot = halves_sum(dot);
    const bool vis = cvalid && tq >= t && tq - t < a.window;
    if (half == 0) xs[t * 32 + col] = vis ? dot * c : -INFINITY;
  };
  if (wave < a.T) new_score(wave, snew + wave * kDDQK * E::kBytes, false);
  if (EXT && tok_hi < a.T) new_score(tok_hi, nullptr, true);
  __syncthreads();  // maxima and new-token scores are in LDS; Q^T is no longer read

  // ---- 2. P of this block against the common maximum ----
  const int head = cvalid ? a.hl.at(g * a.G + cg / a.T) : 0;
  const float sink_l2 = (a.sink && cvalid) ? a.sink[head] * kLog2e : -INFINITY;
  float M = sink_l2;
#pragma unroll
  for (int w = 0; w < kDecNW; ++w) M = fmaxf(M, xm[w * 32 + col]);
  constexpr int kNT = EXT ? 2 * kDecNW : kDecNW;  // new tokens this instance handles
  float snt[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    snt[t] = t < a.T ? xs[t * 32 + col] : -INFINITY;
    M = fmaxf(M, snt[t]);
  }
  const float M_use = (M == -INFINITY) ? 0.f : M;
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = fast_exp2(s[r] - M_use);
    rs += s[r];
  }
  rs = halves_sum(rs);
  char* sp = sq;  // P fragments [block][ks][lane], 16 bytes each, over the Q^T rows
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    st16(sp + ((wave * 2 + ks) * 64 + lane) * 16, __builtin_bit_cast(u32x4, frag_from_acc<E>(s, 8 * ks)));
  if (half == 0) xl[wave * 32 + col] = rs;
  // V rows of tokens 4..7 next to the P fragments, in the part of the Q^T rows P leaves free
  char* snew_hi = sq + kDecNW * 2 * 64 * 16;
  static_assert(kDecNW * 2 * 64 * 16 + 4 * kDDV * 2 <= Lds::kQBytes, "tokens 4..7 fit beside P");
  if (EXT && tid < nvx) st16(snew_hi + tid * 16, vx);
  __syncthreads();  // P fragments, block sums and the V rows of tokens 4..7 are in LDS

  // ---- 3. dv rows 32 wave .. 32 wave + 31 of O^T over all blocks, new tokens, sink ----
  f32x16 acc = zero16();
#pragma unroll
  for (int kb = 0; kb < kDecNW; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, ld16(sp + ((kb * 2 + ks) * 64 + lane) * 16));
      acc = mma(vt_frag_tr(work + kb * Lds::kVBytes, Lds::kVStride, wave, ks, lane), pf, acc);
    }
  float L = a.sink && cvalid ? fast_exp2(sink_l2 - M_use) : 0.f;
#pragma unroll
  for (int w = 0; w < kDecNW; ++w) L += xl[w * 32 + col];
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    if (t >= a.T) break;
    const float pn = fast_exp2(snt[t] - M_use);
    L += pn;
    const char* vrow = t < 4 ? snew + Lds::kNewKBytes + t * kDDV * E::kBytes : snew_hi + (t - 4) * kDDV * E::kBytes;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const u32x2 w2 = *reinterpret_cast<const u32x2*>(vrow + (32 * wave + 8 * gq + 4 * half) * 2);
      acc[4 * gq + 0] = __builtin_fmaf(pn, __uint_as_float(w2[0] << 16), acc[4 * gq + 0]);
      acc[4 * gq + 1] = __builtin_fmaf(pn, __uint_as_float(w2[0] & 0xFFFF0000u), acc[4 * gq + 1]);
      acc[4 * gq + 2] = __builtin_fmaf(pn, __uint_as_float(w2[1] << 16), acc[4 * gq + 2]);
      acc[4 * gq + 3] = __builtin_fmaf(pn, __uint_as_float(w2[1] & 0xFFFF0000u), acc[4 * gq + 3]);
    }
  }
  if (!cvalid) return;
  const float inv = 1.f / L;
  char* orow = (char*)a.o + (((size_t)b * a.T + tq) * a.Hq + head) * kDDV * E::kBytes;
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    u32x2 w2;
    w2[0] = pack_bf16x2(acc[4 * gq] * inv, acc[4 * gq + 1] * inv);
    w2[1] = pack_bf16x2(acc[4 * gq + 2] * inv, acc[4 * gq + 3] * inv);
    *reinterpret_cast<u32x2*>(orow + (32 * wave + 8 * gq + 4 * half) * 2) = w2;
  }
  if (a.lse && wave == 0 && half == 0) a.lse[((size_t)b * a.T + tq) * a.Hq + head] = (M + fast_log2(L)) * kLn2;
}

// Folds the split partials and the sink (once) into O and LSE. A workgroup covers kCombCols query
// columns of one (b, g); thread (column, quad) owns 4 consecutive dv of that column. Pass 1 takes
// the max over the splits' m, pass 2 sums the rescaled l and acc, kCombUnroll splits at a time so
// that their loads are in flight together.
constexpr int kCombCols = 8;
constexpr int kCombUnroll = 8;

template <typename E>
__global__ __launch_bounds__(kCombCols * kDDV / 4) void combine_kernel(const DecodeArgs a) {
  const int quad = threadIdx.x % (kDDV / 4);
  const int c = blockIdx.x * kCombCols + threadIdx.x / (kDDV / 4);  // query column within the group
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  if (c >= a.ncols) return;
  const int ncols_pad = ((a.ncols + 31) / 32) * 32;
  const int t = c % a.T;
  const int head = a.hl.at(g * a.G + c / a.T);
  const float* base = a.ws + (((size_t)b * a.Hkv + g) * a.nsplit * ncols_pad + c) * kRec;
  const size_t stride = (size_t)ncols_pad * kRec;
  const int ns = a.nsplit;

  const float sink_l2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
  float M = sink_l2;
  for (int s0 = 0; s0 < ns; s0 += kCombUnroll) {
    float mv[kCombUnroll];
#pragma unroll
    for (int u = 0; u < kCombUnroll; ++u) mv[u] = base[(size_t)min(s0 + u, ns - 1) * stride + kDDV];
#pragma unroll
    for (int u = 0; u < kCombUnroll; ++u) M = fmaxf(M, mv[u]);  // clamped repeats change no max
  }
  const float M_use = (M == -INFINITY) ? 0.f : M;
  float L = a.sink ? fast_exp2(sink_l2 - M_use) : 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < ns; s0 += kCombUnroll) {
    f32x4 acc[kCombUnroll];
    f32x2 ml[kCombUnroll];
#pragma unroll
    for (int u = 0; u < kCombUnroll; ++u) {
      const float* rec = base + (size_t)min(s0 + u, ns - 1) * stride;
      acc[u] = *reinterpret_cast<const f32x4*>(rec + 4 * quad);
      ml[u] = *reinterpret_cast<const f32x2*>(rec + kDDV);
    }
#pragma unroll
    for (int u = 0; u < kCombUnroll; ++u) {
      // past the last split: weight 0; an empty split has m = -inf, also weight 0
      const float w = s0 + u < ns ? fast_exp2(ml[u][0] - M_use) : 0.f;
      L += ml[u][1] * w;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] += acc[u][i] * w;
    }
  }
  const float inv = 1.f / L;
  char* orow = (char*)a.o + (((size_t)b * a.T + t) * a.Hq + head) * kDDV * E::kBytes;
  if constexpr (E::kBytes == 2) {
    u32x2 w;
    w[0] = pack_bf16x2(o[0] * inv, o[1] * inv);
    w[1] = pack_bf16x2(o[2] * inv, o[3] * inv);
    *reinterpret_cast<u32x2*>(orow + 8 * quad) = w;
  } else {
    f32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = o[i] * inv;
    *reinterpret_cast<f32x4*>(orow + 16 * quad) = w;
  }
  if (a.lse && quad == 0) a.lse[((size_t)b * a.T + t) * a.Hq + head] = (M + fast_log2(L)) * kLn2;
}

// Commits the accepted prefix of a verify step: new tokens 0 .. n_b - 1 of sequence b go to
// positions P_b .. P_b + n_b - 1, i.e. slots (p + off_b) mod C, and cache_len[b] becomes
// P_b + n_b. One workgroup per sequence; 16-byte chunks of K and V rows are spread over its
// threads. Every thread reads cache_len[b] before the barrier, one thread writes it after.
template <typename E>
__global__ __launch_bounds__(256) void cache_append_kernel(const AppendArgs a) {
  constexpr int kKCh = kDDQK / E::kPerChunk, kVCh = kDDV / E::kPerChunk;
  const int b = blockIdx.x;
  int P = a.cache_len[b];
  P = P < 0 ? 0 : (P > a.max_len ? a.max_len : P);
  int n = a.accept ? a.accept[b] : a.T;
  n = n < 0 ? 0 : (n > a.T ? a.T : n);
  n = min(n, a.max_len - P);  // the cache never holds more than max_len positions
  const int off = a.cache_offset ? a.cache_offset[b] : 0;
  const size_t krow_bytes = (size_t)kDDQK * E::kBytes, vrow_bytes = (size_t)kDDV * E::kBytes;
  const int per_tok = a.Hkv * (kKCh + kVCh);
  for (int u = threadIdx.x; u < n * per_tok; u += 256) {
    const int t = u / per_tok, r = u % per_tok;
    const int g = r / (kKCh + kVCh), ch = r % (kKCh + kVCh);
    int slot = (P + t + off) % a.C;
    slot += slot < 0 ? a.C : 0;
    const size_t src = ((size_t)b * a.T + t) * a.Hkv + g;
    const size_t dst = ((size_t)b * a.C + slot) * a.Hkv + g;
    if (ch < kKCh)
      st16((char*)a.k_cache + dst * krow_bytes + ch * 16, ld16((const char*)a.k_new + src * krow_bytes + ch * 16));
    else
      st16((char*)a.v_cache + dst * vrow_bytes + (ch - kKCh) * 16,
           ld16((const char*)a.v_new + src * vrow_bytes + (ch - kKCh) * 16));
  }
  __syncthreads();
  if (threadIdx.x == 0) a.cache_len[b] = P + n;
}

hipError_t cache_append_launch(bool bf16, const AppendArgs& a, hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL(cache_append_kernel<BF16>, dim3(a.B), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(cache_append_kernel<F32>, dim3(a.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

size_t decode_ws_bytes(int B, int Hkv, int ncols, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t ncols_pad = (size_t)((ncols + 31) / 32) * 32;
  return (size_t)B * Hkv * nsplit * ncols_pad * kRec * sizeof(float);
}

// The one-pass window kernel serves a single split of at most four 32-key blocks with at most 32
// query columns per workgroup and at most 4 new tokens (8 without RoPE).
static bool window_kernel_fits(const DecodeArgs& a) {
  const bool cols = a.ncols <= 32 || a.chunk_cols == 32;  // every workgroup's chunk fits one column block
  return a.nsplit == 1 && a.keys_per_split <= 32 * kDecNW && cols && (a.T <= kDecNW || (a.T <= 2 * kDecNW && !a.rope));
}

// With one column block (e.g. 8 query heads x 4 tokens) a wave holds few blocks and fewer
// registers buy a second wave per SIMD; that beats prefetching (measured on the ring workload),
// so the one-column kernel does not prefetch.
constexpr bool kPrefetch1Col = false;

template <bool ROPE>
static void launch_decode_kernel(bool bf16, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, a.Hkv * a.n_chunks, a.B);
  const dim3 block(kDecNW * 64);
  if (bf16 && window_kernel_fits(a)) {
    if (a.T > kDecNW)
      hipLaunchKernelGGL((decode_window_kernel<false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_window_kernel<ROPE, false>), grid, block, 0, stream, a);
    return;
  }
  const bool two = (a.n_chunks > 1 ? a.chunk_cols : a.ncols) > 32;
  if (bf16 && two)
    hipLaunchKernelGGL((decode_kernel<BF16, 2, true, ROPE>), grid, block, 0, stream, a);
  else if (bf16)
    hipLaunchKernelGGL((decode_kernel<BF16, 1, kPrefetch1Col, ROPE>), grid, block, 0, stream, a);
  else if (two)
    hipLaunchKernelGGL((decode_kernel<F32, 2, false, ROPE>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<F32, 1, false, ROPE>), grid, block, 0, stream, a);
}

hipError_t decode_launch(bool bf16, const DecodeArgs& a, hipStream_t stream) {
  if (a.rope)
    launch_decode_kernel<true>(bf16, a, stream);
  else
    launch_decode_kernel<false>(bf16, a, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  const dim3 cgrid((a.ncols + kCombCols - 1) / kCombCols, a.Hkv, a.B);
  const dim3 cblock(kCombCols * kDDV / 4);
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<BF16>, cgrid, cblock, 0, stream, a);
  else
    hipLaunchKernelGGL(combine_kernel<F32>, cgrid, cblock, 0, stream, a);
  return hipGetLastError();
}

}  // namespace mimo
