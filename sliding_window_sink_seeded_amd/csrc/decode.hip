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
// columns of (b, g) - every query head of the group times every new token - are the MFMA columns,
// so each K/V element read from HBM serves all the columns of a chunk. Three kernels:
//   * decode_window_kernel: bf16 single passes over at most four 32-key blocks (the 128-slot ring
//     of a sliding-window layer), one block per wave, 32 or 64 columns per workgroup;
//   * decode_cols_kernel: other bf16 calls with more than 32 columns (64 or 128 per workgroup):
//     the waves split the columns and share each 32-key block staged in LDS;
//   * decode_kernel: 32 columns per workgroup (bf16 up to 32 columns, fp32 in chunks of 32). Q^T
//     sits in LDS, shared by the waves; the split's keys are cut into 32-key blocks dealt
//     round-robin to the waves. Lane (col, half) of a wave fetches half of the K row and half of
//     the V row of key key0 + col: the K half is directly its MFMA A fragment, the V half goes to
//     a wave-private LDS tile that the PV product reads back transposed. A wave keeps an online
//     softmax per column (no sink here), then the waves merge through LDS in a fixed order.
// Single pass (one split): the sink is folded in and O / LSE are written. Several splits: the
// unnormalised (m, l, acc) of each column go to the workspace and combine_kernel folds the splits
// and the sink (counted once) into O / LSE. Keys past the end of a split are fetched from its last
// key (finite data, masked to weight 0). Running maxima are refreshed lazily (see update_max).
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
  // go to the work area after the key loop rather than growing this area)
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
// ROPE (q and k_new arrive before the rotary embedding): load() also fetches the (cos, sin) of
// every rotated chunk (query column c at position P + c % T, new token t at P + t) and store()
// rotates the chunks in registers before writing them. A head vector's chunks go to consecutive
// threads, and every vector starts at a thread index whose rotated chunks stay inside one wave
// (vectors of 24 / 40 chunks for bf16, 48 / 80 for fp32), so a chunk's partner is 32 dims = H
// lanes away in the same wave (rope_chunk_xlane).
template <typename E, int NCB, bool ROPE>
struct QStage {
  using Lds = DecodeLds<E, NCB>;
  static constexpr int kChunksRow = kDDQK / E::kPerChunk;
  static constexpr int kQChunks = NCB * 32 * kChunksRow;
  static constexpr int kQPer = (kQChunks + kDecNW * 64 - 1) / (kDecNW * 64);
  static constexpr int kKCh = kDDQK / E::kPerChunk, kVCh = kDDV / E::kPerChunk;
  static constexpr int kNewPer = (4 * (kKCh + kVCh) + kDecNW * 64 - 1) / (kDecNW * 64);
  static constexpr int H = kRopeH<E>;
  // A thread's Q chunks i = 0, 1, 2, .. sit at chunk (tid + 256 i) % kChunksRow of their rows; 256
  // is 16 mod the row length (24 chunks bf16, 48 fp32) and 48 is 0 mod it, so the chunk indices
  // repeat with period 3 and exactly one of every three, i = ir + 3 k, is a rotated chunk (< 2H).
  static_assert((kDecNW * 64) % kChunksRow == 16 && (3 * 16) % kChunksRow == 0 && 3 * 2 * H == kChunksRow,
                "one rotated chunk in every three");
  static_assert(kQPer % 3 == 0, "whole periods");
  static constexpr int kNR = ROPE ? kQPer / 3 : 1;  // rotated Q chunks per thread
  static constexpr int kCs = ROPE ? 2 * E::kPerChunk : 1;
  u32x4 xq[kQPer], xn[kNewPer];
  float qcs[kNR][kCs], ncs[ROPE ? kNewPer : 1][kCs];
  int ir;  // ROPE: this thread's rotated Q chunks are i = ir + 3 k

  __device__ __forceinline__ void load(const DecodeArgs& a, int tid, int b, int g, int cbase, int ncols, int P) {
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
    if constexpr (ROPE) {
      const int ch0 = tid % kChunksRow;
      ir = ch0 < 2 * H ? 0 : (ch0 + 16 < kChunksRow + 2 * H && ch0 + 16 >= kChunksRow ? 1 : 2);
#pragma unroll
      for (int k = 0; k < kNR; ++k) {
        const int u = tid + (ir + 3 * k) * kDecNW * 64;
        const int c = cbase + min(u / kChunksRow, ncols - 1), ch = u % kChunksRow;
        rope_load<E::kPerChunk>(a.rope, P + c % a.T, (ch % H) * E::kPerChunk, qcs[k]);
      }
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
      // (every lane reads table entries, used only for rotated chunks: no branch around loads)
      if constexpr (ROPE) rope_load<E::kPerChunk>(a.rope, P + t, (ch % H) * E::kPerChunk, ncs[i]);
    }
  }

  // Q^T rows at smem, new tokens 0..3 (K rows, then V rows unless !STAGE_V) right after them; the
  // new tokens only when `last` (the split that folds them in)
  template <bool STAGE_V = true>
  __device__ __forceinline__ void store(char* smem, int tid, int ncols, bool last, int T) const {
    const int lane = tid & 63;
    u32x4 x[kQPer];
#pragma unroll
    for (int i = 0; i < kQPer; ++i) x[i] = xq[i];
    if constexpr (ROPE) {
      // the rotated chunk of each period of three; its partner lane rotates the same i
#pragma unroll
      for (int k = 0; k < kNR; ++k) {
        const u32x4 v = ir == 0 ? x[3 * k] : (ir == 1 ? x[3 * k + 1] : x[3 * k + 2]);
        const int ch = (tid + (ir + 3 * k) * kDecNW * 64) % kChunksRow;
        const u32x4 r = rope_chunk_xlane<E>(v, ch, lane, qcs[k]);
#pragma unroll
        for (int j = 0; j < 3; ++j) x[3 * k + j] = ir == j ? r : x[3 * k + j];
      }
    }
#pragma unroll
    for (int i = 0; i < kQPer; ++i) {
      const int u = tid + i * kDecNW * 64;
      const int c = u / kChunksRow, ch = u % kChunksRow;
      if (u < kQChunks) st16(smem + c * Lds::kQStride * E::kBytes + ch * 16, c < ncols ? x[i] : zero_chunk());
    }
    char* snew = smem + Lds::kQBytes;
#pragma unroll
    for (int i = 0; i < kNewPer; ++i) {
      const int u = tid + i * kDecNW * 64;
      const int t = u / (kKCh + kVCh), ch = u % (kKCh + kVCh);
      u32x4 x = xn[i];
      if constexpr (ROPE) x = rope_chunk_xlane<E>(x, ch < kKCh ? ch : 2 * H, lane, ncs[i]);  // V: as is
      if (last && u < 4 * (kKCh + kVCh) && t < T) {
        if (ch < kKCh)
          st16(snew + t * kDDQK * E::kBytes + ch * 16, x);
        else if (STAGE_V)
          st16(snew + Lds::kNewKBytes + t * kDDV * E::kBytes + (ch - kKCh) * 16, x);
      }
    }
  }
  // !STAGE_V: the V chunk this thread holds (new token t_out, chunk ch_out of its V row), if any
  __device__ __forceinline__ bool new_v_chunk(int tid, int T, u32x4& x, int& t_out, int& ch_out) const {
    static_assert(kNewPer == 1, "one new-token chunk per thread");
    const int t = tid / (kKCh + kVCh), ch = tid % (kKCh + kVCh);
    x = xn[0];
    t_out = t;
    ch_out = ch - kKCh;
    return tid < 4 * (kKCh + kVCh) && t < T && ch >= kKCh;
  }
};

// With one bf16 column block, asking for two waves per SIMD makes the compiler keep the
// accumulators in VGPRs (169 registers, no AGPR copies) instead of 137 VGPRs + 80 AGPRs; both give
// two waves per SIMD, the first runs faster (ring workload).
template <typename E, int NCB, bool PREFETCH, bool ROPE>
__global__ __launch_bounds__(kDecNW * 64)
__attribute__((amdgpu_waves_per_eu(NCB == 1 && E::kBytes == 2 ? 2 : 1))) void decode_kernel(const DecodeArgs a) {
  using Frag = typename E::Frag;
  using Lds = DecodeLds<E, NCB>;
  __shared__ __attribute__((aligned(16))) char smem[Lds::kBytes];
  poison_lds(smem, sizeof(smem));

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
    QStage<E, NCB, ROPE> st;
    st.load(a, tid, b, g, cbase, ncols, P);
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
  // (staging them with the first four costs the whole kernel some 50 registers). With ROPE their
  // K rows are rotated on the way (positions P + 4 ..), laid out as in QStage: a row's chunks on
  // consecutive threads, every row starting where its rotated chunks share one wave. ----
  char* snew_hi = work;  // K rows of tokens 4..7, then their V rows
  if (split == a.nsplit - 1 && a.T > 4) {
    constexpr int kKCh = kDDQK / E::kPerChunk, kVCh = kDDV / E::kPerChunk, kRow = kKCh + kVCh;
    const int n = (a.T - 4) * kRow;
    __syncthreads();  // every wave is done with its V tile
    for (int u0 = 0; u0 < n; u0 += kDecNW * 64) {  // same trip count in every lane (exchange below)
      const int u = min(u0 + tid, n - 1);
      const int t = 4 + u / kRow, ch = u % kRow;
      u32x4 x = ch < kKCh
                    ? ld16((const char*)a.k_new + (((size_t)b * a.T + t) * a.Hkv + g) * krow_bytes + ch * 16)
                    : ld16((const char*)a.v_new + (((size_t)b * a.T + t) * a.Hkv + g) * vrow_bytes + (ch - kKCh) * 16);
      if constexpr (ROPE) {
        constexpr int H = kRopeH<E>;
        float cs[2 * E::kPerChunk];
        if (ch < 2 * H) rope_load<E::kPerChunk>(a.rope, P + t, (ch % H) * E::kPerChunk, cs);
        x = rope_chunk_xlane<E>(x, ch < kKCh ? ch : 2 * H, lane, cs);
      }
      if (u0 + tid < n) {
        if (ch < kKCh)
          st16(snew_hi + (t - 4) * kDDQK * E::kBytes + ch * 16, x);
        else
          st16(snew_hi + Lds::kNewKBytes + (t - 4) * kDDV * E::kBytes + (ch - kKCh) * 16, x);
      }
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

// Sliding-window verify in one pass: at most 128 committed keys (window <= 129), NCB column
// blocks of 32 query columns per workgroup (a column chunk of the G*T columns of (b, g); NCB = 2
// serves 8 heads x 8 tokens in one workgroup) and at most 4 new tokens, or 8 with EXT (block
// drafts), bf16 (the ring workloads' shape). Wave w owns committed-key block w (keys s0 + 32 w ..),
// so each column's maximum over all keys is known after one exchange and no running max is needed:
//   1. every wave forms S^T of its block for every column block (each K fragment feeds NCB
//      products) and its column maxima; wave w also scores new tokens w and w + 4 on the VALU;
//      maxima and new-token scores meet in LDS;
//   2. every wave exponentiates its block against the common maximum and leaves P (bf16 MFMA
//      fragments, over the no longer needed Q^T rows) and its column sums in LDS;
//   3. wave w forms dv rows 32 w .. 32 w + 31 of O^T from all four blocks' V tiles and P (each V^T
//      fragment feeds NCB products), adds the new tokens and the sink, and writes them.
// Against the general kernel this replaces the per-wave (m, l, acc) merge (64 KB of LDS traffic
// and four barriers per workgroup) by two exchanges. A block past the committed keys holds zero V
// rows and masked scores, so the products stay finite. Tokens 4..7 (EXT): LDS is full during
// step 1, so their K rows are fetched into registers at kernel start and their V rows are written
// after the first barrier next to the P fragments.
template <int NCB>
struct WindowLds {
  using L = DecodeLds<BF16, NCB>;
  // new tokens 0..3: K rows only (their V rows stay in the registers they were fetched into until
  // the 16-row V tile is built; the 1 KB saved keeps the one-column-block instance at 52 KB, which
  // with LDS allocated in 2 KB granules is three workgroups per CU instead of two)
  static constexpr int kQBytes = L::kQBytes, kNewBytes = L::kNewKBytes, kVBytes = L::kVBytes;
  static constexpr int kWork = kDecNW * kVBytes;  // the four waves' V tiles
  static constexpr int kX = NCB * 32 * 4;         // one [column block][column] fp32 row
  // exchange: column maxima [wave][cb][col], new-token scores [token][cb][col], sums [wave][cb][col]
  static constexpr int kXBytes = (kDecNW + 2 * kDecNW + kDecNW) * kX;
  static constexpr int kBytes = kQBytes + kNewBytes + kWork + kXBytes;
  static constexpr int kPBytes = kDecNW * 2 * NCB * 64 * 16;  // P fragments over the Q^T rows
  // the new tokens' V rows as a 16-row tile (rows past T zero) beside the P fragments
  static constexpr int kNewVBytes = 16 * L::kVStride * 2;
  static_assert(kPBytes + kNewVBytes <= kQBytes, "P fragments and the new tokens' V tile fit the Q^T rows");
};

template <int NCB, bool ROPE, bool EXT>
__global__ __launch_bounds__(kDecNW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_window_kernel(const DecodeArgs a) {
  using E = BF16;
  using Lds = DecodeLds<E, NCB>;
  using W = WindowLds<NCB>;
  __shared__ __attribute__((aligned(16))) char smem[W::kBytes];
  poison_lds(smem, sizeof(smem));

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
  // ROPE: (cos, sin) of all 32 pairs at that token's position; the rotated dims 0..63 are all in
  // half 0's 96 elements, so a lane holds both chunks of each pair and rotates them itself (just
  // before the token's score, when the loads have long landed)
  constexpr int kXcs = (EXT && ROPE) ? kRopeDims : 1;
  float xcs[kXcs];
  if constexpr (EXT) {
    const int t = min(tok_hi, a.T - 1);
    const char* krow = (const char*)a.k_new + (((size_t)b * a.T + t) * a.Hkv + g) * krow_bytes + half * (kDDQK / 2) * E::kBytes;
#pragma unroll
    for (int i = 0; i < kHalfChunks; ++i) kx[i] = ld16(krow + 16 * i);
    {  // unconditional (threads past nvx re-read a valid chunk, unused), like the K/V rows below
      const int u = min(tid, nvx - 1);  // nvx >= 16: this instance runs only with T > 4
      const int tv = 4 + u / (kDDV / E::kPerChunk), ch = u % (kDDV / E::kPerChunk);
      vx = ld16((const char*)a.v_new + (((size_t)b * a.T + tv) * a.Hkv + g) * vrow_bytes + ch * 16);
    }
    if constexpr (ROPE) rope_load<kRopeDims / 2>(a.rope, P + t, 0, xcs);  // every lane: no branch
  }

  KeyRows<E> cur;
  u32x4 vn;  // a chunk of the V row of new token vn_t (< 4) that this thread fetched, if has_vn
  int vn_t, vn_ch;
  bool has_vn;
  {
    QStage<E, NCB, ROPE> st;
    st.load(a, tid, b, g, cbase, ncols, P);
    // Every wave fetches its K and V rows unconditionally, so the compiler can count them in
    // order behind the Q rows: the Q^T store waits for Q alone and the scores for K alone (with
    // the fetch inside a branch, every wait before the first barrier covered all of them). A
    // wave past the committed keys reads the last committed key; with no committed key at all it
    // reads new token 0 (finite data either way, its scores are masked and P is 0).
    const int pos = max(min(key0 + col, s1 - 1), 0);
    int slot = (pos + off) % a.C;
    slot += slot < 0 ? a.C : 0;
    const size_t kv_row = s1 > 0 ? (row0 + slot) * a.Hkv + g : (size_t)b * a.T * a.Hkv + g;
    cur.load((const char*)(s1 > 0 ? a.k_cache : a.k_new) + kv_row * krow_bytes,
             (const char*)(s1 > 0 ? a.v_cache : a.v_new) + kv_row * vrow_bytes, half);
    st.template store<false>(smem, tid, ncols, true, a.T);
    has_vn = st.new_v_chunk(tid, a.T, vn, vn_t, vn_ch);
  }
  char* sq = smem;
  char* snew = smem + W::kQBytes;
  char* work = snew + W::kNewBytes;
  float* xm = reinterpret_cast<float*>(work + W::kWork);  // [wave][cb][col]
  float* xs = xm + kDecNW * NCB * 32;                     // [token][cb][col], 8 tokens
  float* xl = xs + 2 * kDecNW * NCB * 32;                 // [wave][cb][col]
  __syncthreads();  // Q^T and the new-token rows are in LDS
  if constexpr (EXT && ROPE) {
    if (half == 0) {
#pragma unroll
      for (int j = 0; j < kRopeH<E>; ++j) rope_rotate_chunk<E>(kx[j], kx[j + kRopeH<E>], xcs + 2 * E::kPerChunk * j);
    }
  }

  bool cvalid[NCB];
  int tq[NCB];  // new token of this lane's column in each column block
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    cvalid[cb] = cb * 32 + col < ncols;
    tq[cb] = cvalid[cb] ? (cbase + cb * 32 + col) % a.T : 0;
  }
  const float c = a.scale_log2;

  // ---- 1. S^T of this wave's block, column maxima, new tokens `wave` and `wave + 4` ----
  f32x16 s[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) s[cb] = zero16();
#pragma unroll
  for (int kk = 0; kk < kDDQK / 16; ++kk) {
    const bf16x8 kf = cur.kfrag(kk);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const bf16x8 qf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              sq + ((cb * 32 + col) * Lds::kQStride + 16 * kk + 8 * half) * E::kBytes));
      s[cb] = mma(kf, qf, s[cb]);
    }
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    float bmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int pos = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
      s[cb][r] = (pos < s1 && P + tq[cb] - pos < a.window) ? s[cb][r] * c : -INFINITY;
      bmax = fmaxf(bmax, s[cb][r]);
    }
    bmax = halves_max(bmax);
    if (half == 0) xm[(wave * NCB + cb) * 32 + col] = bmax;
  }
  // score of new token t for this lane's column of every column block: q . k over this half's 96
  // elements (K chunks from `krow` in LDS, or from registers for tokens 4..7), then across halves
  // (EXT: tokens wave and wave + 4 in one pass, sharing the Q^T chunk reads)
  auto new_scores = [&](const char* krow) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const char* qrow = sq + (cb * 32 + col) * Lds::kQStride * E::kBytes;
      float dot = 0.f, dot_hi = 0.f;
#pragma unroll
      for (int i = 0; i < kHalfChunks; ++i) {
        const int e0 = (kDDQK / 2) * half + E::kPerChunk * i;
        const u32x4 qv = *reinterpret_cast<const u32x4*>(qrow + e0 * E::kBytes);
        const u32x4 kv = *reinterpret_cast<const u32x4*>(krow + e0 * E::kBytes);
#pragma unroll
        for (int j = 0; j < 4; ++j) dot = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[j]), as_bf16x2(kv[j]), dot, false);
        if constexpr (EXT) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            dot_hi = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[j]), as_bf16x2(kx[i][j]), dot_hi, false);
        }
      }
      dot = halves_sum(dot);
      const int t = wave;
      const bool vis = cvalid[cb] && tq[cb] >= t && tq[cb] - t < a.window;
      if (half == 0 && t < a.T) xs[(t * NCB + cb) * 32 + col] = vis ? dot * c : -INFINITY;
      if constexpr (EXT) {
        dot_hi = halves_sum(dot_hi);
        const int th = tok_hi;
        const bool vis_hi = cvalid[cb] && tq[cb] >= th && tq[cb] - th < a.window;
        if (half == 0 && th < a.T) xs[(th * NCB + cb) * 32 + col] = vis_hi ? dot_hi * c : -INFINITY;
      }
    }
  };
  // token `wave`'s K row (a clamped, valid row when wave >= T; its score is then not written)
  if (wave < a.T || EXT) new_scores(snew + min(wave, a.T - 1) * kDDQK * E::kBytes);
  // the V half rows (requested after the K half rows) go to the wave's V tile only now, so the
  // scores above wait for K alone (stored before them, every MFMA waited for the V rows too)
  __builtin_amdgcn_sched_barrier(0);
  cur.store_v(work + wave * W::kVBytes, col, half);
  __syncthreads();  // maxima and new-token scores are in LDS; Q^T is no longer read

  // ---- 2. P of this block against the common maximum ----
  constexpr int kNT = EXT ? 2 * kDecNW : kDecNW;  // new tokens this instance handles
  float M[NCB], sink_l2[NCB], snt[kNT][NCB];
  int head[NCB];
  char* sp = sq;  // P fragments [block][ks][cb][lane], 16 bytes each, over the Q^T rows
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    head[cb] = cvalid[cb] ? a.hl.at(g * a.G + (cbase + cb * 32 + col) / a.T) : 0;
    sink_l2[cb] = (a.sink && cvalid[cb]) ? a.sink[head[cb]] * kLog2e : -INFINITY;
    M[cb] = sink_l2[cb];
#pragma unroll
    for (int w = 0; w < kDecNW; ++w) M[cb] = fmaxf(M[cb], xm[(w * NCB + cb) * 32 + col]);
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      snt[t][cb] = t < a.T ? xs[(t * NCB + cb) * 32 + col] : -INFINITY;
      M[cb] = fmaxf(M[cb], snt[t][cb]);
    }
    const float M_use = (M[cb] == -INFINITY) ? 0.f : M[cb];
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[cb][r] = fast_exp2(s[cb][r] - M_use);
      rs += s[cb][r];
    }
    rs = halves_sum(rs);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      st16(sp + (((wave * 2 + ks) * NCB + cb) * 64 + lane) * 16, __builtin_bit_cast(u32x4, frag_from_acc<E>(s[cb], 8 * ks)));
    if (half == 0) xl[(wave * NCB + cb) * 32 + col] = rs;
  }
  // the new tokens' V rows as one 16-row tile next to the P fragments, in the part of the Q^T
  // rows P leaves free (padded rows like the V tiles, rows T..15 zero): they enter O^T through one
  // more MFMA per column block. Rows 0..3 come from the chunks fetched with Q at kernel start,
  // rows 4..7 (EXT) from those fetched with the K rows of tokens 4..7; every chunk of rows 0..T-1
  // has exactly one holder.
  char* vnew = sq + W::kPBytes;
  {
    constexpr int kCh = kDDV / E::kPerChunk;  // 16-byte chunks per V row
    const int r = tid / kCh, ch = tid % kCh;  // 256 threads: rows 0..15
    if (r >= a.T) st16(vnew + (r * Lds::kVStride) * E::kBytes + ch * 16, zero_chunk());
    if (has_vn) st16(vnew + (vn_t * Lds::kVStride) * E::kBytes + vn_ch * 16, vn);
    if (EXT && tid < nvx) st16(vnew + ((4 + tid / kCh) * Lds::kVStride) * E::kBytes + (tid % kCh) * 16, vx);
  }
  __syncthreads();  // P fragments, block sums and the new tokens' V tile are in LDS

  // ---- 3. dv rows 32 wave .. 32 wave + 31 of O^T over all blocks, new tokens, sink ----
  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = zero16();
#pragma unroll
  for (int kb = 0; kb < kDecNW; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 vf = vt_frag_tr(work + kb * W::kVBytes, Lds::kVStride, wave, ks, lane);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const bf16x8 pf = __builtin_bit_cast(bf16x8, ld16(sp + (((kb * 2 + ks) * NCB + cb) * 64 + lane) * 16));
        acc[cb] = mma(vf, pf, acc[cb]);
      }
    }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float M_use = (M[cb] == -INFINITY) ? 0.f : M[cb];
    float L = a.sink && cvalid[cb] ? fast_exp2(sink_l2[cb] - M_use) : 0.f;
#pragma unroll
    for (int w = 0; w < kDecNW; ++w) L += xl[(w * NCB + cb) * 32 + col];
    // new tokens: p of token t for this lane's column; the B fragment of one 16-key MFMA step
    // holds, in lane half h, tokens 4h .. 4h + 3 then four zeros (the key order of the
    // transposing V^T read: keys 4h..4h+3, then 8+4h..8+4h+3, rows 8..15 of the tile being zero)
    auto pnew = [&](int t) { return t < kNT && t < a.T ? fast_exp2(snt[t < kNT ? t : 0][cb] - M_use) : 0.f; };
    {
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = pnew(e), hi = pnew(4 + e);  // scalars: a select of two array elements
        L += lo + hi;                                // became a run-time index into memory
        f[e] = half ? hi : lo;
        f[4 + e] = 0.f;
      }
      const bf16x8 pf = frag_from_f32<E>(f);
      acc[cb] = mma(vt_frag_tr(vnew, Lds::kVStride, wave, 0, lane), pf, acc[cb]);
    }
    if (!cvalid[cb]) continue;
    const float inv = 1.f / L;
    char* orow = (char*)a.o + (((size_t)b * a.T + tq[cb]) * a.Hq + head[cb]) * kDDV * E::kBytes;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      u32x2 w2;
      w2[0] = pack_bf16x2(acc[cb][4 * gq] * inv, acc[cb][4 * gq + 1] * inv);
      w2[1] = pack_bf16x2(acc[cb][4 * gq + 2] * inv, acc[cb][4 * gq + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + (32 * wave + 8 * gq + 4 * half) * 2) = w2;
    }
    if (a.lse && wave == 0 && half == 0)
      a.lse[((size_t)b * a.T + tq[cb]) * a.Hq + head[cb]] = (M[cb] + fast_log2(L)) * kLn2;
  }
}

// ------------------------------------------------------ column-split decode (many query columns)
//
// Decode with more than 32 query columns per KV head (16 heads x 4 or x 8 tokens of a global layer)
// in one pass over the cache. With 128 columns per workgroup, wave w owns query columns
// 32 w .. 32 w + 31; with 64, waves w and w + 2 share column block w and split the dv rows. The
// four waves share every 32-key block of K and V in LDS (two stages). Per block each
// wave forms S^T = K Q^T of its columns (K fragments from LDS, Q^T fragments in registers), runs
// the online softmax of its columns and adds V^T P^T (V^T read transposed from LDS): every cached
// byte is read from HBM once for all 128 columns, and the accumulators of a wave stay at 64
// registers. Blocks are staged through registers two blocks ahead: block i + 2 is requested
// before block i's math, block i + 1 (requested a block earlier) is written to LDS after it.
// (Global -> LDS loads into three stages were slower: the compiler could not tell the stages apart
// for one of the three and made that block's LDS reads wait for every fetch in flight.) The last
// split then takes the T new tokens as one more block (rotated on the way with RoPE). No merge
// between waves: each writes its own columns' O (one split: sink folded, LSE) or split records for
// combine_kernel.
struct ColsTile {
  static constexpr int kKStride = kDDQK + 8, kVStride = kDDV + 16;  // bf16 per LDS row (padded)
  static constexpr int kKBytes = 32 * kKStride * 2, kStageBytes = kKBytes + 32 * kVStride * 2;
  // staging: thread t moves row t / 8 of the block, K chunks 3 (t % 8) .. +2 and V chunks
  // 2 (t % 8) .. +1 (16-byte chunks; 24 per K row, 16 per V row)
  static constexpr int kKPer = kDDQK / 8 / 8, kVPer = kDDV / 8 / 8;
};

struct ColsRegs {
  u32x4 k[ColsTile::kKPer], v[ColsTile::kVPer];
};

// Requests thread tid's chunks of the 32-key block at key0 (keys past s1 - 1 read key s1 - 1,
// masked later); position p is in slot (p + off) mod C.
__device__ __forceinline__ void cols_load(ColsRegs& r, const char* kc, const char* vc, size_t kstride,
                                          size_t vstride, size_t row0, int key0, int s1, int off, int C,
                                          int tid) {
  const int row = min(tid >> 3, s1 - 1 - key0), q = tid & 7;
  int slot = (key0 + row + off) % C;
  slot += slot < 0 ? C : 0;
  const char* kp = kc + (row0 + slot) * kstride + q * ColsTile::kKPer * 16;
  const char* vp = vc + (row0 + slot) * vstride + q * ColsTile::kVPer * 16;
#pragma unroll
  for (int i = 0; i < ColsTile::kKPer; ++i) r.k[i] = ld16(kp + 16 * i);
#pragma unroll
  for (int i = 0; i < ColsTile::kVPer; ++i) r.v[i] = ld16(vp + 16 * i);
}

__device__ __forceinline__ void cols_store(char* stage, const ColsRegs& r, int tid) {
  const int row = tid >> 3, q = tid & 7;
  char* kd = stage + row * ColsTile::kKStride * 2 + q * ColsTile::kKPer * 16;
  char* vd = stage + ColsTile::kKBytes + row * ColsTile::kVStride * 2 + q * ColsTile::kVPer * 16;
#pragma unroll
  for (int i = 0; i < ColsTile::kKPer; ++i) st16(kd + 16 * i, r.k[i]);
#pragma unroll
  for (int i = 0; i < ColsTile::kVPer; ++i) st16(vd + 16 * i, r.v[i]);
}

// NCB column blocks of 32 per workgroup: 4 (128 columns, each wave all 128 dv rows of its block)
// or 2 (64 columns: waves w and w + 2 share column block w and take dv rows 0..63 and 64..127;
// both form the block's scores).
template <int NCB, bool ROPE>
__global__ __launch_bounds__(kColsNW * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_cols_kernel(
    const DecodeArgs a) {
  using E = BF16;
  using T = ColsTile;
  static_assert(NCB == 4 || NCB == 2, "128 or 64 columns per workgroup");
  constexpr int NDB = (kDDV / 32) * NCB / kColsNW;  // dv blocks of 32 per wave
  __shared__ __attribute__((aligned(16))) char smem[2 * T::kStageBytes];
  poison_lds(smem, sizeof(smem));
  char* const st0 = smem;
  char* const st1 = smem + T::kStageBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int split = blockIdx.x;
  const int chunk = blockIdx.y % a.n_chunks;
  const int g = blockIdx.y / a.n_chunks;
  const int b = blockIdx.z;
  const int cbase = chunk * a.chunk_cols;
  const int ncols = min(a.chunk_cols, a.ncols - cbase);

  int P = a.cache_len[b];
  P = P < 0 ? 0 : (P > a.max_len ? a.max_len : P);
  const int off = a.cache_offset ? a.cache_offset[b] : 0;
  const int list0 = max(0, P - a.window + 1);
  // split s takes the 32-key blocks s, s + nsplit, s + 2 nsplit, ... of the keys [list0, P): the
  // splits of a sequence then read neighbouring blocks at the same time instead of each streaming
  // its own contiguous stretch (long-context decode 0.929 -> 0.918 ms)
  const int s1 = P;
  const int nbt = P > list0 ? (P - list0 + 31) / 32 : 0;
  const int nb = split < nbt ? (nbt - 1 - split) / a.nsplit + 1 : 0;
  auto bkey = [&](int i) { return list0 + 32 * (i * a.nsplit + split); };

  const size_t krow_bytes = (size_t)kDDQK * 2, vrow_bytes = (size_t)kDDV * 2;
  const char* kc = (const char*)a.k_cache + (size_t)g * krow_bytes;
  const char* vc = (const char*)a.v_cache + (size_t)g * vrow_bytes;
  const size_t kstride = (size_t)a.Hkv * krow_bytes, vstride = (size_t)a.Hkv * vrow_bytes;
  const size_t row0 = (size_t)b * a.C;

  // this lane's query column (padding columns load a valid row and are never written) and the
  // wave's dv blocks db0 .. db0 + NDB - 1
  const int cl = 32 * (wave % NCB) + col;
  const int db0 = NDB * (wave / NCB);
  const bool cvalid = cl < ncols;
  const int c = cbase + min(cl, ncols - 1);
  const int t = c % a.T;
  const int head = a.hl.at(g * a.G + c / a.T);
  const int qpos = P + t;

  // the first two blocks' requests, then the Q^T fragments (rotated at position P + t with RoPE)
  // With 128 columns every fetch below is unconditional (past the split's last block: that block
  // again, unused), so the compiler's wait counts see one straight-line sequence and the fetch
  // of block i + 2 stays in flight across step i. Under branches (as with 64 columns), each
  // step's LDS store waits for the fetch issued at the top of that same step, and the products
  // for everything in flight: about one block ahead instead of two. Measured: 128 columns (16
  // heads x 8 tokens) 1.035 -> 1.010 ms with the two-ahead fetch; 64 columns 0.947 -> 0.983 ms,
  // so those keep the branches (more fetches in flight from every workgroup read the cache at
  // more places at once).
  constexpr bool kAhead2 = NCB == 4;
  ColsRegs r0, r1;
  if (kAhead2 || nb > 0) cols_load(r0, kc, vc, kstride, vstride, row0, bkey(0), s1, off, a.C, tid);
  if (kAhead2 || nb > 1)
    cols_load(r1, kc, vc, kstride, vstride, row0, bkey(min(1, max(nb - 1, 0))), s1, off, a.C, tid);
  bf16x8 qf[kDDQK / 16];
  {
    const char* qrow = (const char*)a.q + (((size_t)b * a.T + t) * a.Hq + head) * krow_bytes;
#pragma unroll
    for (int kk = 0; kk < kDDQK / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, ld16(qrow + (16 * kk + 8 * half) * 2));
    if constexpr (ROPE) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float cs[16];
        rope_load<8>(a.rope, qpos, 16 * kk + 8 * half, cs);
        rope_rotate_frag<E>(qf[kk], qf[kk + 2], cs);
      }
    }
  }
  if (nb > 0) cols_store(st0, r0, tid);
  if constexpr (kAhead2) wait_all();  // Q^T (fetched last) has landed; the loop counts its own fetches
  __syncthreads();

  const float c2 = a.scale_log2;
  float m = -INFINITY, l = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  // one 32-key block from `stage`: vis(k) says whether key row k (0..31) is visible to this lane's
  // column (only called when the block is not wholly visible)
  auto block = [&](const char* stage, bool full, auto vis) {
    f32x16 s = zero16();
#pragma unroll
    for (int kk = 0; kk < kDDQK / 16; ++kk) {
      const bf16x8 kf = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(stage + (col * T::kKStride + 16 * kk + 8 * half) * 2));
      s = mma(kf, qf[kk], s);
    }
    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = vis(8 * (r >> 2) + 4 * half + (r & 3)) ? s[r] : -INFINITY;
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, s[r]);
    const float mb = halves_max(bmax) * c2;
    // lazy running max (log2 units): rescale only when a candidate exceeds it by more than 8
    if (__builtin_amdgcn_ballot_w64(mb > m + 8.f || (m == -INFINITY && mb > m)) != 0) {
      const float m_new = fmaxf(m, mb);
      const float alpha = fast_exp2(m - (m_new == -INFINITY ? 0.f : m_new));
      l *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
      m = m_new;
    }
    const float m_use = (m == -INFINITY) ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(__builtin_fmaf(s[r], c2, -m_use));
      s[r] = p;
      rs += p;
    }
    l += halves_sum(rs);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pf = frag_from_acc<E>(s, 8 * ks);
#pragma unroll
      for (int d = 0; d < NDB; ++d)
        acc[d] = mma(vt_frag_tr(stage + T::kKBytes, T::kVStride, db0 + d, ks, lane), pf, acc[d]);
    }
  };

  // committed keys: step i requests block i + 2 into the register set that held block i, does
  // block i's math, writes block i + 1 into the other stage (free: read in step i - 1) and closes
  // with a barrier; the register sets and stages alternate, so the loop runs two steps per trip
  auto step = [&](int i, const char* cur, char* other, ColsRegs& mine, const ColsRegs& next) {
    if (kAhead2 || i + 2 < nb)
      cols_load(mine, kc, vc, kstride, vstride, row0, bkey(min(i + 2, nb - 1)), s1, off, a.C, tid);
    __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the math
    const int key0 = bkey(i);
    const bool full = key0 + 32 <= s1 && P + a.T - 1 - key0 < a.window;
    block(cur, full, [&](int k) { return key0 + k < s1 && qpos - (key0 + k) < a.window; });
    if (i + 1 < nb) cols_store(other, next, tid);
    __syncthreads();
  };
  for (int i = 0; i < nb; i += 2) {
    step(i, st0, st1, r0, r1);
    if (i + 1 < nb) step(i + 1, st1, st0, r1, r0);
  }

  // new tokens (last split): rows 0..T-1 of a block hold their K and V (rotated at P + tn with
  // RoPE), rows T..31 zeros; laid out 40 chunks (24 K, 16 V) per row on consecutive threads, so a
  // row's rotated chunks and their partners share one wave
  if (split == a.nsplit - 1) {
    __syncthreads();  // every wave is done with the stages
    constexpr int kKCh = kDDQK / 8, kRow = kKCh + kDDV / 8;
    for (int u = tid; u < 32 * kRow; u += kColsNW * 64) {  // same trip count in every lane
      const int r = u / kRow, ch = u % kRow;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (r < a.T)
        x = ch < kKCh ? ld16((const char*)a.k_new + (((size_t)b * a.T + r) * a.Hkv + g) * krow_bytes + ch * 16)
                      : ld16((const char*)a.v_new + (((size_t)b * a.T + r) * a.Hkv + g) * vrow_bytes + (ch - kKCh) * 16);
      if constexpr (ROPE) {
        constexpr int H = kRopeH<E>;
        float cs[16];
        const bool rot = r < a.T && ch < 2 * H;
        if (rot) rope_load<8>(a.rope, P + r, (ch % H) * 8, cs);
        x = rope_chunk_xlane<E>(x, rot ? ch : 2 * H, lane, cs);
      }
      if (ch < kKCh)
        st16(st0 + (r * T::kKStride) * 2 + ch * 16, x);
      else
        st16(st0 + T::kKBytes + (r * T::kVStride) * 2 + (ch - kKCh) * 16, x);
    }
    __syncthreads();
    block(st0, false, [&](int k) { return k < a.T && k <= t && t - k < a.window; });
  }

  if (!cvalid) return;
  if (a.nsplit == 1) {
    const float s_l2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
    const float M = fmaxf(m, s_l2);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    const float w = fast_exp2(m - M_use);
    const float L = l * w + (a.sink ? fast_exp2(s_l2 - M_use) : 0.f);
    const float sc = w / L;
    char* orow = (char*)a.o + (((size_t)b * a.T + t) * a.Hq + head) * vrow_bytes;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x2 w2;
        w2[0] = pack_bf16x2(acc[d][4 * j] * sc, acc[d][4 * j + 1] * sc);
        w2[1] = pack_bf16x2(acc[d][4 * j + 2] * sc, acc[d][4 * j + 3] * sc);
        *reinterpret_cast<u32x2*>(orow + (32 * (db0 + d) + 8 * j + 4 * half) * 2) = w2;
      }
    if (a.lse && half == 0 && db0 == 0) a.lse[((size_t)b * a.T + t) * a.Hq + head] = (M + fast_log2(L)) * kLn2;
  } else {
    // split record of column c: unnormalised acc against this split's max m, and l
    const int ncols_pad = ((a.ncols + 31) / 32) * 32;
    float* rec = a.ws + ((((size_t)b * a.Hkv + g) * a.nsplit + split) * ncols_pad + c) * kRec;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 w4;
        w4[0] = acc[d][4 * j]; w4[1] = acc[d][4 * j + 1]; w4[2] = acc[d][4 * j + 2]; w4[3] = acc[d][4 * j + 3];
        *reinterpret_cast<f32x4*>(rec + 32 * (db0 + d) + 8 * j + 4 * half) = w4;
      }
    if (half == 0 && db0 == 0) {
      rec[kDDV] = m;
      rec[kDDV + 1] = l;
    }
  }
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

// The one-pass window kernel serves a single split of at most four 32-key blocks with at most
// 64 query columns per workgroup and at most 8 new tokens.
static bool window_kernel_fits(const DecodeArgs& a) {
  const bool cols = a.chunk_cols <= 2 * 32;  // every workgroup's chunk fits two column blocks
  return a.nsplit == 1 && a.keys_per_split <= 32 * kDecNW && cols && a.T <= 2 * kDecNW;
}

// With one column block (e.g. 8 query heads x 4 tokens) a wave holds few blocks and fewer
// registers buy a second wave per SIMD; that beats prefetching (measured on the ring workload),
// so the one-column kernel does not prefetch.
constexpr bool kPrefetch1Col = false;

template <bool ROPE>
static void launch_decode_kernel(bool bf16, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, a.Hkv * a.n_chunks, a.B);
  const dim3 block(kDecNW * 64);
  if (bf16 && a.chunk_cols == kColsCols) {
    hipLaunchKernelGGL((decode_cols_kernel<4, ROPE>), grid, dim3(kColsNW * 64), 0, stream, a);
    return;
  }
  if (bf16 && window_kernel_fits(a)) {
    const bool two = (a.n_chunks > 1 ? a.chunk_cols : a.ncols) > 32;
    if (two && a.T > kDecNW)
      hipLaunchKernelGGL((decode_window_kernel<2, ROPE, true>), grid, block, 0, stream, a);
    else if (two)
      hipLaunchKernelGGL((decode_window_kernel<2, ROPE, false>), grid, block, 0, stream, a);
    else if (a.T > kDecNW)
      hipLaunchKernelGGL((decode_window_kernel<1, ROPE, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_window_kernel<1, ROPE, false>), grid, block, 0, stream, a);
    return;
  }
  // bf16 with 33..64 columns: the column-split kernel (2 column blocks, dv halves per wave)
  const bool two = (a.n_chunks > 1 ? a.chunk_cols : a.ncols) > 32;
  if (bf16 && two)
    hipLaunchKernelGGL((decode_cols_kernel<2, ROPE>), grid, dim3(kColsNW * 64), 0, stream, a);
  else if (bf16)
    hipLaunchKernelGGL((decode_kernel<BF16, 1, kPrefetch1Col, ROPE>), grid, block, 0, stream, a);
  else  // fp32: column chunks of 32
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
