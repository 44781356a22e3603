// Prefill kernels: sink-seeded sliding-window / causal attention on gfx950 MFMA.
//
// Operation: MiMo-V2-Flash Technical Report review (xllm-io), §3.1 (window 128, GQA 64/8 and 64/4,
// head dims 192/128) and §3.2 (per-head sink logit in the softmax denominator); MiMo series notes
// (plmsmile), MiMo-V2-Flash > Learnable Attention Sink > mechanism (real-token weights may sum to
// less than one; the sink carries no value).
//
// Shared structure:
//   * A workgroup owns one KV head g of one sequence b and a group of query heads of g, so every
//     K/V block it stages in LDS serves all of those heads (GQA reuse).
//   * Wave w owns one query head and a tile of 32 consecutive query positions = 32 MFMA columns.
//   * Scores are formed transposed, S^T = K Q^T, so each lane holds one query column: row max and
//     sum need one cross-half exchange, and P^T feeds O^T += V^T P^T straight from registers.
//   * The softmax starts from the sink, m = s_h * log2(e), l = 1 (no sink: m = -inf, l = 0), so
//     the sink is counted once and is never multiplied by the scale. Scores are scaled inside the
//     exponent: p = exp2(s * scale * log2(e) - m), which needs scale > 0 (checked by the host).
//   * Rows or keys past the end of the sequence are read from clamped, valid addresses: their
//     scores are masked to -inf, so they get weight exactly 0 and touch no output.
//
// prefill_swa_kernel (bf16, window <= 129, query heads per KV head a multiple of 8): a workgroup
//   walks a segment of consecutive 32-position tiles. The window of a tile is NB 32-key blocks;
//   they sit in an LDS ring of NB + 1 slots, so each K/V row is fetched once per segment and only
//   the next tile's diagonal block is loaded per step (prefetched under the current tile's math).
//   The whole window is scored before the softmax, so it is single pass (no rescaling).
// prefill_kernel (generic: global attention, fp32, other shapes): streams the union of the
//   workgroup's windows in BK-key blocks, double-buffered in LDS, with an online softmax whose
//   running max is refreshed lazily (see below).
#include <type_traits>

#include "tiles.hpp"

namespace mimo {

// ------------------------------------------------------------------------ generic streaming kernel

constexpr float kLazyRescale = 8.f;  // log2 units

// ROPE: kPreRopeNone (Q and K rotated already), kPreRopeQK (both rotated here: Q once, K at every
// staging), kPreRopeQ (Q rotated here, K rotated beforehand by rope_k_kernel).
constexpr int kPreRopeNone = 0, kPreRopeQK = 1, kPreRopeQ = 2;

template <typename E, int NW, int BK, int ROPE>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(const PrefillArgs a) {
  using Tile = PrefillTile<E, BK>;
  using Frag = typename E::Frag;
  constexpr int NT = NW * 64;
  constexpr int NSB = BK / 32;  // 32-key sub-blocks per block
  __shared__ __attribute__((aligned(16))) char smem[2 * Tile::kStageBytes];
  poison_lds(smem, sizeof(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on it

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
  const int head = a.hl.at(g * a.G + hc * HG + wave % HG);
  const int P0 = qb * kQT * qtiles;
  const int P1 = min(a.L, P0 + kQT * qtiles);
  const int p0 = P0 + kQT * (wave / HG);  // this wave's first query position
  const int qpos = p0 + col;              // this lane's query position

  const size_t krow_stride = (size_t)a.Hkv * kDQK * E::kBytes;
  const size_t vrow_stride = (size_t)a.Hkv * kDV * E::kBytes;
  const char* kbase = (const char*)a.k + ((size_t)b * a.L * a.Hkv + g) * kDQK * E::kBytes;
  const char* vbase = (const char*)a.v + ((size_t)b * a.L * a.Hkv + g) * kDV * E::kBytes;

  Frag qf[kDQK / 16];
  {
    const int qload = min(qpos, a.L - 1);
    const char* qrow = (const char*)a.q + (((size_t)b * a.L + qload) * a.Hq + head) * kDQK * E::kBytes;
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) qf[kk] = global_q_frag<E>(qrow, kk, half);
    if constexpr (ROPE != kPreRopeNone) {
      // fragments 0, 1 hold dims 16 kk + 8 half .. +7 of the rotated slice, 2, 3 their partners
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float cs[16];
        rope_load<8>(a.rope, qload, 16 * kk + 8 * half, cs);
        rope_rotate_frag<E>(qf[kk], qf[kk + 2], cs);
      }
    }
  }

  const float c = a.scale_log2;
  const float sink_l2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
  float m = sink_l2;
  float l = a.sink ? 1.f : 0.f;
  f32x16 acc[kDV / 32];
#pragma unroll
  for (int db = 0; db < kDV / 32; ++db) acc[db] = zero16();

  const int K0 = max(0, P0 - a.window + 1);
  const int kstart = (K0 / BK) * BK;
  const int nblk = (P1 - kstart + BK - 1) / BK;

  // bf16 64-key blocks go global -> LDS directly (no staging registers); the others through
  // registers
  constexpr bool kDMA = E::kBytes == 2 && BK == 64 && ROPE != kPreRopeQK;
  KVStager<E, NT, BK, ROPE == kPreRopeQK ? kRopeMem : kRopeNone> st;
  KVStagerDMA<NW, 64> dma;  // used only when kDMA (BK == 64)
  if constexpr (kDMA) {
    dma.init(krow_stride, vrow_stride, wave, lane);
    dma.load(smem, kbase, vbase, krow_stride, vrow_stride, kstart, a.L, wave, lane);
    wait_vm();
  } else {
    st.init(krow_stride, vrow_stride, tid);
    st.load(kbase, vbase, krow_stride, vrow_stride, kstart, a.L, tid, a.rope);
    st.store(smem, tid);
    wait_all();
  }
  __syncthreads();

  // One block: stage the next block's loads, score, softmax, PV, store the next block, barrier.
  // MASKED is a compile-time copy: blocks that every query of the tile sees in full run without
  // any masking code (left to itself the compiler guards each score with its own branch).
  auto block = [&](int ib, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int key0 = kstart + ib * BK;
    if (ib + 1 < nblk) {
      if constexpr (kDMA)
        dma.load(smem + ((ib + 1) & 1) * Tile::kStageBytes, kbase, vbase, krow_stride, vrow_stride, key0 + BK,
                 a.L, wave, lane);
      else
        st.load(kbase, vbase, krow_stride, vrow_stride, key0 + BK, a.L, tid, a.rope);
    }

    const bool skip = MASKED && ((key0 > p0 + kQT - 1) || (key0 + BK - 1 < p0 - a.window + 1) || (p0 >= a.L));
    if (!skip) {
      // LLVM's interleaving strategy 0 for this scheduling region (K fragment reads spread
      // between the score MFMAs): -2% on the global layer
      __builtin_amdgcn_iglp_opt(0);
      const char* sk = smem + (ib & 1) * Tile::kStageBytes;
      const char* sv = sk + Tile::kKBytes;

      f32x16 s[NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) s[sb] = zero16();
#pragma unroll
      for (int kk = 0; kk < kDQK / 16; ++kk)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
          s[sb] = mma(lds_k_frag<E, BK>(sk, 32 * sb + col, kk, half), qf[kk], s[sb]);

      float bmax = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (MASKED) {
            const int key = key0 + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
            const int d = qpos - key;
            s[sb][r] = (d >= 0 && d < a.window) ? s[sb][r] : -INFINITY;
          }
          bmax = fmaxf(bmax, s[sb][r]);
        }
      }
      // lazy max: rescale only when some lane's block max exceeds its running max by more than
      // kLazyRescale; otherwise exponentiate against the stale max (values stay below
      // 2^kLazyRescale, and the same max scales l and acc, so the result is unchanged)
      const float mb = halves_max(bmax) * c;
      if (__builtin_amdgcn_ballot_w64(mb > m + kLazyRescale || (m == -INFINITY && mb > m)) != 0) {
        const float m_new = fmaxf(m, mb);
        const float alpha = fast_exp2(m - (m_new == -INFINITY ? 0.f : m_new));
        l *= alpha;
#pragma unroll
        for (int db = 0; db < kDV / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        m = m_new;
      }
      const float m_use = (m == -INFINITY) ? 0.f : m;
      float rs = 0.f;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[sb][r], c, -m_use));
          s[sb][r] = p;
          rs += p;
        }
      }
      l += halves_sum(rs);
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const Frag pf = frag_from_acc<E>(s[ks >> 1], 8 * (ks & 1));
#pragma unroll
        for (int db = 0; db < kDV / 32; ++db)
          acc[db] = mma(lds_vt_frag<E, BK>(sv, db, ks, lane), pf, acc[db]);
      }
    }

    if constexpr (kDMA) {
      wait_vm();  // this wave's loads of the next stage have landed
    } else {
      if (ib + 1 < nblk) st.store(smem + ((ib + 1) & 1) * Tile::kStageBytes, tid);
    }
    __syncthreads();
  };

  // Blocks [ib_a, ib_b) are seen in full by every query of this wave's tile: all their keys are
  // at or before the tile's first position and within the window of its last one. Waves may
  // differ in the range: every wave still runs all nblk blocks with the same stage loads, stores
  // and barriers, only its own math takes one copy or the other. Tiles past L take the masked
  // copy (which skips them).
  int ib_a = nblk, ib_b = nblk;
  if (p0 < a.L) {
    const int hi_num = p0 - (BK - 1) - kstart;  // ib < hi  <=>  key0 + BK - 1 <= p0
    const int hi = hi_num >= 0 ? hi_num / BK + 1 : 0;
    const long long lo_num = (long long)p0 + kQT - a.window - kstart;  // ib >= lo  <=>  p0 + kQT - 1 - key0 < window
    const int lo = lo_num <= 0 ? 0 : (int)min<long long>((lo_num + BK - 1) / BK, nblk);
    ib_a = min(lo, nblk);
    ib_b = min(max(hi, ib_a), nblk);
  }
  ib_a = __builtin_amdgcn_readfirstlane(ib_a);
  ib_b = __builtin_amdgcn_readfirstlane(ib_b);
  // runs: masked [0, ib_a), mask-free [ib_a, ib_b), masked [ib_b, nblk); one call site per copy
  for (int ib = 0; ib < nblk;) {
    const int stop = ib < ib_a ? ib_a : (ib < ib_b ? ib : nblk);
    for (; ib < stop; ++ib) block(ib, std::true_type{});
    for (; ib < ib_b; ++ib) block(ib, std::false_type{});
  }

  const bool valid = qpos < a.L;
  char* orow = (char*)a.o + (((size_t)b * a.L + min(qpos, a.L - 1)) * a.Hq + head) * kDV * E::kBytes;
  store_out_row<E>(orow, acc, 1.f / l, half, valid);
  if (a.lse && half == 0 && valid)
    a.lse[((size_t)b * a.Hq + head) * a.L + qpos] = (m + fast_log2(l)) * kLn2;
}

// ------------------------------------------------------------ global (causal) ping-pong kernel

#ifndef MIMO_GA_PINGPONG
#define MIMO_GA_PINGPONG 1
#endif
#ifndef MIMO_GA_BK
#define MIMO_GA_BK 96
#endif
#ifndef MIMO_GA_DEPTH
#define MIMO_GA_DEPTH 2
#endif
#ifndef MIMO_GA_SGB
#define MIMO_GA_SGB 1
#endif
//
// bf16 global attention with 8 query heads per workgroup (wave w = head w of the chunk, all on the
// same 32 query rows; waves w and w + 4 share a SIMD), over key blocks of BK keys. Each wave
// alternates MFMA phases M_k = [O^T += V^T P^T of block k - 1, S^T = K Q^T of block k] and softmax
// phases V_k (masking, running max, exponentials, P to bf16 fragments, rescale). Waves 0-3
// (group A) run one phase ahead of waves 4-7 (group B), so on every SIMD one wave issues MFMAs
// while the other works on the VALU; a barrier closes every phase ("slot"):
//     slot 2k:   A runs M_k,  B runs V_{k-1}          slot 2k + 1:  A runs V_k,  B runs M_k
// With n blocks there are 2n + 2 slots, and every wave passes the same 2n + 3 barriers (one after
// the prologue). K of block k and V of block k - 1 are read in exactly slots 2k and 2k + 1, so they
// share stage k % 2 of two LDS stages; the stage that they overwrite was read last in slot 2k - 3
// (K) or 2k - 1 (V). Staging is global -> LDS (no registers) and happens in softmax phases, which
// read no LDS: group B fetches K of block k + 1 in slot 2k (its V_{k-1}), group A fetches V of
// block k in slot 2k + 1 (its V_k); each waits for its loads before the barrier that closes the
// slot. (The compiler makes a wave's LDS reads wait for all of its loads that target LDS, so loads
// issued before an MFMA phase would stall it.)
// Scheduling-group pattern of an M phase (masks: 0x100 LDS reads, 0x008 MFMA): the reads of the
// first D operand fragments, then product i followed by the reads of fragment i + D. Fragments of
// the first NPV products (V^T) take two transposing reads, the others (K) one.
template <int NPV, int NM, int D, int I>
struct GaReadAhead {
  static constexpr int reads(int i) { return i < NPV ? 2 : 1; }
  static constexpr int first() {
    int r = 0;
    for (int i = 0; i < D && i < NM; ++i) r += reads(i);
    return r;
  }
  __device__ __forceinline__ static void emit() {
    if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(0x100, first(), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (I + D < NM) __builtin_amdgcn_sched_group_barrier(0x100, reads(I + D), 0);
    if constexpr (I + 1 < NM) GaReadAhead<NPV, NM, D, I + 1>::emit();
  }
};

// LDS stage of the ping-pong kernel: K rows [BK][192 + 8], then V rows [BK][128 + 16] (bf16; the
// padding keeps the K rows' 16-byte reads on distinct banks)
template <int BK>
struct GaTile {
  static constexpr int kKStride = kDQK + 8, kVStride = kDV + 16;
  static constexpr int kKBytes = BK * kKStride * 2, kVBytes = BK * kVStride * 2;
  static constexpr int kStageBytes = kKBytes + kVBytes;
};

template <int ROPE, int BK>
__global__ __launch_bounds__(512) void prefill_global_kernel(const PrefillArgs a) {
  using E = BF16;
  using Tile = GaTile<BK>;
  using Frag = bf16x8;
  constexpr int NW = 8, NS = 2;
  constexpr int NKB = BK / 32;  // 32-key MFMA row blocks of a key block
  constexpr int NKS = BK / 16;  // 16-key slices (PV contraction steps)
  static_assert(BK % 32 == 0 && NS * Tile::kStageBytes <= 160 * 1024, "two stages fit LDS");
  __shared__ __attribute__((aligned(16))) char smem[NS * Tile::kStageBytes];
  poison_lds(smem, sizeof(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: one phase ahead, 1: one phase behind

  // heaviest query blocks (latest positions) first; consecutive workgroups differ in (KV head,
  // head chunk)
  const int per_q = a.B * a.Hkv * a.n_hchunks;
  const int qb = a.n_qblocks - 1 - (int)(blockIdx.x / per_q);
  int rest = blockIdx.x % per_q;
  const int hc = rest % a.n_hchunks;
  rest /= a.n_hchunks;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int head = a.hl.at(g * a.G + hc * NW + wave);
  const int p0 = qb * kQT;  // the workgroup's (and every wave's) first query row
  const int qpos = p0 + col;
  const int P1 = min(a.L, p0 + kQT);
  const int n = (P1 + BK - 1) / BK;  // key blocks [0, P1)

  const size_t krow_stride = (size_t)a.Hkv * kDQK * 2;
  const size_t vrow_stride = (size_t)a.Hkv * kDV * 2;
  const char* kbase = (const char*)a.k + ((size_t)b * a.L * a.Hkv + g) * kDQK * 2;
  const char* vbase = (const char*)a.v + ((size_t)b * a.L * a.Hkv + g) * kDV * 2;

  // group B (waves 4-7) stages K, group A (waves 0-3) stages V
  const int gw = wave & 3;
  using KDma = RowsDMA<4, BK, Tile::kKStride * 2 / 16, kDQK / 8>;
  using VDma = RowsDMA<4, BK, Tile::kVStride * 2 / 16, kDV / 8>;
  static_assert(KDma::kChunks * 16 == Tile::kKBytes && VDma::kChunks * 16 == Tile::kVBytes, "regions tile the stage");
  uint32_t doff[KDma::kPer > VDma::kPer ? KDma::kPer : VDma::kPer];
  auto stage_k = [&](int kb) {  // K of block kb into stage kb % 2 (group B)
    KDma::load(doff, smem + (kb % NS) * Tile::kStageBytes, kbase, krow_stride, kb * BK, a.L, gw, lane);
  };
  auto stage_v = [&](int kb) {  // V of block kb into stage (kb + 1) % 2 (group A)
    VDma::load(doff, smem + ((kb + 1) % NS) * Tile::kStageBytes + Tile::kKBytes, vbase, vrow_stride, kb * BK, a.L,
               gw, lane);
  };
  if (grp == 0) {
    VDma::init(doff, vrow_stride, gw, lane);
    stage_v(0);
  } else {
    KDma::init(doff, krow_stride, gw, lane);
    stage_k(0);
    if (n > 1) stage_k(1);
  }
  Frag qf[kDQK / 16];
  {
    const int qload = min(qpos, a.L - 1);
    const char* qrow = (const char*)a.q + (((size_t)b * a.L + qload) * a.Hq + head) * kDQK * 2;
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) qf[kk] = global_q_frag<E>(qrow, kk, half);
    if constexpr (ROPE != kPreRopeNone) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float cs[16];
        rope_load<8>(a.rope, qload, 16 * kk + 8 * half, cs);
        rope_rotate_frag<E>(qf[kk], qf[kk + 2], cs);
      }
    }
  }

  const float c = a.scale_log2;
  const float sink_l2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
  float m = sink_l2;
  float l = a.sink ? 1.f : 0.f;
  f32x16 acc[kDV / 32];
#pragma unroll
  for (int db = 0; db < kDV / 32; ++db) acc[db] = zero16();
  f32x16 s[NKB];
  Frag pf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) pf[ks] = Frag{};

  wait_vm();
  __syncthreads();

  // LDS addresses: the stages' base, and this lane's offsets within a stage for the V^T fragments
  // (transposing reads: row 4 half + (lane % 16) / 4, column 16 ((lane / 16) % 2) + 4 (lane % 4))
  // and the K fragments (row col, column 8 half)
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const uint32_t vt_lane = ((4 * half + ((lane & 15) >> 2)) * Tile::kVStride + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  const uint32_t k_lane = (col * Tile::kKStride + 8 * half) * 2;

  // M_k: the previous block's PV products (PV), then this block's scores (QK). With one wave per
  // SIMD issuing MFMAs at a time, nothing else hides the LDS latency of their operands: every
  // operand fragment is read D products ahead of its use.
  auto mphase = [&](int k, auto pv_tag, auto qk_tag) {
    constexpr bool PV = decltype(pv_tag)::value, QK = decltype(qk_tag)::value;
    constexpr int NPV = PV ? 4 * NKS : 0, NM = NPV + (QK ? NKB * (kDQK / 16) : 0), D = MIMO_GA_DEPTH;
    // this lane's addresses in the stage of pair k (V of block k - 1, K of block k); every
    // fragment is then at a constant offset from them (the LDS read's offset field). The empty asm
    // keeps the compiler from re-associating them into one hoisted register per fragment.
    uint32_t vb = lds_base + (k % NS) * Tile::kStageBytes + Tile::kKBytes + vt_lane;
    uint32_t kb = lds_base + (k % NS) * Tile::kStageBytes + k_lane;
    asm volatile("" : "+v"(vb), "+v"(kb));
    auto frag = [&](int i) -> Frag {  // A operand of product i
      if (i < NPV) {
        const int ks = i / 4, db = i % 4;
        const uint32_t a0 = vb + (16 * ks * Tile::kVStride + 32 * db) * 2;
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)a0);
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(uintptr_t)(a0 + 8 * Tile::kVStride * 2));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        s16x8 u;
        u[0] = x[0]; u[1] = x[1]; u[2] = x[2]; u[3] = x[3];
        u[4] = y[0]; u[5] = y[1]; u[6] = y[2]; u[7] = y[3];
        return __builtin_bit_cast(bf16x8, u);
      }
      const int j = i - NPV;  // score product j: key rows 32 (j % NKB), dims 16 (j / NKB)
      const uint32_t a0 = kb + (32 * (j % NKB) * Tile::kKStride + 16 * (j / NKB)) * 2;
      return __builtin_bit_cast(bf16x8, *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)a0);
    };
    Frag buf[D];
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (i < NM) buf[i] = frag(i);
    if constexpr (QK) {
#pragma unroll
      for (int sb = 0; sb < NKB; ++sb) s[sb] = zero16();
    }
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const Frag x = buf[i % D];
      if (i + D < NM) buf[i % D] = frag(i + D);
      if (i < NPV) {
        acc[i % 4] = mma(x, pf[i / 4], acc[i % 4]);
      } else {
        const int j = i - NPV;
        s[j % NKB] = mma(x, qf[j / NKB], s[j % NKB]);
      }
    }
#if MIMO_GA_SGB
    // keep that order: the first D fragments' reads, then one product and the next reads, ...
    GaReadAhead<NPV, NM, D, 0>::emit();
#endif
  };

  // V_k: softmax of block k (masked only for the last block, which holds the diagonal)
  auto vphase = [&](int k, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float bmax = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < NKB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (MASKED) {
          const int key = k * BK + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
          s[sb][r] = key <= qpos ? s[sb][r] : -INFINITY;
        }
        bmax = fmaxf(bmax, s[sb][r]);
      }
    }
    const float mb = halves_max(bmax) * c;
    if (__builtin_amdgcn_ballot_w64(mb > m + kLazyRescale || (m == -INFINITY && mb > m)) != 0) {
      const float m_new = fmaxf(m, mb);
      const float alpha = fast_exp2(m - (m_new == -INFINITY ? 0.f : m_new));
      l *= alpha;
#pragma unroll
      for (int db = 0; db < kDV / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m = m_new;
    }
    const float m_use = (m == -INFINITY) ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int sb = 0; sb < NKB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[sb][r], c, -m_use));
        s[sb][r] = p;
        rs += p;
      }
    }
    l += halves_sum(rs);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) pf[ks] = frag_from_acc<E>(s[ks >> 1], 8 * (ks & 1));
  };

  // barrier that closes a slot
  auto close_slot = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  const std::false_type no{};
  const std::true_type yes{};
  if (grp == 0) {
    mphase(0, no, yes);
    close_slot();                          // slot 0
    for (int k = 0; k + 1 < n; ++k) {
      if (k >= 1) stage_v(k);
      vphase(k, no);
      wait_vm();
      close_slot();                        // slot 2k + 1
      mphase(k + 1, yes, yes);
      close_slot();                        // slot 2k + 2
    }
    if (n > 1) stage_v(n - 1);
    vphase(n - 1, yes);
    wait_vm();
    close_slot();                          // slot 2n - 1
    mphase(n, yes, no);
    close_slot();                          // slot 2n
    close_slot();                          // slot 2n + 1 (idle)
  } else {
    close_slot();                          // slot 0 (idle)
    mphase(0, no, yes);
    close_slot();                          // slot 1
    for (int k = 0; k + 1 < n; ++k) {
      if (k + 2 < n) stage_k(k + 2);
      vphase(k, no);
      wait_vm();
      close_slot();                        // slot 2k + 2
      mphase(k + 1, yes, yes);
      close_slot();                        // slot 2k + 3
    }
    vphase(n - 1, yes);
    close_slot();                          // slot 2n
    mphase(n, yes, no);
    close_slot();                          // slot 2n + 1
  }

  const bool valid = qpos < a.L;
  char* orow = (char*)a.o + (((size_t)b * a.L + min(qpos, a.L - 1)) * a.Hq + head) * kDV * 2;
  store_out_row<E>(orow, acc, 1.f / l, half, valid);
  if (a.lse && half == 0 && valid) a.lse[((size_t)b * a.Hq + head) * a.L + qpos] = (m + fast_log2(l)) * kLn2;
}

// ---------------------------------------------------------------- sliding-window ring kernel

template <int NB, bool ROPE>
__global__ __launch_bounds__(512) void prefill_swa_kernel(const PrefillArgs a) {
  using E = BF16;
  using Tile = PrefillTile<E, 32>;
  constexpr int NW = 8, NT = 512, R = NB + 1;
  // RoPE: three [32][32][2] fp32 (cos, sin) tables after the ring, for tiles t, t + 1, t + 2 (tile
  // t's rows rotate its Q; tile t + 1's rows rotate the diagonal K block staged at the end of tile
  // t; tile t + 2's rows are written at the end of tile t). The prologue's blocks are rotated in
  // place in the ring.
  constexpr int kHalfRot = kRopeDims / 2;
  constexpr int kTblBytes = kQT * kHalfRot * 2 * 4;
  __shared__ __attribute__((aligned(16))) char smem[R * Tile::kStageBytes + (ROPE ? 3 * kTblBytes : 0)];
  poison_lds(smem, sizeof(smem));
  char* tables = smem + R * Tile::kStageBytes;
  auto table_of = [&](int tile) { return tables + (tile % 3) * kTblBytes; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on it

  // workgroup -> (segment, head chunk, KV head, sequence); segments of one (b, g) are adjacent
  int rest = blockIdx.x;
  const int seg = rest % a.n_segments;
  rest /= a.n_segments;
  const int hc = rest % a.n_hchunks;
  rest /= a.n_hchunks;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int head = a.hl.at(g * a.G + hc * NW + wave);

  const int n_tiles = (a.L + kQT - 1) / kQT;
  const int t0 = seg * a.tiles_per_wg;
  const int t1 = min(n_tiles, t0 + a.tiles_per_wg);

  const size_t krow_stride = (size_t)a.Hkv * kDQK * 2;
  const size_t vrow_stride = (size_t)a.Hkv * kDV * 2;
  const size_t qrow_stride = (size_t)a.Hq * kDQK * 2;
  const size_t orow_stride = (size_t)a.Hq * kDV * 2;
  const char* kbase = (const char*)a.k + ((size_t)b * a.L * a.Hkv + g) * kDQK * 2;
  const char* vbase = (const char*)a.v + ((size_t)b * a.L * a.Hkv + g) * kDV * 2;
  const char* qbase = (const char*)a.q + ((size_t)b * a.L * a.Hq + head) * kDQK * 2;
  char* obase = (char*)a.o + ((size_t)b * a.L * a.Hq + head) * kDV * 2;

  const float c = a.scale_log2;
  const float sink_l2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;
  const int W = a.window;

  // ring slot of key block kb (kb >= -NB + 1)
  auto slot = [](int kb) { return (kb + R) % R; };

  // RoPE: rotate, in place, the rotated dims of the K rows of ring slot `sl`; thread tid takes
  // row r = tid / 16 and the pairs (i, i + 32), (i + 1, i + 33) for i = 2 (tid % 16), with the
  // (cos, sin) row `trow` of that key's position (in LDS or in memory)
  auto rotate_block = [&](int sl, const float* trow) {
    const int r = tid / (kHalfRot / 2), i = 2 * (tid % (kHalfRot / 2));
    uint32_t* row = reinterpret_cast<uint32_t*>(smem + sl * Tile::kStageBytes + r * Tile::kKStride * 2);
    uint32_t lo = row[i / 2], hi = row[(i + kHalfRot) / 2];  // bf16 pairs (i, i+1), (i+32, i+33)
    const f32x4 c = *reinterpret_cast<const f32x4*>(trow + i * 2);
    rope_bf16x2(lo, hi, c[0], c[1], c[2], c[3]);  // the arithmetic of the rotation at staging
    row[i / 2] = lo;
    row[(i + kHalfRot) / 2] = hi;
  };
  static_assert(NT == kQT * kHalfRot / 2, "one thread per two pairs of a 32-row block");
  // this thread's 16 bytes of the (cos, sin) rows of positions p0 .. p0 + 31 (clamped into L)
  auto table_chunk = [&](int p0) {
    const int r = tid / 16, q4 = tid % 16;
    return ld16(reinterpret_cast<const char*>(a.rope) + ((size_t)min(p0 + r, a.L - 1) * kHalfRot * 2 + 4 * q4) * 4);
  };
  // RoPE: rotate a tile's Q fragments in registers with that tile's table rows in LDS
  auto rotate_q = [&](bf16x8(&q)[kDQK / 16], int tile) {
    const float* trow = reinterpret_cast<const float*>(table_of(tile)) + col * kHalfRot * 2;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float cs[16];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(trow + (16 * kk + 8 * half) * 2 + 4 * w);
        cs[4 * w] = v[0]; cs[4 * w + 1] = v[1]; cs[4 * w + 2] = v[2]; cs[4 * w + 3] = v[3];
      }
      rope_rotate_frag<E>(q[kk], q[kk + 2], cs);
    }
  };

  // prologue: zero the slots of blocks before position 0 (they are scored, masked, and must hold
  // finite values), then stage the window of tile t0 (blocks t0 - NB + 1 .. t0) and Q of tile t0
  if (t0 < NB - 1) {
    for (int i = tid; i < R * Tile::kStageBytes / 16; i += NT) st16(smem + 16 * i, zero_chunk());
    __syncthreads();
  }
  {
    KVStager<E, NT, 32> pro[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) pro[j].init(krow_stride, vrow_stride, tid);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (t0 - NB + 1 + j >= 0)
        pro[j].load(kbase, vbase, krow_stride, vrow_stride, 32 * (t0 - NB + 1 + j), a.L, tid);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (t0 - NB + 1 + j >= 0) pro[j].store(smem + slot(t0 - NB + 1 + j) * Tile::kStageBytes, tid);
    if constexpr (ROPE) {
      // the window's blocks, rotated with table rows read from memory; rows of tiles t0 and
      // t0 + 1 to LDS
      st16(table_of(t0) + tid * 16, table_chunk(kQT * t0));
      st16(table_of(t0 + 1) + tid * 16, table_chunk(kQT * min(t0 + 1, t1 - 1)));
      wait_all();
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int kb = t0 - NB + 1 + j;
        if (kb >= 0) rotate_block(slot(kb), a.rope + (size_t)min(32 * kb + tid / 16, a.L - 1) * kHalfRot * 2);
      }
    }
  }
  bf16x8 qf[kDQK / 16];
  {
    const char* qrow = qbase + (size_t)min(kQT * t0 + col, a.L - 1) * qrow_stride;
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) qf[kk] = global_q_frag<E>(qrow, kk, half);
  }
  wait_all();
  __syncthreads();

  KVStager<E, NT, 32, ROPE ? kRopeLds : kRopeNone> st;
  st.init(krow_stride, vrow_stride, tid);
  // one tile; the next tile's Q goes to the second register set, fetched before this tile's score
  // MFMAs (Q of tiles t0, t0 + 2, .. lives in qf, of t0 + 1, t0 + 3, .. in qg)
  auto step = [&](const int t, bf16x8(&qc)[kDQK / 16], bf16x8(&qn)[kDQK / 16]) {
    const int p0 = kQT * t;
    // lanes past the end of the sequence stand in for its last row: same Q, same keys, same
    // result, stored to the same place, so no store or load below needs a per-lane condition
    const int qpos = min(p0 + col, a.L - 1);
    const bool has_next = t + 1 < t1;
    int base[NB];  // byte offset of each window block's ring slot
#pragma unroll
    for (int j = 0; j < NB; ++j) base[j] = slot(t - NB + 1 + j) * Tile::kStageBytes;

    // the next tile's diagonal K/V block and Q stream in under this whole tile. The loads are
    // unconditional (on the last tile: this tile's block again, and one shared Q row, unused), so
    // that the compiler's wait counts see one straight-line sequence of loads and stores.
    st.load(kbase, vbase, krow_stride, vrow_stride, 32 * min(t + 1, t1 - 1), a.L, tid);
    const char* qrow_next = has_next ? qbase + (size_t)min(p0 + kQT + col, a.L - 1) * qrow_stride : qbase;
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) qn[kk] = global_q_frag<E>(qrow_next, kk, half);
    __builtin_amdgcn_sched_barrier(0);  // left alone, the scheduler sinks the Q loads below the MFMAs

    // RoPE: this tile's Q is rotated here, where it is first needed (rotating the next tile's Q at
    // the end of this one would hold the output stores until that Q had arrived)
    if constexpr (ROPE) rotate_q(qc, t);

    // scores of the whole window: block j holds keys 32 * (t - NB + 1 + j) ..
    f32x16 s[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) s[j] = zero16();
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) {
#pragma unroll
      for (int j = 0; j < NB; ++j) s[j] = mma(lds_k_frag<E, 32>(smem + base[j], col, kk, half), qc[kk], s[j]);
    }

    float rmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int kb = t - NB + 1 + j;
      // masked: future keys (diagonal block), keys older than the window, keys before 0
      const bool need_mask = (j == NB - 1) || (kb < 0) || (32 * kb <= p0 + kQT - 1 - W);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const int d = qpos - key;
          s[j][r] = (key >= 0 && d >= 0 && d < W) ? s[j][r] : -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) rmax = fmaxf(rmax, s[j][r]);
    }
    const float m = fmaxf(sink_l2, halves_max(rmax) * c);
    const float m_use = (m == -INFINITY) ? 0.f : m;

    // probabilities go straight to bf16 MFMA fragments (half the registers of fp32 scores)
    float l = 0.f;
    bf16x8 pf[NB][2];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[j][r], c, -m_use));
        s[j][r] = p;
        l += p;
      }
      pf[j][0] = frag_from_acc<E>(s[j], 0);
      pf[j][1] = frag_from_acc<E>(s[j], 8);
    }
    l = halves_sum(l) + (a.sink ? fast_exp2(sink_l2 - m_use) : 0.f);

    f32x16 acc[kDV / 32];
#pragma unroll
    for (int db = 0; db < kDV / 32; ++db) acc[db] = zero16();
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < kDV / 32; ++db)
          acc[db] = mma(lds_vt_frag<E, 32>(smem + base[j] + Tile::kKBytes, db, ks, lane), pf[j][ks],
                        acc[db]);

    // RoPE: this thread's share of the table rows of tile t + 2 (written to LDS below), requested
    // only after the PV products are issued: held across the tile, its four registers spilled and
    // the spill store waited for the load
    u32x4 tchunk;
    if constexpr (ROPE) tchunk = table_chunk(kQT * min(t + 2, t1 - 1));

    // ring update first, output stores last: the stores drain under the barrier and the next
    // tile's score MFMAs instead of holding up the loads that reuse their registers
    u32x4 out[8];
    pack_row_bf16(acc, 1.f / l, out);
    if (has_next) {
      st.store(smem + slot(t + 1) * Tile::kStageBytes, tid, ROPE ? table_of(t + 1) : nullptr);
      if constexpr (ROPE) st16(table_of(t + 2) + tid * 16, tchunk);
    }
    store_packed_row_bf16(obase + (size_t)qpos * orow_stride, out, half);
    if (a.lse) a.lse[((size_t)b * a.Hq + head) * a.L + qpos] = (m + fast_log2(l)) * kLn2;
    __syncthreads();
  };
  bf16x8 qg[kDQK / 16];
  for (int t = t0; t < t1; t += 2) {
    step(t, qf, qg);
    if (t + 1 < t1) step(t + 1, qg, qf);
  }
}

// K [B, L, Hkv, 192] -> k_ws with the leading 64 dims of row l rotated by position l: one thread
// per 16-byte chunk; a thread of a chunk in the first 32 dims rotates it together with its
// partner 32 dims on (the same arithmetic as the rotation at staging), chunks past 64 are copied.
template <typename E>
__global__ __launch_bounds__(256) void rope_k_kernel(const PrefillArgs a) {
  constexpr int NCH = kDQK / E::kPerChunk;        // chunks per row
  constexpr int H = kRopeDims / 2 / E::kPerChunk;  // chunks in 32 dims
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)a.B * a.L * a.Hkv * NCH) return;
  const int c = (int)(idx % NCH);
  const long long row = idx / NCH;                 // (b * L + l) * Hkv + g
  const int l = (int)((row / a.Hkv) % a.L);
  const char* src = (const char*)a.k + row * kDQK * E::kBytes;
  char* dst = (char*)a.k_ws + row * kDQK * E::kBytes;
  if (c < H) {
    u32x4 lo = ld16(src + 16 * c), hi = ld16(src + 16 * (c + H));
    float cs[2 * E::kPerChunk];
    rope_load<E::kPerChunk>(a.rope, l, c * E::kPerChunk, cs);
    rope_rotate_chunk<E>(lo, hi, cs);
    st16(dst + 16 * c, lo);
    st16(dst + 16 * (c + H), hi);
  } else if (c >= 2 * H) {
    st16(dst + 16 * c, ld16(src + 16 * c));
  }
}

template <typename E, int NW, int BK>
static hipError_t launch(const PrefillArgs& a, hipStream_t stream) {
  const long long n_wg = (long long)a.n_qblocks * a.B * a.Hkv * a.n_hchunks;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.rope && a.k_ws) {
    // rotate K once into k_ws; the attention then rotates only Q and stages K as without RoPE
    const long long units = (long long)a.B * a.L * a.Hkv * (kDQK / E::kPerChunk);
    hipLaunchKernelGGL(rope_k_kernel<E>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream, a);
    PrefillArgs r = a;
    r.k = a.k_ws;
    hipLaunchKernelGGL((prefill_kernel<E, NW, BK, kPreRopeQ>), dim3((unsigned)n_wg), dim3(NW * 64), 0, stream, r);
  } else if (a.rope) {
    hipLaunchKernelGGL((prefill_kernel<E, NW, BK, kPreRopeQK>), dim3((unsigned)n_wg), dim3(NW * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((prefill_kernel<E, NW, BK, kPreRopeNone>), dim3((unsigned)n_wg), dim3(NW * 64), 0, stream, a);
  }
  return hipGetLastError();
}


// bf16 global attention, 8 query heads per workgroup: the ping-pong kernel (with RoPE only when K
// is rotated once into k_ws beforehand)
static hipError_t launch_global(const PrefillArgs& a, hipStream_t stream) {
  const long long n_wg = (long long)a.n_qblocks * a.B * a.Hkv * a.n_hchunks;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.rope) {
    const long long units = (long long)a.B * a.L * a.Hkv * (kDQK / 8);
    hipLaunchKernelGGL(rope_k_kernel<BF16>, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream, a);
    PrefillArgs r = a;
    r.k = a.k_ws;
    hipLaunchKernelGGL((prefill_global_kernel<kPreRopeQ, MIMO_GA_BK>), dim3((unsigned)n_wg), dim3(512), 0, stream, r);
  } else {
    hipLaunchKernelGGL((prefill_global_kernel<kPreRopeNone, MIMO_GA_BK>), dim3((unsigned)n_wg), dim3(512), 0, stream, a);
  }
  return hipGetLastError();
}

// Segment sizing of the ring kernel: about this many workgroups per compute unit over the grid
// (one: a single generation of long segments; 1, 2, 4, 8, 16 per CU measured 1.276, 1.284, 1.289,
// 1.315, 1.357 ms on the 4 x 32768 workload),
// and never fewer than this many tiles per segment (each segment re-reads a window of halo).
constexpr int kSwaWgPerCu = 1;
constexpr int kSwaMinTiles = 8;

template <int NB>
static hipError_t launch_swa(PrefillArgs a, hipStream_t stream) {
  const int n_tiles = (a.L + kQT - 1) / kQT;
  const long long units = (long long)a.B * a.Hkv * a.n_hchunks;
  // spread the tiles of every (b, g, head chunk) over segments so that about
  // kSwaWgPerCu workgroups per compute unit run in total
  long long segs = (kSwaWgPerCu * 256LL + units - 1) / units;
  segs = segs < 1 ? 1 : segs;
  long long per = (n_tiles + segs - 1) / segs;
  if (per < kSwaMinTiles) per = kSwaMinTiles;
  a.tiles_per_wg = (int)per;
  a.n_segments = (int)((n_tiles + per - 1) / per);
  const long long n_wg = units * a.n_segments;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.rope)
    hipLaunchKernelGGL((prefill_swa_kernel<NB, true>), dim3((unsigned)n_wg), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_swa_kernel<NB, false>), dim3((unsigned)n_wg), dim3(512), 0, stream, a);
  return hipGetLastError();
}

// One thread per (position, pair): the angle and its cosine / sine in fp64, stored as fp32.
__global__ __launch_bounds__(256) void rope_table_kernel(int n_pos, double base, float* table) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)n_pos * (kRopeDims / 2)) return;
  const int p = (int)(idx / (kRopeDims / 2)), i = (int)(idx % (kRopeDims / 2));
  const double ang = (double)p * pow(base, -2.0 * i / kRopeDims);
  double sn, cs;
  sincos(ang, &sn, &cs);
  reinterpret_cast<f32x2*>(table)[idx] = f32x2{(float)cs, (float)sn};
}

hipError_t rope_table_launch(int n_pos, double base, float* table, hipStream_t stream) {
  const long long n = (long long)n_pos * (kRopeDims / 2);
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, n_pos, base, table);
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
  if (!bf16) {
    // fp32 (the small configurations): four-wave workgroups when eight-wave ones would leave
    // compute units idle (1 x 512 rows x 8 KV heads: 128 workgroups of eight waves)
    if ((long long)a.n_qblocks * a.B * a.Hkv * a.n_hchunks < 2 * 256) {
      constexpr int NW4 = 4;
      int hg4 = 1;
      while (hg4 < NW4 && a.G % (hg4 * 2) == 0) hg4 *= 2;
      a.heads_per_wg = hg4;
      a.n_hchunks = a.G / hg4;
      const int rows4 = kQT * (NW4 / hg4);
      a.n_qblocks = (a.L + rows4 - 1) / rows4;
      return launch<F32, NW4, 32>(a, stream);
    }
    return launch<F32, NW, 32>(a, stream);
  }
  if (!global && hg == NW && a.window <= 129) {
    const int nb = (a.window - 1 + 31) / 32 + 1;  // 32-key blocks in a 32-row tile's window
    switch (nb) {
      case 1:
      case 2: return launch_swa<2>(a, stream);
      case 3: return launch_swa<3>(a, stream);
      case 4: return launch_swa<4>(a, stream);
      default: return launch_swa<5>(a, stream);
    }
  }
  if (global && MIMO_GA_PINGPONG && hg == NW && (!a.rope || a.k_ws)) return launch_global(a, stream);
  if (global) return launch<BF16, NW, 64>(a, stream);
  return launch<BF16, NW, 32>(a, stream);
}

size_t prefill_rope_ws_bytes(bool bf16, int B, int L, int Hq, int Hkv, int window) {
  constexpr int NW = 8;
  const int G = Hq / Hkv;
  int hg = 1;
  while (hg < NW && G % (hg * 2) == 0) hg *= 2;
  const int w = window < L ? window : L;
  if (bf16 && w < L && hg == NW && w <= 129) return 0;  // the ring kernel rotates K once per segment
  return (size_t)B * L * Hkv * kDQK * (bf16 ? 2 : 4);
}

}  // namespace mimo
