// Backward kernels: gradients of sink-seeded sliding-window / causal attention on gfx950 MFMA.
//
// Operation: the gradient of the prefill (MiMo-V2-Flash Technical Report review (xllm-io), §3.1
// and §3.2; MiMo series notes (plmsmile), MiMo-V2-Flash > Learnable Attention Sink: the sink is a
// learned per-head logit in the softmax denominator with no value vector, so training also needs
// its gradient). With the forward's lse (sink included), for query row i and visible key j:
//   P_ij = exp(s_ij - lse_i),  D_i = <dO_i, O_i>,  dS_ij = P_ij (<dO_i, v_j> - D_i)
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i
//   d s_h = -sum_i exp(s_h - lse_i) D_i
// (dK and dV also sum over the query heads of the KV head, and d s_h over the batch).
//
// Three kernels on the caller's stream, no atomics (every output element has one writer, so the
// results do not depend on scheduling):
// bwd_dq_kernel (query-major, the forward's streaming structure): a wave owns one query head and
//   32 query rows (one per MFMA column). It forms D for its rows from dO and O, writes it to the
//   workspace together with its rows' share of the sink gradient, then streams the K/V blocks of
//   the window through LDS: S^T = K Q^T, P^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
// bwd_dkdv_kernel (key-major): a wave owns 32 keys, one per MFMA column, whose K and V rows stay
//   in registers as MFMA operands. The workgroup walks (query head of the group, 32-row query tile)
//   steps; each step's Q, dO, lse and D rows are staged through LDS (double-buffered) and shared by
//   every wave: S = Q K^T, P, dP = dO V^T, dS; dV^T += dO^T P and dK^T += Q^T dS take P and dS
//   straight from the accumulators.
// bwd_sink_kernel: sums the per-tile sink partials of each head in a fixed order.
#include <type_traits>

#include "tiles.hpp"

namespace mimo {

template <typename E>
__device__ __forceinline__ void frag_to_f32(const typename E::Frag& f, float (&x)[8]) {
  if constexpr (E::kBytes == 2) {
    const u32x4 u = __builtin_bit_cast(u32x4, f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = __uint_as_float(u[w] << 16);
      x[2 * w + 1] = __uint_as_float(u[w] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = f[e];
  }
}

// ------------------------------------------------------------------------------------- dQ kernel

template <typename E, int NW, int BK>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(const BackwardArgs a) {
  using Tile = PrefillTile<E, BK, kVRows>;
  using Frag = typename E::Frag;
  constexpr int NT = NW * 64;
  constexpr int NSB = BK / 32;
  // bf16 blocks go global -> LDS directly (no staging registers), fp32 through registers
  constexpr bool kDMA = E::kBytes == 2;
  // bf16: a workgroup whose key blocks fit kAllStages stages (every sliding-window tile) fetches
  // them all at the start and then runs them without waits or barriers; longer ranges (global
  // layers) rotate two stages. (Two stages for all made each workgroup wait for a block's round
  // trip five times after its prologue.)
  constexpr int kAllStages = kDMA ? 6 : 2;
  __shared__ __attribute__((aligned(16))) char smem[kAllStages * Tile::kStageBytes];
  poison_lds(smem, sizeof(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // heaviest query blocks (latest positions) first
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
  const int p0 = P0 + kQT * (wave / HG);
  const int qpos = p0 + col;
  const bool valid = qpos < a.L;
  const int qload = min(qpos, a.L - 1);

  const size_t krow_stride = (size_t)a.Hkv * kDQK * E::kBytes;
  const size_t vrow_stride = (size_t)a.Hkv * kDV * E::kBytes;
  const char* kbase = (const char*)a.k + ((size_t)b * a.L * a.Hkv + g) * kDQK * E::kBytes;
  const char* vbase = (const char*)a.v + ((size_t)b * a.L * a.Hkv + g) * kDV * E::kBytes;

  // Q fragments (B operand of S^T = K Q^T) and dO fragments (B operand of dP^T = V dO^T)
  const size_t row = ((size_t)b * a.L + qload) * a.Hq + head;
  Frag qf[kDQK / 16], df[kDV / 16];
  {
    const char* qrow = (const char*)a.q + row * kDQK * E::kBytes;
    const char* drow = (const char*)a.d_o + row * kDV * E::kBytes;
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) qf[kk] = global_q_frag<E>(qrow, kk, half);
#pragma unroll
    for (int kk = 0; kk < kDV / 16; ++kk) df[kk] = global_q_frag<E>(drow, kk, half);
  }
  const float c = a.scale_log2;
  f32x16 acc[kDQK / 32];
#pragma unroll
  for (int t = 0; t < kDQK / 32; ++t) acc[t] = zero16();

  // the K/V blocks are requested before D is formed, so their latency overlaps that of O
  const int K0 = max(0, P0 - a.window + 1);
  const int kstart = (K0 / BK) * BK;
  const int nblk = (P1 - kstart + BK - 1) / BK;
  const bool all_blocks = kDMA && nblk <= kAllStages;  // uniform

  KVStager<E, NT, BK, kRopeNone, kVRows> st;
  KVStagerDMA<NW, BK, kVRows> dma;
  if constexpr (kDMA) {
    dma.init(krow_stride, vrow_stride, wave, lane);
    if (all_blocks) {
      for (int ib = 0; ib < nblk; ++ib)
        dma.load(smem + ib * Tile::kStageBytes, kbase, vbase, krow_stride, vrow_stride, kstart + ib * BK, a.L,
                 wave, lane);
    } else {
      dma.load(smem, kbase, vbase, krow_stride, vrow_stride, kstart, a.L, wave, lane);
    }
  } else {
    st.init(krow_stride, vrow_stride, tid);
    st.load(kbase, vbase, krow_stride, vrow_stride, kstart, a.L, tid);
    st.store(smem, tid);
    wait_all();
  }
  // D = <dO, O> of this row; each wave half holds 64 of the 128 elements
  float D;
  {
    const char* orow = (const char*)a.o + row * kDV * E::kBytes;
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < kDV / 16; ++kk) {
      float x[8], y[8];
      frag_to_f32<E>(df[kk], x);
      frag_to_f32<E>(global_q_frag<E>(orow, kk, half), y);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf(x[e], y[e], part);
    }
    D = halves_sum(part);
  }
  const size_t lrow = ((size_t)b * a.Hq + head) * a.L + qload;
  const float lse2 = a.lse[lrow] * kLog2e;
  if (half == 0 && valid) a.D[lrow] = D;
  if (a.sink_part && p0 < a.L) {
    // this tile's share of d s_h: -sum_i exp(s_h - lse_i) D_i (the sign is applied at the end)
    float t = (half == 0 && valid) ? fast_exp2(a.sink[head] * kLog2e - lse2) * D : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
    if (lane == 0) a.sink_part[((size_t)head * a.B + b) * a.n_qtiles + p0 / kQT] = t;
  }
  if constexpr (kDMA) wait_vm();  // this wave's K/V fetches have landed
  __syncthreads();

  // One block; MASKED is a compile-time copy, the mask-free one serves blocks that every query of
  // this wave's tile sees in full (see the prefill kernel: waves may differ in the range, all run
  // every block with the same stage loads, stores and barriers).
  auto block = [&](int ib, auto masked_tag, auto all_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool ALL = decltype(all_tag)::value;  // every block already in its own stage
    const int key0 = kstart + ib * BK;
    if (!ALL && ib + 1 < nblk) {
      if constexpr (kDMA)
        dma.load(smem + ((ib + 1) & 1) * Tile::kStageBytes, kbase, vbase, krow_stride, vrow_stride, key0 + BK,
                 a.L, wave, lane);
      else
        st.load(kbase, vbase, krow_stride, vrow_stride, key0 + BK, a.L, tid);
    }

    const bool skip = MASKED && ((key0 > p0 + kQT - 1) || (key0 + BK - 1 < p0 - a.window + 1) || (p0 >= a.L));
    if (!skip) {
      const char* sk = smem + (ALL ? ib : (ib & 1)) * Tile::kStageBytes;
      const char* sv = sk + Tile::kKBytes;

      f32x16 s[NSB], dp[NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) s[sb] = dp[sb] = zero16();
#pragma unroll
      for (int kk = 0; kk < kDQK / 16; ++kk)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
          s[sb] = mma(lds_row_frag<E>(sk, Tile::kKStride, 32 * sb + col, kk, half), qf[kk], s[sb]);
#pragma unroll
      for (int kk = 0; kk < kDV / 16; ++kk)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
          dp[sb] = mma(lds_row_frag<E>(sv, Tile::kVStride, 32 * sb + col, kk, half), df[kk], dp[sb]);

      // dS^T = P^T (dP^T - D), P^T = exp(S^T * scale - lse), zero where masked
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[sb][r], c, -lse2));
          if constexpr (MASKED) {
            const int key = key0 + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
            const int d = qpos - key;
            p = (d >= 0 && d < a.window) ? p : 0.f;
          }
          s[sb][r] = p * (dp[sb][r] - D);
        }
      }
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const Frag dsf = frag_from_acc<E>(s[ks >> 1], 8 * (ks & 1));
#pragma unroll
        for (int t = 0; t < kDQK / 32; ++t)
          acc[t] = mma(lds_t_frag<E>(sk, Tile::kKStride, t, ks, lane), dsf, acc[t]);
      }
    }

    if constexpr (!ALL) {
      if constexpr (kDMA) {
        wait_vm();  // this wave's loads of the next stage have landed
      } else {
        if (ib + 1 < nblk) st.store(smem + ((ib + 1) & 1) * Tile::kStageBytes, tid);
      }
      __syncthreads();
    }
  };

  // blocks [ib_a, ib_b): every key at or before the tile's first row and within the window of
  // its last one
  int ib_a = nblk, ib_b = nblk;
  if (p0 < a.L) {
    const int hi_num = p0 - (BK - 1) - kstart;
    const int hi = hi_num >= 0 ? hi_num / BK + 1 : 0;
    const long long lo_num = (long long)p0 + kQT - a.window - kstart;
    const int lo = lo_num <= 0 ? 0 : (int)min<long long>((lo_num + BK - 1) / BK, nblk);
    ib_a = min(lo, nblk);
    ib_b = min(max(hi, ib_a), nblk);
  }
  ib_a = __builtin_amdgcn_readfirstlane(ib_a);
  ib_b = __builtin_amdgcn_readfirstlane(ib_b);
  if (all_blocks) {
    for (int ib = 0; ib < nblk;) {
      const int stop = ib < ib_a ? ib_a : (ib < ib_b ? ib : nblk);
      for (; ib < stop; ++ib) block(ib, std::true_type{}, std::true_type{});
      for (; ib < ib_b; ++ib) block(ib, std::false_type{}, std::true_type{});
    }
  } else {
    for (int ib = 0; ib < nblk;) {
      const int stop = ib < ib_a ? ib_a : (ib < ib_b ? ib : nblk);
      for (; ib < stop; ++ib) block(ib, std::true_type{}, std::false_type{});
      for (; ib < ib_b; ++ib) block(ib, std::false_type{}, std::false_type{});
    }
  }

  char* dqrow = (char*)a.dq + row * kDQK * E::kBytes;
  store_out_row<E>(dqrow, acc, a.scale, half, valid);
}

// ------------------------------------------------------------ sliding-window dQ: ping-pong walk

// bf16, window <= 129, eight query heads per workgroup (wave w = head w of the chunk). The dQ
// kernel's math on a walk over a segment of consecutive 32-row tiles of one (b, g, head chunk):
// the window of tile t is the 32-key blocks t - 4 .. t, held in an LDS ring (block kb in slot
// kb mod kDqRing), so each K/V row is fetched once per segment. The two halves of the workgroup
// run one phase apart: waves 0-3 take tile t's rows (Q, dO and O: D, the sink partial) and fetch
// K of block t into the ring while waves 4-7 compute tile t - 1, then waves 0-3 compute tile t
// while waves 4-7 take tile t's rows and fetch V of block t + 1; a barrier closes every phase. Each SIMD holds one wave of
// each half, so one of its waves computes while the other waits for memory, and the rows of half
// the heads are always in flight. (The one-tile-per-workgroup kernel above runs one workgroup per
// compute unit, which loads and then computes: per-workgroup timestamps on the 4 x 32768 sliding
// window layer showed 13.6 us of waiting for rows and K/V blocks, then 6.5 us of products and 2 us
// of stores, with most compute units in the same phase at once.)
// Ring slots: block t's slot held block t - 6, last read when waves 4-7 computed tile t - 2; V of
// block t arrives one phase after that (waves 4-7, rows of tile t - 1), K one phase later still
// (waves 0-3, rows of tile t), and both before waves 0-3 compute tile t.
constexpr int kDqRing = 6;

// SHORT: windows shorter than 128 keys, where the middle blocks of a window are masked as well
template <bool SHORT>
__global__ __launch_bounds__(512) void bwd_dq_swa_kernel(const BackwardArgs a) {
  using E = BF16;
  using Tile = PrefillTile<E, 32, kVRows>;
  using Frag = bf16x8;
  __shared__ __attribute__((aligned(16))) char smem[kDqRing * Tile::kStageBytes];
  poison_lds(smem, sizeof(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: takes tile t's rows while 1 computes tile t - 1
  const int gw = wave & 3;

  // workgroup -> (segment, head chunk, KV head, sequence); segments of one (b, g) are adjacent
  int rest = blockIdx.x;
  const int seg = rest % a.n_segments;
  rest /= a.n_segments;
  const int hc = rest % a.n_hchunks;
  rest /= a.n_hchunks;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int head = a.hl.at(g * a.G + hc * 8 + wave);
  const int t0 = seg * a.tiles_per_wg;
  const int t1 = min(a.n_qtiles, t0 + a.tiles_per_wg);

  const size_t krow_stride = (size_t)a.Hkv * kDQK * 2;
  const size_t vrow_stride = (size_t)a.Hkv * kDV * 2;
  const char* kbase = (const char*)a.k + ((size_t)b * a.L * a.Hkv + g) * kDQK * 2;
  const char* vbase = (const char*)a.v + ((size_t)b * a.L * a.Hkv + g) * kDV * 2;
  const float c = a.scale_log2;
  const int W = a.window;
  // ring slot of block kb (kb >= -4)
  auto ring = [&](int kb) { return smem + ((kb + kDqRing) % kDqRing) * Tile::kStageBytes; };

  // the first tiles of a sequence also score the blocks before key 0 (masked): their slots must
  // hold finite values
  if (t0 < 4) {
    for (int i = tid; i < kDqRing * Tile::kStageBytes / 16; i += 512) st16(smem + 16 * i, zero_chunk());
    __syncthreads();
  }
  // waves 0-3 stage the K/V blocks: first the window of tile t0 before its diagonal block
  // Staging global -> LDS by one half (four waves): waves 0-3 fetch K of block t in their rows
  // phase of tile t, waves 4-7 V of block t + 1 in theirs, so both halves' rows phases carry a
  // share of the ring traffic. (The stagers' per-lane offsets are recomputed for every block from
  // an opaque copy of the lane index: held across the walk, they took registers the compute phase
  // needs.)
  using KDma = RowsDMA<4, 32, Tile::kKStride * 2 / 16, kDQK / 8>;
  using VDma = RowsDMA<4, 32, Tile::kVStride * 2 / 16, kDV / 8>;
  static_assert(KDma::kChunks * 16 == Tile::kKBytes && VDma::kChunks * 16 == Tile::kVBytes, "regions tile the stage");
  auto stage_k = [&](int kb) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    uint32_t off[KDma::kPer];
    KDma::init(off, krow_stride, gw, ln);
    KDma::load(off, ring(kb), kbase, krow_stride, 32 * kb, a.L, gw, ln);
  };
  auto stage_v = [&](int kb) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    uint32_t off[VDma::kPer];
    VDma::init(off, vrow_stride, gw, ln);
    VDma::load(off, ring(kb) + Tile::kKBytes, vbase, vrow_stride, 32 * kb, a.L, gw, ln);
  };
  // before the walk (waves 0-3): the window of tile t0 before its diagonal block, and V of t0
  if (grp == 0) {
    for (int kb = max(0, t0 - 4); kb < t0; ++kb) {
      stage_k(kb);
      stage_v(kb);
    }
    stage_v(t0);
  }

  // rows phase of tile t: Q and dO fragments (B operands of S^T = K Q^T and dP^T = V dO^T), D of
  // the rows, their share of the sink gradient; waves 0-3 also fetch K/V block t. Ends when every
  // load of this wave has landed.
  Frag qf[kDQK / 16], df[kDV / 16];
  float D = 0.f, lse2 = 0.f;
  auto rows = [&](int t) __attribute__((always_inline)) {
    // the row addresses come from an opaque copy of the lane index: hoisted out of the walk, the
    // per-lane pointers were spilled and reloaded between the batches of fetches (each reload
    // waiting for every fetch before it; no change in time measured, 60 -> 36 B of scratch)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lcol = ln & 31, lhalf = ln >> 5;
    const int qpos = kQT * t + lcol;
    const bool valid = qpos < a.L;
    const size_t row = ((size_t)b * a.L + min(qpos, a.L - 1)) * a.Hq + head;
    const char* qrow = (const char*)a.q + row * kDQK * 2;
    const char* drow = (const char*)a.d_o + row * kDV * 2;
    const char* orow = (const char*)a.o + row * kDV * 2;
    const size_t lrow = ((size_t)b * a.Hq + head) * a.L + min(qpos, a.L - 1);
    // dO, O and lse first: D and the sink partial are formed while Q and the ring block arrive
    // (requested after Q, they held D back until everything had landed: 5.46 -> 5.37 ms)
    Frag of[kDV / 16];
#pragma unroll
    for (int kk = 0; kk < kDV / 16; ++kk) df[kk] = global_q_frag<E>(drow, kk, lhalf);
#pragma unroll
    for (int kk = 0; kk < kDV / 16; ++kk) of[kk] = global_q_frag<E>(orow, kk, lhalf);
    lse2 = a.lse[lrow] * kLog2e;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) qf[kk] = global_q_frag<E>(qrow, kk, lhalf);
    if (grp == 0)
      stage_k(t);
    else if (t + 1 < t1)
      stage_v(t + 1);
    __builtin_amdgcn_sched_barrier(0);
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < kDV / 16; ++kk) {
      float x[8], y[8];
      frag_to_f32<E>(df[kk], x);
      frag_to_f32<E>(of[kk], y);
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf(x[e], y[e], part);
    }
    D = halves_sum(part);
    if (lhalf == 0 && valid) a.D[lrow] = D;
    if (a.sink_part) {
      // this tile's share of d s_h: -sum_i exp(s_h - lse_i) D_i (the sign is applied at the end)
      float sp = (lhalf == 0 && valid) ? fast_exp2(a.sink[head] * kLog2e - lse2) * D : 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sp += __shfl_xor(sp, off);
      if (lane == 0) a.sink_part[((size_t)head * a.B + b) * a.n_qtiles + t] = sp;
    }
    wait_vm();
  };

  // (the phases are forced inline: called from two runs, the compiler made them functions with a
  // stack frame)
  // compute phase of tile t: blocks t - 4 .. t. The first and the last are masked; the middle
  // ones too (ALL) for the first tiles of a sequence (blocks before key 0) and short windows. The
  // choice is made per run of tiles: inside a tile, a branch between masked and mask-free copies
  // made the compiler spill the accumulators.
  auto compute = [&](int t, auto all_tag) __attribute__((always_inline)) {
    constexpr bool ALL = decltype(all_tag)::value;
    const int qpos = kQT * t + col;
    f32x16 acc[kDQK / 32];
#pragma unroll
    for (int i = 0; i < kDQK / 32; ++i) acc[i] = zero16();
    auto block = [&](int kb, auto masked_tag) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      const char* sk = ring(kb);
      const char* sv = sk + Tile::kKBytes;
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int kk = 0; kk < kDQK / 16; ++kk) s = mma(lds_row_frag<E>(sk, Tile::kKStride, col, kk, half), qf[kk], s);
#pragma unroll
      for (int kk = 0; kk < kDV / 16; ++kk) dp = mma(lds_row_frag<E>(sv, Tile::kVStride, col, kk, half), df[kk], dp);
      // dS^T = P^T (dP^T - D), P^T = exp(S^T * scale - lse), zero where masked (keys before 0
      // read zeroed slots: finite, and masked here)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
        if constexpr (MASKED) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const int d = qpos - key;
          p = (key >= 0 && d >= 0 && d < W) ? p : 0.f;
        }
        s[r] = p * (dp[r] - D);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const Frag dsf = frag_from_acc<E>(s, 8 * ks);
#pragma unroll
        for (int i = 0; i < kDQK / 32; ++i) acc[i] = mma(lds_t_frag<E>(sk, Tile::kKStride, i, ks, lane), dsf, acc[i]);
      }
      __builtin_amdgcn_sched_barrier(0);  // one block at a time
    };
    block(t - 4, std::true_type{});
#pragma unroll
    for (int j = 1; j < 4; ++j) block(t - 4 + j, std::integral_constant<bool, ALL>{});
    block(t, std::true_type{});
    const size_t row = ((size_t)b * a.L + min(qpos, a.L - 1)) * a.Hq + head;
    store_out_row<E>((char*)a.dq + row * kDQK * 2, acc, a.scale, half, qpos < a.L);
  };

  auto close_phase = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  // tiles [ta, tb): rows phase, then compute phase, each closed by a barrier; waves 4-7 start one
  // phase late and waves 0-3 end with an idle phase, so both halves pass the same barriers
  auto run = [&](int ta, int tb, auto all_tag) __attribute__((always_inline)) {
    for (int t = ta; t < tb; ++t) {
      rows(t);
      close_phase();
      compute(t, all_tag);
      close_phase();
    }
  };
  if (grp == 1) close_phase();
  const int tm = SHORT ? t1 : min(t1, max(t0, 4));  // tiles whose window starts before key 0
  run(t0, tm, std::true_type{});
  if constexpr (!SHORT) run(tm, t1, std::false_type{});
  if (grp == 0) close_phase();
}

// ---------------------------------------------------------------------------------- dK/dV kernel

// LDS stage of one step: Q rows [32][kQS], dO rows [32][kOS], then lse * log2(e) [32] and D [32].
// Row strides are padded so that both the 16-byte row reads and the transposing reads of the MFMA
// operands spread over the banks.
template <typename E>
struct DkdvStage {
  static constexpr int kQS = kDQK + 16 / E::kBytes;
  static constexpr int kOS = E::kBytes == 2 ? kDV + 24 : kDV + 4;
  static constexpr int kQBytes = kQT * kQS * E::kBytes;
  static constexpr int kOBytes = kQT * kOS * E::kBytes;
  static constexpr int kBytes = kQBytes + kOBytes + 2 * kQT * 4;
  static_assert(kQBytes % 16 == 0 && kOBytes % 16 == 0, "16-byte aligned rows");
};

// dK/dV: windows up to this many keys run two-wave workgroups (see the launcher); the group-phase
// tile order (see the kernel) applies while a key block sees at most kDkdvMaxGroups tile groups.
constexpr int kDkdvShortWindow = 256;
constexpr int kDkdvMaxGroups = 8;

template <typename E, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(const BackwardArgs a) {
  using Frag = typename E::Frag;
  using St = DkdvStage<E>;
  constexpr int NT = NW * 64;
  static_assert(NT == 128 || NT == 256, "staging: 8 threads per staged row, 1 or 2 rows each");
  constexpr int RPT = 256 / NT;                   // staged rows per thread
  constexpr int QPT = kDQK * E::kBytes / 16 / 8;  // 16-byte Q chunks per thread and row
  constexpr int OPT = kDV * E::kBytes / 16 / 8;   // 16-byte dO chunks per thread and row
  __shared__ __attribute__((aligned(16))) char smem[2 * St::kBytes];
  poison_lds(smem, sizeof(smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // key blocks in ascending order: under causal attention the first ones see the most queries.
  // Paired (global layers): workgroup p takes key block p, walking its query tiles from the last
  // down, then key block n - 1 - p, walking its tiles from the first up. Every workgroup then has
  // the same number of tiles (a generation starts and ends together), and at any moment the first
  // walks of all running workgroups are on one tile and their second walks on another, so they
  // share the Q / dO rows through L2. (Unpaired, a workgroup started when an earlier one finished
  // walked out of phase with the rest and fetched its rows alone: 30 GB per 32768-row global
  // launch.)
  const int pk = (int)(blockIdx.x / (a.B * a.Hkv));
  const int rest = blockIdx.x % (a.B * a.Hkv);
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;
  constexpr bool kPairable = NW == 4 && E::kBytes == 2;  // the launcher pairs only these
  const int n_items = kPairable && a.kv_pairs && a.n_kblocks - 1 - pk != pk ? 2 : 1;
  for (int item = 0; item < n_items; ++item) {
  const bool asc = item == 1;
  const int kb = asc ? a.n_kblocks - 1 - pk : pk;
  if (item == 1) __syncthreads();  // every wave is done with the stages of the first walk
  const int kb0 = kb * 32 * NW;
  const int kw0 = kb0 + 32 * wave;  // this wave's first key
  const int kpos = kw0 + col;       // this lane's key
  const int kload = min(kpos, a.L - 1);

  // K and V rows of this lane's key as MFMA B operands (lane = key column)
  const size_t krow = ((size_t)b * a.L + kload) * a.Hkv + g;
  Frag kf[kDQK / 16], vf[kDV / 16];
  {
    const char* kr = (const char*)a.k + krow * kDQK * E::kBytes;
    const char* vr = (const char*)a.v + krow * kDV * E::kBytes;
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) kf[kk] = global_q_frag<E>(kr, kk, half);
#pragma unroll
    for (int kk = 0; kk < kDV / 16; ++kk) vf[kk] = global_q_frag<E>(vr, kk, half);
  }

  // query tiles that see any key of the block
  const int last_q = min(a.L - 1, kb0 + 32 * NW - 1 + a.window - 1);
  const int qt0 = kb0 / kQT;
  const int ntiles = last_q / kQT - qt0 + 1;
  // Step order: tile-major from the last query tile down, every head of a tile in turn. All
  // workgroups start at the last tile of the sequence, so the ones running together read the
  // same Q / dO rows at about the same time and share them through L2 (head-major order made
  // each workgroup walk its own tiles and re-read Q / dO from HBM).
  //
  // Short windows: the tiles form groups of GS = 32 NW / kQT (the rows of one key block); block kb
  // sees groups kb .. kb + ng - 1 and shares each with the ng - 1 blocks beside it. In one
  // descending order the sharers reach a group at different moments and each fetches it from
  // beyond L2. Instead every block walks its groups in the order of m mod ng (each group's tiles
  // descending), so the ng blocks that share group m, dispatched together, read its tiles in the
  // same steps. Blocks at the end of the sequence also walk the tiles past L (masked rows, clamped
  // loads), which keeps their phases aligned with their neighbours'. Interior (mask-free) tiles do
  // not exist for such windows.
  const int qt_last = last_q / kQT;
  constexpr int GS = 32 * NW / kQT;
  const int ng = (kb0 + 32 * NW - 1 + a.window - 1) / kQT / GS - kb + 1;  // window <= L
  const bool alt = !a.kv_pairs && ng <= kDkdvMaxGroups;
  const int kbm = kb % ng;
  const int nsteps = a.G * (alt ? ng * GS : ntiles);
  auto step_head = [&](int step) { return step % a.G; };
  auto step_row = [&](int step) {
    const int t = step / a.G;
    if (!alt) return (asc ? qt0 + t : qt_last - t) * kQT;
    const int ph = t / GS - kbm;
    const int m = kb + (ph < 0 ? ph + ng : ph);
    return (m * GS + GS - 1 - t % GS) * kQT;
  };

  // staging: thread tid moves rows tid / 8 + NT / 8 * r (r < RPT) of the step's Q and dO tiles;
  // threads 0..63 also move lse (rows 0..31) and D (rows 32..63 -> D of row tid - 32)
  const int srow = tid >> 3, spart = tid & 7;
  const size_t qrow_stride = (size_t)a.Hq * kDQK * E::kBytes;
  const size_t orow_stride = (size_t)a.Hq * kDV * E::kBytes;
  struct Staged {
    u32x4 q[RPT][QPT], o[RPT][OPT];
    float l;
  };
  auto load_step = [&](int step, Staged& r) {
    const int j = step_head(step);
    const int q0 = step_row(step);
    const int head = a.hl.at(g * a.G + j);
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int qrow = min(q0 + srow + NT / 8 * rr, a.L - 1);
      const char* qp = (const char*)a.q + ((size_t)b * a.L + qrow) * qrow_stride + (size_t)head * kDQK * E::kBytes;
      const char* op = (const char*)a.d_o + ((size_t)b * a.L + qrow) * orow_stride + (size_t)head * kDV * E::kBytes;
#pragma unroll
      for (int i = 0; i < QPT; ++i) r.q[rr][i] = ld16(qp + 16 * (spart * QPT + i));
#pragma unroll
      for (int i = 0; i < OPT; ++i) r.o[rr][i] = ld16(op + 16 * (spart * OPT + i));
    }
    {  // every thread loads (threads past 64 re-read a D entry): no branch and no use of the
       // value before store_step, so nothing waits for this load here
      const int rr = min(q0 + (tid & 31), a.L - 1);
      const size_t li = ((size_t)b * a.Hq + head) * a.L + rr;
      r.l = (tid < kQT ? a.lse : a.D)[li];
    }
  };
  auto store_step = [&](char* stage, const Staged& r) {
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int row = srow + NT / 8 * rr;
      char* sq = stage + (row * St::kQS + spart * QPT * (16 / E::kBytes)) * E::kBytes;
      char* so = stage + St::kQBytes + (row * St::kOS + spart * OPT * (16 / E::kBytes)) * E::kBytes;
#pragma unroll
      for (int i = 0; i < QPT; ++i) st16(sq + 16 * i, r.q[rr][i]);
#pragma unroll
      for (int i = 0; i < OPT; ++i) st16(so + 16 * i, r.o[rr][i]);
    }
    if (tid < 2 * kQT)
      reinterpret_cast<float*>(stage + St::kQBytes + St::kOBytes)[tid] = tid < kQT ? r.l * kLog2e : r.l;
  };

  const float c = a.scale_log2;
  Staged ra;
  load_step(0, ra);
  store_step(smem, ra);
  wait_all();
  __syncthreads();

  f32x16 acck[kDQK / 32], accv[kDV / 32];
  // Operand reads go through one per-lane base pointer per step plus compile-time offsets, which
  // become the LDS instructions' immediate offsets (written as lane offset + constant, the
  // compiler kept one hoisted address per read and added the stage to each of them every step).
  const int row_lane = (col * St::kQS + 8 * half) * E::kBytes;                     // Q row reads
  const int orow_lane = St::kQBytes + (col * St::kOS + 8 * half) * E::kBytes;      // dO row reads
  const int tr_row = 4 * half + ((lane & 15) >> 2), tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int qtr_lane = (tr_row * St::kQS + tr_col) * E::kBytes;                    // Q^T reads
  const int otr_lane = St::kQBytes + (tr_row * St::kOS + tr_col) * E::kBytes;      // dO^T reads
  auto row_frag = [&](const char* p) -> Frag {
    if constexpr (E::kBytes == 2) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
    } else {
      const f32x4 x = *reinterpret_cast<const f32x4*>(p);
      const f32x4 y = *reinterpret_cast<const f32x4*>(p + 16);
      Frag f;
      f[0] = x[0]; f[1] = x[1]; f[2] = x[2]; f[3] = x[3];
      f[4] = y[0]; f[5] = y[1]; f[6] = y[2]; f[7] = y[3];
      return f;
    }
  };
  // bf16: rows 16 ks + 4 half + 0..3 and + 8 of columns 32 t + lane % 32, through the
  // transposing read (see vt_frag_tr); p already holds the lane's part of the address
  auto tr_frag = [&](const char* p, int stride) -> bf16x8 {
    const s16x4 x = lds_read_tr16(p);
    const s16x4 y = lds_read_tr16(p + 8 * stride * 2);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 u;
    u[0] = x[0]; u[1] = x[1]; u[2] = x[2]; u[3] = x[3];
    u[4] = y[0]; u[5] = y[1]; u[6] = y[2]; u[7] = y[3];
    return __builtin_bit_cast(bf16x8, u);
  };
  // One step: S = Q K^T and dP = dO V^T for the staged (head, query tile), then P, dS and the
  // dV / dK contributions. A wave none of whose keys the tile sees computes with p = 0 (no
  // branch: branches inside the loop make the compiler move the accumulators between register
  // files on every step).
  // (forced inline: the fp32 instance was otherwise called with a 2.3 KB stack frame)
  auto compute = [&](int step, bool first, auto masked) __attribute__((always_inline)) {
    const int q0 = step_row(step);
    const bool active = (kw0 < a.L) && (q0 + kQT - 1 >= kw0) && (q0 <= kw0 + 31 + a.window - 1);
    const unsigned wlim = active ? (unsigned)a.window : 0u;  // no visible key when inactive
    const char* stage = smem + (step & 1) * St::kBytes;
    const float* sl = reinterpret_cast<const float*>(stage + St::kQBytes + St::kOBytes);

    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int kk = 0; kk < kDQK / 16; ++kk) s = mma(row_frag(stage + row_lane + 16 * kk * E::kBytes), kf[kk], s);
#pragma unroll
    for (int kk = 0; kk < kDV / 16; ++kk) dp = mma(row_frag(stage + orow_lane + 16 * kk * E::kBytes), vf[kk], dp);

    // register r holds query row 8 (r / 4) + 4 half + r % 4 of the tile
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + 8 * gq + 4 * half);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(sl + kQT + 8 * gq + 4 * half);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * gq + i;
        const int qp = q0 + 8 * gq + 4 * half + i;
        float p;
        if constexpr (decltype(masked)::value) {
          const bool vis = (unsigned)(qp - kpos) < wlim && qp < a.L;
          // select the exponent, not the result: exp2(-inf) = 0 needs no branch
          p = fast_exp2(vis ? __builtin_fmaf(s[r], c, -l4[i]) : -INFINITY);
        } else {
          p = fast_exp2(__builtin_fmaf(s[r], c, -l4[i]));
        }
        s[r] = p;
        dp[r] = p * (dp[r] - d4[i]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < kQT / 16; ++ks) {
      const Frag pf = frag_from_acc<E>(s, 8 * ks);
#pragma unroll
      for (int t = 0; t < kDV / 32; ++t) {
        Frag f;
        if constexpr (E::kBytes == 2)
          f = tr_frag(stage + otr_lane + (16 * ks * St::kOS + 32 * t) * 2, St::kOS);
        else
          f = lds_t_frag<E>(stage + St::kQBytes, St::kOS, t, ks, lane);
        accv[t] = mma(f, pf, (first && ks == 0) ? zero16() : accv[t]);
      }
      const Frag dsf = frag_from_acc<E>(dp, 8 * ks);
#pragma unroll
      for (int t = 0; t < kDQK / 32; ++t) {
        Frag f;
        if constexpr (E::kBytes == 2)
          f = tr_frag(stage + qtr_lane + (16 * ks * St::kQS + 32 * t) * 2, St::kQS);
        else
          f = lds_t_frag<E>(stage, St::kQS, t, ks, lane);
        acck[t] = mma(f, dsf, (first && ks == 0) ? zero16() : acck[t]);
      }
    }
    // Issue order: LLVM's interleaving strategy 0 spreads the LDS operand reads between the MFMAs
    // (one wave per SIMD cannot hide an LDS round trip behind another wave's work); it beat
    // explicit scheduling groups with the reads six MFMAs ahead by 3% on the global layer.
    __builtin_amdgcn_iglp_opt(0);
  };

  // Step 0 is peeled so that the accumulators start as MFMA results. The scheduling barriers
  // keep the next step's loads ahead of the math and its LDS stores behind it (left alone, the
  // scheduler pulls the stores up next to the loads and every step waits for global memory).
  //
  // Steps whose tile every key of the workgroup sees in full need no mask: rows at or after the
  // block's last key (q0 >= kb0 + 32 NW - 1), inside the window of its first key, and before L.
  // In the descending or ascending order (long windows) they form one run [s_a, s_b); the steps
  // outside it (the tiles on the diagonal, a partial last tile) take the masked variant. Each loop
  // stays free of branches.
  auto stage = [&](int step) { return smem + (step & 1) * St::kBytes; };
  int s_a = 0, s_b = 0;
  if (!alt) {
    // tile t is interior iff 32 t >= kb0 + 32 NW - 1, 32 t <= kb0 + W - 32 and 32 t <= L - 32
    const int t_lo = (kb0 + 32 * NW - 1 + kQT - 1) / kQT;
    const long long lim = min((long long)kb0 + a.window - kQT, (long long)a.L - kQT);
    if (lim >= 0) {
      const int t_hi = (int)min((long long)qt_last, lim / kQT);
      if (t_lo <= t_hi) {
        s_a = (asc ? t_lo - qt0 : qt_last - t_hi) * a.G;
        s_b = (asc ? t_hi - qt0 + 1 : qt_last - t_lo + 1) * a.G;
      }
    }
  }
  auto run = [&](int s0, int s1, auto masked) {
    for (int step = s0; step < s1; ++step) {
      load_step(min(step + 1, nsteps - 1), ra);
      __builtin_amdgcn_sched_barrier(0);
      compute(step, false, masked);
      __builtin_amdgcn_sched_barrier(0);
      store_step(stage(step + 1), ra);
      __syncthreads();
    }
  };
  load_step(min(1, nsteps - 1), ra);
  __builtin_amdgcn_sched_barrier(0);
  if (s_a == 0 && s_b > 0)
    compute(0, true, BoolTag<false>{});
  else
    compute(0, true, BoolTag<true>{});
  __builtin_amdgcn_sched_barrier(0);
  store_step(stage(1), ra);
  __syncthreads();
  run(1, s_a, BoolTag<true>{});
  run(max(1, s_a), s_b, BoolTag<false>{});
  run(max(1, s_b), nsteps, BoolTag<true>{});

  const bool kvalid = kpos < a.L;
  char* dkrow = (char*)a.dk + krow * kDQK * E::kBytes;
  char* dvrow = (char*)a.dv + krow * kDV * E::kBytes;
  store_out_row<E>(dkrow, acck, a.scale, half, kvalid);
  store_out_row<E>(dvrow, accv, 1.f, half, kvalid);
  }
}

// ---------------------------------------------------------------------------- sink gradient

__global__ __launch_bounds__(256) void bwd_sink_kernel(const BackwardArgs a) {
  __shared__ float red[256];
  poison_lds(red, sizeof(red));
  const int h = blockIdx.x, tid = threadIdx.x;
  const int n = a.B * a.n_qtiles;
  const float* p = a.sink_part + (size_t)h * n;
  float t = 0.f;
  for (int i = tid; i < n; i += 256) t += p[i];
  red[tid] = t;
  __syncthreads();
#pragma unroll
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) a.dsink[h] = -red[0];
}

// ------------------------------------------------------------------------------------ launchers

size_t backward_ws_d_bytes(int B, int L, int Hq) {
  const size_t d = (size_t)B * Hq * L * 4;
  return (d + 255) / 256 * 256;
}

size_t backward_ws_bytes(int B, int L, int Hq) {
  const size_t n_qtiles = ((size_t)L + kQT - 1) / kQT;
  return backward_ws_d_bytes(B, L, Hq) + (size_t)Hq * B * n_qtiles * 4;
}


// windows the sliding-window dQ walk serves (the window of a 32-row tile is then five 32-key
// blocks), and its shortest segment
constexpr int kDqSwaMaxWindow = 129;
constexpr int kDqSwaMinTiles = 8;

template <typename E>
static hipError_t launch_backward(BackwardArgs a, hipStream_t stream) {
  // dQ workgroups of 8 waves (bf16) or 4 (fp32: at 8 waves, two per SIMD, its operands need more
  // than the 256 registers a wave then has, and spilled)
  constexpr int NW = E::kBytes == 2 ? 8 : 4, BK = 32;
  // dK/dV workgroups of 4 waves (128 keys) walk every query tile that sees any of their keys; under
  // a short window each wave sees only some of them (5 of 8 at W = 128) and computes the rest with
  // p = 0. Two-wave workgroups (64 keys, two per CU) walk 6 tiles for the same 5 (bf16; the fp32
  // kernel's doubled staging registers would spill).
  const bool kv2 = E::kBytes == 2 && a.window <= kDkdvShortWindow;
  const int nwk = kv2 ? 2 : 4;
  int hg = 1;
  while (hg < NW && a.G % (hg * 2) == 0) hg *= 2;
  a.heads_per_wg = hg;
  a.n_hchunks = a.G / hg;
  const int rows_per_wg = kQT * (NW / hg);
  a.n_qblocks = (a.L + rows_per_wg - 1) / rows_per_wg;
  a.n_kblocks = (a.L + 32 * nwk - 1) / (32 * nwk);
  a.n_qtiles = (a.L + kQT - 1) / kQT;

  // global layers (the window covers the sequence): key blocks p and n_kblocks - 1 - p share a
  // workgroup (see the kernel)
  a.kv_pairs = E::kBytes == 2 && !kv2 && a.window >= a.L ? 1 : 0;
  const long long n_dq = (long long)a.n_qblocks * a.B * a.Hkv * a.n_hchunks;
  const long long n_kv = (long long)(a.kv_pairs ? (a.n_kblocks + 1) / 2 : a.n_kblocks) * a.B * a.Hkv;
  if (n_dq > 0x7fffffffLL || n_kv > 0x7fffffffLL) return hipErrorInvalidValue;
  if (E::kBytes == 2 && hg == 8 && a.window <= kDqSwaMaxWindow) {
    // sliding window: the ping-pong walk over segments of tiles, about one workgroup per compute
    // unit in total (at least kDqSwaMinTiles tiles per segment, each re-reads a 4-block halo)
    const long long units = (long long)a.B * a.Hkv * a.n_hchunks;
    long long segs = (256 + units - 1) / units;
    long long per = (a.n_qtiles + segs - 1) / segs;
    if (per < kDqSwaMinTiles) per = kDqSwaMinTiles;
    a.tiles_per_wg = (int)per;
    a.n_segments = (int)((a.n_qtiles + per - 1) / per);
    const long long n_wg = units * a.n_segments;
    if (n_wg > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.window >= 128)
      hipLaunchKernelGGL(bwd_dq_swa_kernel<false>, dim3((unsigned)n_wg), dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_dq_swa_kernel<true>, dim3((unsigned)n_wg), dim3(512), 0, stream, a);
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<E, NW, BK>), dim3((unsigned)n_dq), dim3(NW * 64), 0, stream, a);
  }
  if constexpr (E::kBytes == 2) {
    if (kv2)
      hipLaunchKernelGGL((bwd_dkdv_kernel<E, 2>), dim3((unsigned)n_kv), dim3(128), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<E, 4>), dim3((unsigned)n_kv), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, 4>), dim3((unsigned)n_kv), dim3(256), 0, stream, a);
  }
  if (a.dsink) hipLaunchKernelGGL(bwd_sink_kernel, dim3(a.Hq), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t backward_launch(bool bf16, BackwardArgs a, hipStream_t stream) {
  return bf16 ? launch_backward<BF16>(a, stream) : launch_backward<F32>(a, stream);
}

}  // namespace mimo
