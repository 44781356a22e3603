// Argument blocks and launchers shared by the host API and the kernels.
#pragma once

#include "common.hpp"

namespace mimo {

constexpr int kMaxCols = 64;  // decode: query columns per workgroup (query heads per KV head x new tokens)
constexpr int kColsNW = 4;    // column-split decode: waves per workgroup, 32 query columns each
constexpr int kColsCols = 32 * kColsNW;
constexpr int kMaxNew = 8;    // decode: new tokens per sequence (next token + drafts)

// Prefill arguments (kernel argument block, passed by value).
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* sink;
  int B, L, Hq, Hkv, G;
  int window;        // clamped to <= L by the host
  float scale_log2;  // scale * log2(e)
  int heads_per_wg;  // HG
  int n_qblocks;     // ceil(L / (32 * NW / HG))
  int n_hchunks;     // G / HG
  int n_segments;    // sliding-window ring kernel: segments of consecutive tiles per (b, g, chunk)
  int tiles_per_wg;  // sliding-window ring kernel: 32-row tiles per segment
  const float* rope;  // [>= L][32][2] (cos, sin) when Q/K arrive before the rotary embedding, else NULL
  void* k_ws;         // with rope: room for the rotated K ([B, L, Hkv, 192]), or NULL
  HeadList hl;
};

// Decode arguments (kernel argument block, passed by value).
struct DecodeArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cache_len;
  const int32_t* cache_offset;
  const float* sink;
  void* o;
  float* lse;
  float* ws;  // [B][Hkv][nsplit][ncols_pad][kDDV + 4] fp32 when nsplit > 1
  int B, T, Hq, Hkv, G, C;
  int max_len;
  int window;  // clamped to <= max_len + T by the host
  float scale_log2;
  int nsplit;
  int keys_per_split;  // multiple of 32
  int ncols;           // G * T query columns per KV head
  int chunk_cols;      // query columns per workgroup (32 or kMaxCols)
  int n_chunks;        // ceil(ncols / chunk_cols) workgroups share them
  const float* rope;   // [>= max_len + T][32][2] (cos, sin) when q/k_new arrive unrotated, else NULL
  HeadList hl;
};

// Backward arguments (kernel argument block, passed by value).
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;        // forward output
  const void* d_o;      // gradient of the loss with respect to o
  const float* lse;     // [B][Hq][L] natural-log denominators of the forward, sink included
  const float* sink;    // [Hq] or NULL
  void* dq;
  void* dk;
  void* dv;
  float* dsink;         // [Hq] or NULL (sink gradient not wanted)
  float* D;             // workspace [B][Hq][L]: <dO_i, O_i>
  float* sink_part;     // workspace [Hq][B][n_qtiles] per-tile partial sums, NULL if no dsink
  int B, L, Hq, Hkv, G;
  int window;           // clamped to <= L by the host
  float scale;
  float scale_log2;     // scale * log2(e)
  int heads_per_wg;     // dq kernel: query heads per workgroup
  int n_qblocks;        // dq kernel: query blocks per (b, g, head chunk)
  int n_hchunks;        // dq kernel: G / heads_per_wg
  int n_kblocks;        // dk/dv kernel: key blocks per (b, g)
  int kv_pairs;         // dk/dv kernel: 1 = a workgroup takes key blocks p and n_kblocks - 1 - p
  int n_qtiles;         // ceil(L / 32)
  int n_segments;       // sliding-window dq kernel: segments of consecutive tiles per (b, g, chunk)
  int tiles_per_wg;     // sliding-window dq kernel: 32-row tiles per segment
  HeadList hl;
};

// Cache commit arguments (kernel argument block, passed by value).
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  int32_t* cache_len;           // [B], read then advanced
  const int32_t* cache_offset;  // [B] or NULL
  const int32_t* accept;        // [B] or NULL (all T)
  int B, T, Hkv, C, max_len;
};

// Fills table[p][i] = (cos, sin)(p * base^(-2i/64)), p < n_pos, i < 32, evaluated in fp64.
hipError_t rope_table_launch(int n_pos, double base, float* table, hipStream_t stream);
// Picks the prefill variant (fills the tiling fields of `a`) and launches it on `stream`.
hipError_t prefill_launch(bool bf16, PrefillArgs a, hipStream_t stream);
// Bytes of k_ws with which prefill_launch rotates K once instead of at every staging (0: the
// chosen kernel has no use for it).
size_t prefill_rope_ws_bytes(bool bf16, int B, int L, int Hq, int Hkv, int window);
// Launches the decode kernel and, when a.nsplit > 1, the combine kernel on `stream`.
hipError_t decode_launch(bool bf16, const DecodeArgs& a, hipStream_t stream);
// Launches the dq, dk/dv and sink-gradient kernels on `stream` (a.D / a.sink_part point into the
// caller's workspace).
hipError_t backward_launch(bool bf16, BackwardArgs a, hipStream_t stream);
// Workspace bytes of the backward pass: D, then (256-byte aligned) the sink partials.
size_t backward_ws_d_bytes(int B, int L, int Hq);
size_t backward_ws_bytes(int B, int L, int Hq);
// Commits the accepted new tokens of every sequence into its cache on `stream`.
hipError_t cache_append_launch(bool bf16, const AppendArgs& a, hipStream_t stream);
// Workspace bytes for nsplit > 1 partial records (0 otherwise).
size_t decode_ws_bytes(int B, int Hkv, int ncols, int nsplit);

}  // namespace mimo
