// Host side of the C ABI declared in include/mimo_attn.h: argument validation, head grouping,
// decode split planning and kernel launches on the caller's stream. Nothing here allocates,
// frees or synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/mimo_attn.h"
#include "launch.hpp"

namespace {

// Query columns per workgroup of a single-pass decode with more than 32 columns (see decode_impl).
constexpr int kChunkCols1Split = 32;
#ifndef MIMO_WIN_COLS
#define MIMO_WIN_COLS 64
#endif
constexpr int kWindowCols = MIMO_WIN_COLS;


thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Builds the query-head list grouped by KV head; returns 0 or an error code.
int group_heads(int Hq, int Hkv, const int32_t* kv_head_of_q, mimo::HeadList* hl) {
  const int G = Hq / Hkv;
  if (!kv_head_of_q) {
    for (int h = 0; h < Hq; ++h) hl->heads[h] = (int16_t)h;
    hl->identity = 1;
    return MIMO_OK;
  }
  int fill[mimo::kMaxHeads] = {0};
  for (int h = 0; h < Hq; ++h) {
    const int g = kv_head_of_q[h];
    if (g < 0 || g >= Hkv) return fail(MIMO_EINVAL, "kv_head_of_q[%d] = %d is outside [0, %d)", h, g, Hkv);
    if (fill[g] >= G) return fail(MIMO_EINVAL, "KV head %d serves more than Hq/Hkv = %d query heads", g, G);
    hl->heads[g * G + fill[g]++] = (int16_t)h;
  }
  // every KV head now has exactly G heads (counts sum to Hq)
  hl->identity = 1;
  for (int h = 0; h < Hq; ++h) hl->identity &= hl->heads[h] == h;
  return MIMO_OK;
}

int check_common(int dt, int B, int Hq, int Hkv, int d_qk, int d_v, int window, float scale) {
  if (dt != MIMO_F32 && dt != MIMO_BF16) return fail(MIMO_EUNSUPPORTED, "unknown dtype %d", dt);
  if (B < 1 || Hq < 1 || Hkv < 1) return fail(MIMO_EINVAL, "B, Hq and Hkv must be >= 1");
  if (Hq % Hkv) return fail(MIMO_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (Hq > mimo::kMaxHeads) return fail(MIMO_EUNSUPPORTED, "Hq %d exceeds %d", Hq, mimo::kMaxHeads);
  if (window < 1) return fail(MIMO_EINVAL, "window must be >= 1 (got %d)", window);
  // the kernels scale the running max of raw scores, which equals the max of scaled scores only
  // for a positive scale
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(MIMO_EINVAL, "scale must be finite and > 0");
  if (d_qk != 192 || d_v != 128)
    return fail(MIMO_EUNSUPPORTED, "head dims (%d, %d) unsupported; the library supports (192, 128)", d_qk, d_v);
  return MIMO_OK;
}

}  // namespace

extern "C" {

const char* mimo_attn_last_error(void) { return g_err.c_str(); }

int mimo_attn_version(void) { return 10000; }

}  // extern "C"

namespace {

// rope: NULL, or a table of at least L positions for Q/K given before the rotary embedding
int prefill_impl(mimo_dtype dt, int B, int L, int Hq, int Hkv, int d_qk, int d_v, const void* q,
                 const void* k, const void* v, int window, const float* sink,
                 const int32_t* kv_head_of_q, float scale, const float* rope, void* k_ws, void* o,
                 float* lse, hipStream_t stream) {
  g_err.clear();
  if (int rc = check_common(dt, B, Hq, Hkv, d_qk, d_v, window, scale)) return rc;
  if (L < 1) return fail(MIMO_EINVAL, "L must be >= 1");
  if (L > (1 << 30)) return fail(MIMO_EUNSUPPORTED, "L %d exceeds 2^30", L);
  if (!q || !k || !v || !o) return fail(MIMO_EINVAL, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(MIMO_EINVAL, "q, k, v and o must be 16-byte aligned");
  if ((sink && !aligned4(sink)) || (lse && !aligned4(lse)))
    return fail(MIMO_EINVAL, "sink and lse must be 4-byte aligned");
  const double elem = dt == MIMO_BF16 ? 2.0 : 4.0;
  if ((double)B * L * Hq * d_qk * elem > 4.6e18) return fail(MIMO_EINVAL, "tensor too large");

  mimo::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.sink = sink; a.rope = rope; a.k_ws = k_ws;
  a.B = B; a.L = L; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.window = window < L ? window : L;
  a.scale_log2 = scale * mimo::kLog2e;
  if (int rc = group_heads(Hq, Hkv, kv_head_of_q, &a.hl)) return rc;
  const hipError_t e = mimo::prefill_launch(dt == MIMO_BF16, a, stream);
  if (e != hipSuccess) return fail(MIMO_EHIP, "prefill launch failed: %s", hipGetErrorString(e));
  return MIMO_OK;
}

int check_rope(const float* table, int positions, int rot_dims, long long need) {
  if (rot_dims != mimo::kRopeDims)
    return fail(MIMO_EUNSUPPORTED, "rot_dims %d unsupported; the library rotates %d dims", rot_dims,
                mimo::kRopeDims);
  if (!table || !aligned16(table)) return fail(MIMO_EINVAL, "rope_table must be non-NULL and 16-byte aligned");
  if (positions < need)
    return fail(MIMO_EINVAL, "rope_table has %d positions, %lld needed", positions, need);
  return MIMO_OK;
}

}  // namespace

extern "C" {

int mimo_attn_prefill(mimo_dtype dt, int B, int L, int Hq, int Hkv, int d_qk, int d_v,
                      const void* q, const void* k, const void* v, int window, const float* sink,
                      const int32_t* kv_head_of_q, float scale, void* o, float* lse,
                      hipStream_t stream) {
  return prefill_impl(dt, B, L, Hq, Hkv, d_qk, d_v, q, k, v, window, sink, kv_head_of_q, scale,
                      nullptr, nullptr, o, lse, stream);
}

size_t mimo_attn_prefill_rope_workspace_size(mimo_dtype dt, int B, int L, int Hq, int Hkv,
                                             int window) {
  if ((dt != MIMO_BF16 && dt != MIMO_F32) || B < 1 || L < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv ||
      window < 1)
    return 0;
  return mimo::prefill_rope_ws_bytes(dt == MIMO_BF16, B, L, Hq, Hkv, window);
}

int mimo_attn_prefill_rope(mimo_dtype dt, int B, int L, int Hq, int Hkv, int d_qk, int d_v,
                           const void* q, const void* k, const void* v, int window,
                           const float* sink, const int32_t* kv_head_of_q, float scale,
                           const float* rope_table, int rope_positions, int rot_dims,
                           void* workspace, size_t workspace_bytes, void* o, float* lse,
                           hipStream_t stream) {
  g_err.clear();
  if (int rc = check_rope(rope_table, rope_positions, rot_dims, L)) return rc;
  void* k_ws = nullptr;
  if (workspace) {
    if (!aligned16(workspace)) return fail(MIMO_EINVAL, "workspace must be 16-byte aligned");
    const size_t need = mimo_attn_prefill_rope_workspace_size(dt, B, L, Hq, Hkv, window);
    if (workspace_bytes < need)
      return fail(MIMO_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (need > 0) k_ws = workspace;
  }
  return prefill_impl(dt, B, L, Hq, Hkv, d_qk, d_v, q, k, v, window, sink, kv_head_of_q, scale,
                      rope_table, k_ws, o, lse, stream);
}

int mimo_attn_cache_append(mimo_dtype dt, int B, int T, int Hkv, int d_qk, int d_v,
                           const void* k_new, const void* v_new, void* k_cache, void* v_cache, int C,
                           int32_t* cache_len, const int32_t* cache_offset,
                           const int32_t* accept_len, int max_cache_len, hipStream_t stream) {
  g_err.clear();
  if (dt != MIMO_F32 && dt != MIMO_BF16) return fail(MIMO_EUNSUPPORTED, "unknown dtype %d", dt);
  if (B < 1 || Hkv < 1) return fail(MIMO_EINVAL, "B and Hkv must be >= 1");
  if (T < 1 || T > mimo::kMaxNew) return fail(MIMO_EINVAL, "T must be in 1..%d (got %d)", mimo::kMaxNew, T);
  if (d_qk != 192 || d_v != 128)
    return fail(MIMO_EUNSUPPORTED, "head dims (%d, %d) unsupported; the library supports (192, 128)", d_qk, d_v);
  if (C < 1) return fail(MIMO_EINVAL, "C must be >= 1");
  if (max_cache_len < 0 || max_cache_len > (1 << 30) - 8)
    return fail(MIMO_EINVAL, "max_cache_len %d outside [0, 2^30 - 8]", max_cache_len);
  if (!k_new || !v_new || !k_cache || !v_cache || !cache_len)
    return fail(MIMO_EINVAL, "k_new, v_new, k_cache, v_cache and cache_len must be non-NULL");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(MIMO_EINVAL, "k_new, v_new, k_cache and v_cache must be 16-byte aligned");
  if (!aligned4(cache_len) || (cache_offset && !aligned4(cache_offset)) || (accept_len && !aligned4(accept_len)))
    return fail(MIMO_EINVAL, "cache_len, cache_offset and accept_len must be 4-byte aligned");
  const double elem = dt == MIMO_BF16 ? 2.0 : 4.0;
  if ((double)B * C * Hkv * d_qk * elem > 4.6e18) return fail(MIMO_EINVAL, "cache too large");
  mimo::AppendArgs a{};
  a.k_new = k_new; a.v_new = v_new; a.k_cache = k_cache; a.v_cache = v_cache;
  a.cache_len = cache_len; a.cache_offset = cache_offset; a.accept = accept_len;
  a.B = B; a.T = T; a.Hkv = Hkv; a.C = C; a.max_len = max_cache_len;
  const hipError_t e = mimo::cache_append_launch(dt == MIMO_BF16, a, stream);
  if (e != hipSuccess) return fail(MIMO_EHIP, "cache append launch failed: %s", hipGetErrorString(e));
  return MIMO_OK;
}

size_t mimo_attn_prefill_backward_workspace_size(int B, int L, int Hq) {
  if (B < 1 || L < 1 || Hq < 1) return 0;
  return mimo::backward_ws_bytes(B, L, Hq);
}

int mimo_attn_prefill_backward(mimo_dtype dt, int B, int L, int Hq, int Hkv, int d_qk, int d_v,
                               const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* d_o, int window, const float* sink,
                               const int32_t* kv_head_of_q, float scale, void* dq, void* dk,
                               void* dv, float* dsink, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  g_err.clear();
  if (int rc = check_common(dt, B, Hq, Hkv, d_qk, d_v, window, scale)) return rc;
  if (L < 1) return fail(MIMO_EINVAL, "L must be >= 1");
  if (L > (1 << 30)) return fail(MIMO_EUNSUPPORTED, "L %d exceeds 2^30", L);
  if (!q || !k || !v || !o || !lse || !d_o || !dq || !dk || !dv)
    return fail(MIMO_EINVAL, "q, k, v, o, lse, d_o, dq, dk and dv must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_o) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(MIMO_EINVAL, "q, k, v, o, d_o, dq, dk and dv must be 16-byte aligned");
  if (!aligned4(lse) || (sink && !aligned4(sink)) || (dsink && !aligned4(dsink)))
    return fail(MIMO_EINVAL, "lse, sink and dsink must be 4-byte aligned");
  if (dsink && !sink) return fail(MIMO_EINVAL, "dsink given without a sink");
  const double elem = dt == MIMO_BF16 ? 2.0 : 4.0;
  if ((double)B * L * Hq * d_qk * elem > 4.6e18) return fail(MIMO_EINVAL, "tensor too large");
  const size_t need = mimo::backward_ws_bytes(B, L, Hq);
  if (!workspace || !aligned16(workspace))
    return fail(MIMO_EINVAL, "workspace must be non-NULL and 16-byte aligned");
  if (workspace_bytes < need)
    return fail(MIMO_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);

  mimo::BackwardArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.d_o = d_o; a.lse = lse; a.sink = sink;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dsink = dsink;
  a.D = static_cast<float*>(workspace);
  a.sink_part = dsink ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                 mimo::backward_ws_d_bytes(B, L, Hq))
                      : nullptr;
  a.B = B; a.L = L; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.window = window < L ? window : L;
  a.scale = scale;
  a.scale_log2 = scale * mimo::kLog2e;
  if (int rc = group_heads(Hq, Hkv, kv_head_of_q, &a.hl)) return rc;
  const hipError_t e = mimo::backward_launch(dt == MIMO_BF16, a, stream);
  if (e != hipSuccess) return fail(MIMO_EHIP, "backward launch failed: %s", hipGetErrorString(e));
  return MIMO_OK;
}

int mimo_attn_rope_table(int n_pos, int rot_dims, double base, float* table, hipStream_t stream) {
  g_err.clear();
  if (rot_dims != mimo::kRopeDims)
    return fail(MIMO_EUNSUPPORTED, "rot_dims %d unsupported; the library rotates %d dims", rot_dims,
                mimo::kRopeDims);
  if (n_pos < 1 || n_pos > (1 << 30)) return fail(MIMO_EINVAL, "n_pos %d outside [1, 2^30]", n_pos);
  if (!std::isfinite(base) || !(base > 1.0)) return fail(MIMO_EINVAL, "base must be finite and > 1");
  if (!table || !aligned16(table)) return fail(MIMO_EINVAL, "table must be non-NULL and 16-byte aligned");
  const hipError_t e = mimo::rope_table_launch(n_pos, base, table, stream);
  if (e != hipSuccess) return fail(MIMO_EHIP, "rope table launch failed: %s", hipGetErrorString(e));
  return MIMO_OK;
}

}  // extern "C"

namespace {

struct DecodePlan {
  int window;          // clamped
  int nsplit;          // >= 1
  int keys_per_split;  // multiple of 32
  size_t ws_bytes;
};

// Splits: about 8192 committed keys per split, but at least one workgroup per compute unit of an
// MI355X (256), and never fewer than 256 keys per split. Sweeps of explicit split counts: 8 x 262144
// keys (64/4 heads) 16: 968 us, 32: 951 us, 64: 981 us, 128: 1082 us; 64 x 16384 keys 1: 552 us,
// 2: 493 us, 4: 515 us, 8: 558 us; 64 x 127 ring keys 1: 17 us, 2: 32 us. An explicit request is
// honoured up to one 32-key block per split.
DecodePlan plan_decode(int B, int T, int Hq, int Hkv, int max_len, int window, int num_splits) {
  DecodePlan p{};
  const long long wmax = (long long)max_len + T;
  p.window = window < wmax ? window : (int)wmax;
  // committed keys only: the new tokens are folded in by the last split
  long long list_max = (long long)(max_len < p.window - 1 ? max_len : p.window - 1);
  if (list_max < 1) list_max = 1;
  const long long blocks = (list_max + 31) / 32;
  long long ns;
  if (num_splits > 0) {
    ns = num_splits;
  } else {
    const long long chunks = ((long long)(Hq / Hkv) * T + mimo::kMaxCols - 1) / mimo::kMaxCols;
    const long long pairs = (long long)B * Hkv * chunks;
    const long long fill = (256 + pairs - 1) / pairs;
    const long long by_len = (list_max + 8191) / 8192;
    ns = fill > by_len ? fill : by_len;
    const long long cap = (list_max + 255) / 256;
    if (ns > cap) ns = cap;
  }
  if (ns > blocks) ns = blocks;
  if (ns < 1) ns = 1;
  const long long kps_blocks = (blocks + ns - 1) / ns;
  p.keys_per_split = (int)(kps_blocks * 32);
  p.nsplit = (int)((list_max + p.keys_per_split - 1) / p.keys_per_split);
  const int G = Hq / Hkv;
  p.ws_bytes = mimo::decode_ws_bytes(B, Hkv, G * T, p.nsplit);
  return p;
}

}  // namespace

extern "C" {

size_t mimo_attn_decode_workspace_size(int B, int T, int Hq, int Hkv, int d_v, int max_cache_len,
                                       int window, int num_splits) {
  if (B < 1 || T < 1 || T > mimo::kMaxNew || Hq < 1 || Hkv < 1 || Hq % Hkv || d_v != 128 ||
      max_cache_len < 0 || window < 1 || num_splits < 0 || Hq > mimo::kMaxHeads)
    return 0;
  return plan_decode(B, T, Hq, Hkv, max_cache_len, window, num_splits).ws_bytes;
}

}  // extern "C"

// ------------------------------------------------------------------------ decode without allocation
//
// mimo_attn_decode for callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc): the split-KV partial records go to `scratch`, a
// static device array of kNoallocScratchBytes that every GPU the library runs on holds until the
// process ends. Host code never uses the array's name as a device address: its address on each
// device comes from hipGetSymbolAddress, taken once per device (with that device current) on the
// first call there that needs partials, and kept in g_scratch_dev.

constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

// This device's address of `scratch` for launches on `stream` (which must belong to the current
// device, the one the address is taken on).
int scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(MIMO_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  hipDevice_t sdev = 0;
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) return fail(MIMO_EHIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
  if ((int)sdev != cur)
    return fail(MIMO_EINVAL, "the stream belongs to device %d but device %d is current", (int)sdev, cur);
  if (cur < 0 || cur >= kMaxDevices) return fail(MIMO_EUNSUPPORTED, "device %d beyond %d", cur, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[cur]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MIMO_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_dev[cur] = p;
  }
  *out = g_scratch_dev[cur];
  return MIMO_OK;
}

}  // namespace

namespace {

// rope: NULL, or a table of at least max_cache_len + T positions for unrotated q / k_new
// static_ws: the partials go to the library's static scratch (workspace arguments unused)
int decode_impl(mimo_dtype dt, int B, int T, int Hq, int Hkv, int d_qk, int d_v, const void* q,
                const void* k_new, const void* v_new, const void* k_cache, const void* v_cache,
                int C, const int32_t* cache_len, const int32_t* cache_offset, int max_cache_len,
                int window, const float* sink, const int32_t* kv_head_of_q, float scale,
                const float* rope, int num_splits, void* workspace, size_t workspace_bytes,
                void* o, float* lse, hipStream_t stream, bool static_ws = false) {
  if (int rc = check_common(dt, B, Hq, Hkv, d_qk, d_v, window, scale)) return rc;
  if (T < 1 || T > mimo::kMaxNew) return fail(MIMO_EINVAL, "T must be in 1..%d (got %d)", mimo::kMaxNew, T);
  if (max_cache_len < 0 || max_cache_len > (1 << 30) - 8)
    return fail(MIMO_EINVAL, "max_cache_len %d outside [0, 2^30 - 8]", max_cache_len);
  if (C < 1) return fail(MIMO_EINVAL, "C must be >= 1");
  const int need = (window - 1 < max_cache_len) ? window - 1 : max_cache_len;
  if (C < need)
    return fail(MIMO_EINVAL, "cache of %d slots cannot hold the %d committed keys a window of %d needs",
                C, need, window);
  if (num_splits < 0) return fail(MIMO_EINVAL, "num_splits must be >= 0");
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !o || !cache_len)
    return fail(MIMO_EINVAL, "q, k_new, v_new, k_cache, v_cache, cache_len and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(o))
    return fail(MIMO_EINVAL, "q, k_new, v_new, k_cache, v_cache and o must be 16-byte aligned");
  if (!aligned4(cache_len) || (cache_offset && !aligned4(cache_offset)) || (sink && !aligned4(sink)) ||
      (lse && !aligned4(lse)))
    return fail(MIMO_EINVAL, "cache_len, cache_offset, sink and lse must be 4-byte aligned");
  const double elem = dt == MIMO_BF16 ? 2.0 : 4.0;
  if ((double)B * C * Hkv * d_qk * elem > 4.6e18) return fail(MIMO_EINVAL, "cache too large");

  const DecodePlan plan = plan_decode(B, T, Hq, Hkv, max_cache_len, window, num_splits);
  if (static_ws && plan.ws_bytes > 0) {
    if (plan.ws_bytes > kNoallocScratchBytes)
      return fail(MIMO_EWORKSPACE,
                  "the split partials need %zu bytes, the library's static decode scratch holds %zu "
                  "(a smaller num_splits needs less)", plan.ws_bytes, kNoallocScratchBytes);
    if (int rc = scratch_address(stream, &workspace)) return rc;
    workspace_bytes = kNoallocScratchBytes;
  }
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes)
      return fail(MIMO_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes,
                  plan.ws_bytes);
    if (!aligned16(workspace)) return fail(MIMO_EINVAL, "workspace must be 16-byte aligned");
  }

  mimo::DecodeArgs a{};
  a.q = q; a.k_new = k_new; a.v_new = v_new; a.k_cache = k_cache; a.v_cache = v_cache;
  a.cache_len = cache_len; a.cache_offset = cache_offset; a.sink = sink; a.rope = rope;
  a.o = o; a.lse = lse; a.ws = static_cast<float*>(workspace);
  a.B = B; a.T = T; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.C = C;
  a.max_len = max_cache_len;
  a.window = plan.window;
  a.scale_log2 = scale * mimo::kLog2e;
  a.nsplit = plan.nsplit;
  a.keys_per_split = plan.keys_per_split;
  a.ncols = a.G * T;
  // More than kMaxCols query columns per KV head (e.g. 16 heads x 8 tokens) are cut into chunks
  // that run as separate workgroups. A single pass (a sliding-window ring) with more than 32
  // columns takes chunks of 32: the one-block kernel keeps two waves per SIMD, which beats
  // reading the short K/V history once with the 64-column kernel (8 heads x 8 tokens: 107 vs
  // 147 us).
  // fp32 always takes chunks of 32: its 64-column kernel needs more than the 512 registers of a
  // lane (the K and V half rows alone are 160) and spilled.
  a.chunk_cols = (dt == MIMO_F32 || (plan.nsplit == 1 && a.ncols > 32)) ? kChunkCols1Split : mimo::kMaxCols;
  // bf16 single passes over at most four 32-key blocks run the one-pass window kernel, which
  // takes two column blocks per workgroup (each K / V fragment then feeds two products)
  if (dt == MIMO_BF16 && plan.nsplit == 1 && plan.keys_per_split <= 128 && a.ncols > 32)
    a.chunk_cols = kWindowCols;
  // other bf16 calls with more than 64 columns (16 heads x 8 tokens) run the column-split kernel
  // with 128 columns per workgroup, which streams the cache once for all of them (33..64 columns
  // run it with 64)
  else if (dt == MIMO_BF16 && a.ncols > mimo::kMaxCols)
    a.chunk_cols = mimo::kColsCols;
  a.n_chunks = (a.ncols + a.chunk_cols - 1) / a.chunk_cols;
  if ((long long)a.Hkv * a.n_chunks > 65535) return fail(MIMO_EUNSUPPORTED, "too many KV heads x column chunks");
  if (int rc = group_heads(Hq, Hkv, kv_head_of_q, &a.hl)) return rc;
  const hipError_t e = mimo::decode_launch(dt == MIMO_BF16, a, stream);
  if (e != hipSuccess) return fail(MIMO_EHIP, "decode launch failed: %s", hipGetErrorString(e));
  return MIMO_OK;
}

}  // namespace

extern "C" {

int mimo_attn_decode(mimo_dtype dt, int B, int T, int Hq, int Hkv, int d_qk, int d_v,
                     const void* q, const void* k_new, const void* v_new, const void* k_cache,
                     const void* v_cache, int C, const int32_t* cache_len,
                     const int32_t* cache_offset, int max_cache_len, int window,
                     const float* sink, const int32_t* kv_head_of_q, float scale, int num_splits,
                     void* workspace, size_t workspace_bytes, void* o, float* lse,
                     hipStream_t stream) {
  g_err.clear();
  return decode_impl(dt, B, T, Hq, Hkv, d_qk, d_v, q, k_new, v_new, k_cache, v_cache, C, cache_len,
                     cache_offset, max_cache_len, window, sink, kv_head_of_q, scale, nullptr,
                     num_splits, workspace, workspace_bytes, o, lse, stream);
}

int mimo_attn_decode_rope(mimo_dtype dt, int B, int T, int Hq, int Hkv, int d_qk, int d_v,
                          const void* q, const void* k_new, const void* v_new, const void* k_cache,
                          const void* v_cache, int C, const int32_t* cache_len,
                          const int32_t* cache_offset, int max_cache_len, int window,
                          const float* sink, const int32_t* kv_head_of_q, float scale,
                          const float* rope_table, int rope_positions, int rot_dims,
                          int num_splits, void* workspace, size_t workspace_bytes, void* o,
                          float* lse, hipStream_t stream) {
  g_err.clear();
  if (int rc = check_rope(rope_table, rope_positions, rot_dims, (long long)max_cache_len + T)) return rc;
  return decode_impl(dt, B, T, Hq, Hkv, d_qk, d_v, q, k_new, v_new, k_cache, v_cache, C, cache_len,
                     cache_offset, max_cache_len, window, sink, kv_head_of_q, scale, rope_table,
                     num_splits, workspace, workspace_bytes, o, lse, stream);
}

}  // extern "C"

extern "C" {

int mimo_attn_decode_noalloc(mimo_dtype dt, int B, int T, int Hq, int Hkv, int d_qk, int d_v,
                             const void* q, const void* k_new, const void* v_new,
                             const void* k_cache, const void* v_cache, int C,
                             const int32_t* cache_len, const int32_t* cache_offset,
                             int max_cache_len, int window, const float* sink,
                             const int32_t* kv_head_of_q, float scale, int num_splits, void* o,
                             float* lse, hipStream_t stream) {
  g_err.clear();
  return decode_impl(dt, B, T, Hq, Hkv, d_qk, d_v, q, k_new, v_new, k_cache, v_cache, C, cache_len,
                     cache_offset, max_cache_len, window, sink, kv_head_of_q, scale, nullptr,
                     num_splits, nullptr, 0, o, lse, stream, true);
}

}  // extern "C"
