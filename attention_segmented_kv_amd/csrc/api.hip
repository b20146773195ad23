// C ABI of the segment-attention library: argument checks, split planning, launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/seg_attn.h"

namespace segattn {
hipError_t launch_prefill(const void* q, const void* k_pool, const void* v_pool, const void* segs,
                          const int32_t* seg_indptr, const int32_t* cu_q, const int32_t* cu_k,
                          int batch, int max_seqlen_q, int hkv, float scale, int causal, void* out,
                          float* lse, int cu_count, int force_tile, hipStream_t stream);
hipError_t launch_decode(const void* q, const void* k_pool, const void* v_pool,
                         const float* k_scale, const float* v_scale, int fp8, const void* segs,
                         const int32_t* seg_indptr, const int32_t* cu_k, int batch, int hkv,
                         int split_len, int num_splits, float scale, void* out, float* lse,
                         float* ws_o, float* ws_lse, hipStream_t stream);
}  // namespace segattn

namespace {

constexpr int kHeadDim = 128;
constexpr int kGroup = 8;
constexpr int kMaxDevices = 64;
constexpr int kSplitGranule = 64;   // split lengths are multiples of this many keys
constexpr int kMaxAutoSplits = 128;

int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];

// Compute units of the current device (256 on MI355X), read once per device.
int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev]() {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu_count[dev] = n;
  });
  return g_cu_count[dev];
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split plan for decode. A split is the key range one workgroup reduces to one partial result.
// Automatic choice: at least kMinSplit keys per split so each of the workgroup's 4 waves streams
// several tiles, and no more splits than needed to give every compute unit a few workgroups'
// worth of units; split lengths are multiples of 64 keys.
bool plan_splits(int batch, int max_k, int hkv, int fp8, int requested, int* n_out, int* len_out) {
  if (batch < 0 || max_k < 0 || hkv <= 0 || requested < 0) return false;
  if (max_k == 0 || batch == 0) {
    *n_out = 1;
    *len_out = kSplitGranule;
    return true;
  }
  int64_t n;
  if (requested > 0) {
    n = requested;
  } else {
    const int64_t min_split = fp8 ? 1024 : 512;
    const int64_t units_per_level = (int64_t)batch * hkv;
    const int64_t want_units = 4LL * current_cu_count();
    int64_t by_work = ceil_div(want_units, units_per_level);         // splits to fill the chip
    int64_t by_len = ceil_div(max_k, min_split);                      // splits allowed by length
    n = std::max<int64_t>(1, std::min(by_len, std::max<int64_t>(by_work, ceil_div(max_k, 4096))));
    n = std::min<int64_t>(n, kMaxAutoSplits);
  }
  int64_t len = ceil_div(ceil_div(max_k, n), kSplitGranule) * kSplitGranule;
  n = ceil_div(max_k, len);
  *n_out = (int)n;
  *len_out = (int)len;
  return true;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// SEG_ATTN_PREFILL_TILE=128 or 256 pins the prefill tiling (tests use it to cover both).
int prefill_tile_override() {
  const char* v = std::getenv("SEG_ATTN_PREFILL_TILE");
  if (v == nullptr) return 0;
  const int t = std::atoi(v);
  return (t == 128 || t == 256) ? t : 0;
}

size_t workspace_for(int batch, int hq, int n_splits) {
  if (n_splits <= 1) return 0;
  const size_t rows = (size_t)batch * hq * n_splits;
  return align_up(rows * kHeadDim * sizeof(float), 256) + align_up(rows * sizeof(float), 256);
}

seg_attn_status_t check_heads(int32_t hq, int32_t hkv, int32_t head_dim) {
  if (hq <= 0 || hkv <= 0 || head_dim <= 0) return SEG_ATTN_ERR_INVALID_ARG;
  if (hq % hkv != 0) return SEG_ATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || hq / hkv != kGroup) return SEG_ATTN_ERR_UNSUPPORTED;
  return SEG_ATTN_OK;
}

}  // namespace

extern "C" {

const char* seg_attn_status_string(seg_attn_status_t status) {
  switch (status) {
    case SEG_ATTN_OK: return "ok";
    case SEG_ATTN_ERR_INVALID_ARG: return "invalid argument";
    case SEG_ATTN_ERR_UNSUPPORTED: return "unsupported shape (needs head_dim 128 and 8 query heads per kv head)";
    case SEG_ATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
    case SEG_ATTN_ERR_HIP: return "HIP runtime error at launch";
    case SEG_ATTN_ERR_TABLE: return "inconsistent segment / length tables";
    default: return "unknown status";
  }
}

int32_t seg_attn_version(void) { return 1 * 10000 + 0 * 100 + 0; }

seg_attn_status_t seg_attn_prefill(const void* q, const void* k_pool, const void* v_pool,
                                   const seg_attn_segment_t* segs, const int32_t* seg_indptr,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                   int64_t pool_tokens, float softmax_scale, int32_t causal,
                                   void* out, float* lse, seg_attn_stream_t stream) {
  try {
    if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || pool_tokens < 0) return SEG_ATTN_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return SEG_ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return SEG_ATTN_ERR_INVALID_ARG;
    seg_attn_status_t hs = check_heads(num_heads_q, num_heads_kv, head_dim);
    if (hs != SEG_ATTN_OK) return hs;
    if (causal && max_seqlen_q > max_seqlen_k) return SEG_ATTN_ERR_INVALID_ARG;
    if (pool_tokens > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
    if (batch == 0 || max_seqlen_q == 0) return SEG_ATTN_OK;
    if (!q || !k_pool || !v_pool || !segs || !seg_indptr || !cu_seqlens_q || !cu_seqlens_k || !out)
      return SEG_ATTN_ERR_INVALID_ARG;
    const int64_t grid = ceil_div(max_seqlen_q, 16) * (int64_t)num_heads_kv * batch;
    if (grid > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
    hipError_t e = segattn::launch_prefill(q, k_pool, v_pool, segs, seg_indptr, cu_seqlens_q,
                                           cu_seqlens_k, batch, max_seqlen_q, num_heads_kv,
                                           softmax_scale, causal, out, lse, current_cu_count(),
                                           prefill_tile_override(), (hipStream_t)stream);
    return e == hipSuccess ? SEG_ATTN_OK : SEG_ATTN_ERR_HIP;
  } catch (...) {
    return SEG_ATTN_ERR_HIP;
  }
}

int32_t seg_attn_decode_num_splits(int32_t batch, int32_t max_seqlen_k, int32_t num_heads_kv,
                                   int32_t kv_dtype, int32_t num_splits, int32_t* split_len) {
  try {
    if (kv_dtype != SEG_ATTN_KV_BF16 && kv_dtype != SEG_ATTN_KV_FP8_E4M3) return -1;
    int n = 0, len = 0;
    if (!plan_splits(batch, max_seqlen_k, num_heads_kv, kv_dtype == SEG_ATTN_KV_FP8_E4M3, num_splits, &n, &len))
      return -1;
    if (split_len) *split_len = len;
    return n;
  } catch (...) {
    return -1;
  }
}

size_t seg_attn_decode_workspace_bytes(int32_t batch, int32_t max_seqlen_k, int32_t num_heads_q,
                                       int32_t num_heads_kv, int32_t head_dim, int32_t kv_dtype,
                                       int32_t num_splits) {
  try {
    if (check_heads(num_heads_q, num_heads_kv, head_dim) != SEG_ATTN_OK) return 0;
    const int32_t n = seg_attn_decode_num_splits(batch, max_seqlen_k, num_heads_kv, kv_dtype, num_splits, nullptr);
    if (n < 0) return 0;
    return workspace_for(batch, num_heads_q, n);
  } catch (...) {
    return 0;
  }
}

seg_attn_status_t seg_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                                  const float* k_scale, const float* v_scale, int32_t kv_dtype,
                                  const seg_attn_segment_t* segs, const int32_t* seg_indptr,
                                  const int32_t* cu_seqlens_k, int32_t batch,
                                  int32_t max_seqlen_k, int32_t num_heads_q, int32_t num_heads_kv,
                                  int32_t head_dim, int64_t pool_tokens, float softmax_scale,
                                  int32_t num_splits, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, seg_attn_stream_t stream) {
  try {
    if (batch < 0 || max_seqlen_k < 0 || pool_tokens < 0 || num_splits < 0) return SEG_ATTN_ERR_INVALID_ARG;
    if (kv_dtype != SEG_ATTN_KV_BF16 && kv_dtype != SEG_ATTN_KV_FP8_E4M3) return SEG_ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return SEG_ATTN_ERR_INVALID_ARG;
    seg_attn_status_t hs = check_heads(num_heads_q, num_heads_kv, head_dim);
    if (hs != SEG_ATTN_OK) return hs;
    if (pool_tokens > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
    if (batch == 0) return SEG_ATTN_OK;
    const bool fp8 = kv_dtype == SEG_ATTN_KV_FP8_E4M3;
    if (!q || !k_pool || !v_pool || !segs || !seg_indptr || !cu_seqlens_k || !out) return SEG_ATTN_ERR_INVALID_ARG;
    if (fp8 && (!k_scale || !v_scale)) return SEG_ATTN_ERR_INVALID_ARG;
    int n = 0, len = 0;
    if (!plan_splits(batch, max_seqlen_k, num_heads_kv, fp8, num_splits, &n, &len)) return SEG_ATTN_ERR_INVALID_ARG;
    const size_t need = workspace_for(batch, num_heads_q, n);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return SEG_ATTN_ERR_WORKSPACE;
    if ((int64_t)n * num_heads_kv * batch > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
    float* ws_o = nullptr;
    float* ws_lse = nullptr;
    if (n > 1) {
      const size_t rows = (size_t)batch * num_heads_q * n;
      ws_o = (float*)workspace;
      ws_lse = (float*)((char*)workspace + align_up(rows * kHeadDim * sizeof(float), 256));
    }
    hipError_t e = segattn::launch_decode(q, k_pool, v_pool, k_scale, v_scale, fp8 ? 1 : 0, segs,
                                          seg_indptr, cu_seqlens_k, batch, num_heads_kv, len, n,
                                          softmax_scale, out, lse, ws_o, ws_lse, (hipStream_t)stream);
    return e == hipSuccess ? SEG_ATTN_OK : SEG_ATTN_ERR_HIP;
  } catch (...) {
    return SEG_ATTN_ERR_HIP;
  }
}

seg_attn_status_t seg_attn_validate_tables(const seg_attn_segment_t* segs, int64_t nseg,
                                           const int32_t* seg_indptr,
                                           const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_k, int32_t batch,
                                           int64_t pool_tokens, int32_t causal,
                                           int64_t* bad_index) {
  try {
    auto fail = [&](int64_t i) {
      if (bad_index) *bad_index = i;
      return (seg_attn_status_t)SEG_ATTN_ERR_TABLE;
    };
    if (batch < 0 || nseg < 0 || pool_tokens < 0) return SEG_ATTN_ERR_INVALID_ARG;
    if (!seg_indptr || !cu_seqlens_k || (nseg > 0 && !segs)) return SEG_ATTN_ERR_INVALID_ARG;
    if (seg_indptr[0] != 0 || cu_seqlens_k[0] != 0) return fail(0);
    if (cu_seqlens_q && cu_seqlens_q[0] != 0) return fail(0);
    if (seg_indptr[batch] != nseg) return fail(batch);
    for (int32_t b = 0; b < batch; ++b) {
      if (seg_indptr[b + 1] < seg_indptr[b]) return fail(b);
      const int64_t kb = (int64_t)cu_seqlens_k[b + 1] - cu_seqlens_k[b];
      if (kb < 0) return fail(b);
      const int64_t lq = cu_seqlens_q ? (int64_t)cu_seqlens_q[b + 1] - cu_seqlens_q[b] : 1;
      if (lq < 0) return fail(b);
      if (causal && lq > kb) return fail(b);
      int64_t sum = 0;
      for (int32_t s = seg_indptr[b]; s < seg_indptr[b + 1]; ++s) {
        if (segs[s].length < 0 || segs[s].pool_offset < 0 ||
            (int64_t)segs[s].pool_offset + segs[s].length > pool_tokens)
          return fail(s);
        sum += segs[s].length;
      }
      if (sum != kb) return fail(b);
    }
    // no two non-empty segments may share a pool slot
    std::vector<std::pair<int64_t, int64_t>> iv;  // (start, segment index)
    iv.reserve((size_t)nseg);
    for (int64_t s = 0; s < nseg; ++s)
      if (segs[s].length > 0) iv.emplace_back(segs[s].pool_offset, s);
    std::sort(iv.begin(), iv.end());
    for (size_t i = 1; i < iv.size(); ++i) {
      const auto& prev = segs[iv[i - 1].second];
      if ((int64_t)prev.pool_offset + prev.length > iv[i].first) return fail(iv[i].second);
    }
    if (bad_index) *bad_index = -1;
    return SEG_ATTN_OK;
  } catch (...) {
    return SEG_ATTN_ERR_HIP;
  }
}

}  // extern "C"
