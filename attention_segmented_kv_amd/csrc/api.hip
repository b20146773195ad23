// C ABI of the segment-attention library: argument checks, split planning, launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/seg_attn.h"

#ifdef SEG_ATTN_DEBUG
constexpr bool kDebugBuild = true;
#else
constexpr bool kDebugBuild = false;
#endif

namespace segattn {
hipError_t launch_prefill(const void* q, const void* k_pool, const void* v_pool, const void* segs,
                          const int32_t* seg_indptr, const int32_t* cu_q, const int32_t* cu_k,
                          int batch, int max_seqlen_q, int hkv, int64_t pool_size, float scale, int causal,
                          void* out, float* lse, int cu_count, int force_tile, hipStream_t stream);
hipError_t launch_decode(const void* q, const void* k_pool, const void* v_pool,
                         const float* k_scale, const float* v_scale, int kv, const void* segs,
                         const int32_t* seg_indptr, const int32_t* cu_k, int batch, int hkv,
                         int max_k, int forced_len, int min_len, int max_chunks, int cu_count,
                         float scale, void* out, float* lse, int32_t* hdr, int32_t* chunk_base,
                         int32_t* recs, float* ws_o, float* ws_lse, hipStream_t stream);
hipError_t launch_kv_append(const void* k_new, const void* v_new, const void* segs,
                            const int32_t* seg_indptr, const int32_t* cu_new, const int32_t* cu_k,
                            int batch, int total_new, int hkv, int64_t pool_tokens, int fmt,
                            void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                            hipStream_t stream);
hipError_t launch_kv_move(const void* moves, int n_moves, int64_t total_tokens, int hkv,
                          int64_t pool_tokens, int fmt, void* k_pool, void* v_pool, float* k_scale,
                          float* v_scale, hipStream_t stream);
hipError_t launch_linear_prefill(const void* q, const void* k, const void* v, const float* g,
                                 const int32_t* cu, const int32_t* slots, int batch, int heads,
                                 float scale, int initial_state, float* pool, int64_t pool_slots,
                                 void* out, hipStream_t stream);
int linear_fused_max_len();
hipError_t launch_linear_prefill_fused(const void* q, const void* k, const void* v, const float* g,
                                       const int32_t* cu, const int32_t* slots, int batch, int heads,
                                       int max_len, float scale, int initial_state, float* pool,
                                       int64_t pool_slots, void* out, hipStream_t stream);
hipError_t launch_linear_decode(const void* q, const void* k, const void* v, const float* g,
                                const int32_t* slots, int batch, int heads, float scale, float* pool,
                                int64_t pool_slots, void* out, hipStream_t stream);
size_t linear_prefill_ws(int64_t batch, int64_t maxc, int64_t heads, size_t* off);
int64_t decode_auto_chunk_bound(int64_t batch, int hkv, int cu_count);
hipError_t launch_linear_prefill_parallel(const void* q, const void* k, const void* v, const float* g,
                                          const int32_t* cu, const int32_t* slots, int batch, int heads,
                                          int maxc, float scale, int initial_state, float* pool,
                                          int64_t pool_slots, void* out, void* ws, hipStream_t stream);
}  // namespace segattn

namespace {

constexpr int kHeadDim = 128;
constexpr int kGroup = 8;
constexpr int kMaxDevices = 64;
constexpr int kChunkGranule = 64;  // decode chunk lengths are multiples of this many keys

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

bool valid_kv_dtype(int32_t kv) {
  return kv == SEG_ATTN_KV_BF16 || kv == SEG_ATTN_KV_FP8_E4M3 || kv == SEG_ATTN_KV_INT8;
}

// Decode chunk plan. Each request's keys are cut into chunks of one length; a chunk times a kv
// head is one work unit of the split pass. With num_splits > 0 the length is fixed here:
// ceil(max_k / num_splits) rounded up to a multiple of 64, so no request has more than
// num_splits chunks. With 0 the device picks the length from the total key count (so that every
// compute unit gets about a dozen units), never below kMinChunk keys, which bounds the chunks per
// request by ceil(max_k / kMinChunk).
struct DecodePlan {
  int forced_len;        // 0: chosen on the device
  int min_len;           // lower bound of the length
  int64_t per_request;   // upper bound of the chunks of one request
};

bool plan_decode(int batch, int max_k, int one_byte, int requested, DecodePlan* p) {
  if (batch < 0 || max_k < 0 || requested < 0) return false;
  const int min_chunk = one_byte ? 1024 : 512;
  if (requested > 0) {
    const int64_t len = std::max<int64_t>(kChunkGranule, ceil_div(ceil_div(max_k, requested), kChunkGranule) * kChunkGranule);
    p->forced_len = (int)len;
    p->min_len = (int)len;
    p->per_request = std::max<int64_t>(1, ceil_div(max_k, len));
  } else {
    p->forced_len = 0;
    p->min_len = min_chunk;
    p->per_request = std::max<int64_t>(1, ceil_div(max_k, min_chunk));
  }
  return true;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// SEG_ATTN_LINEAR_PREFILL=chunked keeps the chunk-parallel linear prefill for short requests too
// (tests use it to cover both paths); =fused, or unset, takes the closed form up to its length.
bool linear_chunked_forced() {
  const char* v = std::getenv("SEG_ATTN_LINEAR_PREFILL");
  return v != nullptr && std::strcmp(v, "chunked") == 0;
}

// SEG_ATTN_PREFILL_TILE=128 or 256 pins the prefill tiling (tests use it to cover both).
int prefill_tile_override() {
  const char* v = std::getenv("SEG_ATTN_PREFILL_TILE");
  if (v == nullptr) return 0;
  const int t = std::atoi(v);
  return (t == 128 || t == 256) ? t : 0;
}

// Decode workspace: [0, 256) plan header, then chunk offsets [batch + 1] int32, the chunk
// records [max_chunks] x 16 int32, the partial LSEs [max_chunks][Hq] fp32 and the partial
// outputs [max_chunks][Hq][128] fp32, each part 256-byte aligned.
struct DecodeWs {
  size_t base, tab, lse, o, total;
};
DecodeWs decode_ws_layout(int64_t batch, int64_t hq, int64_t max_chunks) {
  DecodeWs w;
  w.base = 256;
  w.tab = w.base + align_up((size_t)(batch + 1) * 4, 256);
  w.lse = w.tab + align_up((size_t)max_chunks * 64, 256);
  w.o = w.lse + align_up((size_t)(max_chunks * hq) * 4, 256);
  w.total = w.o + (size_t)(max_chunks * hq) * kHeadDim * 4;
  return w;
}

// True when p is not a multiple of a (a power of two); NULL counts as aligned.
bool misaligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; }

seg_attn_status_t check_heads(int32_t hq, int32_t hkv, int32_t head_dim) {
  if (hq <= 0 || hkv <= 0 || head_dim <= 0) return SEG_ATTN_ERR_INVALID_ARG;
  if (hq % hkv != 0) return SEG_ATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || hq / hkv != kGroup) return SEG_ATTN_ERR_UNSUPPORTED;
  return SEG_ATTN_OK;
}

seg_attn_status_t check_tables(const seg_attn_segment_t* segs, int64_t nseg,
                                           const int32_t* seg_indptr,
                                           const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_k, int32_t batch,
                                           int64_t pool_tokens, int32_t causal,
                                           int64_t* bad_index, bool disjoint) {
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
    if (!disjoint) {
      if (bad_index) *bad_index = -1;
      return SEG_ATTN_OK;
    }
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

// Debug builds (SEG_ATTN_DEBUG) check the device tables on the host before every attention
// launch: the stream is synchronised, the tables are copied back and checked as
// seg_attn_validate_tables does, except that segments of different requests may share slots
// (attention only reads them); a call on broken tables returns SEG_ATTN_ERR_TABLE and launches
// nothing, so every pool slot a kernel resolves lies inside [0, pool_tokens).
seg_attn_status_t debug_check_tables(const seg_attn_segment_t* segs, const int32_t* seg_indptr,
                                     const int32_t* cu_q, const int32_t* cu_k, int32_t batch,
                                     int64_t pool_tokens, int32_t causal, hipStream_t stream) {
  if (!kDebugBuild) return SEG_ATTN_OK;
  if (hipStreamSynchronize(stream) != hipSuccess) return SEG_ATTN_ERR_HIP;
  const size_t nb = (size_t)batch + 1;
  std::vector<int32_t> ind(nb), ck(nb), cq(cu_q ? nb : 0);
  if (hipMemcpy(ind.data(), seg_indptr, nb * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(ck.data(), cu_k, nb * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      (cu_q && hipMemcpy(cq.data(), cu_q, nb * 4, hipMemcpyDeviceToHost) != hipSuccess))
    return SEG_ATTN_ERR_HIP;
  const int64_t nseg = ind[batch];
  if (nseg < 0 || nseg > (int64_t)1 << 30) return SEG_ATTN_ERR_TABLE;
  std::vector<seg_attn_segment_t> sg((size_t)nseg);
  if (nseg > 0 && hipMemcpy(sg.data(), segs, (size_t)nseg * sizeof(seg_attn_segment_t), hipMemcpyDeviceToHost) != hipSuccess)
    return SEG_ATTN_ERR_HIP;
  return check_tables(sg.data(), nseg, ind.data(), cu_q ? cq.data() : nullptr, ck.data(), batch, pool_tokens,
                      causal, nullptr, false);
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
    case SEG_ATTN_ERR_OUT_OF_MEMORY: return "not enough free pool slots (or host memory)";
    case SEG_ATTN_ERR_SCRATCH: return "call needs more than the fixed scratch of seg_attn_decode_noalloc";
    default: return "unknown status";
  }
}

int32_t seg_attn_debug_build(void) { return kDebugBuild ? 1 : 0; }

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
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return SEG_ATTN_ERR_INVALID_ARG;
    seg_attn_status_t hs = check_heads(num_heads_q, num_heads_kv, head_dim);
    if (hs != SEG_ATTN_OK) return hs;
    if (causal && max_seqlen_q > max_seqlen_k) return SEG_ATTN_ERR_INVALID_ARG;
    if (pool_tokens > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
    if (batch == 0 || max_seqlen_q == 0) return SEG_ATTN_OK;
    if (!q || !k_pool || !v_pool || !segs || !seg_indptr || !cu_seqlens_q || !cu_seqlens_k || !out)
      return SEG_ATTN_ERR_INVALID_ARG;
    // 16-byte loads and HBM->LDS copies of Q, K, V rows and 16-byte stores of output rows;
    // 8-byte segment records; 4-byte table entries and LSE values
    if (misaligned(q, 16) || misaligned(k_pool, 16) || misaligned(v_pool, 16) || misaligned(out, 16) ||
        misaligned(segs, 8) || misaligned(seg_indptr, 4) || misaligned(cu_seqlens_q, 4) ||
        misaligned(cu_seqlens_k, 4) || misaligned(lse, 4))
      return SEG_ATTN_ERR_INVALID_ARG;
    const int64_t grid = ceil_div(max_seqlen_q, 16) * (int64_t)num_heads_kv * batch;
    if (grid > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
    const seg_attn_status_t ts = debug_check_tables(segs, seg_indptr, cu_seqlens_q, cu_seqlens_k, batch,
                                                    pool_tokens, causal, (hipStream_t)stream);
    if (ts != SEG_ATTN_OK) return ts;
    hipError_t e = segattn::launch_prefill(q, k_pool, v_pool, segs, seg_indptr, cu_seqlens_q,
                                           cu_seqlens_k, batch, max_seqlen_q, num_heads_kv, pool_tokens,
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
    if (!valid_kv_dtype(kv_dtype)) return -1;
    if (num_heads_kv <= 0) return -1;
    DecodePlan p;
    if (!plan_decode(batch, max_seqlen_k, kv_dtype != SEG_ATTN_KV_BF16, num_splits, &p)) return -1;
    if (p.per_request > INT32_MAX) return -1;
    if (split_len) *split_len = p.min_len;
    return (int32_t)p.per_request;
  } catch (...) {
    return -1;
  }
}

size_t seg_attn_decode_workspace_bytes(int32_t batch, int32_t max_seqlen_k, int32_t num_heads_q,
                                       int32_t num_heads_kv, int32_t head_dim, int32_t kv_dtype,
                                       int32_t num_splits) {
  try {
    if (check_heads(num_heads_q, num_heads_kv, head_dim) != SEG_ATTN_OK) return 0;
    if (!valid_kv_dtype(kv_dtype)) return 0;
    DecodePlan p;
    if (!plan_decode(batch, max_seqlen_k, kv_dtype != SEG_ATTN_KV_BF16, num_splits, &p)) return 0;
    return decode_ws_layout(batch, num_heads_q, p.per_request * batch).total;
  } catch (...) {
    return 0;
  }
}

}  // extern "C"

namespace {

// Scratch of seg_attn_decode_noalloc: the decode workspace (plan and partial results) in a
// fixed array of every GPU the library runs on, held until the process ends. Host code never
// uses the array's name as an address (in host code it is only a stand-in): its device address
// is looked up once per device, with that device current, and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) char scratch[kScratchBytes];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of the current device's scratch array (nullptr and the HIP error on failure).
void* current_scratch(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev]() {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

// Shared body of the two decode entry points. noalloc: the workspace is the scratch array and
// the automatic plan's chunk count is bounded by decode_auto_chunk_bound instead of the per-request
// worst case, which keeps it small.
seg_attn_status_t decode_impl(const void* q, const void* k_pool, const void* v_pool,
                              const float* k_scale, const float* v_scale, int32_t kv_dtype,
                              const seg_attn_segment_t* segs, const int32_t* seg_indptr,
                              const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen_k,
                              int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                              int64_t pool_tokens, float softmax_scale, int32_t num_splits, void* out,
                              float* lse, void* workspace, size_t workspace_bytes, bool noalloc,
                              hipStream_t stream) {
  if (batch < 0 || max_seqlen_k < 0 || pool_tokens < 0 || num_splits < 0) return SEG_ATTN_ERR_INVALID_ARG;
  if (!valid_kv_dtype(kv_dtype)) return SEG_ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f)) return SEG_ATTN_ERR_INVALID_ARG;
  seg_attn_status_t hs = check_heads(num_heads_q, num_heads_kv, head_dim);
  if (hs != SEG_ATTN_OK) return hs;
  if (pool_tokens > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
  if (batch == 0) return SEG_ATTN_OK;
  const bool scaled = kv_dtype != SEG_ATTN_KV_BF16;  // FP8 or INT8 codes with fp32 scales
  if (!q || !k_pool || !v_pool || !segs || !seg_indptr || !cu_seqlens_k || !out) return SEG_ATTN_ERR_INVALID_ARG;
  if (scaled && (!k_scale || !v_scale)) return SEG_ATTN_ERR_INVALID_ARG;
  // 16-byte HBM->LDS copies of Q rows and pool rows, 4-byte scale copies, 8-byte output
  // stores, 16-byte workspace records and partials
  if (misaligned(q, 16) || misaligned(k_pool, 16) || misaligned(v_pool, 16) || misaligned(out, 8) ||
      misaligned(segs, 8) || misaligned(seg_indptr, 4) || misaligned(cu_seqlens_k, 4) ||
      misaligned(lse, 4) || (scaled && (misaligned(k_scale, 4) || misaligned(v_scale, 4))))
    return SEG_ATTN_ERR_INVALID_ARG;
  DecodePlan p;
  if (!plan_decode(batch, max_seqlen_k, scaled, num_splits, &p)) return SEG_ATTN_ERR_INVALID_ARG;
  {
    const seg_attn_status_t ts = debug_check_tables(segs, seg_indptr, nullptr, cu_seqlens_k, batch, pool_tokens,
                                                    0, stream);
    if (ts != SEG_ATTN_OK) return ts;
  }
  int64_t max_chunks = p.per_request * batch;
  int cu_count = 0;  // read from the device only once the call is going to launch
  if (noalloc && num_splits == 0) {
    cu_count = current_cu_count();
    max_chunks = std::min<int64_t>(max_chunks, segattn::decode_auto_chunk_bound(batch, num_heads_kv, cu_count));
  }
  if (max_chunks * num_heads_kv > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
  const DecodeWs lay = decode_ws_layout(batch, num_heads_q, max_chunks);
  if (noalloc) {
    if (lay.total > kScratchBytes) return SEG_ATTN_ERR_SCRATCH;
    hipError_t e = hipSuccess;
    workspace = current_scratch(&e);
    if (workspace == nullptr) return SEG_ATTN_ERR_HIP;
    workspace_bytes = kScratchBytes;
  }
  if (misaligned(workspace, 16)) return SEG_ATTN_ERR_WORKSPACE;
  if (workspace == nullptr || workspace_bytes < lay.total) return SEG_ATTN_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  if (cu_count == 0) cu_count = current_cu_count();
  hipError_t e = segattn::launch_decode(
      q, k_pool, v_pool, k_scale, v_scale, kv_dtype, segs, seg_indptr, cu_seqlens_k, batch,
      num_heads_kv, max_seqlen_k, p.forced_len, p.min_len, (int)max_chunks, cu_count, softmax_scale,
      out, lse, (int32_t*)ws, (int32_t*)(ws + lay.base), (int32_t*)(ws + lay.tab), (float*)(ws + lay.o),
      (float*)(ws + lay.lse), stream);
  return e == hipSuccess ? SEG_ATTN_OK : SEG_ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

seg_attn_status_t seg_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                                  const float* k_scale, const float* v_scale, int32_t kv_dtype,
                                  const seg_attn_segment_t* segs, const int32_t* seg_indptr,
                                  const int32_t* cu_seqlens_k, int32_t batch,
                                  int32_t max_seqlen_k, int32_t num_heads_q, int32_t num_heads_kv,
                                  int32_t head_dim, int64_t pool_tokens, float softmax_scale,
                                  int32_t num_splits, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, seg_attn_stream_t stream) {
  try {
    return decode_impl(q, k_pool, v_pool, k_scale, v_scale, kv_dtype, segs, seg_indptr, cu_seqlens_k,
                       batch, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, pool_tokens,
                       softmax_scale, num_splits, out, lse, workspace, workspace_bytes, false,
                       (hipStream_t)stream);
  } catch (...) {
    return SEG_ATTN_ERR_HIP;
  }
}

seg_attn_status_t seg_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                          const float* k_scale, const float* v_scale,
                                          int32_t kv_dtype, const seg_attn_segment_t* segs,
                                          const int32_t* seg_indptr, const int32_t* cu_seqlens_k,
                                          int32_t batch, int32_t max_seqlen_k, int32_t num_heads_q,
                                          int32_t num_heads_kv, int32_t head_dim,
                                          int64_t pool_tokens, float softmax_scale,
                                          int32_t num_splits, void* out, float* lse,
                                          seg_attn_stream_t stream) {
  try {
    return decode_impl(q, k_pool, v_pool, k_scale, v_scale, kv_dtype, segs, seg_indptr, cu_seqlens_k,
                       batch, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, pool_tokens,
                       softmax_scale, num_splits, out, lse, nullptr, 0, true, (hipStream_t)stream);
  } catch (...) {
    return SEG_ATTN_ERR_HIP;
  }
}

seg_attn_status_t seg_attn_kv_append(const void* k_new, const void* v_new,
                                     const seg_attn_segment_t* segs, const int32_t* seg_indptr,
                                     const int32_t* cu_seqlens_new, const int32_t* cu_seqlens_k,
                                     int32_t batch, int32_t total_new, int32_t num_heads_kv,
                                     int32_t head_dim, int64_t pool_tokens, int32_t kv_dtype,
                                     void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                     seg_attn_stream_t stream) {
  try {
    if (batch < 0 || total_new < 0 || pool_tokens < 0 || num_heads_kv <= 0 || head_dim <= 0)
      return SEG_ATTN_ERR_INVALID_ARG;
    if (!valid_kv_dtype(kv_dtype)) return SEG_ATTN_ERR_INVALID_ARG;
    if (head_dim != kHeadDim) return SEG_ATTN_ERR_UNSUPPORTED;
    if (pool_tokens > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
    if (batch == 0 && total_new > 0) return SEG_ATTN_ERR_INVALID_ARG;
    if (batch == 0 || total_new == 0) return SEG_ATTN_OK;
    const bool scaled = kv_dtype != SEG_ATTN_KV_BF16;  // FP8 or INT8 codes with fp32 scales
    if (!k_new || !v_new || !segs || !seg_indptr || !cu_seqlens_new || !cu_seqlens_k || !k_pool || !v_pool)
      return SEG_ATTN_ERR_INVALID_ARG;
    if (scaled && (!k_scale || !v_scale)) return SEG_ATTN_ERR_INVALID_ARG;
    // rows move as 16-byte (bf16) or 8-byte (one-byte codes) pieces, scales as 4-byte words
    if (misaligned(k_new, 16) || misaligned(v_new, 16) || misaligned(k_pool, scaled ? 8 : 16) ||
        misaligned(v_pool, scaled ? 8 : 16) || (scaled && (misaligned(k_scale, 4) || misaligned(v_scale, 4))))
      return SEG_ATTN_ERR_INVALID_ARG;
    if ((int64_t)total_new * num_heads_kv > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
    hipError_t e = segattn::launch_kv_append(k_new, v_new, segs, seg_indptr, cu_seqlens_new,
                                             cu_seqlens_k, batch, total_new, num_heads_kv,
                                             pool_tokens, kv_dtype, k_pool, v_pool, k_scale,
                                             v_scale, (hipStream_t)stream);
    return e == hipSuccess ? SEG_ATTN_OK : SEG_ATTN_ERR_HIP;
  } catch (...) {
    return SEG_ATTN_ERR_HIP;
  }
}

seg_attn_status_t seg_attn_kv_move(const seg_attn_move_t* moves, int32_t n_moves,
                                   int64_t total_tokens, int32_t num_heads_kv, int32_t head_dim,
                                   int64_t pool_tokens, int32_t kv_dtype, void* k_pool,
                                   void* v_pool, float* k_scale, float* v_scale,
                                   seg_attn_stream_t stream) {
  try {
    if (n_moves < 0 || total_tokens < 0 || num_heads_kv <= 0 || head_dim <= 0 || pool_tokens < 0)
      return SEG_ATTN_ERR_INVALID_ARG;
    if (!valid_kv_dtype(kv_dtype)) return SEG_ATTN_ERR_INVALID_ARG;
    if (head_dim != kHeadDim) return SEG_ATTN_ERR_UNSUPPORTED;
    if (pool_tokens > INT32_MAX || total_tokens > pool_tokens) return SEG_ATTN_ERR_INVALID_ARG;
    if (n_moves == 0 || total_tokens == 0) return SEG_ATTN_OK;
    const bool scaled = kv_dtype != SEG_ATTN_KV_BF16;
    if (!moves || !k_pool || !v_pool || (scaled && (!k_scale || !v_scale))) return SEG_ATTN_ERR_INVALID_ARG;
    if (misaligned(moves, 16) || misaligned(k_pool, scaled ? 8 : 16) || misaligned(v_pool, scaled ? 8 : 16) ||
        (scaled && (misaligned(k_scale, 4) || misaligned(v_scale, 4))))
      return SEG_ATTN_ERR_INVALID_ARG;
    if (total_tokens * num_heads_kv / 16 + 1 > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
    hipError_t e = segattn::launch_kv_move(moves, n_moves, total_tokens, num_heads_kv, pool_tokens,
                                           kv_dtype, k_pool, v_pool, k_scale, v_scale,
                                           (hipStream_t)stream);
    return e == hipSuccess ? SEG_ATTN_OK : SEG_ATTN_ERR_HIP;
  } catch (...) {
    return SEG_ATTN_ERR_HIP;
  }
}

namespace {
// Shared argument checks of the two linear-attention entry points.
seg_attn_status_t check_linear(const void* q, const void* k, const void* v, const float* g,
                               const int32_t* slots, int32_t batch, int32_t heads, int32_t head_dim,
                               float scale, const float* pool, int64_t pool_slots, const void* out) {
  if (batch < 0 || heads <= 0 || head_dim <= 0 || pool_slots < 0) return SEG_ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return SEG_ATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return SEG_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)batch * heads * 2 > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
  if (batch == 0) return SEG_ATTN_OK;
  if (!q || !k || !v || !g || !slots || !pool || !out) return SEG_ATTN_ERR_INVALID_ARG;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(pool, 16) ||
      misaligned(out, 8) || misaligned(g, 4))
    return SEG_ATTN_ERR_INVALID_ARG;
  return SEG_ATTN_OK;
}
}  // namespace

size_t seg_attn_linear_prefill_workspace_bytes(int32_t batch, int32_t max_seqlen, int32_t num_heads,
                                               int32_t head_dim) {
  if (batch < 0 || max_seqlen < 0 || num_heads <= 0 || head_dim != kHeadDim) return 0;
  return segattn::linear_prefill_ws(batch, ((int64_t)max_seqlen + 63) / 64, num_heads, nullptr);
}

seg_attn_status_t seg_attn_linear_prefill(const void* q, const void* k, const void* v,
                                          const float* g, const int32_t* cu_seqlens,
                                          const int32_t* state_slots, int32_t batch,
                                          int32_t max_seqlen, int32_t num_heads, int32_t head_dim,
                                          float scale, int32_t initial_state, float* state_pool,
                                          int64_t pool_slots, void* out, void* workspace,
                                          size_t workspace_bytes, seg_attn_stream_t stream) {
  try {
    if (initial_state != 0 && initial_state != 1) return SEG_ATTN_ERR_INVALID_ARG;
    if (max_seqlen < 0) return SEG_ATTN_ERR_INVALID_ARG;
    seg_attn_status_t st = check_linear(q, k, v, g, state_slots, batch, num_heads, head_dim, scale,
                                        state_pool, pool_slots, out);
    if (st != SEG_ATTN_OK || batch == 0) return st;
    if (!cu_seqlens) return SEG_ATTN_ERR_INVALID_ARG;
    hipError_t e;
    if (workspace == nullptr) {
      e = segattn::launch_linear_prefill(q, k, v, g, cu_seqlens, state_slots, batch, num_heads, scale,
                                         initial_state, state_pool, pool_slots, out, (hipStream_t)stream);
    } else if (max_seqlen <= segattn::linear_fused_max_len() && !linear_chunked_forced()) {
      e = segattn::launch_linear_prefill_fused(q, k, v, g, cu_seqlens, state_slots, batch, num_heads,
                                               max_seqlen, scale, initial_state, state_pool, pool_slots,
                                               out, (hipStream_t)stream);
    } else {
      const int64_t maxc = ((int64_t)max_seqlen + 63) / 64;
      if ((int64_t)batch * maxc * num_heads * 2 > INT32_MAX) return SEG_ATTN_ERR_UNSUPPORTED;
      if (((uintptr_t)workspace & 255) != 0) return SEG_ATTN_ERR_INVALID_ARG;
      if (workspace_bytes < segattn::linear_prefill_ws(batch, maxc, num_heads, nullptr))
        return SEG_ATTN_ERR_WORKSPACE;
      e = segattn::launch_linear_prefill_parallel(q, k, v, g, cu_seqlens, state_slots, batch, num_heads,
                                                  (int)maxc, scale, initial_state, state_pool, pool_slots,
                                                  out, workspace, (hipStream_t)stream);
    }
    return e == hipSuccess ? SEG_ATTN_OK : SEG_ATTN_ERR_HIP;
  } catch (...) {
    return SEG_ATTN_ERR_HIP;
  }
}

seg_attn_status_t seg_attn_linear_decode(const void* q, const void* k, const void* v, const float* g,
                                         const int32_t* state_slots, int32_t batch,
                                         int32_t num_heads, int32_t head_dim, float scale,
                                         float* state_pool, int64_t pool_slots, void* out,
                                         seg_attn_stream_t stream) {
  try {
    seg_attn_status_t st = check_linear(q, k, v, g, state_slots, batch, num_heads, head_dim, scale,
                                        state_pool, pool_slots, out);
    if (st != SEG_ATTN_OK || batch == 0) return st;
    hipError_t e = segattn::launch_linear_decode(q, k, v, g, state_slots, batch, num_heads, scale,
                                                 state_pool, pool_slots, out, (hipStream_t)stream);
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
  return check_tables(segs, nseg, seg_indptr, cu_seqlens_q, cu_seqlens_k, batch, pool_tokens, causal,
                      bad_index, true);
}

}  // extern "C"
