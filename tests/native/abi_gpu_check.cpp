// The library used from C++ through include/seg_attn.h alone (no Python): device buffers from
// hipMalloc, then prefill, decode and the allocation-free decode on a small segmented workload.
// Checks results that are exact whatever the rounding order, and the argument errors the ABI
// promises to report before launching anything:
//   - a query row that sees one key returns that key's V row bit for bit (probability 1);
//   - its LSE is scale * q.k (a single term);
//   - decode of a request's last query equals prefill's last row of it (both see every key);
//   - seg_attn_decode and seg_attn_decode_noalloc agree bit for bit;
//   - bad arguments return their status and leave the output untouched.
//
//   abi_gpu_check        exit status 0 when every check held; a failed check prints it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <cstdint>
#include <vector>

#include "seg_attn.h"

namespace {

constexpr int kHq = 64, kHkv = 8, kD = 128;

int failures = 0;
void check(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "check failed: %s\n", what);
    ++failures;
  }
}

uint16_t to_bf16(float f) {  // round to nearest even
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFF + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

struct Lcg {  // seeded values in [-2, 2)
  uint64_t s;
  float next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((s >> 40) & 0xFFFFFF) / (float)(1 << 24) * 4.0f - 2.0f;
  }
};

template <class T>
T* dev_copy(const std::vector<T>& h) {
  T* d = nullptr;
  if (hipMalloc((void**)&d, h.size() * sizeof(T)) != hipSuccess) return nullptr;
  if (hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice) != hipSuccess) return nullptr;
  return d;
}
template <class T>
std::vector<T> host_copy(const T* d, size_t n) {
  std::vector<T> h(n);
  if (hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost) != hipSuccess) h.clear();
  return h;
}

}  // namespace

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
    printf("no GPU\n");
    return 2;
  }
  // Three requests: 40 queries on 40 keys in 3 segments; 1 query on 1 key; a chunk of 5
  // queries at the end of 300 keys in 2 segments. Segments sit out of order in the pool.
  const int pool = 1024;
  const std::vector<int32_t> cu_q = {0, 40, 41, 46}, cu_k = {0, 40, 41, 341};
  const std::vector<seg_attn_segment_t> segs = {{700, 10}, {100, 25}, {500, 5},  // request 0
                                                {999, 1},                         // request 1
                                                {200, 250}, {40, 50}};            // request 2
  const std::vector<int32_t> seg_indptr = {0, 3, 4, 6};
  const int batch = 3, total_q = 46;
  const float scale = 1.0f / sqrtf((float)kD);

  Lcg rng{12345};
  std::vector<uint16_t> q((size_t)total_q * kHq * kD), kp((size_t)pool * kHkv * kD), vp(kp.size());
  for (auto& x : q) x = to_bf16(rng.next());
  for (auto& x : kp) x = to_bf16(rng.next());
  for (auto& x : vp) x = to_bf16(rng.next());

  uint16_t* d_q = dev_copy(q);
  uint16_t* d_k = dev_copy(kp);
  uint16_t* d_v = dev_copy(vp);
  seg_attn_segment_t* d_segs = dev_copy(segs);
  int32_t* d_ind = dev_copy(seg_indptr);
  int32_t* d_cq = dev_copy(cu_q);
  int32_t* d_ck = dev_copy(cu_k);
  uint16_t* d_out = nullptr;
  float* d_lse = nullptr;
  check(hipMalloc((void**)&d_out, q.size() * 2) == hipSuccess, "hipMalloc out");
  check(hipMalloc((void**)&d_lse, (size_t)total_q * kHq * 4) == hipSuccess, "hipMalloc lse");
  if (!d_q || !d_k || !d_v || !d_segs || !d_ind || !d_cq || !d_ck || !d_out || !d_lse) {
    fprintf(stderr, "device allocation failed\n");
    return 1;
  }

  // ---- prefill
  seg_attn_status_t st = seg_attn_prefill(d_q, d_k, d_v, d_segs, d_ind, d_cq, d_ck, batch, 40, 300, kHq,
                                          kHkv, kD, pool, scale, 1, d_out, d_lse, nullptr);
  check(st == SEG_ATTN_OK, "prefill status");
  check(hipDeviceSynchronize() == hipSuccess, "prefill ran");
  const std::vector<uint16_t> out = host_copy(d_out, q.size());
  const std::vector<float> lse = host_copy(d_lse, (size_t)total_q * kHq);
  if (out.size() != q.size() || lse.size() != (size_t)total_q * kHq) {
    fprintf(stderr, "copy back failed\n");
    return 1;
  }
  // rows that see exactly one key: request 0's first query (key 0 = slot 700), request 1's
  // only query (slot 999)
  const int one_key_rows[2] = {0, 40}, one_key_slot[2] = {700, 999};
  for (int r = 0; r < 2; ++r) {
    const int row = one_key_rows[r], slot = one_key_slot[r];
    for (int h = 0; h < kHq; ++h) {
      const int g = h / (kHq / kHkv);
      const uint16_t* o = &out[((size_t)row * kHq + h) * kD];
      const uint16_t* v = &vp[((size_t)slot * kHkv + g) * kD];
      check(memcmp(o, v, kD * 2) == 0, "one-key row equals its key's V row");
      double dot = 0;
      for (int d = 0; d < kD; ++d)
        dot += (double)from_bf16(q[((size_t)row * kHq + h) * kD + d]) *
               (double)from_bf16(kp[((size_t)slot * kHkv + g) * kD + d]);
      check(fabs(lse[(size_t)row * kHq + h] - dot * scale) <= 1e-3 * (1.0 + fabs(dot * scale)),
            "one-key row's LSE is scale * q.k");
    }
  }

  // ---- decode of each request's last query against all of its keys
  std::vector<uint16_t> qd((size_t)batch * kHq * kD);
  for (int b = 0; b < batch; ++b)
    memcpy(&qd[(size_t)b * kHq * kD], &q[(size_t)(cu_q[b + 1] - 1) * kHq * kD], (size_t)kHq * kD * 2);
  uint16_t* d_qd = dev_copy(qd);
  uint16_t *d_od = nullptr, *d_od2 = nullptr;
  check(hipMalloc((void**)&d_od, qd.size() * 2) == hipSuccess, "hipMalloc decode out");
  check(hipMalloc((void**)&d_od2, qd.size() * 2) == hipSuccess, "hipMalloc decode out 2");
  const size_t ws_bytes = seg_attn_decode_workspace_bytes(batch, 300, kHq, kHkv, kD, SEG_ATTN_KV_BF16, 0);
  check(ws_bytes > 0, "decode workspace size");
  void* d_ws = nullptr;
  check(hipMalloc(&d_ws, ws_bytes) == hipSuccess, "hipMalloc workspace");
  if (!d_qd || !d_od || !d_od2 || !d_ws) {
    fprintf(stderr, "device allocation failed\n");
    return 1;
  }
  st = seg_attn_decode(d_qd, d_k, d_v, nullptr, nullptr, SEG_ATTN_KV_BF16, d_segs, d_ind, d_ck, batch, 300, kHq,
                       kHkv, kD, pool, scale, 0, d_od, nullptr, d_ws, ws_bytes, nullptr);
  check(st == SEG_ATTN_OK, "decode status");
  st = seg_attn_decode_noalloc(d_qd, d_k, d_v, nullptr, nullptr, SEG_ATTN_KV_BF16, d_segs, d_ind, d_ck, batch,
                               300, kHq, kHkv, kD, pool, scale, 0, d_od2, nullptr, nullptr);
  check(st == SEG_ATTN_OK, "decode_noalloc status");
  check(hipDeviceSynchronize() == hipSuccess, "decode ran");
  const std::vector<uint16_t> od = host_copy(d_od, qd.size()), od2 = host_copy(d_od2, qd.size());
  if (od.size() != qd.size() || od2.size() != qd.size()) {
    fprintf(stderr, "copy back failed\n");
    return 1;
  }
  check(od == od2, "decode and decode_noalloc agree bit for bit");
  double worst = 0;
  for (int b = 0; b < batch; ++b)
    for (int i = 0; i < kHq * kD; ++i) {
      const double a = from_bf16(od[(size_t)b * kHq * kD + i]);
      const double p = from_bf16(out[(size_t)(cu_q[b + 1] - 1) * kHq * kD + i]);
      worst = fmax(worst, fabs(a - p));
    }
  check(worst <= 1e-2, "decode equals prefill's last rows");

  // ---- argument errors: reported before any launch, the output left as it was
  std::vector<uint16_t> sentinel(qd.size(), 0x7FC1);
  check(hipMemcpy(d_od, sentinel.data(), sentinel.size() * 2, hipMemcpyHostToDevice) == hipSuccess, "sentinel");
  check(seg_attn_prefill(d_q, d_k, d_v, d_segs, d_ind, d_cq, d_ck, batch, 40, 300, kHq, kHkv, 64, pool, scale, 1,
                         d_out, nullptr, nullptr) == SEG_ATTN_ERR_UNSUPPORTED,
        "head_dim 64 is unsupported");
  check(seg_attn_prefill(nullptr, d_k, d_v, d_segs, d_ind, d_cq, d_ck, batch, 40, 300, kHq, kHkv, kD, pool,
                         scale, 1, d_out, nullptr, nullptr) == SEG_ATTN_ERR_INVALID_ARG,
        "null q is refused");
  check(seg_attn_prefill(d_q, d_k, d_v, d_segs, d_ind, d_cq, d_ck, batch, 40, 300, kHq, kHkv, kD, pool, scale, 1,
                         (char*)d_out + 2, nullptr, nullptr) == SEG_ATTN_ERR_INVALID_ARG,
        "misaligned out is refused");
  check(seg_attn_decode(d_qd, d_k, d_v, nullptr, nullptr, SEG_ATTN_KV_BF16, d_segs, d_ind, d_ck, batch, 300, kHq,
                        kHkv, kD, pool, scale, 0, d_od, nullptr, d_ws, ws_bytes - 16, nullptr) ==
            SEG_ATTN_ERR_WORKSPACE,
        "a short workspace is refused");
  check(seg_attn_decode(d_qd, d_k, d_v, nullptr, nullptr, 9, d_segs, d_ind, d_ck, batch, 300, kHq, kHkv, kD, pool,
                        scale, 0, d_od, nullptr, d_ws, ws_bytes, nullptr) == SEG_ATTN_ERR_INVALID_ARG,
        "an unknown kv dtype is refused");
  check(hipDeviceSynchronize() == hipSuccess, "sync after refusals");
  check(host_copy(d_od, sentinel.size()) == sentinel, "refused calls left the output untouched");
  check(strlen(seg_attn_status_string(SEG_ATTN_ERR_WORKSPACE)) > 0, "status string");

  for (void* p : {(void*)d_q, (void*)d_k, (void*)d_v, (void*)d_segs, (void*)d_ind, (void*)d_cq, (void*)d_ck,
                  (void*)d_out, (void*)d_lse, (void*)d_qd, (void*)d_od, (void*)d_od2, d_ws})
    check(hipFree(p) == hipSuccess, "hipFree");
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("ok (decode vs prefill max abs %.3g)\n", worst);
  return 0;
}
