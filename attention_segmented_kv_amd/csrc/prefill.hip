// Prefill kernel: GQA attention of query chunks against KV gathered from pool segments.
//
// One workgroup (4 waves) owns one tile of 128 rows: 16 consecutive query positions of one
// request times the 8 query heads that share kv head g ("PackGQA" memory access, FlashPrefill
// V2 abstract): every K/V byte staged into LDS serves all 8 heads of its group. Keys stream
// through LDS in blocks of 64, double-buffered (the double-buffering of "FlashAttention on
// Ascend NPU", optimisation 1): block t+1 is copied from HBM straight into LDS while block t is
// consumed. Each key row of a block is looked up in the request's segment table, so a block
// may span any number of segments at any offsets (Flood README, "Introduction": segmentable
// KV cache).
//
// Per wave (32 rows = 4 positions x 8 heads) and key block, all matrix work is MFMA
// 32x32x16 bf16:
//   S^T[key][row] = K Q^T     keys on the M side, so each lane holds 32 scores of one row
//                             and the row max needs a single cross-lane step (permlane32);
//   O^T[d][row]  += V^T P^T   V^T comes from row-major V in LDS via the transposing read.
// The softmax is the online one: running max m and normaliser l per row, rescaling O by
// exp(m_old - m_new) whenever the max grows ("FlashAttention on Ascend NPU", bottleneck 2).
#include "common.hpp"

namespace segattn {

namespace {

constexpr int kBlockN = 64;      // keys per block
constexpr int kRowsPerWave = 32;
constexpr int kWaves = 4;
constexpr int kPosPerTile = kWaves * kRowsPerWave / kGroup;  // 16 query positions
constexpr int kKBufBytes = kBlockN * kHeadDim * 2;            // 16 KiB
constexpr int kLdsBytes = 4 * kKBufBytes;                      // K x2 + V x2

// LDS layouts (row = key within the block, 256 B = 16 chunks of 16 B per row):
//   K: chunk c of row r is stored at chunk position c ^ (r % 16)
//   V: chunk c of row r is stored at chunk position c ^ vswz(r)
// K is read 16 B per lane for 32 consecutive rows, V with the transposing read over groups
// of 4 consecutive rows; these swizzles keep both free of bank conflicts.
__device__ __forceinline__ int vswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

template <bool kCausal>
__global__ __launch_bounds__(256, 2) void prefill_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_pool,
    const bf16_t* __restrict__ v_pool, const Segment* __restrict__ segs,
    const int32_t* __restrict__ seg_indptr, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int batch, int hkv, int n_qtiles, float scale,
    float scale_log2, bf16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  // Work item. Heaviest (last) query tiles first; kv head fastest so that, with 8 kv heads,
  // every tile of head g lands on the same XCD (workgroups are dealt round-robin over 8 XCDs)
  // and shares its L2.
  const int id = blockIdx.x;
  const int per_tile = hkv * batch;
  const int qtile = n_qtiles - 1 - id / per_tile;
  const int rem = id % per_tile;
  const int b = rem / hkv;
  const int g = rem % hkv;

  const int q0 = cu_q[b];
  const int lq = cu_q[b + 1] - q0;
  const int p0 = qtile * kPosPerTile;
  if (p0 >= lq) return;
  const int K = cu_k[b + 1] - cu_k[b];
  const int hq = hkv * kGroup;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;  // row within the wave
  const int h = lane >> 5;  // which half of the k / m slots this lane holds
  const int pos = p0 + wave * 4 + (n >> 3);
  const int head = g * kGroup + (n & 7);
  const bool row_valid = pos < lq;

  // Keys this tile can see at all, and from which key on masking is needed.
  const int last_pos = min(p0 + kPosPerTile - 1, lq - 1);
  const int kend = kCausal ? min(K, K - lq + last_pos + 1) : K;
  const int kfull = kCausal ? min(K, K - lq + p0 + 1) : K;  // every row sees keys < kfull
  const int n_blocks = (kend + kBlockN - 1) / kBlockN;
  const int row_limit = kCausal ? min(K, K - lq + pos + 1) : K;

  // Q fragments: B operand of S^T = K Q^T. Lane holds d = 16*step + 8*h + (0..7) of its row.
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + ((int64_t)(q0 + pos) * hq + head) * kHeadDim + 8 * h;
#pragma unroll
    for (int step = 0; step < 8; ++step) {
      if (row_valid) {
        qf[step] = *reinterpret_cast<const bf16x8*>(qrow + 16 * step);
      } else {
        qf[step] = bf16x8{};
      }
    }
  }

  // Copy assignment: per block, thread tid copies chunk (tid % 16) of rows 16*i + tid/16.
  SegCursor cur;
  cur.init(segs, seg_indptr[b], seg_indptr[b + 1]);
  const int crow = tid >> 4;  // 0..15
  const int kchunk = (tid & 15) ^ crow;
  const int vchunk = (tid & 15) ^ vswz(crow);
  const int64_t head_off = (int64_t)g * kHeadDim;
  const int64_t tok_stride = (int64_t)hkv * kHeadDim;

  auto issue_block = [&](int blk, int buf) {
    lds_char_t* kb = (lds_char_t*)smem + buf * kKBufBytes;
    lds_char_t* vb = (lds_char_t*)smem + (2 + buf) * kKBufBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = min(blk * kBlockN + 16 * i + crow, K - 1);  // tail rows re-read a real key
      const int64_t base = cur.slot(j) * tok_stride + head_off;
      const int lds_off = (i * 256 + wave * 64) * 16;
      copy16_to_lds(k_pool + base + kchunk * 8, (lds_void_t*)(kb + lds_off));
      copy16_to_lds(v_pool + base + vchunk * 8, (lds_void_t*)(vb + lds_off));
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  if (n_blocks > 0) issue_block(0, 0);

  for (int blk = 0; blk < n_blocks; ++blk) {
    const int buf = blk & 1;
    wait_vmem();
    __syncthreads();
    if (blk + 1 < n_blocks) issue_block(blk + 1, buf ^ 1);

    const lds_char_t* kb = (const lds_char_t*)smem + buf * kKBufBytes;
    const lds_char_t* vb = (const lds_char_t*)smem + (2 + buf) * kKBufBytes;

    // S^T for keys 0..31 (s0) and 32..63 (s1) of the block.
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int step = 0; step < 8; ++step) {
      const int c = 2 * step + h;
      const int r0 = n, r1 = 32 + n;
      bf16x8 a0 = lds_read16(kb + r0 * 256 + ((c ^ (r0 & 15)) << 4));
      bf16x8 a1 = lds_read16(kb + r1 * 256 + ((c ^ (r1 & 15)) << 4));
      s0 = mfma32x32x16(a0, qf[step], s0);
      s1 = mfma32x32x16(a1, qf[step], s1);
    }

    // Mask keys the row may not see (beyond K, or after the row's causal horizon).
    const int kb0 = blk * kBlockN;
    if (kb0 + kBlockN > kfull) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kb0 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (j >= row_limit) s0[i] = -INFINITY;
        if (j + 32 >= row_limit) s1[i] = -INFINITY;
      }
    }

    // Online softmax for this lane's row.
    float mx = s0[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * scale_log2);
    const float neg = -m_use * scale_log2;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = fast_exp2(__builtin_fmaf(s0[i], scale_log2, neg));
      s1[i] = fast_exp2(__builtin_fmaf(s1[i], scale_log2, neg));
      psum += s0[i] + s1[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;

    bf16x8 pb[4];
    pb[0] = to_bf16x8(s0[0], s0[1], s0[2], s0[3], s0[4], s0[5], s0[6], s0[7]);
    pb[1] = to_bf16x8(s0[8], s0[9], s0[10], s0[11], s0[12], s0[13], s0[14], s0[15]);
    pb[2] = to_bf16x8(s1[0], s1[1], s1[2], s1[3], s1[4], s1[5], s1[6], s1[7]);
    pb[3] = to_bf16x8(s1[8], s1[9], s1[10], s1[11], s1[12], s1[13], s1[14], s1[15]);

    // O^T += V^T P^T. Lane (group G = lane/16, index s = lane%16) addresses 4 bf16 of V at
    // row key0 + s/4, column d0 + 4*(s%4); the transposing read hands lane s the 4 keys
    // key0..key0+3 of column d0 + s.
    const int G = lane >> 4;
    const int s = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int dcol = 32 * dt + 16 * (G & 1) + 4 * (s & 3);
      const int chunk = dcol >> 3;
      const int within = (dcol & 7) * 2;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ra = 16 * u + 4 * h + (s >> 2);
        const int rb = ra + 8;
        bf16x4 lo = lds_read_tr16(vb + ra * 256 + ((chunk ^ vswz(ra)) << 4) + within);
        bf16x4 hi = lds_read_tr16(vb + rb * 256 + ((chunk ^ vswz(rb)) << 4) + within);
        bf16x8 a;
        a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
        a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
        o[dt] = mfma32x32x16(a, pb[u], o[dt]);
      }
    }
  }

  // Epilogue: combine the two halves of the row's normaliser, scale, store.
  const float l_tot = sum_xor32(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (row_valid) {
    bf16_t* orow = out + ((int64_t)(q0 + pos) * hq + head) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int d = 32 * dt + 8 * k4 + 4 * h;
        bf16x4 v;
        v[0] = (bf16_t)(o[dt][4 * k4 + 0] * inv);
        v[1] = (bf16_t)(o[dt][4 * k4 + 1] * inv);
        v[2] = (bf16_t)(o[dt][4 * k4 + 2] * inv);
        v[3] = (bf16_t)(o[dt][4 * k4 + 3] * inv);
        *reinterpret_cast<bf16x4*>(orow + d) = v;
      }
    }
    if (lse != nullptr && h == 0) {
      lse[(int64_t)(q0 + pos) * hq + head] = l_tot > 0.f ? m_run * scale + __logf(l_tot) : -INFINITY;
    }
  }
}

}  // namespace

// Launch: grid covers ceil(max_seqlen_q / 16) query tiles x Hkv x batch; tiles past a
// request's query length exit at once.
hipError_t launch_prefill(const void* q, const void* k_pool, const void* v_pool, const void* segs,
                          const int32_t* seg_indptr, const int32_t* cu_q, const int32_t* cu_k,
                          int batch, int max_seqlen_q, int hkv, float scale, int causal, void* out,
                          float* lse, hipStream_t stream) {
  const int n_qtiles = (max_seqlen_q + kPosPerTile - 1) / kPosPerTile;
  const int64_t grid = (int64_t)n_qtiles * hkv * batch;
  if (grid == 0) return hipSuccess;
  const float scale_log2 = scale * 1.4426950408889634f;
  if (causal) {
    hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const bf16_t*)q, (const bf16_t*)k_pool, (const bf16_t*)v_pool,
                       (const Segment*)segs, seg_indptr, cu_q, cu_k, batch, hkv, n_qtiles, scale,
                       scale_log2, (bf16_t*)out, lse);
  } else {
    hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const bf16_t*)q, (const bf16_t*)k_pool, (const bf16_t*)v_pool,
                       (const Segment*)segs, seg_indptr, cu_q, cu_k, batch, hkv, n_qtiles, scale,
                       scale_log2, (bf16_t*)out, lse);
  }
  return hipGetLastError();
}

}  // namespace segattn
