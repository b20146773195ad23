// Prefill kernel: GQA attention of query chunks against KV gathered from pool segments.
//
// Work item: one tile of 128 rows = 16 consecutive query positions of one request times the
// 8 query heads that share kv head g ("PackGQA" memory access, FlashPrefill V2 abstract): every
// K/V byte staged into LDS serves all 8 heads of its group. Each key row of a 64-key block is
// looked up in the request's segment table, so a block may span any number of segments at any
// offsets (Flood README, "Introduction": segmentable KV cache).
//
// The workgroup has 8 waves in two groups of 4. Both groups own the same 128 rows (wave w and
// w + 4 hold the same 32 rows and sit on the same SIMD); group 0 takes the even key blocks,
// group 1 the odd ones, and at the end their online-softmax states are merged. The two groups
// run in opposite phases, switched by workgroup barriers ("ping-pong", FlashPrefill V2
// abstract): while one wave of a SIMD issues its MFMAs,
//     O^T[d][row] += V^T P^T   for its previous block, then
//     S^T[key][row] = K Q^T    for its current block,
// the other wave of that SIMD runs the softmax of its current block on the vector ALU. On
// gfx950 a wave does not overlap its own MFMA and VALU work, so this pairing is what keeps the
// matrix cores busy. K and V blocks are copied from HBM straight into LDS one block pair ahead
// (the double buffering of "FlashAttention on Ascend NPU", optimisation 1).
//
// Softmax is the online one (running max m and normaliser l per row; "FlashAttention on Ascend
// NPU", bottleneck 2), with the running max only moved, and O and l rescaled, when a block's
// max exceeds it by more than 2^8 in exp2 units; O / l is unchanged by the choice of reference
// max, and the bound keeps every probability below 256.
//
// MFMA 32x32x16 bf16 throughout. S^T puts keys on the M side so a lane holds 32 scores of one
// row and the row max needs one cross-lane step (permlane32); V^T comes from row-major V in LDS
// through the transposing read.
#include <type_traits>

#include "common.hpp"

namespace segattn {

namespace {

constexpr int kBlockN = 64;      // keys per block
constexpr int kThreads = 512;    // 8 waves
constexpr int kPosPerTile = 16;  // 4 waves x 32 rows / 8 heads
constexpr int kBlkBytes = kBlockN * kHeadDim * 2;  // 16 KiB
constexpr float kRescaleLog2 = 8.0f;

// LDS layouts (row = key within the block, 256 B = 16 chunks of 16 B per row):
//   K: chunk c of row r is stored at chunk position c ^ (r % 16)
//   V: chunk c of row r is stored at chunk position c ^ vswz(r)
// K is read 16 B per lane over 32 consecutive rows, V with the transposing read over groups of
// 4 consecutive rows; these swizzles keep both free of bank conflicts.
__device__ __forceinline__ int vswz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ void phase_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Scalar cursor over a request's segments; every value is the same in all lanes.
struct BlockCursor {
  const Segment* segs;
  int idx, end, start, off, len;
  __device__ __forceinline__ void fetch() {
    idx = __builtin_amdgcn_readfirstlane(idx);  // uniform index -> scalar (s_load) table read
    if (idx < end) {
      i32x2 v = *reinterpret_cast<const i32x2*>(segs + idx);
      off = __builtin_amdgcn_readfirstlane(v[0]);
      len = __builtin_amdgcn_readfirstlane(v[1]);
    } else {
      off = 0;
      len = 0x7fffffff;
    }
  }
  __device__ __forceinline__ void init(const Segment* s, int first, int last) {
    segs = s;
    idx = first;
    end = last;
    start = 0;
    fetch();
  }
  __device__ __forceinline__ void advance_to(int j) {
    while (j - start >= len) {
      start += len;
      ++idx;
      fetch();
    }
  }
};

template <bool kCausal>
__global__ __launch_bounds__(kThreads) void prefill_split_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_pool,
    const bf16_t* __restrict__ v_pool, const Segment* __restrict__ segs,
    const int32_t* __restrict__ seg_indptr, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int batch, int hkv, int n_qtiles, float scale,
    float scale_log2, bf16_t* __restrict__ out, float* __restrict__ lse) {
  // Eight separate LDS arrays, one per (K|V, pair slot, group). Keeping them separate objects,
  // and every slot index a compile-time constant, lets the compiler see that the blocks being
  // read never alias the blocks being copied in, so it does not wait for the in-flight copies
  // before each read.
  __shared__ __attribute__((aligned(1024))) char kb00[kBlkBytes];  // K, slot 0, group 0
  __shared__ __attribute__((aligned(1024))) char kb01[kBlkBytes];  // K, slot 0, group 1
  __shared__ __attribute__((aligned(1024))) char kb10[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char kb11[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char vb00[kBlkBytes];  // V, slot 0, group 0
  __shared__ __attribute__((aligned(1024))) char vb01[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char vb10[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char vb11[kBlkBytes];

  // Work item: heaviest (last) query tiles first; kv head fastest so that, with 8 kv heads,
  // every tile of head g lands on the same XCD (workgroups are dealt round-robin over the 8
  // XCDs) and shares its L2.
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
  const int grp = wave >> 2;  // 0: even key blocks, 1: odd key blocks
  const int wq = wave & 3;
  const int lane = tid & 63;
  const int n = lane & 31;  // row within the wave
  const int h = lane >> 5;  // which half of the k / m slots this lane holds
  const int pos = p0 + wq * 4 + (n >> 3);
  const int head = g * kGroup + (n & 7);
  const bool row_valid = pos < lq;

  const int last_pos = min(p0 + kPosPerTile - 1, lq - 1);
  const int kend = kCausal ? min(K, K - lq + last_pos + 1) : K;  // keys the tile sees at all
  const int kfull = kCausal ? min(K, K - lq + p0 + 1) : K;        // keys every row sees
  const int n_blocks = max(0, (kend + kBlockN - 1) / kBlockN);
  const int n_pairs = (n_blocks + 1) >> 1;
  const int row_limit = kCausal ? min(K, K - lq + pos + 1) : K;

  // Q fragments: B operand of S^T = K Q^T. Lane holds d = 16*step + 8*h + (0..7) of its row.
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + ((int64_t)(q0 + pos) * hq + head) * kHeadDim + 8 * h;
#pragma unroll
    for (int step = 0; step < 8; ++step)
      qf[step] = row_valid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * step) : bf16x8{};
  }

  // ---- HBM -> LDS copies. Per block, thread tid copies chunk (tid % 16) of rows tid/16 and
  // 32 + tid/16 (the same chunk position in both rows since 32 % 16 == 0).
  // K and V blocks are each copied in increasing block order, each stream with its own cursor.
  BlockCursor kcur, vcur;
  kcur.init(segs, seg_indptr[b], seg_indptr[b + 1]);
  vcur.init(segs, seg_indptr[b], seg_indptr[b + 1]);
  const int crow = tid >> 4;  // 0..31
  const int kchunk = (tid & 15) ^ (crow & 15);
  const int vchunk = (tid & 15) ^ vswz(crow);
  const int64_t tok_stride = (int64_t)hkv * kHeadDim;
  const bf16_t* kbase = k_pool + (int64_t)g * kHeadDim;
  const bf16_t* vbase = v_pool + (int64_t)g * kHeadDim;

  // Where this thread's two rows of block blk live. Fast case (the whole block inside one
  // segment and inside the request's keys, the usual case): row r of the block is pool slot
  // base + r, with base the same for the whole workgroup, so the copy address is a scalar base
  // plus a per-thread constant offset and costs no vector arithmetic. Otherwise each row is
  // resolved on its own (rows past K re-read key K-1).
  struct BlockAddr {
    bool fast;
    int64_t base;    // fast: slot of the block's row 0
    int64_t s0, s1;  // slow: slots of rows crow and 32 + crow
  };
  auto block_addr = [&](BlockCursor& cur, int blk) __attribute__((always_inline)) {
    BlockAddr a;
    const int kb0 = blk * kBlockN;
    const int last = min(kb0 + kBlockN, K) - 1;
    cur.advance_to(kb0);
    a.fast = (kb0 + kBlockN <= K) && (last - cur.start < cur.len);
    a.base = (int64_t)cur.off + (kb0 - cur.start);
    a.s0 = a.s1 = 0;
    if (!a.fast) {
      const int r0 = min(kb0 + crow, last), r1 = min(kb0 + 32 + crow, last);
      SegCursor c2;
      c2.segs = cur.segs;
      c2.idx = cur.idx;
      c2.end = cur.end;
      c2.start = cur.start;
      c2.off = cur.off;
      c2.len = cur.len;
      a.s0 = c2.slot(r0);
      a.s1 = c2.slot(r1);
    }
    return a;
  };
  const uint32_t tok_bytes = (uint32_t)hkv * kHeadDim * 2;
  const uint32_t koff0 = (uint32_t)crow * tok_bytes + kchunk * 16, koff1 = koff0 + 32 * tok_bytes;
  const uint32_t voff0 = (uint32_t)crow * tok_bytes + vchunk * 16, voff1 = voff0 + 32 * tok_bytes;
  // Copy the thread's two rows of a K (or V) block into the 16 KiB at dst; each wave fills its
  // own 1 KiB lines of the block.
  auto copy_k = [&](const BlockAddr& a, char* dst) __attribute__((always_inline)) {
    lds_char_t* lk = (lds_char_t*)dst + wave * 1024;
    if (a.fast) {
      const char* sb = (const char*)(kbase + a.base * tok_stride);
      copy16_to_lds(sb + koff0, (lds_void_t*)lk);
      copy16_to_lds(sb + koff1, (lds_void_t*)(lk + 8192));
    } else {
      copy16_to_lds(kbase + a.s0 * tok_stride + kchunk * 8, (lds_void_t*)lk);
      copy16_to_lds(kbase + a.s1 * tok_stride + kchunk * 8, (lds_void_t*)(lk + 8192));
    }
  };
  auto copy_v = [&](const BlockAddr& a, char* dst) __attribute__((always_inline)) {
    lds_char_t* lv = (lds_char_t*)dst + wave * 1024;
    if (a.fast) {
      const char* sb = (const char*)(vbase + a.base * tok_stride);
      copy16_to_lds(sb + voff0, (lds_void_t*)lv);
      copy16_to_lds(sb + voff1, (lds_void_t*)(lv + 8192));
    } else {
      copy16_to_lds(vbase + a.s0 * tok_stride + vchunk * 8, (lds_void_t*)lv);
      copy16_to_lds(vbase + a.s1 * tok_stride + vchunk * 8, (lds_void_t*)(lv + 8192));
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  bf16x8 pb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = bf16x8{};
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's keys only; the row total is l + l of lane ^ 32

  const int G = lane >> 4;  // 16-lane group for the transposing V read
  const int sl = lane & 15;

  // Matrix phase of this wave for pair i: PV of its block of pair i-1 (V at vprev), then S of
  // its block of pair i (K at kcur).
  auto gemm_phase = [&](int i, const char* vprev, const char* kcurp) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (i >= 1 && 2 * (i - 1) + grp < n_blocks) {
      const lds_char_t* vb = (const lds_char_t*)vprev;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int dcol = 32 * dt + 16 * (G & 1) + 4 * (sl & 3);
        const int chunk = dcol >> 3;
        const int within = (dcol & 7) * 2;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ra = 16 * u + 4 * h + (sl >> 2);
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
    if (i < n_pairs && 2 * i + grp < n_blocks) {
      const lds_char_t* kb = (const lds_char_t*)kcurp;
      s0 = f32x16{};
      s1 = f32x16{};
#pragma unroll
      for (int step = 0; step < 8; ++step) {
        const int c = 2 * step + h;
        const int r0 = n, r1 = 32 + n;
        bf16x8 a0 = lds_read16(kb + r0 * 256 + ((c ^ (r0 & 15)) << 4));
        bf16x8 a1 = lds_read16(kb + r1 * 256 + ((c ^ (r1 & 15)) << 4));
        s0 = mfma32x32x16(a0, qf[step], s0);
        s1 = mfma32x32x16(a1, qf[step], s1);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Vector phase: online softmax of this wave's block of pair ip (scores in s0/s1).
  auto softmax_phase = [&](int ip) __attribute__((always_inline)) {
    const int blk = 2 * ip + grp;
    if (ip < 0 || ip >= n_pairs || blk >= n_blocks) return;
    const int kb0 = blk * kBlockN;
    if (kb0 + kBlockN > kfull) {
      const int thr = row_limit - kb0 - 4 * h;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        // key kb0 + 4h + off_e is hidden iff off_e >= thr (off_e a compile-time constant)
        const int off_e = 8 * (e >> 2) + (e & 3);
        if (off_e >= thr) s0[e] = -INFINITY;
        if (off_e + 32 >= thr) s1[e] = -INFINITY;
      }
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(s0[0], s0[1]), s0[2]);
#pragma unroll
    for (int e = 3; e < 16; ++e) mx = __builtin_fmaxf(mx, s0[e]);
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, s1[e]);
    mx = max_xor32(mx);
    // move the reference max only when the block's max clears it by 2^8 (exp2 units)
    const bool grow = (m_run == -INFINITY) ? (mx != -INFINITY) : ((mx - m_run) * scale_log2 > kRescaleLog2);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * scale_log2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float neg = (m_run == -INFINITY) ? 0.f : -m_run * scale_log2;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = fast_exp2(__builtin_fmaf(s0[e], scale_log2, neg));
      s1[e] = fast_exp2(__builtin_fmaf(s1[e], scale_log2, neg));
      ps0 += s0[e];
      ps1 += s1[e];
    }
    l_run += ps0 + ps1;
    pb[0] = to_bf16x8(s0[0], s0[1], s0[2], s0[3], s0[4], s0[5], s0[6], s0[7]);
    pb[1] = to_bf16x8(s0[8], s0[9], s0[10], s0[11], s0[12], s0[13], s0[14], s0[15]);
    pb[2] = to_bf16x8(s1[0], s1[1], s1[2], s1[3], s1[4], s1[5], s1[6], s1[7]);
    pb[3] = to_bf16x8(s1[8], s1[9], s1[10], s1[11], s1[12], s1[13], s1[14], s1[15]);
  };

  // One pair step = phases 2i (group 0 matrix, group 1 vector) and 2i+1 (the reverse). At
  // phase 2i every thread copies K of pair i+1 and V of pair i; they are first read at phase
  // 2i+2, after the wait and barrier that end this step. Slot = pair index & 1.
  auto pair_step = [&](int i, auto slot_c) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_c)::value;
    char* knext0 = S ? kb00 : kb10;  // K of pair i + 1 (filled now), blocks of group 0 / 1
    char* knext1 = S ? kb01 : kb11;
    char* vnow0 = S ? vb10 : vb00;   // V of pair i (filled now)
    char* vnow1 = S ? vb11 : vb01;
    // Resolve every slot first: a segment-table read issued after the copies would have to
    // wait for them (vector memory operations complete in order).
    BlockAddr ka0{}, ka1{}, va0{}, va1{};
    if (2 * (i + 1) < n_blocks) ka0 = block_addr(kcur, 2 * (i + 1));
    if (2 * (i + 1) + 1 < n_blocks) ka1 = block_addr(kcur, 2 * (i + 1) + 1);
    if (2 * i < n_blocks) va0 = block_addr(vcur, 2 * i);
    if (2 * i + 1 < n_blocks) va1 = block_addr(vcur, 2 * i + 1);
    if (2 * (i + 1) < n_blocks) copy_k(ka0, knext0);
    if (2 * (i + 1) + 1 < n_blocks) copy_k(ka1, knext1);
    if (2 * i < n_blocks) copy_v(va0, vnow0);
    if (2 * i + 1 < n_blocks) copy_v(va1, vnow1);
    // this step reads K of pair i (slot S) and V of pair i - 1 (slot 1 - S)
    if (grp == 0) gemm_phase(i, S ? vb00 : vb10, S ? kb10 : kb00);
    else softmax_phase(i - 1);
    phase_barrier();
    if (grp == 1) gemm_phase(i, S ? vb01 : vb11, S ? kb11 : kb01);
    else softmax_phase(i);
    wait_vmem();
    phase_barrier();
  };

  // Prologue: K of block pair 0.
  {
    BlockAddr a0{}, a1{};
    if (n_blocks > 0) a0 = block_addr(kcur, 0);
    if (n_blocks > 1) a1 = block_addr(kcur, 1);
    if (n_blocks > 0) copy_k(a0, kb00);
    if (n_blocks > 1) copy_k(a1, kb01);
  }
  wait_vmem();
  phase_barrier();
  if (n_blocks > 0) {
    for (int i = 0; i <= n_pairs; i += 2) {
      pair_step(i, std::integral_constant<int, 0>{});
      if (i + 1 <= n_pairs) pair_step(i + 1, std::integral_constant<int, 1>{});
    }
  }

  // ---- merge the two groups' states (same rows, disjoint key blocks) and store.
  // Group 1 parks O (d tiles 0-1 of waves 0-1 in kb00, of waves 2-3 in kb01; d tiles 2-3 in
  // kb10 / kb11), m and l (vb00) per lane.
  char* lo_arr = (wq < 2) ? kb00 : kb01;
  char* hi_arr = (wq < 2) ? kb10 : kb11;
  float* park_lo = reinterpret_cast<float*>(lo_arr) + (size_t)(wq & 1) * (32 * 64);
  float* park_hi = reinterpret_cast<float*>(hi_arr) + (size_t)(wq & 1) * (32 * 64);
  float* park_ml = reinterpret_cast<float*>(vb00) + (size_t)wq * (2 * 64);
  if (grp == 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      park_lo[e * 64 + lane] = o[0][e];
      park_lo[(16 + e) * 64 + lane] = o[1][e];
      park_hi[e * 64 + lane] = o[2][e];
      park_hi[(16 + e) * 64 + lane] = o[3][e];
    }
    park_ml[lane] = m_run;
    park_ml[64 + lane] = l_run;
  }
  phase_barrier();
  if (grp == 0) {
    const float m1 = park_ml[lane];
    const float l1 = park_ml[64 + lane];
    const float m_tot = __builtin_fmaxf(m_run, m1);
    const float m_use = (m_tot == -INFINITY) ? 0.f : m_tot;
    const float a0 = fast_exp2((m_run - m_use) * scale_log2);
    const float a1 = fast_exp2((m1 - m_use) * scale_log2);
    const float l_tot = sum_xor32(a0 * l_run + a1 * l1);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (row_valid) {
      bf16_t* orow = out + ((int64_t)(q0 + pos) * hq + head) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const float* park = (dt < 2 ? park_lo : park_hi) + (dt & 1) * 16 * 64;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int d = 32 * dt + 8 * k4 + 4 * h;
          bf16x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int e = 4 * k4 + t;
            v[t] = (bf16_t)((a0 * o[dt][e] + a1 * park[e * 64 + lane]) * inv);
          }
          *reinterpret_cast<bf16x4*>(orow + d) = v;
        }
      }
      if (lse != nullptr && h == 0)
        lse[(int64_t)(q0 + pos) * hq + head] = l_tot > 0.f ? m_tot * scale + __logf(l_tot) : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Wide tiles: 256 rows (32 query positions x 8 heads) per workgroup. Group 0 owns positions
// 0-15 of the tile, group 1 positions 16-31; both groups consume every K/V block (so each block
// copied into LDS serves 256 rows, half the L2->LDS traffic of the 128-row tiles) and run in
// opposite phases: in step j group 0 issues its MFMAs (PV of block j-1, S of block j) while
// group 1 runs the softmax of block j-1, then the roles swap. K and V blocks are double
// buffered and copied one step ahead of use; the Q tile is staged in LDS.
constexpr int kWidePos = 32;

template <bool kCausal>
__global__ __launch_bounds__(kThreads) void prefill_wide_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_pool,
    const bf16_t* __restrict__ v_pool, const Segment* __restrict__ segs,
    const int32_t* __restrict__ seg_indptr, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int batch, int hkv, int n_qtiles, float scale,
    float scale_log2, bf16_t* __restrict__ out, float* __restrict__ lse) {
  // Separate LDS objects per ring slot, indexed only by compile-time constants, so the compiler
  // can tell the slots being read from the slots being filled.
  __shared__ __attribute__((aligned(1024))) char kr0[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char kr1[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char vr0[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char vr1[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char qlds[2 * kWidePos * kGroup * kHeadDim];  // 256 rows

  // Work item: kv head fastest (with 8 kv heads, head g always runs on XCD g), then the query
  // tiles of one request, heaviest (last) first, then the requests. Workgroups running at the
  // same time on an XCD thus share one request's K/V stream in that XCD's L2.
  const int id = blockIdx.x;
  const int g = id % hkv;
  const int t = id / hkv;
  const int b = t / n_qtiles;
  const int qtile = n_qtiles - 1 - t % n_qtiles;

  const int q0 = cu_q[b];
  const int lq = cu_q[b + 1] - q0;
  const int p0 = qtile * kWidePos;
  if (p0 >= lq) return;
  const int K = cu_k[b + 1] - cu_k[b];
  const int hq = hkv * kGroup;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int grp = wave >> 2;
  const int wq = wave & 3;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int wpos0 = p0 + 16 * grp + 4 * wq;  // first position of this wave's rows
  const int pos = wpos0 + (n >> 3);
  const int head = g * kGroup + (n & 7);
  const bool row_valid = pos < lq;

  const int last_pos = min(p0 + kWidePos - 1, lq - 1);
  const int kend = kCausal ? min(K, K - lq + last_pos + 1) : K;
  const int n_blocks = max(0, (kend + kBlockN - 1) / kBlockN);
  const int kfull = kCausal ? min(K, K - lq + wpos0 + 1) : K;  // every row of this wave sees these
  const int row_limit = kCausal ? min(K, K - lq + pos + 1) : K;

  // Q tile staged in LDS (kept out of registers): LDS row R = wave * 32 + n holds the query row
  // of wave R / 32, lane row n; chunk c of row R sits at chunk position c ^ (R % 16). Thread t
  // copies chunk position t % 16 of rows t / 16 + 32 i; rows past the request re-read its last
  // query row (they are computed but never stored).
  {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int R = (tid >> 4) + 32 * i;
      const int rw = R >> 5, rn = R & 31;
      const int rpos = min(p0 + 16 * (rw >> 2) + 4 * (rw & 3) + (rn >> 3), lq - 1);
      const int rhead = g * kGroup + (rn & 7);
      const int c = (tid & 15) ^ (R & 15);
      const bf16_t* src = q + ((int64_t)(q0 + rpos) * hq + rhead) * kHeadDim + c * 8;
      copy16_to_lds(src, (lds_void_t*)((lds_char_t*)qlds + i * 8192 + wave * 1024));
    }
  }
  const lds_char_t* qmine = (const lds_char_t*)qlds + (wave * 32 + n) * 256;

  BlockCursor kcur, vcur;
  kcur.init(segs, seg_indptr[b], seg_indptr[b + 1]);
  vcur.init(segs, seg_indptr[b], seg_indptr[b + 1]);
  const int crow = tid >> 4;
  const int kchunk = (tid & 15) ^ (crow & 15);
  const int vchunk = (tid & 15) ^ vswz(crow);
  const int64_t tok_stride = (int64_t)hkv * kHeadDim;
  const bf16_t* kbase = k_pool + (int64_t)g * kHeadDim;
  const bf16_t* vbase = v_pool + (int64_t)g * kHeadDim;
  const uint32_t tok_bytes = (uint32_t)hkv * kHeadDim * 2;
  const uint32_t koff0 = (uint32_t)crow * tok_bytes + kchunk * 16, koff1 = koff0 + 32 * tok_bytes;
  const uint32_t voff0 = (uint32_t)crow * tok_bytes + vchunk * 16, voff1 = voff0 + 32 * tok_bytes;

  struct BlockAddr {
    bool fast;
    int64_t base, s0, s1;
  };
  auto block_addr = [&](BlockCursor& cur, int blk) __attribute__((always_inline)) {
    BlockAddr a;
    const int kb0 = blk * kBlockN;
    const int last = min(kb0 + kBlockN, K) - 1;
    cur.advance_to(kb0);
    a.fast = (kb0 + kBlockN <= K) && (last - cur.start < cur.len);
    a.base = (int64_t)cur.off + (kb0 - cur.start);
    a.s0 = a.s1 = 0;
    if (!a.fast) {
      // Walk the segments the block overlaps with a scalar copy of the cursor: every lane
      // takes the same trip and the table is read with scalar loads, so no vector memory
      // wait (which would also wait for the prefetched K/V) is needed.
      const int r0 = min(kb0 + crow, last), r1 = min(kb0 + 32 + crow, last);
      BlockCursor c2 = cur;
      while (true) {
        if (r0 - c2.start >= 0 && r0 - c2.start < c2.len) a.s0 = (int64_t)c2.off + (r0 - c2.start);
        if (r1 - c2.start >= 0 && r1 - c2.start < c2.len) a.s1 = (int64_t)c2.off + (r1 - c2.start);
        if (last - c2.start < c2.len) break;
        c2.start += c2.len;
        ++c2.idx;
        c2.fetch();
      }
    }
    return a;
  };
  // K/V blocks travel HBM -> registers -> LDS. Loading into registers two steps ahead of the
  // LDS write hides the HBM latency of blocks no workgroup has touched yet, and plain register
  // loads let the compiler wait for exactly the data it needs.
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  auto load_rows = [&](BlockCursor& cur, int blk, const bf16_t* pool_base, int chunk, uint32_t off0,
                       uint32_t off1, u32x4& r0, u32x4& r1) __attribute__((always_inline)) {
    const BlockAddr a = block_addr(cur, blk);
    // one load per row on every path (no branch around the loads), from either address form
    const char* sb = (const char*)(pool_base + a.base * tok_stride);
    const char* p0 = a.fast ? sb + off0 : (const char*)(pool_base + a.s0 * tok_stride + chunk * 8);
    const char* p1 = a.fast ? sb + off1 : (const char*)(pool_base + a.s1 * tok_stride + chunk * 8);
    r0 = *(const u32x4*)p0;
    r1 = *(const u32x4*)p1;
  };
  // Thread tid's two 16-byte pieces of a block go to bytes tid*16 and 8192 + tid*16 of its slot
  // (the swizzle is in which global chunk the thread loaded).
  auto store_rows = [&](char* dst, const u32x4& r0, const u32x4& r1) __attribute__((always_inline)) {
    *(__attribute__((address_space(3))) u32x4*)((lds_char_t*)dst + tid * 16) = r0;
    *(__attribute__((address_space(3))) u32x4*)((lds_char_t*)dst + 8192 + tid * 16) = r1;
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  bf16x8 pb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = bf16x8{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const int G = lane >> 4;
  const int sl = lane & 15;

  auto gemm_phase = [&](int j, const char* vprev, const char* kcurp) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (j >= 1) {
      const lds_char_t* vb = (const lds_char_t*)vprev;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int dcol = 32 * dt + 16 * (G & 1) + 4 * (sl & 3);
        const int chunk = dcol >> 3;
        const int within = (dcol & 7) * 2;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int ra = 16 * u + 4 * h + (sl >> 2);
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
    if (j < n_blocks) {
      const lds_char_t* kb = (const lds_char_t*)kcurp;
      s0 = f32x16{};
      s1 = f32x16{};
#pragma unroll
      for (int step = 0; step < 8; ++step) {
        const int c = 2 * step + h;
        const int r0 = n, r1 = 32 + n;
        bf16x8 a0 = lds_read16(kb + r0 * 256 + ((c ^ (r0 & 15)) << 4));
        bf16x8 a1 = lds_read16(kb + r1 * 256 + ((c ^ (r1 & 15)) << 4));
        const bf16x8 qv = lds_read16(qmine + ((c ^ (n & 15)) << 4));
        s0 = mfma32x32x16(a0, qv, s0);
        s1 = mfma32x32x16(a1, qv, s1);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  auto softmax_phase = [&](int j) __attribute__((always_inline)) {
    if (j < 0 || j >= n_blocks) return;
    const int kb0 = j * kBlockN;
    if (kb0 + kBlockN > kfull) {
      const int thr = row_limit - kb0 - 4 * h;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        // key kb0 + 4h + off_e is hidden iff off_e >= thr (off_e a compile-time constant)
        const int off_e = 8 * (e >> 2) + (e & 3);
        if (off_e >= thr) s0[e] = -INFINITY;
        if (off_e + 32 >= thr) s1[e] = -INFINITY;
      }
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(s0[0], s0[1]), s0[2]);
#pragma unroll
    for (int e = 3; e < 16; ++e) mx = __builtin_fmaxf(mx, s0[e]);
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, s1[e]);
    mx = max_xor32(mx);
    const bool grow = (m_run == -INFINITY) ? (mx != -INFINITY) : ((mx - m_run) * scale_log2 > kRescaleLog2);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * scale_log2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float neg = (m_run == -INFINITY) ? 0.f : -m_run * scale_log2;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = fast_exp2(__builtin_fmaf(s0[e], scale_log2, neg));
      s1[e] = fast_exp2(__builtin_fmaf(s1[e], scale_log2, neg));
      ps0 += s0[e];
      ps1 += s1[e];
    }
    l_run += ps0 + ps1;
    pb[0] = to_bf16x8(s0[0], s0[1], s0[2], s0[3], s0[4], s0[5], s0[6], s0[7]);
    pb[1] = to_bf16x8(s0[8], s0[9], s0[10], s0[11], s0[12], s0[13], s0[14], s0[15]);
    pb[2] = to_bf16x8(s1[0], s1[1], s1[2], s1[3], s1[4], s1[5], s1[6], s1[7]);
    pb[3] = to_bf16x8(s1[8], s1[9], s1[10], s1[11], s1[12], s1[13], s1[14], s1[15]);
  };

  // Register staging sets: set e holds K(j+1) and V(j) at the start of step j with j % 2 == e.
  u32x4 stk[2][2], stv[2][2];
  const int last_blk = n_blocks - 1;

  // Step j: K(j) in LDS slot j % 2 is read (S of block j), V(j-1) in slot (j-1) % 2 is read
  // (PV of block j-1). At the start, staging set j % 2 (loaded two steps earlier) is written to
  // LDS: K(j+1) into slot (j+1) % 2 and V(j) into slot j % 2, both last read in step j-1; then
  // the same set is refilled with K(j+3) and V(j+2). Blocks past the end re-load the last one.
  auto step = [&](int j, auto r_c) __attribute__((always_inline)) {
    constexpr int R = decltype(r_c)::value;
    char* kread = R == 0 ? kr0 : kr1;
    char* kwrite = R == 0 ? kr1 : kr0;
    char* vread = R == 0 ? vr1 : vr0;
    char* vwrite = R == 0 ? vr0 : vr1;
    store_rows(kwrite, stk[R][0], stk[R][1]);
    store_rows(vwrite, stv[R][0], stv[R][1]);
    load_rows(kcur, min(j + 3, last_blk), kbase, kchunk, koff0, koff1, stk[R][0], stk[R][1]);
    load_rows(vcur, min(j + 2, last_blk), vbase, vchunk, voff0, voff1, stv[R][0], stv[R][1]);
    if (grp == 0) gemm_phase(j, vread, kread);
    else softmax_phase(j - 1);
    phase_barrier();
    if (grp == 1) gemm_phase(j, vread, kread);
    else softmax_phase(j);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's LDS stores are done
    phase_barrier();
  };

  // Prologue: K(0) into slot 0; staging set 0 = {K(1), V(0)}, set 1 = {K(2), V(1)}.
  if (n_blocks > 0) {
    u32x4 a0, a1;
    // issue order = use order (set 0 before set 1), so each wait covers only what it needs
    load_rows(kcur, 0, kbase, kchunk, koff0, koff1, a0, a1);
    load_rows(kcur, min(1, last_blk), kbase, kchunk, koff0, koff1, stk[0][0], stk[0][1]);
    load_rows(vcur, 0, vbase, vchunk, voff0, voff1, stv[0][0], stv[0][1]);
    load_rows(kcur, min(2, last_blk), kbase, kchunk, koff0, koff1, stk[1][0], stk[1][1]);
    load_rows(vcur, min(1, last_blk), vbase, vchunk, voff0, voff1, stv[1][0], stv[1][1]);
    store_rows(kr0, a0, a1);
  }
  wait_vmem();  // also the Q tile's HBM->LDS copies
  __builtin_amdgcn_s_waitcnt(0xC07F);
  phase_barrier();
  if (n_blocks > 0) {
    // Both steps of a pair unconditionally inside the loop, the odd tail after it: a loop body
    // that may end after its first step would make the compiler assume that step's loads are
    // the most recent ones at the loop head and wait for all of them.
    int j = 0;
    for (; j + 1 <= n_blocks; j += 2) {
      step(j, std::integral_constant<int, 0>{});
      step(j + 1, std::integral_constant<int, 1>{});
    }
    if (j <= n_blocks) step(j, std::integral_constant<int, 0>{});
  }

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
    if (lse != nullptr && h == 0)
      lse[(int64_t)(q0 + pos) * hq + head] = l_tot > 0.f ? m_run * scale + __logf(l_tot) : -INFINITY;
  }
}

}  // namespace

// Launch. Two tilings: 256-row tiles halve the L2->LDS traffic and are used whenever they
// still give at least two workgroups per compute unit; otherwise 128-row tiles split each
// tile's keys between the two wave groups, which keeps more compute units busy on small
// batches. SEG_ATTN_PREFILL_TILE=128|256 forces one of them.
hipError_t launch_prefill(const void* q, const void* k_pool, const void* v_pool, const void* segs,
                          const int32_t* seg_indptr, const int32_t* cu_q, const int32_t* cu_k,
                          int batch, int max_seqlen_q, int hkv, float scale, int causal, void* out,
                          float* lse, int cu_count, int force_tile, hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  const int64_t wide_tiles = (int64_t)((max_seqlen_q + kWidePos - 1) / kWidePos) * hkv * batch;
  const bool wide = force_tile == 256 || (force_tile != 128 && wide_tiles >= 2LL * cu_count);
  if (wide) {
    const int n_qtiles = (max_seqlen_q + kWidePos - 1) / kWidePos;
    if (wide_tiles == 0) return hipSuccess;
    auto kern = causal ? prefill_wide_kernel<true> : prefill_wide_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)wide_tiles), dim3(kThreads), 0, stream, (const bf16_t*)q,
                       (const bf16_t*)k_pool, (const bf16_t*)v_pool, (const Segment*)segs, seg_indptr,
                       cu_q, cu_k, batch, hkv, n_qtiles, scale, scale_log2, (bf16_t*)out, lse);
    return hipGetLastError();
  }
  const int n_qtiles = (max_seqlen_q + kPosPerTile - 1) / kPosPerTile;
  const int64_t grid = (int64_t)n_qtiles * hkv * batch;
  if (grid == 0) return hipSuccess;
  auto kern = causal ? prefill_split_kernel<true> : prefill_split_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, stream, (const bf16_t*)q,
                     (const bf16_t*)k_pool, (const bf16_t*)v_pool, (const Segment*)segs, seg_indptr,
                     cu_q, cu_k, batch, hkv, n_qtiles, scale, scale_log2, (bf16_t*)out, lse);
  return hipGetLastError();
}

}  // namespace segattn
