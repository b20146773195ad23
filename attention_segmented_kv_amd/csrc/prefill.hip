// Prefill kernels: GQA attention of query chunks against KV gathered from pool segments.
//
// Work item: a tile of query rows = consecutive query positions of one request times the 8
// query heads that share kv head g ("PackGQA" memory access, FlashPrefill V2 abstract): every
// K/V byte staged into LDS serves all 8 heads of its group. Each key row of a 64-key block is
// looked up in the request's segment table, so a block may span any number of segments at any
// offsets (Flood README, "Introduction": segmentable KV cache).
//
// Two tilings share the block machinery below:
//   quad: 128 rows (16 positions) per workgroup of 4 waves, two workgroups per CU, each wave
//         running S, softmax and PV of a block back to back; the MFMAs of one workgroup's wave
//         overlap the vector work of the other workgroup's wave on the same SIMD;
//   wide: 256 rows (32 positions) per workgroup of 8 waves in two groups that run in opposite
//         phases, switched by workgroup barriers ("ping-pong", FlashPrefill V2 abstract), so
//         that every K/V block copied into LDS serves twice as many rows.
// On gfx950 a wave does not overlap its own MFMA and VALU work; both tilings rely on the second
// wave of each SIMD for that. K and V blocks are copied from HBM into LDS one block ahead of use
// (the double buffering of "FlashAttention on Ascend NPU", optimisation 1).
//
// Softmax is the online one (running max m and normaliser l per row; "FlashAttention on Ascend
// NPU", bottleneck 2), with the running max only moved, and O and l rescaled, when a block's
// max exceeds it by more than 2^8 in exp2 units; O / l is unchanged by the choice of reference
// max, and the bound keeps every probability below 256.
//
// MFMA 32x32x16 bf16 throughout. S^T puts keys on the M side so a lane holds 32 scores of one
// row and the row max needs one cross-lane step (permlane32); V^T comes from V in LDS through
// the transposing read.
#include <type_traits>

#include "common.hpp"

namespace segattn {

namespace {

constexpr int kBlockN = 64;      // keys per block
constexpr int kThreads = 512;    // 8 waves
constexpr int kPosPerTile = 16;  // 4 waves x 32 rows / 8 heads
constexpr int kBlkBytes = kBlockN * kHeadDim * 2;  // 16 KiB
constexpr float kRescaleLog2 = 8.0f;
// Running-max start: below any score, so that no infinity arithmetic is needed; a row that
// never sees a key keeps it (and l = 0).
constexpr float kNoMax = -3.0e38f;

// LDS layouts (row = key within the block, 256 B = 16 chunks of 16 B per row):
//   K: chunk c of row r is stored at chunk position c ^ (r % 16)
//   V: quarter-major, d quarter q (64 B of every row) of the block's 64 rows occupies bytes
//     q * 4096 + r * 64 .. + 63
// (both tilings use these layouts).
// K is read 16 B per lane over 32 consecutive rows, V with the transposing read over groups of
// 4 consecutive rows. The K swizzle keeps its reads free of bank conflicts; in the quarter-major
// V layout one transposing read covers 8 consecutive rows of one quarter, 512 contiguous bytes,
// and every read of a block is a constant offset from a single per-lane address.

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

// Query rows at or past position `first` of a request (q0: its first row) for the 8 heads of kv
// head g. The grid covers positions below max_seqlen_q, the host's bound of every Lq_b; rows of
// a request that breaks it are never computed, and the workgroup of the last query tile writes
// NaN to them (and to their LSE) so that the broken bound cannot pass unnoticed.
__device__ __forceinline__ void mark_uncovered_rows(bf16_t* out, float* lse, int64_t q0,
                                                    int first, int lq, int hq, int g) {
  const int64_t n = (int64_t)(lq - first) * kGroup * (kHeadDim / 8);  // 16-byte pieces
  const bf16_t nanv = (bf16_t)NAN;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const int64_t r = i / (kGroup * (kHeadDim / 8));
    const int hh = (int)(i / (kHeadDim / 8) % kGroup), c = (int)(i % (kHeadDim / 8));
    const int64_t row = (q0 + first + r) * hq + g * kGroup + hh;
    *reinterpret_cast<bf16x8*>(out + row * kHeadDim + 8 * c) =
        bf16x8{nanv, nanv, nanv, nanv, nanv, nanv, nanv, nanv};
    if (lse != nullptr && c == 0) lse[row] = NAN;
  }
}

// ------------------------------------------------------------------------------------------
// Wide tiles: 256 rows (32 query positions x 8 heads) per workgroup. Group 0 owns positions
// 0-15 of the tile, group 1 positions 16-31; both groups consume every K/V block (so each block
// copied into LDS serves 256 rows, half the L2->LDS traffic of the 128-row tiles) and run in
// opposite phases: in step j group 0 issues its MFMAs (PV of block j-1, S of block j) while
// group 1 runs the softmax of block j-1, then the roles swap. K and V blocks are copied from
// HBM straight into LDS (double buffered): at the start of step j the copies of K(j+1) and V(j)
// are issued into the slots freed by step j-1, and the step's last barrier waits for them. Each
// wave's Q rows stay in registers.
constexpr int kWidePos = 32;

template <bool kCausal, bool kOff32>
__global__ __launch_bounds__(kThreads) void prefill_wide_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_pool,
    const bf16_t* __restrict__ v_pool, const Segment* __restrict__ segs,
    const int32_t* __restrict__ seg_indptr, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int batch, int hkv, int n_qtiles, float scale,
    float scale_log2, bf16_t* __restrict__ out, float* __restrict__ lse) {
  // Separate LDS objects per ring slot, indexed only by compile-time constants, so the compiler
  // can tell the slots being read from the slots being filled. The K and V slots get the larger
  // alignments, which places them below 64 KiB: every K and V read is then a per-lane register
  // plus an immediate offset.
  __shared__ __attribute__((aligned(4096))) char vr0[kBlkBytes];
  __shared__ __attribute__((aligned(4096))) char vr1[kBlkBytes];
  __shared__ __attribute__((aligned(2048))) char kr0[kBlkBytes];
  __shared__ __attribute__((aligned(2048))) char kr1[kBlkBytes];

  // Every pointer argument in scalar registers before the first table read (one round trip).
  asm volatile("" ::"s"(q), "s"(k_pool), "s"(v_pool), "s"(segs), "s"(seg_indptr), "s"(cu_q),
               "s"(cu_k), "s"(out), "s"(lse));

  // Work item: kv head fastest (with 8 kv heads, head g always runs on XCD g), then the query
  // tiles of one request, heaviest (last) first, then the requests. Workgroups running at the
  // same time on an XCD thus share one request's K/V stream in that XCD's L2.
  const int id = blockIdx.x;
  const int g = id % hkv;
  const int t = id / hkv;
  const int b = t / n_qtiles;
  const int qtile = n_qtiles - 1 - t % n_qtiles;

  // The request's six table entries in one vector load (lanes 0-5), then broadcast.
  int tv = 0;
  {
    const int tl = threadIdx.x & 63;
    if (tl < 6) tv = (tl < 2 ? cu_q : (tl < 4 ? cu_k : seg_indptr))[b + (tl & 1)];
  }
  const int q0 = __builtin_amdgcn_readlane(tv, 0);
  const int lq = __builtin_amdgcn_readlane(tv, 1) - q0;
  const int K = __builtin_amdgcn_readlane(tv, 3) - __builtin_amdgcn_readlane(tv, 2);
  const int seg_first = __builtin_amdgcn_readlane(tv, 4);
  const int seg_last = __builtin_amdgcn_readlane(tv, 5);
  const int p0 = qtile * kWidePos;
  if (p0 >= lq) return;
  const int hq = hkv * kGroup;
  if (qtile == n_qtiles - 1 && lq > n_qtiles * kWidePos)
    mark_uncovered_rows(out, lse, q0, n_qtiles * kWidePos, lq, hq, g);

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

  // Q fragments in registers: B operand of S^T = K Q^T. Lane holds d = 16 step + 8 h + (0..7)
  // of its row; rows past the request are zero (computed, never stored).
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + ((int64_t)(q0 + pos) * hq + head) * kHeadDim + 8 * h;
#pragma unroll
    for (int step = 0; step < 8; ++step)
      qf[step] = row_valid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * step) : bf16x8{};
  }

  // ---- HBM -> LDS copies, 16 instructions of 1 KiB per block and tensor, two per wave.
  // K instruction c = 2 w + i fills rows 4c .. 4c + 3 (lane L: row 4c + L / 16, the global chunk
  // (L % 16) ^ (row % 16), so that chunk c of row r lands at chunk position c ^ (r % 16)).
  // V instruction i of wave w fills d quarter w % 4 of rows 16 j .. 16 j + 15, j = 2 (w / 4) + i
  // (lane L: row 16 j + L / 4, 16 bytes at quarter column L % 4): quarter-major.
  BlockCursor kcur, vcur;
  kcur.init(segs, seg_first, seg_last);
  vcur.init(segs, seg_first, seg_last);
  const int64_t tok_stride = (int64_t)hkv * kHeadDim;
  const uint32_t tok_bytes = (uint32_t)hkv * kHeadDim * 2;
  const bf16_t* kbase = k_pool + (int64_t)g * kHeadDim;
  const bf16_t* vbase = v_pool + (int64_t)g * kHeadDim;
  const int krow0 = 8 * wave + (lane >> 4);  // K row of instruction i: krow0 + 4 i
  const int kch = lane & 15;
  const int vrow0 = 32 * (wave >> 2) + (lane >> 2);  // V row of instruction i: vrow0 + 16 i
  const uint32_t vcol = (uint32_t)(wave & 3) * 64 + (lane & 3) * 16;
  const uint32_t vdst0 = (uint32_t)(wave & 3) * 4096 + (uint32_t)(wave >> 2) * 2048;
  uint32_t koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    koff[i] = (uint32_t)(krow0 + 4 * i) * tok_bytes + ((kch ^ ((krow0 + 4 * i) & 15)) << 4);
    voff[i] = (uint32_t)(vrow0 + 16 * i) * tok_bytes + vcol;
  }
  // Fast case (the block inside one segment and inside the request's keys): row r of the block
  // is pool slot base + r, a scalar base plus a fixed per-thread offset. Otherwise every row is
  // looked up on its own (rows past K re-read key K - 1, masked later).
  auto issue_k = [&](int blk, char* dst) __attribute__((always_inline)) {
    const int kb0 = blk * kBlockN;
    const int last = min(kb0 + kBlockN, K) - 1;
    kcur.advance_to(kb0);
    lds_char_t* l = (lds_char_t*)dst + wave * 2048;
    if ((kb0 + kBlockN <= K) && (last - kcur.start < kcur.len)) {
      const auto r = block_rsrc(kbase + ((int64_t)kcur.off + (kb0 - kcur.start)) * tok_stride);
      copy16_buf_at<0>(r, (lds_void_t*)l, koff[0]);
      copy16_buf_at<1024>(r, (lds_void_t*)l, koff[1]);  // koff[1] >= 4 rows >= 1024 bytes
    } else {
      SegCursor c2;
      c2.segs = kcur.segs; c2.idx = kcur.idx; c2.end = kcur.end;
      c2.start = kcur.start; c2.off = kcur.off; c2.len = kcur.len;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = krow0 + 4 * i;
        const int64_t slot = c2.slot(min(kb0 + r, last));
        copy16_row<kOff32>(kbase, slot * tok_bytes + ((kch ^ (r & 15)) << 4), (lds_void_t*)(l + 1024 * i));
      }
    }
  };
  auto issue_v = [&](int blk, char* dst) __attribute__((always_inline)) {
    const int kb0 = blk * kBlockN;
    const int last = min(kb0 + kBlockN, K) - 1;
    vcur.advance_to(kb0);
    lds_char_t* l = (lds_char_t*)dst + vdst0;
    if ((kb0 + kBlockN <= K) && (last - vcur.start < vcur.len)) {
      const auto r = block_rsrc(vbase + ((int64_t)vcur.off + (kb0 - vcur.start)) * tok_stride);
      copy16_buf_at<0>(r, (lds_void_t*)l, voff[0]);
      copy16_buf_at<1024>(r, (lds_void_t*)l, voff[1]);  // voff[1] >= 16 rows >= 1024 bytes
    } else {
      SegCursor c2;
      c2.segs = vcur.segs; c2.idx = vcur.idx; c2.end = vcur.end;
      c2.start = vcur.start; c2.off = vcur.off; c2.len = vcur.len;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int64_t slot = c2.slot(min(kb0 + vrow0 + 16 * i, last));
        copy16_row<kOff32>(vbase, slot * tok_bytes + vcol, (lds_void_t*)(l + 1024 * i));
      }
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  bf16x8 pb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = bf16x8{};
  float m_run = kNoMax;
  float neg = 0.f;  // -m_run * scale_log2 once m_run holds a score
  float l_run = 0.f;
  const float grow_thr = kRescaleLog2 / scale_log2;  // move m_run when a block's max exceeds it by this
  const int G = lane >> 4;
  const int sl = lane & 15;
  // V^T operands (quarter-major V): lane reads rows 16 u + 4 h + sl / 4 (and + 8) at d offset
  // 16 (G % 2) + 4 (sl % 4) of quarter dt; every read is this per-lane offset plus a constant.
  const uint32_t vlane = (uint32_t)(4 * h + (sl >> 2)) * 64 + 32 * (G & 1) + 8 * (sl & 3);
  // K operands: chunk 2 step + h of row n sits at chunk position (2 step + h) ^ (n % 16).
  uint32_t kofs[8];
#pragma unroll
  for (int step = 0; step < 8; ++step) kofs[step] = (uint32_t)(n * 256 + (((2 * step + h) ^ (n & 15)) << 4));

  // MFMA phase of step j: O^T += V^T P^T for block j - 1, then S^T = K Q^T for block j. LDS
  // operands are read ahead of the MFMAs that use them (V one d tile ahead, K two k-steps
  // ahead).
  auto gemm_phase = [&](int j, const char* vprev, const char* kcurp) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (j >= 1) {
      const lds_char_t* vb = (const lds_char_t*)vprev + vlane;
      auto read_vt = [&](int dt, bf16x8 (&dst)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          bf16x4 lo = lds_read_tr16(vb + (dt * 4096 + u * 1024));
          bf16x4 hi = lds_read_tr16(vb + (dt * 4096 + u * 1024 + 512));
          dst[u][0] = lo[0]; dst[u][1] = lo[1]; dst[u][2] = lo[2]; dst[u][3] = lo[3];
          dst[u][4] = hi[0]; dst[u][5] = hi[1]; dst[u][6] = hi[2]; dst[u][7] = hi[3];
        }
      };
      bf16x8 va[2][4];
      read_vt(0, va[0]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        if (dt + 1 < 4) read_vt(dt + 1, va[(dt + 1) & 1]);
#pragma unroll
        for (int u = 0; u < 4; ++u) o[dt] = mfma32x32x16(va[dt & 1][u], pb[u], o[dt]);
        if (dt + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (j < n_blocks) {
      const lds_char_t* kb = (const lds_char_t*)kcurp;
      bf16x8 ka[3][2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        ka[st][0] = lds_read16(kb + kofs[st]);
        ka[st][1] = lds_read16(kb + kofs[st] + 32 * 256);
      }
#pragma unroll
      for (int step = 0; step < 8; ++step) {
        if (step + 2 < 8) {
          ka[(step + 2) % 3][0] = lds_read16(kb + kofs[step + 2]);
          ka[(step + 2) % 3][1] = lds_read16(kb + kofs[step + 2] + 32 * 256);
        }
        s0 = mfma32x32x16(ka[step % 3][0], qf[step], step == 0 ? f32x16{} : s0);
        s1 = mfma32x32x16(ka[step % 3][1], qf[step], step == 0 ? f32x16{} : s1);
        if (step + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
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
    // m_run starts at kNoMax, so the first block with a visible key always moves it (alpha is
    // then 0) and no step tests for infinities; neg stays 0 while a row has seen no key
    if (__builtin_amdgcn_ballot_w64(mx - m_run > grow_thr) != 0) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = fast_exp2((m_run - m_new) * scale_log2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      neg = m_run == kNoMax ? 0.f : -m_run * scale_log2;
    }
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

  // Step j: K(j) in slot j % 2 is read (S of block j), V(j-1) in slot (j-1) % 2 (PV of block
  // j-1). At its start the copies of K(j+1) into slot (j+1) % 2 and of V(j) into slot j % 2 are
  // issued: both slots were last read in step j-1, which ended with a barrier. Its last barrier
  // follows the wait for those copies. (A third slot, copying two steps ahead, measured no
  // faster on the chunked prefill.)
  auto step = [&](int j, auto r_c) __attribute__((always_inline)) {
    constexpr int R = decltype(r_c)::value;
    char* kread = R == 0 ? kr0 : kr1;
    char* kwrite = R == 0 ? kr1 : kr0;
    char* vread = R == 0 ? vr1 : vr0;
    char* vwrite = R == 0 ? vr0 : vr1;
    // Both cursors move first: a segment-table read waits for every vector memory operation
    // in flight, so it must not come after this step's first copies.
    if (j + 1 < n_blocks) kcur.advance_to((j + 1) * kBlockN);
    if (j < n_blocks) vcur.advance_to(j * kBlockN);
    if (j + 1 < n_blocks) issue_k(j + 1, kwrite);
    if (j < n_blocks) issue_v(j, vwrite);
    if (grp == 0) gemm_phase(j, vread, kread);
    else softmax_phase(j - 1);
    phase_barrier();
    if (grp == 1) gemm_phase(j, vread, kread);
    else softmax_phase(j);
    wait_vmem();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    phase_barrier();
  };

  if (n_blocks > 0) issue_k(0, kr0);
  wait_vmem();  // also the Q loads
  phase_barrier();
  if (n_blocks > 0) {
    // Both steps of a pair unconditionally inside the loop, the odd tail after it.
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


// ------------------------------------------------------------------------------------------
// Quad tiles: 128 rows (16 query positions x 8 heads) per workgroup of 4 waves, one wave per
// SIMD, 32 rows per wave, and two workgroups resident per CU (64 KiB of LDS each). Every wave
// runs S = K Q^T, the online softmax and O += P V of a block back to back; the MFMAs of one
// workgroup's wave overlap the vector work of the other workgroup's wave on the same SIMD, with
// no barrier coupling the two, and one workgroup's prologue and epilogue overlap the other's
// main loop. K and V blocks are double buffered: block j + 1 is copied from HBM into LDS while
// block j is consumed, and one barrier per block hands a slot from the readers to the copier.
constexpr int kQuadThreads = 256;

template <bool kCausal, bool kOff32>
__global__ __launch_bounds__(kQuadThreads, 2) void prefill_quad_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_pool,
    const bf16_t* __restrict__ v_pool, const Segment* __restrict__ segs,
    const int32_t* __restrict__ seg_indptr, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int batch, int hkv, int n_qtiles, int fold, float scale,
    float scale_log2, bf16_t* __restrict__ out, float* __restrict__ lse) {
  // One LDS array per (K|V, slot) so that the compiler sees the blocks being read never alias
  // the blocks being copied in. V has the larger alignment, which places it first, below
  // 64 KiB, where a V read is one per-lane register plus an immediate offset.
  __shared__ __attribute__((aligned(4096))) char lv0[kBlkBytes];
  __shared__ __attribute__((aligned(4096))) char lv1[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char lk0[kBlkBytes];
  __shared__ __attribute__((aligned(1024))) char lk1[kBlkBytes];

  // Every pointer argument in scalar registers before the first table read, so that all
  // kernel-argument loads share one memory round trip instead of being fetched as needed.
  asm volatile("" ::"s"(q), "s"(k_pool), "s"(v_pool), "s"(segs), "s"(seg_indptr), "s"(cu_q),
               "s"(cu_k), "s"(out), "s"(lse));

  // Work item: kv head fastest, so that with 8 kv heads every tile of head g lands on the same
  // XCD (workgroups are dealt round-robin over the 8 XCDs) and shares its L2. Query tiles go
  // heaviest (last) first; with fold > 0 (the whole grid resident at once, two workgroups per
  // CU) the second half of the grid goes lightest first instead, so that the workgroups sharing
  // a CU, dispatched one grid-half apart, have causal key counts that add up to about the same
  // total.
  const int id = blockIdx.x;
  const int per_tile = hkv * batch;
  const int rank = id / per_tile;
  const int qtile = (fold == 0 || rank < fold) ? n_qtiles - 1 - rank : rank - fold;
  const int rem = id % per_tile;
  const int b = rem / hkv;
  const int g = rem % hkv;
  // The request's six table entries in one vector load (lanes 0-5), then broadcast: one
  // memory round trip where scalar loads of the three tables would wait on each other.
  int tv = 0;
  {
    const int tl = threadIdx.x & 63;
    if (tl < 6) tv = (tl < 2 ? cu_q : (tl < 4 ? cu_k : seg_indptr))[b + (tl & 1)];
  }
  const int q0 = __builtin_amdgcn_readlane(tv, 0);
  const int lq = __builtin_amdgcn_readlane(tv, 1) - q0;
  const int K = __builtin_amdgcn_readlane(tv, 3) - __builtin_amdgcn_readlane(tv, 2);
  const int seg_first = __builtin_amdgcn_readlane(tv, 4);
  const int seg_last = __builtin_amdgcn_readlane(tv, 5);
  const int p0 = qtile * kPosPerTile;
  if (p0 >= lq) return;
  const int hq = hkv * kGroup;
  if (qtile == n_qtiles - 1 && lq > n_qtiles * kPosPerTile)
    mark_uncovered_rows(out, lse, q0, n_qtiles * kPosPerTile, lq, hq, g);
  const int kfull = kCausal ? min(K, K - lq + p0 + 1) : K;  // keys every row sees
  const int tend = kCausal ? min(K, K - lq + min(p0 + kPosPerTile, lq)) : K;
  const int nblk = max(0, (tend + kBlockN - 1) / kBlockN);  // key blocks the tile sees

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;  // row within the wave
  const int h = lane >> 5;  // which half of the k / m slots this lane holds
  const int head = g * kGroup + (n & 7);

  // Wave w holds positions p0 + 4w .. p0 + 4w + 3 of the tile.
  const int pos = p0 + wave * 4 + (n >> 3);
  const bool row_valid = pos < lq;
  const int row_limit = kCausal ? min(K, K - lq + pos + 1) : K;

  // Q fragments: B operand of S^T = K Q^T. Lane holds d = 16*step + 8*h + (0..7) of its row.
  bf16x8 qf[8];
  {
    const bf16_t* qrow = q + ((int64_t)(q0 + pos) * hq + head) * kHeadDim + 8 * h;
#pragma unroll
    for (int step = 0; step < 8; ++step)
      qf[step] = row_valid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * step) : bf16x8{};
  }

  // ---- HBM -> LDS copies: 16 copy instructions of 1 KiB per block and tensor, four per wave.
  // K instruction c = 4 * wave + k fills rows 4c .. 4c + 3 (256 B each, swizzled: lane L holds
  // chunk (L % 16) ^ (row % 16) of row 4c + L / 16). V instruction c fills rows 16k .. 16k + 15
  // of d quarter `wave` (64 B each): lane L copies 16 B of row 16k + L / 4. Each wave writes
  // only bytes [4096 w, 4096 w + 4096) of every K and V slot.
  BlockCursor cur;
  cur.init(segs, seg_first, seg_last);
  const int64_t tok_stride = (int64_t)hkv * kHeadDim;
  const uint32_t tok_bytes = (uint32_t)hkv * kHeadDim * 2;
  const bf16_t* kbase = k_pool + (int64_t)g * kHeadDim;
  const bf16_t* vbase = v_pool + (int64_t)g * kHeadDim;
  const int krow0 = 16 * wave + (lane >> 4);  // K row of copy k: krow0 + 4k
  const int vrow0 = lane >> 2;                // V row of copy k: vrow0 + 16k
  const uint32_t vcol = (uint32_t)wave * 64 + (lane & 3) * 16;
  uint32_t koff[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    koff[k] = (uint32_t)(krow0 + 4 * k) * tok_bytes + (((lane & 15) ^ ((krow0 + 4 * k) & 15)) << 4);
  const uint32_t voff = (uint32_t)vrow0 * tok_bytes + vcol;

  // Copies of block blk into (kdst, vdst). Fast case (the block inside one segment and inside
  // the request's keys): row r of the block is pool slot base + r for the whole workgroup, a
  // scalar base plus a fixed per-thread offset. Otherwise every row is looked up on its own
  // (rows past K re-read key K - 1).
  // Copies of block blk into (kdst, vdst). Fast case (the block inside one segment and inside
  // the request's keys): row r of the block is pool slot base + r for the whole workgroup, a
  // scalar base plus a fixed per-thread offset; its 8 copies are returned pending, to be issued
  // one after each pair of MFMAs of the next S^T (copy_one). Otherwise every row is looked up on
  // its own (rows past K re-read key K - 1) and the copies are issued at once.
  struct Pending {
    bool fast;
    __amdgpu_buffer_rsrc_t kr, vr;
    lds_char_t *lk, *lv;
  };
  auto copy_one = [&](const Pending& pc, int x) __attribute__((always_inline)) {
    if (x < 4) copy16_buf(pc.kr, (lds_void_t*)(pc.lk + 1024 * x), koff[x]);
    else copy16_buf(pc.vr, (lds_void_t*)(pc.lv + 1024 * (x - 4)), voff + (uint32_t)(16 * (x - 4)) * tok_bytes);
  };
  auto issue_copies = [&](int blk, char* kdst, char* vdst) __attribute__((always_inline)) {
    Pending pc;
    const int kb0 = blk * kBlockN;
    const int last = min(kb0 + kBlockN, K) - 1;
    cur.advance_to(kb0);
    // the wave's LDS destinations as scalars: every copy's M0 is then a scalar add
    lds_char_t* lk = (lds_char_t*)(uintptr_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)((lds_char_t*)kdst + wave * 4096));
    lds_char_t* lv = (lds_char_t*)(uintptr_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)((lds_char_t*)vdst + wave * 4096));
    pc.lk = lk;
    pc.lv = lv;
    pc.fast = (kb0 + kBlockN <= K) && (last - cur.start < cur.len);
    if (pc.fast) {
      const int64_t base = (int64_t)cur.off + (kb0 - cur.start);
      pc.kr = block_rsrc(kbase + base * tok_stride);
      pc.vr = block_rsrc(vbase + base * tok_stride);
    } else {
      pc.kr = block_rsrc(kbase);
      pc.vr = pc.kr;
      SegCursor c2;
      c2.segs = cur.segs;
      c2.idx = cur.idx;
      c2.end = cur.end;
      c2.start = cur.start;
      c2.off = cur.off;
      c2.len = cur.len;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = krow0 + 4 * k;
        const int64_t slot = c2.slot(min(kb0 + r, last));
        copy16_row<kOff32>(kbase, slot * tok_bytes + (((lane & 15) ^ (r & 15)) << 4), (lds_void_t*)(lk + 1024 * k));
      }
      c2.segs = cur.segs;
      c2.idx = cur.idx;
      c2.end = cur.end;
      c2.start = cur.start;
      c2.off = cur.off;
      c2.len = cur.len;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t slot = c2.slot(min(kb0 + vrow0 + 16 * k, last));
        copy16_row<kOff32>(vbase, slot * tok_bytes + vcol, (lds_void_t*)(lv + 1024 * k));
      }
    }
    return pc;
  };

  // LDS operand offsets (K swizzled row-major, V quarter-major; see the layouts at the top).
  const int G = lane >> 4;
  const int sl = lane & 15;
  const uint32_t vlane = (uint32_t)(4 * h + (sl >> 2)) * 64 + 32 * (G & 1) + 8 * (sl & 3);
  uint32_t kofs[8];
#pragma unroll
  for (int step = 0; step < 8; ++step) kofs[step] = n * 256 + (((2 * step + h) ^ (n & 15)) << 4);

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m_run = kNoMax;
  float neg = 0.f;  // -m_run * scale_log2 once m_run holds a score
  float l_run = 0.f;  // this lane's keys only; the row total is l + l of lane ^ 32
  const float grow_thr = kRescaleLog2 / scale_log2;  // move m_run when a block's max exceeds it by this

  // One block: S^T = K Q^T, online softmax, O^T += V^T P^T. LDS operands are read ahead of the
  // MFMAs that use them (K two steps ahead, V one d tile ahead).
  auto block_step = [&](int blk, const char* kslot, const char* vslot, const Pending& pc, bool more) __attribute__((always_inline)) {
    const lds_char_t* kb = (const lds_char_t*)kslot;
    const lds_char_t* vb = (const lds_char_t*)vslot;
    f32x16 s0, s1;
    {
      bf16x8 ka[3][2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        ka[st][0] = lds_read16(kb + kofs[st]);
        ka[st][1] = lds_read16(kb + kofs[st] + 32 * 256);
      }
#pragma unroll
      for (int step = 0; step < 8; ++step) {
        if (step + 2 < 8) {
          ka[(step + 2) % 3][0] = lds_read16(kb + kofs[step + 2]);
          ka[(step + 2) % 3][1] = lds_read16(kb + kofs[step + 2] + 32 * 256);
        }
        s0 = mfma32x32x16(ka[step % 3][0], qf[step], step == 0 ? f32x16{} : s0);
        s1 = mfma32x32x16(ka[step % 3][1], qf[step], step == 0 ? f32x16{} : s1);
        if (more && pc.fast) copy_one(pc, step);
        if (step + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // V^T operand i of the block (d tile i / 4, key step i % 4): two transposing reads. The
    // PV MFMAs take them in order from a ring of 8, each read kLead MFMAs ahead of its use, so
    // that at most 2 * kLead + 2 reads are in flight and the wait before MFMA i can leave the
    // later ones pending (the LDS counter holds at most 15).
    constexpr int kLead = 6;
    auto read_vt = [&](int i) __attribute__((always_inline)) {
      bf16x4 lo = lds_read_tr16(vb + vlane + ((i >> 2) * 4096 + (i & 3) * 1024));
      bf16x4 hi = lds_read_tr16(vb + vlane + ((i >> 2) * 4096 + (i & 3) * 1024 + 512));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    bf16x8 va[8];
#pragma unroll
    for (int i = 0; i < kLead; ++i) va[i] = read_vt(i);

    // ---- online softmax of the block (keys on the M side: a lane holds 32 scores of its row)
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
    // m_run starts at kNoMax, so the first block with a visible key always moves it (alpha is
    // then 0) and no step tests for infinities; neg stays 0 while a row has seen no key
    if (__builtin_amdgcn_ballot_w64(mx - m_run > grow_thr) != 0) {
      const float m_new = __builtin_fmaxf(m_run, mx);
      const float alpha = fast_exp2((m_run - m_new) * scale_log2);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      neg = m_run == kNoMax ? 0.f : -m_run * scale_log2;
    }
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = fast_exp2(__builtin_fmaf(s0[e], scale_log2, neg));
      s1[e] = fast_exp2(__builtin_fmaf(s1[e], scale_log2, neg));
      ps0 += s0[e];
      ps1 += s1[e];
    }
    l_run += ps0 + ps1;
    bf16x8 pb[4];
    pb[0] = to_bf16x8(s0[0], s0[1], s0[2], s0[3], s0[4], s0[5], s0[6], s0[7]);
    pb[1] = to_bf16x8(s0[8], s0[9], s0[10], s0[11], s0[12], s0[13], s0[14], s0[15]);
    pb[2] = to_bf16x8(s1[0], s1[1], s1[2], s1[3], s1[4], s1[5], s1[6], s1[7]);
    pb[3] = to_bf16x8(s1[8], s1[9], s1[10], s1[11], s1[12], s1[13], s1[14], s1[15]);

    // ---- O^T[d][row] += V^T P^T
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      o[i >> 2] = mfma32x32x16(va[i & 7], pb[i & 3], o[i >> 2]);
      if (i + kLead < 16) va[(i + kLead) & 7] = read_vt(i + kLead);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kLead < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- normalise and store the tile's rows. O^T column n is row n of the wave
  // (lane holds d = 32 dt + 8 k4 + 4 h + (0..3)); the rows go through the wave's own 8 KiB of
  // an LDS slot nobody reads any more (rows 0-15 in its K part, 16-31 in its V part, 16-byte
  // chunk c of row r at chunk position c ^ (r % 16)) and leave it as whole 256-byte rows: each
  // store instruction writes 4 heads of one position, 1 KiB contiguous.
  auto store_rows = [&](char* kslot, char* vslot) __attribute__((always_inline)) {
    const float l_tot = sum_xor32(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    lds_char_t* wk = (lds_char_t*)kslot + wave * 4096;
    lds_char_t* wv = (lds_char_t*)vslot + wave * 4096;
    lds_char_t* wrow = (n < 16 ? wk : wv) + (n & 15) * 256 + 8 * h;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (bf16_t)(o[dt][4 * k4 + t] * inv);
        *(lds_bf16x4_t*)(wrow + (((4 * dt + k4) ^ (n & 15)) << 4)) = v;
      }
    }
    if (lse != nullptr && h == 0 && row_valid)
      lse[(int64_t)(q0 + pos) * hq + head] = l_tot > 0.f ? m_run * scale + __logf(l_tot) : -INFINITY;
    const int rr = lane >> 4, cc = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * (i & 3) + rr;  // row within its 16-row half
      const bf16x8 v = lds_read16((i < 4 ? wk : wv) + r * 256 + ((cc ^ r) << 4));
      const int ps = p0 + wave * 4 + (i >> 1);
      if (ps < lq)
        *reinterpret_cast<bf16x8*>(out + ((int64_t)(q0 + ps) * hq + g * kGroup + 4 * (i & 1) + rr) * kHeadDim +
                                   8 * cc) = v;
    }
  };

  // Block j runs from slot j & 1; the copies of block j + 1 go to the other slot, which every
  // wave finished reading before the barrier that ended the step before.
  if (nblk > 0) {
    {
      const Pending p0 = issue_copies(0, lk0, lv0);
      if (p0.fast)
#pragma unroll
        for (int x = 0; x < 8; ++x) copy_one(p0, x);
    }
    wait_vmem();  // also the Q loads
    phase_barrier();
    for (int j = 0; j < nblk; j += 2) {
      const bool more1 = j + 1 < nblk;
      Pending pc = more1 ? issue_copies(j + 1, lk1, lv1) : Pending{};
      block_step(j, lk0, lv0, pc, more1);
      wait_vmem();
      phase_barrier();
      if (!more1) break;
      const bool more2 = j + 2 < nblk;
      pc = more2 ? issue_copies(j + 2, lk0, lv0) : Pending{};
      block_step(j + 1, lk1, lv1, pc, more2);
      wait_vmem();
      phase_barrier();
    }
  }
  // every wave is past the last barrier: all slots are free
  store_rows(lk0, lv0);
}

}  // namespace

// Launch. Two tilings: 256-row tiles halve the L2->LDS traffic and are used whenever they
// still give at least two workgroups per compute unit; otherwise the 128-row quad tiles keep
// more compute units busy on small batches. SEG_ATTN_PREFILL_TILE=128|256 forces one of them.
hipError_t launch_prefill(const void* q, const void* k_pool, const void* v_pool, const void* segs,
                          const int32_t* seg_indptr, const int32_t* cu_q, const int32_t* cu_k,
                          int batch, int max_seqlen_q, int hkv, int64_t pool_size, float scale, int causal,
                          void* out, float* lse, int cu_count, int force_tile, hipStream_t stream) {
  const float scale_log2 = scale * 1.4426950408889634f;
  // Rows looked up one by one are copied through a buffer when every byte offset from a kv head's
  // first pool row fits in 32 bits (pools up to 16M token x kv-head rows), else through flat
  // addresses.
  const bool off32 = pool_size * hkv * kHeadDim * 2 <= 0xFFFFFFF0LL;
  const int64_t wide_tiles = (int64_t)((max_seqlen_q + kWidePos - 1) / kWidePos) * hkv * batch;
  const bool wide = force_tile == 256 || (force_tile != 128 && wide_tiles >= 2LL * cu_count);
  if (wide) {
    const int n_qtiles = (max_seqlen_q + kWidePos - 1) / kWidePos;
    if (wide_tiles == 0) return hipSuccess;
    auto kern = causal ? (off32 ? prefill_wide_kernel<true, true> : prefill_wide_kernel<true, false>)
                       : (off32 ? prefill_wide_kernel<false, true> : prefill_wide_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)wide_tiles), dim3(kThreads), 0, stream, (const bf16_t*)q,
                       (const bf16_t*)k_pool, (const bf16_t*)v_pool, (const Segment*)segs, seg_indptr,
                       cu_q, cu_k, batch, hkv, n_qtiles, scale, scale_log2, (bf16_t*)out, lse);
    return hipGetLastError();
  }
  const int n_qtiles = (max_seqlen_q + kPosPerTile - 1) / kPosPerTile;
  const int64_t grid = (int64_t)n_qtiles * hkv * batch;
  if (grid == 0) return hipSuccess;
  auto kern = causal ? (off32 ? prefill_quad_kernel<true, true> : prefill_quad_kernel<true, false>)
                     : (off32 ? prefill_quad_kernel<false, true> : prefill_quad_kernel<false, false>);
  const int fold = (causal && grid <= 2LL * cu_count) ? (n_qtiles + 1) / 2 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kQuadThreads), 0, stream, (const bf16_t*)q,
                     (const bf16_t*)k_pool, (const bf16_t*)v_pool, (const Segment*)segs, seg_indptr,
                     cu_q, cu_k, batch, hkv, n_qtiles, fold, scale, scale_log2, (bf16_t*)out, lse);
  return hipGetLastError();
}

}  // namespace segattn
