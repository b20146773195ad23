// Decode kernels: one query token per request against all of its segmented keys.
//
// Work units. Each request's keys are cut into chunks of `len` keys (the last one shorter); a
// unit is one (chunk, kv head) pair, whose result is the blockwise partial attention of the
// FlashAccel article ("data layout": attention computed per block of the KV, then reduced per
// request). A one-workgroup plan kernel lists the chunks of all requests on the device, so no
// launch slot is spent on requests shorter than the longest, and chooses `len` from the total
// key count so that every compute unit gets about a dozen units.
//
// Split pass. One persistent workgroup per compute unit walks its share of the units. Its 4
// waves split each unit's tiles round robin (tile i to wave i % 4) and stream them through a
// private double buffer in LDS, filled by direct HBM->LDS copies. A wave issues the copies of
// its next two tiles before it waits for the current one, and its stream runs on across unit
// boundaries, so two tiles per wave stay in flight the whole time: at a unit's end the waves
// only meet to combine their (m, l, O) states while the next unit's tiles are already on their
// way. The 8 query heads of kv head g are the columns of one MFMA tile (PackGQA, FlashPrefill
// V2 abstract): every K/V byte is read from HBM once per group.
//   S^T[key][head] = K Q^T   (MFMA 16x16x32 bf16, keys on M; columns 8..15 are padding)
//   O^T[d][head]  += V^T P^T (V^T via the transposing LDS read)
// A unit that covers a whole request writes the output; otherwise it writes a partial
// (O_s, LSE_s) for the merge pass.
//
// FP8 pools (OCP E4M3FN codes with one fp32 scale per token and kv head) are converted to bf16
// exactly on the way into the MFMAs; the key scale multiplies the scores, the value scale the
// probabilities, so the arithmetic equals bf16 attention over the dequantised pool.
//
// Merge pass: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s per (request, head).
#include "common.hpp"

namespace segattn {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kDecThreads = kWaves * 64;
constexpr int kQBufs = 3;           // Q tiles of the units a wave may be working ahead into
constexpr int kQBytes = kGroup * kHeadDim * 2;  // 2 KiB: the 8 query rows of one unit

template <int kFp8>
struct DecodeCfg;
template <>
struct DecodeCfg<0> {  // bf16: 32 keys per wave tile, 256 B rows
  static constexpr int kTile = 32;
  static constexpr int kRowBytes = 256;
  static constexpr int kChunks = 16;         // 16 B pieces per row
  static constexpr int kRowsPerCopy = 4;     // rows one 64-lane copy instruction covers
  static constexpr int kKBytes = kTile * kRowBytes;  // 8 KiB
  static constexpr int kScaleBytes = 0;
  static constexpr int kCopies = 2 * (kTile / kRowsPerCopy);  // K and V copy instructions per tile
};
template <>
struct DecodeCfg<1> {  // fp8: 64 keys per wave tile, 128 B rows, + k/v scales
  static constexpr int kTile = 64;
  static constexpr int kRowBytes = 128;
  static constexpr int kChunks = 8;
  static constexpr int kRowsPerCopy = 8;
  static constexpr int kKBytes = kTile * kRowBytes;  // 8 KiB
  static constexpr int kScaleBytes = kTile * 4;      // 256 B each
  static constexpr int kCopies = 2 * (kTile / kRowsPerCopy) + 2;
};

template <int kFp8>
struct DecodeLayout {
  using C = DecodeCfg<kFp8>;
  // one wave's stage: K tile, V tile, k scales, v scales
  static constexpr int kStageBytes = 2 * C::kKBytes + 2 * C::kScaleBytes;
  static constexpr int kCombFloats = kGroup * kHeadDim + 4 * kGroup;  // O^T, (m, l) of one wave
};

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt at their no-wait maxima (gfx9 encoding: vmcnt
// bits 3:0 and 15:14).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// bf16 rows: chunk c (16 B) of row r stored at position c ^ (r % 16) for K and c ^ vswz(r) for V.
__device__ __forceinline__ int vswz16(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }

// A operands of O^T += V^T P^T for the 32 keys 32*kk .. 32*kk + 31 of a bf16 V tile in LDS
// (256 B rows, chunk c of row r at c ^ vswz16(r)): vt[dt][j] = V[key(j)][16*dt + col] with
// key(j) = 32*kk + 4*grp + j for j < 4 and 32*kk + 16 + 4*grp + (j - 4) otherwise. Each half is
// one transposing read: lane (grp, col) addresses row 32*kk + 4*grp + col/4 (+16) at column
// 16*dt + 4*(col%4). The 16 reads are issued from one asm block that also waits for them:
// through the builtin the compiler cannot tell which LDS bytes a read touches, and waits for
// every copy still in flight before it.
__device__ __forceinline__ void v_transposed(const lds_char_t* vb, int kk, bf16x8 (&vt)[8]) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int ra = 32 * kk + 4 * grp + (col >> 2);
  const int rb = ra + 16;
  const int within = 8 * (col & 1);
  uint32_t pa[8], pb[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const int chunk = 2 * dt + ((col & 3) >> 1);
    pa[dt] = (uint32_t)(uintptr_t)(vb + ra * 256 + ((chunk ^ vswz16(ra)) << 4) + within);
    pb[dt] = (uint32_t)(uintptr_t)(vb + rb * 256 + ((chunk ^ vswz16(rb)) << 4) + within);
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 r[16];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %17\n\t"
      "ds_read_b64_tr_b16 %2, %18\n\t"
      "ds_read_b64_tr_b16 %3, %19\n\t"
      "ds_read_b64_tr_b16 %4, %20\n\t"
      "ds_read_b64_tr_b16 %5, %21\n\t"
      "ds_read_b64_tr_b16 %6, %22\n\t"
      "ds_read_b64_tr_b16 %7, %23\n\t"
      "ds_read_b64_tr_b16 %8, %24\n\t"
      "ds_read_b64_tr_b16 %9, %25\n\t"
      "ds_read_b64_tr_b16 %10, %26\n\t"
      "ds_read_b64_tr_b16 %11, %27\n\t"
      "ds_read_b64_tr_b16 %12, %28\n\t"
      "ds_read_b64_tr_b16 %13, %29\n\t"
      "ds_read_b64_tr_b16 %14, %30\n\t"
      "ds_read_b64_tr_b16 %15, %31\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]),
        "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(pa[0]), "v"(pb[0]), "v"(pa[1]), "v"(pb[1]), "v"(pa[2]), "v"(pb[2]), "v"(pa[3]),
        "v"(pb[3]), "v"(pa[4]), "v"(pb[4]), "v"(pa[5]), "v"(pb[5]), "v"(pa[6]), "v"(pb[6]),
        "v"(pa[7]), "v"(pb[7])
      : "memory");
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    i32x4 w;
    w[0] = (int)r[2 * dt][0];
    w[1] = (int)r[2 * dt][1];
    w[2] = (int)r[2 * dt + 1][0];
    w[3] = (int)r[2 * dt + 1][1];
    vt[dt] = __builtin_bit_cast(bf16x8, w);
  }
}

// Forward walk over one request's segments with every value wave-uniform, so table reads are
// scalar loads: they never join the vector-memory queue that the tile copies use.
struct ScalarCursor {
  const Segment* segs;
  int idx, end, start, off, len;
  __device__ __forceinline__ void fetch() {
    idx = rfl(idx);
    if (idx < end) {
      i32x2 v = *reinterpret_cast<const i32x2*>(segs + idx);
      off = rfl(v[0]);
      len = rfl(v[1]);
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

// Where a unit's keys are: chunk c of request b holds keys [kbeg, kstop).
struct UnitInfo {
  int valid, c, g, b, kbeg, kstop, n_tiles;
};

// ------------------------------------------------------------------------------------------
// Plan: chunk length, per-request chunk offsets and the chunk -> (request, index) table.
// hdr[0] = len, hdr[1] = number of chunks listed (at most max_chunks).
__global__ __launch_bounds__(1024) void decode_plan_kernel(
    const int32_t* __restrict__ cu_k, int batch, int hkv, int forced_len, int min_len,
    int target_units, int max_chunks, int32_t* __restrict__ hdr, int32_t* __restrict__ chunk_base,
    int32_t* __restrict__ tab) {
  __shared__ int scan[1024];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  int len = forced_len;
  if (len <= 0) {
    const int64_t total = (int64_t)cu_k[batch] - cu_k[0];
    int64_t want = (total * hkv + target_units - 1) / target_units;
    want = (want + 63) / 64 * 64;
    len = (int)(want < min_len ? min_len : (want > (1 << 30) ? (1 << 30) : want));
  }
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int b0 = 0; b0 < batch; b0 += 1024) {
    const int b = b0 + tid;
    int n = 0;
    if (b < batch) {
      const int K = cu_k[b + 1] - cu_k[b];
      n = K > 0 ? (K + len - 1) / len : 0;
    }
    scan[tid] = n;
    __syncthreads();
    for (int s = 1; s < 1024; s <<= 1) {  // inclusive Hillis-Steele scan
      const int add = tid >= s ? scan[tid - s] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int carry = carry_s;
    const int first = carry + scan[tid] - n;
    if (b < batch) {
      chunk_base[b] = first;
      for (int k = 0; k < n && first + k < max_chunks; ++k) {
        tab[2 * (first + k)] = b;
        tab[2 * (first + k) + 1] = k;
      }
    }
    __syncthreads();
    if (tid == 1023) carry_s = carry + scan[1023];
    __syncthreads();
  }
  if (tid == 0) {
    chunk_base[batch] = carry_s;
    hdr[0] = len;
    hdr[1] = carry_s < max_chunks ? carry_s : max_chunks;
  }
}

// ------------------------------------------------------------------------------------------
// Split pass.
template <int kFp8>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const bf16_t* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const Segment* __restrict__ segs, const int32_t* __restrict__ seg_indptr,
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ hdr,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ tab, int hkv,
    int xcd_spread, float scale, float scale_log2, float* __restrict__ ws_o,
    float* __restrict__ ws_lse, bf16_t* __restrict__ out, float* __restrict__ lse) {
  using C = DecodeCfg<kFp8>;
  using L = DecodeLayout<kFp8>;
  // Separate objects for the two stages, the combine area and the Q tiles: the compiler then
  // sees that reading one stage cannot touch the copies still landing in the other, and adds
  // no wait for them.
  __shared__ __attribute__((aligned(1024))) char st0[kWaves * L::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char st1[kWaves * L::kStageBytes];
  __shared__ __attribute__((aligned(16))) float comb[kWaves * L::kCombFloats];
  __shared__ __attribute__((aligned(16))) char qbuf[kQBufs * kQBytes];

  const int len = rfl(hdr[0]);
  const int n_units = rfl(hdr[1]) * hkv;
  const int grid = gridDim.x;
  // Unit order u = c * hkv + g, dealt round robin. With 8 kv heads and a grid that is a
  // multiple of 64, the slot permutation puts the 8 heads of a chunk on workgroups of the same
  // XCD (workgroups go to XCD id % 8), where they share the chunk's scale lines in L2.
  int slot = blockIdx.x;
  if (xcd_spread) {
    const int per = grid >> 3;
    slot = rfl((blockIdx.x % per) * 8 + blockIdx.x / per);
  }
  if (slot >= n_units) return;
  const int my_units = rfl((n_units - slot + grid - 1) / grid);

  const int tid = threadIdx.x;
  const int wave = rfl(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;  // head column of the MFMA tile (>= 8 is padding)
  const int grp = lane >> 4;  // 0..3
  const int hq = hkv * kGroup;
  const int64_t tok_bytes = (int64_t)hkv * C::kRowBytes;

  // Every field is wave-uniform and kept in scalar registers (readfirstlane after each integer
  // division, which the compiler does on the vector ALU).
  auto unit_info = [&](int r) __attribute__((always_inline)) {
    UnitInfo u;
    const int id = slot + r * grid;
    u.valid = r < my_units;
    u.c = u.valid ? rfl(id / hkv) : 0;
    u.g = rfl(id - u.c * hkv);
    const i32x2 t = *reinterpret_cast<const i32x2*>(tab + 2 * u.c);
    u.b = rfl(t[0]);
    const int k = rfl(t[1]);
    const int K = rfl(cu_k[u.b + 1] - cu_k[u.b]);
    u.kbeg = rfl(k * len);
    u.kstop = rfl(min(K, u.kbeg + len));
    u.n_tiles = u.valid ? rfl((u.kstop - u.kbeg + C::kTile - 1) / C::kTile) : 0;
    return u;
  };

  // ---- issue side: this wave's next tile
  UnitInfo iu = unit_info(0);
  int it = wave;  // tile index inside unit iu
  int ir = 0;     // ordinal of unit iu among this workgroup's units
  ScalarCursor cur;
  cur.init(segs, seg_indptr[iu.b], seg_indptr[iu.b + 1]);
  auto q_copy = [&](const UnitInfo& u, int r) __attribute__((always_inline)) {
    // wave 0 copies the unit's 8 query rows (2 KiB, contiguous) into Q buffer r % 3
    const char* src = (const char*)(q + ((int64_t)u.b * hq + u.g * kGroup) * kHeadDim) + lane * 16;
    lds_char_t* dst = (lds_char_t*)qbuf + (r % kQBufs) * kQBytes;
    copy16_to_lds(src, (lds_void_t*)dst);
    copy16_to_lds(src + 1024, (lds_void_t*)(dst + 1024));
  };
  if (wave == 0) q_copy(iu, 0);
  // move to the next unit in which this wave has a tile (wave 0 has one in every unit)
  auto next_unit = [&]() __attribute__((always_inline)) {
    while (true) {
      ++ir;
      iu = unit_info(ir);
      if (!iu.valid) return;
      cur.init(segs, seg_indptr[iu.b], seg_indptr[iu.b + 1]);
      if (wave == 0) q_copy(iu, ir);
      it = wave;
      if (it < iu.n_tiles) return;
    }
  };
  if (it >= iu.n_tiles) next_unit();

  struct Meta {
    int r, k0, kstop;
  };
  // Issue the copies of tile (iu, it) into this wave's part of stage `st`; returns its metadata.
  auto issue = [&](char* st) __attribute__((always_inline)) {
    Meta m;
    m.r = ir;
    m.k0 = iu.kbeg + it * C::kTile;
    m.kstop = iu.kstop;
    lds_char_t* kb = (lds_char_t*)st + wave * L::kStageBytes;
    lds_char_t* vb = kb + C::kKBytes;
    const int last = min(m.k0 + C::kTile, m.kstop) - 1;
    cur.advance_to(m.k0);
    const bool fast = (m.k0 + C::kTile <= m.kstop) && (last - cur.start < cur.len);
    const int rsub = lane / C::kChunks;
    const int cpos = lane % C::kChunks;
    constexpr int kN = C::kTile / C::kRowsPerCopy;
    // pool slot of each of this lane's kN rows
    int64_t slot_of[kN];
    if (fast) {
      const int64_t base = (int64_t)cur.off + (m.k0 - cur.start);
#pragma unroll
      for (int i = 0; i < kN; ++i) slot_of[i] = base + C::kRowsPerCopy * i + rsub;
    } else {
      // Rows of the tile that straddle segments (or lie past the unit's end, which re-read
      // the unit's last key and are masked later): walk the overlapped segments with a
      // scalar copy of the cursor.
#pragma unroll
      for (int i = 0; i < kN; ++i) slot_of[i] = 0;
      ScalarCursor c2 = cur;
      while (true) {
#pragma unroll
        for (int i = 0; i < kN; ++i) {
          const int j = min(m.k0 + C::kRowsPerCopy * i + rsub, last);
          if (j - c2.start >= 0 && j - c2.start < c2.len) slot_of[i] = (int64_t)c2.off + (j - c2.start);
        }
        if (last - c2.start < c2.len) break;
        c2.start += c2.len;
        ++c2.idx;
        c2.fetch();
      }
    }
    const char* kbase = (const char*)k_pool + (int64_t)iu.g * C::kRowBytes;
    const char* vbase = (const char*)v_pool + (int64_t)iu.g * C::kRowBytes;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int r = C::kRowsPerCopy * i + rsub;
      int kc, vc;
      if constexpr (kFp8 == 0) {
        kc = cpos ^ (r & 15);
        vc = cpos ^ vswz16(r);
      } else {
        kc = cpos ^ (r & 7);
        vc = kc;
      }
      const int64_t row = slot_of[i] * tok_bytes;
      copy16_to_lds(kbase + row + kc * 16, (lds_void_t*)(kb + i * 1024));
      copy16_to_lds(vbase + row + vc * 16, (lds_void_t*)(vb + i * 1024));
    }
    if constexpr (kFp8 == 1) {
      // scales: lane L copies those of row L
      const int j = min(m.k0 + lane, last);
      int64_t s;
      if (fast) {
        s = (int64_t)cur.off + (j - cur.start);
      } else {
        s = 0;
        ScalarCursor c2 = cur;
        while (true) {
          if (j - c2.start >= 0 && j - c2.start < c2.len) s = (int64_t)c2.off + (j - c2.start);
          if (last - c2.start < c2.len) break;
          c2.start += c2.len;
          ++c2.idx;
          c2.fetch();
        }
      }
      copy4_to_lds(k_scale + s * hkv + iu.g, (lds_void_t*)(vb + C::kKBytes));
      copy4_to_lds(v_scale + s * hkv + iu.g, (lds_void_t*)(vb + C::kKBytes + C::kScaleBytes));
    }
    // advance to this wave's next tile
    it += kWaves;
    if (it >= iu.n_tiles) next_unit();
    return m;
  };

  // ---- compute side
  bf16x8 qf[4];  // B operand of S^T: lane holds d = 32*step + 8*grp + (0..7) of head `col`
  f32x4 o[8];
  float m_run, l_run;
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{};
    m_run = -INFINITY;
    l_run = 0.f;
  };
  auto load_q = [&](int r) __attribute__((always_inline)) {
    // Read through inline asm: the compiler would otherwise wait for every copy in flight
    // before this read (the copies of wave 0 into qbuf are invisible to the other waves'
    // counters). Its completion was ensured before the barrier that precedes this call.
    const int row = col < kGroup ? col : 0;
    const uint32_t a = (uint32_t)(uintptr_t)((lds_char_t*)qbuf + (r % kQBufs) * kQBytes) +
                       row * (kHeadDim * 2) + grp * 16;
    i32x4 v0, v1, v2, v3;
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:64\n\t"
        "ds_read_b128 %2, %4 offset:128\n\t"
        "ds_read_b128 %3, %4 offset:192\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)  // early clobber: a is read by all four
        : "v"(a)
        : "memory");
    const bool real = col < kGroup;
    qf[0] = real ? __builtin_bit_cast(bf16x8, v0) : bf16x8{};
    qf[1] = real ? __builtin_bit_cast(bf16x8, v1) : bf16x8{};
    qf[2] = real ? __builtin_bit_cast(bf16x8, v2) : bf16x8{};
    qf[3] = real ? __builtin_bit_cast(bf16x8, v3) : bf16x8{};
  };

  // Combine the 4 waves' states for unit r and write the output or the partial.
  auto flush = [&](int r) __attribute__((always_inline)) {
    const UnitInfo u = unit_info(r);
    const int nb = rfl(chunk_base[u.b + 1] - chunk_base[u.b]);
    const float l_col = sum_xor32(sum_xor16(l_run));
    float* red = comb + wave * L::kCombFloats;
    if (col < kGroup) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[col * kHeadDim + 16 * dt + 4 * grp + i] = o[dt][i];
      if (grp == 0) {
        // written through inline asm: this store alone drew a wait for every copy in flight
        // from the compiler, which cannot place it apart from the stage buffers
        f32x4 ml = f32x4{};
        ml[0] = m_run;
        ml[1] = l_col;
        const uint32_t a = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) float*)red + kGroup * kHeadDim + 4 * col);
        asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(ml) : "memory");
      }
    }
    wait_lds();
    wg_barrier();
    const int hh = tid >> 5;        // head 0..7
    const int d4 = (tid & 31) * 4;  // 4 consecutive d
    float mw[kWaves], lw[kWaves];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* rw = comb + w * L::kCombFloats;
      const f32x4 ml = *reinterpret_cast<const f32x4*>(rw + kGroup * kHeadDim + 4 * hh);
      mw[w] = ml[0];
      lw[w] = ml[1];
      M = fmaxf(M, mw[w]);
    }
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float Lsum = 0.f;
    f32x4 acc = f32x4{};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float cw = fast_exp2((mw[w] - M_use) * scale_log2);
      Lsum += cw * lw[w];
      f32x4 v = *(const f32x4*)(comb + w * L::kCombFloats + hh * kHeadDim + d4);
      acc += cw * v;
    }
    const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
    acc *= inv;
    const float lse_v = Lsum > 0.f ? M * scale + __logf(Lsum) : -INFINITY;
    const int head = u.g * kGroup + hh;
    if (nb == 1) {
      bf16x4 v4;
      v4[0] = (bf16_t)acc[0]; v4[1] = (bf16_t)acc[1]; v4[2] = (bf16_t)acc[2]; v4[3] = (bf16_t)acc[3];
      *reinterpret_cast<bf16x4*>(out + ((int64_t)u.b * hq + head) * kHeadDim + d4) = v4;
      if (lse != nullptr && (tid & 31) == 0) lse[(int64_t)u.b * hq + head] = lse_v;
    } else {
      const int64_t row = (int64_t)u.c * hq + head;
      *reinterpret_cast<f32x4*>(ws_o + row * kHeadDim + d4) = acc;
      if ((tid & 31) == 0) ws_lse[row] = lse_v;
    }
    // Q of the next unit: wave 0 waited for its copy before the first barrier. Every wave has
    // it in registers before the second barrier, so wave 0 may reuse its buffer after that.
    if (r + 1 < my_units) load_q(r + 1);
    wait_lds();
    wg_barrier();  // the combine area is free again
  };

  // One tile of this wave's stream from stage `st`.
  auto compute = [&](const char* st, const Meta& m) __attribute__((always_inline)) {
    const lds_char_t* kb = (const lds_char_t*)st + wave * L::kStageBytes;
    const lds_char_t* vb = kb + C::kKBytes;
    constexpr int kMt = C::kTile / 16;  // 16-key M tiles: 2 (bf16) or 4 (fp8)
    // S^T: lane holds keys 16*mt + 4*grp + i (i = 0..3) of head `col`.
    f32x4 s[kMt];
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt) {
      s[mt] = f32x4{};
      const int r = 16 * mt + col;
#pragma unroll
      for (int stp = 0; stp < 4; ++stp) {
        bf16x8 a;
        if constexpr (kFp8 == 0) {
          const int c = 4 * stp + grp;  // d = 32*stp + 8*grp
          a = lds_read16(kb + r * 256 + ((c ^ (r & 15)) << 4));
        } else {
          const int byte = 32 * stp + 8 * grp;
          const int c = byte >> 4;
          const __attribute__((address_space(3))) uint32_t* p =
              (const __attribute__((address_space(3))) uint32_t*)(kb + r * 128 + ((c ^ (r & 7)) << 4) + (byte & 15));
          a = fp8x8_to_bf16x8(p[0], p[1]);
        }
        s[mt] = mfma16x16x32(a, qf[stp], s[mt]);
      }
    }
    if constexpr (kFp8 == 1) {
#pragma unroll
      for (int mt = 0; mt < kMt; ++mt) {
        const __attribute__((address_space(3))) f32x4* sp =
            (const __attribute__((address_space(3))) f32x4*)(vb + C::kKBytes + (16 * mt + 4 * grp) * 4);
        f32x4 sc = *sp;
        s[mt] *= sc;
      }
    }
    // mask keys past the unit's end
    if (m.k0 + C::kTile > m.kstop) {
#pragma unroll
      for (int mt = 0; mt < kMt; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (m.k0 + 16 * mt + 4 * grp + i >= m.kstop) s[mt][i] = -INFINITY;
        }
      }
    }
    // online softmax over this lane's head column
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[mt][i]);
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * scale_log2);
    const float neg = -m_use * scale_log2;
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[mt][i] = fast_exp2(__builtin_fmaf(s[mt][i], scale_log2, neg));
        psum += s[mt][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    if constexpr (kFp8 == 1) {
#pragma unroll
      for (int mt = 0; mt < kMt; ++mt) {
        const __attribute__((address_space(3))) f32x4* sp =
            (const __attribute__((address_space(3))) f32x4*)(vb + C::kKBytes + C::kScaleBytes + (16 * mt + 4 * grp) * 4);
        f32x4 sc = *sp;
        s[mt] *= sc;
      }
    }
    // O^T += V^T P^T, one MFMA k-step per 32 keys (M tiles 2kk and 2kk+1).
#pragma unroll
    for (int kk = 0; kk < kMt / 2; ++kk) {
      bf16x8 vt[8];
      if constexpr (kFp8 == 0) v_transposed(vb, kk, vt);
      bf16x8 pb = to_bf16x8(s[2 * kk][0], s[2 * kk][1], s[2 * kk][2], s[2 * kk][3], s[2 * kk + 1][0],
                            s[2 * kk + 1][1], s[2 * kk + 1][2], s[2 * kk + 1][3]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        bf16x8 a;
        if constexpr (kFp8 == 0) {
          a = vt[dt];
        } else {
          // lane needs V[key][d] for d = 16*dt + col and keys 32kk + 4grp + (0..3), +16
          const int d = 16 * dt + col;
          const int c = d >> 4;
          uint32_t w[2];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            uint32_t acc = 0;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int r = 32 * kk + 16 * half + 4 * grp + jj;
              const uint8_t byte = *((const __attribute__((address_space(3))) uint8_t*)(vb + r * 128 + ((c ^ (r & 7)) << 4) + (d & 15)));
              acc |= (uint32_t)byte << (8 * jj);
            }
            w[half] = acc;
          }
          a = fp8x8_to_bf16x8(w[0], w[1]);
        }
        o[dt] = mfma16x16x32(a, pb, o[dt]);
      }
    }
  };

  // ---- prologue: first two tiles of this wave, then Q of the first unit
  Meta m0{}, m1{};
  bool v0 = false, v1 = false;
  if (iu.valid) {
    m0 = issue(st0);
    v0 = true;
  }
  if (iu.valid) {
    m1 = issue(st1);
    v1 = true;
  }
  if (wave == 0) {
    // Q of unit 0 was copied before both tiles: wait for it alone
    if (v1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C::kCopies));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::kCopies));
  }
  wg_barrier();
  reset();
  load_q(0);
  int cr = 0;  // unit the compute side is in

  auto step = [&](char* st, Meta& m, bool& v, bool next_valid) __attribute__((always_inline)) {
    if (next_valid) __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::kCopies));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    while (cr < m.r) {
      flush(cr);
      ++cr;
      reset();
    }
    compute(st, m);
    if (iu.valid) {
      m = issue(st);
      v = true;
    } else {
      v = false;
    }
  };
  while (v0) {
    step(st0, m0, v0, v1);
    if (!v1) break;
    step(st1, m1, v1, v0);
  }
  while (cr < my_units) {
    flush(cr);
    ++cr;
    reset();
  }
}

// One workgroup per (request, kv head): 256 threads = 8 heads x 32 threads x 4 d. Requests
// listed as one chunk were written by the split pass; requests without keys get O = 0 and
// LSE = -inf.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ws_o,
                                                    const float* __restrict__ ws_lse,
                                                    const int32_t* __restrict__ hdr,
                                                    const int32_t* __restrict__ chunk_base, int hkv,
                                                    bf16_t* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int b = blockIdx.x / hkv;
  const int g = blockIdx.x % hkv;
  const int hq = hkv * kGroup;
  const int tid = threadIdx.x;
  const int head = g * kGroup + (tid >> 5);
  const int d4 = (tid & 31) * 4;
  const int n_chunks = hdr[1];
  const int c0 = chunk_base[b];
  const int c1 = min(chunk_base[b + 1], n_chunks);
  if (c1 - c0 == 1) return;
  const int64_t row = (int64_t)b * hq + head;
  float M = -INFINITY;
  for (int c = c0; c < c1; ++c) M = fmaxf(M, ws_lse[(int64_t)c * hq + head]);
  f32x4 acc = f32x4{};
  float Lsum = 0.f;
  if (M != -INFINITY) {
    for (int c = c0; c < c1; ++c) {
      const float w = __expf(ws_lse[(int64_t)c * hq + head] - M);
      Lsum += w;
      f32x4 v = *(const f32x4*)(ws_o + ((int64_t)c * hq + head) * kHeadDim + d4);
      acc += w * v;
    }
  }
  const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
  acc *= inv;
  bf16x4 v4;
  v4[0] = (bf16_t)acc[0]; v4[1] = (bf16_t)acc[1]; v4[2] = (bf16_t)acc[2]; v4[3] = (bf16_t)acc[3];
  *reinterpret_cast<bf16x4*>(out + row * kHeadDim + d4) = v4;
  if (lse != nullptr && (tid & 31) == 0) lse[row] = Lsum > 0.f ? M + __logf(Lsum) : -INFINITY;
}

}  // namespace

// Units per workgroup the automatic chunk length aims at.
constexpr int kUnitsPerWorkgroup = 12;

hipError_t launch_decode(const void* q, const void* k_pool, const void* v_pool,
                         const float* k_scale, const float* v_scale, int fp8, const void* segs,
                         const int32_t* seg_indptr, const int32_t* cu_k, int batch, int hkv,
                         int forced_len, int min_len, int max_chunks, int cu_count, float scale,
                         void* out, float* lse, int32_t* hdr, int32_t* chunk_base, int32_t* tab,
                         float* ws_o, float* ws_lse, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const int64_t max_units = (int64_t)max_chunks * hkv;
  const int grid = (int)std::min<int64_t>(cu_count, max_units);
  const int target = std::max(1, kUnitsPerWorkgroup * std::max(grid, 1));
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, cu_k, batch, hkv, forced_len,
                     min_len, target, max_chunks, hdr, chunk_base, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (grid > 0) {
    const float scale_log2 = scale * 1.4426950408889634f;
    const int xcd_spread = (hkv == kGroup && grid % 64 == 0) ? 1 : 0;
    if (fp8) {
      hipLaunchKernelGGL(decode_split_kernel<1>, dim3(grid), dim3(kDecThreads), 0, stream,
                         (const bf16_t*)q, k_pool, v_pool, k_scale, v_scale, (const Segment*)segs,
                         seg_indptr, cu_k, hdr, chunk_base, tab, hkv, xcd_spread, scale, scale_log2,
                         ws_o, ws_lse, (bf16_t*)out, lse);
    } else {
      hipLaunchKernelGGL(decode_split_kernel<0>, dim3(grid), dim3(kDecThreads), 0, stream,
                         (const bf16_t*)q, k_pool, v_pool, k_scale, v_scale, (const Segment*)segs,
                         seg_indptr, cu_k, hdr, chunk_base, tab, hkv, xcd_spread, scale, scale_log2,
                         ws_o, ws_lse, (bf16_t*)out, lse);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(batch * hkv)), dim3(256), 0, stream, ws_o, ws_lse,
                     hdr, chunk_base, hkv, (bf16_t*)out, lse);
  return hipGetLastError();
}

}  // namespace segattn
