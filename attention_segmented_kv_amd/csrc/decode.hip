// Decode kernels: one query token per request against all of its segmented keys.
//
// Work units. Each request's keys are cut into chunks of `len` keys (the last one shorter); a
// unit is one (chunk, kv head) pair, whose result is the blockwise partial attention of the
// FlashAccel article ("data layout": attention computed per block of the KV, then reduced per
// request). The chunks of all requests are listed on the device, so no launch slot is spent on
// requests shorter than the longest, with `len` chosen from the total key count so that every
// compute unit gets about 6 units: by each split workgroup itself for up to 256 requests with
// the automatic length, else by a one-workgroup plan kernel launched first.
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
// exactly on the way into the MFMAs (every E4M3FN value is a bf16 value); INT8 pools
// (two's-complement codes, same scales; the INT8 KV cache of "FlashAttention on Ascend NPU",
// optimisation 3) to f16, also exactly, with f16 MFMAs and Q widened to f16 (a conversion of four
// codes costs five instructions, against ten for bf16). The key scale multiplies the scores, the
// value scale the probabilities before their rounding to the operand type, so the arithmetic is
// attention over the dequantised pool with the probabilities rounded to bf16 (f16 for INT8).
//
// Merge pass: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s per (request, head).
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "common.hpp"

namespace segattn {

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kDecThreads = kWaves * 64;
constexpr int kQBufs = 3;           // Q tiles of the units a wave may be working ahead into
constexpr int kQBytes = kGroup * kHeadDim * 2;  // 2 KiB: the 8 query rows of one unit

// kKv: 0 = bf16 pool, 1 = FP8 (E4M3FN) pool, 2 = INT8 pool; 1 and 2 share the 1-byte layout.
template <int kKv>
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
struct DecodeCfg<1> {  // fp8 / int8: 64 keys per wave tile, 128 B rows, + k/v scales
  static constexpr int kTile = 64;
  static constexpr int kRowBytes = 128;
  static constexpr int kChunks = 8;
  static constexpr int kRowsPerCopy = 8;
  static constexpr int kKBytes = kTile * kRowBytes;  // 8 KiB
  static constexpr int kScaleBytes = kTile * 4;      // 256 B each
  static constexpr int kCopies = 2 * (kTile / kRowsPerCopy) + 2;
};
template <>
struct DecodeCfg<2> : DecodeCfg<1> {};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// MFMA operand type of a pool format: bf16 for bf16 and FP8 pools (every E4M3FN value is a bf16
// value), f16 for INT8 pools (every integer of magnitude <= 1024 is an f16 value, and the
// conversion below is two instructions per 4 codes' worth of halves).
template <int kKv>
using OpT = typename std::conditional<kKv == 2, f16x8, bf16x8>::type;

__device__ __forceinline__ f32x4 mfma_op(bf16x8 a, bf16x8 b, f32x4 c) { return mfma16x16x32(a, b, c); }
__device__ __forceinline__ f32x4 mfma_op(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 4 two's-complement codes (one dword) as 4 exact f16 values: u = c + 128 is the code with its
// top bit flipped; the half with bits 0x64 | u, that is 1024 + u, minus 1152 is c exactly.
__device__ __forceinline__ void int8x4_to_f16(uint32_t w, f16x2& a, f16x2& b) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // bytes u0, 64, u1, 64
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // bytes u2, 64, u3, 64
  const f16x2 off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  a = __builtin_bit_cast(f16x2, lo) + off;
  b = __builtin_bit_cast(f16x2, hi) + off;
}

// The same 4 codes as the 4 halves c + 1152 (the conversion above without its subtraction), for
// K: the scores built from them are corrected by 1152 * sum_d q_d of their head afterwards, once
// per score instead of once per code.
__device__ __forceinline__ void int8x4_to_f16_biased(uint32_t w, f16x2& a, f16x2& b) {
  const uint32_t u = w ^ 0x80808080u;
  a = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
  b = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
}
constexpr float kInt8Bias = 1152.0f;

// 8 one-byte codes (bytes 0..3 of lo, then of hi) as 8 exact MFMA operand values.
template <int kKv>
__device__ __forceinline__ OpT<kKv> codes8_to_op(uint32_t lo, uint32_t hi) {
  if constexpr (kKv == 1) {
    return fp8x8_to_bf16x8(lo, hi);
  } else {
    f16x2 r[4];
    int8x4_to_f16(lo, r[0], r[1]);
    int8x4_to_f16(hi, r[2], r[3]);
    return __builtin_bit_cast(f16x8, r);
  }
}

// 8 one-byte K codes as MFMA operands: exact for FP8, plus kInt8Bias for INT8.
template <int kKv>
__device__ __forceinline__ OpT<kKv> kcodes8_to_op(uint32_t lo, uint32_t hi) {
  if constexpr (kKv == 1) {
    return fp8x8_to_bf16x8(lo, hi);
  } else {
    f16x2 r[4];
    int8x4_to_f16_biased(lo, r[0], r[1]);
    int8x4_to_f16_biased(hi, r[2], r[3]);
    return __builtin_bit_cast(f16x8, r);
  }
}

// Eight fp32 values as MFMA operands: bf16 (round to nearest even), or f16 (round to nearest
// even) for the INT8 path.
template <int kKv>
__device__ __forceinline__ OpT<kKv> to_op8(float a0, float a1, float a2, float a3, float a4, float a5,
                                           float a6, float a7) {
  if constexpr (kKv == 2) {
    f16x8 r;
    r[0] = (_Float16)a0; r[1] = (_Float16)a1; r[2] = (_Float16)a2; r[3] = (_Float16)a3;
    r[4] = (_Float16)a4; r[5] = (_Float16)a5; r[6] = (_Float16)a6; r[7] = (_Float16)a7;
    return r;
  } else {
    return to_bf16x8(a0, a1, a2, a3, a4, a5, a6, a7);
  }
}

// Q (bf16 in LDS) as an operand: unchanged, or widened to f16 for the INT8 path (exact for every
// bf16 value of f16's normal range; smaller ones round to f16 subnormals, below 2^-24 absolute).
template <int kKv>
__device__ __forceinline__ OpT<kKv> q_to_op(bf16x8 q) {
  if constexpr (kKv == 2) {
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (_Float16)(float)q[i];
    return r;
  } else {
    return q;
  }
}
template <int kKv>
struct DecodeLayout {
  using C = DecodeCfg<kKv>;
  // one wave's stage: K tile, V tile, k scales, v scales
  static constexpr int kStageBytes = 2 * C::kKBytes + 2 * C::kScaleBytes;
  static constexpr int kCombFloats = kGroup * kHeadDim + 4 * kGroup;  // O^T, (m, l) of one wave
};

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

// A operands of O^T += V^T P^T for the 32 keys 32*kk .. 32*kk + 31 of a 1-byte V tile in LDS
// (128 B rows, 16-byte chunk c of row r at c ^ (r % 8)), still as codes: lane
// (grp, col) gets the 8 codes V[key(j)][16*dt + col], key(j) as for the bf16 tile. The
// transposing 8-bit read hands lane i of a 16-lane group byte i % 8 of the 8 bytes addressed by
// lane 2*j + i / 8, so source lane s of group grp addresses row key(s / 2) at columns
// 16*dt + 8*(s % 2) .. +7. Issued and waited for in one asm block, as in v_transposed.
__device__ __forceinline__ void v_transposed8(const lds_char_t* vb, int kk, uint32_t (&lo)[8], uint32_t (&hi)[8]) {
  const int lane = threadIdx.x & 63;
  const int s = lane & 15, grp = lane >> 4;
  const int j = s >> 1;
  const int key = 32 * kk + 4 * grp + (j < 4 ? j : 12 + j);
  const int half = 8 * (s & 1);
  uint32_t pa[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) pa[dt] = (uint32_t)(uintptr_t)(vb + key * 128 + ((dt ^ (key & 7)) << 4) + half);
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 r[8];
  asm volatile(
      "ds_read_b64_tr_b8 %0, %8\n\t"
      "ds_read_b64_tr_b8 %1, %9\n\t"
      "ds_read_b64_tr_b8 %2, %10\n\t"
      "ds_read_b64_tr_b8 %3, %11\n\t"
      "ds_read_b64_tr_b8 %4, %12\n\t"
      "ds_read_b64_tr_b8 %5, %13\n\t"
      "ds_read_b64_tr_b8 %6, %14\n\t"
      "ds_read_b64_tr_b8 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7])
      : "v"(pa[0]), "v"(pa[1]), "v"(pa[2]), "v"(pa[3]), "v"(pa[4]), "v"(pa[5]), "v"(pa[6]), "v"(pa[7])
      : "memory");
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    lo[dt] = r[dt][0];
    hi[dt] = r[dt][1];
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
  // Positioned on segment i (whose first key is logical key st) from a chunk record.
  __device__ __forceinline__ void init_at(const Segment* s, int i, int last, int st, int o, int l) {
    segs = s;
    idx = i;
    end = last;
    start = st;
    off = o;
    len = l;
  }
  __device__ __forceinline__ void advance_to(int j) {
    while (j - start >= len) {
      start += len;
      ++idx;
      fetch();
    }
  }
};

// Where a unit's keys are: chunk c of request b holds keys [kbeg, kstop); the segment holding
// key kbeg is sidx (its first key is logical key sstart, pool slots [soff, soff + slen)).
struct UnitInfo {
  int valid, c, g, b, kbeg, kstop, single, sidx, send, sstart, soff, slen, n_tiles;
};

// One record per chunk, 16 int32 (64 B, one scalar load), stored in schedule order:
//   0 request b, 1 first key, 2 end key, 3 1 if the chunk is the request's only one,
//   4 index of the segment holding the first key (segment end index if none), 5 segment end
//   index of the request, 6 logical first key of that segment, 7 its pool offset, 8 its
//   length, 9 chunk index (the row of its partial result).
constexpr int kRecInts = 16;
constexpr int kBuckets = 256;

// Plan: chunk length, per-request chunk offsets and the chunk records in schedule order. The
// schedule lists every full-length chunk first, then the shorter last chunks of the requests by
// decreasing length (a counting sort over 256 length buckets); the split pass deals this list
// to its columns in snake order, which spreads the short chunks evenly. One thread per request;
// the table reads are issued together (key counts, segment ranges, then the first segments) so
// the plan costs few memory latencies.
// hdr[0] = len, hdr[1] = number of chunks listed (0 if they would not fit in max_chunks).
constexpr int kPlanSegs = 8;  // segments per request read up front
constexpr int kSpreadMax = 512;  // plan: batches up to this size share each request's chunks

// Inclusive scan over the kW waves of the block of two counts at once: shuffles within each
// wave, then one pass over the wave totals. wtot is LDS scratch of 2 x 16 ints.
template <int kW>
__device__ __forceinline__ void block_scan2(int& a, int& b, int* wtot) {
  static_assert(kW >= 1 && kW <= 16, "at most 16 waves");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int ta = __shfl_up(a, d), tb = __shfl_up(b, d);
    if (lane >= d) {
      a += ta;
      b += tb;
    }
  }
  if (lane == 63) {
    wtot[w] = a;
    wtot[16 + w] = b;
  }
  __syncthreads();
  if (w == 0) {
    int x = lane < kW ? wtot[lane] : 0, y = lane < kW ? wtot[16 + lane] : 0;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int tx = __shfl_up(x, d), ty = __shfl_up(y, d);
      if (lane >= d) {
        x += tx;
        y += ty;
      }
    }
    if (lane < kW) {
      wtot[lane] = x;
      wtot[16 + lane] = y;
    }
  }
  __syncthreads();
  if (w > 0) {
    a += wtot[w - 1];
    b += wtot[16 + w - 1];
  }
}

// Plan: chunk length, per-request chunk offsets and the chunk records in schedule order. The
// schedule lists every full-length chunk first, then the shorter last chunks of the requests by
// decreasing length (a counting sort over 256 length buckets); the split pass deals this list
// to its columns in snake order, which spreads the short chunks evenly. One thread per request;
// the table reads are issued together (key counts, segment ranges, then the first segments) so
// the plan costs few memory latencies.
// hdr[0] = len, hdr[1] = number of chunks listed, hdr[2] = 1 when some K_b exceeds max_k (the
// host's bound, which sized the workspace): then no chunk is listed and the merge pass writes
// NaN to every output and LSE, so that the broken bound cannot pass unnoticed.
__global__ __launch_bounds__(1024) void decode_plan_kernel(
    const int32_t* __restrict__ cu_k, const int32_t* __restrict__ seg_indptr,
    const Segment* __restrict__ segs, int batch, int hkv, int forced_len, int min_len,
    int target_units, int max_chunks, int max_k, int32_t* __restrict__ hdr,
    int32_t* __restrict__ chunk_base, int32_t* __restrict__ recs) {
  __shared__ int wtot[32];
  __shared__ int hist[kBuckets], bucket_base[kBuckets], bucket_fill[kBuckets];
  __shared__ int carry_n, carry_f, too_long;
  // batches of at most kSpreadMax requests: each request's scan results and first segments,
  // for the threads that share its chunks in pass 2
  __shared__ int rq_first[kSpreadMax], rq_ffirst[kSpreadMax], rq_n[kSpreadMax], rq_f[kSpreadMax];
  __shared__ int rq_K[kSpreadMax], rq_sa[kSpreadMax], rq_se[kSpreadMax];
  __shared__ Segment rq_sg[kSpreadMax * kPlanSegs];
  const int tid = threadIdx.x;
  // This thread's request in the first block, read once and kept for both passes. Every load
  // is unconditional, at an index clamped into its table, so that they are all in flight at
  // once (batch >= 1 here).
  const int bq = min(tid, batch - 1);
  const int64_t total = (int64_t)cu_k[batch] - cu_k[0];
  const int nseg = seg_indptr[batch];
  const int ka = cu_k[bq], kb = cu_k[bq + 1];
  const int s0 = tid < batch ? seg_indptr[bq] : 0;
  const int s1 = tid < batch ? seg_indptr[bq + 1] : 0;
  const int K0 = tid < batch ? kb - ka : 0;
  Segment sg0[kPlanSegs];
  if (nseg > 0) {
#pragma unroll
    for (int j = 0; j < kPlanSegs; ++j) sg0[j] = segs[min(s0 + j, nseg - 1)];
  }
#pragma unroll
  for (int j = 0; j < kPlanSegs; ++j)
    if (nseg == 0 || s0 + j >= s1) sg0[j] = Segment{0, 0x7fffffff};
  int len = forced_len;
  if (len <= 0) {
    int64_t want = (total * hkv + target_units - 1) / target_units;
    want = (want + 63) / 64 * 64;
    len = (int)(want < min_len ? min_len : (want > (1 << 30) ? (1 << 30) : want));
  }
  auto counts = [&](int K, int& n, int& f) {
    n = K > 0 ? (K + len - 1) / len : 0;
    f = K > 0 ? K / len : 0;
  };
  if (tid < kBuckets) {
    hist[tid] = 0;
    bucket_fill[tid] = 0;
  }
  if (tid == 0) {
    carry_n = 0;
    carry_f = 0;
    too_long = 0;
  }
  __syncthreads();
  // pass 1: totals and the histogram of the short last chunks
  int n0, f0, sn0 = 0, sf0 = 0;  // counts and inclusive scans of the first block, for pass 2
  counts(K0, n0, f0);
  for (int b0 = 0; b0 < batch; b0 += 1024) {
    const int b = b0 + tid;
    const int K = b0 == 0 ? K0 : (b < batch ? cu_k[b + 1] - cu_k[b] : 0);
    if (K > max_k) too_long = 1;  // any writer stores the same value
    int n, f;
    counts(K, n, f);
    if (n > f) atomicAdd(&hist[(int)((int64_t)(K - f * len) * kBuckets / len)], 1);
    int sn = n, sf = f;
    block_scan2<16>(sn, sf, wtot);
    if (b0 == 0) {
      sn0 = sn;
      sf0 = sf;
    }
    if (tid == 1023) {
      carry_n += sn;
      carry_f += sf;
    }
    __syncthreads();
  }
  const int total_n = carry_n, total_f = carry_f;
  // bucket positions, longest short chunks first: a scan over the buckets in reverse order
  {
    int hcount = tid < kBuckets ? hist[kBuckets - 1 - tid] : 0, dummy = 0;
    block_scan2<16>(hcount, dummy, wtot);
    if (tid < kBuckets) bucket_base[kBuckets - 1 - tid] = total_f + hcount - hist[kBuckets - 1 - tid];
  }
  __syncthreads();
  // pass 2: chunk offsets and records. The record of chunk k of request b: its schedule
  // position (full chunks in request order, then the short last ones by decreasing length) and
  // the segment cursor at its first key, found by walking the request's segments in key order.
  auto write_rec = [&](int b, int k, int K, int n, int f, int first, int ffirst, int idx, int se,
                       int start, const Segment& sg) __attribute__((always_inline)) {
    const int kbeg = k * len;
    int pos = ffirst + k;
    if (k >= f) {
      const int bk = (int)((int64_t)(K - f * len) * kBuckets / len);
      pos = bucket_base[bk] + atomicAdd(&bucket_fill[bk], 1);
    }
    if (pos < max_chunks && first + k < max_chunks) {
      i32x4* r = reinterpret_cast<i32x4*>(recs + (int64_t)pos * kRecInts);
      r[0] = i32x4{b, kbeg, min(K, kbeg + len), n == 1 ? 1 : 0};
      r[1] = i32x4{idx, se, start, sg.pool_offset};
      r[2] = i32x4{sg.length, first + k, 0, 0};
    }
  };
  if (batch <= kSpreadMax) {
    // One block of requests (pass 1 ran once): tpr threads per request take its chunks
    // k = kq, kq + tpr, ..., so that long requests (hundreds of chunks) are not written by one
    // thread in sequence.
    int tpr = 1;
    while (tpr < 64 && batch * tpr * 2 <= 1024) tpr *= 2;
    if (tid < batch) {
      rq_first[tid] = sn0 - n0;
      rq_ffirst[tid] = sf0 - f0;
      rq_n[tid] = n0;
      rq_f[tid] = f0;
      rq_K[tid] = K0;
      rq_sa[tid] = s0;
      rq_se[tid] = s1;
#pragma unroll
      for (int j = 0; j < kPlanSegs; ++j) rq_sg[tid * kPlanSegs + j] = sg0[j];
    }
    __syncthreads();
    const int b = tid / tpr, kq = tid - b * tpr;
    if (b < batch) {
      const int K = rq_K[b], n = rq_n[b], f = rq_f[b], first = rq_first[b], ffirst = rq_ffirst[b];
      const int sa = rq_sa[b], se = rq_se[b];
      if (kq == 0) chunk_base[b] = first;
      int idx = sa, start = 0;
      Segment sg = rq_sg[b * kPlanSegs];
      for (int k = kq; k < n; k += tpr) {
        const int kbeg = k * len;
        while (idx < se && kbeg - start >= sg.length) {
          start += sg.length;
          ++idx;
          const int j = idx - sa;
          sg = j < kPlanSegs ? rq_sg[b * kPlanSegs + j] : (idx < se ? segs[idx] : Segment{0, 0x7fffffff});
        }
        write_rec(b, k, K, n, f, first, ffirst, idx, se, start, sg);
      }
    }
  } else {
  int cn = 0, cf = 0;  // chunks and full chunks of the blocks before
  for (int b0 = 0; b0 < batch; b0 += 1024) {
    const int b = b0 + tid;
    int K = 0, sa = 0, se = 0, n, f, sn, sf;
    if (b0 == 0) {
      K = K0;
      sa = s0;
      se = s1;
      n = n0;
      f = f0;
      sn = sn0;
      sf = sf0;
    } else {
      if (b < batch) {
        K = cu_k[b + 1] - cu_k[b];
        sa = seg_indptr[b];
        se = seg_indptr[b + 1];
      }
      counts(K, n, f);
      sn = n;
      sf = f;
      block_scan2<16>(sn, sf, wtot);
    }
    const int first = cn + sn - n;   // first chunk index of request b
    const int ffirst = cf + sf - f;  // schedule position of its first full chunk
    if (b < batch) {
      chunk_base[b] = first;
      // walk the request's segments once, in key order, recording where each chunk starts
      int idx = sa, start = 0;
      Segment sg = (b0 == 0) ? sg0[0] : (sa < se ? segs[sa] : Segment{0, 0x7fffffff});
      for (int k = 0; k < n; ++k) {
        const int kbeg = k * len;
        while (idx < se && kbeg - start >= sg.length) {
          start += sg.length;
          ++idx;
          const int j = idx - sa;
          if (b0 == 0 && j < kPlanSegs) {
            Segment t = sg0[0];
#pragma unroll
            for (int q = 1; q < kPlanSegs; ++q) t = (j == q) ? sg0[q] : t;
            sg = t;
          } else {
            sg = idx < se ? segs[idx] : Segment{0, 0x7fffffff};
          }
        }
        write_rec(b, k, K, n, f, first, ffirst, idx, se, start, sg);
      }
    }
    // totals of this block for the next one (the last thread holds the block's inclusive sums)
    if (b0 + 1024 < batch) {
      __syncthreads();
      if (tid == 1023) {
        carry_n = cn + sn;
        carry_f = cf + sf;
      }
      __syncthreads();
      cn = carry_n;
      cf = carry_f;
    }
  }
  }
  if (tid == 0) {
    chunk_base[batch] = total_n;
    hdr[0] = len;
    // a key count above the host's bound (which the workspace was sized for): list nothing and
    // let the merge pass mark every output (the scan above ended in a barrier, so too_long is
    // final)
    const int bad = too_long != 0 || total_n > max_chunks;
    hdr[1] = bad ? 0 : total_n;
    hdr[2] = bad ? 1 : 0;
  }
}

// ------------------------------------------------------------------------------------------
// The plan inside the split pass, for batches of at most kInPlanBatch requests with the automatic
// chunk length: every workgroup derives the chunk list from the key counts itself, so the call
// needs no separate plan launch (whose few microseconds, plus the gap before the next launch, are
// a visible share of a short decode). The chunking (length, per-request chunk indices, hence
// every partial and the merge order) is the plan kernel's; the schedule differs only in how the
// short last chunks are ordered: by exact decreasing length, equal lengths by request, a total
// order that every workgroup computes alike.
constexpr int kInPlanBatch = kDecThreads;  // one request per thread
constexpr int kUnitCap = 24;               // unit records per workgroup
// Units per workgroup the automatic chunk length aims at. Measured over 4, 6, 8, 12 and 16 on
// the bf16 batch-128 and the FP8 / INT8 batch-16 long-context decodes: 6 was the fastest or
// within 1% of it on each; 4 leaves the longest requests' chunks too long to balance, 12 and
// more pay for the extra partial results and merge work.
constexpr int kUnitsPerWorkgroup = 6;

// Units of schedule column p out of n_chunks over P columns (positions r * P + p for even r and
// r * P + P - 1 - p for odd r).
__device__ __forceinline__ int column_units(int n_chunks, int P, int p) {
  const int full_rounds = n_chunks / P;
  const int last_pos = (full_rounds & 1) ? P - 1 - p : p;
  return full_rounds + (last_pos < n_chunks - full_rounds * P ? 1 : 0);
}

constexpr int kInPlanScrInts = 6 * 257 + 32;

// All threads of the workgroup call this. scr: LDS for kInPlanScrInts ints that no copy writes
// until it returns; utab: kUnitCap records of 3 x i32x4, laid out as the plan kernel's records.
// Returns the chunk count, or -1 when some K_b exceeds max_k, the chunks would not fit in the
// workspace (max_chunks) or a column would hold more than kUnitCap units; workgroup 0 then
// writes hdr so that the merge pass marks every output NaN. Workgroup 0 also writes hdr and
// chunk_base for the merge pass in the good case.
__device__ int plan_in_workgroup(const int32_t* __restrict__ cu_k, const int32_t* __restrict__ seg_indptr,
                                 const Segment* __restrict__ segs, int batch, int hkv, int min_len,
                                 int target_units, int max_chunks, int max_k, int P, int p, int* scr,
                                 i32x4* utab, int32_t* __restrict__ hdr, int32_t* __restrict__ chunk_base) {
  int* sK = scr;             // [256] key count of each request
  int* sF = sK + 256;        // [257] schedule position of each request's first full chunk
  int* sN = sF + 257;        // [257] index of each request's first chunk
  int* sA = sN + 257;        // [257] segment index range starts (seg_indptr)
  int* sS = sA + 257;        // [256] length of the request's short last chunk, -1 if none
  int* sO = sS + 256;        // [256] requests with a short chunk, longest chunk first
  int* sW = sO + 256;        // [32] scan scratch
  const int t = threadIdx.x;
  const int64_t total = (int64_t)cu_k[batch] - cu_k[0];
  int K = 0, sa = 0, sa_end = 0;
  if (t < batch) {
    K = cu_k[t + 1] - cu_k[t];
    sa = seg_indptr[t];
    if (t == batch - 1) sa_end = seg_indptr[batch];
  }
  int64_t want = (total * hkv + target_units - 1) / target_units;
  want = (want + 63) / 64 * 64;
  const int len = (int)(want < min_len ? min_len : (want > (1 << 30) ? (1 << 30) : want));
  const int n = K > 0 ? (K + len - 1) / len : 0;
  const int f = K > 0 ? K / len : 0;
  int sn = n, sf = f;
  block_scan2<kDecThreads / 64>(sn, sf, sW);
  if (t < batch) {
    sK[t] = K;
    sF[t] = sf - f;
    sN[t] = sn - n;
    sA[t] = sa;
    sS[t] = n > f ? K - f * len : -1;
  }
  if (t == batch - 1) {
    sF[batch] = sf;
    sN[batch] = sn;
    sA[batch] = sa_end;
  }
  const int any_long = __syncthreads_or(t < batch && K > max_k);
  const int total_f = sF[batch], total_n = sN[batch];
  const bool bad = any_long != 0 || total_n > max_chunks || (total_n + P - 1) / P > kUnitCap;
  if (blockIdx.x == 0) {
    if (t == 0) {
      hdr[0] = len;
      hdr[1] = bad ? 0 : total_n;
      hdr[2] = bad ? 1 : 0;
      chunk_base[batch] = total_n;
    }
    if (t < batch) chunk_base[t] = sN[t];
  }
  if (bad) return -1;
  // rank of each short chunk: longer ones first, equal lengths in request order
  if (t < batch && n > f) {
    const int sl = K - f * len;
    int r = 0;
    for (int u = 0; u < batch; ++u) {
      const int su = sS[u];
      r += (su > sl || (su == sl && u < t)) ? 1 : 0;
    }
    sO[r] = t;
  }
  __syncthreads();
  // records of this column's units, one thread each
  const int my_units = column_units(total_n, P, p);
  if (t < my_units) {
    const int r = t;
    const int pos = r * P + ((r & 1) ? P - 1 - p : p);
    int b, k;
    if (pos < total_f) {
      // the last request whose first full chunk is at or before pos owns it
      int lo = 0, hi = batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sF[mid] <= pos) lo = mid;
        else hi = mid - 1;
      }
      b = lo;
      k = pos - sF[b];
    } else {
      b = sO[pos - total_f];
      k = sK[b] / len;
    }
    const int Kb = sK[b];
    const int kbeg = k * len;
    const int kstop = min(Kb, kbeg + len);
    const int single = (Kb + len - 1) / len == 1 ? 1 : 0;
    const int c = sN[b] + k;
    // the segment holding key kbeg: the request's segments in key order, 8 reads at a time
    const int s_first = sA[b], s_end = sA[b + 1];
    int idx = s_first, start = 0, sidx = s_end, soff = 0, slen = 0x7fffffff;
    bool found = false;
    while (!found && idx < s_end) {
      const int m = min(8, s_end - idx);
      Segment sg[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) sg[j] = segs[idx + min(j, m - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (!found && j < m) {
          if (kbeg - start < sg[j].length) {
            found = true;
            sidx = idx + j;
            soff = sg[j].pool_offset;
            slen = sg[j].length;
          } else {
            start += sg[j].length;
          }
        }
      }
      idx += m;
    }
    utab[3 * r + 0] = i32x4{b, kbeg, kstop, single};
    utab[3 * r + 1] = i32x4{sidx, s_end, start, soff};
    utab[3 * r + 2] = i32x4{slen, c, 0, 0};
  }
  __syncthreads();
  return total_n;
}

// ------------------------------------------------------------------------------------------
// Split pass.
// kInPlan: the workgroup plans for itself (plan_in_workgroup, from cu_k and seg_indptr, and
// writes hdr and chunk_base for the merge pass); otherwise hdr and recs come from the plan kernel.
struct InPlanArgs {
  const int32_t* cu_k;
  const int32_t* seg_indptr;
  int32_t* chunk_base;
  int batch, min_len, target_units, max_chunks, max_k;
};

template <int kKv, bool kInPlan>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const bf16_t* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const Segment* __restrict__ segs, int32_t* __restrict__ hdr,
    const int32_t* __restrict__ recs, InPlanArgs ipa, int hkv, float scale, float scale_log2,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, bf16_t* __restrict__ out,
    float* __restrict__ lse) {
  using C = DecodeCfg<kKv>;
  using L = DecodeLayout<kKv>;
  // Separate objects for the two stages, the combine area and the Q tiles: the compiler then
  // sees that reading one stage cannot touch the copies still landing in the other, and adds
  // no wait for them.
  __shared__ __attribute__((aligned(1024))) char st0[kWaves * L::kStageBytes];
  __shared__ __attribute__((aligned(1024))) char st1[kWaves * L::kStageBytes];
  __shared__ __attribute__((aligned(16))) float comb[kWaves * L::kCombFloats];
  __shared__ __attribute__((aligned(16))) char qbuf[kQBufs * kQBytes];
  __shared__ __attribute__((aligned(16))) i32x4 uring[4];
  __shared__ __attribute__((aligned(16))) i32x4 utab[kInPlan ? 3 * kUnitCap : 1];

  // Workgroup = (column p, lane g of the kv heads). Column p takes schedule positions r * P + p
  // for even r and r * P + P - 1 - p for odd r; in round r its workgroups take kv heads
  // (g + r) % hkv, so the 8 heads of each chunk are all done and every workgroup meets every
  // head: the reading speed of a head's slices of the pool rows varies, and this keeps the
  // workgroups even. Workgroups are numbered g * P + p: with P a multiple of 8, the workgroups
  // of one column, which read the same chunk's rows in every round, are dispatched to the same
  // XCD and share its L2 (a 128-byte line of the FP8 / INT8 scale arrays holds 4 tokens x 8
  // heads; spread over 8 XCDs it was fetched 8 times).
  const int P = gridDim.x / hkv;
  const int g = rfl(blockIdx.x / P);
  const int p = rfl(blockIdx.x - g * P);
  int n_chunks;
  if constexpr (kInPlan) {
    // the per-request values go to stage 1, which no copy fills before this returns
    static_assert(kInPlanScrInts * 4 <= (int)sizeof(st1), "plan scratch exceeds stage 1");
    n_chunks = plan_in_workgroup(ipa.cu_k, ipa.seg_indptr, segs, ipa.batch, hkv, ipa.min_len,
                                 ipa.target_units, ipa.max_chunks, ipa.max_k, P, p,
                                 reinterpret_cast<int*>(st1), utab, hdr, ipa.chunk_base);
    if (n_chunks < 0) return;
    n_chunks = rfl(n_chunks);
  } else {
    n_chunks = rfl(hdr[1]);
  }
  const int my_units = column_units(n_chunks, P, p);
  if (my_units == 0) return;

  const int tid = threadIdx.x;
  const int wave = rfl(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15;  // head column of the MFMA tile (>= 8 is padding)
  const int grp = lane >> 4;  // 0..3
  const int hq = hkv * kGroup;
  const int64_t tok_bytes = (int64_t)hkv * C::kRowBytes;
  // Byte offsets of this lane's copies within a tile whose rows are consecutive pool slots:
  // copy i covers rows kRowsPerCopy * i .. + kRowsPerCopy - 1, lane piece lane % kChunks of row
  // kRowsPerCopy * i + lane / kChunks (stored swizzled, so the piece read is chunk position ^ f(r))
  uint32_t koff[C::kTile / C::kRowsPerCopy], voff[C::kTile / C::kRowsPerCopy];
#pragma unroll
  for (int i = 0; i < C::kTile / C::kRowsPerCopy; ++i) {
    const int r = C::kRowsPerCopy * i + lane / C::kChunks;
    const int cpos = lane % C::kChunks;
    int kc, vc;
    if constexpr (kKv == 0) {
      kc = cpos ^ (r & 15);
      vc = cpos ^ vswz16(r);
    } else {
      kc = cpos ^ (r & 7);
      vc = kc;
    }
    koff[i] = (uint32_t)r * (uint32_t)tok_bytes + 16 * kc;
    voff[i] = (uint32_t)r * (uint32_t)tok_bytes + 16 * vc;
  }
  const uint32_t soff = (uint32_t)lane * (uint32_t)hkv * 4;  // scale of row `lane`

  // Every field is wave-uniform and kept in scalar registers (readfirstlane after the integer
  // division, which the compiler does on the vector ALU); the chunk record is one scalar load.
  auto unit_info = [&](int r) __attribute__((always_inline)) {
    UnitInfo u;
    u.valid = r < my_units;
    i32x4 r0, r1, r2;
    if constexpr (kInPlan) {
      // from the LDS table (through inline asm, so that the compiler adds no wait for the copies
      // in flight)
      const uint32_t a = (uint32_t)(uintptr_t)((lds_char_t*)utab + 48 * (u.valid ? r : 0));
      asm volatile(
          "ds_read_b128 %0, %3\n\t"
          "ds_read_b128 %1, %3 offset:16\n\t"
          "ds_read_b128 %2, %3 offset:32\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(r0), "=&v"(r1), "=&v"(r2)
          : "v"(a)
          : "memory");
    } else {
      const int pos = u.valid ? r * P + ((r & 1) ? P - 1 - p : p) : 0;
      const i32x4* rp = reinterpret_cast<const i32x4*>(recs + (int64_t)pos * kRecInts);
      r0 = rp[0];
      r1 = rp[1];
      r2 = rp[2];
    }
    u.g = (g + r) % hkv;
    u.b = rfl(r0[0]);
    u.kbeg = rfl(r0[1]);
    u.kstop = rfl(r0[2]);
    u.single = rfl(r0[3]);
    u.sidx = rfl(r1[0]);
    u.send = rfl(r1[1]);
    u.sstart = rfl(r1[2]);
    u.soff = rfl(r1[3]);
    u.slen = rfl(r2[0]);
    u.c = rfl(r2[1]);
    u.n_tiles = u.valid ? rfl((u.kstop - u.kbeg + C::kTile - 1) / C::kTile) : 0;
    return u;
  };
  // Unit identities for the combine, written by wave 0 when it enters a unit (it has a tile in
  // every unit) and read by all waves between the combine's barriers. Entry r % 4 is rewritten
  // only once wave 0 works on unit r + 2, after every wave has left the combine of unit r.
  auto ring_put = [&](const UnitInfo& u, int r) __attribute__((always_inline)) {
    if (wave == 0 && lane == 0) {
      i32x4 v = i32x4{u.c, u.g, u.b, u.single};
      const uint32_t a = (uint32_t)(uintptr_t)((lds_char_t*)uring + 16 * (r & 3));
      asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
    }
  };

  // ---- issue side: this wave's next tile
  UnitInfo iu = unit_info(0);
  int it = wave;  // tile index inside unit iu
  int ir = 0;     // ordinal of unit iu among this workgroup's units
  ScalarCursor cur;
  cur.init_at(segs, iu.sidx, iu.send, iu.sstart, iu.soff, iu.slen);
  ring_put(iu, 0);
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
      cur.init_at(segs, iu.sidx, iu.send, iu.sstart, iu.soff, iu.slen);
      ring_put(iu, ir);
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
    constexpr int kN = C::kTile / C::kRowsPerCopy;
    const char* kbase = (const char*)k_pool + (int64_t)iu.g * C::kRowBytes;
    const char* vbase = (const char*)v_pool + (int64_t)iu.g * C::kRowBytes;
    if (fast) {
      // rows k0 .. k0 + kTile - 1 are consecutive pool slots from base: one buffer per tensor
      // based at the tile's first row, and per-lane offsets fixed for the whole kernel
      const int64_t base = (int64_t)cur.off + (m.k0 - cur.start);
      const auto kr = block_rsrc(kbase + base * tok_bytes);
      const auto vr = block_rsrc(vbase + base * tok_bytes);
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        copy16_buf_stream(kr, (lds_void_t*)(kb + i * 1024), koff[i]);
        copy16_buf_stream(vr, (lds_void_t*)(vb + i * 1024), voff[i]);
      }
      if constexpr (kKv != 0) {
        // scales: lane L copies those of row L
        const int64_t s0 = base * hkv + iu.g;
        copy4_buf(block_rsrc(k_scale + s0), (lds_void_t*)(vb + C::kKBytes), soff);
        copy4_buf(block_rsrc(v_scale + s0), (lds_void_t*)(vb + C::kKBytes + C::kScaleBytes), soff);
      }
    } else {
      // Rows of the tile that straddle segments (or lie past the unit's end, which re-read
      // the unit's last key and are masked later): walk the overlapped segments with a
      // scalar copy of the cursor.
      const int rsub = lane / C::kChunks;
      const int cpos = lane % C::kChunks;
      int64_t slot_of[kN];
#pragma unroll
      for (int i = 0; i < kN; ++i) slot_of[i] = 0;
      {
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
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        const int r = C::kRowsPerCopy * i + rsub;
        int kc, vc;
        if constexpr (kKv == 0) {
          kc = cpos ^ (r & 15);
          vc = cpos ^ vswz16(r);
        } else {
          kc = cpos ^ (r & 7);
          vc = kc;
        }
        const int64_t row = slot_of[i] * tok_bytes;
        copy16_to_lds_stream(kbase + row + kc * 16, (lds_void_t*)(kb + i * 1024));
        copy16_to_lds_stream(vbase + row + vc * 16, (lds_void_t*)(vb + i * 1024));
      }
      if constexpr (kKv != 0) {
        // scales: lane L copies those of row L
        const int j = min(m.k0 + lane, last);
        int64_t s = 0;
        ScalarCursor c2 = cur;
        while (true) {
          if (j - c2.start >= 0 && j - c2.start < c2.len) s = (int64_t)c2.off + (j - c2.start);
          if (last - c2.start < c2.len) break;
          c2.start += c2.len;
          ++c2.idx;
          c2.fetch();
        }
        copy4_to_lds(k_scale + s * hkv + iu.g, (lds_void_t*)(vb + C::kKBytes));
        copy4_to_lds(v_scale + s * hkv + iu.g, (lds_void_t*)(vb + C::kKBytes + C::kScaleBytes));
      }
    }
    // advance to this wave's next tile
    it += kWaves;
    if (it >= iu.n_tiles) next_unit();
    return m;
  };

  // ---- compute side
  OpT<kKv> qf[4];  // B operand of S^T: lane holds d = 32*step + 8*grp + (0..7) of head `col`
  float kbias = 0.f;  // INT8: kInt8Bias * sum_d q_d of head `col` (the f16 q the MFMAs see)
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
    qf[0] = q_to_op<kKv>(real ? __builtin_bit_cast(bf16x8, v0) : bf16x8{});
    qf[1] = q_to_op<kKv>(real ? __builtin_bit_cast(bf16x8, v1) : bf16x8{});
    qf[2] = q_to_op<kKv>(real ? __builtin_bit_cast(bf16x8, v2) : bf16x8{});
    qf[3] = q_to_op<kKv>(real ? __builtin_bit_cast(bf16x8, v3) : bf16x8{});
    if constexpr (kKv == 2) {
      float qs = 0.f;
#pragma unroll
      for (int stp = 0; stp < 4; ++stp)
#pragma unroll
        for (int i = 0; i < 8; ++i) qs += (float)qf[stp][i];
      kbias = kInt8Bias * sum_xor32(sum_xor16(qs));
    }
  };

  // Combine the 4 waves' states for unit r and write the output or the partial.
  auto flush = [&](int r) __attribute__((always_inline)) {
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
    i32x4 id4;
    {
      const uint32_t a = (uint32_t)(uintptr_t)((lds_char_t*)uring + 16 * (r & 3));
      asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(id4) : "v"(a) : "memory");
    }
    const int uc = rfl(id4[0]), ug = rfl(id4[1]), ub = rfl(id4[2]), usingle = rfl(id4[3]);
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
    const int head = ug * kGroup + hh;
    if (usingle) {
      bf16x4 v4;
      v4[0] = (bf16_t)acc[0]; v4[1] = (bf16_t)acc[1]; v4[2] = (bf16_t)acc[2]; v4[3] = (bf16_t)acc[3];
      *reinterpret_cast<bf16x4*>(out + ((int64_t)ub * hq + head) * kHeadDim + d4) = v4;
      if (lse != nullptr && (tid & 31) == 0) lse[(int64_t)ub * hq + head] = lse_v;
    } else {
      const int64_t row = (int64_t)uc * hq + head;
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
    constexpr int kMt = C::kTile / 16;  // 16-key M tiles: 2 (bf16) or 4 (fp8, int8)
    // S^T: lane holds keys 16*mt + 4*grp + i (i = 0..3) of head `col`.
    f32x4 s[kMt];
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt) {
      s[mt] = f32x4{};
      const int r = 16 * mt + col;
#pragma unroll
      for (int stp = 0; stp < 4; ++stp) {
        OpT<kKv> a;
        if constexpr (kKv == 0) {
          const int c = 4 * stp + grp;  // d = 32*stp + 8*grp
          a = lds_read16(kb + r * 256 + ((c ^ (r & 15)) << 4));
        } else {
          const int byte = 32 * stp + 8 * grp;
          const int c = byte >> 4;
          const __attribute__((address_space(3))) uint32_t* p =
              (const __attribute__((address_space(3))) uint32_t*)(kb + r * 128 + ((c ^ (r & 7)) << 4) + (byte & 15));
          a = kcodes8_to_op<kKv>(p[0], p[1]);
        }
        s[mt] = mfma_op(a, qf[stp], s[mt]);
      }
    }
    if constexpr (kKv != 0) {
#pragma unroll
      for (int mt = 0; mt < kMt; ++mt) {
        const __attribute__((address_space(3))) f32x4* sp =
            (const __attribute__((address_space(3))) f32x4*)(vb + C::kKBytes + (16 * mt + 4 * grp) * 4);
        f32x4 sc = *sp;
        if constexpr (kKv == 2) s[mt] -= f32x4{kbias, kbias, kbias, kbias};  // biased K codes
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
    if constexpr (kKv != 0) {
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
      uint32_t v8lo[8], v8hi[8];
      if constexpr (kKv == 0) v_transposed(vb, kk, vt);
      else v_transposed8(vb, kk, v8lo, v8hi);
      const OpT<kKv> pb = to_op8<kKv>(s[2 * kk][0], s[2 * kk][1], s[2 * kk][2], s[2 * kk][3],
                                      s[2 * kk + 1][0], s[2 * kk + 1][1], s[2 * kk + 1][2],
                                      s[2 * kk + 1][3]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        OpT<kKv> a;
        if constexpr (kKv == 0) {
          a = vt[dt];
        } else {
          a = codes8_to_op<kKv>(v8lo[dt], v8hi[dt]);
        }
        o[dt] = mfma_op(a, pb, o[dt]);
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
// LSE = -inf. The 32 threads of a head first find the largest partial LSE together, then each
// accumulates its 4 columns over the chunks four at a time, so the loads overlap.
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
  const int64_t row = (int64_t)b * hq + head;
  if (hdr[2] != 0) {
    // the plan found a key count above max_seqlen_k: nothing was computed
    const bf16_t nan_bf16 = (bf16_t)NAN;
    *reinterpret_cast<bf16x4*>(out + row * kHeadDim + d4) = bf16x4{nan_bf16, nan_bf16, nan_bf16, nan_bf16};
    if (lse != nullptr && (tid & 31) == 0) lse[row] = NAN;
    return;
  }
  const int c0 = chunk_base[b];
  const int c1 = min(chunk_base[b + 1], n_chunks);
  if (c1 - c0 == 1) return;
  float M = -INFINITY;
  for (int c = c0 + (tid & 31); c < c1; c += 32) M = fmaxf(M, ws_lse[(int64_t)c * hq + head]);
#pragma unroll
  for (int sh = 1; sh < 32; sh <<= 1) M = fmaxf(M, __shfl_xor(M, sh, 32));
  f32x4 acc = f32x4{};
  float Lsum = 0.f;
  if (M != -INFINITY) {
    int c = c0;
    for (; c + 4 <= c1; c += 4) {
      float l[4];
      f32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l[i] = ws_lse[(int64_t)(c + i) * hq + head];
        v[i] = *(const f32x4*)(ws_o + ((int64_t)(c + i) * hq + head) * kHeadDim + d4);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float w = __expf(l[i] - M);
        Lsum += w;
        acc += w * v[i];
      }
    }
    for (; c < c1; ++c) {
      const float w = __expf(ws_lse[(int64_t)c * hq + head] - M);
      Lsum += w;
      acc += w * *(const f32x4*)(ws_o + ((int64_t)c * hq + head) * kHeadDim + d4);
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


// An upper bound of the chunks the automatic plan lists (num_splits = 0), whatever the key
// counts: the length it picks is at least total * hkv / target, target = kUnitsPerWorkgroup *
// grid, grid = columns * hkv with at most max(1, cu_count / hkv) columns, so the whole chunks
// number at most kUnitsPerWorkgroup * columns and each request adds at most one short chunk;
// at the 2^30 length cap a request of fewer than 2^31 keys has at most two chunks.
int64_t decode_auto_chunk_bound(int64_t batch, int hkv, int cu_count) {
  const int64_t cols = std::max(1, cu_count / std::max(1, hkv));
  return kUnitsPerWorkgroup * cols + 2 * batch;
}

// SEG_ATTN_DECODE_PLAN=kernel keeps the separate plan launch for every call (tests compare the
// two ways of planning).
bool decode_plan_kernel_forced() {
  const char* v = std::getenv("SEG_ATTN_DECODE_PLAN");
  return v != nullptr && std::strcmp(v, "kernel") == 0;
}

hipError_t launch_decode(const void* q, const void* k_pool, const void* v_pool,
                         const float* k_scale, const float* v_scale, int kv, const void* segs,
                         const int32_t* seg_indptr, const int32_t* cu_k, int batch, int hkv,
                         int max_k, int forced_len, int min_len, int max_chunks, int cu_count,
                         float scale, void* out, float* lse, int32_t* hdr, int32_t* chunk_base,
                         int32_t* recs, float* ws_o, float* ws_lse, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  // columns: one workgroup per (column, kv head), about one workgroup per compute unit
  const int cols = (int)std::max<int64_t>(1, std::min<int64_t>(cu_count / hkv, max_chunks));
  const int grid = max_chunks > 0 ? cols * hkv : 0;
  const int target = std::max(1, kUnitsPerWorkgroup * std::max(grid, 1));
  // The split workgroups plan for themselves when the batch fits one request per thread, the
  // chunk length is automatic and every column's units fit the LDS table: at most
  // (kUnitsPerWorkgroup * cols + 2 * batch) / cols of them (decode_auto_chunk_bound).
  const bool in_plan = grid > 0 && forced_len <= 0 && batch <= kInPlanBatch &&
                       kUnitsPerWorkgroup + (2 * batch + cols - 1) / cols <= kUnitCap &&
                       !decode_plan_kernel_forced();
  hipError_t e = hipSuccess;
  if (!in_plan) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, cu_k, seg_indptr,
                       (const Segment*)segs, batch, hkv, forced_len, min_len, target, max_chunks, max_k,
                       hdr, chunk_base, recs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (grid > 0) {
    const float scale_log2 = scale * 1.4426950408889634f;
    const InPlanArgs ipa{cu_k, seg_indptr, chunk_base, batch, min_len, target, max_chunks, max_k};
    auto split = in_plan
        ? (kv == 2 ? decode_split_kernel<2, true> : (kv == 1 ? decode_split_kernel<1, true> : decode_split_kernel<0, true>))
        : (kv == 2 ? decode_split_kernel<2, false> : (kv == 1 ? decode_split_kernel<1, false> : decode_split_kernel<0, false>));
    hipLaunchKernelGGL(split, dim3(grid), dim3(kDecThreads), 0, stream, (const bf16_t*)q, k_pool,
                       v_pool, k_scale, v_scale, (const Segment*)segs, hdr, recs, ipa, hkv, scale,
                       scale_log2, ws_o, ws_lse, (bf16_t*)out, lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(batch * hkv)), dim3(256), 0, stream, ws_o, ws_lse,
                     hdr, chunk_base, hkv, (bf16_t*)out, lse);
  return hipGetLastError();
}

}  // namespace segattn
