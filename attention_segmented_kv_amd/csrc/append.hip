// KV append: a batch's new tokens' K and V rows written into their requests' segments, the step
// ahead of attention. Each request's cache is a few contiguous segments of one shared pool
// (Flood README, "Introduction"); the FP8 and INT8 variants quantise on write, one fp32 scale
// per (token, kv head) row, for the FP8 KV cache of the same README's feature list and the
// INT8 KV cache of "FlashAttention on Ascend NPU", optimisation 3.
//
// Request b appends n_b = cu_new[b+1] - cu_new[b] tokens and cu_k counts its keys after the
// append, so its new tokens are its last n_b keys, logical positions K_b - n_b .. K_b - 1.
//
// One 16-lane group per (token, kv head) row of 128 values, 16 rows per 256-thread workgroup.
// The group loads its row (8 values per lane, 16-byte pieces), finds the token's request and
// the key's pool slot with its lanes working together on the tables, and stores the row there.
// The FP8 row scale is max|x| / 448 (1 for an all-zero row); each value is divided by it in
// fp32, correctly rounded, clamped to +-448 and converted to E4M3FN (round to nearest, ties to
// even). INT8 is the same with 127 in place of 448 and a rounding to the nearest integer, ties
// to even. The kernels reach the same bits by cheaper means: both divisions are replaced by
// sequences that give the same scale and the same codes for every bf16 input, and the clamp is
// left out where it cannot change a code (below).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace segattn {

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Seg {
  int32_t off, len;
};

constexpr int kRowsPerBlock = 16;

// The row scale RN(a / M) for a bf16 row maximum a > 0: s0 = a c with c = RN(1 / M), then one
// residual step s0 - (s0 M - a) c, the residual exact in an fma. Equal to the correctly
// rounded quotient for every positive finite bf16 a, for M = 448 and M = 127 (checked
// exhaustively over the 32640 values).
template <int kM>
__device__ __forceinline__ float row_scale(float a) {
  constexpr float c = 1.0f / (float)kM;
  const float s0 = a * c;
  return __builtin_fmaf(-__builtin_fmaf(s0, (float)kM, -a), c, s0);
}

// The code of x / s, from any reciprocal r within one ulp of 1 / s (the hardware reciprocal):
// q = x r, then one residual step q - (q s - x) r. For a bf16 x with |x| <= a, the row's bf16
// maximum, and s = RN(a / M) in [2^-80, 2^80], q may differ from the correctly rounded quotient
// in its last bit, but never across a rounding boundary of the code: its E4M3FN code (M = 448)
// or its nearest integer (M = 127) equals that of the correctly rounded quotient. Checked
// exhaustively, every such (x, a) pair and each of the three reciprocals RN(1 / s) and its two
// neighbours; a second residual step (Markstein's correctly rounded division) would change no
// code. Written with the negated residual so that x = -0 keeps its sign.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float q = __fmul_rn(x, r);
  return __builtin_fmaf(-__builtin_fmaf(q, s, -x), r, q);
}

// Lane data movement inside the 16-lane DPP rows, which are the row groups: kCtrl is a DPP
// control (quad_perm 0x00-0xFF, row_shr 0x111-0x11F, row_mirror 0x140, row_half_mirror 0x141).
// A lane whose source lies outside its row reads 0.
template <int kCtrl>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}

// Maximum over the 16 lanes of a row group of non-negative floats (their bit patterns order
// like the values): swap neighbours, then pairs, then quads (half-row mirror), then halves.
__device__ __forceinline__ float group_max_nonneg(float v) {
  int b = __builtin_bit_cast(int, v);
  b = max(b, dpp<0xB1>(b));   // quad_perm [1, 0, 3, 2]
  b = max(b, dpp<0x4E>(b));   // quad_perm [2, 3, 0, 1]
  b = max(b, dpp<0x141>(b));  // row_half_mirror
  b = max(b, dpp<0x140>(b));  // row_mirror
  return __builtin_bit_cast(float, b);
}

// Inclusive prefix sum over the 16 lanes of a row group.
__device__ __forceinline__ int group_inclusive_sum(int v) {
  v += dpp<0x111>(v);  // row_shr 1
  v += dpp<0x112>(v);  // row_shr 2
  v += dpp<0x114>(v);  // row_shr 4
  v += dpp<0x118>(v);  // row_shr 8
  return v;
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4 raw, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __builtin_bit_cast(float, raw[i] << 16);
    x[2 * i + 1] = __builtin_bit_cast(float, raw[i] & 0xFFFF0000u);
  }
}

// No clamp is needed before either encoding: with |x| <= a and s = RN(a / M) >= (a / M)(1 - 2^-24)
// every quotient has |q| <= M (1 + 2^-22), which still rounds to +-M.

// Eight quotients as E4M3FN codes (byte i = value i): the hardware conversion, two values per
// instruction, the second pair into the high half of the word.
__device__ __forceinline__ u32x2 encode_fp8x8(const float (&y)[8]) {
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i], y[4 * i + 1], 0, false);
    w[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i + 2], y[4 * i + 3], lo, true);
  }
  return u32x2{w[0], w[1]};
}

// Eight quotients rounded to the nearest integer (ties to even), as two's-complement bytes
// (byte i = value i). Adding 1.5 * 2^23 rounds a float of magnitude below 2^22 to an integer
// in the fp32 addition itself (round to nearest even), and the sum's low byte is that integer
// modulo 256; byte permutes gather the four low bytes of a word.
__device__ __forceinline__ u32x2 encode_int8x8(const float (&y)[8]) {
  uint32_t w[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = __builtin_bit_cast(uint32_t, y[4 * i + q] + 0x1.8p23f);
    const uint32_t p01 = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);  // b0.byte0, b1.byte0
    const uint32_t p23 = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);
    w[i] = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
  }
  return u32x2{w[0], w[1]};
}

// Mask of the calling lane's 16-lane group (bit i = group lane i) of a predicate.
__device__ __forceinline__ uint32_t group_ballot(bool p) {
  const int shift = __lane_id() & 48;
  return (uint32_t)(__ballot(p) >> shift) & 0xFFFFu;
}

// Pool slot of new token t (all 16 lanes of the calling group take part and get the result), or
// -1 when the tables do not give it one.
__device__ __forceinline__ int64_t find_slot(int t, int sub, const Seg* __restrict__ segs,
                                             const int32_t* __restrict__ seg_indptr,
                                             const int32_t* __restrict__ cu_new,
                                             const int32_t* __restrict__ cu_k, int batch) {
  // Request of token t: the largest b with cu_new[b] <= t (requests without new tokens have
  // cu_new[b] == cu_new[b + 1] and are passed over). The group's 16 lanes probe 16 evenly
  // spaced entries of [lo, hi) at once, which shrinks the range 16-fold per step: one step for
  // up to 17 requests, two for up to 257.
  int lo = 0, hi = batch;
  while (hi - lo > 1) {
    const int step = (hi - lo + 14) >> 4;  // ceil((hi - lo - 1) / 16)
    const int idx = lo + (sub + 1) * step;
    const uint32_t le = group_ballot(idx < hi && cu_new[idx] <= t);  // a prefix of the lanes
    const int c = __popc(le);
    hi = min(hi, lo + (c + 1) * step);
    lo += c * step;
  }
  const int b = lo;
  const int n0 = cu_new[b], n1 = cu_new[b + 1];
  const int j = (cu_k[b + 1] - cu_k[b]) - (n1 - n0) + (t - n0);  // logical key of token t
  const int seg_end = seg_indptr[b + 1];

  // Its pool slot: the group reads 16 of the request's segments at once, and the lane whose
  // key range [start, start + len) holds j gives the slot (empty segments hold nothing).
  int64_t slot = -1;
  int before = 0;  // keys in the request's segments ahead of this batch of 16
  for (int first = seg_indptr[b]; first < seg_end; first += 16) {
    const int idx = first + sub;
    const Seg sg = idx < seg_end ? segs[idx] : Seg{0, 0};
    const int incl = group_inclusive_sum(sg.len);
    const int start = before + incl - sg.len;
    const uint32_t hit = group_ballot(j >= start && j < before + incl);
    if (hit != 0) {
      const int src_lane = __ffs(hit) - 1;
      slot = (int64_t)__shfl(sg.off, src_lane, 16) + (j - __shfl(start, src_lane, 16));
      break;
    }
    before += __shfl(incl, 15, 16);
  }
  return j < 0 ? -1 : slot;
}

// Quantise one (token, kv head) row of K and of V (8 values per lane of the 16-lane group) and
// store codes and scales at pool row dst_row.
template <int kFmt>
__device__ __forceinline__ void quantise_row_pair(const u32x4 kraw, const u32x4 vraw, int sub,
                                                  int64_t dst_row, uint8_t* __restrict__ k_pool,
                                                  uint8_t* __restrict__ v_pool,
                                                  float* __restrict__ k_scale,
                                                  float* __restrict__ v_scale) {
    // K and V rows side by side: row maxima over the group, scales, quotients, codes
    float xk[8], xv[8];
    unpack_bf16x8(kraw, xk);
    unpack_bf16x8(vraw, xv);
    float ak = 0.f, av = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ak = fmaxf(ak, fabsf(xk[i]));
      av = fmaxf(av, fabsf(xv[i]));
    }
    ak = group_max_nonneg(ak);
    av = group_max_nonneg(av);
    constexpr int kM = kFmt == 1 ? 448 : 127;
    const float sk = ak > 0.f ? row_scale<kM>(ak) : 1.0f;
    const float sv = av > 0.f ? row_scale<kM>(av) : 1.0f;
    float yk[8], yv[8];
    auto in_range = [](float s) { return s >= 0x1p-80f && s <= 0x1p80f; };
    if (in_range(sk) && in_range(sv)) {  // the same for the whole group
      const float rk = __builtin_amdgcn_rcpf(sk), rv = __builtin_amdgcn_rcpf(sv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        yk[i] = div_by_scale(xk[i], sk, rk);
        yv[i] = div_by_scale(xv[i], sv, rv);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        yk[i] = xk[i] / sk;
        yv[i] = xv[i] / sv;
      }
    }
    const int64_t dst = dst_row * 128 + 8 * sub;
    const u32x2 ck = kFmt == 1 ? encode_fp8x8(yk) : encode_int8x8(yk);
    const u32x2 cv = kFmt == 1 ? encode_fp8x8(yv) : encode_int8x8(yv);
    __builtin_nontemporal_store(ck, reinterpret_cast<u32x2*>(k_pool + dst));
    __builtin_nontemporal_store(cv, reinterpret_cast<u32x2*>(v_pool + dst));
    if (sub == 0) {
      k_scale[dst_row] = sk;
      v_scale[dst_row] = sv;
    }
}

// kFmt: 0 = bf16 pool (copy), 1 = FP8 (E4M3FN) pool, 2 = INT8 pool.
template <int kFmt>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const Seg* __restrict__ segs, const int32_t* __restrict__ seg_indptr,
    const int32_t* __restrict__ cu_new, const int32_t* __restrict__ cu_k, int batch, int total_new,
    int hkv, int64_t pool_tokens, void* __restrict__ k_pool, void* __restrict__ v_pool,
    float* __restrict__ k_scale, float* __restrict__ v_scale) {
  // rows number fewer than 2^31 (checked by the caller), so 32-bit index arithmetic suffices
  const uint32_t row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  if (row >= (uint32_t)total_new * (uint32_t)hkv) return;  // whole 16-lane groups leave together
  const int sub = threadIdx.x & 15;                         // values 8 sub .. 8 sub + 7 of the row
  const int t = (int)(row / (uint32_t)hkv);
  const int h = (int)(row - (uint32_t)t * (uint32_t)hkv);

  // the row's values are loaded first: they do not depend on where the row goes
  const int64_t src = (int64_t)row * 128 + 8 * sub;
  const u32x4 kraw = *reinterpret_cast<const u32x4*>(k_new + src);
  const u32x4 vraw = *reinterpret_cast<const u32x4*>(v_new + src);

  const int64_t slot = find_slot(t, sub, segs, seg_indptr, cu_new, cu_k, batch);
  // a key outside the request's segments or the pool means inconsistent tables: nothing is
  // written for it rather than a write out of bounds
  if (slot < 0 || slot >= pool_tokens) return;

  const int64_t dst_row = slot * hkv + h;
  if constexpr (kFmt == 0) {
    __builtin_nontemporal_store(kraw, reinterpret_cast<u32x4*>((uint16_t*)k_pool + dst_row * 128 + 8 * sub));
    __builtin_nontemporal_store(vraw, reinterpret_cast<u32x4*>((uint16_t*)v_pool + dst_row * 128 + 8 * sub));
  } else {
    quantise_row_pair<kFmt>(kraw, vraw, sub, dst_row, (uint8_t*)k_pool, (uint8_t*)v_pool, k_scale, v_scale);
  }
}

// FP8 / INT8 pools: one 16-lane group per new token, all of its kv heads. The slot lookup is
// done once per token, and the rows of up to 8 heads are loaded before any is quantised.
constexpr int kHeadsPerPass = 8;
constexpr int kTokenPathMin = 4096;  // new tokens from which the per-token kernel is used

template <int kFmt>
__global__ __launch_bounds__(256) void kv_append_token_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const Seg* __restrict__ segs, const int32_t* __restrict__ seg_indptr,
    const int32_t* __restrict__ cu_new, const int32_t* __restrict__ cu_k, int batch, int total_new,
    int hkv, int64_t pool_tokens, uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    float* __restrict__ k_scale, float* __restrict__ v_scale) {
  const int t = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  if (t >= total_new) return;  // whole 16-lane groups leave together
  const int sub = threadIdx.x & 15;
  const int64_t src0 = (int64_t)t * hkv * 128 + 8 * sub;
  u32x4 kraw[kHeadsPerPass], vraw[kHeadsPerPass];
  auto load_pass = [&](int h0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kHeadsPerPass; ++i) {
      if (h0 + i < hkv) {
        kraw[i] = *reinterpret_cast<const u32x4*>(k_new + src0 + (int64_t)(h0 + i) * 128);
        vraw[i] = *reinterpret_cast<const u32x4*>(v_new + src0 + (int64_t)(h0 + i) * 128);
      }
    }
  };
  load_pass(0);  // in flight during the lookup
  const int64_t slot = find_slot(t, sub, segs, seg_indptr, cu_new, cu_k, batch);
  // a key outside the request's segments or the pool means inconsistent tables: nothing is
  // written for it rather than a write out of bounds
  if (slot < 0 || slot >= pool_tokens) return;
  for (int h0 = 0; h0 < hkv; h0 += kHeadsPerPass) {
    if (h0 > 0) load_pass(h0);
#pragma unroll
    for (int i = 0; i < kHeadsPerPass; ++i) {
      if (h0 + i < hkv)
        quantise_row_pair<kFmt>(kraw[i], vraw[i], sub, slot * hkv + h0 + i, k_pool, v_pool, k_scale,
                                v_scale);
    }
  }
}

// ------------------------------------------------------------------------------------------
// KV move: the pool side of the allocator's compaction. A move copies the rows of `len`
// consecutive pool slots (every kv head; K, V and, for one-byte pools, their scales) from
// slot src to slot dst. Moves are listed with `first`, the number of slots of all earlier moves,
// so flattened slot t of the list belongs to the last move whose first <= t. The allocator only
// plans moves whose sources and destinations are pairwise disjoint, so every row is copied
// independently: one 16-lane group per (slot, kv head) row, 16 rows per workgroup.
struct Move {
  int32_t src, dst, len, first;
};

template <bool kOneByte>
__global__ __launch_bounds__(256) void kv_move_kernel(const Move* __restrict__ moves, int n_moves,
                                                      int64_t total_rows, int hkv, int64_t pool_tokens,
                                                      char* __restrict__ k_pool, char* __restrict__ v_pool,
                                                      float* __restrict__ k_scale,
                                                      float* __restrict__ v_scale) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  if (row >= total_rows) return;
  const int l16 = threadIdx.x & 15;
  const int64_t t = row / hkv;
  const int g = (int)(row - t * hkv);
  // the last move with first <= t
  int lo = 0, hi = n_moves - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (moves[mid].first <= t) lo = mid;
    else hi = mid - 1;
  }
  const Move mv = moves[lo];
  const int64_t k = t - mv.first;
  if (k < 0 || k >= mv.len) return;  // a list whose `first` values do not add up
  const int64_t src = (int64_t)mv.src + k, dst = (int64_t)mv.dst + k;
  if (src < 0 || src >= pool_tokens || dst < 0 || dst >= pool_tokens) return;
  constexpr int64_t kRowBytes = kOneByte ? 128 : 256;
  const int64_t so = (src * hkv + g) * kRowBytes, dO = (dst * hkv + g) * kRowBytes;
  if constexpr (kOneByte) {
    const u32x2 kv = *reinterpret_cast<const u32x2*>(k_pool + so + 8 * l16);
    const u32x2 vv = *reinterpret_cast<const u32x2*>(v_pool + so + 8 * l16);
    *reinterpret_cast<u32x2*>(k_pool + dO + 8 * l16) = kv;
    *reinterpret_cast<u32x2*>(v_pool + dO + 8 * l16) = vv;
    if (l16 == 0) {
      k_scale[dst * hkv + g] = k_scale[src * hkv + g];
      v_scale[dst * hkv + g] = v_scale[src * hkv + g];
    }
  } else {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(k_pool + so + 16 * l16);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(v_pool + so + 16 * l16);
    *reinterpret_cast<u32x4*>(k_pool + dO + 16 * l16) = kv;
    *reinterpret_cast<u32x4*>(v_pool + dO + 16 * l16) = vv;
  }
}

}  // namespace

hipError_t launch_kv_move(const void* moves, int n_moves, int64_t total_tokens, int hkv,
                          int64_t pool_tokens, int fmt, void* k_pool, void* v_pool, float* k_scale,
                          float* v_scale, hipStream_t stream) {
  const int64_t rows = total_tokens * hkv;
  const int64_t grid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (grid == 0 || n_moves == 0) return hipSuccess;
  auto kern = fmt != 0 ? kv_move_kernel<true> : kv_move_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, stream, (const Move*)moves, n_moves, rows,
                     hkv, pool_tokens, (char*)k_pool, (char*)v_pool, k_scale, v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, const void* segs,
                            const int32_t* seg_indptr, const int32_t* cu_new, const int32_t* cu_k,
                            int batch, int total_new, int hkv, int64_t pool_tokens, int fmt,
                            void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                            hipStream_t stream) {
  const int64_t rows = (int64_t)total_new * hkv;
  if (rows == 0) return hipSuccess;
  if (rows > INT32_MAX) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  // FP8 / INT8: one group per token (one lookup per token) once there are enough tokens to fill
  // the chip with it; below that, one group per (token, head) row keeps more groups in flight.
  if (fmt == 0 || total_new < kTokenPathMin) {
    auto kern = fmt == 2 ? kv_append_kernel<2> : (fmt == 1 ? kv_append_kernel<1> : kv_append_kernel<0>);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, stream, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, (const Seg*)segs, seg_indptr, cu_new, cu_k, batch,
                       total_new, hkv, pool_tokens, k_pool, v_pool, k_scale, v_scale);
  } else {
    const unsigned tgrid = (unsigned)((total_new + kRowsPerBlock - 1) / kRowsPerBlock);
    auto kern = fmt == 2 ? kv_append_token_kernel<2> : kv_append_token_kernel<1>;
    hipLaunchKernelGGL(kern, dim3(tgrid), dim3(256), 0, stream, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, (const Seg*)segs, seg_indptr, cu_new, cu_k, batch,
                       total_new, hkv, pool_tokens, (uint8_t*)k_pool, (uint8_t*)v_pool, k_scale, v_scale);
  }
  return hipGetLastError();
}

}  // namespace segattn
