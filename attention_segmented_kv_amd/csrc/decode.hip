// Decode kernels: one query token per request against all of its segmented keys.
//
// Split pass: each workgroup owns a (request b, kv head g, key block s) unit — the blockwise
// partial attention of the FlashAccel article ("data layout": attention computed per block,
// then reduced per request). Its 4 waves stream disjoint tiles of the unit's keys, each wave
// through a private double buffer in LDS filled by direct HBM->LDS copies, so no wave waits for
// another until the unit's end. The 8 query heads of kv head g are the columns of one MFMA tile
// (PackGQA, FlashPrefill V2 abstract): every K/V byte is read from HBM once per group.
//   S^T[key][head] = K Q^T   (MFMA 16x16x32 bf16, keys on M; columns 8..15 are padding)
//   O^T[d][head]  += V^T P^T (V^T via the transposing LDS read)
// At the unit's end the 4 per-wave states (m, l, O) are combined in LDS; the result is either
// the final output (one block per request) or a partial (O_s, LSE_s) for the merge kernel.
//
// FP8 pools (OCP E4M3FN codes with one fp32 scale per token and kv head) are converted to bf16
// exactly on the way into the MFMAs; the key scale multiplies the scores, the value scale the
// probabilities, so the arithmetic equals bf16 attention over the dequantised pool.
//
// Merge pass: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s per (request, head).
#include "common.hpp"

namespace segattn {

namespace {

constexpr int kWaves = 4;

template <int kFp8>
struct DecodeCfg;
template <>
struct DecodeCfg<0> {  // bf16: 32 keys per wave tile, 256 B rows
  static constexpr int kTile = 32;
  static constexpr int kRowBytes = 256;
  static constexpr int kKBytes = kTile * kRowBytes;  // 8 KiB
  static constexpr int kScaleBytes = 0;
};
template <>
struct DecodeCfg<1> {  // fp8: 64 keys per wave tile, 128 B rows, + k/v scales
  static constexpr int kTile = 64;
  static constexpr int kRowBytes = 128;
  static constexpr int kKBytes = kTile * kRowBytes;  // 8 KiB
  static constexpr int kScaleBytes = kTile * 4;      // 256 B each
};

template <int kFp8>
struct DecodeLayout {
  using C = DecodeCfg<kFp8>;
  // one stage: K tile, V tile, k scales, v scales
  static constexpr int kStageBytes = 2 * C::kKBytes + 2 * C::kScaleBytes;
  static constexpr int kWaveBytes = 2 * kStageBytes;
  static constexpr int kLdsBytes = kWaves * kWaveBytes;
};

// bf16 rows: chunk c (16 B) of row r stored at position c ^ (r % 16) for K and c ^ vswz(r) for V.
__device__ __forceinline__ int vswz16(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

template <int kFp8>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const bf16_t* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const Segment* __restrict__ segs, const int32_t* __restrict__ seg_indptr,
    const int32_t* __restrict__ cu_k, int batch, int hkv, int split_len, int num_splits,
    float scale, float scale_log2, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    bf16_t* __restrict__ out, float* __restrict__ lse) {
  using C = DecodeCfg<kFp8>;
  using L = DecodeLayout<kFp8>;
  __shared__ __attribute__((aligned(1024))) char smem[L::kLdsBytes];

  const int id = blockIdx.x;
  const int per_split = hkv * batch;
  const int split = id / per_split;
  const int rem = id % per_split;
  const int b = rem / hkv;
  const int g = rem % hkv;
  const int hq = hkv * kGroup;

  const int K = cu_k[b + 1] - cu_k[b];
  const int kbeg = split * split_len;
  if (kbeg >= K && !(num_splits == 1 && split == 0)) return;  // nothing for this block
  const int kstop = min(K, kbeg + split_len);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 15;   // head column of the MFMA tile (>= 8 is padding)
  const int grp = lane >> 4;   // 0..3

  // Q fragments (B operand of S^T): lane holds d = 32*step + 8*grp + (0..7) of head `col`.
  bf16x8 qf[4];
  {
    const bool real = col < kGroup;
    const bf16_t* qrow = q + ((int64_t)b * hq + g * kGroup + (real ? col : 0)) * kHeadDim + 8 * grp;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      qf[st] = real ? *reinterpret_cast<const bf16x8*>(qrow + 32 * st) : bf16x8{};
    }
  }

  char* wave_lds = smem + wave * L::kWaveBytes;
  const int64_t tok_stride = (int64_t)hkv * kHeadDim;  // elements per pool token
  const int n_tiles_unit = (kstop - kbeg + C::kTile - 1) / C::kTile;
  // this wave's tiles: wave, wave + 4, ...
  const int my_tiles = n_tiles_unit > wave ? (n_tiles_unit - wave + kWaves - 1) / kWaves : 0;

  SegCursor cur;   // K/V rows
  cur.init(segs, seg_indptr[b], seg_indptr[b + 1]);
  SegCursor scur;  // FP8 scale rows
  if constexpr (kFp8 == 1) scur.init(segs, seg_indptr[b], seg_indptr[b + 1]);

  auto issue_tile = [&](int t, int stage) {
    const int tile_k0 = kbeg + (wave + t * kWaves) * C::kTile;
    lds_char_t* st = (lds_char_t*)wave_lds + stage * L::kStageBytes;
    lds_char_t* kb = st;
    lds_char_t* vb = st + C::kKBytes;
    if constexpr (kFp8 == 0) {
      // 32 rows x 16 chunks; instruction i covers rows 4i .. 4i+3.
      const int rsub = lane >> 4;
      const int cpos = lane & 15;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + rsub;
        const int j = min(tile_k0 + r, kstop - 1);
        const int64_t base = cur.slot(j) * tok_stride + (int64_t)g * kHeadDim;
        const bf16_t* kp = (const bf16_t*)k_pool + base + ((cpos ^ (r & 15)) << 3);
        const bf16_t* vp = (const bf16_t*)v_pool + base + ((cpos ^ vswz16(r)) << 3);
        copy16_to_lds(kp, (lds_void_t*)(kb + i * 1024));
        copy16_to_lds(vp, (lds_void_t*)(vb + i * 1024));
      }
    } else {
      // 64 rows x 8 chunks of 16 B; instruction i covers rows 8i .. 8i+7.
      const int rsub = lane >> 3;
      const int cpos = lane & 7;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * i + rsub;
        const int j = min(tile_k0 + r, kstop - 1);
        const int64_t tok = cur.slot(j);
        const int64_t base = tok * tok_stride + (int64_t)g * kHeadDim;  // bytes (1 B / element)
        const uint8_t* kp = (const uint8_t*)k_pool + base + ((cpos ^ (r & 7)) << 4);
        const uint8_t* vp = (const uint8_t*)v_pool + base + ((cpos ^ (r & 7)) << 4);
        copy16_to_lds(kp, (lds_void_t*)(kb + i * 1024));
        copy16_to_lds(vp, (lds_void_t*)(vb + i * 1024));
      }
      // scales: lane L loads the scales of row L (its own cursor keeps lookups monotone)
      {
        const int j = min(tile_k0 + lane, kstop - 1);
        const int64_t tok = scur.slot(j);
        copy4_to_lds(k_scale + tok * hkv + g, (lds_void_t*)(st + 2 * C::kKBytes));
        copy4_to_lds(v_scale + tok * hkv + g, (lds_void_t*)(st + 2 * C::kKBytes + C::kScaleBytes));
      }
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{};
  float m_run = -INFINITY;
  float l_run = 0.f;  // partial: this lane's keys only

  if (my_tiles > 0) issue_tile(0, 0);
  for (int t = 0; t < my_tiles; ++t) {
    const int stage = t & 1;
    wait_vmem();
    if (t + 1 < my_tiles) issue_tile(t + 1, stage ^ 1);
    const lds_char_t* st = (const lds_char_t*)wave_lds + stage * L::kStageBytes;
    const lds_char_t* kb = st;
    const lds_char_t* vb = st + C::kKBytes;
    const int tile_k0 = kbeg + (wave + t * kWaves) * C::kTile;
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
            (const __attribute__((address_space(3))) f32x4*)(st + 2 * C::kKBytes + (16 * mt + 4 * grp) * 4);
        f32x4 sc = *sp;
        s[mt] *= sc;
      }
    }
    // mask keys past the unit's end
    if (tile_k0 + C::kTile > kstop) {
#pragma unroll
      for (int mt = 0; mt < kMt; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (tile_k0 + 16 * mt + 4 * grp + i >= kstop) s[mt][i] = -INFINITY;
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
            (const __attribute__((address_space(3))) f32x4*)(st + 2 * C::kKBytes + C::kScaleBytes + (16 * mt + 4 * grp) * 4);
        f32x4 sc = *sp;
        s[mt] *= sc;
      }
    }

    // O^T += V^T P^T, one MFMA k-step per 32 keys (M tiles 2kk and 2kk+1).
#pragma unroll
    for (int kk = 0; kk < kMt / 2; ++kk) {
      bf16x8 pb = to_bf16x8(s[2 * kk][0], s[2 * kk][1], s[2 * kk][2], s[2 * kk][3], s[2 * kk + 1][0],
                            s[2 * kk + 1][1], s[2 * kk + 1][2], s[2 * kk + 1][3]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        bf16x8 a;
        if constexpr (kFp8 == 0) {
          // lane (grp, s=col) addresses row key0 + s/4, column 16*dt + 4*(s%4)
          const int dcol = 16 * dt + 4 * (col & 3);
          const int chunk = dcol >> 3;
          const int within = (dcol & 7) * 2;
          const int ra = 32 * kk + 4 * grp + (col >> 2);
          const int rb = ra + 16;
          bf16x4 lo = lds_read_tr16(vb + ra * 256 + ((chunk ^ vswz16(ra)) << 4) + within);
          bf16x4 hi = lds_read_tr16(vb + rb * 256 + ((chunk ^ vswz16(rb)) << 4) + within);
          a[0] = lo[0]; a[1] = lo[1]; a[2] = lo[2]; a[3] = lo[3];
          a[4] = hi[0]; a[5] = hi[1]; a[6] = hi[2]; a[7] = hi[3];
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
  }

  // ---- combine the 4 waves' states in LDS
  // per wave: m[8], l[8], O[8][128]
  const float l_col = sum_xor32(sum_xor16(l_run));
  __syncthreads();  // all waves done with their tile buffers
  float* red = (float*)(smem + wave * (8 * kHeadDim * 4 + 64));
  if (col < kGroup) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[col * kHeadDim + 16 * dt + 4 * grp + i] = o[dt][i];
    if (grp == 0) {
      red[8 * kHeadDim + col] = m_run;
      red[8 * kHeadDim + 8 + col] = l_col;
    }
  }
  __syncthreads();
  {
    const int hh = tid >> 5;         // head 0..7
    const int d4 = (tid & 31) * 4;   // 4 consecutive d
    float mw[kWaves], lw[kWaves];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* rw = (const float*)(smem + w * (8 * kHeadDim * 4 + 64));
      mw[w] = rw[8 * kHeadDim + hh];
      lw[w] = rw[8 * kHeadDim + 8 + hh];
      M = fmaxf(M, mw[w]);
    }
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float Lsum = 0.f;
    f32x4 acc = f32x4{};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float cw = fast_exp2((mw[w] - M_use) * scale_log2);
      Lsum += cw * lw[w];
      const float* rw = (const float*)(smem + w * (8 * kHeadDim * 4 + 64));
      f32x4 v = *(const f32x4*)(rw + hh * kHeadDim + d4);
      acc += cw * v;
    }
    const float inv = Lsum > 0.f ? 1.0f / Lsum : 0.f;
    acc *= inv;
    const float lse_v = Lsum > 0.f ? M * scale + __logf(Lsum) : -INFINITY;
    const int head = g * kGroup + hh;
    if (num_splits == 1) {
      bf16x4 v4;
      v4[0] = (bf16_t)acc[0]; v4[1] = (bf16_t)acc[1]; v4[2] = (bf16_t)acc[2]; v4[3] = (bf16_t)acc[3];
      *reinterpret_cast<bf16x4*>(out + ((int64_t)b * hq + head) * kHeadDim + d4) = v4;
      if (lse != nullptr && (tid & 31) == 0) lse[(int64_t)b * hq + head] = lse_v;
    } else {
      const int64_t slot = ((int64_t)b * hq + head) * num_splits + split;
      *reinterpret_cast<f32x4*>(ws_o + slot * kHeadDim + d4) = acc;
      if ((tid & 31) == 0) ws_lse[slot] = lse_v;
    }
  }
}

// One workgroup per (request, kv head): 256 threads = 8 heads x 32 threads x 4 d.
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ ws_o,
                                                    const float* __restrict__ ws_lse,
                                                    const int32_t* __restrict__ cu_k, int hkv,
                                                    int split_len, int num_splits,
                                                    bf16_t* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int b = blockIdx.x / hkv;
  const int g = blockIdx.x % hkv;
  const int hq = hkv * kGroup;
  const int tid = threadIdx.x;
  const int head = g * kGroup + (tid >> 5);
  const int d4 = (tid & 31) * 4;
  const int K = cu_k[b + 1] - cu_k[b];
  const int ns = min(num_splits, (K + split_len - 1) / split_len);
  const int64_t row = (int64_t)b * hq + head;
  const float* lrow = ws_lse + row * num_splits;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, lrow[s]);
  f32x4 acc = f32x4{};
  float Lsum = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < ns; ++s) {
      const float w = __expf(lrow[s] - M);
      Lsum += w;
      f32x4 v = *(const f32x4*)(ws_o + (row * num_splits + s) * kHeadDim + d4);
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

hipError_t launch_decode(const void* q, const void* k_pool, const void* v_pool,
                         const float* k_scale, const float* v_scale, int fp8, const void* segs,
                         const int32_t* seg_indptr, const int32_t* cu_k, int batch, int hkv,
                         int split_len, int num_splits, float scale, void* out, float* lse,
                         float* ws_o, float* ws_lse, hipStream_t stream) {
  const int64_t grid = (int64_t)num_splits * hkv * batch;
  if (grid == 0) return hipSuccess;
  const float scale_log2 = scale * 1.4426950408889634f;
  if (fp8) {
    hipLaunchKernelGGL(decode_split_kernel<1>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const bf16_t*)q, k_pool, v_pool, k_scale, v_scale, (const Segment*)segs,
                       seg_indptr, cu_k, batch, hkv, split_len, num_splits, scale, scale_log2,
                       ws_o, ws_lse, (bf16_t*)out, lse);
  } else {
    hipLaunchKernelGGL(decode_split_kernel<0>, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const bf16_t*)q, k_pool, v_pool, k_scale, v_scale, (const Segment*)segs,
                       seg_indptr, cu_k, batch, hkv, split_len, num_splits, scale, scale_log2,
                       ws_o, ws_lse, (bf16_t*)out, lse);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || num_splits == 1) return e;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(batch * hkv)), dim3(256), 0, stream, ws_o, ws_lse,
                     cu_k, hkv, split_len, num_splits, (bf16_t*)out, lse);
  return hipGetLastError();
}

int decode_lds_bytes(int fp8) { return fp8 ? DecodeLayout<1>::kLdsBytes : DecodeLayout<0>::kLdsBytes; }

}  // namespace segattn
