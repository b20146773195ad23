// Segment linear attention: simple gated linear attention over a pool of per-request states, the
// kernel family of the Flood README's "Seg-linear-attn" table (16 heads, 16 kv heads, d = 128,
// measured against flash-linear-attention's chunked prefill and recurrent decode). Per request
// and head, with a scalar log decay g_t <= 0 per token:
//   S_t = exp(g_t) S_{t-1} + k_t^T v_t      (S: d_k x d_v, fp32)
//   o_t = scale * q_t S_t
// A request's state lives in one slot of the pool [slots, H, 128, 128] (d_k rows, d_v columns
// contiguous).
//
// Prefill works in chunks of 64 tokens. With G_t the running sum of g within the chunk (G_last
// for its last token) and S the state before the chunk:
//   O   = scale * ( diag(exp(G)) Q S + P V ),  P[t][s] = (q_t . k_s) exp(G_t - G_s) for s <= t
//   S' = exp(G_last) S + K~^T V,              K~[s] = exp(G_last - G_s) k_s
// which is the recurrence regrouped. The d_v columns of S and V split into independent halves,
// so a workgroup handles one (request, head, 64-column half) and walks the request's chunks in
// order, holding its half of the state in MFMA accumulators (fp32) and feeding it to Q S as
// bf16. MFMA 32x32x16 bf16 throughout, everything transposed so that the chunk's tokens sit on
// the N side: O^T = S^T Q^T + V^T P^T, P^T from K Q^T, and S'^T = exp(G_last) S^T + V^T K~.
//
// Decode (one token per request) streams each state once: a workgroup per (request, head) reads
// S, writes exp(g) S + k^T v and reduces q . S' over the rows.
#include "common.hpp"

namespace segattn {

namespace {

constexpr int kLaDim = 128;
constexpr int kChunk = 64;
constexpr int kLaThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __builtin_bit_cast(float, b << 16); }
// float -> bf16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------------------------------- decode

__global__ __launch_bounds__(kLaThreads) void la_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const int32_t* __restrict__ slots, int H, float scale,
    float* __restrict__ pool, int64_t pool_slots, uint16_t* __restrict__ out) {
  __shared__ float qk[2][kLaDim];
  __shared__ f32x4v red[8][32];
  const int b = blockIdx.x / H, h = blockIdx.x - b * H;
  const int tid = threadIdx.x;
  const int64_t slot = slots[b];
  if (slot < 0 || slot >= pool_slots) return;  // the whole workgroup leaves together
  const int64_t row = (int64_t)b * H + h;
  qk[tid >> 7][tid & 127] = bf16_bits_to_float((tid < 128 ? q : k)[row * kLaDim + (tid & 127)]);
  const int j4 = tid & 31;  // columns 4 j4 .. 4 j4 + 3
  const int ig = tid >> 5;  // rows ig, ig + 8, ..., ig + 120
  const u32x2 vb = *reinterpret_cast<const u32x2*>(v + row * kLaDim + 4 * j4);
  const f32x4v vv = {bf16_bits_to_float(vb[0] & 0xFFFFu), bf16_bits_to_float(vb[0] >> 16),
                     bf16_bits_to_float(vb[1] & 0xFFFFu), bf16_bits_to_float(vb[1] >> 16)};
  const float decay = __expf(g[row]);
  f32x4v* st = reinterpret_cast<f32x4v*>(pool + (slot * H + h) * (int64_t)(kLaDim * kLaDim)) + j4;
  f32x4v s[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = st[(ig + 8 * r) * 32];
  __syncthreads();
  f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = ig + 8 * r;
    const float ki = qk[1][i], qi = qk[0][i];
    s[r] = s[r] * decay + ki * vv;
    st[i * 32] = s[r];
    acc += qi * s[r];
  }
  red[ig][j4] = acc;
  __syncthreads();
  if (tid < 128) {
    const float* rf = reinterpret_cast<const float*>(&red[0][0]);
    float o = 0.f;
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) o += rf[gi * 128 + tid];
    out[row * kLaDim + tid] = (uint16_t)float_to_bf16_bits(o * scale);
  }
}

// ------------------------------------------------------------------------------------ prefill

// LDS layouts (bf16):
//   Qs, Ks [64 t][128 i]: 16-byte chunk c of row r at chunk position c ^ (r % 16)
//   St     [64 d][128 i]: the bf16 state half, S^T, same swizzle
//   Vt     [64 d][64 s]:  V^T of the half, 8-byte unit u of row r at u ^ (r % 16)
//   Kt     [128 i][64 s]: K~^T, same 8-byte swizzle
//   Gs     [64] fp32:      the chunk's running decay sums
// Ordered so that the chunk-output kernel, which needs only Qs, Ks, Vt and Gs, takes the first
// 40.25 KiB, and the chunk-state kernel, which needs Vt and Kt, the first 56.25 KiB.
constexpr int kQsOff = 0;                              // Qs: 16 KiB
constexpr int kKsOff = kQsOff + kChunk * kLaDim * 2;   // Ks: 16 KiB
constexpr int kVtOff = kKsOff + kChunk * kLaDim * 2;   // Vt: 8 KiB
constexpr int kGsOff = kVtOff + 64 * kChunk * 2;       // Gs: 256 B
constexpr int kOutLds = kGsOff + kChunk * 4;           // 40.25 KiB
constexpr int kKtOff = kOutLds;                        // Kt: 16 KiB
constexpr int kStateLds = kKtOff + kLaDim * kChunk * 2;  // 56.25 KiB
constexpr int kStOff = kStateLds;                      // St: 16 KiB
constexpr int kLaLds = kStOff + 64 * kLaDim * 2;       // 72.25 KiB in all

__device__ __forceinline__ int chunk16(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
__device__ __forceinline__ int unit8(int r, int u) { return r * 128 + ((u ^ (r & 15)) << 3); }

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_sum(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

__global__ __launch_bounds__(kLaThreads) void la_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const int32_t* __restrict__ cu, const int32_t* __restrict__ slots,
    int H, float scale, int initial_state, float* __restrict__ pool, int64_t pool_slots,
    uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kLaLds];
  lds_char_t* lds = (lds_char_t*)lds_raw;
  // the two d_v halves of a (request, head) are workgroups bh and bh + gridDim.x / 2: with
  // gridDim.x / 2 a multiple of 8 they are dispatched to the same XCD and read q, k through
  // one L2
  const int half_grid = gridDim.x >> 1;
  const int vs = blockIdx.x >= half_grid;
  const int bh = blockIdx.x - vs * half_grid;
  const int b = bh / H, h = bh - b * H;
  const int64_t slot = slots[b];
  if (slot < 0 || slot >= pool_slots) return;  // the whole workgroup leaves together
  const int t_begin = cu[b], n = cu[b + 1] - t_begin;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int md = wave & 1;   // d tile (32 columns of the half) of this wave's O^T and S^T tiles
  const int nt = wave >> 1;  // t tile of this wave's O^T tile
  const int np = wave >> 1;  // S^T tiles ni = 2 np, 2 np + 1 (i = 32 ni + l32)

  // ---- the state half S^T[d][i], d = 32 md + 8 (e >> 2) + 4 hh + (e & 3), i = 32 ni + l32
  float* sbase = pool + (slot * H + h) * (int64_t)(kLaDim * kLaDim) + 64 * vs;
  f32x16 st[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = 32 * (2 * np + u) + l32;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      f32x4v x = {0.f, 0.f, 0.f, 0.f};
      if (initial_state) x = *reinterpret_cast<const f32x4v*>(sbase + i * kLaDim + 32 * md + 8 * qd + 4 * hh);
#pragma unroll
      for (int c = 0; c < 4; ++c) st[u][4 * qd + c] = x[c];
    }
  }

  // ---- staging registers for one chunk: Q, K rows (4 x 16 B each), V half (2 x 16 B), g
  const int srow = tid >> 2;  // token row of the chunk this thread stages
  u32x4 rq[4], rk[4], rv[2];
  float rg = 0.f;
  const int64_t hstride = (int64_t)H * kLaDim;
  auto fetch = [&](int c0) __attribute__((always_inline)) {
    const int t = c0 + srow;
    const bool ok = t < n;
    const int64_t base = (int64_t)(t_begin + t) * hstride + (int64_t)h * kLaDim;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = 4 * (tid & 3) + c;
      rq[c] = ok ? *reinterpret_cast<const u32x4*>(q + base + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
      rk[c] = ok ? *reinterpret_cast<const u32x4*>(k + base + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ch = 2 * (tid & 3) + c;
      rv[c] = ok ? *reinterpret_cast<const u32x4*>(v + base + 64 * vs + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
    }
    const int tg = c0 + lane;
    rg = tg < n ? g[(int64_t)(t_begin + tg) * H + h] : 0.f;
  };

  const int nchunks = (n + kChunk - 1) / kChunk;
  if (nchunks > 0) fetch(0);
  for (int ci = 0; ci < nchunks; ++ci) {
    const int c0 = ci * kChunk;
    // ---- running decay sums of the chunk (every wave holds them, lane t = token t)
    const float G = wave_inclusive_sum(rg);
    const float Glast = __shfl(G, 63, 64);
    // ---- stage the chunk and the state half into LDS
    {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int ch = 4 * (tid & 3) + c;
        *(__attribute__((address_space(3))) u32x4*)(lds + kQsOff + chunk16(srow, ch)) = rq[c];
        *(__attribute__((address_space(3))) u32x4*)(lds + kKsOff + chunk16(srow, ch)) = rk[c];
      }
      // K~^T[i][s] = bf16(k_s[i] * exp(G_last - G_s)), s = srow
      const float ws = __expf(Glast - __shfl(G, srow, 64));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int ch = 4 * (tid & 3) + c;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (rk[c][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          const int i = 8 * ch + e;
          *(__attribute__((address_space(3))) uint16_t*)(lds + kKtOff + unit8(i, srow >> 2) + 2 * (srow & 3)) =
              (uint16_t)float_to_bf16_bits(bf16_bits_to_float(bits) * ws);
        }
      }
      // V^T[d][s], s = srow
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ch = 2 * (tid & 3) + c;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * ch + e;
          *(__attribute__((address_space(3))) uint16_t*)(lds + kVtOff + unit8(d, srow >> 2) + 2 * (srow & 3)) =
              (uint16_t)((rv[c][e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
      }
      if (wave == 0) *(__attribute__((address_space(3))) float*)(lds + kGsOff + 4 * lane) = G;
      // S^T as bf16
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = 32 * (2 * np + u) + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int d = 32 * md + 8 * (e >> 2) + 4 * hh + (e & 3);
          *(__attribute__((address_space(3))) uint16_t*)(lds + kStOff + chunk16(d, i >> 3) + 2 * (i & 7)) =
              (uint16_t)float_to_bf16_bits(st[u][e]);
        }
      }
    }
    __syncthreads();
    if (ci + 1 < nchunks) fetch(c0 + kChunk);  // in flight during the chunk's math

    const int t = 32 * nt + l32;              // this lane's token (column of the O^T tile)
    const float Gt = __shfl(G, t, 64);
    // ---- O^T = S^T Q^T (state before the chunk), scaled by exp(G_t) per column
    f32x16 o = {};
    if (ci > 0 || initial_state) {
#pragma unroll
      for (int stp = 0; stp < 8; ++stp) {
        const bf16x8 a = lds_read16(lds + kStOff + chunk16(32 * md + l32, 2 * stp + hh));
        const bf16x8 bq = lds_read16(lds + kQsOff + chunk16(t, 2 * stp + hh));
        o = mfma32x32x16(a, bq, o);
      }
      const float et = __expf(Gt);
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] *= et;
    }
    // ---- V^T fragments of the wave's d tile: A operands for s = 16 stp + {4hh..4hh+3, 8+4hh..}
    bf16x8 vt[4];
#pragma unroll
    for (int stp = 0; stp < 4; ++stp) {
      const int r = 32 * md + l32;
      const u32x2 lo = *(const __attribute__((address_space(3))) u32x2*)(lds + kVtOff + unit8(r, 4 * stp + hh));
      const u32x2 hi = *(const __attribute__((address_space(3))) u32x2*)(lds + kVtOff + unit8(r, 4 * stp + 2 + hh));
      const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
      vt[stp] = __builtin_bit_cast(bf16x8, w);
    }
    // ---- P^T = (K Q^T) * exp(G_t - G_s) for s <= t, and O^T += V^T P^T
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      if (ms > nt) break;  // keys s >= 32 > t: all masked for the first t tile
      f32x16 a = {};
#pragma unroll
      for (int stp = 0; stp < 8; ++stp) {
        const bf16x8 ka = lds_read16(lds + kKsOff + chunk16(32 * ms + l32, 2 * stp + hh));
        const bf16x8 qb = lds_read16(lds + kQsOff + chunk16(t, 2 * stp + hh));
        a = mfma32x32x16(ka, qb, a);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int s = 32 * ms + 8 * (e >> 2) + 4 * hh + (e & 3);
        const float Gs = *(const __attribute__((address_space(3))) float*)(lds + kGsOff + 4 * s);
        a[e] = s <= t ? a[e] * __builtin_amdgcn_exp2f((Gt - Gs) * kLog2e) : 0.f;
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int e0 = 8 * half;
        const bf16x8 pb = to_bf16x8(a[e0], a[e0 + 1], a[e0 + 2], a[e0 + 3], a[e0 + 4], a[e0 + 5],
                                    a[e0 + 6], a[e0 + 7]);
        o = mfma32x32x16(vt[2 * ms + half], pb, o);
      }
    }
    // ---- store the chunk's outputs: lane holds O^T[d][t], d = 32 md + 8 (e >> 2) + 4 hh + (e & 3)
    if (c0 + t < n) {
      uint16_t* orow = out + (int64_t)(t_begin + c0 + t) * hstride + (int64_t)h * kLaDim + 64 * vs + 32 * md + 4 * hh;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const uint32_t lo = float_to_bf16_bits(o[4 * qd] * scale) | (float_to_bf16_bits(o[4 * qd + 1] * scale) << 16);
        const uint32_t hi = float_to_bf16_bits(o[4 * qd + 2] * scale) | (float_to_bf16_bits(o[4 * qd + 3] * scale) << 16);
        *reinterpret_cast<u32x2*>(orow + 8 * qd) = u32x2{lo, hi};
      }
    }
    // ---- S'^T = exp(G_last) S^T + V^T K~, for the wave's two i tiles
    const float el = __expf(Glast);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 32 * (2 * np + u) + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) st[u][e] *= el;
#pragma unroll
      for (int stp = 0; stp < 4; ++stp) {
        const u32x2 lo = *(const __attribute__((address_space(3))) u32x2*)(lds + kKtOff + unit8(i, 4 * stp + hh));
        const u32x2 hi = *(const __attribute__((address_space(3))) u32x2*)(lds + kKtOff + unit8(i, 4 * stp + 2 + hh));
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        st[u] = mfma32x32x16(vt[stp], __builtin_bit_cast(bf16x8, w), st[u]);
      }
    }
    __syncthreads();  // every LDS read of this chunk is done before the next chunk is staged
  }

  // ---- the final state half back to the slot
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = 32 * (2 * np + u) + l32;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const f32x4v x = {st[u][4 * qd], st[u][4 * qd + 1], st[u][4 * qd + 2], st[u][4 * qd + 3]};
      *reinterpret_cast<f32x4v*>(sbase + i * kLaDim + 32 * md + 8 * qd + 4 * hh) = x;
    }
  }
}


// ---------------------------------------------------------------- chunk-parallel prefill
//
// The sequential kernel walks a request's chunks in order, so B = 1 keeps 32 workgroups busy.
// With a workspace the same arithmetic runs in three launches over (request, chunk) pairs:
//   1. every chunk's own state contribution dS^T = V^T K~ (fp32) and its decay sum G_last;
//   2. a scan per (request, head, 32 d_v columns): S_before(c) written as bf16 S^T, then
//      S <- exp(G_last(c)) S + dS(c); the final state goes back to the slot;
//   3. every chunk's outputs, O^T = exp(G) S_before^T Q^T + V^T P^T.
// Workspace: dS^T [B][maxc][H][128 d][128 i] fp32, S_before^T [B][maxc][H][128 d][128 i] bf16,
// G_last [B][maxc][H] fp32.

// Stage a chunk's K rows (row-major, swizzled) / K~^T / V^T half and return G for lane t.
struct ChunkIn {
  u32x4 rq[4], rk[4], rv[2];
  float rg;
};

__device__ __forceinline__ void load_chunk(ChunkIn& in, const uint16_t* q, const uint16_t* k,
                                           const uint16_t* v, const float* g, int t_begin, int n,
                                           int c0, int h, int H, int vs, bool want_q) {
  const int tid = threadIdx.x, lane = tid & 63, srow = tid >> 2;
  const int t = c0 + srow;
  const bool ok = t < n;
  const int64_t hstride = (int64_t)H * kLaDim;
  const int64_t base = (int64_t)(t_begin + t) * hstride + (int64_t)h * kLaDim;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ch = 4 * (tid & 3) + c;
    in.rq[c] = (ok && want_q) ? *reinterpret_cast<const u32x4*>(q + base + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
    in.rk[c] = ok ? *reinterpret_cast<const u32x4*>(k + base + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ch = 2 * (tid & 3) + c;
    in.rv[c] = ok ? *reinterpret_cast<const u32x4*>(v + base + 64 * vs + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
  }
  const int tg = c0 + lane;
  in.rg = tg < n ? g[(int64_t)(t_begin + tg) * H + h] : 0.f;
}

// Writes V^T (always), K~^T (with_kt) and Qs/Ks (with_qk) of the staged chunk into LDS.
__device__ __forceinline__ void stage_chunk(const ChunkIn& in, lds_char_t* lds, float G, float Glast,
                                            bool with_kt, bool with_qk) {
  const int tid = threadIdx.x, srow = tid >> 2;
  if (with_qk) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = 4 * (tid & 3) + c;
      *(__attribute__((address_space(3))) u32x4*)(lds + kQsOff + chunk16(srow, ch)) = in.rq[c];
      *(__attribute__((address_space(3))) u32x4*)(lds + kKsOff + chunk16(srow, ch)) = in.rk[c];
    }
  }
  if (with_kt) {
    const float ws = __expf(Glast - __shfl(G, srow, 64));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = 4 * (tid & 3) + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (in.rk[c][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const int i = 8 * ch + e;
        *(__attribute__((address_space(3))) uint16_t*)(lds + kKtOff + unit8(i, srow >> 2) + 2 * (srow & 3)) =
            (uint16_t)float_to_bf16_bits(bf16_bits_to_float(bits) * ws);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ch = 2 * (tid & 3) + c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * ch + e;
      *(__attribute__((address_space(3))) uint16_t*)(lds + kVtOff + unit8(d, srow >> 2) + 2 * (srow & 3)) =
          (uint16_t)((in.rv[c][e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    }
  }
}

// V^T fragments (A operands) of d tile md, s = 16 stp + {4hh..4hh+3, 8+4hh..8+4hh+3}
__device__ __forceinline__ void read_vt_frags(const lds_char_t* lds, int md, bf16x8 (&vt)[4]) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int stp = 0; stp < 4; ++stp) {
    const int r = 32 * md + l32;
    const u32x2 lo = *(const __attribute__((address_space(3))) u32x2*)(lds + kVtOff + unit8(r, 4 * stp + hh));
    const u32x2 hi = *(const __attribute__((address_space(3))) u32x2*)(lds + kVtOff + unit8(r, 4 * stp + 2 + hh));
    const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
    vt[stp] = __builtin_bit_cast(bf16x8, w);
  }
}

__global__ __launch_bounds__(kLaThreads) void la_chunk_state_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ g,
    const int32_t* __restrict__ cu, int H, int maxc, float* __restrict__ ds, float* __restrict__ glast) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kStateLds];
  lds_char_t* lds = (lds_char_t*)lds_raw;
  // halves of a (request, chunk, head) as in la_prefill_kernel: same XCD, one L2 for q and k
  const int half_grid = gridDim.x >> 1;
  const int vs = blockIdx.x >= half_grid;
  const int rest = blockIdx.x - vs * half_grid;
  const int h = rest % H;
  const int bc = rest / H;  // b * maxc + c
  const int b = bc / maxc, c = bc - b * maxc;
  const int t_begin = cu[b], n = cu[b + 1] - t_begin;
  const int c0 = c * kChunk;
  if (c0 >= n) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int md = wave & 1, np = wave >> 1;
  ChunkIn in;
  load_chunk(in, k, k, v, g, t_begin, n, c0, h, H, vs, false);
  const float G = wave_inclusive_sum(in.rg);
  const float Glast = __shfl(G, 63, 64);
  stage_chunk(in, lds, G, Glast, true, false);
  __syncthreads();
  bf16x8 vt[4];
  read_vt_frags(lds, md, vt);
  float* out = ds + ((int64_t)bc * H + h) * (kLaDim * kLaDim);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = 32 * (2 * np + u) + l32;
    f32x16 acc = {};
#pragma unroll
    for (int stp = 0; stp < 4; ++stp) {
      const u32x2 lo = *(const __attribute__((address_space(3))) u32x2*)(lds + kKtOff + unit8(i, 4 * stp + hh));
      const u32x2 hi = *(const __attribute__((address_space(3))) u32x2*)(lds + kKtOff + unit8(i, 4 * stp + 2 + hh));
      const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
      acc = mfma32x32x16(vt[stp], __builtin_bit_cast(bf16x8, w), acc);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int d = 64 * vs + 32 * md + 8 * (e >> 2) + 4 * hh + (e & 3);
      out[d * kLaDim + i] = acc[e];
    }
  }
  if (vs == 0 && tid == 0) glast[(int64_t)bc * H + h] = Glast;
}

// One workgroup per (request, head, 8 d_v columns); thread: column d = 8 db + (tid >> 5), rows
// i = 4 (tid & 31) .. + 3 of S^T. The chain S <- exp(G_last) S + dS is one fma per chunk, so the
// loop is bounded by the loads: the next kScanDepth chunks' dS and G_last are always in flight.
constexpr int kScanCols = 8;
constexpr int kScanDepth = 8;

__global__ __launch_bounds__(kLaThreads) void la_scan_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, int H, int maxc,
    int initial_state, float* __restrict__ pool, int64_t pool_slots, const float* __restrict__ ds,
    const float* __restrict__ glast, uint16_t* __restrict__ sb) {
  constexpr int kGroups = kLaDim / kScanCols;
  const int db = blockIdx.x % kGroups;
  const int bh = blockIdx.x / kGroups;
  const int b = bh / H, h = bh - b * H;
  const int64_t slot = slots[b];
  if (slot < 0 || slot >= pool_slots) return;
  const int n = cu[b + 1] - cu[b];
  // chunks beyond the workspace's maxc (a max_seqlen below a request's length) are not read
  const int nch = min((n + kChunk - 1) / kChunk, maxc);
  const int tid = threadIdx.x, i4 = tid & 31;
  const int d = kScanCols * db + (tid >> 5);
  float* sp = pool + (slot * H + h) * (int64_t)(kLaDim * kLaDim);
  f32x4v S;
#pragma unroll
  for (int e = 0; e < 4; ++e) S[e] = initial_state ? sp[(4 * i4 + e) * kLaDim + d] : 0.f;
  const int64_t blk0 = (int64_t)b * maxc * H + h;  // block of chunk c: blk0 + c * H
  const float* dsrc = ds + blk0 * (kLaDim * kLaDim) + d * kLaDim + 4 * i4;
  const int64_t cstride = (int64_t)H * kLaDim * kLaDim;
  f32x4v ring[kScanDepth];
  float gring[kScanDepth];
#pragma unroll
  for (int j = 0; j < kScanDepth; ++j) {
    if (j < nch) {
      ring[j] = *reinterpret_cast<const f32x4v*>(dsrc + j * cstride);
      gring[j] = glast[blk0 + (int64_t)j * H];
    }
  }
  uint16_t* dst = sb + blk0 * (kLaDim * kLaDim) + d * kLaDim + 4 * i4;
  for (int cb = 0; cb < nch; cb += kScanDepth) {
#pragma unroll
    for (int j = 0; j < kScanDepth; ++j) {
      const int c = cb + j;
      if (c < nch) {
        const uint32_t lo = float_to_bf16_bits(S[0]) | (float_to_bf16_bits(S[1]) << 16);
        const uint32_t hi = float_to_bf16_bits(S[2]) | (float_to_bf16_bits(S[3]) << 16);
        *reinterpret_cast<u32x2*>(dst + c * cstride) = u32x2{lo, hi};
        S = S * __expf(gring[j]) + ring[j];
        if (c + kScanDepth < nch) {
          ring[j] = *reinterpret_cast<const f32x4v*>(dsrc + (c + kScanDepth) * cstride);
          gring[j] = glast[blk0 + (int64_t)(c + kScanDepth) * H];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) sp[(4 * i4 + e) * kLaDim + d] = S[e];
}

__global__ __launch_bounds__(kLaThreads) void la_chunk_out_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const int32_t* __restrict__ cu, const int32_t* __restrict__ slots,
    int H, int maxc, float scale, int initial_state, int64_t pool_slots,
    const uint16_t* __restrict__ sb, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kOutLds];
  lds_char_t* lds = (lds_char_t*)lds_raw;
  // halves of a (request, chunk, head) as in la_prefill_kernel: same XCD, one L2 for q and k
  const int half_grid = gridDim.x >> 1;
  const int vs = blockIdx.x >= half_grid;
  const int rest = blockIdx.x - vs * half_grid;
  const int h = rest % H;
  const int bc = rest / H;
  const int b = bc / maxc, c = bc - b * maxc;
  const int64_t slot = slots[b];
  if (slot < 0 || slot >= pool_slots) return;
  const int t_begin = cu[b], n = cu[b + 1] - t_begin;
  const int c0 = c * kChunk;
  if (c0 >= n) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int md = wave & 1, nt = wave >> 1;
  ChunkIn in;
  load_chunk(in, q, k, v, g, t_begin, n, c0, h, H, vs, true);
  const float G = wave_inclusive_sum(in.rg);
  stage_chunk(in, lds, G, 0.f, false, true);
  if (wave == 0) *(__attribute__((address_space(3))) float*)(lds + kGsOff + 4 * lane) = G;
  // S_before^T fragments straight from the workspace (A operands: row d, i = 16 stp + 8 hh ..)
  const bool has_state = c > 0 || initial_state;
  bf16x8 sa[8];
  if (has_state) {
    const uint16_t* src = sb + ((int64_t)bc * H + h) * (kLaDim * kLaDim) +
                          (int64_t)(64 * vs + 32 * md + l32) * kLaDim + 8 * hh;
#pragma unroll
    for (int stp = 0; stp < 8; ++stp) sa[stp] = *reinterpret_cast<const bf16x8*>(src + 16 * stp);
  }
  __syncthreads();
  const int t = 32 * nt + l32;
  const float Gt = __shfl(G, t, 64);
  f32x16 o = {};
  if (has_state) {
#pragma unroll
    for (int stp = 0; stp < 8; ++stp)
      o = mfma32x32x16(sa[stp], lds_read16(lds + kQsOff + chunk16(t, 2 * stp + hh)), o);
    const float et = __expf(Gt);
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] *= et;
  }
  bf16x8 vt[4];
  read_vt_frags(lds, md, vt);
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    if (ms > nt) break;
    f32x16 a = {};
#pragma unroll
    for (int stp = 0; stp < 8; ++stp) {
      const bf16x8 ka = lds_read16(lds + kKsOff + chunk16(32 * ms + l32, 2 * stp + hh));
      const bf16x8 qb = lds_read16(lds + kQsOff + chunk16(t, 2 * stp + hh));
      a = mfma32x32x16(ka, qb, a);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int s = 32 * ms + 8 * (e >> 2) + 4 * hh + (e & 3);
      const float Gs = *(const __attribute__((address_space(3))) float*)(lds + kGsOff + 4 * s);
      a[e] = s <= t ? a[e] * __builtin_amdgcn_exp2f((Gt - Gs) * kLog2e) : 0.f;
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int e0 = 8 * half;
      const bf16x8 pb = to_bf16x8(a[e0], a[e0 + 1], a[e0 + 2], a[e0 + 3], a[e0 + 4], a[e0 + 5],
                                  a[e0 + 6], a[e0 + 7]);
      o = mfma32x32x16(vt[2 * ms + half], pb, o);
    }
  }
  if (c0 + t < n) {
    const int64_t hstride = (int64_t)H * kLaDim;
    uint16_t* orow = out + (int64_t)(t_begin + c0 + t) * hstride + (int64_t)h * kLaDim + 64 * vs + 32 * md + 4 * hh;
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const uint32_t lo = float_to_bf16_bits(o[4 * qd] * scale) | (float_to_bf16_bits(o[4 * qd + 1] * scale) << 16);
      const uint32_t hi = float_to_bf16_bits(o[4 * qd + 2] * scale) | (float_to_bf16_bits(o[4 * qd + 3] * scale) << 16);
      *reinterpret_cast<u32x2*>(orow + 8 * qd) = u32x2{lo, hi};
    }
  }
}

}  // namespace

hipError_t launch_linear_prefill(const void* q, const void* k, const void* v, const float* g,
                                 const int32_t* cu, const int32_t* slots, int batch, int heads,
                                 float scale, int initial_state, float* pool, int64_t pool_slots,
                                 void* out, hipStream_t stream) {
  const int64_t grid = (int64_t)batch * heads * 2;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(la_prefill_kernel, dim3((unsigned)grid), dim3(kLaThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, g, cu, slots, heads,
                     scale, initial_state, pool, pool_slots, (uint16_t*)out);
  return hipGetLastError();
}

// Workspace of the chunk-parallel prefill: dS^T (fp32), S_before^T (bf16), G_last, each part
// 256-byte aligned. Returns the byte size; fills the part offsets if `off` is not null.
size_t linear_prefill_ws(int64_t batch, int64_t maxc, int64_t heads, size_t* off) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t blocks = (size_t)(batch * maxc * heads);
  const size_t ds = 0, sb = al(ds + blocks * kLaDim * kLaDim * 4), gl = al(sb + blocks * kLaDim * kLaDim * 2);
  if (off) { off[0] = ds; off[1] = sb; off[2] = gl; }
  return al(gl + blocks * 4);
}

hipError_t launch_linear_prefill_parallel(const void* q, const void* k, const void* v, const float* g,
                                          const int32_t* cu, const int32_t* slots, int batch, int heads,
                                          int maxc, float scale, int initial_state, float* pool,
                                          int64_t pool_slots, void* out, void* ws, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  size_t off[3];
  linear_prefill_ws(batch, maxc, heads, off);
  char* w = (char*)ws;
  float* ds = (float*)(w + off[0]);
  uint16_t* sb = (uint16_t*)(w + off[1]);
  float* gl = (float*)(w + off[2]);
  const int64_t chunk_grid = (int64_t)batch * maxc * heads * 2;
  if (chunk_grid > 0) {
    hipLaunchKernelGGL(la_chunk_state_kernel, dim3((unsigned)chunk_grid), dim3(kLaThreads), 0, stream,
                       (const uint16_t*)k, (const uint16_t*)v, g, cu, heads, maxc, ds, gl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(la_scan_kernel, dim3((unsigned)((int64_t)batch * heads * (kLaDim / kScanCols))),
                     dim3(kLaThreads), 0,
                     stream, cu, slots, heads, maxc, initial_state, pool, pool_slots, ds, gl, sb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || chunk_grid == 0) return e;
  hipLaunchKernelGGL(la_chunk_out_kernel, dim3((unsigned)chunk_grid), dim3(kLaThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, g, cu, slots, heads, maxc,
                     scale, initial_state, pool_slots, sb, (uint16_t*)out);
  return hipGetLastError();
}

hipError_t launch_linear_decode(const void* q, const void* k, const void* v, const float* g,
                                const int32_t* slots, int batch, int heads, float scale, float* pool,
                                int64_t pool_slots, void* out, hipStream_t stream) {
  const int64_t grid = (int64_t)batch * heads;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(la_decode_kernel, dim3((unsigned)grid), dim3(kLaThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, g, slots, heads, scale,
                     pool, pool_slots, (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace segattn
