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
    const float* __restrict__ glast, uint16_t* __restrict__ sb, uint16_t* __restrict__ out) {
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
  if (n > maxc * kChunk) {
    // A request longer than max_seqlen, the host's bound that sized the workspace: its tokens
    // past the bound are not computed. They and the final state get NaN (this workgroup's
    // columns), so that the broken bound cannot pass unnoticed.
    for (int t = maxc * kChunk + i4; t < n; t += 32)
      out[((int64_t)cu[b] + t) * H * kLaDim + (int64_t)h * kLaDim + d] = 0x7FC0;  // bf16 NaN
#pragma unroll
    for (int e = 0; e < 4; ++e) S[e] = NAN;
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

// ------------------------------------------------------------ fused prefill (closed form)
//
// For requests of up to kFusedMaxLen tokens one launch computes the outputs and the final states
// from the closed form of the recurrence, with G_t = g_0 + ... + g_t the decay sum from the
// request's first token:
//   o_t = scale * ( exp(G_t) q_t S_0 + sum_{s <= t} (q_t . k_s) exp(G_t - G_s) v_s )
//   S_n = exp(G_{n-1}) S_0 + sum_s exp(G_{n-1} - G_s) k_s^T v_s
// The cost grows with the square of the length, as causal attention's does, where the chunked
// form's grows linearly; but no state is carried from chunk to chunk, so every term can be
// computed at once, without a scan and without a workspace. Both sums are split over the waves
// of a workgroup by key blocks, and since the terms simply add (no normalisation) the waves'
// partial sums are added through LDS at the end. Workgroups of 8 waves:
//   output workgroups, one per (64-query tile, request, head), heaviest tile first: wave w takes
//     the 32 queries 32 (w / 4) .. + 31 of the tile and the 32-key blocks w % 4, w % 4 + 4, ...;
//     the two waves with the same w % 4 share each block, copied once into LDS (K row-major and
//     V, read back transposed), one workgroup barrier per step;
//   state workgroups, four per (request, head), one per 64 x 64 quarter of the state: wave w
//     takes the 32-key blocks w, w + 8, ... on its own (no barrier in the key loop), K scaled by
//     its decay weight on the way into LDS.
// Each workgroup forms the decay sums it needs by a prefix sum over the request's g (at most
// kFusedMaxLen values) into LDS. With a stored initial state the state workgroups run in a second
// launch, after every output workgroup has read S_0 from the slot they overwrite.

constexpr int kFusedMaxLen = 4096;
constexpr int kFThreads = 256;                  // 4 waves
constexpr int kFQ = 64;                         // queries per output tile
constexpr int kNT = kFQ / 32;                   // 32-query halves of a tile
constexpr int kFKB = 32;                        // keys per block
constexpr int kFGOff = 131072;                  // key-block slots and the partial sums below
constexpr int kFLds = kFGOff + kFusedMaxLen * 4 + 16;  // then the decay sums and 4 wave totals

typedef __attribute__((address_space(3))) float lds_f32_t;
typedef __attribute__((address_space(3))) f32x4v lds_f32x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;

// Blocks of 256-byte rows (128 bf16): K with 16-byte chunk c of row r at c ^ (r % 16), read 16
// bytes per lane along rows; V and S_0 with chunk c at c ^ 4 (r % 4), read transposed.
__device__ __forceinline__ int ksw(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }
__device__ __forceinline__ int vsw(int r, int c) { return r * 256 + ((c ^ ((r & 3) << 2)) << 4); }
// Blocks of 128-byte rows (64 bf16), read transposed: chunk c of row r at c ^ 4 ((r / 2) % 2).
__device__ __forceinline__ int hsw(int r, int c) { return r * 128 + ((c ^ (((r >> 1) & 1) << 2)) << 4); }

// This lane's address for the transposing read of rows r0 + rstride * (lane / 32) + jj (jj =
// 0..3) and columns 32 tile + lane % 32 of a vsw (wide) or hsw (half-width) block: after the read
// the lane holds those four values of its column. Each group of 16 lanes reads 4 rows x 16
// columns; over the wave the 64 pieces of 8 bytes fall on every 8-byte bank pair exactly twice.
template <bool kHalf>
__device__ __forceinline__ int tr_addr(int r0, int rstride, int tile) {
  const int l = threadIdx.x & 63;
  const int grp = l >> 4, jj = (l >> 2) & 3, u = l & 3;
  const int r = r0 + rstride * (grp >> 1) + jj;
  const int c = 4 * tile + 2 * (grp & 1) + (u >> 1);
  return (kHalf ? hsw(r, c) : vsw(r, c)) + 8 * (u & 1);
}

// Two transposing reads, off_hi bytes apart, as one 8-value MFMA operand.
__device__ __forceinline__ bf16x8 tr_pair(const lds_char_t* p, int off_hi) {
  const bf16x4 lo = lds_read_tr16(p), hi = lds_read_tr16(p + off_hi);
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Gl[t] = log2(e) (g_0 + ... + g_t) for the request's tokens t < cnt of head h (cnt <=
// kFusedMaxLen), in two parts so that the loads can be issued first and the scan done later:
// decay_load gives each thread the running sums of its (up to 16) consecutive tokens, decay_scan
// adds the totals of the threads before it and writes Gl; every thread of the workgroup takes
// part, and decay_scan ends with a barrier.
struct DecayPart {
  float vals[16];
};
__device__ __forceinline__ void decay_load(const float* __restrict__ g, int t_begin, int H, int h, int cnt,
                                           DecayPart& d) {
  const int tid = threadIdx.x;
  const int per = (cnt + kFThreads - 1) / kFThreads;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = tid * per + i;
    d.vals[i] = (i < per && t < cnt) ? g[(int64_t)(t_begin + t) * H + h] : 0.f;
  }
}
__device__ __forceinline__ void decay_scan(int cnt, DecayPart& d, lds_f32_t* Gl, lds_f32_t* wsum) {
  const int tid = threadIdx.x;
  const int per = (cnt + kFThreads - 1) / kFThreads;
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    run += d.vals[i];
    d.vals[i] = run;
  }
  const float incl = wave_inclusive_sum(run);
  if ((tid & 63) == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  float off = incl - run;
  for (int w = 0; w < (tid >> 6); ++w) off += wsum[w];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = tid * per + i;
    if (i < per && t < cnt) Gl[t] = (d.vals[i] + off) * kLog2e;
  }
  __syncthreads();
}

__device__ __forceinline__ void sched_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void fused_outputs(
    lds_char_t* lds, lds_f32_t* Gl, lds_f32_t* wsum, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ g,
    int t_begin, int n, int H, int h, int j, int n_tiles, int64_t slot, float scale,
    int initial_state, const float* __restrict__ pool, uint16_t* __restrict__ out) {
  const int q0 = j * kFQ;
  if (q0 >= n) return;  // the whole workgroup leaves together
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t hstride = (int64_t)H * kLaDim;
  const int cnt = min(n, q0 + kFQ);  // keys the tile sees; also one past its last query
  DecayPart dec;
  decay_load(g, t_begin, H, h, cnt, dec);  // first: the decay sums are on the longest path
  if (j == n_tiles - 1 && n > n_tiles * kFQ) {
    // tokens past the covered length (a request longer than max_seqlen): NaN
    const int first = n_tiles * kFQ;
    for (int x = tid; x < (n - first) * 64; x += kFThreads)
      *reinterpret_cast<uint32_t*>(out + (int64_t)(t_begin + first + x / 64) * hstride + h * kLaDim + 2 * (x % 64)) =
          0x7FC07FC0u;
  }

  // Q^T (B operands of P^T = K Q^T) of the tile's two 32-query halves: lane holds
  // q_t[16 step + 8 hh + 0..7] of query t = q0 + 32 nt + l32
  bf16x8 qf[kNT][8];
  int tq[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    tq[nt] = min(q0 + 32 * nt + l32, n - 1);
    const uint16_t* qrow = q + (int64_t)(t_begin + tq[nt]) * hstride + h * kLaDim + 8 * hh;
#pragma unroll
    for (int step = 0; step < 8; ++step) qf[nt][step] = *reinterpret_cast<const bf16x8*>(qrow + 16 * step);
  }

  // ---- key blocks: wave w takes blocks w, w + 4, ... of the tile's keys, in two slots of its
  // own (16 KiB each: K at +0, V at +8 KiB); no workgroup barrier in the loop
  const int nkb = (cnt + kFKB - 1) / kFKB;
  const int mine = nkb > wave ? (nkb - 1 - wave) / 4 + 1 : 0;
  lds_char_t* slot0 = lds + wave * 32768;
  lds_char_t* slot1 = slot0 + 16384;
  const int cr = lane >> 4;  // copy instruction c fills rows 4 c + cr, chunk position lane % 16
  const uint32_t rowb = (uint32_t)hstride * 2;
  uint32_t kco[8];  // K: chunk (lane % 16) ^ (row % 16) of the row; V: chunk (lane % 16) ^ 4 cr
#pragma unroll
  for (int c = 0; c < 8; ++c) kco[c] = (uint32_t)((lane & 15) ^ ((4 * c + cr) & 15)) << 4;
  const uint32_t vco = (uint32_t)((lane & 15) ^ (cr << 2)) << 4;
  // Block kb's copies (rows 4 c + cr of K and of V, c = 0..7), from buffers based at the
  // block's first row; rows past the tile's keys re-read its last key. copy_one(x) issues copy
  // x (0..15) of the 16, so that they can be spread between the MFMAs.
  struct Copies {
    __amdgpu_buffer_rsrc_t kr, vr;
    int lim;
    lds_char_t* dst;
  };
  auto copies_of = [&](int kb, lds_char_t* dst) __attribute__((always_inline)) {
    const int s0 = kb * kFKB;
    const int64_t base = (int64_t)(t_begin + s0) * hstride + h * kLaDim;
    return Copies{block_rsrc(k + base), block_rsrc(v + base), cnt - 1 - s0, dst};
  };
  auto copy_one = [&](const Copies& cp, int x) __attribute__((always_inline)) {
    const int c = x >> 1;
    const uint32_t ro = (uint32_t)min(4 * c + cr, cp.lim) * rowb;
    if ((x & 1) == 0) copy16_buf(cp.kr, (lds_void_t*)(cp.dst + 1024 * c), ro + kco[c]);
    else copy16_buf(cp.vr, (lds_void_t*)(cp.dst + 8192 + 1024 * c), ro + vco);
  };

  f32x16 o[4][kNT];
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) o[md][nt] = f32x16{};

  if (initial_state) {
    // exp(G_t) q_t S_0 for d_v tile `wave`, both query halves: S_0 as bf16 [128 i][128 d] (vsw)
    // in the first 32 KiB, before any key block is copied there
    const float* s0 = pool + (slot * H + h) * (int64_t)(kLaDim * kLaDim);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int qd = tid + kFThreads * c;
      const int i = qd >> 4, ch = qd & 15;
      const f32x4v a = *reinterpret_cast<const f32x4v*>(s0 + i * kLaDim + 8 * ch);
      const f32x4v b = *reinterpret_cast<const f32x4v*>(s0 + i * kLaDim + 8 * ch + 4);
      *(lds_bf16x8_t*)(lds + vsw(i, ch)) = to_bf16x8(a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]);
    }
    __syncthreads();
    // A = S_0^T rows d, k = i in the order of qf: rows 16 st + 8 hh + jj, then + 4
    const int a0 = tr_addr<false>(0, 8, wave);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 a = tr_pair(lds + a0 + 4096 * st, 1024);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int md = 0; md < 4; ++md)
          if (md == wave) o[md][nt] = mfma32x32x16(a, qf[nt][st], o[md][nt]);
    }
    __syncthreads();  // the key blocks below overwrite S_0; the exp(G_t) factor comes with G
  }
  if (mine > 0) {  // in flight during the decay sums
    const Copies cp = copies_of(wave, slot0);
#pragma unroll
    for (int x = 0; x < 16; ++x) copy_one(cp, x);
  }
  decay_scan(cnt, dec, Gl, wsum);
  float Gt[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) Gt[nt] = Gl[tq[nt]];
  if (initial_state) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const float et = fast_exp2(Gt[nt]);
#pragma unroll
      for (int md = 0; md < 4; ++md)
        if (md == wave) o[md][nt] *= et;
    }
  }

  int kofs[8];
#pragma unroll
  for (int step = 0; step < 8; ++step) kofs[step] = ksw(l32, 2 * step + hh);
  int vaddr[4];
#pragma unroll
  for (int md = 0; md < 4; ++md) vaddr[md] = 8192 + tr_addr<false>(0, 4, md);

  // block kb from src; the next block's 16 copies (if nxt_kb >= 0) go out one after each MFMA of
  // P^T = K Q^T, so that no copy instruction waits long for the memory pipeline (the wave issues
  // in order) and they have the rest of the block to land
  auto compute = [&](int kb, const lds_char_t* src, int nxt_kb, lds_char_t* nxt) __attribute__((always_inline)) {
    bf16x8 kf[8];
#pragma unroll
    for (int step = 0; step < 8; ++step) kf[step] = lds_read16(src + kofs[step]);
    const int s0 = kb * kFKB;
    f32x4v gs[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) gs[g4] = *(const lds_f32x4_t*)(Gl + s0 + 8 * g4 + 4 * hh);
    f32x16 p[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) p[nt] = f32x16{};
    const Copies cp = copies_of(nxt_kb < 0 ? kb : nxt_kb, nxt);
#pragma unroll
    for (int step = 0; step < 8; ++step)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        p[nt] = mfma32x32x16(kf[step], qf[nt][step], p[nt]);
        if (nxt_kb >= 0)
#pragma unroll
          for (int x = 0; x < 2 / kNT; ++x) copy_one(cp, (step * kNT + nt) * (2 / kNT) + x);
      }
    bf16x8 vf[4][2];
#pragma unroll
    for (int md = 0; md < 4; ++md) {
      vf[md][0] = tr_pair(src + vaddr[md], 2048);
      vf[md][1] = tr_pair(src + vaddr[md] + 4096, 2048);
    }
    // P^T[s][t] *= exp(G_t - G_s), s = s0 + 8 (e / 4) + 4 hh + e % 4; keys after t hidden
    bf16x8 pb[kNT][2];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int tw = q0 + 32 * nt;  // first query of the half
      const bool diag = s0 + kFKB - 1 > tw;
      const int t = tw + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = p[nt][e] * fast_exp2(Gt[nt] - gs[e >> 2][e & 3]);
        p[nt][e] = (!diag || s0 + 8 * (e >> 2) + 4 * hh + (e & 3) <= t) ? pe : 0.f;
      }
      pb[nt][0] = to_bf16x8(p[nt][0], p[nt][1], p[nt][2], p[nt][3], p[nt][4], p[nt][5], p[nt][6], p[nt][7]);
      pb[nt][1] = to_bf16x8(p[nt][8], p[nt][9], p[nt][10], p[nt][11], p[nt][12], p[nt][13], p[nt][14], p[nt][15]);
    }
#pragma unroll
    for (int stp = 0; stp < 2; ++stp)
#pragma unroll
      for (int md = 0; md < 4; ++md)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) o[md][nt] = mfma32x32x16(vf[md][stp], pb[nt][stp], o[md][nt]);
  };

  // Double buffered per wave: block i + 1's copies are issued during block i's MFMAs, and block
  // i + 1 is waited for (all copies done) just before it is used.
  for (int i = 0; i < mine; ++i) {
    sched_fence();
    wait_vmem();
    sched_fence();
    const bool more = i + 1 < mine;
    compute(wave + 4 * i, (i & 1) ? slot1 : slot0, more ? wave + 4 * (i + 1) : -1, (i & 1) ? slot0 : slot1);
  }

  // ---- add the 4 waves' partials through LDS; wave w finishes d_v tile w of all 64 queries
  __syncthreads();
  lds_f32x4_t* red = (lds_f32x4_t*)lds;  // [wave][md][nt][e / 4][lane]: 128 KiB
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        red[(((wave * 4 + md) * kNT + nt) * 4 + e4) * 64 + lane] =
            f32x4v{o[md][nt][4 * e4], o[md][nt][4 * e4 + 1], o[md][nt][4 * e4 + 2], o[md][nt][4 * e4 + 3]};
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int t = q0 + 32 * nt + l32;
    if (t >= n) continue;
    uint16_t* orow = out + (int64_t)(t_begin + t) * hstride + h * kLaDim + 32 * wave + 4 * hh;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      f32x4v x = red[(((0 * 4 + wave) * kNT + nt) * 4 + e4) * 64 + lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) x += red[(((w * 4 + wave) * kNT + nt) * 4 + e4) * 64 + lane];
      const uint32_t lo = float_to_bf16_bits(x[0] * scale) | (float_to_bf16_bits(x[1] * scale) << 16);
      const uint32_t hi = float_to_bf16_bits(x[2] * scale) | (float_to_bf16_bits(x[3] * scale) << 16);
      *reinterpret_cast<u32x2*>(orow + 8 * e4) = u32x2{lo, hi};
    }
  }
}

// One 64 x 64 quarter of a request's final state: d_v columns 64 dh .., d_k rows 64 ih ...
__device__ __forceinline__ void fused_state(
    lds_char_t* lds, lds_f32_t* Gl, lds_f32_t* wsum, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g, int t_begin, int n, int H, int h,
    int part, int max_len, int64_t slot, int initial_state, float* __restrict__ pool) {
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dh = part >> 1, ih = part & 1;
  const int64_t hstride = (int64_t)H * kLaDim;
  float* st = pool + (slot * H + h) * (int64_t)(kLaDim * kLaDim);
  if (n > max_len) {  // a request longer than max_seqlen: its state is NaN
    for (int x = tid; x < 64 * 64; x += kFThreads)
      st[(64 * ih + (x >> 6)) * kLaDim + 64 * dh + (x & 63)] = __builtin_nanf("");
    return;
  }

  // wave w: blocks w, w + 4, ... (block i of the wave: w + 4 i); V copies two blocks ahead into
  // a ring of 3 slots of 4 KiB, K rows two blocks ahead in registers, scaled into one K~ slot
  // (4 KiB) just before use: 16 KiB per wave
  DecayPart dec;
  decay_load(g, t_begin, H, h, n, dec);  // first: the decay sums are on the longest path
  const int nkb = (n + kFKB - 1) / kFKB;
  const int mine = nkb > wave ? (nkb - 1 - wave) / 4 + 1 : 0;
  lds_char_t* wbase = lds + wave * 16384;
  lds_char_t* ktl = wbase + 12288;
  // K rows (64 d_k values, 128 bytes): copy c takes chunk (lane + 64 c) of the block, row
  // (lane + 64 c) / 8; V rows: copy instruction c fills rows 8 c + lane / 8, position lane % 8.
  u32x4 kreg[2][4];
  const uint32_t rowb = (uint32_t)hstride * 2;
  auto load_k = [&](int kb, u32x4 (&kr)[4]) __attribute__((always_inline)) {
    const int lim = n - 1 - kb * kFKB;
    const auto rs = block_rsrc(k + (int64_t)(t_begin + kb * kFKB) * hstride + h * kLaDim + 64 * ih);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qd = lane + 64 * c;
      kr[c] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)min(qd >> 3, lim) * rowb + 16 * (qd & 7), 0, 0);
    }
  };
  auto dma_v = [&](int kb, lds_char_t* dst) __attribute__((always_inline)) {
    const int lim = n - 1 - kb * kFKB;
    const auto rs = block_rsrc(v + (int64_t)(t_begin + kb * kFKB) * hstride + h * kLaDim + 64 * dh);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = 8 * c + (lane >> 3);
      const int ch = (lane & 7) ^ (((r >> 1) & 1) << 2);
      copy16_buf(rs, (lds_void_t*)(dst + 1024 * c), (uint32_t)min(r, lim) * rowb + 16 * ch);
    }
  };
  const int blk0 = wave, blk1 = wave + 4;
  if (mine > 0) {
    load_k(blk0, kreg[0]);
    dma_v(blk0, wbase);
  }
  if (mine > 1) {
    load_k(blk1, kreg[1]);
    dma_v(blk1, wbase + 4096);
  }
  decay_scan(n, dec, Gl, wsum);
  const float Gn = n > 0 ? Gl[n - 1] : 0.f;

  // S^T partial [dt][it]: d = 64 dh + 32 dt + 8 (e / 4) + 4 hh + e % 4, i = 64 ih + 32 it + l32
  f32x16 acc[2][2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int it = 0; it < 2; ++it) acc[dt][it] = f32x16{};
  int va[2], ka[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    va[x] = tr_addr<true>(0, 4, x);
    ka[x] = tr_addr<true>(0, 4, x);
  }
  // K~[s] = exp(G_{n-1} - G_s) k_s, zero past the request (where V re-reads the last row)
  auto store_k = [&](int kb, const u32x4 (&kr)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int qd = lane + 64 * c;
      const int r = qd >> 3, s = kb * kFKB + r;
      const float w = s < n ? fast_exp2(Gn - Gl[s]) : 0.f;
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_bits_to_float(kr[c][e] & 0xFFFFu) * w;
        x[2 * e + 1] = bf16_bits_to_float(kr[c][e] >> 16) * w;
      }
      *(lds_bf16x8_t*)(ktl + hsw(r, qd & 7)) = to_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    }
  };
  auto compute = [&](const lds_char_t* vsrc) __attribute__((always_inline)) {
#pragma unroll
    for (int stp = 0; stp < 2; ++stp) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        a[x] = tr_pair(vsrc + va[x] + 2048 * stp, 1024);
        b[x] = tr_pair(ktl + ka[x] + 2048 * stp, 1024);
      }
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int it = 0; it < 2; ++it) acc[dt][it] = mfma32x32x16(a[dt], b[it], acc[dt][it]);
    }
  };
  // step i: K~ of block i from registers, block i + 2 requested (K into the registers just
  // freed, V into the ring slot block i - 1 used), then block i's V waited for: 8 or 16
  // operations of later blocks may still be in flight
  auto step = [&](int i, u32x4 (&kr)[4]) __attribute__((always_inline)) {
    const int kb = wave + 4 * i;
    store_k(kb, kr);
    const bool more2 = i + 2 < mine;
    if (more2) {
      load_k(kb + 8, kr);
      dma_v(kb + 8, wbase + 4096 * ((i + 2) % 3));
    }
    sched_fence();
    if (more2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));
    else if (i + 1 < mine) __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));
    else wait_vmem();
    sched_fence();
    compute(wbase + 4096 * (i % 3));
  };
  for (int i = 0; i < mine; i += 2) {
    step(i, kreg[0]);
    if (i + 1 < mine) step(i + 1, kreg[1]);
  }

  // ---- add the 4 waves' partials through LDS; wave w finishes tile (w / 2, w % 2)
  __syncthreads();
  lds_f32x4_t* red = (lds_f32x4_t*)lds;  // [wave][tile][e / 4][lane]: 64 KiB
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        red[((wave * 4 + dt * 2 + it) * 4 + e4) * 64 + lane] =
            f32x4v{acc[dt][it][4 * e4], acc[dt][it][4 * e4 + 1], acc[dt][it][4 * e4 + 2], acc[dt][it][4 * e4 + 3]};
  __syncthreads();
  {
    const int dt = wave >> 1, it = wave & 1;
    const int i = 64 * ih + 32 * it + l32;
    const float en = fast_exp2(Gn);
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int d = 64 * dh + 32 * dt + 8 * e4 + 4 * hh;
      f32x4v x = {0.f, 0.f, 0.f, 0.f};
      if (initial_state) x = *reinterpret_cast<const f32x4v*>(st + i * kLaDim + d) * en;
#pragma unroll
      for (int w = 0; w < 4; ++w) x += red[((w * 4 + wave) * 4 + e4) * 64 + lane];
      *reinterpret_cast<f32x4v*>(st + i * kLaDim + d) = x;
    }
  }
}

// roles: 1 = output workgroups, 2 = state workgroups (placed first in the grid), 3 = both.
__global__ __launch_bounds__(kFThreads) void la_fused_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const int32_t* __restrict__ cu, const int32_t* __restrict__ slots,
    int batch, int H, int max_len, int n_tiles, int roles, float scale, int initial_state,
    float* __restrict__ pool, int64_t pool_slots, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kFLds];
  lds_char_t* lds = (lds_char_t*)lds_raw;
  lds_f32_t* Gl = (lds_f32_t*)(lds + kFGOff);
  lds_f32_t* wsum = Gl + kFusedMaxLen;  // the 4 wave totals of the prefix sum
  // Every pointer argument in scalar registers before the first table read, so that the
  // kernel-argument loads share one round trip instead of following the tables one by one.
  asm volatile("" ::"s"(q), "s"(k), "s"(v), "s"(g), "s"(cu), "s"(slots), "s"(pool), "s"(out));
  // workgroup order: the state workgroups (quarter-major), then output tiles heaviest first,
  // (request, head) fastest throughout, so that with 8 | H every workgroup of head h runs on XCD
  // h % 8 and shares its L2
  const int bh_count = batch * H;
  const int n_state = (roles & 2) ? 4 * bh_count : 0;
  const int id = blockIdx.x;
  const bool state_role = id < n_state;
  const int bh = state_role ? id % bh_count : (id - n_state) % bh_count;
  const int b = bh / H, h = bh - b * H;
  // The request's slot and token range in one vector load (lanes 0-2), then broadcast: one
  // round trip, where scalar loads would wait for the slot before reading cu.
  int tv = 0;
  {
    const int tl = threadIdx.x & 63;
    if (tl < 3) tv = tl == 0 ? slots[b] : cu[b + tl - 1];
  }
  const int64_t slot = __builtin_amdgcn_readlane(tv, 0);
  const int t_begin = __builtin_amdgcn_readlane(tv, 1), t_end = __builtin_amdgcn_readlane(tv, 2);
  if (slot < 0 || slot >= pool_slots) return;  // the whole workgroup leaves together
  const int n = t_end - t_begin;
  if (state_role) {
    fused_state(lds, Gl, wsum, k, v, g, t_begin, n, H, h, id / bh_count, max_len, slot, initial_state, pool);
  } else {
    const int j = n_tiles - 1 - (id - n_state) / bh_count;
    fused_outputs(lds, Gl, wsum, q, k, v, g, t_begin, n, H, h, j, n_tiles, slot, scale, initial_state,
                  pool, out);
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
                     stream, cu, slots, heads, maxc, initial_state, pool, pool_slots, ds, gl, sb,
                     (uint16_t*)out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || chunk_grid == 0) return e;
  hipLaunchKernelGGL(la_chunk_out_kernel, dim3((unsigned)chunk_grid), dim3(kLaThreads), 0, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, g, cu, slots, heads, maxc,
                     scale, initial_state, pool_slots, sb, (uint16_t*)out);
  return hipGetLastError();
}

int linear_fused_max_len() { return kFusedMaxLen; }

hipError_t launch_linear_prefill_fused(const void* q, const void* k, const void* v, const float* g,
                                       const int32_t* cu, const int32_t* slots, int batch, int heads,
                                       int max_len, float scale, int initial_state, float* pool,
                                       int64_t pool_slots, void* out, hipStream_t stream) {
  const int n_tiles = (max_len + kFQ - 1) / kFQ;
  const int64_t bh = (int64_t)batch * heads;
  if (bh == 0) return hipSuccess;
  auto go = [&](int roles) {
    const int64_t grid = ((roles & 2) ? 4 * bh : 0) + ((roles & 1) ? bh * n_tiles : 0);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(la_fused_kernel, dim3((unsigned)grid), dim3(kFThreads), 0, stream, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, g, cu, slots, batch, heads, max_len, n_tiles,
                       roles, scale, initial_state, pool, pool_slots, (uint16_t*)out);
    return hipGetLastError();
  };
  if (!initial_state) return go(3);
  // the output workgroups read S_0 from the slots the state workgroups overwrite
  const hipError_t e = go(1);
  return e != hipSuccess ? e : go(2);
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
