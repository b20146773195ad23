// Shared device helpers for the gfx950 segment-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace segattn {

typedef __bf16 bf16_t;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr int kHeadDim = 128;
constexpr int kGroup = 8;  // query heads per kv head, packed into one tile

struct Segment {
  int32_t pool_offset;
  int32_t length;
};

// Walks a request's segment table forward. Keys are looked up in non-decreasing order, so the
// cursor only ever advances; zero-length segments are stepped over.
struct SegCursor {
  const Segment* segs;
  int idx, end;
  int start;  // logical key index of the current segment's first key
  int off, len;

  __device__ __forceinline__ void init(const Segment* s, int first, int last) {
    segs = s;
    idx = first;
    end = last;
    start = 0;
    fetch();
  }
  __device__ __forceinline__ void fetch() {
    if (idx < end) {
      i32x2 v = *reinterpret_cast<const i32x2*>(segs + idx);
      off = v[0];
      len = v[1];
    } else {
      off = 0;
      len = 0x7fffffff;
    }
  }
  // Pool slot of logical key j (j must lie inside the request's keys).
  __device__ __forceinline__ int64_t slot(int j) {
    while (j - start >= len) {
      start += len;
      ++idx;
      fetch();
    }
    return (int64_t)off + (j - start);
  }
};

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 bytes from global memory straight into LDS: lane L's bytes land at lds_base + 16 * L.
// lds_base must be the same for the whole wave.
__device__ __forceinline__ void copy16_to_lds(const void* g, lds_void_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, lds_base, 16, 0, 0);
}
// 4 bytes per lane: lane L's dword lands at lds_base + 4 * L.
__device__ __forceinline__ void copy4_to_lds(const void* g, lds_void_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, lds_base, 4, 0, 0);
}
// The same two copies marked non-temporal (the nt cache-policy bit), for data read exactly once
// in a stream. Measured on the decode read pattern (a kv head's 256-byte slices of consecutive
// pool rows): about 6.8 TB/s with the bit against 6.0 TB/s without.
__device__ __forceinline__ void copy16_to_lds_stream(const void* g, lds_void_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, lds_base, 16, 0, 2);
}
__device__ __forceinline__ void copy4_to_lds_stream(const void* g, lds_void_t* lds_base) {
  __builtin_amdgcn_global_load_lds(g, lds_base, 4, 0, 2);
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their "no wait" maxima). Issued through the
// builtin, not inline asm, so the compiler's own wait insertion knows every earlier vector
// memory operation, HBM->LDS copies included, has completed here.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(n) with expcnt and lgkmcnt at their no-wait maxima (gfx9 encoding: vmcnt
// bits 3:0 and 15:14).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// A block's pool rows as a raw buffer whose base is the block's first row (a scalar 64-bit add
// per block): every lane's row offset is then a 32-bit register added by the load itself, with
// no 64-bit address arithmetic on the vector ALU, and the LDS destination (M0) is scalar.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
// 16 bytes per lane from the buffer at byte offset voff into LDS: lane L's bytes land at
// lds_base + 16 * L.
__device__ __forceinline__ void copy16_buf(__amdgpu_buffer_rsrc_t r, lds_void_t* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, 0, 0, 0);
}
// copy16_buf into lds_base + kImm, from byte offset voff (>= kImm): the instruction's immediate
// offset moves both the LDS and the memory address, so copies into one region at constant
// distances share one LDS base (M0) and the wave writes M0 once for all of them.
// 16 bytes per lane at byte offset off from base into LDS (lane L's bytes at lds_base + 16 * L),
// for rows looked up one by one. With kOff32 (every offset used is below 4 GiB - 16) the load
// goes through a raw buffer based at base; otherwise through a flat 64-bit address. The two land
// the same bytes, but a flat copy into LDS makes the compiler treat every later LDS read as
// possibly out of order and wait for all of them (lgkmcnt(0)) wherever one is used, while with
// buffer copies only the kernel's own flat copies remain and it waits just for the reads needed.
template <bool kOff32>
__device__ __forceinline__ void copy16_row(const void* base, int64_t off, lds_void_t* lds_base) {
  if constexpr (kOff32) {
    const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xFFFFFFFF, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, (uint32_t)off, 0, 0, 0);
  } else {
    __builtin_amdgcn_global_load_lds((const char*)base + off, lds_base, 16, 0, 0);
  }
}
template <int kImm>
__device__ __forceinline__ void copy16_buf_at(__amdgpu_buffer_rsrc_t r, lds_void_t* lds_base, uint32_t voff) {
  static_assert(kImm >= 0 && kImm < 4096, "immediate offset range");
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff - kImm, 0, kImm, 0);
}
// The same with the non-temporal bit (data read once, in a stream), and 4 bytes per lane.
__device__ __forceinline__ void copy16_buf_stream(__amdgpu_buffer_rsrc_t r, lds_void_t* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, 0, 0, 2);
}
__device__ __forceinline__ void copy4_buf(__amdgpu_buffer_rsrc_t r, lds_void_t* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 4, voff, 0, 0, 0);
}

// Transposing LDS read: within each group of 16 lanes, lane i receives element (i % 4) of the
// 4 bf16 values addressed by lane 4 * jj + i / 4, for jj = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const lds_char_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p);
}

__device__ __forceinline__ bf16x8 lds_read16(const lds_char_t* p) {
  return *(const __attribute__((address_space(3))) bf16x8*)p;
}

// Value of x in lane (l ^ 32), via v_permlane32_swap.
__device__ __forceinline__ float xor32(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)((threadIdx.x & 32) ? r[0] : r[1]));
}
// max / sum of x over lanes l and l ^ 32
__device__ __forceinline__ float max_xor32(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}
// max / sum over lanes l and l ^ 16 (v_permlane16_swap pairs lanes 0-15 with 16-31, 32-47 with 48-63)
__device__ __forceinline__ float max_xor16(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                            float a6, float a7) {
  bf16x8 r;
  r[0] = (bf16_t)a0; r[1] = (bf16_t)a1; r[2] = (bf16_t)a2; r[3] = (bf16_t)a3;
  r[4] = (bf16_t)a4; r[5] = (bf16_t)a5; r[6] = (bf16_t)a6; r[7] = (bf16_t)a7;
  return r;
}

// Eight OCP E4M3FN codes (little-endian in two dwords) to bf16, exactly: every E4M3FN value is
// a bf16 value. The conversion's scale operand is 1.0, so no scaling happens here.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

}  // namespace segattn
