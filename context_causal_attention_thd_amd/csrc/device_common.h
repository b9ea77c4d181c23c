// Device-side helpers for the gfx950 kernels: bf16 vector types, MFMA
// wrappers and small conversions. CDNA4 wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace thdcp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane l holds row l%32 of A and column l%32 of B, k-slots 8*(l/32)..+7;
// accumulator element i of lane l is row 8*(i/4) + 4*(l/32) + i%4, column l%32.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate. Lane l holds
// row l%16 of A and column l%16 of B, k-slots 8*(l/16)..+7; accumulator
// element i of lane l is row 4*(l/16) + i, column l%16.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Round two 16x16 accumulators' entries (4 each) to one bf16x8 operand
// (round to nearest even, two values per conversion instruction).
__device__ __forceinline__ bf16x8 pack8(const f32x4& x, const f32x4& y) {
  return __builtin_shufflevector(__builtin_convertvector(x, bf16x4),
                                 __builtin_convertvector(y, bf16x4), 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void store_bf16x8(bf16* p, const bf16x8& v) {
  *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}

__device__ __forceinline__ bf16x4 load_bf16x4(const bf16* p) {
  return __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(p));
}

__device__ __forceinline__ bf16x8 concat4(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round-to-nearest-even float -> bf16 for 8 consecutive accumulator values
// (base 0 or 8), two per conversion instruction.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& v, int base) {
  const f32x8 x = base == 0 ? __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, 6, 7)
                            : __builtin_shufflevector(v, v, 8, 9, 10, 11, 12, 13, 14, 15);
  return __builtin_convertvector(x, bf16x8);
}

__device__ __forceinline__ uint32_t pack_bf16x2(bf16 lo, bf16 hi) {
  uint16_t a = __builtin_bit_cast(uint16_t, lo);
  uint16_t b = __builtin_bit_cast(uint16_t, hi);
  return (uint32_t)a | ((uint32_t)b << 16);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16). Within each group of 16
// lanes, lane i receives element i%4 of the 8 bytes that lane 4j + i/4 of the
// group addressed, as its element j. So if source lane s of the group points
// at row R[s/4], columns c0 + 4*(s%4) .. +3 of a row-major b16 matrix, lane i
// receives column c0 + i of rows R[0..3]: a column slice, as MFMA operands
// want, read straight from row-major tiles. All 64 lanes must be active.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value known to be the same in every lane of the wave, moved to a scalar
// register so that branches on it are scalar (no exec-mask divergence).
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }


__device__ __forceinline__ void store_bf16x4(bf16* p, const bf16x4& v) {
  *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float shfl_xor32(float x) {
  // exchange with the lane 32 away (the other half of the wave64)
  return __shfl_xor(x, 32, 64);
}


// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3):
// loads at offsets past the end return 0 without touching memory, so a tile
// whose last rows fall outside the data needs no branch around its loads.
// `bytes` stays below 2^31 (checked on the host), so an offset of 0xFFFFFFF0
// is always past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// gfx950 LDS DMA: 16 bytes per lane from buffer r at byte offset off straight
// into LDS, lane i at lds + 16 i (lds wave-uniform). No register holds the
// data and the wave writes nothing to LDS itself; the write lands
// asynchronously and is counted by vmcnt. An offset past the descriptor
// writes zeros (as a plain buffer load reads them).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, (int)off, 0, 0, 0);
}

// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Maximum (or sum) over the four 16-lane groups of a wave with the gfx950
// lane-swap instructions (VALU, no LDS traffic): permlane16_swap exchanges
// 16-lane rows 0<->1 and 2<->3, permlane32_swap the two halves of the wave.
__device__ __forceinline__ float group_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t u2 = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group_sum4(float x) {
  const uint32_t u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t u2 = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Gated tail zeroing by whole workgroups: workgroup b of the zeroing part of
// a grid writes 0 to kZeroRowsPerBlock of the dK/dV rows no local query
// attends (all heads), found among the plan's untouched ranges (`before` is
// the count of such rows ahead of each range). Key row g is row
// (kv_row ? kv_row[g] : g) - kv_sub of dk and dv.
constexpr int kZeroRowsPerBlock = 8;

__device__ inline void zero_untouched_block(int64_t b, const ZeroRange* __restrict__ zr,
                                            int32_t n_zr, int64_t zero_rows,
                                            const int32_t* __restrict__ kv_row, int32_t kv_sub,
                                            int64_t row_floats, float* __restrict__ dk,
                                            float* __restrict__ dv) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const int64_t vpr = row_floats / 4;
  for (int rr = 0; rr < kZeroRowsPerBlock; ++rr) {
    const int64_t lin = b * kZeroRowsPerBlock + rr;  // index among all untouched rows
    if (lin >= zero_rows) break;
    int32_t lo = 0, hi = n_zr - 1;  // last range with before <= lin
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if ((int64_t)zr[mid].before <= lin) lo = mid; else hi = mid - 1;
    }
    const int64_t g = zr[lo].r0 + (lin - zr[lo].before);
    const int64_t row = (kv_row ? kv_row[g] : g) - kv_sub;  // global row -> row of dk/dv
    f32x4* a = reinterpret_cast<f32x4*>(dk + row * row_floats);
    f32x4* c = reinterpret_cast<f32x4*>(dv + row * row_floats);
    for (int64_t i = threadIdx.x; i < vpr; i += blockDim.x) {
      a[i] = z;
      c[i] = z;
    }
  }
}

// Split key walks: every thread of a part's workgroup calls this after
// writing the part's partial result. Each wave waits until its stores have
// reached the L2; one agent-scope release (a write-back of the XCD's L2)
// then publishes the whole workgroup's stores before the workgroup is counted
// on *cnt. The workgroup that completes the count of nparts gets true in
// every thread: it resets the counter for the next launch and performs one
// agent-scope acquire (invalidating its CU's L1 and its XCD's L2) before any
// of its waves reads the other parts' results. No workgroup waits for
// another. One release and one acquire per workgroup, not per wave: the
// cache maintenance is cache-wide, and per-wave fences measured several
// times slower.
__device__ inline bool split_arrive(int32_t* cnt, int32_t nparts) {
  __shared__ int32_t s_last;
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int32_t before =
        __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == nparts - 1;
    if (s_last) {
      __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
  }
  __syncthreads();
  return s_last != 0;
}

// Scratch of one part of a split key walk (slot x, head h) of a kernel whose
// tiles hold ROWS query rows of D dims.
template <int D, int ROWS>
__device__ inline float* split_slot(float* part, int32_t x, int32_t h, int32_t H) {
  return part + ((int64_t)x * H + h) * kSplitFloats(D, ROWS);
}

}  // namespace thdcp
