// Shared device-side definitions for the gfx950 kernels of the policy step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace vla {

typedef uint16_t bf16_t;  // bfloat16 bit pattern in memory

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int i32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bfloat16, round to nearest, ties to even (NaN stays a quiet NaN):
// gfx950 converts in hardware (v_cvt_pk_bf16_f32, two values per instruction)
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}

// A workgroup-uniform int from device memory that no kernel writes while this
// one runs, through the scalar cache: a vector load here would make the
// compiler wait for every load issued before it (loads retire in order).
__device__ __forceinline__ int uniform_ld(const int* p, int i) {
  return *((const __attribute__((address_space(4))) int*)(uintptr_t)p + i);
}

// 2^x on the hardware exponential unit (one instruction; results below the
// normal range flush to zero, 2^-inf = 0).  Used for softmax weights in (0, 1].
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// GELU in its error-function form, 0.5 x (1 + erf(x / sqrt 2)) = 0.5 x
// erfc(-x / sqrt 2).  erfc(z) for z >= 0 comes from the Chebyshev-fitted
// exponential form of Numerical Recipes (Press et al., function erfcc),
// whose fractional error is below 1.2e-7 for every z, so the product keeps
// fp32-level relative error on both tails.  It has no branches: in a GEMM
// epilogue every lane evaluates a different argument, and a wave64 VALU
// instruction costs four cycles, so this is about a quarter of the cost of
// the library erff there.
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float q = fmaf(t, 0.17087277f, -0.82215223f);
  q = fmaf(t, q, 1.48851587f);
  q = fmaf(t, q, -1.13520398f);
  q = fmaf(t, q, 0.27886807f);
  q = fmaf(t, q, -0.18628806f);
  q = fmaf(t, q, 0.09678418f);
  q = fmaf(t, q, 0.37409196f);
  q = fmaf(t, q, 1.00002368f);
  q = fmaf(t, q, -1.26551223f);
  const float ec = t * fast_exp2(fmaf(-z, z, q) * 1.4426950408889634f);  // erfc(|x| / sqrt 2)
  return 0.5f * x * (x >= 0.f ? 2.0f - ec : ec);
}

// ---------------------------------------------------------------- reductions
// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 lane-swap instructions: each swap pairs lane l with l^32
// (l^16) as its two results, a VALU round trip instead of an LDS permute.
__device__ __forceinline__ float group4_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Whole-wave reductions: inside each 16-lane row with DPP lane moves (pairs
// i ^ 1, then i ^ 2, then the mirrored quad of each half row, then the
// mirrored half row), then across the four rows with the lane swaps above.
// Every step adds two equal-rank partial sums, so every lane ends with the same
// bits, and no step goes through the LDS permute unit.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return group4_sum(v);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return group4_max(v);
}

// Sum over a block of `NT` threads (NT a multiple of 64); every thread gets the result.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red /* >= NT/64 floats of LDS */) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) s = fmaxf(s, red[i]);
  return s;
}

// ---------------------------------------------------------------- MFMA wrappers
// 32x32x16 bf16 -> f32.  Lane l supplies A row (l % 32), k = (l / 32) * 8 + [0, 8);
// B column (l % 32), same k; accumulator element i of lane l is row
// (i / 4) * 8 + (l / 32) * 4 + (i % 4), column (l % 32).
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 16x16x32 bf16 -> f32.  Lane l supplies A row (l % 16), k = (l / 16) * 8 + [0, 8);
// accumulator element i of lane l is row (l / 16) * 4 + i, column (l % 16).
__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 32x32x32 int8 -> int32.  Lane l supplies 16 bytes: row (l % 32), k = (l / 32) * 16 + [0, 16);
// accumulator layout as for 32x32x16.
__device__ __forceinline__ i32x16_t mfma32x32x32_i8(i32x4_t a, i32x4_t b, i32x16_t c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// Fragment layout of a [rows][K] bf16 matrix for the 16x16x32 MFMA: blocks of
// 16 rows x 32 columns, each block 1 KB in the order the 64 lanes of a wave
// consume it (lane = row % 16 + 16 * ((col % 32) / 8), 8 consecutive columns per
// lane), blocks row-block major.  One wave loads one block as one contiguous 1 KB.
__host__ __device__ __forceinline__ long frag_idx(int m, int k, int K) {
  return ((((long)(m >> 4) * (K >> 5) + (k >> 5)) * 64 + ((m & 15) + ((k >> 3) & 3) * 16)) << 3) + (k & 7);
}

// Value layout for the P V product of attention, O^T += V^T P^T on the 16x16x32
// MFMA, for a [keys][D] matrix V: one 1 KB block per 32-key tile and 16 columns
// d, holding V^T's A-operand fragment.  Lane (d % 16) + 16 * g supplies 8 keys
// of the tile, {4 g .. 4 g + 3} then {16 + 4 g .. 16 + 4 g + 3}: the order in
// which the transposed score accumulator (rows = keys) hands P^T to the B operand.
__host__ __device__ __forceinline__ long vfrag_idx(int t, int d, int D) {
  const int kin = t & 31;
  const long blk = (long)(t >> 5) * (D >> 4) + (d >> 4);
  return ((blk * 64 + (d & 15) + 16 * ((kin & 15) >> 2)) << 3) + (kin >> 4) * 4 + (kin & 3);
}

// Workgroup `blk` of `nblk` reads its share of the ranges, 16 loads of 16 bytes
// per thread in flight, and folds them so the loads are kept.
// Extra workgroups [first, first + count) of a kernel (linear ids) read the
// byte ranges of `f` once and drop them, so the kernel after finds them in
// cache: a range without a group is shared by all of them; a grouped range is
// read XCD by XCD (see Prefetch), each workgroup taking a share of the groups
// of its own XCD (linear id % 8); groups that are not a power of two in size
// are read like ungrouped ranges.  Sixteen 16-byte loads per thread are in
// flight at a time.  Ranges are below 32 GB.
__device__ __forceinline__ void prefetch_share(const Prefetch& f, int L, int first, int count) {
  constexpr int U = 16;
  const int c = L & 7;
  const int fc = first + ((c - first) & 7);                      // first prefetch workgroup on this XCD
  const int nc = fc < first + count ? (first + count - 1 - fc) / 8 + 1 : 1;
  const int rc = (L - fc) >> 3;
  unsigned x = 0;
  auto range = [&](const void* p, size_t bytes, size_t group) {
    if (!p || bytes < 16) return;
    const u32x4_t* v = (const u32x4_t*)p;
    // vector i of this workgroup's share maps to v[(i >> sh) * jump + (i & mk)]:
    // groups of 2^sh vectors, of which every eighth is this XCD's (jump = 8
    // groups, starting at group c), or the whole range (sh = 31)
    uint32_t n, part, stride, sh = 31, mk = 0xffffffffu;
    size_t jump = 0;
    const u32x4_t* v0 = v;
    if (group >= 16 && !(group & (group - 1))) {
      sh = 31 - __builtin_clz((uint32_t)(group >> 4));
      mk = (1u << sh) - 1;
      const uint32_t ng = (uint32_t)(bytes / group);
      n = ng > (uint32_t)c ? (((ng - 1 - c) >> 3) + 1) << sh : 0;  // vectors of the groups c, c + 8, ...
      jump = (size_t)8 << sh;
      v0 = v + ((size_t)c << sh);
      part = rc; stride = nc;
    } else {
      n = (uint32_t)(bytes >> 4);
      part = L - first; stride = count;
    }
    const uint32_t step = stride * blockDim.x;
    for (uint32_t base = part * blockDim.x + threadIdx.x; base < n; base += step * U) {
      u32x4_t t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = min(base + u * step, n - 1);
        t[u] = v0[(i >> sh) * jump + (i & mk)];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) x ^= t[u][0] ^ t[u][3];
    }
  };
  range(f.p, f.bytes, f.group);
  range(f.p2, f.bytes2, f.group2);
  range(f.p3, f.bytes3, f.group3);
  if (x == 0x9E3779B9u) f.sink[L & 63] = x;
}

// A kernel's own workgroups form grid layer z = 0; its prefetch workgroups
// follow in layers z >= 1 (workgroups are numbered x fastest, then y, then z,
// which is the order they reach the XCDs).  The test reads the dispatch index
// register: a test on a kernel argument made the kernel's own work wait for a
// first scalar load before its remaining arguments were even requested.
__device__ __forceinline__ bool prefetch_layer(const Prefetch& f) {
  if (!blockIdx.z) return false;
  const int per = gridDim.x * gridDim.y;
  prefetch_share(f, per * blockIdx.z + gridDim.x * blockIdx.y + blockIdx.x, per, per * (gridDim.z - 1));
  return true;
}

// acc row index of element i for lane l in a 32x32 MFMA block
__device__ __forceinline__ int mfma32_row(int i, int lane) { return (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3); }

}  // namespace vla
