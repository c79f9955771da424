// mfma_util.hpp -- device helpers of the matrix-core (MFMA) kernels for gfx950:
// operand types, the 32x32x16 bf16 MFMA, LDS transpose-reads, bf16 packing,
// streaming loads and the LDS-only barrier.
//
// MFMA 32x32x16 bf16 operand layout (lane l, half h = l / 32):
//   A[m][k]: lane holds m = l % 32, k = 8h .. 8h+7
//   B[k][n]: lane holds n = l % 32, k = 8h .. 8h+7
//   C[m][n]: element r holds m = 8(r/4) + 4h + r%4, n = l % 32
// Any consistent relabelling of k between A and B gives the same sum.
#pragma once

#include "common.hpp"

namespace gla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.
// Renumbering so that XCD x runs a contiguous range of work items keeps
// neighbouring frames (which share their group's carried state) on one L2.
// A bijection on [0, n): the first 8 * floor(n / 8) ids are remapped, the
// remainder keep their id.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_contiguous(int64_t w, int64_t n) {
  const int64_t per = n / kXcds;
  if (w >= per * kXcds) return w;
  return (w % kXcds) * per + w / kXcds;
}

template <bool kNt>
__device__ __forceinline__ uint4 ld_stream16(const uint4 *p) {
  if constexpr (kNt) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
  } else {
    return *p;
  }
}

// Workgroup barrier for data exchanged through LDS only. __syncthreads() also
// fences global memory, which on this architecture waits for every
// outstanding global load and store (vmcnt(0)) -- including the prefetch of
// the next tile and the stores of the previous one -- before the barrier.
// Waiting for LDS operations alone (lgkmcnt(0)) is enough for LDS data.
__device__ __forceinline__ void sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for every global load and store issued so far (vmcnt(0); expcnt and
// lgkmcnt at their maximum: no wait). Placed in front of a tile loop whose
// first tile was loaded ahead of it: then no path enters the loop with a load
// outstanding. Otherwise the compiler, which counts loads and stores on one
// counter, waits inside the loop for that load by count -- vmcnt(0) -- and so
// each iteration waits for the previous tile's stores, or for the next tile's
// prefetch, as well.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int kCtrl>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                          0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over each aligned group of kLanes lanes (2, 4, 8 or 16), in every lane of
// the group, by DPP moves on the vector ALU: swap neighbours and pairs within
// quads, then mirror half-rows (lane i of 8 takes 7 - i) and rows (i of 16
// takes 15 - i). A shuffle (__shfl_xor) goes through the LDS crossbar instead,
// a round trip per step.
template <int kLanes>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(kLanes == 2 || kLanes == 4 || kLanes == 8 || kLanes == 16, "group of 2 to 16");
  x = dpp_add<0xB1>(x);                           // quad_perm [1, 0, 3, 2]
  if constexpr (kLanes >= 4) x = dpp_add<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  if constexpr (kLanes >= 8) x = dpp_add<0x141>(x);  // row_half_mirror
  if constexpr (kLanes >= 16) x = dpp_add<0x140>(x); // row_mirror
  return x;
}

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 (lane l, g = l / 16):
//   A[m][k]: m = l % 16, k = 8g .. 8g+7;  B[k][n]: n = l % 16, k = 8g .. 8g+7
//   C[m][n]: element r holds m = 4g + r, n = l % 16
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ReLU of two packed bf16: as signed 16-bit integers every negative bf16
// (including -0) is negative, so max(x, 0) in int16 is max(x, +0) in bf16.
__device__ __forceinline__ uint32_t relu2(uint32_t w) {
  i16x2 v = __builtin_bit_cast(i16x2, w);
  v = __builtin_elementwise_max(v, (i16x2){0, 0});
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint4 relu8(uint4 x) {
  return make_uint4(relu2(x.x), relu2(x.y), relu2(x.z), relu2(x.w));
}

// Gate and normaliser of the epilogue with the hardware reciprocal (v_rcp_f32,
// 1 ulp) rather than an IEEE division (~10 instructions each): the result is
// rounded to bf16 right after. exp overflow still gives sigmoid = 0 exactly.
__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ bf16x8 tr_fragment(const lds_char *tile, int row, int col, int pitch) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4 *)(tile + row * pitch + col * 2));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4 *)(tile + (row + 4) * pitch + col * 2));
  const i16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}


// x = hi + lo, both bf16: returns hi in the low half, lo in the high half
__device__ __forceinline__ uint32_t split_hl(float x) {
  const uint16_t h = f32_to_bf16_rne(x);
  return (uint32_t)h | ((uint32_t)f32_to_bf16_rne(x - bf16_to_f32(h)) << 16);
}

// (x0, x1) = hi + lo with both parts bf16, as packed pairs: v_cvt_pk_bf16_f32
// rounds to nearest even, like split_hl, two values per instruction
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(x0, x1);
  lo = pack_bf16x2(x0 - lo_bf16(hi), x1 - hi_bf16(hi));
}

// A fragments (hi, lo) of M^T for output block mb: A[m = j][k = i] = M[i][j]
template <int D>
__device__ __forceinline__ void frag_transposed(const float *M, int mb, int lane, bf16x8 *hi,
                                                bf16x8 *lo) {
  const int h = lane >> 5, col = 32 * mb + (lane & 31);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    i16x8 hv, lv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t x = split_hl(M[(16 * ks + 8 * h + e) * D + col]);
      hv[e] = (short)(x & 0xFFFFu);
      lv[e] = (short)(x >> 16);
    }
    hi[ks] = __builtin_bit_cast(bf16x8, hv);
    lo[ks] = __builtin_bit_cast(bf16x8, lv);
    asm volatile("" ::: "memory");  // one k-step of loads in flight at a time (registers)
  }
}

// A fragments (hi, lo) of M for output block mb: A[m = i][k = j] = M[i][j]
// (each lane reads 8 consecutive floats of a row)
template <int D>
__device__ __forceinline__ void frag_direct(const float *M, int mb, int lane, bf16x8 *hi,
                                            bf16x8 *lo) {
  const int h = lane >> 5, row = 32 * mb + (lane & 31);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const float4 a = *reinterpret_cast<const float4 *>(M + row * D + 16 * ks + 8 * h);
    const float4 b = *reinterpret_cast<const float4 *>(M + row * D + 16 * ks + 8 * h + 4);
    const float xs[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    i16x8 hv, lv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t x = split_hl(xs[e]);
      hv[e] = (short)(x & 0xFFFFu);
      lv[e] = (short)(x >> 16);
    }
    hi[ks] = __builtin_bit_cast(bf16x8, hv);
    lo[ks] = __builtin_bit_cast(bf16x8, lv);
  }
}

__device__ __forceinline__ void st_stream16(uint4 *p, uint4 v) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(p));
}

}  // namespace gla
