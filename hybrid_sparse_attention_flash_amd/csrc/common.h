// Shared device helpers for the gfx950 kernels of the HySparse hot path.
//
// Element storage types:
//   float     - fp32
//   uint16_t  - bf16 bits
//   uint8_t   - OCP fp8 e4m3fn bits (value = decode(byte) * per-tensor scale)
//
// MFMA lane layouts used throughout (wave64, checked on gfx950):
//   v_mfma_f32_32x32x16_bf16: lane l holds A[m=l%32][k=8*(l/32)+j], B[k=8*(l/32)+j][n=l%32]
//                             (j = 0..7) and C[m=8*(i/4)+4*(l/32)+i%4][n=l%32] (i = 0..15)
//   v_mfma_f32_32x32x2_f32:   lane l holds A[m=l%32][k=l/32], B[k=l/32][n=l%32], same C
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hys {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// Slack of the online softmax's reference maximum, in base-2 exponent units:
// a row's reference moves only when a tile maximum exceeds it by more than
// this, so probabilities stay below 2^kLazyLog2 and O is rescaled rarely.
constexpr float kLazyLog2 = 8.0f;

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}

// round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two fp32 -> packed bf16x2, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// OCP e4m3fn -> bf16, exact: v_cvt_scalef32_pk_bf16_fp8 with scale 1
// decodes two e4m3fn bytes of a dword (the low or the high half) straight to
// two bf16 (one instruction; every finite e4m3 value has at most 4
// significant bits and an exponent well inside bf16's range, so nothing
// rounds).  Checked bit for bit against the format definition for every
// finite code through the attention path.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi_word) {
  return __builtin_bit_cast(uint32_t, hi_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

// Four fp8 bytes (one dword) -> four bf16 (two dwords).
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = fp8x2_to_bf16x2(w, false);
  hi = fp8x2_to_bf16x2(w, true);
}

// Four fp8 bytes -> four fp32.
__device__ __forceinline__ f32x4 fp8x4_to_f32x4(uint32_t w) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  f32x4 r = {a[0], a[1], b[0], b[1]};
  return r;
}

// IEEE maximum of two floats in one instruction.  Values that crossed lanes
// come back as integers, and fmaxf on them would first quiet them (an extra
// v_max per operand); the logits handled here are never NaN.
__device__ __forceinline__ float fmax_nc(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max(v[l], v[l ^ 32]) for every lane l: v_permlane32_swap of v with itself
// leaves the two 32-lane halves exchanged between its two results.
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nc(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max(v[l], v[l ^ 16]) for every lane l (v_permlane16_swap exchanges odd and
// even 16-lane rows).
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nc(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Column maxima of a 32 x 32 block held one column value per register:
// lane l (l = 32h + r) holds v[x] = M_h[r][x] for a 32 x 32 matrix M_h per
// half h, and the result is max over r of M_h[r][x] for the four columns
// x = (r & 28) + c, c = 0..3, returned in element c (all four lanes of a quad
// receive the same four maxima).  A reduce-scatter: the row bit 4 step pairs
// registers x and x + 16 through v_permlane16_swap; the bit 3 and bit 2 steps
// use DPP row_mirror / row_half_mirror with bank masks, so each lane half of a
// bank pair updates only the register range it keeps; bits 1 and 0 are then
// all-reduced with quad permutes.  32 VALU operations and no LDS traffic.
__device__ __forceinline__ f32x4 colmax32(const float (&v)[32]) {
  float w[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[x]), __float_as_uint(v[x + 16]), false, false);
    w[x] = fmax_nc(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  // One block so the ordering below holds: every DPP read is at least two
  // instructions after the write of its source (the s_nop covers the VALU
  // writes before the block).  A disabled bank keeps its destination value.
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %0, %8, %8 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %1, %1, %1 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %1, %9, %9 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %2, %2, %2 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %2, %10, %10 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %3, %3, %3 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %3, %11, %11 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %4, %4, %4 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %4, %12, %12 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %5, %5, %5 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %5, %13, %13 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %6, %6, %6 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %6, %14, %14 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      "v_max_f32_dpp %7, %7, %7 row_mirror row_mask:0xf bank_mask:0x3\n\t"
      "v_max_f32_dpp %7, %15, %15 row_mirror row_mask:0xf bank_mask:0xc\n\t"
      // bit 2: banks 0, 2 keep registers 0..3, banks 1, 3 take 4..7
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %0, %4, %4 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_max_f32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %1, %5, %5 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_max_f32_dpp %2, %2, %2 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %2, %6, %6 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      "v_max_f32_dpp %3, %3, %3 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_max_f32_dpp %3, %7, %7 row_half_mirror row_mask:0xf bank_mask:0xa\n\t"
      // bits 1 and 0: all-reduce inside each quad
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %2, %2, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_max_f32_dpp %3, %3, %3 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]), "+v"(w[6]), "+v"(w[7])
      : "v"(w[8]), "v"(w[9]), "v"(w[10]), "v"(w[11]), "v"(w[12]), "v"(w[13]), "v"(w[14]), "v"(w[15]));
  const f32x4 o = {w[0], w[1], w[2], w[3]};
  return o;
}

// max over aligned groups of W consecutive lanes (W in {2,4,8,16,32}), every
// lane of a group receiving the group max.  Lane pairs are exchanged with DPP
// (quad_perm, row_half_mirror, row_mirror) inside a 16-lane row; the 32-wide
// step crosses rows with v_permlane16_swap.
template <int W> __device__ __forceinline__ float group_max(float v) {
  if (W >= 2)
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  if (W >= 4)
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  if (W >= 8)
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  if (W >= 16)
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
  if (W >= 32) v = xor16_max(v);
  return v;
}

// Inclusive prefix sum of an int over the 64 lanes of a wave, by DPP:
// row_shr 1, 2, 3 (from the original values), 4 and 8 within each 16-lane
// row, then row_bcast 15 / 31 across rows.  Invalid DPP sources read 0.
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  int x = v + __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);       // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);              // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, v, 0x113, 0xF, 0xF, true);              // row_shr:3
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xE, true);              // row_shr:4, banks 1-3
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xC, true);              // row_shr:8, banks 2-3
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, true);              // row_bcast:15, rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, true);              // row_bcast:31, rows 2, 3
  return x;
}

// Sum of an int over the 64 lanes of a wave (wave-uniform): the last lane of
// the inclusive scan.
__device__ __forceinline__ int wave_sum_i32(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan_i32(v), 63);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
// -inf maps below every finite value; NaN is handled by callers.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 consecutive stored elements as raw registers
template <typename KT> struct Raw8;
template <> struct Raw8<float> { uint4 a, b; };
template <> struct Raw8<uint16_t> { uint4 a; };
template <> struct Raw8<uint8_t> { uint2 a; };

template <typename KT> __device__ __forceinline__ Raw8<KT> load8(const KT* p);
template <> __device__ __forceinline__ Raw8<float> load8<float>(const float* p) {
  Raw8<float> r; r.a = *(const uint4*)p; r.b = *(const uint4*)(p + 4); return r;
}
template <> __device__ __forceinline__ Raw8<uint16_t> load8<uint16_t>(const uint16_t* p) {
  Raw8<uint16_t> r; r.a = *(const uint4*)p; return r;
}
template <> __device__ __forceinline__ Raw8<uint8_t> load8<uint8_t>(const uint8_t* p) {
  Raw8<uint8_t> r; r.a = *(const uint2*)p; return r;
}
template <typename KT> __device__ __forceinline__ Raw8<KT> zero8() { Raw8<KT> r; __builtin_memset(&r, 0, sizeof(r)); return r; }

// Zero a staged unit whose slot is empty.  Staging loads are issued
// unconditionally from a clamped, in-bounds address (a branch around each
// load makes the compiler wait for every earlier load before issuing the
// next, which serialises the whole prefetch); the select happens when the
// data is consumed.
__device__ __forceinline__ uint32_t sel0(uint32_t x, bool ok) { return ok ? x : 0u; }
__device__ __forceinline__ void keep_if(Raw8<float>& r, bool ok) {
  r.a = make_uint4(sel0(r.a.x, ok), sel0(r.a.y, ok), sel0(r.a.z, ok), sel0(r.a.w, ok));
  r.b = make_uint4(sel0(r.b.x, ok), sel0(r.b.y, ok), sel0(r.b.z, ok), sel0(r.b.w, ok));
}
__device__ __forceinline__ void keep_if(Raw8<uint16_t>& r, bool ok) {
  r.a = make_uint4(sel0(r.a.x, ok), sel0(r.a.y, ok), sel0(r.a.z, ok), sel0(r.a.w, ok));
}
__device__ __forceinline__ void keep_if(Raw8<uint8_t>& r, bool ok) {
  r.a = make_uint2(sel0(r.a.x, ok), sel0(r.a.y, ok));
}

// 8 elements in compute layout: bf16 -> one uint4, fp32 -> two uint4
template <typename CT> struct Cvt8;
template <> struct Cvt8<uint16_t> { uint4 a; };
template <> struct Cvt8<float> { uint4 a, b; };

__device__ __forceinline__ Cvt8<uint16_t> to_ct(const Raw8<uint16_t>& r) { Cvt8<uint16_t> c; c.a = r.a; return c; }
__device__ __forceinline__ Cvt8<uint16_t> to_ct(const Raw8<uint8_t>& r) {
  Cvt8<uint16_t> c;
  fp8x4_to_bf16x4(r.a.x, c.a.x, c.a.y);
  fp8x4_to_bf16x4(r.a.y, c.a.z, c.a.w);
  return c;
}
__device__ __forceinline__ Cvt8<float> to_ct(const Raw8<float>& r) { Cvt8<float> c; c.a = r.a; c.b = r.b; return c; }

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

}  // namespace hys
