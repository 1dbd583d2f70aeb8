// Device-side helpers shared by the kernels of libmqa_int8 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// v_mfma_f32_16x16x32_bf16. Lane l = 16*g + c (g = l/16, c = l%16):
//   A (16x32, M x K): lane holds A[c][8g .. 8g+7]
//   B (32x16, K x N): lane holds B[8g .. 8g+7][c]
//   C (16x16, M x N): lane holds C[4g + r][c], r = 0..3
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_f16, same lane layout as the bf16 form.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
// int8 x int8 -> int32, 16x16x64: each lane supplies 16 bytes of A and of B.
__device__ __forceinline__ i32x4 mfma16_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ u32x4 cat(u32x2 a, u32x2 b) { return u32x4{a[0], a[1], b[0], b[1]}; }

// Pack the bf16 patterns of two fp32 values whose low 16 bits are zero (for
// example small integers): result = hi16(b) << 16 | hi16(a).
__device__ __forceinline__ uint32_t pack_hi16(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// Four int8 codes (one 32-bit word) -> four exact bf16 values, as two words.
// Every int8 value (including -128) has at most 8 significant bits, so the
// fp32 conversion is exact and its upper half is the exact bf16 pattern.
// (float)(signed char)(w >> 8k) is a single v_cvt_f32_i32 with an SDWA
// sign-extended byte select on gfx950.
__device__ __forceinline__ u32x2 i8x4_to_bf16(uint32_t w) {
  const float f0 = (float)(signed char)(w);
  const float f1 = (float)(signed char)(w >> 8);
  const float f2 = (float)(signed char)(w >> 16);
  const float f3 = (float)(signed char)(w >> 24);
  return u32x2{pack_hi16(f0, f1), pack_hi16(f2, f3)};
}

// Byte `sel` (0..3) of a word as an exact fp32 value of the signed int8.
__device__ __forceinline__ float i8_byte(uint32_t w, int sel) {
  return (float)(signed char)(w >> (8 * sel));
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 of two values, packed (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Split two fp32 values into bf16 hi + lo parts, both rounded to nearest
// even: x = hi + lo + e with |e| <= 2^-18 |x| (hi keeps 8 significant bits,
// the exact fp32 remainder x - hi is rounded to 8 more). Returns {hi, lo}
// as packed pairs.
__device__ __forceinline__ u32x2 split_bf16(float a, float b) {
  const uint32_t h = cvt_pk_bf16(a, b);
  return u32x2{h, cvt_pk_bf16(a - bf16_lo_to_f32(h), b - bf16_hi_to_f32(h))};
}

// Round-to-nearest-even fp32 -> fp16 of two values, packed (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t cvt_pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// int8 -> fp16, exact, one instruction per byte: an SDWA convert sign-extends
// the selected byte of a word and writes the low half (upper half cleared) or
// the high half (low half kept) of the result. hipcc does not form these
// itself, so they are written as inline asm, and the compiler's hazard
// tracking does not see asm as vector ALU work: each block below therefore
// keeps its own wait states. A half written through dst_sel is read by the
// next instruction only after one wait state (the four low halves come first,
// so every high-half write is at least three instructions after the low half
// it keeps), and a vector ALU result may feed an MFMA source only after two;
// each block ends with three (s_nop 2) before anything can read its results.

// One MFMA operand of four fp16 pairs: pair i = {byte SEL of w[2i], byte SEL
// of w[2i + 1]}.
template <int SEL>
__device__ __forceinline__ u32x4 f16_pairs_of_bytes(const uint32_t (&w)[8]) {
  uint32_t d0, d1, d2, d3;
#define MQA_LO(D, W) "v_cvt_f16_i16_sdwa " D ", sext(" W ") dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_%12\n\t"
#define MQA_HI(D, W) "v_cvt_f16_i16_sdwa " D ", sext(" W ") dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_%12\n\t"
  asm(MQA_LO("%0", "%4") MQA_LO("%1", "%6") MQA_LO("%2", "%8") MQA_LO("%3", "%10")
      MQA_HI("%0", "%5") MQA_HI("%1", "%7") MQA_HI("%2", "%9") MQA_HI("%3", "%11") "s_nop 2"
      : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
      : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(w[4]), "v"(w[5]), "v"(w[6]), "v"(w[7]), "i"(SEL));
  return u32x4{d0, d1, d2, d3};
}
// Eight int8 codes (two words) -> eight fp16 values (one MFMA operand), in order.
__device__ __forceinline__ u32x4 i8x8_to_f16(uint32_t w0, uint32_t w1) {
  uint32_t d0, d1, d2, d3;
  asm("v_cvt_f16_i16_sdwa %0, sext(%4) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
      "v_cvt_f16_i16_sdwa %1, sext(%4) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
      "v_cvt_f16_i16_sdwa %2, sext(%5) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0\n\t"
      "v_cvt_f16_i16_sdwa %3, sext(%5) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
      "v_cvt_f16_i16_sdwa %0, sext(%4) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
      "v_cvt_f16_i16_sdwa %1, sext(%4) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3\n\t"
      "v_cvt_f16_i16_sdwa %2, sext(%5) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1\n\t"
      "v_cvt_f16_i16_sdwa %3, sext(%5) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3\n\t"
      "s_nop 2"
      : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3)
      : "v"(w0), "v"(w1));
  return u32x4{d0, d1, d2, d3};
}
#undef MQA_LO
#undef MQA_HI

// Split two fp32 values into fp16 hi + lo parts, both rounded to nearest
// even: hi = fp16(x), lo = fp16(x - hi) with the difference formed exactly in
// fp32 by a mixed-precision FMA (v_fma_mix{lo,hi}_f16). For |x| >= 2^-3 the
// pair carries 22 significant bits; below that lo is subnormal and the
// absolute error stays under 2^-25. Returns {hi, lo} as packed pairs.
__device__ __forceinline__ u32x2 split_f16(float a, float b) {
  const uint32_t hi = cvt_pk_f16(a, b);
  uint32_t lo;
  // asm, so its wait states are its own (as for the conversions above): one
  // after the low-half write, three before the result may feed an MFMA
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "s_nop 0\n\t"
      "v_fma_mixhi_f16 %0, %1, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
      "s_nop 2"
      : "=&v"(lo)
      : "v"(hi), "v"(a), "v"(b));
  return u32x2{hi, lo};
}

// int8 KV encoding of one value (the library's quantizer and the fused append
// share these, so both write identical bytes): scale s = fl32(absmax / 127),
// code = clamp(rint(fl32(x / s)), -127, 127); both divisions are IEEE
// correctly rounded fp32 divisions and rintf rounds half to even. A row whose
// scale is 0 is all zero codes.
__device__ __forceinline__ float kv_row_scale(float absmax) { return absmax / 127.0f; }
__device__ __forceinline__ int kv_code(float x, float s) {
  if (s == 0.0f) return 0;
  const float qv = rintf(x / s);
  return (int)fminf(fmaxf(qv, -127.0f), 127.0f);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [I0, I1).
template <int I0, int I1, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < I1) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, I1>(f);
  }
}

// Max of 8 values as a chain the compiler turns into v_max3_f32.
__device__ __forceinline__ float max8(const float (&x)[8]) {
  float m = fmaxf(fmaxf(x[0], x[1]), x[2]);
  m = fmaxf(fmaxf(m, x[3]), x[4]);
  m = fmaxf(fmaxf(m, x[5]), x[6]);
  return fmaxf(m, x[7]);
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (v_permlane{16,32}_swap).
__device__ __forceinline__ float quad_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ int quad_max_i(int v) {
  const auto a = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  v = max((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  return max((int)b[0], (int)b[1]);
}
// Max over all 64 lanes, in every lane: two lane-half swaps, then rotations
// within each row of 16 lanes and quad permutations (DPP, no LDS traffic).
__device__ __forceinline__ float wave_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));  // row_ror:8
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));  // row_ror:4
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false)));   // quad [2,3,0,1]
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false)));   // quad [1,0,3,2]
  return v;
}
__device__ __forceinline__ float quad_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^x with the hardware instruction (no denormal range handling: results
// below the normal range flush to 0, which only drops negligible weights).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A pointer every lane holds alike, moved to scalar registers. A buffer
// resource built from a value the compiler keeps in vector registers (it
// does so under scalar register pressure) is re-made in every load by a
// loop over the distinct values of the wave.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Buffer resource over [base, base + bytes): loads beyond it return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// s_waitcnt immediate for "at most n vector memory operations outstanding"
// (gfx9 encoding; expcnt and lgkmcnt left at no-wait).
__device__ __forceinline__ constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

// Physical row of token position t of sequence b in a paged KV buffer:
// block table[b][(t >> log2_bs) % table_len], entry clamped into the pool.
__device__ __forceinline__ int64_t paged_row(const int32_t* table, int table_len, int log2_bs, int num_blocks,
                                             int b, int t) {
  int e = table[(int64_t)b * table_len + (t >> log2_bs) % table_len];
  e = e < 0 ? 0 : (e >= num_blocks ? num_blocks - 1 : e);
  return ((int64_t)e << log2_bs) | (t & ((1 << log2_bs) - 1));
}

// Streaming variants: the non-temporal hint (nt) for data read once per call.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicyNT));
}
__device__ __forceinline__ u32x2 buf_load8_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kCachePolicyNT));
}
__device__ __forceinline__ uint32_t buf_load4_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kCachePolicyNT);
}

}  // namespace mqa
