// Device helpers shared by the LLoPS kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llops {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---- bf16 <-> f32 --------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Round-to-nearest-even fp32 -> bf16 pair (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return static_cast<uint16_t>(pack_bf16x2(x, 0.f) & 0xFFFFu);
}

// ---- 16-byte vector memory ------------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// ---- buffer loads ----------------------------------------------------------
// A raw buffer resource over [base, base + bytes): loads address it with a
// 32-bit lane offset plus a scalar offset (no per-lane 64-bit address math)
// and read zeros past `bytes` (range-checked by the hardware).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// The same load marked non-temporal (streamed once: kept from displacing
// data that is read again, such as Theta, in the caches).
__device__ __forceinline__ u32x4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                             uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
__device__ __forceinline__ u32x2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
}
__device__ __forceinline__ uint32_t buf_ld4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}
__device__ __forceinline__ uint32_t buf_ld2(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}

// ---- cross-half lane exchange ---------------------------------------------
// v_permlane32_swap: lanes 32..63 of x trade values with lanes 0..31 of y;
// lanes 0..31 of x and lanes 32..63 of y keep theirs.
__device__ __forceinline__ void swap_halves(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}

// ---- MFMA ------------------------------------------------------------------
// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l (g = l / 16, c = l % 16): A holds row c, k = 8g..8g+7; B holds
// column c, k = 8g..8g+7; D holds column c, rows 4g..4g+3. Any permutation
// of k applied to both A and B leaves D unchanged.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l (h = l / 32, c = l % 32): A holds row c, k = 8h..8h+7; B holds
// column c, k = 8h..8h+7; D element 4i+e holds row 8i + 4h + e of column c.
// On gfx950 this shape issues twice the flops per cycle of 16x16x32.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---- MFMA operand fragments from LDS (v_mfma_f32_32x32x16_bf16) -----------
// "P16" k-order: a 16-deep k-slice puts k = {4hh..4hh+3, 8+4hh..8+4hh+3} in
// lane half hh (hh = lane / 32). An accumulator tile's elements [8h, 8h+8)
// have exactly that order over its rows 16h..16h+15, so accumulators can be
// reused as operands; every other operand of such a product is read in P16
// order too.
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 lds_tr64(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>(
          reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(uint2, v);
}

// B-style fragment (column = lane % 32, k in P16 order) of the matrix
// M[k][col] stored row-major in LDS: rows kbase..kbase+15, columns
// cbase..cbase+31. Within each 16-lane group the transposing read hands lane
// q column q of 4 consecutive rows supplied by lanes q/4 + 4i.
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* base, int stride, int kbase, int cbase,
                                          int lane) {
  const int s = lane & 15, G = lane >> 4;
  const int row = kbase + 4 * (G >> 1) + (s >> 2);
  const int col = cbase + (G & 1) * 16 + 4 * (s & 3);
  const uint2 lo = lds_tr64(base + row * stride + col);
  const uint2 hi = lds_tr64(base + (row + 8) * stride + col);
  return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

// The same read with k in natural order (k = kbase + 8 * (lane / 32) + 0..7):
// the 4-row groups start 8 rows apart per lane half instead of 4, so this
// operand pairs with rows of the other operand read as 16 contiguous bytes.
__device__ __forceinline__ bf16x8 frag_tr_nat(const uint16_t* base, int stride, int kbase,
                                              int cbase, int lane) {
  const int s = lane & 15, G = lane >> 4;
  const int row = kbase + 8 * (G >> 1) + (s >> 2);
  const int col = cbase + (G & 1) * 16 + 4 * (s & 3);
  const uint2 lo = lds_tr64(base + row * stride + col);
  const uint2 hi = lds_tr64(base + (row + 4) * stride + col);
  return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

// A-style fragment with k in P16 order from row-major M[row][k] in LDS:
// row = rbase + lane % 32, k = kbase + {4hh..4hh+3, 8+4hh..8+4hh+3}.
__device__ __forceinline__ bf16x8 frag_p16(const uint16_t* base, int stride, int rbase, int kbase,
                                           int lane) {
  const uint16_t* p = base + (rbase + (lane & 31)) * stride + kbase + 4 * (lane >> 5);
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
  return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

// frag_p16 as two separate ds_read_b64. Two 8-byte reads from one base
// register are otherwise merged into one ds_read2_b64, which on gfx950 takes
// twice the LDS cycles of the two single reads (8 against 4 per wave, and 16
// against 8 when rows sit 16 or 48 bytes apart modulo 256). The empty asm
// statements emit nothing; their memory clobber keeps each read a separate
// instruction, since no access may be moved across them to pair with another.
__device__ __forceinline__ bf16x8 frag_p16_sep(const uint16_t* base, int stride, int rbase,
                                               int kbase, int lane) {
  const uint16_t* p = base + (rbase + (lane & 31)) * stride + kbase + 4 * (lane >> 5);
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  asm volatile("" ::: "memory");
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
  asm volatile("" ::: "memory");
  return as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
}

// Natural-order fragment (k = kbase + 8hh .. +7) of row-major M[row][k].
__device__ __forceinline__ bf16x8 frag_nat(const uint16_t* base, int stride, int rbase, int kbase,
                                           int lane) {
  return as_bf16x8(ld16(base + (rbase + (lane & 31)) * stride + kbase + 8 * (lane >> 5)));
}

// Accumulator elements [8h, 8h+8) of a fp32 tile as a bf16 operand (P16).
__device__ __forceinline__ bf16x8 acc_frag(const f32x16& t, int h) {
  return as_bf16x8(u32x4{pack_bf16x2(t[8 * h + 0], t[8 * h + 1]),
                         pack_bf16x2(t[8 * h + 2], t[8 * h + 3]),
                         pack_bf16x2(t[8 * h + 4], t[8 * h + 5]),
                         pack_bf16x2(t[8 * h + 6], t[8 * h + 7])});
}

// a if first else b, for two elements of one accumulator tile and a
// wave-uniform condition. The values pass through an empty asm first: a plain
// select between elements of one vector is rewritten into an indexed register
// read (M0-relative moves or a select chain over the whole tile).
__device__ __forceinline__ float pick(float a, float b, bool first) {
  asm volatile("" : "+v"(a), "+v"(b));
  return first ? a : b;
}


// ---- 8x8 bf16 transpose in registers --------------------------------------
// in[r] holds row r (8 bf16 = 4 dwords; dword w = elements 2w, 2w+1).
// out[c] receives column c (8 bf16: rows 0..7).
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = in[2 * q][w], hi = in[2 * q + 1][w];
      out[2 * w][q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      out[2 * w + 1][q] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
    }
  }
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace llops
