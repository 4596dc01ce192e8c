// Shared device helpers for the gfx950 MoE kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA 16x16x32 operand
typedef __attribute__((ext_vector_type(4))) float f32x4_t;     // MFMA 16x16 accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;  // 16-byte load
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

#define MOE_WAVE 64

namespace moe {

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 16) and B column (l % 16), 8 consecutive k
// values each; the k assignment only has to agree between A and B.  Lane l
// receives D[4*(l/16) + q][l % 16] for q = 0..3.
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two fp32 -> packed bf16 pair (lo in bits 0-15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Streaming (read-once) 16-byte load: non-temporal hint for weights.
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Rank-16 LoRA term of one 16 x 16 output tile, D[row][col] = sum_j
// P[row][j] Q[col][j] (fp32 adapters), as four fp32 MFMA 16x16x4 steps:
// lane (r, g) supplies P[row r][4g .. 4g+3] and Q[col r][4g .. 4g+3] (step c
// multiplies j = 4g + c) and receives D[4g + q][r], the accumulator layout of
// the bf16 16x16 tiles.  Every expert kernel (16-row and MFMA, bf16 and
// 4-bit) adds scale * D with this same sequence, so a row gets the same bits
// whichever kernel its batch size selects.
__device__ __forceinline__ f32x4_t lora_tile(f32x4_t prow, f32x4_t qrow) {
  f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) d = __builtin_amdgcn_mfma_f32_16x16x4f32(prow[c], qrow[c], d, 0, 0, 0);
  return d;
}

// Gathered token fragments (16 rows x 32 k of bf16) in LDS, as the LDS-tiled
// MFMA kernels fetch them row by row: slot 4p + c (16 bytes) holds k chunk
// xchunk(p, c) of row p, so lanes 4p .. 4p+3 of the copy read one 64-byte
// row segment.  xchunk(p, .) is an involution on 0..3 (c ^ s(p)), so chunk
// g of row r sits in slot 4r + xchunk(r, g) = xslot(lane) for the MFMA lane
// (r, g).  The 16-byte reads are served 8 lanes at a time; s(r) = bits 1, 2
// of r takes 4 distinct values over each 8 consecutive rows, so 8
// consecutive lanes of an operand read (8 rows, one chunk) cover 8 distinct
// 16-byte bank groups (no bank conflicts in the counters; a swizzle built
// for 16-lane groups showed 4 conflict cycles per read).
__device__ __forceinline__ int xchunk(int p, int c) { return c ^ ((p >> 1) & 3); }
__device__ __forceinline__ int xslot(int lane) {
  const int r = lane & 15, g = lane >> 4;
  return 4 * r + xchunk(r, g);
}

__device__ __forceinline__ f32x4_t ld4f(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }

// acc += scale * d, elementwise
__device__ __forceinline__ void add_scaled(f32x4_t& acc, f32x4_t d, float scale) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] += scale * d[q];
}

}  // namespace moe
