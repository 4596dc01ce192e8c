// 4-bit blockwise weights: the code-pair table and the per-lane loads shared
// by the 16-row and the LDS-tiled 4-bit expert kernels (internal to the
// library).
#pragma once
#include "common.hpp"

namespace moe {

// A weight is codebook[code] * absmax(row, 64-block), the codebook holding
// 16 fp32 values.  Each entry enters the MFMA as two bf16 parts, hi =
// RNE(cb) and lo = RNE(cb - hi) (cb - hi is exact in fp32), so the operand
// hi + lo carries cb to within 2^-18 of its magnitude (17 significant bits
// where a single bf16 holds 8): a bf16-valued entry has lo = 0 and enters
// exactly.  Here the tokens are the MFMA A operand and the weights the B
// operand, D[token][weight row], so a lane's four outputs all belong to its
// own weight row and the absmax is applied to MFMA partial sums: each 32-k
// MFMA step lies in one 64-block (steps 0,1 of a 128-k block use block 2kb,
// steps 2,3 block 2kb+1), and
//   D[t][row] = sum_h absmax(row, h) * sum_{k in h} x[t][k] (lo[code] + hi[code])
// (the lo products are accumulated first, then the hi ones, into one fp32
// accumulator).  The per-weight work is one 8-byte table read per two codes:
// entry b of the table holds the packed bf16 pairs (hi[b & 15], hi[b >> 4])
// and (lo[b & 15], lo[b >> 4]) of code byte b.  The table is held kLutRep
// times over (copy c of entry b at entry b * kLutRep + c) and lane l reads
// copy l % kLutRep, so within each group of kLutRep consecutive lanes the
// reads land in distinct LDS banks whatever bytes they look up (one shared
// copy puts several lanes of each read in one bank: random code bytes over
// 64 lanes); lanes kLutRep apart share a copy and can still collide.
//
// Lane (g, r) feeds token row r and weight row r, k = 128kb + 32st + 8g + 0..7
// for step st = 0..3 (dword st of its 16-byte chunk in the tiled layout; four
// 4-byte loads from a row-major row), and receives D[token 4g + q][row r].

#ifndef MOE_LUT_REP
#define MOE_LUT_REP 16
#endif
constexpr int kLutRep = MOE_LUT_REP;  // copies of the code-pair table
static_assert((kLutRep & (kLutRep - 1)) == 0 && kLutRep <= 32, "table copies");

// thread tid < 256 writes every copy of entry tid, starting at copy
// tid % kLutRep so that the lanes of each store fall in distinct banks
__device__ __forceinline__ void build_lut(u32x2_t* s_lut, const float* cb, int tid) {
  if (tid < 256) {
    const float c0 = cb[tid & 15], c1 = cb[tid >> 4];
    const uint32_t hi = pack_bf16x2(c0, c1);
    const u32x2_t v = {hi, pack_bf16x2(c0 - bf16lo(hi), c1 - bf16hi(hi))};
#pragma unroll 8
    for (int c = 0; c < kLutRep; ++c) s_lut[tid * kLutRep + ((c + tid) & (kLutRep - 1))] = v;
  }
}

// this lane's copy of the table
__device__ __forceinline__ const u32x2_t* lut_copy(const u32x2_t* s_lut, int lane) {
  return s_lut + (lane & (kLutRep - 1));
}

// 8 codes (one dword, element 2i in the low nibble of byte i) -> the hi and
// lo parts of their 8 entries, read from the lane's copy of the table
__device__ __forceinline__ void lut8(const u32x2_t* s_lutl, uint32_t w, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x2_t v = s_lutl[((w >> (8 * i)) & 0xffu) * kLutRep];
    hi[i] = v[0];
    lo[i] = v[1];
  }
}

// codes of one 128-k block for this lane: tiled = one 16-byte chunk,
// row-major = dwords 16kb + 4st + g of the row
template <bool TILED>
__device__ __forceinline__ u32x4_t load_codes(const uint8_t* q, int kb, int g) {
  if (TILED) return ld16_stream(q + (size_t)kb * 1024);
  const uint32_t* d = reinterpret_cast<const uint32_t*>(q) + 16 * kb + g;
  return u32x4_t{d[0], d[4], d[8], d[12]};
}

// absmax of this lane's weight row for the two 64-blocks of 128-k block kb
// (tiled: floats kb*32 + 2r, +1 of the row tile; row-major: 2kb, 2kb+1)
template <bool TILED>
__device__ __forceinline__ u32x2_t load_scales(const float* s, int kb) {
  return *reinterpret_cast<const u32x2_t*>(s + (size_t)kb * (TILED ? 32 : 2));
}

}  // namespace moe
