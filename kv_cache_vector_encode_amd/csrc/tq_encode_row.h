// Per-row pieces of the vector-unit encoder (one 128-d vector per 16-lane
// row, 8 coordinates per lane): signed loads, the bucketed threshold search
// and bit packing.  Shared by the encode kernels and the decode step that
// appends each sequence's new token before attending over it.
#pragma once

#include "tq_device.h"

namespace tq {

// 8 input coordinates of one lane with the rotation's sign flips applied
// through the raw bits: m[i] holds the sign masks of the i-th 32-bit word
// (bits 15 / 31 for two 16-bit inputs, bit 31 for one fp32 input).
template <int DT>
__device__ __forceinline__ void load8_signed(const void* base, int64_t elem, const uint32_t (&m)[8], float (&x)[8]) {
  if constexpr (DT == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
    const uint4 a = p[0], b = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(w[e] ^ m[e]);
  } else {
    const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {r.x ^ m[0], r.y ^ m[1], r.z ^ m[2], r.w ^ m[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == 2) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        x[2 * i] = __half2float(__ushort_as_half((unsigned short)(w[i] & 0xFFFFu)));
        x[2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(w[i] >> 16)));
      }
    }
  }
}

// Bucketed threshold search for one row (8 coordinates per lane): z = y_raw
// * zs + lut_off in bucket units, bucket = nearest integer to z clamped to
// [0, 255] by the conversion, code = base + (z > bucket threshold).
template <int BITS>
__device__ __forceinline__ void row_codes(const float (&x)[8], float zs, float lut_off, const uint2* s_lut,
                                          uint32_t (&code)[8]) {
  float z[8];
  uint32_t key4[2] = {0u, 0u};   // four bucket indices per word
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    z[e] = __builtin_fmaf(x[e], zs, lut_off);
    key4[e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(z[e], e & 3, key4[e >> 2]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint2 ent = s_lut[(key4[e >> 2] >> (8 * (e & 3))) & 0xFFu];
    code[e] = ent.y + (z[e] > __uint_as_float(ent.x) ? 1u : 0u);
  }
}

// Lane L of a row holds the codes of coordinates 8L..8L+7; every lane of the
// row takes part in the DPP exchanges.  Returns the 32-bit word this lane
// stores (if store_lane) at byte store_off of the vector's record.
template <int BITS>
__device__ __forceinline__ uint32_t row_pack(const uint32_t (&code)[8], int L, bool& store_lane, int& store_off) {
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) word |= code[e] << (BITS * e);
  store_lane = true;
  store_off = 4 * L;
  if constexpr (BITS == 2) {
    const uint32_t nb = dpp_u<kDppXor1>(word);
    store_lane = (L & 1) == 0;
    store_off = 2 * L;
    return word | (nb << 16);
  } else if constexpr (BITS == 3) {
    const uint32_t nb = dpp_u<kDppQuadNext>(word);
    const int q = L & 3;
    store_lane = q < 3;
    store_off = 12 * (L >> 2) + 4 * q;
    return (word >> (8 * q)) | (q < 3 ? nb << (24 - 8 * q) : 0u);
  }
  return word;
}

// 256-entry bucket table in threshold-search units (entries past lut_n
// repeat the last bucket, which holds no threshold).
__device__ __forceinline__ void fill_lut(uint2* s_lut, const CodecTables& tab, float lut_scale, float lut_off, int tid) {
  const int k = min(tid, tab.lut_n - 1);
  s_lut[tid] = make_uint2(__float_as_uint(__builtin_fmaf(tab.lut_thr[k], lut_scale, lut_off)),
                          (uint32_t)tab.lut_base[k]);
}

}  // namespace tq
