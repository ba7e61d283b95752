// Device helpers shared by the gfx950 kernels: DPP lane exchanges, the
// 128-point Walsh-Hadamard transform held in one 16-lane row, row reductions
// and small load/convert helpers.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

// DPP controls (CDNA): quad_perm [1,0,3,2] = lane^1, [2,3,0,1] = lane^2,
// row_half_mirror = lane^7 inside 8-lane halves, row_mirror = lane^15 inside
// a 16-lane row, quad_perm [1,2,3,3] = next lane of the quad (last repeats).
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppQuadNext = 0xF9;
constexpr int kDppRor8 = 0x128;     // row_ror:8

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// ---------------------------------------------------------------------------
// FWHT-128 in one 16-lane row, 8 elements per lane.
//
// Three butterfly stages run inside the lane (element bits 1, 2, 4).  Four run
// across lanes along the xor masks 1, 2, 7, 15, which DPP provides directly
// (quad_perm, quad_perm, row_half_mirror, row_mirror).  Those masks form a
// basis of the 4-bit lane index, so the row computes a Walsh-Hadamard
// transform in the virtual lane coordinates v = A^{-1} L (A = [1 2 7 15]).
// Each cross-lane stage is one fma per element, new = own + m * partner, with
// m = +-1 per lane; this leaves each lane's values multiplied by a known sign
// sig(L) (the "upper" lane of every butterfly ends up negated).
//
// Loading lane L with the input coordinates 8*kPerm(L) + e makes the output
// come out in natural Sylvester order: lane L holds (H x)_{8L+e} * sig(L).
// Loading natural input (lane L holds 8L+e) leaves lane L holding output
// lane kPerm(L), i.e. (H x)_{8*kPerm(L)+e} * sig(L).
// kPerm (as nibbles, lane 0 lowest), the per-stage negative-multiplier masks
// and the final sign mask follow from A by GF(2) algebra; they were checked by
// a host model of this exact data flow against a dense Hadamard matrix.
constexpr uint64_t kPerm = 0x8DEB7214C9AF3650ull;
constexpr uint32_t kStageNeg0 = 0x5A5A, kStageNeg1 = 0x3C3C, kStageNeg2 = 0x0FF0,
                   kStageNeg3 = 0xFF00, kSigNeg = 0x9696;

__device__ __forceinline__ int perm16(int L) { return (int)((kPerm >> (4 * L)) & 15); }

struct FwhtLane {
  float m0, m1, m2, m3, sig;
};

__device__ __forceinline__ FwhtLane fwht_lane(int L) {
  auto pm = [L](uint32_t neg) { return ((neg >> L) & 1u) ? -1.0f : 1.0f; };
  return {pm(kStageNeg0), pm(kStageNeg1), pm(kStageNeg2), pm(kStageNeg3), pm(kSigNeg)};
}

// x[e] += m * x[e] of the partner lane, for 8 elements: one v_fmac_f32_dpp
// each.  (The compiler does not fold a DPP move into a tied-operand fmac, so
// the stage is written out.)  The leading s_nop 1 provides the two wait
// states the hardware needs between a VALU write of a VGPR and a DPP read of
// it; inside the block every DPP source was written at least 7 instructions
// earlier or not at all.
#define TQ_FMAC_DPP8(CTRL)                                                        \
  asm("s_nop 1\n"                                                                 \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"           \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"           \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"           \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"           \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"           \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"           \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"           \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"           \
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),   \
        "+v"(x[6]), "+v"(x[7])                                                     \
      : "v"(m))

template <int STAGE>
__device__ __forceinline__ void fmac_dpp8(float (&x)[8], float m) {
  if constexpr (STAGE == 0) TQ_FMAC_DPP8("quad_perm:[1,0,3,2]");
  else if constexpr (STAGE == 1) TQ_FMAC_DPP8("quad_perm:[2,3,0,1]");
  else if constexpr (STAGE == 2) TQ_FMAC_DPP8("row_half_mirror");
  else TQ_FMAC_DPP8("row_mirror");
}

// All 16 lanes of the row must execute this together.
__device__ __forceinline__ void fwht_row(float (&x)[8], const FwhtLane& c) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!(e & h)) {
        const float a = x[e], b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
    }
  }
  fmac_dpp8<0>(x, c.m0);
  fmac_dpp8<1>(x, c.m1);
  fmac_dpp8<2>(x, c.m2);
  fmac_dpp8<3>(x, c.m3);
}

// Sum / max over the 16 lanes of a row; every lane receives the result.
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return v;
}
// Sum / max over the four 16-lane rows (lanes j, j + 16, j + 32, j + 48);
// every lane receives the result.  permlane16/32_swap exchange rows on the
// vector ALU: with both operands v, the two results hold v of the lane and
// of its partner 16 (32) lanes away, in some order.
__device__ __forceinline__ float sum_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float w = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t uw = __float_as_uint(w);
  const auto b = __builtin_amdgcn_permlane32_swap(uw, uw, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float max_rows(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float w = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t uw = __float_as_uint(w);
  const auto b = __builtin_amdgcn_permlane32_swap(uw, uw, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

// Sign-flip masks (bit 31) for the 8 coordinates 8*g .. 8*g+7 of a SignMask.
__device__ __forceinline__ uint32_t sign_byte(const SignMask& m, int g) {
  return (m.neg[g >> 2] >> (8 * (g & 3))) & 0xFFu;
}
__device__ __forceinline__ float flip(float v, uint32_t byte, int e) {
  return __uint_as_float(__float_as_uint(v) ^ (((byte >> e) & 1u) << 31));
}

// Load 8 consecutive elements of dtype (0 f32, 1 f16, 2 bf16) as floats.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&x)[8]) {
  if constexpr (DT == 0) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == 2) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      } else {
        x[2 * i] = __half2float(__ushort_as_half((unsigned short)(w[i] & 0xFFFF)));
        x[2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(w[i] >> 16)));
      }
    }
  }
}

// The b-bit codes of coordinates 8*g .. 8*g+7 of a code record.
template <int BITS>
__device__ __forceinline__ uint32_t load_codes8(const uint8_t* rec, int g) {
  if constexpr (BITS == 4) {
    return *reinterpret_cast<const uint32_t*>(rec + 4 * g);
  } else if constexpr (BITS == 2) {
    return *reinterpret_cast<const uint16_t*>(rec + 2 * g);
  } else {
    // 24 bits at byte 3g: two aligned dwords and a funnel shift.  The second
    // dword can run past the record end; it stays inside the (block, head)
    // chunk because other regions always follow the code regions.
    const int byte = 3 * g, al = byte & ~3, sh = 8 * (byte & 3);
    const uint32_t lo = *reinterpret_cast<const uint32_t*>(rec + al);
    const uint32_t hi = *reinterpret_cast<const uint32_t*>(rec + al + 4);
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> sh) & 0xFFFFFFu;
  }
}

__device__ __forceinline__ float load_half(const uint8_t* p) {
  return __half2float(__ushort_as_half(*reinterpret_cast<const unsigned short*>(p)));
}

// floor(n / d) for 0 <= n < 2^31 with a host-computed multiplier
// (Granlund-Montgomery: l = ceil(log2 d), m = ceil(2^(31+l) / d),
// q = (n * m) >> (31 + l)).
__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)n * f.mul) >> f.shift);
}

constexpr float kInvSqrtD = 0.08838834764831845f;   // 1/sqrt(128)
constexpr float kSqrtHalfPi = 1.2533141373155003f;  // sqrt(pi/2)

}  // namespace tq
