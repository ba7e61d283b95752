// tq_minmax: the comparison codec of the deep-dive page's value path (Step 3
// compress_value / decompress_value): rotate the whole vector with the same
// seeded randomized Hadamard transform, y = R x; per vector lo = min_j y_j,
// scale = (max_j y_j - lo) / (2^b - 1), code_j = round half to even of
// (y_j - lo) / scale, fp16 scale and zero point.  Decoding forms
// code * scale + zero and applies R^T.  Built to measure against the
// Lloyd-Max codec (per-coordinate codebook and fp16 norm).
//
// One vector per 16-lane row, 8 coordinates per lane, the in-register
// 16-lane FWHT of the encoder.  The code decision is taken in fp32.

#include <hip/hip_bf16.h>

#include "tq_device.h"
#include "tq_encode_row.h"

namespace tq {

__device__ __forceinline__ float row_min(float v) { return -row_max(-v); }

// Codes of coordinates 8g .. 8g+7 from a flat record of 16 * BITS bytes.
// With 3-bit codes the 24 bits at byte 3g need a second dword only when
// they cross one (byte 3g mod 4 >= 2), and that dword is always inside the
// record, so nothing is read past the buffer's last record.
template <int BITS>
__device__ __forceinline__ uint32_t load_codes8_flat(const uint8_t* rec, int g) {
  if constexpr (BITS == 3) {
    const int byte = 3 * g, al = byte & ~3, sh = 8 * (byte & 3);
    const uint32_t lo = *reinterpret_cast<const uint32_t*>(rec + al);
    const uint32_t hi = sh > 8 ? *reinterpret_cast<const uint32_t*>(rec + al + 4) : 0u;
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> sh) & 0xFFFFFFu;
  } else {
    return load_codes8<BITS>(rec, g);
  }
}

template <int BITS, int DT>
__global__ __launch_bounds__(256) void minmax_encode_kernel(const MinmaxArgs a) {
  const int tid = threadIdx.x;
  const int L = tid & 15, ell = perm16(L);
  const int64_t v = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const int64_t vc = v < a.n ? v : a.n - 1;   // past the end: recompute the last vector, store nothing
  const uint32_t sneg = sign_byte(a.rot, ell);
  uint32_t smask[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (DT == 0) smask[i] = ((sneg >> i) & 1u) << 31;
    else smask[i] = i < 4 ? (((sneg >> (2 * i)) & 1u) << 15) | (((sneg >> (2 * i + 1)) & 1u) << 31) : 0u;
  }
  float x[8];
  load8_signed<DT>(a.src, vc * kD + 8 * ell, smask, x);
  const FwhtLane fc = fwht_lane(L);
  fwht_row(x, fc);   // lane L now holds coordinates 8L..8L+7 (times fc.sig * sqrt(d))
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] *= fc.sig * kInvSqrtD;
    lo = fminf(lo, x[e]);
    hi = fmaxf(hi, x[e]);
  }
  lo = row_min(lo) + 0.f;   // + 0: a zero vector's sign flips leave -0, stored as +0
  hi = row_max(hi);
  constexpr int kLevels = (1 << BITS) - 1;
  const float scale = (hi - lo) / (float)kLevels;
  // (y - lo) / scale as a product with the hardware reciprocal (1 ulp): it
  // differs from the page's division only within a few ulps of a rounding
  // tie, and the row's 8 divisions were most of the kernel's vector work
  const float inv = scale > 0.f ? __builtin_amdgcn_rcpf(scale) : 0.f;
  uint32_t code[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float u = (x[e] - lo) * inv;
    code[e] = (uint32_t)fminf(fmaxf(rintf(u), 0.f), (float)kLevels);
  }
  bool store_lane;
  int store_off;
  const uint32_t word = row_pack<BITS>(code, L, store_lane, store_off);
  if (v < a.n) {
    if (store_lane) *reinterpret_cast<uint32_t*>(a.codes + v * (16 * BITS) + store_off) = word;
    if (L == 0) {
      const uint32_t s16 = __half_as_ushort(__float2half_rn(fminf(scale, 65504.f)));
      const uint32_t z16 = __half_as_ushort(__float2half_rn(fminf(fmaxf(lo, -65504.f), 65504.f)));
      *reinterpret_cast<uint32_t*>(a.params + 2 * v) = s16 | (z16 << 16);
    }
  }
}

template <int BITS, int OUT>
__global__ __launch_bounds__(256) void minmax_decode_kernel(const MinmaxArgs a) {
  const int tid = threadIdx.x;
  const int L = tid & 15, ell = perm16(L);
  const int64_t v = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const int64_t vc = v < a.n ? v : a.n - 1;
  const uint32_t cw = load_codes8_flat<BITS>(a.codes + vc * (16 * BITS), ell);
  const uint32_t p = *reinterpret_cast<const uint32_t*>(a.params + 2 * vc);
  const float s = __half2float(__ushort_as_half((unsigned short)(p & 0xFFFFu)));
  const float z = __half2float(__ushort_as_half((unsigned short)(p >> 16)));
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf((float)((cw >> (BITS * e)) & ((1u << BITS) - 1)), s, z);
  const FwhtLane fc = fwht_lane(L);
  fwht_row(x, fc);
  const float g = fc.sig * kInvSqrtD;
  const uint32_t sb = sign_byte(a.rot, L);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = flip(x[e] * g, sb, e);
  if (v >= a.n) return;   // after the row's exchanges
  if constexpr (OUT == 0) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + v * kD + 8 * L);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
  } else {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (OUT == 2)
        w[e] = (uint32_t)__builtin_bit_cast(unsigned short, __float2bfloat16(o[2 * e])) |
               ((uint32_t)__builtin_bit_cast(unsigned short, __float2bfloat16(o[2 * e + 1])) << 16);
      else
        w[e] = (uint32_t)__half_as_ushort(__float2half_rn(o[2 * e])) |
               ((uint32_t)__half_as_ushort(__float2half_rn(o[2 * e + 1])) << 16);
    }
    // written once, not read here: non-temporal stores (measured 39.0 -> 34.6 us
    // on 2^18 vectors, 194 -> 148 us on 2^20)
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store((u32x4){w[0], w[1], w[2], w[3]},
                                reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.out) + (v * kD + 8 * L) * 2));
  }
}

template <int BITS>
static void enc_bits(const MinmaxArgs& a, dim3 grid, hipStream_t s) {
  if (a.in_dtype == 0) hipLaunchKernelGGL((minmax_encode_kernel<BITS, 0>), grid, dim3(256), 0, s, a);
  else if (a.in_dtype == 1) hipLaunchKernelGGL((minmax_encode_kernel<BITS, 1>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((minmax_encode_kernel<BITS, 2>), grid, dim3(256), 0, s, a);
}

template <int BITS>
static void dec_bits(const MinmaxArgs& a, dim3 grid, hipStream_t s) {
  if (a.out_dtype == 0) hipLaunchKernelGGL((minmax_decode_kernel<BITS, 0>), grid, dim3(256), 0, s, a);
  else if (a.out_dtype == 1) hipLaunchKernelGGL((minmax_decode_kernel<BITS, 1>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((minmax_decode_kernel<BITS, 2>), grid, dim3(256), 0, s, a);
}

int launch_minmax_encode(const MinmaxArgs& a, int bits, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t groups = (a.n + 15) / 16;
  if (a.n <= 0 || groups > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)groups);
  switch (bits) {
    case 2: enc_bits<2>(a, grid, s); break;
    case 3: enc_bits<3>(a, grid, s); break;
    case 4: enc_bits<4>(a, grid, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_minmax_decode(const MinmaxArgs& a, int bits, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t groups = (a.n + 15) / 16;
  if (a.n <= 0 || groups > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)groups);
  switch (bits) {
    case 2: dec_bits<2>(a, grid, s); break;
    case 3: dec_bits<3>(a, grid, s); break;
    case 4: dec_bits<4>(a, grid, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace tq
