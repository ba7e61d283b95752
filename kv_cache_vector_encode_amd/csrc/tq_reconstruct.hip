// tq_reconstruct: dequantise cached vectors back to the original frame,
// x_hat = gamma16 * R^T c[codes] = gamma16 * D H c[codes] / sqrt(d)
// (Bit-Axon "TurboQuant: KV Cache Compression", dequantisation K_hat = DQ(K_q);
// deep-dive blog Step 2 decompress_key = magnitude * codebook direction).
//
// One vector per 16-lane row: lane L gathers the codes of coordinates
// 8*kPerm(L)+e so the FWHT leaves it holding output coordinates 8L..8L+7.

#include <hip/hip_bf16.h>

#include "tq_device.h"

namespace tq {

template <int BITS>
__global__ __launch_bounds__(256) void reconstruct_kernel(const ReconArgs a) {
  __shared__ float s_cent[16];
  const int tid = threadIdx.x;
  if (tid < 16) s_cent[tid] = a.centroid[tid];
  __syncthreads();
  const int L = tid & 15;
  const int64_t v = (int64_t)blockIdx.x * 16 + (tid >> 4);
  if (v >= a.n_vectors) return;   // whole rows leave together
  const int64_t H = a.num_heads;
  const uint32_t i = fast_div((uint32_t)v, a.div_heads);
  const int64_t h = v - (int64_t)i * H;
  const int32_t slot = a.slots[i];
  float* dst = a.out + v * kD + 8 * L;
  if (slot < 0 || slot >= a.num_slots) {
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = 0.f;
    return;
  }
  const uint8_t* base = a.pool + ((int64_t)(slot >> 4) * H + h) * a.block_bytes;
  const int row = slot & 15;
  const int ell = perm16(L);
  const uint32_t cw = load_codes8<BITS>(base + a.rec_off + (int64_t)row * a.rec_bytes, ell);
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = s_cent[(cw >> (BITS * e)) & ((1u << BITS) - 1)];
  const FwhtLane fc = fwht_lane(L);
  fwht_row(x, fc);
  const float g = load_half(base + a.norm_off + 2 * row) * fc.sig * kInvSqrtD;
  const uint32_t sb = sign_byte(a.rot, L);
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = flip(x[e] * g, sb, e);
}

int launch_reconstruct(const ReconArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t groups = (a.n_vectors + 15) / 16;
  if (groups > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  switch (a.bits) {
    case 2: hipLaunchKernelGGL(reconstruct_kernel<2>, dim3((unsigned)groups), dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(reconstruct_kernel<3>, dim3((unsigned)groups), dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(reconstruct_kernel<4>, dim3((unsigned)groups), dim3(256), 0, s, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// decompress_kernel: the same dequantisation for whole cache rows, keys and
// values in one launch (blockIdx.y picks the stream), written as 16-bit
// floats (round to nearest even) for attention over a compressed prefix.
// Every output vector is one 256-byte store per 16-lane row (16 bytes per
// lane); a workgroup takes kDecompVpr vectors per row, all loads issued first.
// Per vector it reads d*b/8 + 2 bytes and writes 256.
// ---------------------------------------------------------------------------
template <int OUT>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
  if constexpr (OUT == 2) {
    return (uint32_t)__builtin_bit_cast(unsigned short, __float2bfloat16(lo)) |
           ((uint32_t)__builtin_bit_cast(unsigned short, __float2bfloat16(hi)) << 16);
  } else {
    return (uint32_t)__half_as_ushort(__float2half_rn(lo)) | ((uint32_t)__half_as_ushort(__float2half_rn(hi)) << 16);
  }
}

template <int BITS, int OUT, int kDecompVpr>
__global__ __launch_bounds__(256) void decompress_kernel(const DecompArgs a) {
  const DecompStream& st = a.stream[blockIdx.y];
  __shared__ float s_cent[16];
  const int tid = threadIdx.x;
  const int L = tid & 15;
  const int ell = perm16(L);
  const int64_t H = a.num_heads;
  // ---- loads first: slots, then codes and norms of this row's vectors
  int64_t v[kDecompVpr];
  int32_t slot[kDecompVpr];
#pragma unroll
  for (int u = 0; u < kDecompVpr; ++u) {
    v[u] = ((int64_t)blockIdx.x * kDecompVpr + u) * 16 + (tid >> 4);
    const int64_t vc = v[u] < a.n_vectors ? v[u] : a.n_vectors - 1;
    slot[u] = a.slots[fast_div((uint32_t)vc, a.div_heads)];
  }
  uint32_t cw[kDecompVpr];
  float g[kDecompVpr];
#pragma unroll
  for (int u = 0; u < kDecompVpr; ++u) {
    const int64_t vc = v[u] < a.n_vectors ? v[u] : a.n_vectors - 1;
    const uint32_t i = fast_div((uint32_t)vc, a.div_heads);
    const int64_t h = vc - (int64_t)i * H;
    const bool ok = slot[u] >= 0 && slot[u] < a.num_slots;
    const int32_t sl = ok ? slot[u] : 0;   // invalid slots read slot 0; written as zeros
    const uint8_t* base = a.pool + ((int64_t)(sl >> 4) * H + h) * a.block_bytes;
    const int row = sl & 15;
    cw[u] = load_codes8<BITS>(base + st.rec_off + (int64_t)row * st.rec_bytes, ell);
    g[u] = ok ? load_half(base + st.norm_off + 2 * row) : 0.f;
  }
  if (tid < 16) s_cent[tid] = st.centroid[tid];
  __syncthreads();
  const FwhtLane fc = fwht_lane(L);
  const uint32_t sb = sign_byte(a.rot, L);
#pragma unroll
  for (int u = 0; u < kDecompVpr; ++u) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s_cent[(cw[u] >> (BITS * e)) & ((1u << BITS) - 1)];
    fwht_row(x, fc);   // every lane of the row takes part, also past the end
    const float gs = g[u] * fc.sig * kInvSqrtD;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack16<OUT>(flip(x[2 * e] * gs, sb, 2 * e), flip(x[2 * e + 1] * gs, sb, 2 * e + 1));
    if (v[u] < a.n_vectors) {
      // the output is written once and not read here: non-temporal stores
      // (measured 177.9 -> 171.7 us on every key and value of 16 x 8192 tokens)
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint8_t*>(st.out) + (v[u] * kD + 8 * L) * 2);
      __builtin_nontemporal_store((u32x4){w[0], w[1], w[2], w[3]}, dst);
    }
  }
}

// Vectors per 16-lane row: 4 below 2^20 vectors per stream, 8 from there
// (measured on keys and values of 2^18 vectors each: 46 us at 4 against 50
// at 8; of 2^20 each: 180 us at 4 against 170 at 8).
template <int BITS, int VPR>
static void launch_decomp_vpr(const DecompArgs& a, dim3 grid, hipStream_t s) {
  if (a.out_dtype == 2) hipLaunchKernelGGL((decompress_kernel<BITS, 2, VPR>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((decompress_kernel<BITS, 1, VPR>), grid, dim3(256), 0, s, a);
}

template <int BITS>
static void launch_decomp_bits(const DecompArgs& a, dim3 grid, int vpr, hipStream_t s) {
  if (vpr == 8) launch_decomp_vpr<BITS, 8>(a, grid, s);
  else launch_decomp_vpr<BITS, 4>(a, grid, s);
}

int launch_decompress(const DecompArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int vpr = a.n_vectors >= ((int64_t)1 << 20) ? 8 : 4;
  const int64_t groups = (a.n_vectors + 16 * vpr - 1) / (16 * vpr);
  if (groups > 0x7FFFFFFF || a.n_vectors >= ((int64_t)1 << 31)) return (int)hipErrorInvalidValue;
  // one launch per distinct bit width (keys and values share one when equal)
  DecompArgs b = a;
  int streams = 0;
  for (int k = 0; k < 2; ++k)
    if (a.stream[k].out) b.stream[streams++] = a.stream[k];
  if (streams == 0) return 0;
  const bool same = streams == 1 || b.stream[0].bits == b.stream[1].bits;
  for (int part = 0; part < (same ? 1 : 2); ++part) {
    DecompArgs c = b;
    if (!same) c.stream[0] = b.stream[part];
    const dim3 grid((unsigned)groups, (unsigned)(same ? streams : 1));
    switch (c.stream[0].bits) {
      case 2: launch_decomp_bits<2>(c, grid, vpr, s); break;
      case 3: launch_decomp_bits<3>(c, grid, vpr, s); break;
      case 4: launch_decomp_bits<4>(c, grid, vpr, s); break;
      default: return (int)hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace tq
