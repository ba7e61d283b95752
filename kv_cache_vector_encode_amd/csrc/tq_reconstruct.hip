// tq_reconstruct: dequantise cached vectors back to the original frame,
// x_hat = gamma16 * R^T c[codes] = gamma16 * D H c[codes] / sqrt(d)
// (Bit-Axon "TurboQuant: KV Cache Compression", dequantisation K_hat = DQ(K_q);
// deep-dive blog Step 2 decompress_key = magnitude * codebook direction).
//
// One vector per 16-lane row: lane L gathers the codes of coordinates
// 8*kPerm(L)+e so the FWHT leaves it holding output coordinates 8L..8L+7.

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

}  // namespace tq
