// tq_merge: second step of decode-attend.  The split kernels leave, for every
// (sequence, query head) and split of the sequence, the unnormalised
// rotated-frame output o_rot (128 floats), the split's running max m
// (natural-log units) and exp-sum l.  One workgroup per (sequence, query head)
// merges them in a fixed order (deterministic), normalises and rotates back:
// o = R^T o_rot / L = D H o_rot / (sqrt(d) L)  (Bit-Axon "TurboQuant: KV Cache
// Compression", attention softmax(Q K_hat^T / sqrt(d_h)) V_hat; deep-dive
// blog Step 1, the inverse of the orthogonal rotation is its transpose).
// A separate launch makes the partials visible with ordinary loads.

#include "tq_device.h"

namespace tq {

template <int U>
__global__ __launch_bounds__(256) void merge_kernel(const DecodeArgs a) {
  __shared__ float s_m[8], s_l[8];
  __shared__ float4 s_part[8][32];
  __shared__ float4 s_o[32];
  __shared__ float s_L;
  const int tid = threadIdx.x;
  const int hq = blockIdx.x, n = blockIdx.y;
  const int h = hq / a.group, g = hq - h * a.group;
  const int nsplit = a.num_splits;
  const int64_t stride = (int64_t)a.group * kPartStride;   // between splits
  const float* base = a.partials + ((int64_t)n * a.num_kv_heads + h) * nsplit * stride + (int64_t)g * kPartStride;

  // 1. thread (c4, sg) takes dims 4c4..4c4+3 of splits sg, sg+8, ...: U of
  // them per round (U covers the split count when it is at most 128), all
  // loads issued before any arithmetic (one memory round trip), then a local
  // max / weights / sums in registers
  {
    const int c4 = tid & 31, sg = tid >> 5;
    float M = -INFINITY, L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = sg; s0 < nsplit; s0 += 8 * U) {
      float ms[U], ls[U];
      float4 v[U];
      // unconditional loads (indices past the end re-read the last split and
      // are masked below): a branch per load would serialise them
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float* pp = base + min(s0 + 8 * u, nsplit - 1) * stride;
        const float2 ml = *reinterpret_cast<const float2*>(pp + 128);
        ms[u] = ml.x;
        ls[u] = s0 + 8 * u < nsplit ? ml.y : 0.f;
        v[u] = *reinterpret_cast<const float4*>(pp + 4 * c4);
      }
      float Mn = M;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ls[u] > 0.f) Mn = fmaxf(Mn, ms[u]);
      if (Mn == -INFINITY) continue;   // nothing in these splits yet
      const float r = M == -INFINITY ? 0.f : __expf(M - Mn);
      L *= r;
      o.x *= r; o.y *= r; o.z *= r; o.w *= r;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = ls[u] > 0.f ? __expf(ms[u] - Mn) : 0.f;
        L = __builtin_fmaf(ls[u], w, L);
        o.x = __builtin_fmaf(w, v[u].x, o.x);
        o.y = __builtin_fmaf(w, v[u].y, o.y);
        o.z = __builtin_fmaf(w, v[u].z, o.z);
        o.w = __builtin_fmaf(w, v[u].w, o.w);
      }
      M = Mn;
    }
    s_part[sg][c4] = o;
    if (c4 == 0) {
      s_m[sg] = M;
      s_l[sg] = L;
    }
  }
  __syncthreads();
  // 2. combine the 8 groups (in fixed order)
  if (tid < 32) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) M = fmaxf(M, s_m[k]);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = s_m[k] == -INFINITY ? 0.f : __expf(s_m[k] - M);
      const float4 v = s_part[k][tid];
      L = __builtin_fmaf(s_l[k], w, L);
      o.x = __builtin_fmaf(w, v.x, o.x);
      o.y = __builtin_fmaf(w, v.y, o.y);
      o.z = __builtin_fmaf(w, v.z, o.z);
      o.w = __builtin_fmaf(w, v.w, o.w);
    }
    s_o[tid] = o;
    if (tid == 0) s_L = L;
  }
  __syncthreads();
  const float L = s_L;

  // 3. normalise and rotate back in one 16-lane row
  if (tid >= 16) return;
  const int p = tid;
  const float invl = L > 0.f ? 1.f / L : 0.f;
  const float4 o0 = s_o[2 * p], o1 = s_o[2 * p + 1];
  float o[8] = {o0.x * invl, o0.y * invl, o0.z * invl, o0.w * invl,
                o1.x * invl, o1.y * invl, o1.z * invl, o1.w * invl};
  // natural input leaves lane p holding output lane perm16(p)
  const FwhtLane fc = fwht_lane(p);
  fwht_row(o, fc);
  const int lo = perm16(p);
  const uint32_t sb = sign_byte(a.rot, lo);
  float* dst = a.out + ((int64_t)n * a.num_q_heads + hq) * kD + 8 * lo;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = flip(o[e] * fc.sig * kInvSqrtD, sb, e);
}

int launch_merge(const DecodeArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)a.num_q_heads, (unsigned)a.num_seqs);
  const int per = (a.num_splits + 7) / 8;   // splits per thread group
  if (per <= 1) hipLaunchKernelGGL(merge_kernel<1>, grid, dim3(256), 0, s, a);
  else if (per <= 2) hipLaunchKernelGGL(merge_kernel<2>, grid, dim3(256), 0, s, a);
  else if (per <= 4) hipLaunchKernelGGL(merge_kernel<4>, grid, dim3(256), 0, s, a);
  else if (per <= 8) hipLaunchKernelGGL(merge_kernel<8>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<16>, grid, dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace tq
