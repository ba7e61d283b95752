// tq_merge: second step of decode-attend.  The split kernels leave, for every
// (sequence, query head) and split of the sequence, the unnormalised
// rotated-frame output o_rot (128 floats), the split's running max m
// (natural-log units) and exp-sum l.  One workgroup per (sequence, query head)
// merges them in split order (deterministic), normalises and rotates back:
// o = R^T o_rot / L = D H o_rot / (sqrt(d) L)  (Bit-Axon "TurboQuant: KV Cache
// Compression", attention softmax(Q K_hat^T / sqrt(d_h)) V_hat; deep-dive
// blog Step 1, the inverse of the orthogonal rotation is its transpose).
// A separate launch makes the partials visible with ordinary loads.

#include "tq_device.h"

namespace tq {

__global__ __launch_bounds__(256) void merge_kernel(const DecodeArgs a) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[2][8];
  __shared__ float4 s_part[8][32];
  __shared__ float4 s_o[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hq = blockIdx.x, n = blockIdx.y;
  const int h = hq / a.group, g = hq - h * a.group;
  const int nsplit = a.num_splits;
  const int64_t stride = (int64_t)a.group * kPartStride;   // between splits
  const float* base = a.partials + ((int64_t)n * a.num_kv_heads + h) * nsplit * stride + (int64_t)g * kPartStride;

  // 1. running max M and total L over the splits
  float M = -INFINITY;
  for (int s = tid; s < nsplit; s += 256) {
    const float* pp = base + s * stride;
    if (pp[129] > 0.f) M = fmaxf(M, pp[128]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) s_red[0][wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  float L = 0.f;
  for (int s = tid; s < nsplit; s += 256) {
    const float* pp = base + s * stride;
    const float l = pp[129];
    const float w = l > 0.f ? __expf(pp[128] - M) : 0.f;
    s_w[s] = w;
    L = __builtin_fmaf(l, w, L);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
  if (lane == 0) s_red[1][wave] = L;
  __syncthreads();
  L = s_red[1][0] + s_red[1][1] + s_red[1][2] + s_red[1][3];

  // 2. weighted sum of o_rot: thread -> (4 dims c4, every 8th split from sg)
  {
    const int c4 = tid & 31, sg = tid >> 5;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = sg;
    for (; s + 24 < nsplit; s += 32) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float4*>(base + (s + 8 * u) * stride + 4 * c4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = s_w[s + 8 * u];
        o.x = __builtin_fmaf(w, v[u].x, o.x);
        o.y = __builtin_fmaf(w, v[u].y, o.y);
        o.z = __builtin_fmaf(w, v[u].z, o.z);
        o.w = __builtin_fmaf(w, v[u].w, o.w);
      }
    }
    for (; s < nsplit; s += 8) {
      const float4 v = *reinterpret_cast<const float4*>(base + s * stride + 4 * c4);
      const float w = s_w[s];
      o.x = __builtin_fmaf(w, v.x, o.x);
      o.y = __builtin_fmaf(w, v.y, o.y);
      o.z = __builtin_fmaf(w, v.z, o.z);
      o.w = __builtin_fmaf(w, v.w, o.w);
    }
    s_part[sg][c4] = o;
  }
  __syncthreads();
  if (tid < 32) {
    float4 o = s_part[0][tid];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      const float4 v = s_part[k][tid];
      o.x += v.x; o.y += v.y; o.z += v.z; o.w += v.w;
    }
    s_o[tid] = o;
  }
  __syncthreads();

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
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)a.num_q_heads, (unsigned)a.num_seqs), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace tq
