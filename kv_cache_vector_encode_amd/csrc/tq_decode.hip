// tq_decode: attention of one decode query per sequence over the compressed
// paged cache, computed in the rotated frame, plus the keys-only logits path.
//
// Method: Bit-Axon "TurboQuant: KV Cache Compression", attention under
// quantisation softmax(Q K_hat^T / sqrt(d_h)) V_hat; deep-dive blog Step 1
// (the rotation is orthogonal, so inner products and hence attention scores
// can be taken in the rotated frame without undoing it first); OCTOPUS
// summary contributions (the decoder never materialises K_hat; the optional
// QJL residual adds a correction to q^T k_hat).
//
// In the rotated frame <q, k_hat_t> = gamma_t <R q, c[codes_t]>, so q is
// rotated once, every logit is a centroid-lookup dot product, and the value
// sum o_rot = sum_t p_t gamma_v,t c[codes_v,t] is rotated back once:
// o = R^T o_rot = D H o_rot / sqrt(d).
//
// Grid: (split, kv-head slice, sequence).  A workgroup (256 threads = 16 rows
// of 16 lanes) owns up to 8 query heads of one KV head and a contiguous range
// of blocks of one sequence.  Lane p of a row handles coordinates 8p..8p+7.
//   A. logits: each row takes one token at a time; per-lane partial dot
//      products are summed over the row with DPP; scores go to LDS.
//   B. per head: max and exp-sum over the split (one row per head).
//   C. values: each row accumulates p_t * gamma_v * c[codes] for its tokens.
//   D. rows are reduced (shuffles inside a wave, LDS across waves) and the
//      split's (m, l, o_rot) goes to the workspace; merge_kernel
//      (tq_merge.hip), a second launch, combines the splits in a fixed order
//      (deterministic results), applies R^T and writes the output.

#include "tq_device.h"

namespace tq {

constexpr int kMaxSplitTokens = 1024;

template <int DT>
__device__ __forceinline__ void load_q8(const DecodeArgs& a, int64_t elem, float (&x)[8]) {
  load8<DT>(a.q, elem, x);
}

template <int BK, int BV, bool QJL, int GMAX, bool ATTEND>
__global__ __launch_bounds__(256) void decode_kernel(const DecodeArgs a, int ns, int gs) {
  __shared__ float s_q[GMAX][kD];
  __shared__ float s_w[QJL ? GMAX : 1][kD];
  __shared__ float s_ck[16];
  __shared__ float s_cv[16];
  __shared__ float s_p[ATTEND ? kMaxSplitTokens * GMAX : 1];
  __shared__ float s_ml[2][GMAX];
  __shared__ float s_red[ATTEND ? 4 : 1][GMAX][kD];
  __shared__ int s_bt[kMaxSplitTokens / kBlock];   // the split's blocks, clamped into the pool

  const int tid = threadIdx.x;
  const int r = tid >> 4, p = tid & 15;
  const int split = blockIdx.x, unit = blockIdx.y, n = blockIdx.z;
  const int h = unit / ns, slice = unit - h * ns;
  const int g0 = slice * gs;
  const int gcount = min(gs, a.group - g0);
  const int seq_len = max(0, min(a.seq_lens[n], a.max_blocks * kBlock));
  const int t0 = split * a.blocks_per_split * kBlock;
  const int t1 = min(seq_len, t0 + a.blocks_per_split * kBlock);
  const FwhtLane fc = fwht_lane(p);
  const int64_t Hq = a.num_q_heads;

  if (tid < 16) {
    s_ck[tid] = a.cent_k[tid];
    s_cv[tid] = a.cent_v[tid];
  }
  const int32_t* btab = a.block_tables + (int64_t)n * a.max_blocks;
  const int nb = t1 > t0 ? (t1 - t0 + kBlock - 1) / kBlock : 0;   // t0 is a block multiple
  for (int i = tid; i < nb; i += 256) {
    const int b = btab[t0 / kBlock + i];
    s_bt[i] = (b >= 0 && b < a.num_blocks) ? b : 0;
  }

  // ---- D0: rotate this slice's queries, q_rot = H D q / sqrt(d) (and R' q_rot)
  if (r < gcount) {
    const int64_t hq = (int64_t)h * a.group + g0 + r;
    const int ell = perm16(p);
    float x[8];
    const int64_t elem = ((int64_t)n * Hq + hq) * kD + 8 * ell;
    if (a.q_dtype == 0) load_q8<0>(a, elem, x);
    else if (a.q_dtype == 1) load_q8<1>(a, elem, x);
    else load_q8<2>(a, elem, x);
    const uint32_t sb = sign_byte(a.rot, ell);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = flip(x[e], sb, e);
    fwht_row(x, fc);
    const float sc = fc.sig * kInvSqrtD;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] *= sc;
      s_q[r][8 * p + e] = x[e];
    }
    if constexpr (QJL) {
      const uint32_t qb = sign_byte(a.rot_qjl, p);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = flip(x[e], qb, e);
      fwht_row(x, fc);
      const int lo = perm16(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) s_w[r][8 * lo + e] = x[e] * sc;
    }
  }
  __syncthreads();

  float qreg[GMAX][8];
  float wreg[QJL ? GMAX : 1][8];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qreg[g][e] = g < gcount ? s_q[g][8 * p + e] : 0.f;
      if constexpr (QJL) wreg[g][e] = g < gcount ? s_w[g][8 * p + e] : 0.f;
    }

  const int64_t Hkv = a.num_kv_heads;
  // Rows take token row r of the split's blocks in turn, kU blocks at a
  // time with every load of the batch issued before the first use (a loop
  // that loads and uses one token at a time waits out a memory round trip
  // per token); blocks past the split's end re-read its last block and are
  // not used
  constexpr int kU = 4;
  auto blk_base = [&](int i) {
    return a.pool + ((int64_t)s_bt[min(i, nb - 1)] * Hkv + h) * a.lay.block_bytes;
  };

  // ---- A: logits
  for (int i0 = 0; i0 < nb; i0 += kU) {
    uint32_t cwb[kU], sbb[kU];
    unsigned short gkb[kU], rhb[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint8_t* base = blk_base(i0 + u);
      cwb[u] = load_codes8<BK>(base + a.lay.off_k + (int64_t)r * a.lay.k_rec, p);
      gkb[u] = *reinterpret_cast<const unsigned short*>(base + a.lay.off_gk + 2 * r);
      if constexpr (QJL) {
        sbb[u] = base[a.lay.off_sign + r * 16 + p];
        rhb[u] = *reinterpret_cast<const unsigned short*>(base + a.lay.off_rho + 2 * r);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
    const int tok = t0 + (i0 + u) * kBlock + r;
    if (i0 + u >= nb || tok >= t1) break;   // uniform across rows but for the last block
    const uint32_t cw = cwb[u];
    float c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = s_ck[(cw >> (BK * e)) & ((1u << BK) - 1)];
    const float gk = __half2float(__ushort_as_half(gkb[u]));
    float qj_rho = 0.f;
    uint32_t sbits = 0;
    if constexpr (QJL) {
      sbits = sbb[u];
      qj_rho = __half2float(__ushort_as_half(rhb[u])) * (kSqrtHalfPi * kInvSqrtD);
    }
    // the residual estimate's weights +-tau rho of this token's 8 sign bits,
    // shared by every head: it joins the lane's part of the logit before the
    // row sum (one 16-lane sum per head instead of two)
    [[maybe_unused]] float cs[8];
    if constexpr (QJL) {
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[e] = flip(qj_rho, sbits, e);
    }
    float mine = 0.f;
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(c[e], qreg[g][e], dot);
      if constexpr (QJL) {
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(cs[e], wreg[g][e], dot);
      }
      const float sg = a.scale * gk * row_sum(dot);
      if (p == g) mine = sg;
    }
    if (p < gcount) {
      if (a.logits)
        a.logits[((int64_t)n * Hq + (int64_t)h * a.group + g0 + p) * a.logits_stride + tok] = mine;
      if constexpr (ATTEND) s_p[(tok - t0) * GMAX + p] = mine;
    }
    }
  }
  if constexpr (!ATTEND) return;
  __syncthreads();

  // ---- B: per-head max / exp-sum over the split
  const int ntok = max(0, t1 - t0);
  if (r < gcount) {
    float m = -INFINITY;
    for (int t = p; t < ntok; t += 16) m = fmaxf(m, s_p[t * GMAX + r]);
    m = row_max(m);
    float l = 0.f;
    for (int t = p; t < ntok; t += 16) {
      const float e = __expf(s_p[t * GMAX + r] - m);
      s_p[t * GMAX + r] = e;
      l += e;
    }
    l = row_sum(l);
    if (p == 0) {
      s_ml[0][r] = m;
      s_ml[1][r] = l;
    }
  }
  __syncthreads();

  // ---- C: values
  float acc[GMAX][8];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  for (int i0 = 0; i0 < nb; i0 += kU) {
    uint32_t cwb[kU];
    unsigned short gvb[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint8_t* base = blk_base(i0 + u);
      cwb[u] = load_codes8<BV>(base + a.lay.off_v + (int64_t)r * a.lay.v_rec, p);
      gvb[u] = *reinterpret_cast<const unsigned short*>(base + a.lay.off_gv + 2 * r);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
    const int tok = t0 + (i0 + u) * kBlock + r;
    if (i0 + u >= nb || tok >= t1) break;
    const uint32_t cw = cwb[u];
    const float gv = __half2float(__ushort_as_half(gvb[u]));
    float c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = s_cv[(cw >> (BV * e)) & ((1u << BV) - 1)];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      const float pw = s_p[(tok - t0) * GMAX + g] * gv;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = __builtin_fmaf(pw, c[e], acc[g][e]);
    }
    }
  }

  // ---- D: reduce the 16 rows (4 per wave, then 4 waves)
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[g][e] = sum_rows(acc[g][e]);
    }
  const int wave = tid >> 6;
  if ((tid & 63) < 16) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_red[wave][g][8 * p + e] = acc[g][e];
  }
  __syncthreads();
  const int64_t nsplit = a.num_splits;
  float* part_base = a.partials + (((int64_t)n * Hkv + h) * nsplit) * a.group * kPartStride;
  for (int i = tid; i < gcount * kD; i += 256) {
    const int g = i / kD, j = i - g * kD;
    const float v = s_red[0][g][j] + s_red[1][g][j] + s_red[2][g][j] + s_red[3][g][j];
    part_base[((int64_t)split * a.group + g0 + g) * kPartStride + j] = v;
  }
  if (tid < gcount) {
    float* pp = part_base + ((int64_t)split * a.group + g0 + tid) * kPartStride;
    pp[128] = s_ml[0][tid];
    pp[129] = s_ml[1][tid];
  }

}

template <int BK, int BV, bool QJL, bool ATTEND>
static int launch_g(const DecodeArgs& a, int ns, int gs, hipStream_t s) {
  dim3 grid((unsigned)a.num_splits, (unsigned)(a.num_kv_heads * ns), (unsigned)a.num_seqs);
  if (gs <= 1) hipLaunchKernelGGL((decode_kernel<BK, BV, QJL, 1, ATTEND>), grid, dim3(256), 0, s, a, ns, gs);
  else if (gs <= 2) hipLaunchKernelGGL((decode_kernel<BK, BV, QJL, 2, ATTEND>), grid, dim3(256), 0, s, a, ns, gs);
  else if (gs <= 4) hipLaunchKernelGGL((decode_kernel<BK, BV, QJL, 4, ATTEND>), grid, dim3(256), 0, s, a, ns, gs);
  else hipLaunchKernelGGL((decode_kernel<BK, BV, QJL, 8, ATTEND>), grid, dim3(256), 0, s, a, ns, gs);
  return (int)hipGetLastError();
}

template <int B, bool ATTEND>
static int launch_b(const DecodeArgs& a, bool qjl, int ns, int gs, hipStream_t s) {
  if (qjl) return launch_g<B, ATTEND ? B : 2, true, ATTEND>(a, ns, gs, s);
  return launch_g<B, ATTEND ? B : 2, false, ATTEND>(a, ns, gs, s);
}

int launch_decode(const DecodeArgs& a, int bits_k, int bits_v, int qjl, int attend, int mfma, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int ns = (a.group + 7) / 8;
  const int gs = (a.group + ns - 1) / ns;
  if (attend && bits_v != bits_k) return (int)hipErrorInvalidValue;
  if (attend && mfma) {
    const int e = launch_decode_mfma(a, bits_k, qjl != 0, ns, gs, stream);
    return e ? e : launch_merge(a, stream);
  }
  int e = 0;
  switch (bits_k) {
    case 2: e = attend ? launch_b<2, true>(a, qjl, ns, gs, s) : launch_b<2, false>(a, qjl, ns, gs, s); break;
    case 3: e = attend ? launch_b<3, true>(a, qjl, ns, gs, s) : launch_b<3, false>(a, qjl, ns, gs, s); break;
    case 4: e = attend ? launch_b<4, true>(a, qjl, ns, gs, s) : launch_b<4, false>(a, qjl, ns, gs, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (e == 0 && attend) ? launch_merge(a, stream) : e;
}

int decode_slices(int group) { return (group + 7) / 8; }

}  // namespace tq
