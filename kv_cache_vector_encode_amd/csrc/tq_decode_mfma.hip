// tq_decode_mfma: decode-attend for grouped queries on the gfx950 matrix
// cores.  Same computation as decode_kernel (tq_decode.hip): logits in the
// rotated frame, s_t = scale * gamma_t * <R q, c[codes_t]>, softmax, value
// sum in the rotated frame, one inverse rotation per query head at the end
// (Bit-Axon "TurboQuant: KV Cache Compression", attention under quantisation;
// deep-dive blog Step 1, attention directly on the rotated data).
//
// With 8 query heads per KV head every code is used by 8 dot products, so
// both contractions are dense; they run as v_mfma_f32_16x16x32 products and
// the vector units only dequantise codes and run the softmax.
//
//   logits  C[16 tokens x 16] = A[16 tokens x 32] * B[32 x 16], 8 steps over
//           the 128 dims.  A slots hold (hi, lo) bf16 pairs of centroid
//           values (c = hi + lo to 2^-17); B columns hold q_hi (heads 0..7)
//           and q_lo (residual of q, heads 0..7); logit = col h + col h+8.
//   values  C[16 dims x 16] += A[16 dims x 32 tokens] * B[32 tokens x 16] in
//           f16, one product per 8-dim tile over a pair of blocks; B columns
//           hold p*gamma_v in f16 (heads 0..7) and its f16 residual.
// Operand layout (16x16x32, checked on the device): lane l holds
// A[l%16][8(l/16)+s], B[8(l/16)+s][l%16] and C[4(l/16)+r][l%16].
//
// Work: grid (split, KV-head slice of <= 8 query heads, sequence); 4 waves
// per workgroup, each takes pairs of 16-token blocks of the split in turn
// and keeps its own running max / sum / accumulator.  The waves are merged
// in LDS, the split's (m, l, o_rot) goes to the workspace, and the last
// workgroup of the (sequence, slice) merges the splits in fixed order and
// applies R^T (shared with decode_kernel).

#include <hip/hip_bf16.h>

#include "tq_device.h"

namespace tq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_bits(float v) {
  return (uint32_t)__builtin_bit_cast(unsigned short, __float2bfloat16(v));
}
__device__ __forceinline__ float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint32_t f16_bits(float v) {
  return (uint32_t)__half_as_ushort(__float2half_rn(v));
}

// code i of a packed little-endian bit string held in words w[]
template <int BITS, int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N], int i) {
  const int bit = BITS * i, wi = bit >> 5, sh = bit & 31;
  constexpr uint32_t mask = (1u << BITS) - 1;
  if (sh + BITS <= 32) return (w[wi] >> sh) & mask;
  return ((w[wi] >> sh) | (w[wi + 1] << (32 - sh))) & mask;
}

// c + c of the lane 8 columns away (row_ror:8 inside each 16-lane row), for
// the four C registers of a logit tile: adds the q_hi and q_lo columns.
// Written out because the compiler, combining a DPP move with an add, fed
// all four registers from the first.  The C registers come straight from the
// matrix core, and the compiler does not pad inline asm for that hazard: the
// s_nops give 20 wait states (an 8-pass matrix-core write needs 10 before a
// vector read, a 16-pass one 18), which also cover the 2 a DPP read of a
// vector-unit result needs.
__device__ __forceinline__ void add_col_pairs(const f32x4& c, float (&o)[4]) {
  asm("s_nop 7\n\ts_nop 7\n\ts_nop 3\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %2, %6, %6 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_add_f32_dpp %3, %7, %7 row_ror:8 row_mask:0xf bank_mask:0xf"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]));
}

template <int BITS>
struct BlockRegs {
  uint32_t k[BITS];     // 32 codes: dims 32g .. 32g+31 of token row m
  uint32_t v[4];        // 8 codes each: dims 8m .. 8m+7 of tokens 4g .. 4g+3
  uint32_t gk[2];       // fp16 norms of tokens 4g .. 4g+3
  uint32_t gv[2];
};

// Per-lane byte offsets inside a (block, KV head) chunk, fixed for the whole
// kernel: loads then take a wave-uniform base plus a 32-bit lane offset.
struct LaneOffsets {
  uint32_t k;      // K code chunk of row m, dims 32g..
  uint32_t v[4];   // V codes of tokens 4g+i, dims 8m..
  uint32_t gk, gv; // norms of tokens 4g..4g+3
};

template <int BITS>
__device__ __forceinline__ LaneOffsets lane_offsets(const Layout& lay, int m, int g) {
  LaneOffsets o;
  o.k = (uint32_t)(lay.off_k + m * lay.k_rec + g * (4 * BITS));
#pragma unroll
  for (int i = 0; i < 4; ++i) o.v[i] = (uint32_t)(lay.off_v + (4 * g + i) * lay.v_rec + ((BITS * 8 * m) >> 3));
  o.gk = (uint32_t)(lay.off_gk + 8 * g);
  o.gv = (uint32_t)(lay.off_gv + 8 * g);
  return o;
}

template <int BITS>
__device__ __forceinline__ void load_block(BlockRegs<BITS>& r, const uint8_t* base, const LaneOffsets& o, int m) {
  if constexpr (BITS == 4) {
    const uint4 t = *reinterpret_cast<const uint4*>(base + o.k);
    r.k[0] = t.x; r.k[1] = t.y; r.k[2] = t.z; r.k[3] = t.w;
  } else if constexpr (BITS == 3) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(base + o.k);
    r.k[0] = p[0]; r.k[1] = p[1]; r.k[2] = p[2];
  } else {
    const uint2 t = *reinterpret_cast<const uint2*>(base + o.k);
    r.k[0] = t.x; r.k[1] = t.y;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BITS == 4) {
      r.v[i] = *reinterpret_cast<const uint32_t*>(base + o.v[i]);
    } else if constexpr (BITS == 2) {
      r.v[i] = *reinterpret_cast<const uint16_t*>(base + o.v[i]);
    } else {
      // 24 bits at byte 3m: two aligned dwords and a funnel shift (the
      // second can run past the record; other regions follow the codes)
      const uint32_t al = o.v[i] & ~3u, sh = 8 * (o.v[i] & 3u);
      const uint32_t lo = *reinterpret_cast<const uint32_t*>(base + al);
      const uint32_t hi = *reinterpret_cast<const uint32_t*>(base + al + 4);
      r.v[i] = (uint32_t)((((uint64_t)hi << 32) | lo) >> sh) & 0xFFFFFFu;
    }
  }
  const uint2 a = *reinterpret_cast<const uint2*>(base + o.gk);
  const uint2 b = *reinterpret_cast<const uint2*>(base + o.gv);
  r.gk[0] = a.x; r.gk[1] = a.y;
  r.gv[0] = b.x; r.gv[1] = b.y;
}

__device__ __forceinline__ float half_lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xFFFF))); }
__device__ __forceinline__ float half_hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }

template <int BITS, bool LOGITS>
__global__ __launch_bounds__(256) void decode_mfma_kernel(const DecodeArgs a, int ns, int gs) {
  // Dequantisation tables, indexed by a pair of codes (2*BITS bits):
  //  keys:   (hi | lo << 16, hi | lo << 16) bf16 of the two centroids,
  //  values: f16(c[first]) | f16(c[second]) << 16.
  __shared__ uint2 s_tk2[1 << (2 * BITS)];
  __shared__ uint32_t s_tv2[1 << (2 * BITS)];
  __shared__ float s_q[8][kD];
  __shared__ u32x4 s_qb[8][64];        // logit B operands [step][lane]
  __shared__ float s_acc[4][16][kD];   // per wave: [column][dim]
  __shared__ float s_wm[4][8], s_wl[4][8];
  __shared__ float s_ml[2][8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;     // row / column index and lane group
  const int split = blockIdx.x, unit = blockIdx.y, n = blockIdx.z;
  const int h = unit / ns, slice = unit - h * ns;
  const int g0 = slice * gs;
  const int gcount = min(gs, a.group - g0);
  const int seq_len = max(0, min(a.seq_lens[n], a.max_blocks * kBlock));
  const int nblk_seq = (seq_len + kBlock - 1) / kBlock;
  const int sb0 = split * a.blocks_per_split;
  const int sb1 = min(nblk_seq, sb0 + a.blocks_per_split);
  const int64_t Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const float LOG2E = 1.4426950408889634f;

  for (int i = tid; i < (1 << (2 * BITS)); i += 256) {
    constexpr uint32_t mask = (1u << BITS) - 1;
    const float c0 = a.cent_k[i & mask], c1 = a.cent_k[i >> BITS];
    const uint32_t h0 = bf16_bits(c0), h1 = bf16_bits(c1);
    s_tk2[i] = make_uint2(h0 | (bf16_bits(c0 - bf16_val(h0)) << 16), h1 | (bf16_bits(c1 - bf16_val(h1)) << 16));
    s_tv2[i] = f16_bits(a.cent_v[i & mask]) | (f16_bits(a.cent_v[i >> BITS]) << 16);
  }

  // ---- rotate this slice's queries (rows of 16 lanes, one head each)
  {
    const int r = tid >> 4, p = tid & 15;
    if (r < gcount) {
      const FwhtLane fc = fwht_lane(p);
      const int64_t hq = (int64_t)h * a.group + g0 + r;
      const int ell = perm16(p);
      float x[8];
      const int64_t elem = ((int64_t)n * Hq + hq) * kD + 8 * ell;
      if (a.q_dtype == 0) load8<0>(a.q, elem, x);
      else if (a.q_dtype == 1) load8<1>(a.q, elem, x);
      else load8<2>(a.q, elem, x);
      const uint32_t sb = sign_byte(a.rot, ell);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = flip(x[e], sb, e);
      fwht_row(x, fc);
      const float sc = fc.sig * kInvSqrtD;
#pragma unroll
      for (int e = 0; e < 8; ++e) s_q[r][8 * p + e] = x[e] * sc;
    }
  }
  __syncthreads();

  // ---- B operands of the logit product: column m -> head m%8, part m/8;
  // step st, slots (2e, 2e+1) both carry dim 32g + 4st + e.  Kept in LDS
  // (each lane reads back its own 8 x 16 bytes per block) to spare VGPRs.
  {
    const int hd = m & 7;
    const bool lo = m >= 8;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st % 4 != wave) continue;   // the 4 waves fill 2 steps each
      u32x4 q4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float qv = hd < gcount ? s_q[hd][32 * g + 4 * st + e] : 0.f;
        const uint32_t hb = bf16_bits(qv);
        const uint32_t v = lo ? bf16_bits(qv - bf16_val(hb)) : hb;
        q4[e] = v | (v << 16);
      }
      s_qb[st][lane] = q4;
    }
  }
  __syncthreads();
  const float sscale = a.scale * LOG2E;       // scores kept in log2 units
  const bool col_lo = m >= 8;
  const bool col_live = (m & 7) < gcount;
  const uint32_t live_mask = col_live ? 0xFFFFu : 0u;

  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float run_m = -INFINITY, run_l = 0.f;

  const int32_t* btab = a.block_tables + (int64_t)n * a.max_blocks;
  const int npairs = max(0, (sb1 - sb0 + 1) / 2);
  // wave-uniform indices: block-table reads become scalar loads, which do not
  // hold up the vector-memory counter the prefetched data waits on
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  auto block_base = [&](int lb) -> const uint8_t* {
    int blk = (lb < sb1) ? btab[lb] : 0;
    blk = (blk >= 0 && blk < a.num_blocks) ? blk : 0;
    return a.pool + ((int64_t)blk * Hkv + h) * a.lay.block_bytes;
  };
  const LaneOffsets lo_off = lane_offsets<BITS>(a.lay, m, g);
  auto load_pair = [&](BlockRegs<BITS>(&r)[2], int pi) {
    load_block<BITS>(r[0], block_base(sb0 + 2 * pi), lo_off, m);
    load_block<BITS>(r[1], block_base(sb0 + 2 * pi + 1), lo_off, m);
  };
  auto compute_pair = [&](const BlockRegs<BITS>(&cur)[2], int pi) {
    // ---- logits of the two blocks
    float s[2][4];
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const uint2 t0 = s_tk2[field<2 * BITS>(cur[X].k, 2 * st)];
        const uint2 t1 = s_tk2[field<2 * BITS>(cur[X].k, 2 * st + 1)];
        const u32x4 av = {t0.x, t0.y, t1.x, t1.y};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                    __builtin_bit_cast(bf16x8, s_qb[st][lane]), c, 0, 0, 0);
      }
      const int lb = sb0 + 2 * pi + X;
      float cs[4];
      add_col_pairs(c, cs);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = cs[j];
        const float gk = (j & 1) ? half_hi(cur[X].gk[j >> 1]) : half_lo(cur[X].gk[j >> 1]);
        const int tok = lb * kBlock + 4 * g + j;
        v = (lb < sb1 && tok < seq_len) ? v * gk * sscale : -INFINITY;
        s[X][j] = v;
        if (LOGITS && !col_lo && col_live && lb < sb1 && tok < seq_len)
          a.logits[((int64_t)n * Hq + (int64_t)h * a.group + g0 + m) * a.logits_stride + tok] = v * (1.f / LOG2E);
      }
    }
    // ---- online softmax over the 32 tokens (per head = per column pair)
    float bm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float new_m = fmaxf(run_m, bm);
    // rescale only when some head's running max moved (rare after the first
    // blocks); the accumulators stay in the matrix-core registers otherwise
    if (__builtin_amdgcn_ballot_w64(new_m > run_m) != 0) {
      const float alpha = (run_m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(run_m - new_m);
      run_l *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= alpha;
    }
    run_m = new_m;
    uint32_t pw[2][2];
#pragma unroll
    for (int X = 0; X < 2; ++X) {
      uint32_t hv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = (new_m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[X][j] - new_m);
        run_l += p;
        const float gv = (j & 1) ? half_hi(cur[X].gv[j >> 1]) : half_lo(cur[X].gv[j >> 1]);
        const float pv = p * gv;
        // columns 0..7 take f16(pv), columns 8..15 its f16 residual; no
        // branches here (a branch would make the compiler wait for every
        // outstanding load, including the prefetched block pair)
        const float hi = __half2float(__float2half_rn(pv));
        hv[j] = f16_bits(col_lo ? pv - hi : pv) & live_mask;
      }
      pw[X][0] = hv[0] | (hv[1] << 16);
      pw[X][1] = hv[2] | (hv[3] << 16);
    }
    const u32x4 pb = {pw[0][0], pw[0][1], pw[1][0], pw[1][1]};
    // ---- values: one product per 8-dim tile t (dims 8m+t); the A operand
    // pairs tokens (4g, 4g+1), (4g+2, 4g+3) of each block
    uint32_t iv[4][8];   // [word pair][t]: code(first) | code(second) << BITS
#pragma unroll
    for (int X = 0; X < 2; ++X)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t wa = cur[X].v[2 * q], wb = cur[X].v[2 * q + 1];
        if constexpr (BITS == 4) {
          // interleave nibbles: byte k of ev = (a_{2k}, b_{2k}), of od = (a_{2k+1}, b_{2k+1})
          const uint32_t ev = (wa & 0x0F0F0F0Fu) | ((wb & 0x0F0F0F0Fu) << 4);
          const uint32_t od = ((wa >> 4) & 0x0F0F0F0Fu) | (wb & 0xF0F0F0F0u);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            iv[2 * X + q][2 * k] = (ev >> (8 * k)) & 0xFFu;
            iv[2 * X + q][2 * k + 1] = (od >> (8 * k)) & 0xFFu;
          }
        } else {
          constexpr uint32_t mask = (1u << BITS) - 1;
#pragma unroll
          for (int t = 0; t < 8; ++t)
            iv[2 * X + q][t] = ((wa >> (BITS * t)) & mask) | (((wb >> (BITS * t)) & mask) << BITS);
        }
      }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x4 av = {s_tv2[iv[0][t]], s_tv2[iv[1][t]], s_tv2[iv[2][t]], s_tv2[iv[3][t]]};
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av),
                                                     __builtin_bit_cast(f16x8, pb), acc[t], 0, 0, 0);
    }
  };

  // Two register sets in turn (no copies, so a wait only covers the older
  // set).  Prefetches are unconditional, past the split's end they re-read
  // block 0 (never used): with a fixed number of loads in flight the
  // compiler can wait for just the older set.
  BlockRegs<BITS> ra[2], rb[2];
  int pi = wv;
  load_pair(ra, pi);
  for (; pi < npairs; pi += 8) {
    load_pair(rb, pi + 4);
    compute_pair(ra, pi);
    if (pi + 4 >= npairs) break;
    load_pair(ra, pi + 8);
    compute_pair(rb, pi + 4);
  }

  // ---- merge the 4 waves of the workgroup
  run_l += __shfl_xor(run_l, 16);
  run_l += __shfl_xor(run_l, 32);
  if (g == 0 && m < 8) {
    s_wm[wave][m] = run_m;
    s_wl[wave][m] = run_l;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) s_acc[wave][m][8 * (4 * g + j) + t] = acc[t][j];
  __syncthreads();

  const int64_t nsplit = a.num_splits;
  float* part_base = a.partials + (((int64_t)n * Hkv + h) * nsplit) * a.group * kPartStride;
  if (tid < 8) {
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_wm[w][tid]);
    float L = 0.f;
    for (int w = 0; w < 4; ++w)
      if (s_wm[w][tid] != -INFINITY) L += s_wl[w][tid] * __builtin_amdgcn_exp2f(s_wm[w][tid] - M);
    s_ml[0][tid] = M;
    s_ml[1][tid] = L;
  }
  __syncthreads();
  for (int i = tid; i < gcount * kD; i += 256) {
    const int hd = i >> 7, d = i & (kD - 1);
    const float M = s_ml[0][hd];
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_wm[w][hd];
      if (mw != -INFINITY) o += __builtin_amdgcn_exp2f(mw - M) * (s_acc[w][hd][d] + s_acc[w][hd + 8][d]);
    }
    part_base[((int64_t)split * a.group + g0 + hd) * kPartStride + d] = o;
  }
  if (tid < gcount) {
    float* pp = part_base + ((int64_t)split * a.group + g0 + tid) * kPartStride;
    // the merge step works in natural-log units
    pp[128] = s_ml[0][tid] * (1.f / LOG2E);
    pp[129] = s_ml[1][tid];
  }

}

int launch_decode_mfma(const DecodeArgs& a, int bits, int ns, int gs, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((unsigned)a.num_splits, (unsigned)(a.num_kv_heads * ns), (unsigned)a.num_seqs);
  const bool lg = a.logits != nullptr;
  switch (bits) {
    case 2:
      if (lg) hipLaunchKernelGGL((decode_mfma_kernel<2, true>), grid, dim3(256), 0, s, a, ns, gs);
      else hipLaunchKernelGGL((decode_mfma_kernel<2, false>), grid, dim3(256), 0, s, a, ns, gs);
      break;
    case 3:
      if (lg) hipLaunchKernelGGL((decode_mfma_kernel<3, true>), grid, dim3(256), 0, s, a, ns, gs);
      else hipLaunchKernelGGL((decode_mfma_kernel<3, false>), grid, dim3(256), 0, s, a, ns, gs);
      break;
    case 4:
      if (lg) hipLaunchKernelGGL((decode_mfma_kernel<4, true>), grid, dim3(256), 0, s, a, ns, gs);
      else hipLaunchKernelGGL((decode_mfma_kernel<4, false>), grid, dim3(256), 0, s, a, ns, gs);
      break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace tq
