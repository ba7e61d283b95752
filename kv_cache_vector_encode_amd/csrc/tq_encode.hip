// tq_encode: norm / direction split, seeded sign flip, FWHT-128, threshold
// search against the Lloyd-Max codebook, b-bit packing into the paged cache,
// optional 1-bit QJL residual sketch.
//
// Method: "TurboQuant: KV Cache Vector Quantization" card, three stages
// (split, rotate, codebook); OCTOPUS summary, Method steps 1, 2 and 6 and the
// "Optional 1-bit QJL residual" contribution; Bit-Axon "TurboQuant: KV Cache
// Compression", quantisation function (nearest codeword); deep-dive blog
// Step 1 (sign flip, Hadamard, 1/sqrt(d)) and Step 2 (fp16 magnitude plus
// direction indices).
//
// Two kernels:
//  * encode_mx_kernel (bf16 / f16 input, with or without the QJL sidecar):
//    the Hadamard product on the matrix cores, 16 vectors per wave; the norm,
//    the bucketed threshold search and the packing stay on the vector ALUs
//    (described at the kernel).  The sidecar's second Hadamard product runs on
//    the matrix cores too.
//  * encode_kernel (fp32 input): one vector (d = 128)
//    per 16-lane row, 8 coordinates per lane, the FWHT as in-lane butterflies
//    plus DPP lane stages, so a wave64 encodes 4 vectors at once and a
//    256-thread workgroup 16.  A workgroup handles kIters such groups; all
//    their input loads are issued before any arithmetic.  A row's 16 lanes
//    read the vector's 256 contiguous bytes (permuted among the lanes, still
//    one coalesced request) and write its code record.

#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "tq_device.h"
#include "tq_encode_row.h"

namespace tq {

constexpr int kIters = 4;

template <int BITS, int DT, bool QJL>
__global__ __launch_bounds__(256) void encode_kernel(const EncodeArgs a) {
  // Threshold search in bucket units: z = y * lut_scale + lut_offset - 1/2,
  // bucket k = round-to-nearest(z) clamped to [0, 255] by the conversion
  // (the floor of y * lut_scale + lut_offset away from bucket edges, which
  // hold no threshold), code = base[k] + (z > threshold of bucket k in the
  // same units).  Entries past the host's lut_n repeat its last bucket.
  __shared__ uint2 s_lut[256];
  __shared__ float s_cent[16];
  const int tid = threadIdx.x;
  const float lut_scale = a.tab.lut_scale, lut_off = a.tab.lut_offset - 0.5f;
  fill_lut(s_lut, a.tab, lut_scale, lut_off, tid);
  if (tid < 16) s_cent[tid] = a.tab.centroid[tid];

  const EncodeStream st = a.stream[blockIdx.y];
  const int L = tid & 15;
  const int ell = perm16(L);
  const uint32_t sneg = sign_byte(a.rot, ell);       // signs of my inputs 8*ell+e
  uint32_t smask[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (DT == 0) smask[i] = ((sneg >> i) & 1u) << 31;
    else smask[i] = i < 4 ? (((sneg >> (2 * i)) & 1u) << 15) | (((sneg >> (2 * i + 1)) & 1u) << 31) : 0u;
  }
  const FwhtLane fc = fwht_lane(L);
  const int32_t H = a.num_heads;

  // ---- issue every load of this workgroup first
  float x[kIters][8];
  int32_t slot[kIters];
  uint32_t head[kIters];
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    const int64_t v = ((int64_t)blockIdx.x * kIters + i) * 16 + (tid >> 4);
    const bool ok = v < a.num_vectors;
    const uint32_t vl = ok ? (uint32_t)v : 0u;
    load8_signed<DT>(st.src, (int64_t)vl * kD + 8 * ell, smask, x[i]);
    const uint32_t t = fast_div(vl, a.div_heads);
    head[i] = vl - t * (uint32_t)H;
    const int32_t sm = ok ? a.slot_mapping[t] : -1;
    slot[i] = (sm >= 0 && sm < a.num_slots) ? sm : -1;
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[i][e], x[i][e], ss);
    ss = row_sum(ss);
    fwht_row(x[i], fc);                 // lane L now holds coordinates 8L..8L+7
    // 1-ulp hardware sqrt / reciprocal: their error (~1e-7 relative) is far
    // inside the decision band the encoder is held to
    const float gamma = __builtin_amdgcn_sqrtf(ss);
    const float inv = ss > 0.f ? fc.sig * __builtin_amdgcn_rcpf(gamma * 11.313708498984761f) : 0.f;

    uint32_t code[8];
    row_codes<BITS>(x[i], inv * lut_scale, lut_off, s_lut, code);
    bool store_lane;
    int store_off;
    const uint32_t store_word = row_pack<BITS>(code, L, store_lane, store_off);

    // ---- optional QJL sketch of the rotated-frame residual (keys)
    uint32_t sbits = 0;
    float rho = 0.f;
    if constexpr (QJL) {
      if (st.qjl) {
        float r[8];
        float rr = 0.f;
        const uint32_t qneg = sign_byte(a.rot_qjl, L);   // natural coords 8L+e
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          r[e] = x[i][e] * inv - s_cent[code[e]];
          rr = __builtin_fmaf(r[e], r[e], rr);
        }
        rr = row_sum(rr);
        rho = __builtin_amdgcn_sqrtf(rr);
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = flip(r[e], qneg, e);
        fwht_row(r, fc);                 // lane L holds output lane perm16(L)
#pragma unroll
        for (int e = 0; e < 8; ++e) sbits |= ((fc.sig * r[e]) < 0.f ? 1u : 0u) << e;
      }
    }

    if (slot[i] >= 0) {
      const int64_t h = head[i];
      const int s = slot[i];
      uint8_t* base = a.pool + ((int64_t)(s >> 4) * H + h) * a.block_bytes;
      const int row = s & 15;
      uint8_t* rec = base + st.rec_off + (int64_t)row * st.rec_bytes;
      if (store_lane) *reinterpret_cast<uint32_t*>(rec + store_off) = store_word;
      if (L == 0) {
        const __half g16 = __float2half_rn(fminf(gamma, 65504.f));
        *reinterpret_cast<__half*>(base + st.norm_off + 2 * row) = g16;
      }
      if constexpr (QJL) {
        if (st.qjl) {
          base[a.sign_off + row * 16 + perm16(L)] = (uint8_t)sbits;
          if (L == 0)
            *reinterpret_cast<__half*>(base + a.rho_off + 2 * row) = __float2half_rn(fminf(rho, 65504.f));
        }
      }
    }
  }
}

// two-term dot product of packed 16-bit pairs with a zero accumulator (the
// three-operand form; the builtin spends a move on the zero)
template <int DT>
__device__ __forceinline__ float dot2_zero(uint32_t w, uint32_t b) {
  float r;
  if constexpr (DT == 2)
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(w), "v"(b));
  else
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(w), "v"(b));
  return r;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ float dot2_acc(uint32_t w, uint32_t b, float c) {
  if constexpr (DT == 2)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), __builtin_bit_cast(f16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------
// Matrix-core encode for 16-bit inputs.
//
// The Hadamard part of the rotation is the dense product Y = H X' for a batch
// of 16 vectors: X' is the 128 x 16 input with the sign flips applied as an
// xor of sign bits (exact), H has entries +-1 (exact in 16 bits), and the
// products accumulate in fp32.  Output coordinates form 8 tiles of 16, input
// dims 4 steps of 32, one v_mfma_f32_16x16x32 per (tile, step).
//
// Row i of tile n stands for coordinate 32 (n >> 1) + 8 (i >> 2) + 4 (n & 1)
// + (i & 3).  With that order accumulator lane (g, j) (g = lane / 16,
// j = lane % 16) of tiles 2m and 2m + 1 holds coordinates 32 m + 8 g .. +7
// of vector j: the eight consecutive coordinates of one packed code group,
// so codes are searched and packed where they are produced.
//
// The H operand of tile n, step k at lane (g', i), element s is
// (-1)^popcount(p & d) for coordinate p above and input dim d = 32 k + 8 g' + s:
//   popcount(p & d) = i0 s0 + i1 s1 + i2 g'0 + i3 g'1   lane and element
//                   + n0 s2                             odd tiles: elements 4..7
//                   + n1 k0 + n2 k1                     same for the whole tile and step
// so each operand is one of +-B0, +-B1, B1 being B0 with elements 4..7 negated.
//
// QJL sidecar (keys of a QJL cache): the residual r = y / (|x| sqrt(128)) -
// centroid(code) of the lane's coordinates 32 m + 8 g .. +7 sits exactly
// where step m of a second product with H reads its input, so H D' r is the
// same 8 tiles x 4 steps with D' (the sketch's signs) applied as sign-bit
// xors.  r is not exact in 16 bits: it is scaled by 2^10 and split into f16
// high and low parts (high truncated, low = the rest, both in f16), and the
// two products accumulate in fp32.  What the split drops is below 2^-22 of
// each |r_i|, so each output is off by at most 2^-22 sqrt(128) |r| < 3e-6 |r|
// from the fp32 product, and only such near-zero outputs can take the other
// sign bit.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#ifndef TQ_MX_BATCHES
#define TQ_MX_BATCHES 1
#endif
constexpr int kMxBatches = TQ_MX_BATCHES;   // 16-vector batches per wave

template <int DT>
__device__ __forceinline__ f32x4_t mfma_h(const u32x4_t& h, const u32x4_t& x, const f32x4_t& c) {
  if constexpr (DT == 2)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, h), __builtin_bit_cast(bf16x8_t, x), c,
                                                   0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, h), __builtin_bit_cast(f16x8_t, x), c,
                                                  0, 0, 0);
}

template <int BITS>
struct MxShared {
  static constexpr int kRecStride = 16 * BITS + 16;   // padded staging record
  uint2 lut[256];
  u32x4_t smask[4][4];                                // [g][k]: sign-bit masks of dims 32 k + 8 g + 0..7
  __align__(16) uint8_t rec[4][16 * kRecStride];      // per wave: 16 packed records
};

// QJL sidecar: the sketch's sign-bit masks (as smask) and 2^10 x the centroids.
struct MxQjlShared {
  u32x4_t qmask[4][4];
  float cent[16];
};

// Bucket table, sign masks (shared) and the H operands B0, B1, -B0, -B1 of
// this lane (lane = (g', i) of the A layout).
template <int BITS, int DT, bool QJL>
__device__ __forceinline__ void mx_setup(const EncodeArgs& a, MxShared<BITS>& sh, MxQjlShared& shq, u32x4_t (&B)[4],
                                         int tid) {
  fill_lut(sh.lut, a.tab, a.tab.lut_scale, a.tab.lut_offset - 0.5f, tid);
  if constexpr (QJL) {
    if (tid >= 64 && tid < 128) {
      const int gg = (tid >> 4) & 3, k = (tid >> 2) & 3, q = tid & 3;
      const uint32_t n0 = __builtin_amdgcn_readfirstlane(a.rot_qjl.neg[0]);
      const uint32_t n1 = __builtin_amdgcn_readfirstlane(a.rot_qjl.neg[1]);
      const uint32_t n2 = __builtin_amdgcn_readfirstlane(a.rot_qjl.neg[2]);
      const uint32_t n3 = __builtin_amdgcn_readfirstlane(a.rot_qjl.neg[3]);
      const uint32_t wd = k == 0 ? n0 : k == 1 ? n1 : k == 2 ? n2 : n3;
      const uint32_t sb = (wd >> (8 * gg)) & 0xFFu;
      shq.qmask[gg][k][q] = (((sb >> (2 * q)) & 1u) << 15) | (((sb >> (2 * q + 1)) & 1u) << 31);
    }
    if (tid >= 128 && tid < 144) shq.cent[tid - 128] = 1024.f * a.tab.centroid[tid - 128];   // 2^10 c, exact
  }
  if (tid < 64) {
    const int gg = tid >> 4, k = (tid >> 2) & 3, q = tid & 3;
    // sign byte 4 k + gg, picked among wave-uniform (scalar) loads of the
    // four mask words: a per-lane load of the argument block would be one
    // more memory round trip before the batch can start
    // (readfirstlane keeps the compiler from turning the select into a
    // per-lane address)
    const uint32_t n0 = __builtin_amdgcn_readfirstlane(a.rot.neg[0]), n1 = __builtin_amdgcn_readfirstlane(a.rot.neg[1]);
    const uint32_t n2 = __builtin_amdgcn_readfirstlane(a.rot.neg[2]), n3 = __builtin_amdgcn_readfirstlane(a.rot.neg[3]);
    const uint32_t wd = k == 0 ? n0 : k == 1 ? n1 : k == 2 ? n2 : n3;
    const uint32_t sb = (wd >> (8 * gg)) & 0xFFu;
    sh.smask[gg][k][q] = (((sb >> (2 * q)) & 1u) << 15) | (((sb >> (2 * q + 1)) & 1u) << 31);
  }
  // Element e = 2 w + h of B0 at lane (g', i) is negative iff
  // i0 e0 + i1 e1 + i2 g'0 + i3 g'1 is odd.  Elements e and e + 4 agree, so
  // B0 = {w0, w1, w0, w1}: w0 (e = 0, 1) carries the lane parity c in both
  // halves and i0 in the high half, w1 (e = 2, 3) also i1 in both halves.
  const uint32_t one2 = DT == 2 ? 0x3F803F80u : 0x3C003C00u;
  const uint32_t lane = (uint32_t)(tid & 63);
  const uint32_t y = (lane >> 2) & (lane >> 4);            // bit 0: i2 g'0, bit 1: i3 g'1
  const uint32_t c = (y ^ (y >> 1)) & 1u;
  const uint32_t w0 = one2 ^ (c ? 0x80008000u : 0u) ^ ((lane & 1u) << 31);
  const uint32_t w1 = w0 ^ ((lane & 2u) ? 0x80008000u : 0u);
  const uint32_t n0 = w0 ^ 0x80008000u, n1 = w1 ^ 0x80008000u;
  B[0] = (u32x4_t){w0, w1, w0, w1};
  B[1] = (u32x4_t){w0, w1, n0, n1};
  B[2] = (u32x4_t){n0, n1, n0, n1};
  B[3] = (u32x4_t){n0, n1, w0, w1};
}

// One batch: this lane's share of vector j (dims 32 k + 8 g .. +7 in X[k]),
// its slot (-1: nothing stored) and head.
struct MxBatch {
  u32x4_t X[4];
  int32_t slot;
  uint32_t head;
};

__device__ __forceinline__ void mx_load(const EncodeArgs& a, const void* src, uint32_t batch, int g, int j,
                                        MxBatch& o) {
  // past the last vector a lane re-reads the last one (nothing is stored)
  const uint32_t nvec = (uint32_t)a.num_vectors;
  const uint32_t v = 16u * batch + j;
  const uint32_t vc = min(v, nvec - 1u);
  const u32x4_t* p =
      reinterpret_cast<const u32x4_t*>(static_cast<const uint8_t*>(src) + (uint64_t)vc * (2 * kD) + 16 * g);
#pragma unroll
  for (int k = 0; k < 4; ++k) o.X[k] = p[4 * k];
  const uint32_t t = fast_div(vc, a.div_heads);
  o.head = vc - t * (uint32_t)a.num_heads;
  o.slot = v < nvec ? a.slot_mapping[t] : -1;
}

template <int BITS, int DT, bool OFF32, bool QJL>
__device__ __forceinline__ void mx_batch(const EncodeArgs& a, const EncodeStream& st, const MxBatch& in,
                                         const u32x4_t (&B)[4], MxShared<BITS>& sh, const MxQjlShared& shq, int wave,
                                         int g, int j) {
  constexpr int kRecStride = MxShared<BITS>::kRecStride;
  const float lut_scale = a.tab.lut_scale, lut_off = a.tab.lut_offset - 0.5f;
  uint8_t* rec_w = sh.rec[wave];
  // |x|^2 of vector j: this lane holds 32 of its 128 dims
  float ss = dot2_zero<DT>(in.X[0][0], in.X[0][0]);
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int q = (k == 0 ? 1 : 0); q < 4; ++q) ss = dot2_acc<DT>(in.X[k][q], in.X[k][q], ss);
  ss = sum_rows(ss);
  const float gamma = __builtin_amdgcn_sqrtf(ss);
  // 1-ulp hardware square root and reciprocal square root: ~1e-7 relative,
  // far inside the decision band
  const float zs = ss > 0.f ? lut_scale * kInvSqrtD * __builtin_amdgcn_rsqf(ss) : 0.f;
  u32x4_t xs[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) xs[k] = in.X[k] ^ sh.smask[g][k];
  // QJL: 2^10 r as f16 high and low parts with the sketch's signs applied,
  // and the lane's share of |2^10 r|^2
  const bool qjl = QJL && st.qjl != 0;
  const float zu = ss > 0.f ? kInvSqrtD * __builtin_amdgcn_rsqf(ss) : 0.f;
  u32x4_t rh[4], rl[4];
  float rr = 0.f;

#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int neg = ((m & k) ^ ((m >> 1) & (k >> 1))) & 1;
      c0 = mfma_h<DT>(B[2 * neg], xs[k], c0);
      c1 = mfma_h<DT>(B[1 + 2 * neg], xs[k], c1);
    }
    const float y[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    uint32_t code[8];
    row_codes<BITS>(y, zs, lut_off, sh.lut, code);
    if constexpr (QJL) {
      if (qjl) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // 1024 (y zu - c) as one fma: scaling by a power of two is exact
          const float r0 = __builtin_fmaf(y[2 * w], 1024.f * zu, -shq.cent[code[2 * w]]);
          const float r1 = __builtin_fmaf(y[2 * w + 1], 1024.f * zu, -shq.cent[code[2 * w + 1]]);
          rr = __builtin_fmaf(r0, r0, __builtin_fmaf(r1, r1, rr));
          const auto h = __builtin_amdgcn_cvt_pkrtz(r0, r1);
          const auto l = __builtin_amdgcn_cvt_pkrtz(r0 - (float)h[0], r1 - (float)h[1]);
          rh[m][w] = __builtin_bit_cast(uint32_t, h) ^ shq.qmask[g][m][w];
          rl[m][w] = __builtin_bit_cast(uint32_t, l) ^ shq.qmask[g][m][w];
        }
      }
    }
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) word |= code[e] << (BITS * e);
    // codes of coordinates 32 m + 8 g .. +7 sit at record byte BITS (4 m + g)
    uint8_t* dst = rec_w + j * kRecStride + BITS * (4 * m + g);
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint32_t*>(dst) = word;
    } else if constexpr (BITS == 2) {
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)word;
    } else {
      // 3 bytes at an odd or even address: a 16-bit and an 8-bit write
      const bool odd = (g & 1) != 0;
      *reinterpret_cast<uint16_t*>(dst + (odd ? 1 : 0)) = (uint16_t)(odd ? word >> 8 : word);
      dst[odd ? 0 : 2] = (uint8_t)(odd ? word : word >> 16);
    }
  }
  float rho = 0.f;
  if constexpr (QJL) {
    if (qjl) {
      rho = __builtin_amdgcn_sqrtf(sum_rows(rr)) * (1.f / 1024.f);
      // the H operands in f16 (+-1 has the same sign bit in both formats)
      u32x4_t Bh[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) Bh[i] = DT == 2 ? B[i] ^ (0x3F803F80u ^ 0x3C003C00u) : B[i];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int neg = ((m & k) ^ ((m >> 1) & (k >> 1))) & 1;
          c0 = mfma_h<1>(Bh[2 * neg], rh[k], c0);
          c1 = mfma_h<1>(Bh[1 + 2 * neg], rh[k], c1);
          c0 = mfma_h<1>(Bh[2 * neg], rl[k], c0);
          c1 = mfma_h<1>(Bh[1 + 2 * neg], rl[k], c1);
        }
        uint32_t bits = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) bits |= (c0[e] < 0.f ? 1u : 0u) << e | (c1[e] < 0.f ? 1u : 0u) << (e + 4);
        // sign byte of coordinates 32 m + 8 g .. +7 in the record's padding
        rec_w[j * kRecStride + 16 * BITS + 4 * m + g] = (uint8_t)bits;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  using Off = typename std::conditional<OFF32, uint32_t, uint64_t>::type;
  const int32_t sm = in.slot;
  if (sm >= 0 && sm < a.num_slots) {
    const uint32_t row = (uint32_t)sm & 15u;
    const uint32_t blk_bytes = (uint32_t)(a.num_heads * a.block_bytes);
    const uint32_t bb = (uint32_t)a.block_bytes;
    Off off;
    if constexpr (OFF32)
      off = __umul24((uint32_t)sm >> 4, blk_bytes) + __umul24(in.head, bb);
    else
      off = (uint64_t)((uint32_t)sm >> 4) * blk_bytes + (uint64_t)in.head * bb;
    if (g < BITS) {
      const u32x4_t r = *reinterpret_cast<const u32x4_t*>(rec_w + j * kRecStride + 16 * g);
      const Off ro = off + (uint32_t)st.rec_off + __umul24(row, (uint32_t)st.rec_bytes) + 16u * (uint32_t)g;
      // non-temporal: the cache is read by later launches, not this one
      // (measured -2% on 2^19 and 2^21 vectors; the same for the 2-byte norm
      // stores was +3%)
      __builtin_nontemporal_store(r, reinterpret_cast<u32x4_t*>(a.pool + ro));
    }
    if (g == 0) {
      const Off no = off + (uint32_t)st.norm_off + 2u * row;
      *reinterpret_cast<__half*>(a.pool + no) = __float2half_rn(fminf(gamma, 65504.f));
    }
    if constexpr (QJL) {
      if (qjl && g == 3) {
        const u32x4_t sg = *reinterpret_cast<const u32x4_t*>(rec_w + j * kRecStride + 16 * BITS);
        const Off so = off + (uint32_t)a.sign_off + 16u * row;
        __builtin_nontemporal_store(sg, reinterpret_cast<u32x4_t*>(a.pool + so));
      }
      if (qjl && g == 1) {
        const Off ro = off + (uint32_t)a.rho_off + 2u * row;
        *reinterpret_cast<__half*>(a.pool + ro) = __float2half_rn(fminf(rho, 65504.f));
      }
    }
  }
  // the next batch rewrites this wave's staging records
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// kMxBatches batches per wave, all loads issued up front.
template <int BITS, int DT, bool OFF32, bool QJL>
__global__ __launch_bounds__(256) void encode_mx_kernel(const EncodeArgs a) {
  __shared__ MxShared<BITS> sh;
  __shared__ MxQjlShared shq;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  // the input loads go first: the set-up's per-lane reads of the argument
  // tables (and their waits) then overlap them instead of preceding them
  const EncodeStream& st = a.stream[blockIdx.y];
  const uint32_t b0 = (blockIdx.x * 4u + (uint32_t)wave) * kMxBatches;
  MxBatch in[kMxBatches];
#pragma unroll
  for (int u = 0; u < kMxBatches; ++u) mx_load(a, st.src, b0 + u, g, j, in[u]);
  u32x4_t B[4];
  mx_setup<BITS, DT, QJL>(a, sh, shq, B, tid);
  __syncthreads();   // bucket table and sign masks
#pragma unroll
  for (int u = 0; u < kMxBatches; ++u) mx_batch<BITS, DT, OFF32, QJL>(a, st, in[u], B, sh, shq, wave, g, j);
}

// TQ_ENCODE_GENERIC=1 keeps 16-bit inputs on encode_kernel (comparison only).
static bool encode_generic_only() {
  static const bool v = [] {
    const char* e = std::getenv("TQ_ENCODE_GENERIC");
    return e && std::atoi(e) == 1;
  }();
  return v;
}

template <int BITS, int DT>
static int launch_bits_dt(const EncodeArgs& a, int streams, bool qjl, hipStream_t s) {
  // 16-byte record stores need 16-byte aligned chunks and record regions
  // (the layout's sizes are multiples of 16; the pool base is checked)
  const bool mx = DT != 0 && !encode_generic_only() && a.num_vectors < ((int64_t)1 << 31) &&
                  a.block_bytes % 16 == 0 && a.stream[0].rec_off % 16 == 0 && a.stream[1].rec_off % 16 == 0 &&
                  (!qjl || a.sign_off % 16 == 0) && (reinterpret_cast<uintptr_t>(a.pool) & 15) == 0;
  if (mx) {
    constexpr int DT16 = DT == 0 ? 1 : DT;
    // 32-bit cache offsets: the whole pool below 4 GiB, block index and
    // per-block bytes below 2^24 (24-bit multiplies)
    const int64_t blocks = a.num_slots / 16, per_block = a.num_heads * a.block_bytes;
    const bool off32 = blocks < ((int64_t)1 << 24) && per_block < ((int64_t)1 << 24) &&
                       blocks * per_block <= ((int64_t)1 << 32) - per_block;
    dim3 gmx((unsigned)((a.num_vectors + 64 * kMxBatches - 1) / (64 * kMxBatches)), (unsigned)streams);
    if (qjl && off32)
      hipLaunchKernelGGL((encode_mx_kernel<BITS, DT16, true, true>), gmx, dim3(256), 0, s, a);
    else if (qjl)
      hipLaunchKernelGGL((encode_mx_kernel<BITS, DT16, false, true>), gmx, dim3(256), 0, s, a);
    else if (off32)
      hipLaunchKernelGGL((encode_mx_kernel<BITS, DT16, true, false>), gmx, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((encode_mx_kernel<BITS, DT16, false, false>), gmx, dim3(256), 0, s, a);
    return (int)hipGetLastError();
  }
  const int64_t groups = (a.num_vectors + 16 * kIters - 1) / (16 * kIters);   // 64 vectors each
  dim3 grid((unsigned)groups, (unsigned)streams);
  if (qjl)
    hipLaunchKernelGGL((encode_kernel<BITS, DT, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((encode_kernel<BITS, DT, false>), grid, dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

template <int BITS>
static int launch_bits(const EncodeArgs& a, int streams, int dt, bool qjl, hipStream_t s) {
  switch (dt) {
    case 0: return launch_bits_dt<BITS, 0>(a, streams, qjl, s);
    case 1: return launch_bits_dt<BITS, 1>(a, streams, qjl, s);
    default: return launch_bits_dt<BITS, 2>(a, streams, qjl, s);
  }
}

int launch_encode(const EncodeArgs& a, int num_streams, int in_dtype, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool qjl = a.stream[0].qjl != 0;
  if (a.num_vectors > (int64_t)(16 * kIters) * 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  switch (a.tab.bits) {
    case 2: return launch_bits<2>(a, num_streams, in_dtype, qjl, s);
    case 3: return launch_bits<3>(a, num_streams, in_dtype, qjl, s);
    case 4: return launch_bits<4>(a, num_streams, in_dtype, qjl, s);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace tq
