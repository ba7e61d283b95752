// tq_octo: the octahedral triplet codec of the OCTOPUS summary (the
// Contributions list: the triplet direction quantizer with norm marginals
// and the uneven bit split; and the Method list): the rotated unit
// direction y = R k / ||k|| is cut into 43 triplets (the last is
// (y126, y127, 0)); each triplet t = rho n keeps its norm rho and the
// direction n mapped by the equal-area octahedral map to (xi, eta) in
// [-1, 1]^2.  xi and eta take (b+1)-bit uniform codes, rho a (b-1)-bit
// Lloyd-Max code, and a 3x3 joint rounding over the nearest direction cell
// and its neighbours picks the codes with the least ||t - rho_hat n_hat||^2.
//
// Encode: one vector per 16-lane row (the in-register FWHT of the encoder),
// the rotated coordinates staged in LDS, then the workgroup's threads take
// the 16 vectors' triplets as one flat list; the direction table sits in LDS.
// Logits: a matrix-core product of the group's rotated queries with keys
// decoded in registers (16 keys x 16 queries per tile); each triplet's
// direction comes from the LDS table scaled by its norm code, and no K_hat
// is written anywhere.

#include <hip/hip_bf16.h>

#include <algorithm>

#include "tq_device.h"
#include "tq_encode_row.h"

namespace tq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 bits of x rounded to nearest even (x finite)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// x = hi + lo + e, hi and lo bf16 (hi = bf16(x), lo = bf16(x - hi)), |e| <=
// 2^-17 |x|: the two halves of a split operand
__device__ __forceinline__ void bf16_split(float x, uint32_t& hi, uint32_t& lo) {
  hi = bf16_bits(x);
  lo = bf16_bits(x - __uint_as_float(hi << 16));
}

template <int B>
struct Octo {
  static constexpr int kBd = B + 1;                  // bits of xi and of eta
  static constexpr int kBn = B - 1;                  // bits of rho
  static constexpr int kNd = 1 << kBd;               // grid cells per axis
  static constexpr int kNr = 1 << kBn;               // norm codes
  static constexpr int kField = 2 * kBd + kBn;       // bits per triplet
  static constexpr int kWords = (kOctoTri * kField + 31) / 32;
  static constexpr int kRec = 4 * kWords;            // bytes per record
};

constexpr int kOctoRowPad = 132;   // LDS floats per row: 128 coordinates, zero pad

// The lower of the two grid columns whose centres -1 + (2 j + 1) / nd
// bracket v: with v in cell j = floor((v + 1) nd / 2), columns j - 1, j when
// v lies in the lower half of the cell, j, j + 1 in the upper half; i.e.
// floor((v + 1) nd / 2 - 1/2).  Clamped to [0, nd - 2], so both columns lie
// on the grid: next to an outer column the pair is that column and its
// neighbour, a superset of the pair's part on the grid.  |v| <= 1 keeps the
// argument at or above -1/2, where truncation toward zero and the floor
// differ only on (-1, 0), which the clamp takes to 0 either way.
__device__ __forceinline__ int octo_block_lo(float v, int nd) {
  const int h = (int)__builtin_fmaf(v, 0.5f * (float)nd, 0.5f * (float)nd - 0.5f);
  return min(max(h, 0), nd - 2);
}

// A buffer resource over the n bytes at p (raw, stride 0, 32-bit data
// format): a load whose offset lies at or past n returns zero and touches
// no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
}

// Copy the direction table ([xi code][eta code] of (x, y, z, 0), nd x nd
// entries) to LDS with every load issued before the first store (a loop
// that stores as it loads waits one memory round trip per iteration);
// indices past the table re-read its last entry and store nothing.  With
// kT the copy is transposed to [eta code][xi code], so that the low 2 kBd
// bits of a triplet field (xi code, then eta code) index it directly.
template <int ND, bool kT>
__device__ __forceinline__ void load_dirs(float4* s_dir, const float* dirs, int tid) {
  constexpr int N = ND * ND, kIt = (N + 255) / 256;
  const float4* src = reinterpret_cast<const float4*>(dirs);
  float4 t[kIt];
#pragma unroll
  for (int r = 0; r < kIt; ++r) t[r] = src[min(tid + 256 * r, N - 1)];
#pragma unroll
  for (int r = 0; r < kIt; ++r) {
    const int i = tid + 256 * r;   // = a ND + c
    if (i < N) s_dir[kT ? (i % ND) * ND + i / ND : i] = t[r];
  }
}

// atan(a) for a in [0, 1] as a * P(a^2), P of degree 7: the odd polynomial
// of kv_cache_vector_encode_amd/fit_atan.py (Lawson's reweighted least
// squares toward the minimax fit), coefficients rounded to fp32; largest
// error 1.34e-7 rad in this fp32 evaluation.
__device__ __forceinline__ float atan01(float a) {
  const float s = a * a;
  float p = -4.054567311e-03f;
  p = __builtin_fmaf(p, s, 2.186295763e-02f);
  p = __builtin_fmaf(p, s, -5.591232702e-02f);
  p = __builtin_fmaf(p, s, 9.642197192e-02f);
  p = __builtin_fmaf(p, s, -1.390862912e-01f);
  p = __builtin_fmaf(p, s, 1.994656622e-01f);
  p = __builtin_fmaf(p, s, -3.332985938e-01f);
  p = __builtin_fmaf(p, s, 9.999993443e-01f);
  return a * p;
}

// atan2(|y|, |x|) (0 when both are 0), through atan01 of the smaller
// magnitude over the larger (the larger floored at 1e-30, so 0 / 0 gives 0).
// The larger and smaller are one max3 and one min with absolute-value
// operands, written out: fmaxf / fminf first canonicalise operands the
// compiler cannot prove canonical (one more instruction each); x and y are
// finite here.
__device__ __forceinline__ float atan2_abs(float y, float x) {
  float mx, mn;
  asm("v_max3_f32 %0, |%2|, |%3|, %4\n\tv_min_f32_e64 %1, |%2|, |%3|"
      : "=&v"(mx), "=&v"(mn)
      : "v"(x), "v"(y), "v"(1e-30f));
  const float t = atan01(mn * __builtin_amdgcn_rcpf(mx));
  return fabsf(y) > fabsf(x) ? 1.57079632679489662f - t : t;
}

// Equal-area octahedral map of the direction of (nx, ny, .) with unit-vector
// z component nz (nx and ny may carry any common positive scale; |nz| may
// exceed 1 by a rounding error): L1 radius sqrt(1 - |nz|), the azimuth
// atan2(|ny|, |nx|) spread linearly along the diamond edge, the lower
// hemisphere reflected across the edge, the signs of nx and ny copied (a
// coordinate of -0 takes the negative side: the map's two sides agree there).
__device__ __forceinline__ void oct_map(float nx, float ny, float nz, float& xi, float& eta) {
  const float r = __builtin_amdgcn_sqrtf(fmaxf(1.f - fabsf(nz), 0.f));
  const float phi = atan2_abs(ny, nx);
  float ae = r * phi * 0.636619772367581343f;   // 2 / pi
  float ax = r - ae;
  if (nz < 0.f) {
    const float t = ax;
    ax = 1.f - ae;
    ae = 1.f - t;
  }
  xi = __builtin_copysignf(ax, nx);
  eta = __builtin_copysignf(ae, ny);
}

template <int B, int DT, bool QJL>
__global__ __launch_bounds__(256) void octo_encode_kernel(const OctoArgs a) {
  using C = Octo<B>;
  // direction table [xi code][eta code], (x, y, z, 0) per entry
  constexpr int kNd = C::kNd;
  __shared__ float4 s_dir[kNd * kNd];
  __shared__ float s_y[16][kOctoRowPad];
  __shared__ uint32_t s_rec[16][C::kWords];
  __shared__ float s_crho[8];
  const int tid = threadIdx.x, row = tid >> 4;
  const int L = tid & 15, ell = perm16(L);
  load_dirs<kNd, true>(s_dir, a.dirs, tid);   // [eta code][xi code]
  if (QJL && tid < 8) s_crho[tid] = a.crho[tid];
  const uint32_t sneg = sign_byte(a.rot, ell);
  uint32_t smask[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (DT == 0) smask[i] = ((sneg >> i) & 1u) << 31;
    else smask[i] = i < 4 ? (((sneg >> (2 * i)) & 1u) << 15) | (((sneg >> (2 * i + 1)) & 1u) << 31) : 0u;
  }
  const FwhtLane fc = fwht_lane(L);
  const int64_t groups = (a.n + 15) / 16;
  // the next group's 8 coordinates are loaded while this one is coded
  constexpr int kRaw = DT == 0 ? 8 : 4;
  uint32_t raw[kRaw];
  auto fetch = [&](int64_t grp) {
    const int64_t vv = grp * 16 + row;
    const int64_t vc = vv < a.n ? vv : a.n - 1;
    const uint4* p = DT == 0 ? reinterpret_cast<const uint4*>(static_cast<const float*>(a.src) + vc * kD + 8 * ell)
                             : reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src) + vc * kD + 8 * ell);
    const uint4 r0 = p[0];
    raw[0] = r0.x; raw[1] = r0.y; raw[2] = r0.z; raw[3] = r0.w;
    if constexpr (DT == 0) {
      const uint4 r1 = p[1];
      raw[4] = r1.x; raw[5] = r1.y; raw[6] = r1.z; raw[7] = r1.w;
    }
  };
  if (blockIdx.x < groups) fetch(blockIdx.x);
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const int64_t v = grp * 16 + row;
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (DT == 0) {
        x[i] = __uint_as_float(raw[i] ^ smask[i]);
      } else {
        const uint32_t wv = raw[i >> 1] ^ smask[i >> 1];
        const uint32_t h = (i & 1) ? (wv >> 16) : (wv & 0xFFFFu);
        if constexpr (DT == 2) x[i] = __uint_as_float(h << 16);
        else x[i] = __half2float(__ushort_as_half((unsigned short)h));
      }
    }
    if (grp + gridDim.x < groups) fetch(grp + gridDim.x);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
    const float gamma = sqrtf(row_sum(ss));
    fwht_row(x, fc);   // lane L: coordinates 8L..8L+7 of H s.x, times fc.sig
    const float g = gamma > 0.f ? fc.sig * kInvSqrtD / gamma : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s_y[row][8 * L + e] = x[e] * g;
    if (L < kOctoRowPad - kD) s_y[row][kD + L] = 0.f;
    for (int w = L; w < C::kWords; w += 16) s_rec[row][w] = 0u;
    __syncthreads();
    // the group's 16 x 43 triplets in one flat list over the 256 threads:
    // 2.69 passes, so the last wave has no third pass (with 43 per 16-lane
    // row every wave ran three)
    // (unrolled, so each pass's row and triplet index are computed once)
#pragma unroll
    for (int f = tid; f < 16 * kOctoTri; f += 256) {
      const int rw = f / kOctoTri, i = f - rw * kOctoTri;
      const float tx = s_y[rw][3 * i], ty = s_y[rw][3 * i + 1], tz = s_y[rw][3 * i + 2];
      const float rr = tx * tx + ty * ty + tz * tz;
      // the map needs z / rho only; the azimuth is scale-free
      const float nz = rr > 0.f ? tz * __builtin_amdgcn_rsqf(rr) : 1.f;
      float xi, eta;
      oct_map(tx, ty, nz, xi, eta);
      const int a0 = octo_block_lo(xi, kNd), c0 = octo_block_lo(eta, kNd);
      // For a unit direction n_hat the error with the best norm code is
      // rho^2 + min_k (c_k^2 - 2 c_k p), p = t . n_hat; every c_k > 0, so
      // that minimum falls as p grows: the 3x3 joint rounding takes the
      // candidate of largest projection (first on ties, xi-major), then the
      // norm code nearest to its p.  That candidate always lies in the 2x2
      // block of the window on the side of the point's quadrant of its cell
      // (columns a0, a0 + 1 and rows c0, c0 + 1): a dense float64 scan of the
      // (xi, eta) square at every bit width finds the best projection of the
      // other five cells never above the block's, equal only on the folds of
      // the map, where mirror cells tie.  So only the block is scanned.
      // In the transposed table the entry of (xi code a, eta code c) sits at
      // a + c nd, which is also the field's direction bits a | c << kBd; so
      // the candidates are base + {0, nd, 1, nd + 1} (xi-major: (a0, c0),
      // (a0, c0 + 1), (a0 + 1, c0), (a0 + 1, c0 + 1)), and the winner's
      // offset is its field's offset as well
      const int base = a0 + (c0 << C::kBd);
      float best = 0.f;
      int bo = 0;
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        const int off = (o >> 1) + (o & 1) * kNd;
        const float4 d = s_dir[base + off];
        const float p = tx * d.x + ty * d.y + tz * d.z;
        if (o == 0 || p > best) {
          best = p;
          bo = off;
        }
      }
      // norm code: the number of ascending thresholds below p (seven
      // independent compares at b = 4; a binary search's dependent chain of
      // compares and selects measured 10% slower, a bucketed table search 0.5%
      // faster)
      uint32_t k = 0;
#pragma unroll
      for (int j = 0; j + 1 < C::kNr; ++j) k += best > a.trho[j] ? 1u : 0u;
      const uint32_t field = (uint32_t)(base + bo) + (k << (2 * C::kBd));
      if constexpr (QJL) {
        // what the codes leave out of the triplet, in place of it (the lane
        // owns these three coordinates)
        const float4 d = s_dir[base + bo];
        const float rk = s_crho[k];
        s_y[rw][3 * i] = __builtin_fmaf(-rk, d.x, tx);
        s_y[rw][3 * i + 1] = __builtin_fmaf(-rk, d.y, ty);
        s_y[rw][3 * i + 2] = __builtin_fmaf(-rk, d.z, tz);
      }
      const int bit = i * C::kField, w = bit >> 5, sh = bit & 31;
      atomicOr(&s_rec[rw][w], field << sh);
      if (sh + C::kField > 32) atomicOr(&s_rec[rw][w + 1], field >> (32 - sh));
    }
    __syncthreads();
    if constexpr (QJL) {
      // one-bit sketch of the residual r (coordinates 0..127 of the row):
      // lane L takes coordinates 8L..8L+7, flips them by the second
      // rotation's signs and runs the row FWHT, after which it holds output
      // coordinates 8 perm16(L) + e of R' r (times fc.sig); bit e of byte
      // perm16(L) of the sign record is [(R' r)_j < 0], rho = ||r||
      float r[8];
      float rr = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        r[e] = s_y[row][8 * L + e];
        rr = __builtin_fmaf(r[e], r[e], rr);
      }
      const float rho = __builtin_amdgcn_sqrtf(row_sum(rr));
      const uint32_t qneg = sign_byte(a.rot_qjl, L);
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = flip(r[e], qneg, e);
      fwht_row(r, fc);
      uint32_t sbits = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) sbits |= ((fc.sig * r[e]) < 0.f ? 1u : 0u) << e;
      if (v < a.n) {
        a.qjl_signs[v * 16 + perm16(L)] = (uint8_t)sbits;
        if (L == 0) a.qjl_rho[v] = __half_as_ushort(__float2half_rn(fminf(rho, 65504.f)));
      }
    }
    if (v < a.n) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + v * C::kRec);
      for (int w = L; w < C::kWords; w += 16) dst[w] = s_rec[row][w];
      if (L == 0) a.gamma[v] = __half_as_ushort(__float2half_rn(fminf(gamma, 65504.f)));
    }
    __syncthreads();   // s_y and s_rec are rewritten by the next group
  }
}

// Logits of a head's group of 1..16 queries against n keys: out = scale *
// gamma * sum_i rho_hat_i (R q)_i . n_hat_i, as a matrix-core product per
// 16-key tile, C[16 keys x 16 queries] += A[16 keys x K] * B[K x 16 queries]
// over the 132 rotated dims (128 plus the zero pad) in an order of the
// kernel's choosing.  Each A element is one decoded coordinate rho_hat *
// n_hat[comp] of key l%16, unpacked from the tile's records in LDS; the B
// operands (the rotated, scaled queries) stay in registers for the whole
// kernel; C[4(l/16)+r][l%16] sits in lane l.  Each wave takes 16-key tiles
// in turn.
//  - 5 steps of 32 dims on v_mfma_f32_16x16x32_bf16, each operand split
//    into bf16 high and low halves (three products per step): 15
//    instructions of 16 cycles per tile instead of 33 fp32 ones of 32.  At
//    b <= 3 the key's halves are read from a table of every field value's
//    products; at b = 4 (a 128 KB table) they are formed in registers.
//  - With the sketch at b = 4: 33 steps of 4 dims on
//    v_mfma_f32_16x16x4f32, fp32 in and out.
//  - The sketch (OCTOPUS-QJL) adds 4 steps of 32 coordinates on bf16-split
//    operands to the same accumulator.
constexpr int kOctoMfmaTile = 128;   // keys per tile step (2 tiles of 16 per wave)

// Waves per SIMD: 4 at b = 2; 3 at b = 3 (the bf16 operands take 134
// VGPRs: 154 against 166 us at 4 waves with 3 spills, on the 4.2M keys of
// llama70b), at b = 4 (the split in registers takes 168) and with the
// sketch (its 32 more query registers)
template <int B, bool QJL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QJL || B >= 3 ? 3 : 4))) void octo_logits_mfma_kernel(
    const OctoArgs a) {
  using C = Octo<B>;
  constexpr int kStride = C::kWords + 1;
  constexpr int kQd = 132;
  __shared__ float4 s_dir[C::kNd * C::kNd];
  // the rotated queries are read into registers once, before the first
  // tile's records are staged: the two share their LDS
  __shared__ union {
    struct {
      float q[16][kQd];
      float w[QJL ? 16 : 1][kD];   // OCTOPUS-QJL: R' R q (scaled), natural order
    } qw;
    struct {                       // one tile of keys, zeros past the last
      uint32_t rec[kOctoMfmaTile * kStride];
      float g[kOctoMfmaTile];                  // norms
      uint4 sg[QJL ? kOctoMfmaTile : 1];       // OCTOPUS-QJL: sign sketches
      float sk[QJL ? kOctoMfmaTile : 1];       // and sqrt(pi/2)/sqrt(d) times their norms
    } t;
  } s_u;
  auto& s_q = s_u.qw.q;
  auto& s_w = s_u.qw.w;
  static_assert(sizeof(s_u.qw) == sizeof(float) * (16 * kQd + (QJL ? 16 : 1) * kD), "q and w are contiguous");
  uint32_t* const s_rec = s_u.t.rec;
  __shared__ float s_rho[8];
  // b <= 3: by field value (the field's bits as the index), the products
  // (x, y, z) = rho n of its norm code and direction, split into bf16
  // halves: (x, y), (y, z) of the high parts, then of the low parts
  constexpr int kPtN = C::kNr * C::kNd * C::kNd;
  constexpr bool kPT = kPtN <= 1024;
  __shared__ uint4 s_pt[kPT ? kPtN : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  load_dirs<C::kNd, true>(s_dir, a.dirs, tid);
  if (tid < 8) s_rho[tid] = a.crho[tid];
  // queries past the group (and, with the sketch, their R' R q) stay zero
  float* qf = &s_q[0][0];
  for (int i = tid; i < 16 * kQd + (QJL ? 16 * kD : 0); i += 256) qf[i] = 0.f;
  __syncthreads();
  if constexpr (kPT) {   // read after the tile barriers below
    for (int e = tid; e < kPtN; e += 256) {
      const float4 d = s_dir[e & (C::kNd * C::kNd - 1)];
      const float r = s_rho[e >> (2 * C::kBd)];
      uint32_t xh, xl, yh, yl, zh, zl;
      bf16_split(r * d.x, xh, xl);
      bf16_split(r * d.y, yh, yl);
      bf16_split(r * d.z, zh, zl);
      s_pt[e] = make_uint4(xh | (yh << 16), yh | (zh << 16), xl | (yl << 16), yl | (zl << 16));
    }
  }
  {
    const int row = tid >> 4, L = tid & 15, ell = perm16(L);
    const int rq = row < a.group ? row : 0;
    const uint32_t sneg = sign_byte(a.rot, ell);
    uint32_t smask[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) smask[i] = ((sneg >> i) & 1u) << 31;
    float x[8];
    load8_signed<0>(a.q, ((int64_t)head * a.group + rq) * kD + 8 * ell, smask, x);
    const FwhtLane fc = fwht_lane(L);
    fwht_row(x, fc);
    const float g = fc.sig * kInvSqrtD * a.scale;
    if (row < a.group) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_q[row][8 * L + e] = x[e] * g;
    }
    if constexpr (QJL) {
      // the residual sketch is read against R' (R q): the second rotation
      // of the lane's natural coordinates 8L..8L+7, after which the lane
      // holds coordinates 8 perm16(L) + e (times fc.sig), as in the encoder
      const uint32_t qneg = sign_byte(a.rot_qjl, L);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = flip(x[e] * g, qneg, e);
      fwht_row(x, fc);
      if (row < a.group) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s_w[row][8 * perm16(L) + e] = x[e] * fc.sig * kInvSqrtD;
      }
    }
  }
  __syncthreads();
  // The contraction runs over the 44 triplets (the last all-zero in q) in
  // an order of our choosing: lanes with l/16 = kk take triplets kk, kk+4,
  // ..., kk+40, one per 3 consecutive steps (components x, y, z), so each
  // lane decodes a triplet once and feeds it to 3 products.
  const int col = lane & 15, kk = lane >> 4;
  // bf16-split operands everywhere but with the sketch at b = 4 (the
  // sketch's 32 query registers beside them spilled there: 45 against 42 us
  // on decode_1x32768); that case keeps fp32 operands, step 3m + c taking
  // component c of triplet 4m + kk
  constexpr bool kSplit = kPT || !QJL;
  float qb[kSplit ? 1 : 33];
  // bf16 operands: K slot 8s + e of step s (e < 8) is component
  // c % 3 of triplet 4 (c / 3) + kk, c = 8s + e < 33 (zero past 32); the
  // queries split into bf16 high and low halves, the products
  // hi.hi + hi.lo + lo.hi lose |q_lo k_lo| and the halves' rounding, about
  // 2^-15 |q_i k_i| a term
  u32x4 qh[kSplit ? 5 : 1], ql[kSplit ? 5 : 1];
  if constexpr (kSplit) {
#pragma unroll
    for (int st = 0; st < 5; ++st)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t h[2], l[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int c = 8 * st + 2 * w + hf, dim = 3 * (4 * (c / 3) + kk) + c % 3;
          bf16_split(c < 33 && dim < kD ? s_q[col][dim] : 0.f, h[hf], l[hf]);
        }
        qh[st][w] = h[0] | (h[1] << 16);
        ql[st][w] = l[0] | (l[1] << 16);
      }
  } else {
#pragma unroll
    for (int m = 0; m < 11; ++m)
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const int dim = 3 * (4 * m + kk) + c;
        qb[3 * m + c] = dim < kD ? s_q[col][dim] : 0.f;
      }
  }
  // OCTOPUS-QJL: 4 more steps of 32 sketch coordinates on bf16-split
  // operands; word w of lane kk in step s holds coordinates j = 32 s + 4 kk
  // + w and j + 16, whose sign bits sit at bits 4 kk + w and 4 kk + w + 16
  // of word s of the key's sign record
  u32x4 wh[QJL ? 4 : 1], wl[QJL ? 4 : 1];
  if constexpr (QJL) {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t h0, l0, h1, l1;
        bf16_split(s_w[col][32 * st + 4 * kk + w], h0, l0);
        bf16_split(s_w[col][32 * st + 4 * kk + w + 16], h1, l1);
        wh[st][w] = h0 | (h1 << 16);
        wl[st][w] = l0 | (l1 << 16);
      }
  }
  // the workgroup walks tiles blockIdx.x, blockIdx.x + gridDim.x, ... of
  // its head, so the table and the queries are set up once per workgroup;
  // the next tile's records (and sketches) are loaded into registers while
  // this one is multiplied, its norms once the products are done (a
  // register fewer held through them), so the products read LDS only (the
  // barrier at the top of the tile loop also orders the reads of s_q above
  // before the first records overwrite it)
  const int64_t ntiles = (a.n + kOctoMfmaTile - 1) / kOctoMfmaTile;
  constexpr int kPre = (kOctoMfmaTile * C::kWords + 255) / 256;
  uint32_t pre[kPre];
  uint16_t pg, pr;              // norm and sketch norm of key tid % 128
  uint32_t ps[QJL ? 2 : 1];     // sketch words tid and tid + 256 of the tile
  auto fetch = [&](int64_t tl) {
    const int64_t k0 = tl * kOctoMfmaTile;
    const int n_ = (int)(a.n - k0 < kOctoMfmaTile ? a.n - k0 : kOctoMfmaTile);
    const int64_t kb = (int64_t)head * a.n + k0;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.codes + kb * C::kRec);
#pragma unroll
    for (int r = 0; r < kPre; ++r) {
      const int i = tid + 256 * r;
      pre[r] = i < n_ * C::kWords ? src[i] : 0u;
    }
    // indices past the tile's last key re-read it (stored as zeros, or
    // multiplied by a zero norm)
    if constexpr (QJL) {
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(a.qjl_signs + kb * 16);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = tid + 256 * r;
        ps[r] = sp[4 * min(i >> 2, n_ - 1) + (i & 3)];
      }
    }
  };
  auto fetch_norms = [&](int64_t tl) {
    const int64_t k0 = tl * kOctoMfmaTile;
    const int n_ = (int)(a.n - k0 < kOctoMfmaTile ? a.n - k0 : kOctoMfmaTile);
    const int64_t kg = (int64_t)head * a.n + k0 + min(tid & (kOctoMfmaTile - 1), n_ - 1);
    pg = a.gamma[kg];
    if constexpr (QJL) pr = a.qjl_rho[kg];
  };
  if (blockIdx.x < ntiles) {
    fetch(blockIdx.x);
    fetch_norms(blockIdx.x);
  }
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
  const int64_t key0 = tile * kOctoMfmaTile;
  const int nk = (int)(a.n - key0 < kOctoMfmaTile ? a.n - key0 : kOctoMfmaTile);
  __syncthreads();   // the previous tile's records are no longer read
#pragma unroll
  for (int r = 0; r < kPre; ++r) {
    const int i = tid + 256 * r;
    if (i < kOctoMfmaTile * C::kWords) {
      const int k = i / C::kWords, w = i - k * C::kWords;
      s_rec[k * kStride + w] = pre[r];   // rows past the end hold zeros
    }
  }
  if (tid < kOctoMfmaTile) {
    s_u.t.g[tid] = tid < nk ? __half2float(__ushort_as_half(pg)) : 0.f;
    if constexpr (QJL) s_u.t.sk[tid] = tid < nk ? 0.1107783657f * __half2float(__ushort_as_half(pr)) : 0.f;
  }
  if constexpr (QJL) {
#pragma unroll
    for (int r = 0; r < 2; ++r) reinterpret_cast<uint32_t*>(s_u.t.sg)[tid + 256 * r] = ps[r];
  }
  __syncthreads();
  if (tile + gridDim.x < ntiles) fetch(tile + gridDim.x);
  for (int t = wave; t * 16 < nk; t += 4) {
    const uint32_t* rec = s_rec + (t * 16 + col) * kStride;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto field = [&](int m) -> uint32_t {
      const int j = 4 * m + kk;               // triplet 43 reads zero record bits; its q is 0
      const int bit = j * C::kField, wi = bit >> 5, sh = bit & 31;
      return (uint32_t)((((uint64_t)rec[wi + 1] << 32) | rec[wi]) >> sh) & ((1u << C::kField) - 1u);
    };
    if constexpr (kPT) {
      // A in the slot order of qh/ql: per pair of triplets m, m+1 the words
      // (x_m, y_m), (z_m, x_m+1), (y_m+1, z_m+1), from the table's (x, y)
      // and (y, z) words and one byte permute; triplet 10 ends the list
      uint4 e[11];
      uint32_t ah[20], al[20];
      auto word = [&](int w) {   // the words of slots 2w, 2w + 1, high and low parts
        const int p = w / 3, r = w % 3;
        if (w >= 17) {
          ah[w] = al[w] = 0u;
        } else if (w >= 15) {    // triplet 10: (x, y), (z, 0)
          ah[w] = w == 15 ? e[10].x : e[10].y >> 16;
          al[w] = w == 15 ? e[10].z : e[10].w >> 16;
        } else if (r == 0) {
          ah[w] = e[2 * p].x;
          al[w] = e[2 * p].z;
        } else if (r == 1) {
          ah[w] = __builtin_amdgcn_perm(e[2 * p + 1].x, e[2 * p].y, 0x05040302u);
          al[w] = __builtin_amdgcn_perm(e[2 * p + 1].z, e[2 * p].w, 0x05040302u);
        } else {
          ah[w] = e[2 * p + 1].y;
          al[w] = e[2 * p + 1].w;
        }
      };
      // step st reads triplets up to (8 st + 7) / 3 (and 10 at st = 3), so
      // the table reads are issued one step ahead and few are live at once
      constexpr int kLast[5] = {2, 5, 7, 10, 10};
#pragma unroll
      for (int m = 0; m <= kLast[0]; ++m) e[m] = s_pt[field(m)];
#pragma unroll
      for (int st = 0; st < 5; ++st) {
        if (st + 1 < 5) {
#pragma unroll
          for (int m = kLast[st] + 1; m <= kLast[st + 1]; ++m) e[m] = s_pt[field(m)];
        }
#pragma unroll
        for (int w = 4 * st; w < 4 * st + 4; ++w) word(w);
        const u32x4 h = {ah[4 * st], ah[4 * st + 1], ah[4 * st + 2], ah[4 * st + 3]};
        const u32x4 l = {al[4 * st], al[4 * st + 1], al[4 * st + 2], al[4 * st + 3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, qh[st]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, ql[st]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, l), __builtin_bit_cast(bf16x8, qh[st]), acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (kSplit) {
      // b = 4: the key's products formed in registers and split there (hi
      // the value truncated to bf16, lo = bf16(x - hi), |lo| <= 2^-8 |x|),
      // slot c = component c % 3 of triplet c / 3, zero past 32
      float v[40];
#pragma unroll
      for (int c = 33; c < 40; ++c) v[c] = 0.f;
      auto trip = [&](int m) {
        const uint32_t f = field(m);
        const float4 d = s_dir[f & (C::kNd * C::kNd - 1)];
        const float r = s_rho[f >> (2 * C::kBd)];
        v[3 * m] = r * d.x;
        v[3 * m + 1] = r * d.y;
        v[3 * m + 2] = r * d.z;
      };
      constexpr int kLast[5] = {2, 5, 7, 10, 10};
#pragma unroll
      for (int m = 0; m <= kLast[0]; ++m) trip(m);
#pragma unroll
      for (int st = 0; st < 5; ++st) {
        if (st + 1 < 5) {
#pragma unroll
          for (int m = kLast[st] + 1; m <= kLast[st + 1]; ++m) trip(m);
        }
        u32x4 h, l;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const float x0 = v[8 * st + 2 * w4], x1 = v[8 * st + 2 * w4 + 1];
          const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
          h[w4] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          const bf16x2 lo = {(__bf16)(x0 - __uint_as_float(b0 & 0xFFFF0000u)), (__bf16)(x1 - __uint_as_float(b1 & 0xFFFF0000u))};
          l[w4] = __builtin_bit_cast(uint32_t, lo);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, qh[st]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, ql[st]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, l), __builtin_bit_cast(bf16x8, qh[st]), acc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 11; ++m) {
        const uint32_t f = field(m);
        const float4 d = s_dir[f & (C::kNd * C::kNd - 1)];
        const float r = s_rho[f >> (2 * C::kBd)];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r * d.x, qb[3 * m], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r * d.y, qb[3 * m + 1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r * d.z, qb[3 * m + 2], acc, 0, 0, 0);
      }
    }
    if constexpr (QJL) {
      // A[key][j] = +-sqrt(pi/2)/sqrt(d) rho16 by the key's sign bit j
      // (set: negative), so the products add the residual estimate
      // sqrt(pi/2)/sqrt(d) rho16 sum_j sgn_j (R' R q)_j to the logit
      const uint4 sg = s_u.t.sg[t * 16 + col];
      const float sk = s_u.t.sk[t * 16 + col];   // zero past the last key
      uint32_t skh, skl;
      bf16_split(sk, skh, skl);
      const uint32_t bh = skh * 0x10001u, bl = skl * 0x10001u;   // both halves
      const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        u32x4 h, l;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // sign bits 4kk + w and 4kk + w + 16 moved to 15 and 31 (negating
          // both halves of a split value negates it exactly)
          const uint32_t neg = (sw[st] << (15 - 4 * kk - w)) & 0x80008000u;
          h[w] = bh ^ neg;
          l[w] = bl ^ neg;
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, wh[st]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, wl[st]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, l), __builtin_bit_cast(bf16x8, wh[st]), acc, 0, 0, 0);
      }
    }
    if (col < a.group) {
      float* o = a.out + ((int64_t)head * a.group + col) * a.n + key0 + t * 16 + 4 * kk;
      const float4 g = *reinterpret_cast<const float4*>(&s_u.t.g[t * 16 + 4 * kk]);
      const float gr[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (t * 16 + 4 * kk + r < nk) o[r] = acc[r] * gr[r];
    }
  }
  if (tile + gridDim.x < ntiles) fetch_norms(tile + gridDim.x);
  }
}

template <int B, bool QJL>
static void octo_enc_q(const OctoArgs& a, dim3 grid, hipStream_t s) {
  if (a.dtype == 0) hipLaunchKernelGGL((octo_encode_kernel<B, 0, QJL>), grid, dim3(256), 0, s, a);
  else if (a.dtype == 1) hipLaunchKernelGGL((octo_encode_kernel<B, 1, QJL>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((octo_encode_kernel<B, 2, QJL>), grid, dim3(256), 0, s, a);
}
template <int B>
static void octo_enc(const OctoArgs& a, dim3 grid, hipStream_t s) {
  if (a.qjl_signs) octo_enc_q<B, true>(a, grid, s);
  else octo_enc_q<B, false>(a, grid, s);
}

int launch_octo_encode(const OctoArgs& a, int bits, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t groups = (a.n + 15) / 16;
  if (a.n <= 0) return (int)hipErrorInvalidValue;
  // The direction table is loaded once per workgroup, and each workgroup
  // loops over groups of 16 vectors.  As many workgroups as fit on the 256
  // CUs at once, so the whole grid is resident in one round: 6 per CU at
  // b = 4 (25.6 KB of LDS each), 8 (the wave limit) at b = 2, 3.  Measured
  // against 4 per CU: 746 against 850 us (b = 3, 4.2M vectors); b = 4 with
  // a bordered 28 KB table, 5 per CU: 64.4 against 69.8 us (262k vectors).
  const int64_t cap = 256 * (bits == 4 ? 6 : 8);
  const dim3 grid((unsigned)(groups < cap ? groups : cap));
  switch (bits) {
    case 2: octo_enc<2>(a, grid, s); break;
    case 3: octo_enc<3>(a, grid, s); break;
    case 4: octo_enc<4>(a, grid, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <int B>
static void octo_log_mfma(const OctoArgs& a, dim3 grid, hipStream_t s) {
  if (a.qjl_signs) hipLaunchKernelGGL((octo_logits_mfma_kernel<B, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((octo_logits_mfma_kernel<B, false>), grid, dim3(256), 0, s, a);
}

int launch_octo_logits(const OctoArgs& a, int bits, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.n <= 0 || a.heads < 1 || a.heads > 65535 || a.group < 1 || a.group > kOctoMaxGroup)
    return (int)hipErrorInvalidValue;
  // about as many workgroups as are resident at once (waves per SIMD: 4 at
  // b = 2, 3 at b = 3, 4 and with the sketch; one workgroup's wave on each
  // SIMD), spread over
  // the heads, each looping over tiles of its head (the table and the
  // queries are set up once per workgroup)
  const int64_t wgs = 256 * (a.qjl_signs || bits >= 3 ? 3 : 4);
  const int64_t tiles = std::min((a.n + kOctoMfmaTile - 1) / kOctoMfmaTile, std::max<int64_t>(1, wgs / a.heads));
  const dim3 grid((unsigned)tiles, (unsigned)a.heads);
  switch (bits) {
    case 2: octo_log_mfma<2>(a, grid, s); break;
    case 3: octo_log_mfma<3>(a, grid, s); break;
    case 4: octo_log_mfma<4>(a, grid, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}


// Decode-attend over triplet-coded keys and values of one head per
// workgroup row ([P3] Method step 7: every score and every value from its
// triplets' norms and directions, no K_hat or V_hat written; [P2] attention
// softmax(q K^T scale) V): a split of split_len keys per workgroup, staged
// 128 keys at a time (records and norms of keys and values), each wave
// taking a 32-key sub-tile of the chunk and keeping its own online softmax,
// in log2 units (scale * log2(e) folded into the queries), and accumulators.
//  - Scores: the logits kernel's product at b = 4, C[16 keys x 16 queries]
//    over 5 steps of 32 rotated dims on bf16-split operands (three bf16
//    products per step, about 2^-15 relative a term), twice, times gamma_k.
//  - Values: C[16 rows x 16 queries] += A[16 rows x 32 keys] * B[32 keys x 16
//    queries] on 16-bit operands with fp32 accumulation, B = f16(p gamma_v)
//    through LDS.  The 144 rows of the 9 row tiles are (triplet, component)
//    pairs: row m of tile 3u + c is component c of triplet 16u + m, so a
//    lane decodes triplet 16u + col of its 8 keys once for three products:
//    at b <= 3 from an LDS table of the three f16 products rho_k n for every
//    field value (one read per triplet); at b = 4, where that table would
//    take 64 KB, from the field's direction and norm (f16 direction and
//    norm tables multiplied in f16 measured 3% slower).  Rows past dim 127
//    (triplet 42's pad component, triplets 43..47) are never stored.  The
//    operands' rounding (2^-11 relative) is far inside the output bar.
//  - The 4 waves' (o_rot, m, l) are merged in LDS in a fixed order, and the
//    split writes one partial (m in natural-log units); merge_kernel
//    combines a head's splits, normalises and rotates back.
// 2 waves per SIMD (190-206 VGPRs) and about two workgroups per CU in all:
// at 3 waves the split scores spilled 80 registers; against the fp32 scores
// at 3 waves, 40 against 44 us on decode_1x32768, 307 against 311 us on
// llama70b
template <int B>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void octo_attend_kernel(const OctoArgs a) {
  using C = Octo<B>;
  constexpr int kStride = C::kWords + 1;
  constexpr int kQd = 132;
  constexpr int kCh = kOctoAttChunk;
  __shared__ float4 s_dir[C::kNd * C::kNd];
  __shared__ union {
    float q[16][kQd];
    struct {
      uint32_t rec[2][kCh * kStride];   // key, value records of the chunk
      float g[2][kCh];                  // their norms (0 past the chunk's end)
    } ch;
  } s_u;
  __shared__ float s_rho[8];
  __shared__ float s_p[4][16][36];      // per wave: p * gamma_v, [query][key of the 32-key sub-tile]
  __shared__ float s_wml[4][2][16];     // per wave: m (log2 units), l of each query, for the final merge
  // b <= 3: by field value (the field's bits as the index), the f16 values
  // rho n_x, rho n_y (low, high half of .x), rho n_z (low half of .y)
  constexpr int kVtN = C::kNr * C::kNd * C::kNd;
  constexpr bool kVT = kVtN <= 1024;
  __shared__ uint2 s_vt[kVT ? kVtN : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y, split = blockIdx.x;
  const int64_t kb0 = (int64_t)split * a.split_len;
  const int64_t kb1 = a.n < kb0 + a.split_len ? a.n : kb0 + a.split_len;
  const float LOG2E = 1.4426950408889634f;
  load_dirs<C::kNd, true>(s_dir, a.dirs, tid);
  if (tid < 8) s_rho[tid] = a.crho[tid];
  float* qf = &s_u.q[0][0];
  for (int i = tid; i < 16 * kQd; i += 256) qf[i] = 0.f;   // queries past the group stay zero
  __syncthreads();
  if constexpr (kVT) {
    for (int e = tid; e < kVtN; e += 256) {
      const float4 d = s_dir[e & (C::kNd * C::kNd - 1)];
      const float r = s_rho[e >> (2 * C::kBd)];
      const _Float16 hx = (_Float16)(r * d.x), hy = (_Float16)(r * d.y), hz = (_Float16)(r * d.z);
      s_vt[e] = make_uint2((uint32_t)__builtin_bit_cast(uint16_t, hx) | ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16),
                           (uint32_t)__builtin_bit_cast(uint16_t, hz));
    }
  }
  {
    const int row = tid >> 4, L = tid & 15, ell = perm16(L);
    const int rq = row < a.group ? row : 0;
    const uint32_t sneg = sign_byte(a.rot, ell);
    uint32_t smask[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) smask[i] = ((sneg >> i) & 1u) << 31;
    float x[8];
    load8_signed<0>(a.q, ((int64_t)head * a.group + rq) * kD + 8 * ell, smask, x);
    const FwhtLane fc = fwht_lane(L);
    fwht_row(x, fc);
    const float g = fc.sig * kInvSqrtD * a.scale * LOG2E;
    if (row < a.group) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_u.q[row][8 * L + e] = x[e] * g;
    }
  }
  __syncthreads();
  const int col = lane & 15, kk = lane >> 4;
  // bf16-split query operands: K slot 8s + e of step s is component c % 3
  // of triplet 4 (c / 3) + kk, c = 8s + e < 33 (zero past 32)
  u32x4 qh[5], ql[5];
#pragma unroll
  for (int st = 0; st < 5; ++st)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t h[2], l[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int c = 8 * st + 2 * w + hf, dim = 3 * (4 * (c / 3) + kk) + c % 3;
        bf16_split(c < 33 && dim < kD ? s_u.q[col][dim] : 0.f, h[hf], l[hf]);
      }
      qh[st][w] = h[0] | (h[1] << 16);
      ql[st][w] = l[0] | (l[1] << 16);
    }
  float run_m = -INFINITY, run_l = 0.f;
  f32x4 acc[9];
#pragma unroll
  for (int T = 0; T < 9; ++T) acc[T] = (f32x4){0.f, 0.f, 0.f, 0.f};
  auto field_of = [&](const uint32_t* rec, int j) -> uint32_t {
    const int bit = j * C::kField, wi = bit >> 5, sh = bit & 31;
    return (uint32_t)((((uint64_t)rec[wi + 1] << 32) | rec[wi]) >> sh) & ((1u << C::kField) - 1u);
  };
  const uint8_t* kcod = a.codes + (int64_t)head * a.n * C::kRec;
  const uint8_t* vcod = a.vcodes + (int64_t)head * a.n * C::kRec;
  const uint16_t* kg = a.gamma + (int64_t)head * a.n;
  const uint16_t* vg = a.vgamma + (int64_t)head * a.n;
  for (int64_t c0 = kb0; c0 < kb1; c0 += kCh) {   // the same trip count in every wave
    const int nk = (int)(kb1 - c0 < kCh ? kb1 - c0 : kCh);
    // the chunk's records and norms, every load issued before the first
    // store: the nk records are nk * kWords consecutive words, read through
    // a range of that many words (slots past them load as zeros)
    constexpr int kIt = (kCh * C::kWords + 255) / 256;
    const int nb = 4 * nk * C::kWords;   // bytes of the chunk's records
    const uint8_t* kc = kcod + c0 * C::kRec;
    const uint8_t* vc = vcod + c0 * C::kRec;
    uint32_t kr[kIt], vr[kIt];
#pragma unroll
    for (int r = 0; r < kIt; ++r) {   // pass r reads bytes [1024 r, 1024 r + 1024)
      // the same for every lane: read it from the first so the range stays scalar
      const int left = __builtin_amdgcn_readfirstlane(max(nb - 1024 * r, 0));
      kr[r] = __builtin_amdgcn_raw_buffer_load_b32(byte_range(kc + 1024 * r, left), 4 * tid, 0, 0);
      vr[r] = __builtin_amdgcn_raw_buffer_load_b32(byte_range(vc + 1024 * r, left), 4 * tid, 0, 0);
    }
    const int tc = min(tid & (kCh - 1), nk - 1);
    const uint16_t gk16 = kg[c0 + tc], gv16 = vg[c0 + tc];
    __syncthreads();   // the previous chunk (or the queries) is no longer read
#pragma unroll
    for (int r = 0; r < kIt; ++r) {
      const int i = tid + 256 * r;
      if (i < kCh * C::kWords) {
        const int k = i / C::kWords, w = i - k * C::kWords;
        s_u.ch.rec[0][k * kStride + w] = kr[r];
        s_u.ch.rec[1][k * kStride + w] = vr[r];
      }
    }
    if (tid < kCh) {
      const bool in = tid < nk;
      s_u.ch.g[0][tid] = in ? __half2float(__ushort_as_half(gk16)) : 0.f;
      s_u.ch.g[1][tid] = in ? __half2float(__ushort_as_half(gv16)) : 0.f;
    }
    __syncthreads();
    for (int t = wave; t * 32 < nk; t += 4) {
      // ---- scores of keys 32t .. 32t+31, two 16-key products: row 4kk + r
      // of half X is key 32t + 16X + 4kk + r, for query col
      f32x4 sl[2];
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        const uint32_t* rk = s_u.ch.rec[0] + (t * 32 + 16 * X + col) * kStride;
        sl[X] = (f32x4){0.f, 0.f, 0.f, 0.f};
        float v[40];   // slot c: component c % 3 of triplet c / 3, zero past 32
#pragma unroll
        for (int c = 33; c < 40; ++c) v[c] = 0.f;
        auto trip = [&](int m) {
          const uint32_t f = field_of(rk, 4 * m + kk);   // triplet 43 reads zero bits; its q is 0
          const float4 d = s_dir[f & (C::kNd * C::kNd - 1)];
          const float r = s_rho[f >> (2 * C::kBd)];
          v[3 * m] = r * d.x;
          v[3 * m + 1] = r * d.y;
          v[3 * m + 2] = r * d.z;
        };
        constexpr int kLast[5] = {2, 5, 7, 10, 10};
#pragma unroll
        for (int m = 0; m <= kLast[0]; ++m) trip(m);
#pragma unroll
        for (int st = 0; st < 5; ++st) {
          if (st + 1 < 5) {
#pragma unroll
            for (int m = kLast[st] + 1; m <= kLast[st + 1]; ++m) trip(m);
          }
          u32x4 h, l;
#pragma unroll
          for (int w4 = 0; w4 < 4; ++w4) {
            const float x0 = v[8 * st + 2 * w4], x1 = v[8 * st + 2 * w4 + 1];
            const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
            h[w4] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 lo = {(__bf16)(x0 - __uint_as_float(b0 & 0xFFFF0000u)), (__bf16)(x1 - __uint_as_float(b1 & 0xFFFF0000u))};
            l[w4] = __builtin_bit_cast(uint32_t, lo);
          }
          sl[X] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, qh[st]), sl[X], 0, 0, 0);
          sl[X] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, ql[st]), sl[X], 0, 0, 0);
          sl[X] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, l), __builtin_bit_cast(bf16x8, qh[st]), sl[X], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float sc[8];
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = t * 32 + 16 * X + 4 * kk + r;
          sc[4 * X + r] = key < nk ? sl[X][r] * s_u.ch.g[0][key] : -INFINITY;
        }
      // ---- online softmax for query col over the 32 keys
      float bm = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) bm = fmaxf(bm, sc[i]);
      bm = max_rows(bm);
      const float new_m = fmaxf(run_m, bm);
      if (__builtin_amdgcn_ballot_w64(new_m > run_m) != 0) {
        const float alpha = run_m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(run_m - new_m);
        run_l *= alpha;
#pragma unroll
        for (int T = 0; T < 9; ++T) acc[T] *= alpha;
      }
      run_m = new_m;
      const float mref = new_m == -INFINITY ? 0.f : new_m;
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * X + 4 * kk + r;
          const float p = __builtin_amdgcn_exp2f(sc[4 * X + r] - mref);   // exp2(-inf) = 0
          run_l += p;
          s_p[wave][col][key] = p * s_u.ch.g[1][t * 32 + key];
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // ---- values: one 32-key product per row tile on 16-bit operands
      // (fp32 accumulation).  Lane (kk, col) holds K slots 8kk .. 8kk+7,
      // keys 32t + 8kk + i: B = f16(p gamma_v) of query col, A = f16 of the
      // components of triplet 16u + col of those keys (row col of tiles 3u,
      // 3u+1, 3u+2)
      f16x8 bv;
#pragma unroll
      for (int i = 0; i < 8; ++i) bv[i] = (_Float16)s_p[wave][col][8 * kk + i];
      if constexpr (kVT) {
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          // rows of triplets past 42 and triplet 42's z land in dims >= 128,
          // which the partial store skips: their table reads need only stay
          // inside the record
          const int jc = min(16 * u + col, kOctoTri - 1);
          uint32_t xy[8], zz[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint2 e = s_vt[field_of(s_u.ch.rec[1] + (t * 32 + 8 * kk + i) * kStride, jc)];
            xy[i] = e.x;
            zz[i] = e.y;
          }
          u32x4 px, py, pz;   // f16 pairs (key 2w, key 2w + 1)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            px[w] = __builtin_amdgcn_perm(xy[2 * w + 1], xy[2 * w], 0x05040100u);
            py[w] = __builtin_amdgcn_perm(xy[2 * w + 1], xy[2 * w], 0x07060302u);
            pz[w] = __builtin_amdgcn_perm(zz[2 * w + 1], zz[2 * w], 0x05040100u);
          }
          acc[3 * u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, px), bv, acc[3 * u], 0, 0, 0);
          acc[3 * u + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, py), bv, acc[3 * u + 1], 0, 0, 0);
          acc[3 * u + 2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, pz), bv, acc[3 * u + 2], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 3; ++u) {
          const int jc = min(16 * u + col, kOctoTri - 1);   // as above
          uint32_t xy[8], zz[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t f = field_of(s_u.ch.rec[1] + (t * 32 + 8 * kk + i) * kStride, jc);
            const float4 d = s_dir[f & (C::kNd * C::kNd - 1)];
            const float r = s_rho[f >> (2 * C::kBd)];
            const f16x2 hxy = {(_Float16)(r * d.x), (_Float16)(r * d.y)};
            xy[i] = __builtin_bit_cast(uint32_t, hxy);
            zz[i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(r * d.z));
          }
          u32x4 px, py, pz;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            px[w] = __builtin_amdgcn_perm(xy[2 * w + 1], xy[2 * w], 0x05040100u);
            py[w] = __builtin_amdgcn_perm(xy[2 * w + 1], xy[2 * w], 0x07060302u);
            pz[w] = __builtin_amdgcn_perm(zz[2 * w + 1], zz[2 * w], 0x05040100u);
          }
          acc[3 * u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, px), bv, acc[3 * u], 0, 0, 0);
          acc[3 * u + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, py), bv, acc[3 * u + 1], 0, 0, 0);
          acc[3 * u + 2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, pz), bv, acc[3 * u + 2], 0, 0, 0);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();   // s_p is rewritten by the next sub-tile
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  // ---- the split's partial: the 4 waves' (m, l, o_rot) merged in LDS in a
  // fixed order (w0 + w1 + w2 + w3, deterministic), written by wave 3.
  // Rows 4kk + r of tile 3u + c are component c of triplet 16u + 4kk + r,
  // i.e. dim 3 (16u + 4kk + r) + c.
  run_l = sum_rows(run_l);
  __syncthreads();   // every wave is done with the chunk buffers
  if (kk == 0) {
    s_wml[wave][0][col] = run_m;
    s_wml[wave][1][col] = run_l;
  }
  __syncthreads();
  float M = s_wml[0][0][col], L = 0.f;
#pragma unroll
  for (int w = 1; w < 4; ++w) M = fmaxf(M, s_wml[w][0][col]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = s_wml[w][0][col];
    L += (mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M)) * s_wml[w][1][col];
  }
  const float alpha = run_m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(run_m - M);   // M >= run_m
  float* const buf = reinterpret_cast<float*>(&s_u);   // [query][145]: rows T * 16 + 4kk + r
  static_assert(sizeof(s_u) >= 16 * 145 * sizeof(float), "merge buffer");
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    if (wave == w) {
#pragma unroll
      for (int T = 0; T < 9; ++T)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float& b = buf[col * 145 + T * 16 + 4 * kk + r];
          b = (w == 0 ? 0.f : b) + alpha * acc[T][r];
        }
    }
    __syncthreads();
  }
  if (wave == 3 && col < a.group) {
    float* pp = a.partials + (((int64_t)head * a.num_splits + split) * a.group + col) * kPartStride;
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
      for (int c = 0; c < 3; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int T = 3 * u + c, dim = 3 * (16 * u + 4 * kk + r) + c;
          if (dim < kD) pp[dim] = buf[col * 145 + T * 16 + 4 * kk + r] + alpha * acc[T][r];
        }
    if (kk == 0) {
      pp[128] = M * (1.f / LOG2E);   // natural-log units for the merge
      pp[129] = L;
    }
  }
}

int launch_octo_attend(const OctoArgs& a, int bits, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.n < 0 || a.heads < 1 || a.heads > 65535 || a.group < 1 || a.group > kOctoMaxGroup || a.num_splits < 1 ||
      a.split_len < kOctoAttChunk || a.split_len % kOctoAttChunk != 0 || (int64_t)a.num_splits * a.split_len < a.n)
    return (int)hipErrorInvalidValue;
  const dim3 grid((unsigned)a.num_splits, (unsigned)a.heads);
  switch (bits) {
    case 2: hipLaunchKernelGGL((octo_attend_kernel<2>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((octo_attend_kernel<3>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((octo_attend_kernel<4>), grid, dim3(256), 0, s, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace tq
