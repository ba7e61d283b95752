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
// the rotated coordinates staged in LDS, then each lane takes triplets
// L, L+16, L+32 of its row; the direction table sits in LDS.
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
// neighbour, a superset of the pair's part on the grid.
__device__ __forceinline__ int octo_block_lo(float v, int nd) {
  const int h = (int)floorf(__builtin_fmaf(v, 0.5f * (float)nd, 0.5f * (float)nd - 0.5f));
  return min(max(h, 0), nd - 2);
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

// atan2(y, x) for y, x >= 0 (0 when both are 0), through atan01 of the
// smaller over the larger (the larger floored at 1e-30, so 0 / 0 gives 0)
__device__ __forceinline__ float atan2_pos(float y, float x) {
  const float mx = fmaxf(x, y), mn = fminf(x, y);
  const float t = atan01(mn * __builtin_amdgcn_rcpf(fmaxf(mx, 1e-30f)));
  return y > x ? 1.57079632679489662f - t : t;
}

// Equal-area octahedral map of the direction of (nx, ny, .) with unit-vector
// z component nz (nx and ny may carry any common positive scale; |nz| may
// exceed 1 by a rounding error): L1 radius sqrt(1 - |nz|), the azimuth
// atan2(|ny|, |nx|) spread linearly along the diamond edge, the lower
// hemisphere reflected across the edge, the signs of nx and ny copied (a
// coordinate of -0 takes the negative side: the map's two sides agree there).
__device__ __forceinline__ void oct_map(float nx, float ny, float nz, float& xi, float& eta) {
  const float r = __builtin_amdgcn_sqrtf(fmaxf(1.f - fabsf(nz), 0.f));
  const float phi = atan2_pos(fabsf(ny), fabsf(nx));
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
  for (int i = tid; i < kNd * kNd; i += 256) s_dir[i] = reinterpret_cast<const float4*>(a.dirs)[i];
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
    for (int i = L; i < kOctoTri; i += 16) {
      const float tx = s_y[row][3 * i], ty = s_y[row][3 * i + 1], tz = s_y[row][3 * i + 2];
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
      const int base = a0 * kNd + c0;
      float best = -INFINITY;
      int bo = 0;
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        const float4 d = s_dir[base + (o >> 1) * kNd + (o & 1)];
        const float p = tx * d.x + ty * d.y + tz * d.z;
        if (p > best) {
          best = p;
          bo = o;
        }
      }
      const int ca = a0 + (bo >> 1), cc = c0 + (bo & 1);
      // norm code: the number of ascending thresholds below p (seven
      // independent compares at b = 4; a binary search's dependent chain of
      // compares and selects measured 10% slower, a bucketed table search 0.5%
      // faster)
      uint32_t k = 0;
#pragma unroll
      for (int j = 0; j + 1 < C::kNr; ++j) k += best > a.trho[j] ? 1u : 0u;
      const uint32_t field = (uint32_t)ca | ((uint32_t)cc << C::kBd) | (k << (2 * C::kBd));
      if constexpr (QJL) {
        // what the codes leave out of the triplet, in place of it (the lane
        // owns these three coordinates)
        const float4 d = s_dir[ca * kNd + cc];
        const float rk = s_crho[k];
        s_y[row][3 * i] = __builtin_fmaf(-rk, d.x, tx);
        s_y[row][3 * i + 1] = __builtin_fmaf(-rk, d.y, ty);
        s_y[row][3 * i + 2] = __builtin_fmaf(-rk, d.z, tz);
      }
      const int bit = i * C::kField, w = bit >> 5, sh = bit & 31;
      atomicOr(&s_rec[row][w], field << sh);
      if (sh + C::kField > 32) atomicOr(&s_rec[row][w + 1], field >> (32 - sh));
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
// gamma * sum_i rho_hat_i (R q)_i . n_hat_i, as a matrix-core product per 16-key tile,
// C[16 keys x 16 queries] += A[16 keys x 4 dims] * B[4 dims x 16 queries]
// over 33 steps of 4 rotated dims (132: 128 plus the zero pad), fp32 in and
// out (v_mfma_f32_16x16x4f32).  Lane l holds A[l%16][l/16], B[l/16][l%16]
// and C[4(l/16)+r][l%16]: the B operands (the rotated, scaled queries) stay
// in 33 registers for the whole kernel; each A element is one decoded
// coordinate rho_hat * n_hat[comp] of key l%16, unpacked from the tile's
// records in LDS.  Each wave takes 16-key tiles in turn.
constexpr int kOctoMfmaTile = 128;   // keys per tile step (2 tiles of 16 per wave)

// 5 waves per SIMD at b = 2, 3 (the kernel held to 96 VGPRs: 248 against
// 263 us on the 4.2M keys of llama70b at b = 3); at b = 4 that limit spills
// and measured slower, so it keeps 4; the QJL variant's 32 more query
// registers leave room for 3
template <int B, bool QJL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(QJL ? 3 : B == 4 ? 4 : 5))) void octo_logits_mfma_kernel(
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
    uint32_t rec[kOctoMfmaTile * kStride];
  } s_u;
  auto& s_q = s_u.qw.q;
  auto& s_w = s_u.qw.w;
  static_assert(sizeof(s_u.qw) == sizeof(float) * (16 * kQd + (QJL ? 16 : 1) * kD), "q and w are contiguous");
  uint32_t* const s_rec = s_u.rec;
  __shared__ float s_rho[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  for (int i = tid; i < C::kNd * C::kNd; i += 256) s_dir[i] = reinterpret_cast<const float4*>(a.dirs)[i];
  if (tid < 8) s_rho[tid] = a.crho[tid];
  // queries past the group (and, with the sketch, their R' R q) stay zero
  float* qf = &s_q[0][0];
  for (int i = tid; i < 16 * kQd + (QJL ? 16 * kD : 0); i += 256) qf[i] = 0.f;
  __syncthreads();
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
  float qb[33];
#pragma unroll
  for (int m = 0; m < 11; ++m)
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const int dim = 3 * (4 * m + kk) + c;
      qb[3 * m + c] = dim < kD ? s_q[col][dim] : 0.f;
    }
  // OCTOPUS-QJL: 32 more steps of 4 sketch coordinates, lane kk taking
  // coordinate 4 s + kk of step s
  float qw[QJL ? 32 : 1];
  if constexpr (QJL) {
#pragma unroll
    for (int st = 0; st < 32; ++st) qw[st] = s_w[col][4 * st + kk];
  }
  // the workgroup walks tiles blockIdx.x, blockIdx.x + gridDim.x, ... of
  // its head, so the table and the queries are set up once per workgroup;
  // the next tile's records are loaded into registers while this one is
  // multiplied (the barrier at the top of the tile loop also orders the
  // reads of s_q above before the first records overwrite it)
  const int64_t ntiles = (a.n + kOctoMfmaTile - 1) / kOctoMfmaTile;
  constexpr int kPre = (kOctoMfmaTile * C::kWords + 255) / 256;
  uint32_t pre[kPre];
  auto fetch = [&](int64_t tl) {
    const int64_t k0 = tl * kOctoMfmaTile;
    const int n_ = (int)(a.n - k0 < kOctoMfmaTile ? a.n - k0 : kOctoMfmaTile);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.codes + ((int64_t)head * a.n + k0) * C::kRec);
#pragma unroll
    for (int r = 0; r < kPre; ++r) {
      const int i = tid + 256 * r;
      pre[r] = i < n_ * C::kWords ? src[i] : 0u;
    }
  };
  if (blockIdx.x < ntiles) fetch(blockIdx.x);
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
  __syncthreads();
  if (tile + gridDim.x < ntiles) fetch(tile + gridDim.x);
  for (int t = wave; t * 16 < nk; t += 4) {
    const uint32_t* rec = s_rec + (t * 16 + col) * kStride;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 11; ++m) {
      const int j = 4 * m + kk;               // triplet 43 reads zero record bits; its q is 0
      const int bit = j * C::kField, wi = bit >> 5, sh = bit & 31;
      const uint32_t f = (uint32_t)((((uint64_t)rec[wi + 1] << 32) | rec[wi]) >> sh) & ((1u << C::kField) - 1u);
      const float4 d = s_dir[(int)(f & (C::kNd - 1)) * C::kNd + (int)((f >> C::kBd) & (C::kNd - 1))];
      const float r = s_rho[f >> (2 * C::kBd)];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r * d.x, qb[3 * m], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r * d.y, qb[3 * m + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r * d.z, qb[3 * m + 2], acc, 0, 0, 0);
    }
    if constexpr (QJL) {
      // A[key][j] = +-sqrt(pi/2)/sqrt(d) rho16 by the key's sign bit j
      // (set: negative), so the products add the residual estimate
      // sqrt(pi/2)/sqrt(d) rho16 sum_j sgn_j (R' R q)_j to the logit
      const int key = t * 16 + col;
      const int64_t kg = (int64_t)head * a.n + key0 + (key < nk ? key : 0);
      const uint4 sg = *reinterpret_cast<const uint4*>(a.qjl_signs + kg * 16);
      const float sk = key < nk ? 0.1107783657f * __half2float(__ushort_as_half(a.qjl_rho[kg])) : 0.f;
      const uint32_t sgs[4] = {sg.x >> kk, sg.y >> kk, sg.z >> kk, sg.w >> kk};
      const uint32_t skb = __float_as_uint(sk);
#pragma unroll
      for (int st = 0; st < 32; ++st) {
        const uint32_t neg = ((sgs[st >> 3] >> (4 * (st & 7))) & 1u) << 31;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(skb ^ neg), qw[st], acc, 0, 0, 0);
      }
    }
    if (col < a.group) {
      float* o = a.out + ((int64_t)head * a.group + col) * a.n + key0 + t * 16 + 4 * kk;
      const uint16_t* gp = a.gamma + (int64_t)head * a.n + key0 + t * 16 + 4 * kk;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (t * 16 + 4 * kk + r < nk) o[r] = acc[r] * __half2float(__ushort_as_half(gp[r]));
    }
  }
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
  // b = 4, 5 at b = 2, 3, one workgroup's wave on each SIMD), spread over
  // the heads, each looping over tiles of its head (the table and the
  // queries are set up once per workgroup)
  const int64_t wgs = 256 * (a.qjl_signs ? 3 : bits == 4 ? 4 : 5);
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

}  // namespace tq
