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
// Work mapping: one vector (d = 128) per 16-lane row, 8 coordinates per lane,
// so a wave64 encodes 4 vectors at once and a 256-thread workgroup 16.  A
// workgroup handles kIters such groups; all their input loads are issued
// before any arithmetic so each lane has kIters 16-byte loads in flight.
// A row's 16 lanes read the vector's 256 contiguous bytes (permuted among
// the lanes, still one coalesced request) and write its code record.

#include "tq_device.h"

namespace tq {

constexpr int kIters = 4;

template <int BITS, int DT, bool QJL>
__global__ __launch_bounds__(256) void encode_kernel(const EncodeArgs a) {
  __shared__ uint2 s_lut[kLutMax];
  __shared__ float s_cent[16];
  const int tid = threadIdx.x;
  if (tid < a.tab.lut_n) s_lut[tid] = make_uint2(__float_as_uint(a.tab.lut_thr[tid]), (uint32_t)a.tab.lut_base[tid]);
  if (tid < 16) s_cent[tid] = a.tab.centroid[tid];

  const EncodeStream st = a.stream[blockIdx.y];
  const int L = tid & 15;
  const int ell = perm16(L);
  const uint32_t sneg = sign_byte(a.rot, ell);       // signs of my inputs 8*ell+e
  const FwhtLane fc = fwht_lane(L);
  const float lut_scale = a.tab.lut_scale, lut_off = a.tab.lut_offset;
  const float lut_top = (float)(a.tab.lut_n - 1);
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
    load8<DT>(st.src, (int64_t)vl * kD + 8 * ell, x[i]);
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
    for (int e = 0; e < 8; ++e) {
      x[i][e] = flip(x[i][e], sneg, e);
      ss = __builtin_fmaf(x[i][e], x[i][e], ss);
    }
    ss = row_sum(ss);
    fwht_row(x[i], fc);                 // lane L now holds coordinates 8L..8L+7
    // 1-ulp hardware sqrt / reciprocal: their error (~1e-7 relative) is far
    // inside the decision band the encoder is held to
    const float gamma = __builtin_amdgcn_sqrtf(ss);
    const float inv = ss > 0.f ? fc.sig * __builtin_amdgcn_rcpf(gamma * 11.313708498984761f) : 0.f;

    uint32_t code[8];
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = x[i][e] * inv;
      const float kf = __builtin_amdgcn_fmed3f(__builtin_fmaf(y[e], lut_scale, lut_off), 0.f, lut_top);
      const uint2 ent = s_lut[(int)kf];
      code[e] = ent.y + (y[e] > __uint_as_float(ent.x) ? 1u : 0u);
    }

    // ---- pack (every lane of the row takes part in the DPP exchanges)
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) word |= code[e] << (BITS * e);
    uint32_t store_word = word;
    bool store_lane = true;
    int store_off = 4 * L;
    if constexpr (BITS == 2) {
      const uint32_t nb = dpp_u<kDppXor1>(word);
      store_word = word | (nb << 16);
      store_lane = (L & 1) == 0;
      store_off = 2 * L;
    } else if constexpr (BITS == 3) {
      const uint32_t nb = dpp_u<kDppQuadNext>(word);
      const int q = L & 3;
      store_word = (word >> (8 * q)) | (q < 3 ? nb << (24 - 8 * q) : 0u);
      store_lane = q < 3;
      store_off = 12 * (L >> 2) + 4 * q;
    }

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
          r[e] = y[e] - s_cent[code[e]];
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

template <int BITS, int DT>
static int launch_bits_dt(const EncodeArgs& a, int streams, bool qjl, hipStream_t s) {
  const int64_t groups = (a.num_vectors + 16 * kIters - 1) / (16 * kIters);
  dim3 grid((unsigned)groups, (unsigned)streams);
  if (qjl) hipLaunchKernelGGL((encode_kernel<BITS, DT, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((encode_kernel<BITS, DT, false>), grid, dim3(256), 0, s, a);
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
