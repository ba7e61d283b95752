// tq_decode_mfma: decode-attend for grouped queries on the gfx950 matrix
// cores.  Same computation as decode_kernel (tq_decode.hip): logits in the
// rotated frame, s_t = scale * gamma_t * <R q, c[codes_t]>, softmax, value
// sum in the rotated frame; the inverse rotation runs in merge_kernel
// (Bit-Axon "TurboQuant: KV Cache Compression", attention under quantisation;
// deep-dive blog Step 1, attention directly on the rotated data).
//
// With 8 query heads per KV head every code is used by 8 dot products, so
// both contractions are dense; they run as matrix-core products and the
// vector units only dequantise codes and run the softmax.
//
//   logits, 4-bit keys: C[16 tokens x 16] = A[16 tokens x 64] * B[64 x 16]
//           in 8-bit integers, 2 steps over the 128 dims for each of the two
//           byte planes of the integer centroids (c ~ (256 hi + lo + 128.5)
//           * 2^-s, |error| <= 2^-(s+1), s = 17 at d = 128); B columns hold
//           the bytes of a 16-bit integer query, Qh (heads 0..7) and Ql.
//           The planes are built from the codes with byte permutes, so the
//           keys need no table lookups.  Exact int32 sums, combined in fp32.
//   logits, 2-/3-bit keys: C[16 x 16] = A[16 x 32] * B[32 x 16] in bf16, 8
//           steps over the 128 dims.  A slots hold (hi, lo) bf16 pairs of
//           centroid values (c = hi + lo to 2^-17); B columns hold q_hi
//           (heads 0..7) and q_lo (residual of q).  Logit = col h + col h+8.
//   values  C[16 dims x 16] += A[16 dims x 32 tokens] * B[32 tokens x 16] in
//           f16, one product per 8-dim tile over a pair of blocks; B columns
//           hold p*gamma_v in f16 (heads 0..7) and its f16 residual.
// Operand layout (checked on the device): for 16x16x32 lane l holds
// A[l%16][8(l/16)+s], B[8(l/16)+s][l%16] and C[4(l/16)+r][l%16]; the
// 16x16x64 integer product pairs byte s of lane l's A operand with byte s of
// lane l's B operand the same way, so only the two must agree on the dims.
//
// Work: grid (split, KV-head slice of <= 8 query heads, sequence); 8 waves
// per workgroup, each takes pairs of 16-token blocks of the split in turn and
// keeps its own running max / sum / accumulator.
//
// Memory: every wave streams its (block, KV head) chunks into a private ring
// of LDS stages with global_load_lds (global memory straight to LDS, no
// registers held while the data is in flight), several block pairs ahead,
// and waits for a stage with an explicit vmcnt.  The loop issues no other
// vector-memory loads, so the count is exact.  The waves are merged in LDS
// and the split's (m, l, o_rot) goes to the workspace for merge_kernel.

#include <hip/hip_bf16.h>

#include <type_traits>

#include "tq_device.h"
#include "tq_encode_row.h"

namespace tq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

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

// Exchanges with the lane 8 columns away inside each 16-lane row
// (row_ror:8), written out so that the compiler cannot fold the DPP move
// into the arithmetic around it (it once fed four such folded adds from the
// first register).  The sources are vector-unit results: the leading s_nop 1
// gives the two wait states a DPP read of such a result needs.
//   r[j] += ror8(x[j]) * w
__device__ __forceinline__ void fmac_ror8_4(float (&r)[4], const float (&x)[4], float w) {
  asm("s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %4, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %5, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %6, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %7, %8 row_ror:8 row_mask:0xf bank_mask:0xf"
      : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3])
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(w));
}
//   o[j] = x[j] of the lane 8 columns away
__device__ __forceinline__ void ror8_2(const uint32_t (&x)[2], uint32_t (&o)[2]) {
  asm("s_nop 1\n\t"
      "v_mov_b32_dpp %0, %2 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32_dpp %1, %3 row_ror:8 row_mask:0xf bank_mask:0xf"
      : "=&v"(o[0]), "=&v"(o[1])
      : "v"(x[0]), "v"(x[1]));
}

// Maxima written out: the compiler's fmaxf first canonicalises operands it
// cannot prove canonical (an extra v_max per operand); the softmax values here
// are products, exponentials or -inf, never signalling NaNs.
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max of v and v of the lane 8 columns away (the source is a vector-unit
// result: s_nop 1 gives the DPP read its two wait states)
__device__ __forceinline__ float vmax_ror8(float v) {
  float r;
  asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(v));
  return r;
}
// max over the four 16-lane rows (every lane receives it), with m folded in
__device__ __forceinline__ float vmax_rows(float v, float m) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float w = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t uw = __float_as_uint(w);
  const auto b = __builtin_amdgcn_permlane32_swap(uw, uw, false, false);
  return vmax3(__uint_as_float(b[0]), __uint_as_float(b[1]), m);
}

// 4-bit key codes -> the two signed-byte planes of their integer centroids,
// on the vector unit (no table in LDS).  A word holds 8 codes, one nibble
// each; byte k of the "even" results belongs to the low nibble of byte k of
// the word, byte k of the "odd" results to its high nibble.
//  - m: 0xFF in the bytes whose code has bit 3 set (positive half).  v_perm
//    selectors 8..11 replicate bit 7 of bytes 1, 3 of either source, so the
//    words are shifted until each code's bit 3 sits in such a bit 7.
//  - sel = (code ^ m) & 7: the code itself in the negative half, 15 - code
//    (its mirror) in the positive half.
//  - plane byte = table[sel] ^ m: the mirror's bytes, NOT-ed for positives.
// The tables hold the eight negative-half bytes: t0 = entries 0..3, t1 = 4..7.
struct KeyI8Tab {
  uint32_t h0, h1, l0, l1;
};
__device__ __forceinline__ void key_planes_b4(uint32_t w, const KeyI8Tab& t, uint32_t& he, uint32_t& ho,
                                              uint32_t& le, uint32_t& lo) {
  constexpr uint32_t kSignSel = 0x090B080Au;   // bytes 0..3 <- bit 7 of src0 b1, src1 b1, src0 b3, src1 b3
  const uint32_t me = __builtin_amdgcn_perm(w << 12, w << 4, kSignSel);
  const uint32_t mo = __builtin_amdgcn_perm(w << 8, w, kSignSel);
  const uint32_t se = __builtin_amdgcn_bitop3_b32(w, me, 0x07070707u, 0x28);        // (a ^ b) & c
  const uint32_t so = __builtin_amdgcn_bitop3_b32(w >> 4, mo, 0x07070707u, 0x28);
  he = __builtin_amdgcn_perm(t.h1, t.h0, se) ^ me;
  le = __builtin_amdgcn_perm(t.l1, t.l0, se) ^ me;
  ho = __builtin_amdgcn_perm(t.h1, t.h0, so) ^ mo;
  lo = __builtin_amdgcn_perm(t.l1, t.l0, so) ^ mo;
}

// Geometry of one (block, KV head) chunk of a cache with values (K codes
// [16][16b] | V codes [16][16b] | gamma_k [16] | gamma_v [16], fp16 norms;
// with the QJL sidecar also rho [16], fp16 residual norms, and signs
// [16][16 B]), and of its LDS stage slot.  The chunk is copied by kFull 1 KiB
// pieces (64 lanes x 16 B) and one tail piece of kRem bytes by the first
// kRem / 16 lanes, so a slot holds exactly one chunk.  kStages block pairs
// per wave.
template <int BITS, bool QJL = false>
struct Chunk {
  static constexpr int kBytes = 512 * BITS + 64 + (QJL ? 32 + 256 : 0);
  static constexpr int kOffV = 256 * BITS, kOffGK = 512 * BITS, kOffGV = 512 * BITS + 32;
  static constexpr int kOffRho = 512 * BITS + 64, kOffSign = kOffRho + 32;
  static constexpr int kFull = kBytes / 1024;
  static constexpr int kRem = kBytes - 1024 * kFull;
  static constexpr int kTailLanes = kRem / 16;
  static constexpr int kSlot = kBytes;
  static constexpr int kDma = kFull + 1;     // copy instructions per chunk
  static constexpr int kStages = BITS == 2 && !QJL ? 4 : 2;
  static constexpr int kWaveRing = kStages * 2 * kSlot;
  static_assert(kRem > 0 && kRem % 16 == 0 && kTailLanes <= 64, "tail piece");
  // exec mask of the tail copy
  static constexpr uint32_t kTailLo = kTailLanes >= 32 ? 0xFFFFFFFFu : (1u << kTailLanes) - 1u;
  static constexpr uint32_t kTailHi = kTailLanes > 32 ? (kTailLanes == 64 ? 0xFFFFFFFFu : (1u << (kTailLanes - 32)) - 1u) : 0u;
};

// Copy one chunk from global memory (wave-uniform src) to LDS byte address
// lds, with non-temporal loads (the cache is streamed once per call: random
// 1.6-2.1 KB chunks read 5.6 TB/s plain and 6.2-6.3 TB/s non-temporal in a
// streaming probe on this chip).  v16 = 16 * lane.  The LDS address of a piece is m0 + instruction
// offset + lane * 16 (the offset applies to both sides), so every piece
// lands at its offset inside the slot.  The tail piece runs with the exec
// mask narrowed to its lanes (inactive lanes neither read nor write); m0 and
// exec are saved and restored inside the asm.
template <int BITS, bool QJL>
__device__ __forceinline__ void dma_chunk(uint32_t lds, const uint8_t* src, uint32_t v16, uint32_t vv) {
  using C = Chunk<BITS, QJL>;
  uint32_t save;
  uint64_t esave;
  if constexpr (BITS == 4) {
    // the V piece (codes of the 16 values) goes through the swizzled lane
    // offsets vv (see v_slot_src)
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %4 nt\n\t"
        "global_load_lds_dwordx4 %5, %4 offset:1024 nt\n\t"
        "s_mov_b64 %1, exec\n\ts_mov_b32 exec_lo, %6\n\ts_mov_b32 exec_hi, %7\n\ts_nop 1\n\t"
        "global_load_lds_dwordx4 %3, %4 offset:2048 nt\n\t"
        "s_mov_b64 exec, %1\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save), "=&s"(esave)
        : "s"(lds), "v"(v16), "s"(src), "v"(vv), "i"(C::kTailLo), "i"(C::kTailHi)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %4 nt\n\t"
        "s_mov_b64 %1, exec\n\ts_mov_b32 exec_lo, %5\n\ts_mov_b32 exec_hi, %6\n\ts_nop 1\n\t"
        "global_load_lds_dwordx4 %3, %4 offset:1024 nt\n\t"
        "s_mov_b64 exec, %1\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save), "=&s"(esave)
        : "s"(lds), "v"(v16), "s"(src), "i"(C::kTailLo), "i"(C::kTailHi)
        : "memory");
    (void)vv;
  }
}

// One 16 B-per-lane copy: LDS lds + 16 lane <- global src + voff.
__device__ __forceinline__ void dma_x4(uint32_t lds, const void* src, uint32_t voff) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save) : "s"(lds), "v"(voff), "s"(src) : "memory");
}

// One dword per lane from global memory (wave-uniform base + lane offset),
// written as asm so that the compiler neither tracks nor waits for it: the
// caller orders it before the copies it waits for.
__device__ __forceinline__ uint32_t load_dword_untracked(const void* base, uint32_t voff) {
  uint32_t v;
  asm volatile("global_load_dword %0, %1, %2" : "=v"(v) : "v"(voff), "s"(base) : "memory");
  return v;
}

// Wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait for the oldest staged pair while `behind` younger pairs stay in flight
template <int BITS, bool QJL>
__device__ __forceinline__ void wait_pairs_behind(int behind) {
  constexpr int P = 2 * Chunk<BITS, QJL>::kDma;
  if (behind <= 0) wait_vm<0>();
  else if (behind == 1) wait_vm<P>();
  else if (behind == 2) wait_vm<2 * P>();
  else if (behind == 3) wait_vm<3 * P>();
  else wait_vm<4 * P>();
}

// With 4-bit codes the V region (16 records of 64 B, 64 pieces of 16 B) is
// staged transposed by token: piece (token T, quarter d) of the record goes
// to slot 16 (T % 4) + 4 (T / 4) + d, so the reads below (lane (m, g) takes
// 4 B of token 4g + i at a time) hit 64 different banks.  Lane L of the copy
// fetches the piece that belongs in slot L.
__device__ __forceinline__ uint32_t v_slot_src(int L) {
  const int T = 4 * ((L >> 2) & 3) + (L >> 4), d = L & 3;
  return (uint32_t)(16 * (4 * T + d));
}

template <int BITS>
struct BlockRegs {
  uint32_t k[BITS];     // 32 codes: dims 32g .. 32g+31 of token row m
  uint32_t v[4];        // 8 codes each: dims 8m .. 8m+7 of tokens 4g .. 4g+3
};
// fp16 norms of tokens 4g .. 4g+3 of the lane's own block of the pair
struct PairNorms {
  uint32_t gk[2];
  uint32_t gv[2];
};
// QJL sidecar of both blocks of a pair: word g of token m's sign record, and
// the fp16 residual norms of tokens 4g .. 4g+3
struct PairQjl {
  uint32_t sw[2];
  uint32_t rh[2][2];
};

// this lane's codes and norms of one chunk staged in LDS at st
template <int BITS>
__device__ __forceinline__ void read_chunk(BlockRegs<BITS>& r, const uint8_t* st, int m, int g) {
  using C = Chunk<BITS>;
  if constexpr (BITS == 4) {
    const uint4 t = *reinterpret_cast<const uint4*>(st + m * 64 + g * 16);
    r.k[0] = t.x; r.k[1] = t.y; r.k[2] = t.z; r.k[3] = t.w;
  } else if constexpr (BITS == 3) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(st + m * 48 + g * 12);
    r.k[0] = p[0]; r.k[1] = p[1]; r.k[2] = p[2];
  } else {
    const uint2 t = *reinterpret_cast<const uint2*>(st + m * 32 + g * 8);
    r.k[0] = t.x; r.k[1] = t.y;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int off = C::kOffV + (4 * g + i) * 16 * BITS + BITS * m;
    if constexpr (BITS == 4) {
      // transposed staging: token 4g + i, dims 8m.. at 256 i + 64 g + 4 m
      r.v[i] = *reinterpret_cast<const uint32_t*>(st + C::kOffV + 256 * i + 64 * g + 4 * m);
    } else if constexpr (BITS == 2) {
      r.v[i] = *reinterpret_cast<const uint16_t*>(st + off);
    } else {
      // 24 bits at byte off (4 pair fields), funnel-shifted so that pair
      // field T lands at bit 7 + 6T: field 0 is then already where the table
      // address wants it (v_field_addr).  The two aligned dwords start 1-4
      // bytes below off, so the shift 8 (off - base) - 7 is never negative;
      // the lower one may hold K codes, the upper one may reach into the
      // gamma_k region of the slot (bits outside the fields are masked off).
      const int dm = off & 3;
      const int base = off - (dm ? dm : 4);
      const uint32_t lo = *reinterpret_cast<const uint32_t*>(st + base);
      const uint32_t hi = *reinterpret_cast<const uint32_t*>(st + base + 4);
      r.v[i] = __builtin_amdgcn_alignbit(hi, lo, (uint32_t)(8 * (off - base) - 7));
    }
  }
}

// the norms of the lane's own block: own = st + (lane's block of the pair) * slot
template <int BITS>
__device__ __forceinline__ void read_norms(PairNorms& r, const uint8_t* own, int g) {
  using C = Chunk<BITS>;
  const uint2 a = *reinterpret_cast<const uint2*>(own + C::kOffGK + 8 * g);
  const uint2 b = *reinterpret_cast<const uint2*>(own + C::kOffGV + 8 * g);
  r.gk[0] = a.x; r.gk[1] = a.y;
  r.gv[0] = b.x; r.gv[1] = b.y;
}

// a * (the fp16 value in the low / high half of h), left to the compiler so
// that it forms a mixed-precision product (v_fma_mix) and pads its hazards
// (a product right after a transcendental needs a wait state)
__device__ __forceinline__ float mul_h_lo(float a, uint32_t h) {
  return a * (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}
__device__ __forceinline__ float mul_h_hi(float a, uint32_t h) {
  return a * (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> 16));
}

// LDS of one workgroup, in one object so the tables sit at address 0 (a
// lookup address then fits the instruction's offset field).
template <int BITS, bool QJL = false>
struct DecodeSmem {
  // 4-bit codes: the logits take 8-bit integer operands built on the vector
  // unit (key_planes_b4), no key table; values read a table of code pairs,
  // f16(c[first]) | f16(c[second]) << 16.
  // 2- and 3-bit codes: keys and values both read tables of code pairs
  // (index = the pair's 2b-bit field), entry = the two scaled halves, kept in
  // 32 copies laid out so that lane L reads copy L % 32 from bank L % 32:
  // entry e of copy r is word 32 e + r, so any 32 lanes of a read hit 32
  // different banks whatever codes they look up.
  static constexpr bool kI8 = BITS == 4;
  static constexpr bool kTab = BITS <= 3;
  static constexpr int kRep = 32;
  static constexpr int kPairs = 1 << (2 * BITS);
  static constexpr int kTk = kI8 ? 4 : kPairs * kRep;
  static constexpr int kTv = kI8 ? kPairs : kPairs * kRep;
  static constexpr int kQSteps = kI8 ? 2 : 4;
  // waves per workgroup: 8, so the per-workgroup set-up (tables, query
  // rotation) and the split partials are shared by 8 waves; two workgroups
  // (16 waves) fit on a CU
  static constexpr int kWaves = 8;
  uint32_t tk[kTk];
  uint32_t tv[kTv];
  float qcorr[8], qmult[8];            // 8-bit logits: per-head offset and scale
  // the slice's queries as loaded, then (after a barrier) the logit B
  // operands [step][lane] built from them
  union {
    alignas(16) uint8_t qs[8 * kD * 4];
    u32x4 qb[kQSteps][64];
  };
  float cent[2][16];                   // key / value centroids (4-bit)
  uint32_t half[2][16];                // key / value scaled halves (2-, 3-bit)
  float wm[kWaves][8], wl[kWaves][8], ml[2][8];
  alignas(16) uint8_t ring[kWaves * Chunk<BITS, QJL>::kWaveRing];
};

// Byte address of the table entry for the W-bit field i of a packed
// little-endian bit string w[] (lane copy r4 = 4 (lane % 32)): the field is
// moved to bit 7 (entry stride 128 bytes) with one shift or funnel shift and
// merged with r4 by one and-or.
template <int W, int N>
__device__ __forceinline__ uint32_t pair_addr(const uint32_t (&w)[N], int i, uint32_t r4) {
  const int bit = W * i, wi = bit >> 5, sh = bit & 31;
  constexpr uint32_t mask = ((1u << W) - 1u) << 7;
  uint32_t x;
  if (sh + W <= 32) x = sh >= 7 ? (w[wi] >> (sh - 7)) : (w[wi] << (7 - sh));
  else x = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], (uint32_t)(sh - 7));
  return (x & mask) | r4;
}
// The same for the value codes of 2- and 3-bit caches as read_chunk leaves
// them: 2-bit, field T at bit 4T (pair_addr); 3-bit, at bit 7 + 6T, so field
// 0 needs no shift.
template <int BITS>
__device__ __forceinline__ uint32_t v_field_addr(uint32_t w, int T, uint32_t r4) {
  if constexpr (BITS == 3) {
    constexpr uint32_t mask = 0x3Fu << 7;
    return ((T ? w >> (6 * T) : w) & mask) | r4;
  } else {
    const uint32_t w1[1] = {w};
    return pair_addr<2 * BITS>(w1, T, r4);
  }
}
__device__ __forceinline__ uint32_t lds_word(const uint32_t* table, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(table) + byte_addr);
}

// s[j] = gamma_k * logit of token 4g + j, from the two blocks' logit
// products f0 / f1 of the table path (column m of a block holds the q_hi
// part of head m % 8 for m < 8, the q_lo part for m >= 8).  Lanes m < 8 take
// block 0, lanes m >= 8 block 1: each adds its own column and the one 8
// columns away, as two adds that write one lane half each (banks 0, 1 /
// banks 2, 3 of every row); then the product with the fp16 norm (low / high
// half of gk[j / 2]) as one mixed-precision multiply-add.  f0 and f1 are
// matrix-core results read here by DPP: the leading s_nops give that read
// more wait states than the 16x16x32 products need.
__device__ __forceinline__ void logits_tab(const f32x4& f0, const f32x4& f1, const uint32_t (&gk)[2], float (&s)[4]) {
  float c0, c1, c2, c3;
  asm volatile("s_nop 7\n\ts_nop 4\n\t"
      "v_add_f32_dpp %4, %8, %8 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %4, %12, %12 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %5, %9, %9 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %5, %13, %13 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %6, %10, %10 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %6, %14, %14 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %7, %11, %11 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %7, %15, %15 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_fma_mix_f32 %0, %4, %16, 0 op_sel_hi:[0,1,0]\n\t"
      "v_fma_mix_f32 %1, %5, %16, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]\n\t"
      "v_fma_mix_f32 %2, %6, %17, 0 op_sel_hi:[0,1,0]\n\t"
      "v_fma_mix_f32 %3, %7, %17, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
      : "=&v"(s[0]), "=&v"(s[1]), "=&v"(s[2]), "=&v"(s[3]), "=&v"(c0), "=&v"(c1), "=&v"(c2), "=&v"(c3)
      : "v"(f0[0]), "v"(f0[1]), "v"(f0[2]), "v"(f0[3]), "v"(f1[0]), "v"(f1[1]), "v"(f1[2]), "v"(f1[3]),
        "v"(gk[0]), "v"(gk[1]));
}

// s[j] = c[j] * the fp16 norm in the low / high half of gk[j / 2], as
// mixed-precision multiply-adds (c are ordinary vector results, not
// transcendental ones, so no extra wait state is needed)
__device__ __forceinline__ void scale_by_norms(const float (&c)[4], const uint32_t (&gk)[2], float (&s)[4]) {
  asm("v_fma_mix_f32 %0, %4, %8, 0 op_sel_hi:[0,1,0]\n\t"
      "v_fma_mix_f32 %1, %5, %8, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]\n\t"
      "v_fma_mix_f32 %2, %6, %9, 0 op_sel_hi:[0,1,0]\n\t"
      "v_fma_mix_f32 %3, %7, %9, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
      : "=&v"(s[0]), "=&v"(s[1]), "=&v"(s[2]), "=&v"(s[3])
      : "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]), "v"(gk[0]), "v"(gk[1]));
}

// B operands of the table path's two value products, built from hv[j] (f16
// bits of p gamma_v of token 4g + j in the low half, high half zero) and
// hi[j] = hv[j] << 16:
//   block 0 (becomes hv): lanes c < 8 keep their own hv; lanes c >= 8 take
//     the hv of lane c - 8 times 65536 (its high half);
//   block 1 (becomes hi): lanes c >= 8 keep their own hv << 16; lanes c < 8
//     take the hv of lane c + 8.
// The block-1 copies run first, while every lane's hv is still its own.
// m holds 65536 in the lanes c >= 8.  The leading s_nop gives the DPP reads
// of hv their two wait states; the closing one separates the last DPP write
// from the matrix-core reads of the operands.
__device__ __forceinline__ void value_b_tab(uint32_t (&hv)[4], uint32_t (&hi)[4], uint32_t m) {
  asm("s_nop 1\n\t"
      "v_mov_b32_dpp %4, %0 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_mov_b32_dpp %5, %1 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_mov_b32_dpp %6, %2 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_mov_b32_dpp %7, %3 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_mul_u32_u24_dpp %0, %0, %8 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_mul_u32_u24_dpp %1, %1, %8 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_mul_u32_u24_dpp %2, %2, %8 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_mul_u32_u24_dpp %3, %3, %8 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "s_nop 1"
      : "+v"(hv[0]), "+v"(hv[1]), "+v"(hv[2]), "+v"(hv[3]), "+v"(hi[0]), "+v"(hi[1]), "+v"(hi[2]), "+v"(hi[3])
      : "v"(m));
}

// Decode step: encode the sequence's new token (keys and values of KV head
// h) into row `row` of block `blk`, with the vector encoder's row algorithm
// (FWHT in one 16-lane row, bucketed threshold search, packing, fp16 norm):
// lanes 0..15 of wave 0 take the key, lanes 16..31 the value.  `lut` is 2 KB
// of LDS not otherwise in use; every thread of the workgroup calls this.
// The stores are performed (vmcnt 0) before the closing barrier, so the
// workgroup's copies of the block that follow read the new rows.
template <int BITS>
__device__ __forceinline__ void append_token(const DecodeArgs& a, const AppendArgs& ap, int n, int h, int blk, int row,
                                             uint2* lut, int tid) {
  const float lut_scale = ap.tab.lut_scale, lut_off = ap.tab.lut_offset - 0.5f;
  fill_lut(lut, ap.tab, lut_scale, lut_off, tid);
  __syncthreads();
  if (tid < 32) {
    const int r = tid >> 4, L = tid & 15, ell = perm16(L);
    // sign byte ell of the rotation, picked among wave-uniform words
    const uint32_t n0 = __builtin_amdgcn_readfirstlane(a.rot.neg[0]), n1 = __builtin_amdgcn_readfirstlane(a.rot.neg[1]);
    const uint32_t n2 = __builtin_amdgcn_readfirstlane(a.rot.neg[2]), n3 = __builtin_amdgcn_readfirstlane(a.rot.neg[3]);
    const int wsel = ell >> 2;
    const uint32_t wd = wsel == 0 ? n0 : wsel == 1 ? n1 : wsel == 2 ? n2 : n3;
    const uint32_t sneg = (wd >> (8 * (ell & 3))) & 0xFFu;
    uint32_t smask[8];
    float x[8];
    const int64_t elem = ((int64_t)n * a.num_kv_heads + h) * kD + 8 * ell;
    const void* src = r ? ap.v_new : ap.k_new;
    if (ap.dtype == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) smask[i] = ((sneg >> i) & 1u) << 31;
      load8_signed<0>(src, elem, smask, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        smask[i] = i < 4 ? (((sneg >> (2 * i)) & 1u) << 15) | (((sneg >> (2 * i + 1)) & 1u) << 31) : 0u;
      if (ap.dtype == 1) load8_signed<1>(src, elem, smask, x);
      else load8_signed<2>(src, elem, smask, x);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
    ss = row_sum(ss);
    const FwhtLane fc = fwht_lane(L);
    fwht_row(x, fc);   // lane L now holds coordinates 8L..8L+7
    const float gamma = __builtin_amdgcn_sqrtf(ss);
    const float inv = ss > 0.f ? fc.sig * __builtin_amdgcn_rcpf(gamma * 11.313708498984761f) : 0.f;
    uint32_t code[8];
    row_codes<BITS>(x, inv * lut_scale, lut_off, lut, code);
    bool store_lane;
    int store_off;
    const uint32_t word = row_pack<BITS>(code, L, store_lane, store_off);
    uint8_t* base = const_cast<uint8_t*>(a.pool) + ((int64_t)blk * a.num_kv_heads + h) * a.lay.block_bytes;
    uint8_t* rec = base + (r ? a.lay.off_v + (int64_t)row * a.lay.v_rec : a.lay.off_k + (int64_t)row * a.lay.k_rec);
    if (store_lane) *reinterpret_cast<uint32_t*>(rec + store_off) = word;
    if (L == 0)
      *reinterpret_cast<__half*>(base + (r ? a.lay.off_gv : a.lay.off_gk) + 2 * row) =
          __float2half_rn(fminf(gamma, 65504.f));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// 4 waves per SIMD (two 8-wave workgroups per CU); a 4-bit QJL chunk ring
// leaves room for one workgroup per CU, so that variant may take the
// registers of 2
template <int BITS, bool LOGITS, bool APPEND, bool QJL = false>
__global__ __launch_bounds__(64 * DecodeSmem<BITS>::kWaves) __attribute__((amdgpu_waves_per_eu(QJL && BITS == 4 ? 2 : 4))) void decode_mfma_kernel(
    const DecodeArgs a, int ns, int gs, const typename std::conditional<APPEND, AppendArgs, NoAppend>::type ap) {
  static_assert(!QJL || !APPEND, "the decode step takes caches without the QJL sidecar");
  using C = Chunk<BITS, QJL>;
  constexpr int NS = C::kStages;
  __shared__ DecodeSmem<BITS, QJL> sm;
  const uint32_t* const s_tv2 = sm.tv;
  auto& s_qb = sm.qb;
  auto& s_wm = sm.wm;
  auto& s_wl = sm.wl;
  auto& s_ml = sm.ml;
  uint8_t* const s_ring = sm.ring;
  // per-wave [column][dim] accumulator rows, padded where the ring has room
  // (16 columns; 8 on the table path, whose columns of one head are merged
  // by dim parity)
  constexpr int kAccRows = DecodeSmem<BITS>::kTab ? 8 : 16;
  constexpr int kAccRow = kAccRows * (kD + 4) * 4 <= C::kWaveRing ? kD + 4 : kD;
  static_assert(kAccRows * kAccRow * 4 <= C::kWaveRing, "wave accumulator must fit in the wave's ring");

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
  const int tok_end = min(seq_len, sb1 * kBlock);
  const int64_t Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const float LOG2E = 1.4426950408889634f;

  // ---- this wave's block pairs: wave, wave + NW, ... of the split
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int npairs = max(0, (sb1 - sb0 + 1) / 2);
  constexpr int NW = DecodeSmem<BITS>::kWaves;
  constexpr int NT = 64 * NW;
  const int my_n = npairs > wv ? (npairs - wv + NW - 1) / NW : 0;
  // the block table is read through the constant address space: it does not
  // change during the launch, so its wave-uniform reads stay scalar loads
  // (the asm around them would otherwise force vector loads and full waits)
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const const_i32_ptr btab = (const_i32_ptr)(a.block_tables + (int64_t)n * a.max_blocks);
  const uint32_t nblocks = (uint32_t)min(a.num_blocks, (int64_t)INT32_MAX);
  const uint8_t* const pool_h = a.pool + (int64_t)h * C::kBytes;
  const int64_t blk_stride = Hkv * C::kBytes;
  // block-table entries of this wave's k-th pair (the second block of a
  // split's odd tail re-reads the first; its data is never used)
  auto fetch_pair = [&](int k, int& b0, int& b1) {
    const int lb = sb0 + 2 * (wv + NW * k);
    b0 = btab[lb];
    b1 = btab[lb + 1 < sb1 ? lb + 1 : lb];
  };
  auto chunk_src = [&](int blk) -> const uint8_t* {
    return pool_h + (int64_t)((uint32_t)blk < nblocks ? blk : 0) * blk_stride;   // out-of-range ids read block 0
  };
  const uint32_t ring_lds = (uint32_t)reinterpret_cast<uintptr_t>(s_ring) + (uint32_t)(wv * C::kWaveRing);
  const uint32_t v16 = 16u * lane;
  const uint32_t vv = v_slot_src(lane);
  auto dma_pair = [&](int k, int b0, int b1) {   // k-th pair of this wave into stage k % NS
    const uint32_t st = ring_lds + (uint32_t)((k % NS) * 2 * C::kSlot);
    dma_chunk<BITS, QJL>(st, chunk_src(b0), v16, vv);
    dma_chunk<BITS, QJL>(st + C::kSlot, chunk_src(b1), v16, vv);
  };
  // Block-table entries of this wave's pairs for the loop: lane j holds
  // those of pair j (at most 64 pairs per wave, by the split size), read
  // here with per-lane loads issued before every copy, so each wait for a
  // copy below also covers them.  (Scalar loads in the loop would share the
  // LDS wait counter and, completing out of order, force a full wait on
  // every table read.)  Lanes past the wave's pairs re-read its first entry.
  uint32_t ids0 = 0, ids1 = 0;
  if (my_n > 0) {
    const int j = min(lane, my_n - 1);
    const int lb = sb0 + 2 * (wv + NW * j);
    const void* row = a.block_tables + (int64_t)n * a.max_blocks;
    ids0 = load_dword_untracked(row, 4u * (uint32_t)lb);
    ids1 = load_dword_untracked(row, 4u * (uint32_t)(lb + 1 < sb1 ? lb + 1 : lb));
  }
  // The kernel issues no other vector-memory loads of its own: the slice's
  // queries and the first stages are copied to LDS here, before the set-up
  // below, whose latency they hide; centroids and signs come through scalar
  // loads.  Wave 0 copies the queries (gcount heads of 128 elements,
  // contiguous) first, so it can wait for them alone.
  const int qsize = a.q_dtype == 0 ? 4 : 2;
  if (wv == 0) {
    const int qbytes = gcount * kD * qsize;   // a multiple of 256
    const uint8_t* qsrc = static_cast<const uint8_t*>(a.q) + ((int64_t)n * Hq + (int64_t)h * a.group + g0) * kD * qsize;
    const uint32_t qs_lds = (uint32_t)reinterpret_cast<uintptr_t>(sm.qs);
    for (int j = 0; 1024 * j < qbytes; ++j)
      dma_x4(qs_lds + 1024u * j, qsrc, (uint32_t)min(16 * lane + 1024 * j, qbytes - 16));
  }
  // decode step: the split holding the new token's block encodes it first,
  // and copies nothing before that
  bool owner = false;
  int new_blk = 0, new_row = 0;
  if constexpr (APPEND) {
    const int t_new = seq_len - 1;
    if (t_new >= 0 && t_new / kBlock >= sb0 && t_new / kBlock < sb1) {
      new_blk = btab[t_new / kBlock];
      new_row = t_new & (kBlock - 1);
      owner = (uint32_t)new_blk < nblocks;
    }
  }
  const int k_pro = min(NS, my_n);
  auto prologue_copies = [&]() {
    for (int k = 0; k < k_pro; ++k) {
      int b0, b1;
      fetch_pair(k, b0, b1);
      dma_pair(k, b0, b1);
    }
  };
  if (!owner) prologue_copies();

  constexpr bool kI8 = DecodeSmem<BITS>::kI8;
  constexpr bool kTab = DecodeSmem<BITS>::kTab;
  constexpr int kLevels = 1 << BITS;
  // codebooks through LDS: one lane writes them from wave-uniform (scalar)
  // loads of the arguments, so no per-lane argument load is needed
  if (tid == 0) {
#pragma unroll
    for (int i = 0; i < kLevels; ++i) {
      if constexpr (kTab) {
        sm.half[0][i] = a.f16_k.h[i];
        sm.half[1][i] = a.f16_v.h[i];
      } else {
        sm.cent[0][i] = a.cent_k[i];
        sm.cent[1][i] = a.cent_v[i];
      }
    }
  }
  __syncthreads();
  if constexpr (kTab) {
    // pair tables, 32 copies each (entry e of copy r at word 32 e + r)
    constexpr int mask = kLevels - 1;
    for (int i = tid; i < DecodeSmem<BITS>::kPairs * DecodeSmem<BITS>::kRep; i += NT) {
      const int e = i >> 5;
      sm.tk[i] = sm.half[0][e & mask] | (sm.half[0][e >> BITS] << 16);
      sm.tv[i] = sm.half[1][e & mask] | (sm.half[1][e >> BITS] << 16);
    }
  } else {
    for (int i = tid; i < (1 << (2 * BITS)); i += NT) {
      constexpr int mask = kLevels - 1;
      sm.tv[i] = f16_bits(sm.cent[1][i & mask]) | (f16_bits(sm.cent[1][i >> BITS]) << 16);
    }
  }
  if (wv == 0) wait_pairs_behind<BITS, QJL>(owner ? 0 : k_pro);   // the query copy has landed
  __syncthreads();

  // ---- rotate this slice's queries (rows of 16 lanes, one head each; the
  // logit scale and log2(e) are folded in, so logits come out in log2 units)
  // and scatter them into the B operands of the logit product.  Columns of
  // heads past the slice are zero.
  // QJL: w = R' (R q) of the rotation rows' heads, lane p holding
  // coordinates 8 perm16(p) + e (zero for heads past the slice)
  [[maybe_unused]] float wq[QJL ? 8 : 1];
  if constexpr (QJL) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wq[e] = 0.f;
  }
  {
    const int r = tid >> 4, p = tid & 15;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (r < 8 && r < gcount) {
      const FwhtLane fc = fwht_lane(p);
      const int ell = perm16(p);
      const int elem = r * kD + 8 * ell;
      if (a.q_dtype == 0) load8<0>(sm.qs, elem, x);
      else if (a.q_dtype == 1) load8<1>(sm.qs, elem, x);
      else load8<2>(sm.qs, elem, x);
      // sign byte ell of the rotation: word picked among uniform loads
      const int wsel = ell >> 2;
      const uint32_t wd = wsel == 0 ? a.rot.neg[0] : wsel == 1 ? a.rot.neg[1] : wsel == 2 ? a.rot.neg[2] : a.rot.neg[3];
      const uint32_t sb = (wd >> (8 * (ell & 3))) & 0xFFu;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = flip(x[e], sb, e);
      fwht_row(x, fc);   // lane p now holds dims 8p .. 8p+7
      const float sc = fc.sig * kInvSqrtD * a.scale * LOG2E;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= sc;
      if constexpr (QJL) {
        // the residual sketch is read against R' applied to the scaled
        // R q: flip dims 8p..8p+7 by byte p of R' and run the row FWHT again
        const int ws = p >> 2;
        const uint32_t wd2 = ws == 0 ? a.rot_qjl.neg[0] : ws == 1 ? a.rot_qjl.neg[1] : ws == 2 ? a.rot_qjl.neg[2] : a.rot_qjl.neg[3];
        const uint32_t sq = (wd2 >> (8 * (p & 3))) & 0xFFu;
#pragma unroll
        for (int e = 0; e < 8; ++e) wq[e] = flip(x[e], sq, e);
        fwht_row(wq, fc);
#pragma unroll
        for (int e = 0; e < 8; ++e) wq[e] *= fc.sig * kInvSqrtD;
      }
    }
    // every read of the staged queries is done before the B operands,
    // which share their storage, are written
    __syncthreads();
    if (r < 8) {
      if constexpr (kI8) {
        // 16-bit integer query Q = rint(x S), S = 32512 / max|x| over the
        // head, split as Q = 256 Qh + Ql into signed bytes: column r takes
        // Qh, column r + 8 takes Ql.  In the operand of lane (c, g) at step
        // st, byte s carries dim 32g + 16st + 8(s>>3) + 2(s&3) + ((s>>2)&1),
        // the order key_planes_b4 leaves the key codes in.  The sum of Q
        // restores the 128.5-unit offset of the key values.
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[e]));
        mx = row_max(mx);
        const float S = mx > 0.f ? 32512.f / mx : 1.f;
        uint8_t* qb = reinterpret_cast<uint8_t*>(s_qb);
        int qsum = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int Q = (int)rintf(x[e] * S);
          const int qh = (Q + 128) >> 8, ql = Q - 256 * qh;
          qsum += Q;
          const int d = 8 * p + e, gq = d >> 5, st = (d >> 4) & 1;
          const int sl = 8 * ((d >> 3) & 1) + 4 * (d & 1) + ((d >> 1) & 3);
          qb[(st * 64 + r + 16 * gq) * 16 + sl] = (uint8_t)qh;
          qb[(st * 64 + r + 8 + 16 * gq) * 16 + sl] = (uint8_t)ql;
        }
        const float qsf = row_sum((float)qsum);
        if (p == 0) {
          sm.qcorr[r] = 128.5f * qsf;
          sm.qmult[r] = a.ki8_unit / S;
        }
      } else {
        // column c -> head c%8, part c/8 (f16 q_hi, f16 residual); in the
        // operand of lane (c, g) at step st, slot s carries dim
        // 32g + 8st + s, the order of the lane's key codes.  The key table
        // holds S c, so 1/S is folded in here.
        uint16_t* qb = reinterpret_cast<uint16_t*>(s_qb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * p + e, gq = d >> 5, st = (d >> 3) & 3, sl = d & 7;
          const float xv = x[e] * a.f16_k.unscale;
          const _Float16 hh = (_Float16)xv;
          const _Float16 hl = (_Float16)(xv - (float)hh);
          qb[(st * 64 + r + 16 * gq) * 8 + sl] = __builtin_bit_cast(uint16_t, hh);
          qb[(st * 64 + r + 8 + 16 * gq) * 8 + sl] = __builtin_bit_cast(uint16_t, hl);
        }
      }
    }
  }
  __syncthreads();
  if constexpr (APPEND) {
    if (owner) {   // workgroup-uniform; no copy is in flight, so the ring is free
      append_token<BITS>(a, ap, n, h, new_blk, new_row, reinterpret_cast<uint2*>(s_ring), tid);
      prologue_copies();
    }
  }
  const bool col_lo = m >= 8;
  const bool col_live = (m & 7) < gcount;

  // value accumulators: 8-dim tiles t (4-bit), or dim-pair tiles T of the
  // table path (row R = 4g + r holds dims 8R + 2T and 8R + 2T + 1, by the
  // column's parity)
  constexpr int kTiles = kTab ? 4 : 8;
  f32x4 acc[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const uint32_t r4 = (uint32_t)(lane & 31) << 2;             // this lane's table copy
  const uint32_t par_mul = col_lo ? 65536u : 1u;
  const float v_unscale = a.f16_v.unscale;
  float run_m = -INFINITY, run_l = 0.f;

  // logit B operands stay in registers for the whole loop
  constexpr int QS = DecodeSmem<BITS>::kQSteps;
  u32x4 qreg[QS];
#pragma unroll
  for (int st = 0; st < QS; ++st) qreg[st] = s_qb[st][lane];
  // QJL: B operands of the sketch product, built in the same storage once
  // every wave holds its query operands.  Column c -> head c % 8, part c / 8
  // (f16 w_hi, f16 residual); in the operand of lane (c, g) at step st, slot
  // 2k carries coordinate j = 32g + 4st + k and slot 2k + 1 coordinate j + 16,
  // whose sign bits sit at bits 4st + k and 4st + k + 16 of word g of the
  // token's sign record.
  [[maybe_unused]] u32x4 wreg[QJL ? 4 : 1];
  if constexpr (QJL) {
    __syncthreads();
    const int r = tid >> 4, p = tid & 15;
    if (r < 8) {
      uint16_t* wb = reinterpret_cast<uint16_t*>(sm.qs);   // 4 KB: 4 steps x 64 lanes x 16 B
      const int lo = perm16(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * lo + e, gq = d >> 5, j = d & 31;
        const int st = (j & 15) >> 2, sl = 2 * (j & 3) + (j >> 4);
        const _Float16 hh = (_Float16)wq[e];
        const _Float16 hl = (_Float16)(wq[e] - (float)hh);
        wb[(st * 64 + r + 16 * gq) * 8 + sl] = __builtin_bit_cast(uint16_t, hh);
        wb[(st * 64 + r + 8 + 16 * gq) * 8 + sl] = __builtin_bit_cast(uint16_t, hl);
      }
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 4; ++st) wreg[st] = reinterpret_cast<const u32x4*>(sm.qs)[st * 64 + lane];
  }
  // After the logit products, the two 8-lane halves of every row hold the
  // two parts of the same head's sums (column m: q_hi / Qh for m < 8, q_lo /
  // Ql for m >= 8).  Each half keeps one block of the pair: lanes m < 8 take
  // block 0, lanes m >= 8 block 1, and receive the other part of their block
  // from the lane 8 columns away, so the softmax runs once per logit.
  //  8-bit logits: v = 256 hi-plane sum + lo-plane sum of a column (exact
  //  int32); head logit = (256 v[Qh column] + v[Ql column] + offset) * unit.
  const int xo = col_lo ? 1 : 0;   // this lane's block of the pair
  const float kmult = kI8 ? sm.qmult[m & 7] : 1.f;
  const float w_own = kI8 ? (col_lo ? 1.f : 256.f) * kmult : 1.f;
  const float w_par = kI8 ? (col_lo ? 256.f : 1.f) * kmult : 1.f;
  const float kc = kI8 ? sm.qcorr[m & 7] * kmult : 0.f;
  const KeyI8Tab kt = {a.ki8_hi[0], a.ki8_hi[1], a.ki8_lo[0], a.ki8_lo[1]};

  // QJL: the residual estimate of both blocks of a pair, C[16 tokens x 16]
  // = S[16 x 128] W[128 x 16], S = the tokens' sign bits as f16 +-1 (exact),
  // W = R' R q split into f16 halves like the query; each word's two sign
  // bits move to the two f16 sign positions with one shift and one and-or
  [[maybe_unused]] auto sketch_pair = [&](const PairQjl& qj, f32x4(&cq)[2]) {
#pragma unroll
    for (int X = 0; X < 2; ++X) cq[X] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        u32x4 sa;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int sh = 15 - 4 * st - q;
          sa[q] = ((sh ? qj.sw[X] << sh : qj.sw[X]) & 0x80008000u) | 0x3C003C00u;
        }
        cq[X] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, sa),
                                                       __builtin_bit_cast(f16x8, wreg[st]), cq[X], 0, 0, 0);
      }
  };
  constexpr float kTau = 0.1107783657f;   // sqrt(pi/2) / sqrt(128)
  auto compute_pair = [&](const BlockRegs<BITS>(&cur)[2], const PairNorms& nrm, [[maybe_unused]] const PairQjl& qj, int lb0) {
    // ---- logits of the two blocks (log2 units)
    float fv[2][4];   // 8-bit path: this lane's column of each block's product
    f32x4 ck[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // table path: the products
    if constexpr (kI8) {
      // signed-byte planes of the centroids built on the vector unit, two
      // 64-dim steps per block, one product chain per (block, plane)
      i32x4 c1[2], c2[2];
#pragma unroll
      for (int X = 0; X < 2; ++X) c1[X] = c2[X] = (i32x4){0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int X = 0; X < 2; ++X) {
          uint32_t h[4], l[4];
          key_planes_b4(cur[X].k[2 * st], kt, h[0], h[1], l[0], l[1]);
          key_planes_b4(cur[X].k[2 * st + 1], kt, h[2], h[3], l[2], l[3]);
          const u32x4 ah = {h[0], h[1], h[2], h[3]}, al = {l[0], l[1], l[2], l[3]};
          c1[X] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, ah),
                                                        __builtin_bit_cast(i32x4, qreg[st]), c1[X], 0, 0, 0);
          c2[X] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, al),
                                                        __builtin_bit_cast(i32x4, qreg[st]), c2[X], 0, 0, 0);
        }
      // |hi-plane sum| <= 128 * 2^14, so 256 * it + the lo-plane sum fits in int32
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int j = 0; j < 4; ++j) fv[X][j] = (float)((c1[X][j] << 8) + c2[X][j]);
    } else {
      // f16 products over the pair tables: in step st the lane's A operand
      // holds the scaled halves of its codes 8st .. 8st+7 (dims 32g + 8st +
      // 0..7 of token row m), one table read per two codes
      const uint32_t* const tk = sm.tk;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int X = 0; X < 2; ++X) {
          u32x4 av;
#pragma unroll
          for (int q = 0; q < 4; ++q) av[q] = lds_word(tk, pair_addr<2 * BITS>(cur[X].k, 4 * st + q, r4));
          ck[X] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av),
                                                         __builtin_bit_cast(f16x8, qreg[st]), ck[X], 0, 0, 0);
        }
      if constexpr (QJL) {
        // each logit gains sqrt(pi/2)/sqrt(d) rho_t times its sketch sum,
        // before the two halves are added and the key norm applied
        f32x4 cq[2];
        sketch_pair(qj, cq);
#pragma unroll
        for (int X = 0; X < 2; ++X)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float tr = (j & 1) ? mul_h_hi(kTau, qj.rh[X][j >> 1]) : mul_h_lo(kTau, qj.rh[X][j >> 1]);
            ck[X][j] = __builtin_fmaf(tr, cq[X][j], ck[X][j]);
          }
      }
    }
    // own block's part, plus the other part from the lane 8 columns away,
    // times the token's key norm: the table path does both in logits_tab
    float s[4];
    if constexpr (kTab) {
      logits_tab(ck[0], ck[1], nrm.gk, s);
    } else {
      float cs[4], send[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cs[j] = fmaf(col_lo ? fv[1][j] : fv[0][j], w_own, kc);
        send[j] = col_lo ? fv[0][j] : fv[1][j];
      }
      fmac_ror8_4(cs, send, w_par);
      if constexpr (QJL) {
        // the own block's sketch sum: own column plus the partner's column
        // (the lane 8 away keeps the other block), times tau rho_t
        f32x4 cq[2];
        sketch_pair(qj, cq);
        float qo[4], qs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          qo[j] = col_lo ? cq[1][j] : cq[0][j];
          qs[j] = col_lo ? cq[0][j] : cq[1][j];
        }
        fmac_ror8_4(qo, qs, 1.f);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t rh = col_lo ? qj.rh[1][j >> 1] : qj.rh[0][j >> 1];
          const float tr = (j & 1) ? mul_h_hi(kTau, rh) : mul_h_lo(kTau, rh);
          cs[j] = __builtin_fmaf(tr, qo[j], cs[j]);
        }
      }
      scale_by_norms(cs, nrm.gk, s);
    }
    // ---- value operands: table reads issued before the softmax needs them
    u32x4 va[8];
    if constexpr (kTab) {
      // product (block X, tile T) is va[4X + T]: rows = dim pairs (8m + 2T,
      // 8m + 2T + 1), K slots (2j, 2j + 1) of lane group g = the pair's two
      // dims of token 4g + j, so one table read gives one operand word
      const uint32_t* const tv = sm.tv;
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int T = 0; T < 4; ++T)
#pragma unroll
          for (int j = 0; j < 4; ++j) va[4 * X + T][j] = lds_word(tv, v_field_addr<BITS>(cur[X].v[j], T, r4));
    } else {
      // tile t = dims 8m+t; the A operand pairs tokens (4g, 4g+1),
      // (4g+2, 4g+3) of each block
      uint32_t iv[4][8];   // [word pair][t]: code(first) | code(second) << BITS
#pragma unroll
      for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t wa = cur[X].v[2 * q], wb = cur[X].v[2 * q + 1];
          // whole-word masks: byte k of ze / zo is the pair index of dim
          // 2k / 2k + 1 (the low nibble from wa, the high one from wb)
          constexpr uint32_t M = 0x0F0F0F0Fu;
          uint32_t ze = (wa & M) | ((wb << 4) & ~M);
          uint32_t zo = ((wa >> 4) & M) | (wb & ~M);
          // built once: each index below is one byte-select shift of these
          asm volatile("" : "+v"(ze), "+v"(zo));
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            iv[2 * X + q][2 * k] = (ze >> (8 * k)) & 0xFFu;
            iv[2 * X + q][2 * k + 1] = (zo >> (8 * k)) & 0xFFu;
          }
        }
#pragma unroll
      for (int t = 0; t < 8; ++t) va[t] = (u32x4){s_tv2[iv[0][t]], s_tv2[iv[1][t]], s_tv2[iv[2][t]], s_tv2[iv[3][t]]};
    }

    // ---- this lane's 4 logits: tokens 4g .. 4g+3 of block xo, head m % 8
    const uint32_t(&gv2)[2] = nrm.gv;
    const int tok0 = (lb0 + xo) * kBlock + 4 * g;
    if ((lb0 + 2) * kBlock > tok_end) {   // pair reaches past the split's last token
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (tok0 + j >= tok_end) s[j] = -INFINITY;
    }
    if constexpr (LOGITS) {
      if (col_live) {
        float* lrow = a.logits + ((int64_t)n * Hq + (int64_t)h * a.group + g0 + (m & 7)) * a.logits_stride;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (tok0 + j < tok_end) lrow[tok0 + j] = s[j] * (1.f / LOG2E);
      }
    }
    // ---- online softmax over the 32 tokens (per head: both row halves)
    float bm = vmax(vmax3(s[0], s[1], s[2]), s[3]);
    bm = vmax_ror8(bm);
    const float new_m = vmax_rows(bm, run_m);
    // rescale only when some head's running max moved (rare after the first
    // blocks); the accumulators stay in the matrix-core registers otherwise
    if (__builtin_amdgcn_ballot_w64(new_m > run_m) != 0) {
      const float alpha = (run_m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(run_m - new_m);
      run_l *= alpha;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) acc[t] *= alpha;
    }
    run_m = new_m;
    // all masked: exp2(-inf) = 0; heads past the slice: +inf, so p = 0
    const float mref = !col_live ? INFINITY : (new_m == -INFINITY) ? 0.f : new_m;
    if constexpr (kTab) {
      // B of the value product for block X: K slots (2j, 2j + 1) = (token
      // 4g + j, dim parity 0 / 1); column c takes head c % 8 at parity c / 8,
      // so its f16(p gamma_v) sits in the low half (c < 8) or the high half
      // (c >= 8) of slot pair j and the other half is zero.  Lanes hold
      // their own block's p: the other block's comes from the lane 8 columns
      // away (block 0 into lanes c >= 8, block 1 into lanes c < 8).
      // (the value table holds S_v c: 1/S_v is applied when the waves merge)
      uint32_t hv[4], hi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = __builtin_amdgcn_exp2f(s[j] - mref);
        run_l += p;
        const uint32_t gw = gv2[j >> 1];
        const _Float16 gh = __builtin_bit_cast(_Float16, (uint16_t)((j & 1) ? (gw >> 16) : (gw & 0xFFFFu)));
        hv[j] = __builtin_bit_cast(uint16_t, (_Float16)(p * (float)gh));
        hi[j] = hv[j] << 16;
      }
      value_b_tab(hv, hi, par_mul);
      const u32x4 b0 = {hv[0], hv[1], hv[2], hv[3]}, b1 = {hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, va[T]),
                                                       __builtin_bit_cast(f16x8, b0), acc[T], 0, 0, 0);
        acc[T] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, va[4 + T]),
                                                       __builtin_bit_cast(f16x8, b1), acc[T], 0, 0, 0);
      }
    } else {
      uint32_t hi[2], lo[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float pv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const float p = __builtin_amdgcn_exp2f(s[2 * q + u] - mref);
          run_l += p;
          pv[u] = u ? mul_h_hi(p, gv2[q]) : mul_h_lo(p, gv2[q]);
        }
        // f16(pv) (rounded toward zero) and the f16 of its residual, exact in f32
        const auto ph = __builtin_amdgcn_cvt_pkrtz(pv[0], pv[1]);
        const auto pl = __builtin_amdgcn_cvt_pkrtz(pv[0] - (float)ph[0], pv[1] - (float)ph[1]);
        hi[q] = __builtin_bit_cast(uint32_t, ph);
        lo[q] = __builtin_bit_cast(uint32_t, pl);
      }
      // B columns 0..7 take f16(p gamma_v) of both blocks, columns 8..15 its
      // residual: lanes m < 8 send their block-0 residuals across, lanes m >= 8
      // their block-1 high parts
      uint32_t snd[2] = {col_lo ? hi[0] : lo[0], col_lo ? hi[1] : lo[1]}, rcv[2];
      ror8_2(snd, rcv);
      const u32x4 pb = col_lo ? (u32x4){rcv[0], rcv[1], lo[0], lo[1]} : (u32x4){hi[0], hi[1], rcv[0], rcv[1]};
      // ---- values: one product per 8-dim tile
#pragma unroll
      for (int t = 0; t < 8; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, va[t]),
                                                       __builtin_bit_cast(f16x8, pb), acc[t], 0, 0, 0);
    }
  };

  // ---- main loop: wait for stage k, read it, refill it with pair k + NS
  // (its block-table entries were fetched one iteration earlier)
  // The loop is unrolled by the ring depth, so each stage's LDS offset is a
  // constant of the read instructions.
  const uint8_t* ring = s_ring + wv * C::kWaveRing;
  const int own_slot = col_lo ? C::kSlot : 0;   // the lane's block of the pair
  auto step = [&](int k, int u) {   // pair k sits in stage u = k % NS
    wait_pairs_behind<BITS, QJL>(min(NS - 1, my_n - 1 - k));
    // the block-table loads are older than the copy just waited for; this
    // keeps their uses below that wait
    asm volatile("" : "+v"(ids0), "+v"(ids1));
    const uint8_t* st = ring + u * 2 * C::kSlot;
    BlockRegs<BITS> cur[2];
    PairNorms nrm;
    read_chunk<BITS>(cur[0], st, m, g);
    read_chunk<BITS>(cur[1], st + C::kSlot, m, g);
    read_norms<BITS>(nrm, st + own_slot, g);
    PairQjl qj;
    if constexpr (QJL) {
#pragma unroll
      for (int X = 0; X < 2; ++X) {
        const uint8_t* sx = st + X * C::kSlot;
        qj.sw[X] = *reinterpret_cast<const uint32_t*>(sx + C::kOffSign + 16 * m + 4 * g);
        const uint2 rr = *reinterpret_cast<const uint2*>(sx + C::kOffRho + 8 * g);
        qj.rh[X][0] = rr.x;
        qj.rh[X][1] = rr.y;
      }
    }
    if (k + NS < my_n) {
      // the stage is overwritten only after this wave's reads of it are done
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      dma_pair(k + NS, (int)__builtin_amdgcn_readlane(ids0, k + NS), (int)__builtin_amdgcn_readlane(ids1, k + NS));
    }
    compute_pair(cur, nrm, qj, sb0 + 2 * (wv + NW * k));
  };
  for (int k0 = 0; k0 < my_n; k0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u)
      if (k0 + u < my_n) step(k0 + u, u);
  }

  // ---- merge the NW waves of the workgroup (each wave's accumulator goes
  // into its own ring, whose copies have all been waited for)
  run_l = sum_rows(run_l);
  run_l += dpp<kDppRor8>(run_l);   // the two row halves hold the pair's two blocks
  if (g == 0 && m < 8) {
    s_wm[wave][m] = run_m;
    s_wl[wave][m] = run_l;
  }
  float* s_acc = reinterpret_cast<float*>(s_ring + wave * C::kWaveRing);   // [column][kAccRow]
  if constexpr (kTab) {
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j) s_acc[(m & 7) * kAccRow + 8 * (4 * g + j) + 2 * T + (m >> 3)] = acc[T][j] * v_unscale;
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) s_acc[m * kAccRow + 8 * (4 * g + j) + t] = acc[t][j];
  }
  __syncthreads();

  const int64_t nsplit = a.num_splits;
  float* part_base = a.partials + (((int64_t)n * Hkv + h) * nsplit) * a.group * kPartStride;
  if (tid < 8) {
    float M = -INFINITY;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_wm[w][tid]);
    float L = 0.f;
    for (int w = 0; w < NW; ++w)
      if (s_wm[w][tid] != -INFINITY) L += s_wl[w][tid] * __builtin_amdgcn_exp2f(s_wm[w][tid] - M);
    s_ml[0][tid] = M;
    s_ml[1][tid] = L;
  }
  __syncthreads();
  for (int i = tid; i < gcount * kD; i += NT) {
    const int hd = i >> 7, d = i & (kD - 1);
    const float M = s_ml[0][hd];
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_wm[w][hd];
      const float* sa = reinterpret_cast<const float*>(s_ring + w * C::kWaveRing);
      if (mw != -INFINITY)
        o += __builtin_amdgcn_exp2f(mw - M) * (kTab ? sa[hd * kAccRow + d] : sa[hd * kAccRow + d] + sa[(hd + 8) * kAccRow + d]);
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

static int check_mfma_args(const DecodeArgs& a, int bits, bool qjl) {
  // the kernel's chunk geometry is fixed at compile time: values, and the
  // QJL sidecar right after the norms
  const int64_t expect = 512 * bits + 64 + (qjl ? 32 + 256 : 0);
  if (a.lay.block_bytes != expect || a.lay.off_k != 0 || a.lay.off_v != 256 * bits ||
      a.lay.off_gk != 512 * bits || a.lay.off_gv != 512 * bits + 32 ||
      (qjl && (a.lay.off_rho != 512 * bits + 64 || a.lay.off_sign != 512 * bits + 96)) ||
      (reinterpret_cast<uintptr_t>(a.pool) & 15) != 0)
    return (int)hipErrorInvalidValue;
  if (bits < 2 || bits > 4) return (int)hipErrorInvalidValue;
  // 4-bit keys need the integer form of the key codebook (odd-symmetric)
  if (bits == 4 && !(a.ki8_unit > 0.f)) return (int)hipErrorInvalidValue;
  // a wave keeps the block-table entries of its pairs one per lane
  const int nw = bits == 4 ? DecodeSmem<4>::kWaves : DecodeSmem<3>::kWaves;
  if (a.blocks_per_split < 1 || a.blocks_per_split > 2 * nw * 64) return (int)hipErrorInvalidValue;
  return 0;
}

template <bool APPEND, typename AP>
static void launch_mfma(const DecodeArgs& a, const AP& ap, int bits, bool qjl, int ns, int gs, hipStream_t s) {
  const dim3 grid((unsigned)a.num_splits, (unsigned)(a.num_kv_heads * ns), (unsigned)a.num_seqs);
  const bool lg = a.logits != nullptr;
  if constexpr (!APPEND) {
    if (qjl) {
      if (bits == 2) {
        if (lg) hipLaunchKernelGGL((decode_mfma_kernel<2, true, false, true>), grid, dim3(64 * DecodeSmem<2>::kWaves), 0, s, a, ns, gs, ap);
        else hipLaunchKernelGGL((decode_mfma_kernel<2, false, false, true>), grid, dim3(64 * DecodeSmem<2>::kWaves), 0, s, a, ns, gs, ap);
      } else if (bits == 4) {
        if (lg) hipLaunchKernelGGL((decode_mfma_kernel<4, true, false, true>), grid, dim3(64 * DecodeSmem<4>::kWaves), 0, s, a, ns, gs, ap);
        else hipLaunchKernelGGL((decode_mfma_kernel<4, false, false, true>), grid, dim3(64 * DecodeSmem<4>::kWaves), 0, s, a, ns, gs, ap);
      } else {
        if (lg) hipLaunchKernelGGL((decode_mfma_kernel<3, true, false, true>), grid, dim3(64 * DecodeSmem<3>::kWaves), 0, s, a, ns, gs, ap);
        else hipLaunchKernelGGL((decode_mfma_kernel<3, false, false, true>), grid, dim3(64 * DecodeSmem<3>::kWaves), 0, s, a, ns, gs, ap);
      }
      return;
    }
  }
  switch (bits) {
    case 2:
      if (lg) hipLaunchKernelGGL((decode_mfma_kernel<2, true, APPEND>), grid, dim3(64 * DecodeSmem<2>::kWaves), 0, s, a, ns, gs, ap);
      else hipLaunchKernelGGL((decode_mfma_kernel<2, false, APPEND>), grid, dim3(64 * DecodeSmem<2>::kWaves), 0, s, a, ns, gs, ap);
      break;
    case 3:
      if (lg) hipLaunchKernelGGL((decode_mfma_kernel<3, true, APPEND>), grid, dim3(64 * DecodeSmem<3>::kWaves), 0, s, a, ns, gs, ap);
      else hipLaunchKernelGGL((decode_mfma_kernel<3, false, APPEND>), grid, dim3(64 * DecodeSmem<3>::kWaves), 0, s, a, ns, gs, ap);
      break;
    default:
      if (lg) hipLaunchKernelGGL((decode_mfma_kernel<4, true, APPEND>), grid, dim3(64 * DecodeSmem<4>::kWaves), 0, s, a, ns, gs, ap);
      else hipLaunchKernelGGL((decode_mfma_kernel<4, false, APPEND>), grid, dim3(64 * DecodeSmem<4>::kWaves), 0, s, a, ns, gs, ap);
      break;
  }
}

int launch_decode_mfma(const DecodeArgs& a, int bits, bool qjl, int ns, int gs, void* stream) {
  const int e = check_mfma_args(a, bits, qjl);
  if (e) return e;
  launch_mfma<false>(a, NoAppend{}, bits, qjl, ns, gs, static_cast<hipStream_t>(stream));
  return (int)hipGetLastError();
}

// Decode step: append each sequence's new token, attend, merge.
int launch_decode_step(const DecodeArgs& a, const AppendArgs& ap, int bits, void* stream) {
  const int e = check_mfma_args(a, bits, false);
  if (e) return e;
  const int ns = decode_slices(a.group);
  const int gs = (a.group + ns - 1) / ns;
  launch_mfma<true>(a, ap, bits, false, ns, gs, static_cast<hipStream_t>(stream));
  const hipError_t le = hipGetLastError();
  if (le != hipSuccess) return (int)le;
  return launch_merge(a, stream);
}

}  // namespace tq
