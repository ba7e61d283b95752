// Internal structures shared by the host code (tq_host.cpp) and the HIP
// kernels.  Everything a kernel needs about a cache travels by value in its
// kernel-argument struct (a few hundred bytes): codebooks, the bucket lookup
// table of the threshold search, and the rotation signs as bit masks.
#pragma once

#include <stdint.h>

namespace tq {

constexpr int kD = 128;          // head dimension supported by the kernels
constexpr int kBlock = 16;       // tokens per cache block
constexpr int kLutMax = 96;      // buckets of the threshold-search table
constexpr int kMaxGroup = 16;    // query heads per KV head
constexpr int kPartStride = 132; // floats per (split, head) partial: o_rot[128], m, l, pad
constexpr int kMaxSplits = 4096; // splits per (sequence, KV head) of a decode launch

// Codebook of one bit width, plus the bucket table used by the encoder's
// threshold search: for y in bucket k = clamp(floor(y*lut_scale+lut_offset)),
// code = lut_base[k] + (y > lut_thr[k]).  The host builds the grid so that a
// bucket holds at most one threshold and every threshold sits at least 1e-6
// away from a bucket edge; a y that rounds into a neighbouring bucket then
// still gets the exact threshold count.
struct CodecTables {
  int32_t bits;
  int32_t lut_n;
  float lut_scale;
  float lut_offset;
  float centroid[16];           // ascending, fp32
  float threshold[15];          // fp32 midpoints
  float lut_thr[kLutMax];       // +inf when the bucket holds no threshold
  int32_t lut_base[kLutMax];
};

// Rotation signs as a bit mask: bit j of neg[j/32] set <=> s_j = -1.
struct SignMask {
  uint32_t neg[kD / 32];
};

// Exact division by a runtime constant for numerators below 2^31.
struct FastDiv {
  uint32_t mul;
  uint32_t shift;
};

inline FastDiv make_fast_div(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const unsigned __int128 num = (unsigned __int128)1 << (31 + l);
  const uint64_t m = (uint64_t)((num + d - 1) / d);
  return FastDiv{(uint32_t)m, 31 + l};
}

struct Layout {
  int64_t block_bytes;
  int64_t off_k, off_v, off_gk, off_gv, off_rho, off_sign;
  int32_t k_rec, v_rec;
};

// ---------------------------------------------------------------- encode --
struct EncodeStream {
  const void* src;        // [tokens][heads][128]
  int64_t rec_off;        // code region offset inside (block, head)
  int64_t norm_off;       // fp16 norm region offset
  int32_t rec_bytes;
  int32_t qjl;            // 1: also write the QJL sidecar (keys only)
};

struct EncodeArgs {
  EncodeStream stream[2];   // gridDim.y streams (K, then V)
  const int32_t* slot_mapping;
  uint8_t* pool;
  int64_t num_vectors;      // tokens * heads
  int64_t num_slots;        // num_blocks * 16; larger slots are skipped
  int64_t block_bytes;
  int64_t rho_off, sign_off;
  int32_t num_heads;
  FastDiv div_heads;
  SignMask rot, rot_qjl;
  CodecTables tab;
};

// ---------------------------------------------------------------- decode --
// A codebook as IEEE half operands of the matrix-core decode: h[i] is the
// half nearest S c_i for the host-chosen scale S; unscale = 1/S.  max_err =
// max_i |h_i / S - c_i|.
struct F16Codebook {
  uint32_t h[16];
  float unscale;
  float max_err;
};

struct DecodeArgs {
  const void* q;            // [seqs][q_heads][128]
  const uint8_t* pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* out;               // [seqs][q_heads][128] (attend)
  float* logits;            // [seqs][q_heads][logits_stride] or null
  float* partials;          // [seqs][kv_heads][splits][group][kPartStride]
  int64_t logits_stride;
  Layout lay;
  int64_t num_blocks;       // block-table entries outside [0, num_blocks) read as block 0
  int32_t q_dtype;
  int32_t num_seqs, num_q_heads, num_kv_heads, group;
  int32_t max_blocks, blocks_per_split, num_splits;
  float scale;
  SignMask rot, rot_qjl;
  float cent_k[16];
  float cent_v[16];
  // Keys as 8-bit integer planes for the matrix-core logits: centroid i of
  // the negative half (i < 2^(b-1)) is (256*hi_i + lo_i + 128.5) * ki8_unit,
  // bytes hi_i / lo_i packed four to a word; a code of the positive half
  // takes the bitwise NOT of both bytes of its mirror 2^b-1-i, which is the
  // mirror's value negated because the codebook is odd-symmetric.
  uint32_t ki8_hi[2], ki8_lo[2];
  float ki8_unit;
  // 2- and 3-bit keys and values: the codebooks as scaled halves
  F16Codebook f16_k, f16_v;
};

// Decode step with append: each sequence's new token (position seq_len - 1,
// its slot taken from the block table) is encoded into the cache by the
// split that holds its block, before that split streams the block.
struct AppendArgs {
  const void* k_new;        // [seqs][kv_heads][128]
  const void* v_new;
  int32_t dtype;            // 0 fp32, 1 fp16, 2 bf16
  CodecTables tab;          // keys and values share the bit width
};
struct NoAppend {};

// ----------------------------------------------------------- reconstruct --
struct ReconArgs {
  const uint8_t* pool;
  const int32_t* slots;
  float* out;               // [n][heads][128]
  int64_t n_vectors;        // n * heads
  int64_t num_slots;        // slots outside [0, num_slots) give zero vectors
  int64_t rec_off, norm_off, block_bytes;
  int32_t rec_bytes, bits, num_heads;
  FastDiv div_heads;
  SignMask rot;
  float centroid[16];
};

// Decompression of cache rows to 16-bit floats (keys and values in one launch).
struct DecompStream {
  void* out;                // [n][heads][128] of out_dtype; nullptr: stream skipped
  int64_t rec_off, norm_off;
  int32_t rec_bytes, bits;
  float centroid[16];
};
struct DecompArgs {
  const uint8_t* pool;
  const int32_t* slots;
  int64_t n_vectors;        // n * heads
  int64_t num_slots;        // slots outside [0, num_slots) give zero vectors
  int64_t block_bytes;
  int32_t num_heads, out_dtype;   // TQ_F16 = 1, TQ_BF16 = 2
  FastDiv div_heads;
  SignMask rot;
  DecompStream stream[2];   // keys, values
};

// Min/max comparison codec on flat buffers: per vector, d*b/8 bytes of codes
// (LSB first) and two fp16 words (scale, zero point).
struct MinmaxArgs {
  const void* src;          // encode: [n][128] of in_dtype
  uint8_t* codes;           // [n][16 * bits]
  uint16_t* params;         // [n][2]: fp16 scale, fp16 zero point
  void* out;                // decode: [n][128] of out_dtype
  int64_t n;
  int32_t in_dtype, out_dtype;   // 0 fp32, 1 fp16, 2 bf16
  SignMask rot;
};

// Triplet codec on flat buffers.  Per vector: kOctoTri fields of
// 2 (b+1) + (b-1) bits (xi code | eta code << (b+1) | norm code << 2(b+1)),
// triplet i at bit i * field_bits, LSB first, in a record of whole 32-bit
// words; the norm gamma as fp16 beside it.
constexpr int kOctoTri = 43;        // ceil(128 / 3); the last triplet is (y126, y127, 0)
constexpr int kOctoMaxGroup = 16;   // queries per head of a logits launch
struct OctoArgs {
  const void* src;          // encode: [n][128] of dtype
  const float* dirs;        // [nd * nd][4] unit directions (x, y, z, 0), nd = 2^(b+1)
  uint8_t* codes;           // [heads][n][rec_bytes]
  uint16_t* gamma;          // [heads][n] fp16
  const float* q;           // logits: [heads][group][128] fp32
  float* out;               // logits: [heads][group][n]
  int64_t n;
  int32_t dtype, heads, group;
  float scale;
  SignMask rot;
  float crho[8];            // norm centroids (2^(b-1) used)
  float trho[8];            // thresholds, +inf past the last
  // OCTOPUS-QJL (null: the plain codec): per vector 16 bytes of residual
  // sketch signs and the residual norm (fp16); written by the encoder, read
  // by the logits
  uint8_t* qjl_signs;       // [heads][n][16]
  uint16_t* qjl_rho;        // [heads][n] fp16
  SignMask rot_qjl;
  // decode-attend over triplet-coded keys (codes, gamma) and values
  const uint8_t* vcodes;    // [heads][n][rec_bytes]
  const uint16_t* vgamma;   // [heads][n] fp16
  float* partials;          // [heads][splits][group][kPartStride]
  int64_t split_len;        // keys per split, a multiple of kOctoAttChunk
  int32_t num_splits;
};
constexpr int kOctoAttChunk = 128;   // keys a decode-attend workgroup stages at a time

// The fixed decode scratch of tq_decode_attend_noalloc (tq_scratch.hip):
// 16 MiB per GPU.  scratch_buffer returns this device's copy (resolved on
// the first call per device, with it current) and its size; hipError_t value.
constexpr int64_t kScratchBytes = 16 << 20;
int scratch_buffer(void** ptr, int64_t* bytes);

// Launchers implemented in the .hip files; return a hipError_t value.
int launch_encode(const EncodeArgs& a, int num_streams, int in_dtype, void* stream);
int launch_decode(const DecodeArgs& a, int bits_k, int bits_v, int qjl, int attend, int mfma, void* stream);
int decode_slices(int group);
int launch_decode_mfma(const DecodeArgs& a, int bits, bool qjl, int ns, int gs, void* stream);
int launch_merge(const DecodeArgs& a, void* stream);
int launch_decode_step(const DecodeArgs& a, const AppendArgs& ap, int bits, void* stream);
int launch_reconstruct(const ReconArgs& a, void* stream);
int launch_decompress(const DecompArgs& a, void* stream);
int launch_minmax_encode(const MinmaxArgs& a, int bits, void* stream);
int launch_minmax_decode(const MinmaxArgs& a, int bits, void* stream);
int launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);
int launch_octo_encode(const OctoArgs& a, int bits, void* stream);
int launch_octo_logits(const OctoArgs& a, int bits, void* stream);
int launch_octo_attend(const OctoArgs& a, int bits, void* stream);   // then launch_merge

}  // namespace tq
