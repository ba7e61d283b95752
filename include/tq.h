/*
 * tq.h - C ABI of libtq: rotation-preconditioned (TurboQuant-style) KV-cache
 * compression for one AMD MI355X (gfx950).
 *
 * Sources of the operations (page titles as printed on the pages):
 *   [P1] "TurboQuant: KV Cache Vector Quantization" (llm-engineer card):
 *        three stages Split / Rotate / Codebook, online compression.
 *   [P2] "TurboQuant: KV Cache Compression" (Bit-Axon docs): quantisation
 *        function Q(K) = argmin over the codebook, dequantisation, attention
 *        over the quantised cache softmax(Q K^T / sqrt(d_h)) V, planned API
 *        TurboQuant(bits).compress / decompress.
 *   [P3] OCTOPUS summary (aitrends.kr): Method steps 1-2 (norm/direction
 *        split, R = H diag(s)), glossary entries "Walsh-Hadamard rotation" and
 *        "Lloyd-Max quantization", contribution "Optional 1-bit QJL residual
 *        for unbiased dot-product".
 *   [P4] TurboQuant deep-dive blog (cell-devlog): Step 1 randomized Hadamard
 *        transform (sign flip, Hadamard, 1/sqrt(d)); Step 2 compress_key
 *        (fp16 magnitude + direction indices, 128*4+16 = 528 bits); the
 *        TurboQuantConfig(key_bits, value_bits, hadamard_seed) example.
 *
 * Conventions for every entry point:
 *   - Return value: TQ_OK (0) or a negative tq_status.  Nothing aborts and no
 *     C++ exception crosses the ABI.  tq_last_error() gives a thread-local
 *     text for the last failure on the calling thread.
 *   - "device" pointers are HIP device memory on the current device, owned by
 *     the caller; the library never frees them.  "host" pointers are ordinary
 *     process memory.
 *   - GPU work is enqueued on the caller's hipStream_t (passed as void*; NULL
 *     is the default stream) and is asynchronous: the caller synchronises.
 *     Argument checks are synchronous; kernel faults surface as HIP errors on
 *     the stream and are reported as TQ_ERR_HIP by the next call that checks.
 *   - Every array is densely packed in the stated row-major shape.
 *   - Supported now: head dimension d = 128, bits in {2, 3, 4}, 16-token
 *     blocks.  Other values return TQ_ERR_UNSUPPORTED.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_LAYOUT_VERSION 1
#define TQ_BLOCK_TOKENS 16

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1,   /* null/negative/inconsistent argument        */
  TQ_ERR_UNSUPPORTED = -2,   /* valid but not implemented (d, bits, block)  */
  TQ_ERR_BITS_MISMATCH = -3, /* bits argument differs from the cache's      */
  TQ_ERR_OOM = -4,           /* host allocation failed                      */
  TQ_ERR_NO_DEVICE = -5,     /* no usable HIP device                        */
  TQ_ERR_HIP = -6,           /* a HIP runtime call or launch failed         */
  TQ_ERR_WORKSPACE = -7      /* workspace missing or too small              */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_F16 = 1, TQ_BF16 = 2 } tq_dtype;

/* Static text for a status code ("TQ_OK", ...). */
const char* tq_status_string(int status);
/* Detail text of the last failure on this thread ("" if none). */
const char* tq_last_error(void);
/* Cache layout version implemented (TQ_LAYOUT_VERSION). */
int tq_layout_version(void);

/* ---------------------------------------------------------------------------
 * Seeded random rotation R = H diag(s) / sqrt(d)   ([P4] Step 1; [P3] Method
 * step 2 and glossary "Walsh-Hadamard rotation").
 * s_j = +1 if the top bit of the j-th SplitMix64 output for `seed` is 0, else
 * -1 (SplitMix64: Steele, Lea & Flood 2014).  H is the Sylvester Hadamard
 * matrix.  The object is host memory owned by the library, immutable, and
 * freed by tq_rotation_destroy.  d must be a power of two in [2, 4096]. */
typedef struct tq_rotation tq_rotation;
int tq_make_rotation(uint64_t seed, int32_t d, tq_rotation** out);
/* Copies the d signs (+1/-1) into host_out[d]. */
int tq_rotation_signs(const tq_rotation* rot, int8_t* host_out);
int32_t tq_rotation_dim(const tq_rotation* rot);
void tq_rotation_destroy(tq_rotation* rot);

/* ---------------------------------------------------------------------------
 * Lloyd-Max codebook ([P3] glossary "Lloyd-Max quantization": alternating
 * centroid / boundary updates minimising MSE for a 1-D density; [P3] key idea:
 * per-coordinate Lloyd-Max on the rotated marginals).  The density is the
 * coordinate marginal of a uniform unit vector in R^d,
 * f(x) = K_d (1 - x^2)^((d-3)/2).  Outputs (host arrays):
 *   centroids[2^bits]    fp32, ascending (code i <-> centroids[i]);
 *   thresholds[2^bits-1] fp32 midpoints of adjacent fp32 centroids.
 * Computed in float64 on the host, cached per (d, bits). bits in [1, 4]. */
int tq_codebook(int32_t d, int32_t bits, float* centroids, float* thresholds);

/* ---------------------------------------------------------------------------
 * Compressed paged cache.  The pool is caller-owned device memory of
 * tq_cache_bytes() bytes laid out (layout version 1) as
 *   [num_blocks][num_kv_heads][block_bytes], 16 tokens per block;
 *   block = K codes [16][d*bits_k/8] | V codes [16][d*bits_v/8] (bits_v > 0)
 *         | gamma_K [16] fp16 | gamma_V [16] fp16 (bits_v > 0)
 *         | (qjl) rho [16] fp16 | sign bits [16][d/8].
 * A token's code record stores code j at bits [j*b, j*b+b) of the record read
 * as a little-endian bit string; codes are ascending centroid ranks.  QJL sign
 * bit j (bit j of the sign record) is 1 when (R' r)_j < 0. */
typedef struct {
  int32_t d;            /* head dimension (128)                                  */
  int32_t num_kv_heads; /* >= 1                                                  */
  int32_t bits_k;       /* 2..4                                                  */
  int32_t bits_v;       /* 2..4, or 0 for a keys-only cache                      */
  int32_t qjl;          /* 0/1: 1-bit QJL residual sidecar on keys               */
  int32_t block_size;   /* must be 16                                            */
  int64_t num_blocks;   /* >= 1                                                  */
  const tq_rotation* rot;     /* R (shared by keys and values); not owned        */
  const tq_rotation* rot_qjl; /* R' (independent seed) if qjl, else NULL         */
  int32_t layout_version;     /* TQ_LAYOUT_VERSION                               */
} tq_cache_config;

typedef struct {
  int64_t block_bytes;     /* bytes of one (block, kv head)                       */
  int64_t k_rec_bytes, v_rec_bytes;
  int64_t off_k, off_v, off_gamma_k, off_gamma_v, off_rho, off_sign;
  int64_t pool_bytes;
} tq_cache_layout;

/* Pool size in bytes (>= 0) or a negative tq_status. */
int64_t tq_cache_bytes(const tq_cache_config* cfg);
/* Region offsets of layout version 1 for cfg (host only). */
int tq_cache_layout_query(const tq_cache_config* cfg, tq_cache_layout* out);

/* Binds a descriptor to a device pool of tq_cache_bytes(cfg) bytes.  Host only:
 * builds the codebooks and lookup tables; allocates no device memory.  The
 * descriptor copies the rotation signs, so the rotations may be destroyed
 * afterwards.  Freed by tq_cache_destroy (never frees the pool). */
typedef struct tq_cache tq_cache;
int tq_cache_create(const tq_cache_config* cfg, void* device_pool, tq_cache** out);
void tq_cache_destroy(tq_cache* cache);

/* ---------------------------------------------------------------------------
 * Encode ([P1] Split / Rotate / Codebook; [P3] Method steps 1, 2, 6; [P2]
 * Q(K) = argmin; [P4] Step 2 compress_key; optional [P3] QJL residual).
 * For every token t with slot_mapping[t] >= 0 and every KV head h:
 *   gamma = ||x||, y = R x / gamma, code_j = #{i : y_j > thresholds[i]},
 *   stored with fp16(gamma) (round to nearest even, saturated at 65504) at
 *   block slot/16, row slot%16.  With qjl: r = y - c[code], rho = fp16(||r||),
 *   sign bits of R' r.
 *   K, V: device [num_tokens][num_kv_heads][d] of `dtype`; V may be NULL only
 *         for a keys-only cache (and must be NULL then).
 *   slot_mapping: device int32[num_tokens]; -1 skips the token; other values
 *         must be < num_blocks*16 (not checked on the device).
 *   bits: must equal cache bits_k (and bits_v when V is given), else
 *         TQ_ERR_BITS_MISMATCH.
 * Decisions are taken in fp32.  A vector whose fp32 squared norm underflows
 * to 0 is stored as the zero vector (codes 2^(b-1)-1, gamma 0).  Non-finite
 * input is outside the contract. */
int tq_encode_kv(const void* K, const void* V, int32_t dtype, int64_t num_tokens,
                 const int32_t* slot_mapping, int32_t bits, tq_cache* cache,
                 void* hip_stream);

/* ---------------------------------------------------------------------------
 * Decode-attend in the rotated frame ([P2] attention under quantisation;
 * [P4] "RHT preserves inner products, attention can be computed without
 * restoring"; [P3] contribution: the decoder never materialises K_hat).
 *   q:            device [num_seqs][num_q_heads][d], TQ_F32/TQ_F16/TQ_BF16,
 *                 16-byte aligned.
 *                 Query head h reads KV head h / (num_q_heads/num_kv_heads);
 *                 num_q_heads must be a multiple of num_kv_heads with a group
 *                 of at most 16.
 *   block_tables: device int32[num_seqs][max_blocks_per_seq] physical blocks.
 *   seq_lens:     device int32[num_seqs], each in [0, max_blocks_per_seq*16].
 *   scale:        logit scale; <= 0 selects 1/sqrt(d).
 *   out:          device f32 [num_seqs][num_q_heads][d]:
 *                 o = R^T( sum_t softmax_t(s) gamma_v,t c[codes_v,t] ) with
 *                 s_t = scale * gamma_k,t * <R q, c[codes_k,t]> (+ QJL term
 *                 scale*gamma_k,t*rho_t*sqrt(pi/2)/sqrt(d)*<sign_t, R' R q>).
 *                 A sequence of length 0 gets o = 0.
 *   logits_out:   NULL or device f32 [num_seqs][num_q_heads][max_blocks_per_seq*16];
 *                 receives s_t for t < seq_len (other entries untouched).
 *   workspace:    device memory of tq_decode_workspace_bytes() bytes, 16-byte
 *                 aligned, no initial contents needed: it receives the
 *                 per-split partial results (two launches on hip_stream: the
 *                 split pass, then the merge).  Calls that share a workspace
 *                 must not overlap in time.
 * Requires a cache with values (bits_v > 0). */
int64_t tq_decode_workspace_bytes(const tq_cache* cache, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_blocks_per_seq);
int tq_decode_attend(const void* q, int32_t q_dtype, const tq_cache* cache,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_blocks_per_seq, float scale, float* out,
                     float* logits_out, void* workspace, int64_t workspace_bytes,
                     void* hip_stream);

/* Decode-attend without allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops or harnesses that
 * forbid hipMalloc).  The same computation, kernels and arguments as
 * tq_decode_attend, minus the workspace: the per-split partials go to a
 * fixed buffer inside the library, TQ_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU,
 * held from the library's first such call on that GPU until the process
 * ends.  A call whose partials need more (tq_decode_workspace_bytes) returns
 * TQ_ERR_WORKSPACE before touching the device.  The call itself allocates
 * nothing.  Every call on one GPU shares that GPU's buffer: calls that
 * overlap in time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller.  The buffer needs no initial contents
 * (each split writes its partials before the merge reads them). */
#define TQ_NOALLOC_SCRATCH_BYTES (16ll << 20)
int tq_decode_attend_noalloc(const void* q, int32_t q_dtype, const tq_cache* cache,
                             const int32_t* block_tables, const int32_t* seq_lens,
                             int32_t num_seqs, int32_t num_q_heads,
                             int32_t max_blocks_per_seq, float scale, float* out,
                             float* logits_out, void* hip_stream);

/* ---------------------------------------------------------------------------
 * One decode step: append each sequence's new token to the compressed cache
 * and attend over the whole sequence, new token included, in one call with
 * one attend launch ([P1] online compression as tokens arrive, no
 * calibration; [P2] Implementation plan, cache update then attention).
 * Same result as tq_encode_kv of the new tokens followed by tq_decode_attend.
 *   K_new, V_new: device [num_seqs][num_kv_heads][d], kv_dtype TQ_F32 /
 *                 TQ_F16 / TQ_BF16, 16-byte aligned: the new token of every
 *                 sequence;
 *   seq_lens:     counts the new token, which sits at position seq_len - 1:
 *                 slot block_tables[n][(seq_len-1)/16] * 16 + (seq_len-1) % 16
 *                 (the block must be allocated; sequences of length 0 are
 *                 skipped);
 *   other arguments, the workspace and the outputs as tq_decode_attend.
 * The split of the attend kernel that holds the new token's block encodes it
 * (the vector-unit encoder's arithmetic) before streaming that block.  Needs
 * a cache with values of the key bit width and no QJL sidecar
 * (TQ_ERR_BITS_MISMATCH, TQ_ERR_UNSUPPORTED otherwise).  Asynchronous on
 * hip_stream. */
int tq_decode_step(const void* q, int32_t q_dtype, const void* K_new,
                   const void* V_new, int32_t kv_dtype, tq_cache* cache,
                   const int32_t* block_tables, const int32_t* seq_lens,
                   int32_t num_seqs, int32_t num_q_heads,
                   int32_t max_blocks_per_seq, float scale, float* out,
                   float* logits_out, void* workspace, int64_t workspace_bytes,
                   void* hip_stream);

/* Keys-only scores ([P2] Q K_hat^T / sqrt(d_h); [P4] attention logits):
 * logits_out device f32 [num_seqs][num_q_heads][max_blocks_per_seq*16],
 * s_t as in tq_decode_attend for t < seq_len.  Works on any cache. */
int tq_decode_logits(const void* q, int32_t q_dtype, const tq_cache* cache,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_blocks_per_seq, float scale, float* logits_out,
                     void* hip_stream);

/* ---------------------------------------------------------------------------
 * Reconstruct cached vectors in the original frame ([P2] K_hat = DQ(K_q);
 * [P4] Step 2 decompress_key): x_hat = fp16 gamma * R^T c[codes].
 *   slots: device int32[n]; which: 0 = keys, 1 = values;
 *   out:   device f32 [n][num_kv_heads][d]. */
int tq_reconstruct(const tq_cache* cache, const int32_t* slots, int64_t n,
                   int32_t which, float* out, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Decompress cache rows to 16-bit floats, keys and values in one call, for
 * attention over a compressed prefix ([P2] Implementation plan, the planned
 * decompress call; [P2] Math, K_hat = DQ(K_q); [P4] Step 2 decompress_key).
 * For row i of slots and KV head h:
 *   K_out[i][h][:] = round(gamma16_k * R^T c_k[codes_k]),  V_out likewise,
 * computed in fp32 and rounded to nearest even in out_dtype.
 *   slots:     device int32[n], slot = block*16 + row; a slot < 0 or past
 *              the pool gives zero vectors;
 *   out_dtype: TQ_BF16 or TQ_F16;
 *   K_out, V_out: device [n][num_kv_heads][d] of out_dtype, 16-byte aligned,
 *              caller-owned; either may be NULL (not written); V_out must be
 *              NULL for a keys-only cache.
 * Asynchronous on hip_stream.  Errors: TQ_ERR_INVALID_ARG (null cache, n < 0,
 * bad dtype, misaligned output, values asked of a keys-only cache, more than
 * 2^31 vectors), TQ_ERR_NO_DEVICE, TQ_ERR_HIP (launch failure). */
/* ---------------------------------------------------------------------------
 * Comparison codec: per-vector min/max uniform quantiser after the same
 * rotation ([P4] Step 3 compress_value / decompress_value).  y = R x;
 * lo = min_j y_j; scale = (max_j y_j - lo) / (2^bits - 1);
 * code_j = round half to even of (y_j - lo) / scale, in [0, 2^bits - 1]
 * (all codes 0 when scale = 0); scale and lo stored as fp16 (round to
 * nearest even, saturating at +-65504).  Flat buffers, caller-owned:
 *   X:      device [n][128] of dtype (TQ_F32 / TQ_F16 / TQ_BF16), 16-byte aligned;
 *   codes:  device [n][16 * bits] bytes, code j of a vector in bits
 *           [j*bits, (j+1)*bits) LSB first, 4-byte aligned;
 *   params: device [n][2] fp16 words (scale, zero point), 4-byte aligned.
 * bits in {2, 3, 4}; rot: dimension 128.  Asynchronous on hip_stream.
 * Errors: TQ_ERR_INVALID_ARG (null pointer, bad dtype, misalignment, n < 0,
 * n >= 2^31), TQ_ERR_UNSUPPORTED (bits, rotation dimension), TQ_ERR_NO_DEVICE,
 * TQ_ERR_HIP. */
int tq_minmax_encode(const void* X, int32_t dtype, int64_t n, int32_t bits,
                     const tq_rotation* rot, void* codes, void* params,
                     void* hip_stream);

/* Decode of the same buffers: x_hat = R^T (code * scale16 + zero16), in
 * fp32 then written as out_dtype (TQ_F32, or TQ_F16 / TQ_BF16 rounded to
 * nearest even); out: device [n][128], 16-byte aligned. */
int tq_minmax_decode(const void* codes, const void* params, int64_t n,
                     int32_t bits, const tq_rotation* rot, int32_t out_dtype,
                     void* out, void* hip_stream);

int tq_decompress_kv(const tq_cache* cache, const int32_t* slots, int64_t n,
                     int32_t out_dtype, void* K_out, void* V_out,
                     void* hip_stream);

/* ---------------------------------------------------------------------------
 * Octahedral triplet codec ([P3] "Octahedral triplet direction quantizer
 * with norm marginals", "MSE-optimal non-uniform bit allocation", Method
 * steps 1-7), d = 128, budget bits b in {2, 3, 4}.  gamma = ||x||; the
 * rotated direction y = R x / gamma is cut into 43 triplets t_i (the last is
 * (y126, y127, 0)); rho_i = ||t_i||, n_i = t_i / rho_i ((0, 0, 1) when
 * rho_i = 0); (xi, eta) = the equal-area octahedral map of n_i.  xi and eta
 * take (b+1)-bit codes on the uniform grid c_j = -1 + (2j+1)/2^(b+1) (the
 * Lloyd-Max quantiser of their uniform marginal); rho takes a (b-1)-bit
 * Lloyd-Max code for its marginal (rho^2 ~ Beta(3/2, 125/2)).  Joint
 * rounding: among the nearest grid cell and its in-grid neighbours in xi and
 * eta (xi-major, ascending), with n_hat the table direction and the norm code
 * nearest to t_i . n_hat, the first of least ||t_i - rho_hat n_hat||^2 wins.
 *
 * Record of one vector (tq_octo_record_bytes: 40 / 56 / 72 bytes): 43 fields
 * of 2(b+1) + (b-1) bits, field i at bit 7i / 10i / 13i, LSB first, holding
 * xi code | eta code << (b+1) | rho code << 2(b+1); unused bits zero.  gamma
 * is stored beside it as fp16 (round to nearest even, saturating at 65504). */

/* Bytes of one record; negative status for unsupported d or bits. */
int64_t tq_octo_record_bytes(int32_t d, int32_t bits);

/* Bytes of the device direction table of bit budget `bits`:
 * 16 * 4^(bits+1) (4 / 16 / 64 KiB). */
int64_t tq_octo_table_bytes(int32_t bits);

/* Host copies of the tables (computed in float64, rounded to fp32, cached):
 *   dirs:          [4^(bits+1)][4], entry a * 2^(bits+1) + c = the unit
 *                  direction of grid point (c_a, c_c): x, y, z, 0; may be NULL;
 *   rho_centroids: [2^(bits-1)] ascending; may be NULL. */
int tq_octo_codebook(int32_t d, int32_t bits, float* dirs, float* rho_centroids);

/* Fill a caller-owned device buffer of tq_octo_table_bytes(bits) bytes
 * (16-byte aligned) with the direction table; asynchronous on hip_stream.
 * The buffer is what the encode and logits calls of the same bits read. */
int tq_octo_tables(int32_t bits, void* dev_tables, void* hip_stream);

/* Encode n vectors.  X: device [n][128] of dtype (TQ_F32 / TQ_F16 /
 * TQ_BF16), 16-byte aligned; codes: device [n][record bytes], 8-byte aligned;
 * gamma: device [n] fp16; dev_tables / table_bytes: the buffer filled by
 * tq_octo_tables(bits) and its size, at least tq_octo_table_bytes(bits).  All
 * caller-owned.  Asynchronous on hip_stream.  Errors: TQ_ERR_INVALID_ARG
 * (null pointer, dtype, alignment, table too small, n < 0, n >= 2^31),
 * TQ_ERR_UNSUPPORTED (bits, rotation dimension), TQ_ERR_NO_DEVICE, TQ_ERR_HIP. */
int tq_octo_encode(const void* X, int32_t dtype, int64_t n, int32_t bits,
                   const tq_rotation* rot, const void* dev_tables,
                   int64_t table_bytes, void* codes, void* gamma,
                   void* hip_stream);

/* Logits straight from the records, no reconstructed key written ([P3]
 * Method step 7: the dot product from each triplet's norm and direction):
 *   out[h][g][j] = scale * gamma_hj * sum_i rho_hat_hji ((R q_hg)_i . n_hat_hji)
 * which equals scale * q_hg . x_hat_hj.  q: device fp32 [heads][group][128],
 * 16-byte aligned; codes: [heads][n][record bytes]; gamma: [heads][n] fp16;
 * out: fp32 [heads][group][n]; group in 1..16, heads in 1..65535,
 * heads * n < 2^31.  Errors as tq_octo_encode (group > 16 is
 * TQ_ERR_UNSUPPORTED; a non-finite scale is TQ_ERR_INVALID_ARG). */
int tq_octo_logits(const float* q, const void* codes, const void* gamma,
                   int32_t heads, int32_t group, int64_t n, int32_t bits,
                   const tq_rotation* rot, const void* dev_tables,
                   int64_t table_bytes, float scale, float* out,
                   void* hip_stream);

/* OCTOPUS-QJL ([P3] Method step 8, the optional residual sketch that makes
 * the dot-product estimate unbiased).  tq_octo_encode_qjl writes what
 * tq_octo_encode writes, plus a one-bit sketch of what the codes leave out:
 * with y = R k / ||k|| (coordinates 0..127) and y_hat its reconstruction
 * from the codes, r = y - y_hat, z = R' r through the independent rotation
 * rot_qjl, and per vector
 *   signs: 16 bytes, bit j (byte j / 8, bit j % 8) = [z_j < 0];
 *   rho:   fp16 ||r|| (round to nearest even, saturating at 65504).
 * signs: device [n][16], 16-byte aligned; rho: device [n] fp16, 2-byte
 * aligned; both caller-owned.  tq_octo_logits_qjl adds the sketch's
 * estimate of the residual's share to every logit:
 *   out[h][g][j] = scale * gamma_hj * (sum_i rho_hat_hji (R q_hg)_i . n_hat_hji
 *                  + sqrt(pi/2) / sqrt(128) * rho_hj * sum_j' sgn_j' (R' R q_hg)_j')
 * with sgn = +1 for a clear bit, -1 for a set one; signs [heads][n][16] and
 * rho [heads][n] as the encoder wrote them.  Arguments and errors otherwise
 * as tq_octo_encode / tq_octo_logits; a missing or non-128 rot_qjl is
 * TQ_ERR_UNSUPPORTED, a null or misaligned signs / rho TQ_ERR_INVALID_ARG. */
int tq_octo_encode_qjl(const void* X, int32_t dtype, int64_t n, int32_t bits,
                       const tq_rotation* rot, const tq_rotation* rot_qjl,
                       const void* dev_tables, int64_t table_bytes,
                       void* codes, void* gamma, void* signs, void* rho,
                       void* hip_stream);
int tq_octo_logits_qjl(const float* q, const void* codes, const void* gamma,
                       const void* signs, const void* rho, int32_t heads,
                       int32_t group, int64_t n, int32_t bits,
                       const tq_rotation* rot, const tq_rotation* rot_qjl,
                       const void* dev_tables, int64_t table_bytes,
                       float scale, float* out, void* hip_stream);

/* Decode-attend over triplet-coded keys and values ([P3] Method step 7:
 * scores and values straight from each triplet's norm and direction codes,
 * no reconstructed key or value written; [P2] attention
 * softmax(q K_hat^T scale) V_hat), on the flat per-head buffers of
 * tq_octo_encode (keys and values coded with the same rotation and bits):
 *   out[h][g] = sum_j softmax_j(scale * q_hg . k_hat_hj) v_hat_hj
 * q: device fp32 [heads][group][128], 16-byte aligned; k_codes / v_codes:
 * [heads][n][record bytes], 8-byte aligned; k_gamma / v_gamma: [heads][n]
 * fp16; out: fp32 [heads][group][128], 16-byte aligned (n = 0 gives zeros);
 * workspace: device, 16-byte aligned, at least
 * tq_octo_attend_workspace_bytes(heads, group, n) bytes, for the split
 * partials.  All caller-owned; asynchronous on hip_stream (a split kernel and
 * a merge).  group in 1..16, heads in 1..65535, heads * n < 2^31.  Errors as
 * tq_octo_logits, plus TQ_ERR_WORKSPACE for a short workspace. */
int64_t tq_octo_attend_workspace_bytes(int32_t heads, int32_t group, int64_t n);
int tq_octo_attend(const float* q, const void* k_codes, const void* k_gamma,
                   const void* v_codes, const void* v_gamma, int32_t heads,
                   int32_t group, int64_t n, int32_t bits,
                   const tq_rotation* rot, const void* dev_tables,
                   int64_t table_bytes, float scale, float* out,
                   void* workspace, int64_t workspace_bytes, void* hip_stream);

/* ---------------------------------------------------------------------------
 * Measurement aid (not part of the codec): read `bytes` of device memory at
 * `src` as a plain stream (grid-stride 16-byte non-temporal loads) and write
 * one folded word to `sink` (device, 4 bytes).  Timing it gives the on-box
 * read ceiling that the read-dominated decode is compared with, beside the
 * vendor's 8 TB/s.  src 16-byte aligned; bytes is rounded down to a multiple
 * of 32 KiB (less than that: nothing is read).  Asynchronous on hip_stream. */
int tq_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H_ */
