// Host side of libtq: status/error handling, seeded rotations, the float64
// Lloyd-Max codebook, cache layout, argument validation and kernel launch.
// No device memory is owned here: per-cache tables travel in kernel arguments.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "../../include/tq.h"
#include "tq_internal.h"

struct tq_rotation {
  uint64_t seed;
  int32_t d;
  std::vector<int8_t> signs;
};

struct tq_cache {
  tq_cache_config cfg;
  tq_cache_layout lay;
  void* pool;
  tq::SignMask rot;
  tq::SignMask rot_qjl;
  tq::CodecTables tab_k;
  tq::CodecTables tab_v;
  tq::F16Codebook f16_k;      // scaled fp16 forms of the codebooks (decode operands)
  tq::F16Codebook f16_v;
};

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int hip_fail(int err, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(static_cast<hipError_t>(err));
  return TQ_ERR_HIP;
}

// ---------------------------------------------------------------- signs ----
// SplitMix64 (Steele, Lea & Flood 2014; Vigna's splitmix64.c): the j-th output
// of the generator seeded with `seed`.
uint64_t splitmix64_nth(uint64_t seed, uint64_t j) {
  uint64_t z = seed + (j + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// ------------------------------------------------------------- codebook ----
// Coordinate marginal of a uniform unit vector in R^d:
// f(x) = K_d (1 - x^2)^((d-3)/2).  With x = sin(phi) the mass of [0, x] is
// K_d * J_{d-2}(phi), J_n(phi) = integral_0^phi cos^n, which obeys
// J_n = cos^{n-1} sin / n + (n-1)/n J_{n-2} (J_0 = phi, J_1 = sin phi).
double cos_power_integral(int n, double phi) {
  const double s = std::sin(phi), c = std::cos(phi);
  double j = (n % 2 == 0) ? phi : s;      // J_0 or J_1
  double cpow = (n % 2 == 0) ? c : c * c; // cos^{k-1} for the first k
  for (int k = (n % 2 == 0) ? 2 : 3; k <= n; k += 2) {
    j = cpow * s / k + (double)(k - 1) / k * j;
    cpow *= c * c;
  }
  return j;
}

struct Marginal {
  int d;
  double kd;   // normaliser
  explicit Marginal(int d_) : d(d_) {
    kd = 1.0 / (2.0 * cos_power_integral(d - 2, M_PI / 2));
  }
  // mass of [-1, x]
  double cdf(double x) const {
    if (x <= -1.0) return 0.0;
    if (x >= 1.0) return 1.0;
    return 0.5 + kd * cos_power_integral(d - 2, std::asin(x));
  }
  // integral of x f(x) over [a, b] = K_d/(d-1) [cos^{d-1}(asin a) - cos^{d-1}(asin b)]
  double first_moment(double a, double b) const {
    auto cp = [&](double x) {
      x = std::fmin(1.0, std::fmax(-1.0, x));
      return std::pow(std::sqrt(std::fmax(0.0, 1.0 - x * x)), d - 1);
    };
    return kd / (d - 1) * (cp(a) - cp(b));
  }
};

// Lloyd-Max iteration in float64: thresholds at midpoints, centroids at cell
// conditional means, centroids symmetrised every step, until no centroid
// moves by more than 1e-14 of the largest (or the step stops shrinking at the
// float64 noise floor).  The start is the quantiles at (i + 1/2) / 2^bits,
// found by bisection on the CDF; the fixed point is unique for this
// log-concave density, so the start only changes the step count.
void lloyd_max(int d, int bits, std::vector<double>& c) {
  const int n = 1 << bits;
  Marginal m(d);
  c.resize(n);
  for (int i = 0; i < n; ++i) {
    const double target = (i + 0.5) / n;
    double lo = -1.0, hi = 1.0;
    for (int k = 0; k < 80; ++k) {
      const double mid = 0.5 * (lo + hi);
      (m.cdf(mid) < target ? lo : hi) = mid;
    }
    c[i] = 0.5 * (lo + hi);
  }
  std::vector<double> nc(n), edge(n + 1), cdf(n + 1);
  double best = 1e300;
  int stale = 0;
  for (int it = 0; it < 1000000; ++it) {
    edge[0] = -1.0;
    edge[n] = 1.0;
    for (int i = 1; i < n; ++i) edge[i] = 0.5 * (c[i - 1] + c[i]);
    for (int i = 0; i <= n; ++i) cdf[i] = m.cdf(edge[i]);
    for (int i = 0; i < n; ++i)
      nc[i] = m.first_moment(edge[i], edge[i + 1]) / (cdf[i + 1] - cdf[i]);
    double moved = 0.0, cmax = 0.0;
    for (int i = 0; i < n / 2; ++i) {
      const double v = 0.5 * (nc[n - 1 - i] - nc[i]);   // symmetric pair
      moved = std::fmax(moved, std::fabs(v - c[n - 1 - i]));
      c[n - 1 - i] = v;
      c[i] = -v;
      cmax = std::fmax(cmax, v);
    }
    if (moved < 1e-14 * cmax) return;
    if (moved < best) {
      best = moved;
      stale = 0;
    } else if (++stale > 2000) {
      return;
    }
  }
}

struct Codebook {
  std::vector<float> c;
  std::vector<float> t;
};

const Codebook* codebook_cached(int d, int bits) {
  static std::mutex mu;
  static std::map<std::pair<int, int>, Codebook> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(d, bits);
  auto it = cache.find(key);
  if (it != cache.end()) return &it->second;
  std::vector<double> c;
  lloyd_max(d, bits, c);
  Codebook cb;
  const int n = 1 << bits;
  cb.c.resize(n);
  cb.t.resize(n - 1);
  for (int i = 0; i < n; ++i) cb.c[i] = (float)c[i];
  for (int i = 0; i < n - 1; ++i)
    cb.t[i] = (float)(0.5 * ((double)cb.c[i] + (double)cb.c[i + 1]));
  return &cache.emplace(key, std::move(cb)).first->second;
}

// --------------------------------------------------------- triplet codec --
// Norm of one triplet of a uniform unit vector in R^d: rho^2 ~ Beta(3/2,
// (d-3)/2), density proportional to r^2 (1 - r^2)^((d-5)/2).  With
// r = sin(phi) the mass of [0, r] is proportional to
// integral_0^phi sin^2 cos^(d-4) = J_{d-4}(phi) - J_{d-2}(phi), and the first
// moment to integral_0^phi sin^3 cos^(d-4)
//   = (1 - cos^(d-3) phi)/(d-3) - (1 - cos^(d-1) phi)/(d-1).
struct RhoMarginal {
  int d;
  double norm;
  explicit RhoMarginal(int d_) : d(d_) {
    norm = 1.0 / (cos_power_integral(d - 4, M_PI / 2) - cos_power_integral(d - 2, M_PI / 2));
  }
  double cdf(double r) const {
    if (r <= 0.0) return 0.0;
    if (r >= 1.0) return 1.0;
    const double phi = std::asin(r);
    return norm * (cos_power_integral(d - 4, phi) - cos_power_integral(d - 2, phi));
  }
  double first_moment(double a, double b) const {
    auto m = [&](double r) {
      r = std::fmin(1.0, std::fmax(0.0, r));
      const double c = std::sqrt(std::fmax(0.0, 1.0 - r * r));
      return (1.0 - std::pow(c, d - 3)) / (d - 3) - (1.0 - std::pow(c, d - 1)) / (d - 1);
    };
    return norm * (m(b) - m(a));
  }
};

// Lloyd-Max for rho on [0, 1]: the same iteration as lloyd_max without the
// symmetry (this density is log-concave too, so the fixed point is unique).
void rho_lloyd_max(int d, int bits, std::vector<double>& c) {
  const int n = 1 << bits;
  RhoMarginal m(d);
  c.resize(n);
  for (int i = 0; i < n; ++i) {
    const double target = (i + 0.5) / n;
    double lo = 0.0, hi = 1.0;
    for (int k = 0; k < 80; ++k) {
      const double mid = 0.5 * (lo + hi);
      (m.cdf(mid) < target ? lo : hi) = mid;
    }
    c[i] = 0.5 * (lo + hi);
  }
  std::vector<double> edge(n + 1), cdf(n + 1);
  double best = 1e300;
  int stale = 0;
  for (int it = 0; it < 1000000; ++it) {
    edge[0] = 0.0;
    edge[n] = 1.0;
    for (int i = 1; i < n; ++i) edge[i] = 0.5 * (c[i - 1] + c[i]);
    for (int i = 0; i <= n; ++i) cdf[i] = m.cdf(edge[i]);
    double moved = 0.0, cmax = 0.0;
    for (int i = 0; i < n; ++i) {
      const double v = m.first_moment(edge[i], edge[i + 1]) / (cdf[i + 1] - cdf[i]);
      moved = std::fmax(moved, std::fabs(v - c[i]));
      c[i] = v;
      cmax = std::fmax(cmax, v);
    }
    if (moved < 1e-14 * cmax) return;
    if (moved < best) {
      best = moved;
      stale = 0;
    } else if (++stale > 2000) {
      return;
    }
  }
}

// Inverse of the equal-area octahedral map, (xi, eta) in [-1, 1]^2 to a unit
// vector: past the diamond |xi| + |eta| = 1 the point is reflected back
// ((|xi|, |eta|) -> (1 - |eta|, 1 - |xi|)) and lands in the lower hemisphere;
// the L1 radius r gives z = 1 - r^2, the position along the diamond edge the
// azimuth phi = (pi/2) |eta| / r, and sqrt(1 - z^2) = r sqrt(2 - r^2).
void oct_unmap(double xi, double eta, double out[3]) {
  double ax = std::fabs(xi), ae = std::fabs(eta);
  const bool lower = ax + ae > 1.0;
  if (lower) {
    const double t = ax;
    ax = 1.0 - ae;
    ae = 1.0 - t;
  }
  const double r = ax + ae;
  const double z = 1.0 - r * r;
  const double phi = r > 0.0 ? (M_PI / 2) * ae / r : 0.0;
  const double s = r * std::sqrt(std::fmax(2.0 - r * r, 0.0));
  out[0] = (xi < 0 ? -1.0 : 1.0) * s * std::cos(phi);
  out[1] = (eta < 0 ? -1.0 : 1.0) * s * std::sin(phi);
  out[2] = lower ? -z : z;
}

// Tables of the triplet codec with budget b: directions of the (b+1)-bit
// uniform grid c_j = -1 + (2j + 1) / 2^(b+1) in xi and eta (entry a * nd + c
// is the direction of (c_a, c_c), x y z 0 as fp32), and the (b-1)-bit
// Lloyd-Max norm codebook with fp32 midpoint thresholds.
struct OctoTables {
  std::vector<float> dirs;   // [nd * nd][4]
  std::vector<float> crho;   // [2^(b-1)]
  std::vector<float> trho;   // [2^(b-1) - 1]
};

const OctoTables* octo_tables_cached(int d, int b) {
  static std::mutex mu;
  static std::map<std::pair<int, int>, OctoTables> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(d, b);
  auto it = cache.find(key);
  if (it != cache.end()) return &it->second;
  OctoTables t;
  const int nd = 1 << (b + 1);
  t.dirs.resize((size_t)nd * nd * 4);
  for (int a = 0; a < nd; ++a)
    for (int c = 0; c < nd; ++c) {
      double v[3];
      oct_unmap(-1.0 + (2.0 * a + 1.0) / nd, -1.0 + (2.0 * c + 1.0) / nd, v);
      float* e = &t.dirs[((size_t)a * nd + c) * 4];
      e[0] = (float)v[0];
      e[1] = (float)v[1];
      e[2] = (float)v[2];
      e[3] = 0.f;
    }
  std::vector<double> c;
  rho_lloyd_max(d, b - 1, c);
  for (double v : c) t.crho.push_back((float)v);
  for (size_t i = 0; i + 1 < t.crho.size(); ++i)
    t.trho.push_back((float)(0.5 * ((double)t.crho[i] + (double)t.crho[i + 1])));
  return &cache.emplace(key, std::move(t)).first->second;
}

// Bucket table of the encoder's threshold search (see tq::CodecTables).
int build_codec_tables(int d, int bits, tq::CodecTables& tab) {
  const Codebook* cb = codebook_cached(d, bits);
  std::memset(&tab, 0, sizeof(tab));
  tab.bits = bits;
  const int n = 1 << bits, nt = n - 1;
  for (int i = 0; i < n; ++i) tab.centroid[i] = cb->c[i];
  for (int i = 0; i < nt; ++i) tab.threshold[i] = cb->t[i];
  double gap = 1e300;
  for (int i = 0; i + 1 < nt; ++i) gap = std::fmin(gap, (double)cb->t[i + 1] - cb->t[i]);
  if (nt == 1) gap = 2.0 * std::fabs((double)cb->c[1]);
  const double w = 0.5 * gap;
  const double lo0 = (double)cb->t[0] - 2.0 * w;
  double best_margin = -1.0;
  float best_s = 0.f, best_o = 0.f;
  int best_n = 0;
  for (int ph = 0; ph < 64; ++ph) {
    const double lo = lo0 - w * ph / 64.0;
    const float S = (float)(1.0 / w);
    const float O = (float)(-lo / w);
    const double hi = (double)cb->t[nt - 1] + 2.0 * w;
    const int nb = (int)std::ceil(((double)hi * S + O)) + 1;
    if (nb > tq::kLutMax) continue;
    double margin = 1e300;
    for (int i = 0; i < nt; ++i) {
      const double u = (double)cb->t[i] * S + O;   // position in bucket units
      margin = std::fmin(margin, std::fabs(u - std::nearbyint(u)) / S);
    }
    if (margin > best_margin) {
      best_margin = margin;
      best_s = S;
      best_o = O;
      best_n = nb;
    }
  }
  if (best_margin < 1e-6) return fail(TQ_ERR_UNSUPPORTED, "no bucket grid with enough threshold margin");
  tab.lut_n = best_n;
  tab.lut_scale = best_s;
  tab.lut_offset = best_o;
  for (int k = 0; k < best_n; ++k) {
    const double e0 = ((double)k - best_o) / best_s;        // lower edge
    const double e1 = ((double)k + 1 - best_o) / best_s;    // upper edge
    int base = 0;
    float thr = std::numeric_limits<float>::infinity();
    for (int i = 0; i < nt; ++i) {
      const double t = cb->t[i];
      if (t < e0) ++base;
      else if (t < e1) thr = cb->t[i];
    }
    tab.lut_base[k] = base;
    tab.lut_thr[k] = thr;
  }
  // the clamped end buckets must not hold thresholds
  if (tab.lut_base[0] != 0 || tab.lut_thr[0] != std::numeric_limits<float>::infinity() ||
      tab.lut_thr[best_n - 1] != std::numeric_limits<float>::infinity() ||
      tab.lut_base[best_n - 1] != nt)
    return fail(TQ_ERR_UNSUPPORTED, "bucket table end check failed");
  return TQ_OK;
}

int layout_of(const tq_cache_config* cfg, tq_cache_layout* lay) {
  if (!cfg || !lay) return fail(TQ_ERR_INVALID_ARG, "null argument");
  if (cfg->layout_version != TQ_LAYOUT_VERSION)
    return fail(TQ_ERR_UNSUPPORTED, "layout_version must be 1");
  if (cfg->d != tq::kD) return fail(TQ_ERR_UNSUPPORTED, "only d = 128 is supported");
  if (cfg->block_size != tq::kBlock) return fail(TQ_ERR_UNSUPPORTED, "block_size must be 16");
  if (cfg->num_kv_heads < 1) return fail(TQ_ERR_INVALID_ARG, "num_kv_heads < 1");
  if (cfg->num_blocks < 1) return fail(TQ_ERR_INVALID_ARG, "num_blocks < 1");
  if (cfg->bits_k < 2 || cfg->bits_k > 4) return fail(TQ_ERR_UNSUPPORTED, "bits_k must be 2..4");
  if (cfg->bits_v != 0 && (cfg->bits_v < 2 || cfg->bits_v > 4))
    return fail(TQ_ERR_UNSUPPORTED, "bits_v must be 0 or 2..4");
  if (cfg->bits_v != 0 && cfg->bits_v != cfg->bits_k)
    return fail(TQ_ERR_UNSUPPORTED, "bits_v must be 0 or equal to bits_k");
  if (cfg->qjl != 0 && cfg->qjl != 1) return fail(TQ_ERR_INVALID_ARG, "qjl must be 0/1");
  const int64_t B = tq::kBlock, d = cfg->d;
  lay->k_rec_bytes = d * cfg->bits_k / 8;
  lay->v_rec_bytes = d * cfg->bits_v / 8;
  lay->off_k = 0;
  lay->off_v = B * lay->k_rec_bytes;
  lay->off_gamma_k = lay->off_v + B * lay->v_rec_bytes;
  lay->off_gamma_v = lay->off_gamma_k + 2 * B;
  lay->off_rho = lay->off_gamma_v + (cfg->bits_v > 0 ? 2 * B : 0);
  lay->off_sign = lay->off_rho + 2 * B;
  lay->block_bytes = lay->off_rho + (cfg->qjl ? 2 * B + B * d / 8 : 0);
  const int64_t per_block = lay->block_bytes * cfg->num_kv_heads;
  if (cfg->num_blocks > std::numeric_limits<int64_t>::max() / per_block)
    return fail(TQ_ERR_INVALID_ARG, "pool size overflows int64");
  lay->pool_bytes = per_block * cfg->num_blocks;
  return TQ_OK;
}

void to_mask(const std::vector<int8_t>& s, tq::SignMask& m) {
  std::memset(&m, 0, sizeof(m));
  for (int j = 0; j < tq::kD; ++j)
    if (s[j] < 0) m.neg[j / 32] |= 1u << (j % 32);
}

int check_device() {
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return fail(TQ_ERR_NO_DEVICE, "no HIP device");
  }
  return TQ_OK;
}

// Blocks per split of a decode launch.  The matrix-core kernel keeps no
// per-split score buffer, so its splits are sized for one round of two
// workgroups per CU (256 CUs); the vector kernel stages its split's scores in
// LDS and caps a split at 64 blocks.  A decode-attend launch has at most
// kMaxSplits splits per (sequence, KV head), which bounds the workspace.
// TQ_BLOCKS_PER_SPLIT overrides (tuning only).  Returns 0 when no valid split
// size exists.
int blocks_per_split_for(const tq_cache* c, int32_t num_seqs, int32_t group, int32_t max_blocks, bool mfma,
                         bool attend) {
  const int64_t units = (int64_t)num_seqs * c->cfg.num_kv_heads * tq::decode_slices(group);
  // matrix-core kernel: at most 64 block pairs per wave, the block-table
  // entries a wave keeps one per lane; 8 waves per workgroup
  const int64_t waves = 8;
  const int64_t cap = mfma ? 2 * 64 * waves : 64;
  int64_t bps;
  if (mfma) {
    // two 8-wave workgroups fit on a CU: aim for one such round of them
    // (4-bit codes: 3-4% faster than four 4-wave workgroups on 16 x 8192 and
    // 1 x 32768 tokens x 8 KV heads).  Short splits (a few pairs per wave)
    // pay the per-workgroup set-up and merge more than they gain from the
    // extra workgroups: there aim for half as many, with a whole number of
    // pairs per wave.
    const int64_t wgs = 256 * 2;
    const int64_t unit = 2 * waves;
    bps = ((int64_t)max_blocks * units + wgs - 1) / wgs;
    if (bps <= 32) bps = (((int64_t)max_blocks * units + wgs / 2 - 1) / (wgs / 2) + unit - 1) / unit * unit;
    if (bps < unit) bps = unit;
  } else {
    bps = ((int64_t)max_blocks * units + 1023) / 1024;
    if (bps < 4) bps = 4;
  }
  if (const char* env = std::getenv("TQ_BLOCKS_PER_SPLIT")) {
    const int v = std::atoi(env);
    if (v >= 1) bps = v;
  }
  if (attend) {
    const int64_t min_bps = ((int64_t)max_blocks + tq::kMaxSplits - 1) / tq::kMaxSplits;
    if (bps < min_bps) bps = min_bps;
  }
  if (mfma) bps = (bps + 1) & ~(int64_t)1;
  if (bps > cap) bps = cap;
  if (attend && ((int64_t)max_blocks + bps - 1) / bps > tq::kMaxSplits) bps = 0;
  return (int)bps;
}

// Decode-attend runs on the matrix cores, with or without the QJL sidecar.
// TQ_DECODE_VALU=1 selects the vector-unit kernel instead (comparison only).
bool decode_uses_mfma(const tq_cache*, bool attend) {
  if (const char* env = std::getenv("TQ_DECODE_VALU"))
    if (std::atoi(env) == 1) return false;
  return attend;
}

int validate_decode(const void* q, int32_t q_dtype, const tq_cache* cache,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "null cache");
  if (num_seqs < 0 || max_blocks < 0) return fail(TQ_ERR_INVALID_ARG, "negative size");
  if (num_seqs > 0 && (!q || !block_tables || !seq_lens))
    return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (q_dtype != TQ_F32 && q_dtype != TQ_F16 && q_dtype != TQ_BF16)
    return fail(TQ_ERR_INVALID_ARG, "bad q dtype");
  if (num_seqs > 0 && (reinterpret_cast<uintptr_t>(q) & 15) != 0)
    return fail(TQ_ERR_INVALID_ARG, "q must be 16-byte aligned");
  const int hkv = cache->cfg.num_kv_heads;
  if (num_q_heads < hkv || num_q_heads % hkv != 0)
    return fail(TQ_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (num_q_heads / hkv > tq::kMaxGroup)
    return fail(TQ_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
  return TQ_OK;
}

// 8-bit integer form of an odd-symmetric key codebook (the matrix-core
// logits).  With unit = 2^-s, s the largest power keeping the centroids
// within 32000 units, centroid i of the negative half is approximated by
// Y_i = V_i + 128.5 units, V_i = 256*hi_i + lo_i an integer with signed bytes
// hi_i, lo_i, and |Y_i - c_i / unit| <= 1/2.  The mirror code 2^b-1-i holds
// the bitwise NOT of both bytes, V = -V_i - 257, so its Y is exactly -Y_i.
// The kernel adds the constant 128.5 units back through the query sum.
// Returns false if the codebook is not exactly odd-symmetric.
bool make_key_i8_tables(const float* c, int bits, uint32_t hi[2], uint32_t lo[2], float* unit) {
  const int n = 1 << bits, half = n / 2;
  double cmax = 0.0;
  for (int i = 0; i < n; ++i) {
    if (c[n - 1 - i] != -c[i]) return false;
    cmax = std::max(cmax, std::fabs((double)c[i]));
  }
  if (!(cmax > 0.0)) return false;
  const int s = (int)std::floor(std::log2(32000.0 / cmax));
  hi[0] = hi[1] = lo[0] = lo[1] = 0;
  for (int i = 0; i < half; ++i) {
    const int64_t v = (int64_t)std::llround(std::ldexp((double)c[i], s) - 128.5);
    const int64_t h = (v + 128) >> 8;          // floor: lo in [-128, 127]
    const int64_t l = v - 256 * h;
    if (h < -127 || h > 127) return false;
    hi[i / 4] |= (uint32_t)(uint8_t)(int8_t)h << (8 * (i % 4));
    lo[i / 4] |= (uint32_t)(uint8_t)(int8_t)l << (8 * (i % 4));
  }
  *unit = (float)std::ldexp(1.0, -s);
  return true;
}

// IEEE half (binary16) bits of a finite double, round to nearest even,
// with subnormals; |v| past the largest half gives infinity.
uint16_t half_bits_rne(double v) {
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e;
  const double m = std::frexp(a, &e);          // a = m 2^e, m in [0.5, 1)
  int E = e + 14;                               // biased exponent of 1.f 2^(e-1)
  if (E <= 0) return sign | (uint16_t)std::nearbyint(std::ldexp(a, 24));   // subnormal (1024 = smallest normal)
  double q = std::nearbyint(std::ldexp(m, 11)); // 11 significant bits, in [1024, 2048]
  if (q == 2048.0) {
    q = 1024.0;
    ++E;
  }
  if (E >= 31) return sign | 0x7C00;
  return sign | (uint16_t)(E << 10) | (uint16_t)((int)q - 1024);
}

double half_value(uint16_t h) {
  const int E = (h >> 10) & 31, f = h & 1023;
  const double v = E == 0 ? std::ldexp((double)f, -24) : std::ldexp(1024.0 + f, E - 25);
  return (h & 0x8000) ? -v : v;
}

// fp16 form of a codebook for the matrix-core decode: h_i = half(S c_i),
// with S = s 2^k, k putting S max|c| in [1, 2) and s in [1, 2) searched
// over 4096 steps for the least max_i |h_i / S - c_i|.  Half rounding is
// relative, so a scale at which every centroid lands near a half grid
// point leaves far less than the plain half-ulp error (d = 128: at most
// 1.5e-6 for 3-bit and 1.2e-5 for 4-bit codebooks, in the units of the
// unit-vector coordinates, against 4.3e-5 / 5e-5 at S = 1).
tq::F16Codebook make_f16_codebook(const float* c, int bits) {
  tq::F16Codebook f{};
  const int n = 1 << bits;
  double cmax = 0.0;
  for (int i = 0; i < n; ++i) cmax = std::max(cmax, std::fabs((double)c[i]));
  const double base = cmax > 0.0 ? std::ldexp(1.0, -(int)std::floor(std::log2(cmax))) : 1.0;
  double best = std::numeric_limits<double>::infinity(), best_s = base;
  for (int step = 0; step < 4096; ++step) {
    const double S = base * (1.0 + step / 4096.0);
    double err = 0.0;
    for (int i = 0; i < n; ++i) err = std::max(err, std::fabs(half_value(half_bits_rne(S * c[i])) / S - c[i]));
    if (err < best) {
      best = err;
      best_s = S;
    }
  }
  for (int i = 0; i < 16; ++i) f.h[i] = i < n ? half_bits_rne(best_s * c[i]) : 0;
  f.unscale = (float)(1.0 / best_s);
  f.max_err = (float)best;
  return f;
}

void fill_decode_args(tq::DecodeArgs& a, const void* q, int32_t q_dtype, const tq_cache* c,
                      const int32_t* bt, const int32_t* sl, int32_t num_seqs,
                      int32_t num_q_heads, int32_t max_blocks, float scale) {
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.q_dtype = q_dtype;
  a.pool = static_cast<const uint8_t*>(c->pool);
  a.block_tables = bt;
  a.seq_lens = sl;
  a.lay.block_bytes = c->lay.block_bytes;
  a.lay.off_k = c->lay.off_k;
  a.lay.off_v = c->lay.off_v;
  a.lay.off_gk = c->lay.off_gamma_k;
  a.lay.off_gv = c->lay.off_gamma_v;
  a.lay.off_rho = c->lay.off_rho;
  a.lay.off_sign = c->lay.off_sign;
  a.lay.k_rec = (int32_t)c->lay.k_rec_bytes;
  a.lay.v_rec = (int32_t)c->lay.v_rec_bytes;
  a.num_blocks = c->cfg.num_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = c->cfg.num_kv_heads;
  a.group = num_q_heads / c->cfg.num_kv_heads;
  a.max_blocks = max_blocks;
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)c->cfg.d);
  a.rot = c->rot;
  a.rot_qjl = c->rot_qjl;
  for (int i = 0; i < 16; ++i) {
    a.cent_k[i] = i < (1 << c->cfg.bits_k) ? c->tab_k.centroid[i] : 0.f;
    a.cent_v[i] = (c->cfg.bits_v > 0 && i < (1 << c->cfg.bits_v)) ? c->tab_v.centroid[i] : 0.f;
  }
  if (!make_key_i8_tables(c->tab_k.centroid, c->cfg.bits_k, a.ki8_hi, a.ki8_lo, &a.ki8_unit)) a.ki8_unit = 0.f;
  a.f16_k = c->f16_k;
  a.f16_v = c->f16_v;
}

}  // namespace

extern "C" {

const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_BITS_MISMATCH: return "TQ_ERR_BITS_MISMATCH";
    case TQ_ERR_OOM: return "TQ_ERR_OOM";
    case TQ_ERR_NO_DEVICE: return "TQ_ERR_NO_DEVICE";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
    case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE";
    default: return "TQ_ERR_UNKNOWN";
  }
}

const char* tq_last_error(void) { return g_last_error.c_str(); }

int tq_layout_version(void) { return TQ_LAYOUT_VERSION; }

int tq_make_rotation(uint64_t seed, int32_t d, tq_rotation** out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "null out");
  *out = nullptr;
  if (d < 2 || d > 4096 || (d & (d - 1))) return fail(TQ_ERR_INVALID_ARG, "d must be a power of two in [2, 4096]");
  tq_rotation* r = new (std::nothrow) tq_rotation;
  if (!r) return fail(TQ_ERR_OOM, "out of host memory");
  r->seed = seed;
  r->d = d;
  try {
    r->signs.resize(d);
  } catch (...) {
    delete r;
    return fail(TQ_ERR_OOM, "out of host memory");
  }
  for (int j = 0; j < d; ++j) r->signs[j] = (splitmix64_nth(seed, j) >> 63) ? -1 : 1;
  *out = r;
  return TQ_OK;
}

int tq_rotation_signs(const tq_rotation* rot, int8_t* host_out) {
  if (!rot || !host_out) return fail(TQ_ERR_INVALID_ARG, "null argument");
  std::memcpy(host_out, rot->signs.data(), rot->d);
  return TQ_OK;
}

int32_t tq_rotation_dim(const tq_rotation* rot) { return rot ? rot->d : 0; }

void tq_rotation_destroy(tq_rotation* rot) { delete rot; }

int tq_codebook(int32_t d, int32_t bits, float* centroids, float* thresholds) {
  if (!centroids || !thresholds) return fail(TQ_ERR_INVALID_ARG, "null output");
  if (d < 4 || d > 65536) return fail(TQ_ERR_INVALID_ARG, "d out of range [4, 65536]");
  if (bits < 1 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits must be 1..4");
  const Codebook* cb = codebook_cached(d, bits);
  std::memcpy(centroids, cb->c.data(), sizeof(float) * cb->c.size());
  std::memcpy(thresholds, cb->t.data(), sizeof(float) * cb->t.size());
  return TQ_OK;
}

int64_t tq_cache_bytes(const tq_cache_config* cfg) {
  tq_cache_layout lay;
  const int s = layout_of(cfg, &lay);
  return s != TQ_OK ? s : lay.pool_bytes;
}

int tq_cache_layout_query(const tq_cache_config* cfg, tq_cache_layout* out) {
  return layout_of(cfg, out);
}

int tq_cache_create(const tq_cache_config* cfg, void* device_pool, tq_cache** out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "null out");
  *out = nullptr;
  tq_cache_layout lay;
  int s = layout_of(cfg, &lay);
  if (s != TQ_OK) return s;
  if (!device_pool) return fail(TQ_ERR_INVALID_ARG, "null device pool");
  if (reinterpret_cast<uintptr_t>(device_pool) % 16 != 0)
    return fail(TQ_ERR_INVALID_ARG, "device pool must be 16-byte aligned");
  if (!cfg->rot || cfg->rot->d != cfg->d) return fail(TQ_ERR_INVALID_ARG, "rotation missing or of wrong dimension");
  if (cfg->qjl && (!cfg->rot_qjl || cfg->rot_qjl->d != cfg->d))
    return fail(TQ_ERR_INVALID_ARG, "qjl needs rot_qjl of dimension d");
  tq_cache* c = new (std::nothrow) tq_cache;
  if (!c) return fail(TQ_ERR_OOM, "out of host memory");
  std::memset(c, 0, sizeof(*c));
  c->cfg = *cfg;
  c->cfg.rot = nullptr;       // signs are copied; the rotations may be freed
  c->cfg.rot_qjl = nullptr;
  c->lay = lay;
  c->pool = device_pool;
  to_mask(cfg->rot->signs, c->rot);
  if (cfg->qjl) to_mask(cfg->rot_qjl->signs, c->rot_qjl);
  if ((s = build_codec_tables(cfg->d, cfg->bits_k, c->tab_k)) != TQ_OK ||
      (cfg->bits_v > 0 && (s = build_codec_tables(cfg->d, cfg->bits_v, c->tab_v)) != TQ_OK)) {
    delete c;
    return s;
  }
  c->f16_k = make_f16_codebook(c->tab_k.centroid, cfg->bits_k);
  if (cfg->bits_v > 0) c->f16_v = make_f16_codebook(c->tab_v.centroid, cfg->bits_v);
  *out = c;
  return TQ_OK;
}

void tq_cache_destroy(tq_cache* cache) { delete cache; }

int tq_encode_kv(const void* K, const void* V, int32_t dtype, int64_t num_tokens,
                 const int32_t* slot_mapping, int32_t bits, tq_cache* cache, void* hip_stream) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "null cache");
  if (num_tokens < 0) return fail(TQ_ERR_INVALID_ARG, "num_tokens < 0");
  if (dtype != TQ_F32 && dtype != TQ_F16 && dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "bad dtype");
  const tq_cache_config& cfg = cache->cfg;
  if (cfg.bits_v == 0 && V) return fail(TQ_ERR_INVALID_ARG, "V given for a keys-only cache");
  if (cfg.bits_v > 0 && !V) return fail(TQ_ERR_INVALID_ARG, "V missing for a cache with values");
  if (bits != cfg.bits_k || (V && bits != cfg.bits_v))
    return fail(TQ_ERR_BITS_MISMATCH, "bits differs from the cache's bit width");
  if (num_tokens == 0) return TQ_OK;
  if (!K || !slot_mapping) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  const int64_t nvec = num_tokens * cfg.num_kv_heads;
  if (nvec / cfg.num_kv_heads != num_tokens || nvec >= ((int64_t)1 << 31))
    return fail(TQ_ERR_INVALID_ARG, "too many vectors");
  int s = check_device();
  if (s != TQ_OK) return s;
  tq::EncodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.slot_mapping = slot_mapping;
  a.pool = static_cast<uint8_t*>(cache->pool);
  a.num_vectors = nvec;
  a.num_slots = cfg.num_blocks * tq::kBlock;
  a.block_bytes = cache->lay.block_bytes;
  a.rho_off = cache->lay.off_rho;
  a.sign_off = cache->lay.off_sign;
  a.num_heads = cfg.num_kv_heads;
  a.div_heads = tq::make_fast_div((uint32_t)cfg.num_kv_heads);
  a.rot = cache->rot;
  a.rot_qjl = cache->rot_qjl;
  a.tab = cache->tab_k;
  a.stream[0] = {K, cache->lay.off_k, cache->lay.off_gamma_k, (int32_t)cache->lay.k_rec_bytes, cfg.qjl};
  a.stream[1] = {V, cache->lay.off_v, cache->lay.off_gamma_v, (int32_t)cache->lay.v_rec_bytes, 0};
  const int streams = V ? 2 : 1;
  int err = tq::launch_encode(a, streams, dtype, hip_stream);
  if (err != 0) return hip_fail(err, "encode launch");
  return TQ_OK;
}

int64_t tq_decode_workspace_bytes(const tq_cache* cache, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_blocks_per_seq) {
  if (!cache || num_seqs < 0 || max_blocks_per_seq < 0 || num_q_heads < cache->cfg.num_kv_heads ||
      num_q_heads % cache->cfg.num_kv_heads != 0)
    return fail(TQ_ERR_INVALID_ARG, "bad workspace query");
  const int group = num_q_heads / cache->cfg.num_kv_heads;
  const int bps = blocks_per_split_for(cache, num_seqs, group, max_blocks_per_seq, decode_uses_mfma(cache, true), true);
  if (bps <= 0) return fail(TQ_ERR_UNSUPPORTED, "sequence too long for this cache's decode kernel");
  const int64_t splits = std::max<int64_t>(1, (max_blocks_per_seq + bps - 1) / bps);
  const int64_t nsh = (int64_t)num_seqs * cache->cfg.num_kv_heads;
  return nsh * splits * group * tq::kPartStride * 4;
}

// Decode-attend with its partials in `workspace` (caller memory, or the
// library's fixed scratch when workspace == nullptr and no_alloc is set).
static int decode_attend_impl(const void* q, int32_t q_dtype, const tq_cache* cache,
                              const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                              int32_t num_q_heads, int32_t max_blocks_per_seq, float scale, float* out,
                              float* logits_out, void* workspace, int64_t workspace_bytes, bool no_alloc,
                              void* hip_stream) {
  int s = validate_decode(q, q_dtype, cache, block_tables, seq_lens, num_seqs, num_q_heads,
                          max_blocks_per_seq);
  if (s != TQ_OK) return s;
  if (cache->cfg.bits_v == 0) return fail(TQ_ERR_INVALID_ARG, "decode_attend needs a cache with values");
  if (num_seqs == 0) return TQ_OK;
  if (!out) return fail(TQ_ERR_INVALID_ARG, "null out");
  const int64_t need = tq_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_blocks_per_seq);
  if (need < 0) return (int)need;
  if (no_alloc) {
    if (need > tq::kScratchBytes)
      return fail(TQ_ERR_WORKSPACE, "the call needs " + std::to_string(need) +
                                        " bytes of split partials; the fixed scratch holds " +
                                        std::to_string(tq::kScratchBytes) + " (use tq_decode_attend with a workspace)");
    if ((s = check_device()) != TQ_OK) return s;
    const int e = tq::scratch_buffer(&workspace, &workspace_bytes);
    if (e != 0) return hip_fail(e, "scratch address");
  } else {
    if (!workspace || workspace_bytes < need) return fail(TQ_ERR_WORKSPACE, "workspace too small");
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return fail(TQ_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if ((s = check_device()) != TQ_OK) return s;
  }
  tq::DecodeArgs a;
  fill_decode_args(a, q, q_dtype, cache, block_tables, seq_lens, num_seqs, num_q_heads,
                   max_blocks_per_seq, scale);
  a.out = out;
  a.logits = logits_out;
  a.logits_stride = (int64_t)max_blocks_per_seq * tq::kBlock;
  a.blocks_per_split = blocks_per_split_for(cache, num_seqs, a.group, max_blocks_per_seq, decode_uses_mfma(cache, true), true);
  if (a.blocks_per_split <= 0) return fail(TQ_ERR_UNSUPPORTED, "sequence too long for this cache's decode kernel");
  a.num_splits = std::max(1, (max_blocks_per_seq + a.blocks_per_split - 1) / a.blocks_per_split);
  a.partials = static_cast<float*>(workspace);
  int err = tq::launch_decode(a, cache->cfg.bits_k, cache->cfg.bits_v, cache->cfg.qjl, 1,
                              decode_uses_mfma(cache, true) ? 1 : 0, hip_stream);
  if (err != 0) return hip_fail(err, "decode launch");
  return TQ_OK;
}

int tq_decode_attend(const void* q, int32_t q_dtype, const tq_cache* cache,
                     const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t max_blocks_per_seq, float scale, float* out,
                     float* logits_out, void* workspace, int64_t workspace_bytes, void* hip_stream) {
  return decode_attend_impl(q, q_dtype, cache, block_tables, seq_lens, num_seqs, num_q_heads, max_blocks_per_seq,
                            scale, out, logits_out, workspace, workspace_bytes, false, hip_stream);
}

int tq_decode_attend_noalloc(const void* q, int32_t q_dtype, const tq_cache* cache,
                             const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t max_blocks_per_seq, float scale, float* out,
                             float* logits_out, void* hip_stream) {
  return decode_attend_impl(q, q_dtype, cache, block_tables, seq_lens, num_seqs, num_q_heads, max_blocks_per_seq,
                            scale, out, logits_out, nullptr, 0, true, hip_stream);
}

int tq_decode_step(const void* q, int32_t q_dtype, const void* K_new, const void* V_new, int32_t kv_dtype,
                   tq_cache* cache, const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                   int32_t num_q_heads, int32_t max_blocks_per_seq, float scale, float* out, float* logits_out,
                   void* workspace, int64_t workspace_bytes, void* hip_stream) {
  int s = validate_decode(q, q_dtype, cache, block_tables, seq_lens, num_seqs, num_q_heads, max_blocks_per_seq);
  if (s != TQ_OK) return s;
  const tq_cache_config& cfg = cache->cfg;
  if (cfg.bits_v == 0) return fail(TQ_ERR_INVALID_ARG, "decode_step needs a cache with values");
  if (cfg.bits_v != cfg.bits_k) return fail(TQ_ERR_BITS_MISMATCH, "decode_step needs keys and values of one bit width");
  if (!decode_uses_mfma(cache, true) || cache->cfg.qjl)
    return fail(TQ_ERR_UNSUPPORTED, "decode_step runs on the matrix-core decode (no QJL sidecar)");
  if (kv_dtype != TQ_F32 && kv_dtype != TQ_F16 && kv_dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "bad kv_dtype");
  if (num_seqs == 0) return TQ_OK;
  if (!out || !K_new || !V_new) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if ((reinterpret_cast<uintptr_t>(K_new) | reinterpret_cast<uintptr_t>(V_new)) % 16 != 0)
    return fail(TQ_ERR_INVALID_ARG, "K_new and V_new must be 16-byte aligned");
  const int64_t need = tq_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_blocks_per_seq);
  if (!workspace || workspace_bytes < need) return fail(TQ_ERR_WORKSPACE, "workspace too small");
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return fail(TQ_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  if ((s = check_device()) != TQ_OK) return s;
  tq::DecodeArgs a;
  fill_decode_args(a, q, q_dtype, cache, block_tables, seq_lens, num_seqs, num_q_heads, max_blocks_per_seq, scale);
  a.out = out;
  a.logits = logits_out;
  a.logits_stride = (int64_t)max_blocks_per_seq * tq::kBlock;
  a.blocks_per_split = blocks_per_split_for(cache, num_seqs, a.group, max_blocks_per_seq, true, true);
  if (a.blocks_per_split <= 0) return fail(TQ_ERR_UNSUPPORTED, "sequence too long for this cache's decode kernel");
  a.num_splits = std::max(1, (max_blocks_per_seq + a.blocks_per_split - 1) / a.blocks_per_split);
  a.partials = static_cast<float*>(workspace);
  tq::AppendArgs ap;
  std::memset(&ap, 0, sizeof(ap));
  ap.k_new = K_new;
  ap.v_new = V_new;
  ap.dtype = kv_dtype;
  ap.tab = cache->tab_k;
  int err = tq::launch_decode_step(a, ap, cfg.bits_k, hip_stream);
  if (err != 0) return hip_fail(err, "decode step launch");
  return TQ_OK;
}

int tq_decode_logits(const void* q, int32_t q_dtype, const tq_cache* cache,
                     const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                     int32_t num_q_heads, int32_t max_blocks_per_seq, float scale,
                     float* logits_out, void* hip_stream) {
  int s = validate_decode(q, q_dtype, cache, block_tables, seq_lens, num_seqs, num_q_heads,
                          max_blocks_per_seq);
  if (s != TQ_OK) return s;
  if (num_seqs == 0 || max_blocks_per_seq == 0) return TQ_OK;
  if (!logits_out) return fail(TQ_ERR_INVALID_ARG, "null logits_out");
  if ((s = check_device()) != TQ_OK) return s;
  tq::DecodeArgs a;
  fill_decode_args(a, q, q_dtype, cache, block_tables, seq_lens, num_seqs, num_q_heads,
                   max_blocks_per_seq, scale);
  a.logits = logits_out;
  a.logits_stride = (int64_t)max_blocks_per_seq * tq::kBlock;
  a.blocks_per_split = blocks_per_split_for(cache, num_seqs, a.group, max_blocks_per_seq, false, false);
  a.num_splits = std::max(1, (max_blocks_per_seq + a.blocks_per_split - 1) / a.blocks_per_split);
  int err = tq::launch_decode(a, cache->cfg.bits_k, 0, cache->cfg.qjl, 0, 0, hip_stream);
  if (err != 0) return hip_fail(err, "logits launch");
  return TQ_OK;
}

int tq_decompress_kv(const tq_cache* cache, const int32_t* slots, int64_t n, int32_t out_dtype,
                     void* K_out, void* V_out, void* hip_stream) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "null cache");
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n < 0");
  if (out_dtype != TQ_BF16 && out_dtype != TQ_F16) return fail(TQ_ERR_INVALID_ARG, "out_dtype must be TQ_BF16 or TQ_F16");
  if (V_out && cache->cfg.bits_v == 0) return fail(TQ_ERR_INVALID_ARG, "V_out given for a keys-only cache");
  if ((reinterpret_cast<uintptr_t>(K_out) | reinterpret_cast<uintptr_t>(V_out)) % 16 != 0)
    return fail(TQ_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  if (n == 0 || (!K_out && !V_out)) return TQ_OK;
  if (!slots) return fail(TQ_ERR_INVALID_ARG, "null slots");
  if (n * cache->cfg.num_kv_heads >= ((int64_t)1 << 31)) return fail(TQ_ERR_INVALID_ARG, "too many vectors");
  int s = check_device();
  if (s != TQ_OK) return s;
  tq::DecompArgs a;
  std::memset(&a, 0, sizeof(a));
  a.pool = static_cast<const uint8_t*>(cache->pool);
  a.slots = slots;
  a.n_vectors = n * cache->cfg.num_kv_heads;
  a.num_slots = cache->cfg.num_blocks * tq::kBlock;
  a.block_bytes = cache->lay.block_bytes;
  a.num_heads = cache->cfg.num_kv_heads;
  a.out_dtype = out_dtype;
  a.div_heads = tq::make_fast_div((uint32_t)cache->cfg.num_kv_heads);
  a.rot = cache->rot;
  for (int k = 0; k < 2; ++k) {
    tq::DecompStream& st = a.stream[k];
    const tq::CodecTables& tab = k ? cache->tab_v : cache->tab_k;
    st.out = k ? V_out : K_out;
    st.rec_off = k ? cache->lay.off_v : cache->lay.off_k;
    st.norm_off = k ? cache->lay.off_gamma_v : cache->lay.off_gamma_k;
    st.rec_bytes = (int32_t)(k ? cache->lay.v_rec_bytes : cache->lay.k_rec_bytes);
    st.bits = k ? cache->cfg.bits_v : cache->cfg.bits_k;
    for (int i = 0; i < 16; ++i) st.centroid[i] = (st.out && i < (1 << st.bits)) ? tab.centroid[i] : 0.f;
  }
  int err = tq::launch_decompress(a, hip_stream);
  if (err != 0) return hip_fail(err, "decompress launch");
  return TQ_OK;
}

int tq_minmax_encode(const void* X, int32_t dtype, int64_t n, int32_t bits, const tq_rotation* rot, void* codes,
                     void* params, void* hip_stream) {
  if (!rot || rot->d != 128) return fail(TQ_ERR_UNSUPPORTED, "the min/max codec needs a rotation of dimension 128");
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n < 0");
  if (bits < 2 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits must be 2..4");
  if (dtype != TQ_F32 && dtype != TQ_F16 && dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "bad dtype");
  if (n == 0) return TQ_OK;
  if (!X || !codes || !params) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (reinterpret_cast<uintptr_t>(X) % 16 != 0 || reinterpret_cast<uintptr_t>(codes) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(params) % 4 != 0)
    return fail(TQ_ERR_INVALID_ARG, "X must be 16-byte aligned, codes and params 4-byte aligned");
  if (n >= ((int64_t)1 << 31)) return fail(TQ_ERR_INVALID_ARG, "too many vectors");
  int s = check_device();
  if (s != TQ_OK) return s;
  tq::MinmaxArgs a;
  std::memset(&a, 0, sizeof(a));
  a.src = X;
  a.codes = static_cast<uint8_t*>(codes);
  a.params = static_cast<uint16_t*>(params);
  a.n = n;
  a.in_dtype = dtype;
  to_mask(rot->signs, a.rot);
  int err = tq::launch_minmax_encode(a, bits, hip_stream);
  if (err != 0) return hip_fail(err, "min/max encode launch");
  return TQ_OK;
}

int tq_minmax_decode(const void* codes, const void* params, int64_t n, int32_t bits, const tq_rotation* rot,
                     int32_t out_dtype, void* out, void* hip_stream) {
  if (!rot || rot->d != 128) return fail(TQ_ERR_UNSUPPORTED, "the min/max codec needs a rotation of dimension 128");
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n < 0");
  if (bits < 2 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits must be 2..4");
  if (out_dtype != TQ_F32 && out_dtype != TQ_F16 && out_dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "bad out_dtype");
  if (n == 0) return TQ_OK;
  if (!codes || !params || !out) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (reinterpret_cast<uintptr_t>(out) % 16 != 0 || reinterpret_cast<uintptr_t>(codes) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(params) % 4 != 0)
    return fail(TQ_ERR_INVALID_ARG, "out must be 16-byte aligned, codes and params 4-byte aligned");
  if (n >= ((int64_t)1 << 31)) return fail(TQ_ERR_INVALID_ARG, "too many vectors");
  int s = check_device();
  if (s != TQ_OK) return s;
  tq::MinmaxArgs a;
  std::memset(&a, 0, sizeof(a));
  a.codes = const_cast<uint8_t*>(static_cast<const uint8_t*>(codes));
  a.params = const_cast<uint16_t*>(static_cast<const uint16_t*>(params));
  a.out = out;
  a.n = n;
  a.out_dtype = out_dtype;
  to_mask(rot->signs, a.rot);
  int err = tq::launch_minmax_decode(a, bits, hip_stream);
  if (err != 0) return hip_fail(err, "min/max decode launch");
  return TQ_OK;
}

int tq_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* hip_stream) {
  if (bytes < 0) return fail(TQ_ERR_INVALID_ARG, "bytes < 0");
  if (bytes < 16 * 256 * 8) return TQ_OK;   // less than one thread-group's pass: nothing to time
  if (!src || !sink) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return fail(TQ_ERR_INVALID_ARG, "src must be 16-byte aligned");
  int s = check_device();
  if (s != TQ_OK) return s;
  int err = tq::launch_stream_read(src, bytes, sink, hip_stream);
  if (err != 0) return hip_fail(err, "stream read launch");
  return TQ_OK;
}

int64_t tq_octo_record_bytes(int32_t d, int32_t bits) {
  if (d != tq::kD) return fail(TQ_ERR_UNSUPPORTED, "the triplet codec supports d = 128");
  if (bits < 2 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits must be 2..4");
  const int64_t field = 2 * (bits + 1) + (bits - 1);
  return 4 * ((tq::kOctoTri * field + 31) / 32);
}

int64_t tq_octo_table_bytes(int32_t bits) {
  if (bits < 2 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits must be 2..4");
  return (int64_t)16 << (2 * (bits + 1));
}

int tq_octo_codebook(int32_t d, int32_t bits, float* dirs, float* rho_centroids) {
  if (d != tq::kD) return fail(TQ_ERR_UNSUPPORTED, "the triplet codec supports d = 128");
  if (bits < 2 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits must be 2..4");
  const OctoTables* t = octo_tables_cached(d, bits);
  if (dirs) std::memcpy(dirs, t->dirs.data(), sizeof(float) * t->dirs.size());
  if (rho_centroids) std::memcpy(rho_centroids, t->crho.data(), sizeof(float) * t->crho.size());
  return TQ_OK;
}

int tq_octo_tables(int32_t bits, void* dev_tables, void* hip_stream) {
  if (bits < 2 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits must be 2..4");
  if (!dev_tables) return fail(TQ_ERR_INVALID_ARG, "null table buffer");
  if (reinterpret_cast<uintptr_t>(dev_tables) % 16 != 0) return fail(TQ_ERR_INVALID_ARG, "table buffer must be 16-byte aligned");
  int s = check_device();
  if (s != TQ_OK) return s;
  const OctoTables* t = octo_tables_cached(tq::kD, bits);   // cached for the process: a valid copy source
  hipError_t e = hipMemcpyAsync(dev_tables, t->dirs.data(), sizeof(float) * t->dirs.size(), hipMemcpyHostToDevice,
                                static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail((int)e, "table copy");
  return TQ_OK;
}

namespace {
int octo_args(int32_t bits, const tq_rotation* rot, const void* dev_tables, int64_t table_bytes, tq::OctoArgs& a) {
  if (!rot || rot->d != tq::kD) return fail(TQ_ERR_UNSUPPORTED, "the triplet codec needs a rotation of dimension 128");
  if (bits < 2 || bits > 4) return fail(TQ_ERR_UNSUPPORTED, "bits must be 2..4");
  if (!dev_tables || reinterpret_cast<uintptr_t>(dev_tables) % 16 != 0)
    return fail(TQ_ERR_INVALID_ARG, "tables must be a 16-byte aligned device buffer filled by tq_octo_tables");
  if (table_bytes < ((int64_t)16 << (2 * (bits + 1))))
    return fail(TQ_ERR_INVALID_ARG, "table buffer smaller than tq_octo_table_bytes(bits)");
  std::memset(&a, 0, sizeof(a));
  const OctoTables* t = octo_tables_cached(tq::kD, bits);
  a.dirs = static_cast<const float*>(dev_tables);
  for (int i = 0; i < 8; ++i) {
    a.crho[i] = i < (int)t->crho.size() ? t->crho[i] : 0.f;
    a.trho[i] = i < (int)t->trho.size() ? t->trho[i] : std::numeric_limits<float>::infinity();
  }
  to_mask(rot->signs, a.rot);
  return TQ_OK;
}
}  // namespace

namespace {
// The sketch buffers of OCTOPUS-QJL (all null for the plain codec): the
// second rotation, 16-byte aligned sign records, 2-byte aligned norms.
int octo_qjl_args(const tq_rotation* rot_qjl, const void* signs, const void* rho, bool want, tq::OctoArgs& a) {
  if (!want) return TQ_OK;
  if (!rot_qjl || rot_qjl->d != tq::kD) return fail(TQ_ERR_UNSUPPORTED, "the residual sketch needs a rotation of dimension 128");
  if (!signs || !rho) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (reinterpret_cast<uintptr_t>(signs) % 16 != 0 || reinterpret_cast<uintptr_t>(rho) % 2 != 0)
    return fail(TQ_ERR_INVALID_ARG, "signs must be 16-byte aligned, rho 2-byte");
  a.qjl_signs = const_cast<uint8_t*>(static_cast<const uint8_t*>(signs));
  a.qjl_rho = const_cast<uint16_t*>(static_cast<const uint16_t*>(rho));
  to_mask(rot_qjl->signs, a.rot_qjl);
  return TQ_OK;
}

int octo_encode_impl(const void* X, int32_t dtype, int64_t n, int32_t bits, const tq_rotation* rot,
                     const tq_rotation* rot_qjl, const void* dev_tables, int64_t table_bytes, void* codes, void* gamma,
                     void* signs, void* rho, bool qjl, void* hip_stream) {
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n < 0");
  if (dtype != TQ_F32 && dtype != TQ_F16 && dtype != TQ_BF16) return fail(TQ_ERR_INVALID_ARG, "bad dtype");
  tq::OctoArgs a;
  int s = octo_args(bits, rot, dev_tables, table_bytes, a);
  if (s != TQ_OK) return s;
  if (qjl && (!rot_qjl || rot_qjl->d != tq::kD))
    return fail(TQ_ERR_UNSUPPORTED, "the residual sketch needs a rotation of dimension 128");
  if (n == 0) return TQ_OK;
  if (!X || !codes || !gamma) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (reinterpret_cast<uintptr_t>(X) % 16 != 0 || reinterpret_cast<uintptr_t>(codes) % 8 != 0 ||
      reinterpret_cast<uintptr_t>(gamma) % 2 != 0)
    return fail(TQ_ERR_INVALID_ARG, "X must be 16-byte aligned, codes 8-byte, gamma 2-byte");
  if ((s = octo_qjl_args(rot_qjl, signs, rho, qjl, a)) != TQ_OK) return s;
  if (n >= ((int64_t)1 << 31)) return fail(TQ_ERR_INVALID_ARG, "too many vectors");
  if ((s = check_device()) != TQ_OK) return s;
  a.src = X;
  a.codes = static_cast<uint8_t*>(codes);
  a.gamma = static_cast<uint16_t*>(gamma);
  a.n = n;
  a.dtype = dtype;
  a.heads = 1;
  int err = tq::launch_octo_encode(a, bits, hip_stream);
  if (err != 0) return hip_fail(err, "triplet encode launch");
  return TQ_OK;
}

int octo_logits_impl(const float* q, const void* codes, const void* gamma, const void* signs, const void* rho,
                     int32_t heads, int32_t group, int64_t n, int32_t bits, const tq_rotation* rot,
                     const tq_rotation* rot_qjl, const void* dev_tables, int64_t table_bytes, float scale, float* out,
                     bool qjl, void* hip_stream) {
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n < 0");
  if (heads < 1 || heads > 65535) return fail(TQ_ERR_INVALID_ARG, "heads must be 1..65535");
  if (group < 1 || group > tq::kOctoMaxGroup) return fail(TQ_ERR_UNSUPPORTED, "group must be 1..16");
  if (!std::isfinite(scale)) return fail(TQ_ERR_INVALID_ARG, "scale must be finite");
  tq::OctoArgs a;
  int s = octo_args(bits, rot, dev_tables, table_bytes, a);
  if (s != TQ_OK) return s;
  if (qjl && (!rot_qjl || rot_qjl->d != tq::kD))
    return fail(TQ_ERR_UNSUPPORTED, "the residual sketch needs a rotation of dimension 128");
  if (n == 0) return TQ_OK;
  if (!q || !codes || !gamma || !out) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(codes) % 8 != 0 ||
      reinterpret_cast<uintptr_t>(gamma) % 2 != 0 || reinterpret_cast<uintptr_t>(out) % 4 != 0)
    return fail(TQ_ERR_INVALID_ARG, "q must be 16-byte aligned, codes 8-byte, gamma 2-byte, out 4-byte");
  if ((s = octo_qjl_args(rot_qjl, signs, rho, qjl, a)) != TQ_OK) return s;
  if (n * heads >= ((int64_t)1 << 31)) return fail(TQ_ERR_INVALID_ARG, "too many keys");
  if ((s = check_device()) != TQ_OK) return s;
  a.q = q;
  a.codes = const_cast<uint8_t*>(static_cast<const uint8_t*>(codes));
  a.gamma = const_cast<uint16_t*>(static_cast<const uint16_t*>(gamma));
  a.out = out;
  a.n = n;
  a.heads = heads;
  a.group = group;
  a.scale = scale;
  int err = tq::launch_octo_logits(a, bits, hip_stream);
  if (err != 0) return hip_fail(err, "triplet logits launch");
  return TQ_OK;
}
}  // namespace

int tq_octo_encode(const void* X, int32_t dtype, int64_t n, int32_t bits, const tq_rotation* rot,
                   const void* dev_tables, int64_t table_bytes, void* codes, void* gamma, void* hip_stream) {
  return octo_encode_impl(X, dtype, n, bits, rot, nullptr, dev_tables, table_bytes, codes, gamma, nullptr, nullptr,
                          false, hip_stream);
}

int tq_octo_encode_qjl(const void* X, int32_t dtype, int64_t n, int32_t bits, const tq_rotation* rot,
                       const tq_rotation* rot_qjl, const void* dev_tables, int64_t table_bytes, void* codes,
                       void* gamma, void* signs, void* rho, void* hip_stream) {
  return octo_encode_impl(X, dtype, n, bits, rot, rot_qjl, dev_tables, table_bytes, codes, gamma, signs, rho, true,
                          hip_stream);
}

int tq_octo_logits(const float* q, const void* codes, const void* gamma, int32_t heads, int32_t group, int64_t n,
                   int32_t bits, const tq_rotation* rot, const void* dev_tables, int64_t table_bytes, float scale,
                   float* out, void* hip_stream) {
  return octo_logits_impl(q, codes, gamma, nullptr, nullptr, heads, group, n, bits, rot, nullptr, dev_tables,
                          table_bytes, scale, out, false, hip_stream);
}

int tq_octo_logits_qjl(const float* q, const void* codes, const void* gamma, const void* signs, const void* rho,
                       int32_t heads, int32_t group, int64_t n, int32_t bits, const tq_rotation* rot,
                       const tq_rotation* rot_qjl, const void* dev_tables, int64_t table_bytes, float scale,
                       float* out, void* hip_stream) {
  return octo_logits_impl(q, codes, gamma, signs, rho, heads, group, n, bits, rot, rot_qjl, dev_tables, table_bytes,
                          scale, out, true, hip_stream);
}

namespace {
// Splits of a triplet decode-attend: about two workgroups per CU in all
// (the kernel's registers allow two waves per SIMD; 768 splits, one and a
// half rounds, measured 20-30% slower), each split a multiple of the 128
// keys a workgroup stages at a time; at most 1024.
void octo_attend_split(int32_t heads, int64_t n, int64_t& split_len, int32_t& nsplit) {
  const int64_t ch = tq::kOctoAttChunk;
  const int64_t want = std::max<int64_t>(1, (n * heads + 511) / 512);
  split_len = std::max<int64_t>(ch, (want + ch - 1) / ch * ch);
  if ((n + split_len - 1) / split_len > 1024) split_len = ((n + 1023) / 1024 + ch - 1) / ch * ch;
  nsplit = (int32_t)std::max<int64_t>(1, (n + split_len - 1) / split_len);
}
}  // namespace

int64_t tq_octo_attend_workspace_bytes(int32_t heads, int32_t group, int64_t n) {
  if (heads < 1 || heads > 65535 || group < 1 || group > tq::kOctoMaxGroup || n < 0)
    return fail(TQ_ERR_INVALID_ARG, "heads 1..65535, group 1..16, n >= 0");
  int64_t split_len;
  int32_t nsplit;
  octo_attend_split(heads, n, split_len, nsplit);
  return (int64_t)heads * nsplit * group * tq::kPartStride * (int64_t)sizeof(float);
}

int tq_octo_attend(const float* q, const void* k_codes, const void* k_gamma, const void* v_codes,
                   const void* v_gamma, int32_t heads, int32_t group, int64_t n, int32_t bits,
                   const tq_rotation* rot, const void* dev_tables, int64_t table_bytes, float scale, float* out,
                   void* workspace, int64_t workspace_bytes, void* hip_stream) {
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n < 0");
  if (heads < 1 || heads > 65535) return fail(TQ_ERR_INVALID_ARG, "heads must be 1..65535");
  if (group < 1 || group > tq::kOctoMaxGroup) return fail(TQ_ERR_UNSUPPORTED, "group must be 1..16");
  if (!std::isfinite(scale)) return fail(TQ_ERR_INVALID_ARG, "scale must be finite");
  tq::OctoArgs a;
  int s = octo_args(bits, rot, dev_tables, table_bytes, a);
  if (s != TQ_OK) return s;
  if (!q || !out || !workspace || (n > 0 && (!k_codes || !k_gamma || !v_codes || !v_gamma)))
    return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(k_codes) % 8 != 0 ||
      reinterpret_cast<uintptr_t>(v_codes) % 8 != 0 || reinterpret_cast<uintptr_t>(k_gamma) % 2 != 0 ||
      reinterpret_cast<uintptr_t>(v_gamma) % 2 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(TQ_ERR_INVALID_ARG, "q, out and workspace must be 16-byte aligned, codes 8-byte, norms 2-byte");
  if (n * heads >= ((int64_t)1 << 31)) return fail(TQ_ERR_INVALID_ARG, "too many keys");
  const int64_t need = tq_octo_attend_workspace_bytes(heads, group, n);
  if (workspace_bytes < need) return fail(TQ_ERR_WORKSPACE, "workspace smaller than tq_octo_attend_workspace_bytes");
  if ((s = check_device()) != TQ_OK) return s;
  a.q = q;
  a.codes = const_cast<uint8_t*>(static_cast<const uint8_t*>(k_codes));
  a.gamma = const_cast<uint16_t*>(static_cast<const uint16_t*>(k_gamma));
  a.vcodes = static_cast<const uint8_t*>(v_codes);
  a.vgamma = static_cast<const uint16_t*>(v_gamma);
  a.partials = static_cast<float*>(workspace);
  a.n = n;
  a.heads = heads;
  a.group = group;
  a.scale = scale;
  octo_attend_split(heads, n, a.split_len, a.num_splits);
  int err = tq::launch_octo_attend(a, bits, hip_stream);
  if (err != 0) return hip_fail(err, "triplet attend launch");
  // the main decode's merge: num_kv_heads = heads, one partial per split
  tq::DecodeArgs m;
  std::memset(&m, 0, sizeof(m));
  m.out = out;
  m.partials = a.partials;
  m.num_seqs = 1;
  m.num_kv_heads = heads;
  m.num_q_heads = heads * group;
  m.group = group;
  m.num_splits = a.num_splits;
  m.rot = a.rot;
  err = tq::launch_merge(m, hip_stream);
  if (err != 0) return hip_fail(err, "merge launch");
  return TQ_OK;
}

int tq_reconstruct(const tq_cache* cache, const int32_t* slots, int64_t n, int32_t which,
                   float* out, void* hip_stream) {
  if (!cache) return fail(TQ_ERR_INVALID_ARG, "null cache");
  if (n < 0) return fail(TQ_ERR_INVALID_ARG, "n < 0");
  if (which != 0 && which != 1) return fail(TQ_ERR_INVALID_ARG, "which must be 0 (K) or 1 (V)");
  if (which == 1 && cache->cfg.bits_v == 0) return fail(TQ_ERR_INVALID_ARG, "cache has no values");
  if (n == 0) return TQ_OK;
  if (!slots || !out) return fail(TQ_ERR_INVALID_ARG, "null pointer");
  if (n * cache->cfg.num_kv_heads >= ((int64_t)1 << 31)) return fail(TQ_ERR_INVALID_ARG, "too many vectors");
  int s = check_device();
  if (s != TQ_OK) return s;
  tq::ReconArgs a;
  std::memset(&a, 0, sizeof(a));
  a.pool = static_cast<const uint8_t*>(cache->pool);
  a.slots = slots;
  a.out = out;
  a.n_vectors = n * cache->cfg.num_kv_heads;
  a.num_slots = cache->cfg.num_blocks * tq::kBlock;
  a.block_bytes = cache->lay.block_bytes;
  a.num_heads = cache->cfg.num_kv_heads;
  a.div_heads = tq::make_fast_div((uint32_t)cache->cfg.num_kv_heads);
  a.rot = cache->rot;
  const tq::CodecTables& tab = which ? cache->tab_v : cache->tab_k;
  a.bits = tab.bits;
  for (int i = 0; i < 16; ++i) a.centroid[i] = tab.centroid[i];
  a.rec_off = which ? cache->lay.off_v : cache->lay.off_k;
  a.norm_off = which ? cache->lay.off_gamma_v : cache->lay.off_gamma_k;
  a.rec_bytes = (int32_t)(which ? cache->lay.v_rec_bytes : cache->lay.k_rec_bytes);
  int err = tq::launch_reconstruct(a, hip_stream);
  if (err != 0) return hip_fail(err, "reconstruct launch");
  return TQ_OK;
}

}  // extern "C"
