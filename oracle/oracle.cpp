/*
 * CPU ORACLE for the batch-invariant MoE layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This code is the checker that the GPU library is
 * compared against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product path (the HIP library and its
 * Python binding) never does, and shares no code, header, table or constant
 * generator with it.
 *
 * Plain C++17, OpenMP only over independent tokens / rows (every output value
 * is computed by one thread in one fixed order), built with -O2
 * -ffp-contract=off, no fast-math, IEEE round-to-nearest-even, no FTZ/DAZ.
 * Floating point is carried in double between the rounding points that the
 * method fixes (expert hidden h, expert output o, shared output s, layer output
 * y); the routing arithmetic is fp32 in a pinned order because the method
 * requires bit-exact routing.
 *
 * Sources (web pages; cited by title and section):
 *  [FW]  "MoE 模型中的訓練與推論一致性：數值漂移發生之處" (Fireworks AI post on
 *        train/inference numerical parity in MoE models, easyvibecoding.app/curated/746)
 *  [MT]  "美团把训练和推理的概率做到逐位相同:分歧藏在一个加法顺序里"
 *        (LongCat bitwise train/inference parity, bbs.huaweicloud.com/blogs/524918)
 *  [DS]  "6 基建与训练稳定性优化" (DeepSeek-V4 infrastructure walkthrough,
 *        liyongzhi.xyz deepseek_v4 sections/06-infra), sections 6.1, 6.2, 6.3, 6.5
 *  [LD]  MoE FLOPs / shared experts / SiTU-GLU forum article (feedbbs.com/linuxdo/72580),
 *        sections "MoE FLOPs/参数量", "共享专家", "SiTU-GLU", "MoE是如何影响输出确定性的"
 *  [V4]  open "V4" MoE model article (nxmr.cn/news/146660), section 2.2 (routing)
 *
 * Readings where the pages leave a step open (each one is a definition of this
 * library, pinned by tests rather than by the pages):
 *  - router logit: 64 fp32 partial sums, element d goes to partial (d/8) mod 64
 *    in increasing d with fmaf, then a pairwise halving tree j += j+m for
 *    m = 32..1 (the xor-butterfly shape of [FW] trap 2, fixed for every batch).
 *  - exp for routing: Cody–Waite reduction + degree-7 Taylor/Horner in fp32
 *    (orc_exp below); sigmoid s = 1/(1+exp(-l)) with IEEE division.
 *  - softmax routing selects on logits and normalises exp over the selected k;
 *    sigmoid routing selects on s + bias and normalises the unbiased s; ties
 *    in the key go to the lower expert id; sums for the normaliser run in
 *    ascending expert id.
 *  - hash routing: slot j takes fmix32(tid + j*0x9E3779B9) mod E, probing
 *    forward past experts already taken; weight 1/k.
 *  - rounding points: h, o, s rounded to the activation type (bf16 RNE or
 *    fp32), combine in fp32 in ascending expert id with fmaf, shared added
 *    last, one final rounding.
 *  - gated-activation variants (glu_value below) replace SiLU(g) * u in every
 *    SwiGLU of the layer, routed experts and the shared expert alike.
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

enum { ACT_F32 = 0, ACT_BF16 = 1, W_MXFP4 = 2 };
enum { ROUTE_SOFTMAX = 0, ROUTE_SIGMOID = 1, ROUTE_HASH = 2 };

inline float f_from_bits(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint32_t bits_of(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}
inline float bf16_value(uint16_t b) { return f_from_bits((uint32_t)b << 16); }

/* double -> bf16 bits, one rounding (round to nearest, ties to even). */
uint16_t bf16_round(double d) {
  if (std::isnan(d)) return 0x7fc0;
  if (std::isinf(d)) return d > 0 ? 0x7f80 : 0xff80;
  if (d == 0.0) return std::signbit(d) ? 0x8000 : 0x0000;
  int e = std::ilogb(d);                   // floor(log2 |d|)
  int qe = std::max(e, -126) - 7;          // bf16 quantum at this binade
  double q = std::ldexp(1.0, qe);
  double r = std::nearbyint(d / q) * q;    // exact scaling, RNE to an integer
  if (std::fabs(r) >= std::ldexp(1.0, 128)) return d > 0 ? 0x7f80 : 0xff80;
  return (uint16_t)(bits_of((float)r) >> 16);  // r has <= 8 significant bits
}

/* One value of activation storage type `act` (fp32 or bf16 bits) as double. */
inline double act_at(const void* p, int act, int64_t i) {
  if (act == ACT_F32) return (double)static_cast<const float*>(p)[i];
  return (double)bf16_value(static_cast<const uint16_t*>(p)[i]);
}
inline float act_at_f(const void* p, int act, int64_t i) {
  if (act == ACT_F32) return static_cast<const float*>(p)[i];
  return bf16_value(static_cast<const uint16_t*>(p)[i]);
}
inline void act_store(void* p, int act, int64_t i, double v) {
  if (act == ACT_F32)
    static_cast<float*>(p)[i] = (float)v;  // C cast: IEEE round to nearest even
  else
    static_cast<uint16_t*>(p)[i] = bf16_round(v);
}

/* E2M1 code (4 bits) times the E8M0 scale 2^(s-127), exactly, from the
 * format's bit fields: sign | 2 exponent bits (bias 1) | 1 mantissa bit,
 * exponent field 0 = subnormal 0.m. */
double mxfp4_value(uint8_t code, uint8_t scale) {
  if (scale == 0xff) return std::nan("");
  int sign = (code >> 3) & 1, ef = (code >> 1) & 3, m = code & 1;
  double mag = (ef == 0) ? 0.5 * m : (1.0 + 0.5 * m) * std::ldexp(1.0, ef - 1);
  double v = std::ldexp(mag, (int)scale - 127);
  return sign ? -v : v;
}

/* Weight matrix [rows, cols] of one expert as double, rows-major. */
std::vector<double> weight_matrix(const void* w, const uint8_t* scale, int wdtype,
                                  int64_t rows, int64_t cols) {
  std::vector<double> out((size_t)(rows * cols));
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      double v;
      if (wdtype == ACT_F32) {
        v = static_cast<const float*>(w)[r * cols + c];
      } else if (wdtype == ACT_BF16) {
        v = bf16_value(static_cast<const uint16_t*>(w)[r * cols + c]);
      } else {
        uint8_t byte = static_cast<const uint8_t*>(w)[r * (cols / 2) + c / 2];
        uint8_t code = (c & 1) ? (byte >> 4) : (byte & 0xf);
        v = mxfp4_value(code, scale[r * (cols / 32) + c / 32]);
      }
      out[(size_t)(r * cols + c)] = v;
    }
  return out;
}

/* ---- routing exp: Cody–Waite + degree-7 Taylor, all fp32 ---------------- */
const float kLog2e = 0x1.715476p+0f;     // fp32(log2 e)
const float kLn2Hi = 0x1.62e430p-1f;     // fp32(ln 2)
const float kLn2Lo = -0x1.05c610p-29f;   // fp32(ln 2 - kLn2Hi)
const float kInvFact[8] = {0x1p+0f,         0x1p+0f,         0x1p-1f,
                           0x1.555556p-3f,  0x1.555556p-5f,  0x1.111112p-7f,
                           0x1.6c16c2p-10f, 0x1.a01a02p-13f};  // fp32(1/j!)

inline float pow2f(int m) { return f_from_bits((uint32_t)(m + 127) << 23); }  // -126..127

float routing_exp(float x) {
  if (x != x) return x;
  if (x > 89.0f) return INFINITY;
  if (x < -104.0f) return 0.0f;
  float n = std::rint(x * kLog2e);  // ties to even (default rounding mode)
  float r = std::fma(-n, kLn2Hi, x);
  r = std::fma(-n, kLn2Lo, r);
  float p = kInvFact[7];
  for (int j = 6; j >= 0; --j) p = std::fma(p, r, kInvFact[j]);
  int ni = (int)n;
  if (ni > 127) return (p * pow2f(ni - 64)) * pow2f(64);
  if (ni < -126) return (p * pow2f(ni + 64)) * pow2f(-64);
  return p * pow2f(ni);
}

inline float routing_sigmoid(float l) { return 1.0f / (1.0f + routing_exp(-l)); }

/* Router logit of one (token, expert) pair in the pinned order. */
float router_logit(const void* x, const void* w, int act, int64_t xoff, int64_t woff,
                   int D) {
  float p[64];
  for (int j = 0; j < 64; ++j) p[j] = 0.0f;
  for (int d = 0; d < D; ++d) {
    int j = (d / 8) % 64;
    p[j] = std::fma(act_at_f(x, act, xoff + d), act_at_f(w, act, woff + d), p[j]);
  }
  for (int m = 32; m >= 1; m /= 2)
    for (int j = 0; j < m; ++j) p[j] = p[j] + p[j + m];
  return p[0];
}

uint32_t fmix32(uint32_t h) {  // MurmurHash3 finaliser (A. Appleby, public domain)
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

struct Sel {
  float key;
  int id;
};
inline bool sel_before(const Sel& a, const Sel& b) {
  return a.key > b.key || (a.key == b.key && a.id < b.id);
}

/* Route one token from its logits (or token id). Writes k ids in rank order
 * and their weights; keys_out (optional) receives all E selection keys. */
void route_token(const float* logits, const float* bias, int32_t tid, int E, int k,
                 int mode, int32_t* idx, float* wout, float* keys_out) {
  if (mode == ROUTE_HASH) {
    std::vector<char> taken((size_t)E, 0);
    for (int j = 0; j < k; ++j) {
      uint32_t c = fmix32((uint32_t)tid + (uint32_t)j * 0x9E3779B9u) % (uint32_t)E;
      while (taken[c]) c = (c + 1) % (uint32_t)E;
      taken[c] = 1;
      idx[j] = (int32_t)c;
      wout[j] = 1.0f / (float)k;
    }
    return;
  }
  std::vector<float> score((size_t)E);
  std::vector<Sel> all((size_t)E);
  for (int e = 0; e < E; ++e) {
    score[e] = (mode == ROUTE_SIGMOID) ? routing_sigmoid(logits[e]) : logits[e];
    float key = bias ? score[e] + bias[e] : score[e];
    all[e] = Sel{key, e};
    if (keys_out) keys_out[e] = key;
  }
  std::sort(all.begin(), all.end(), sel_before);
  std::vector<int> asc((size_t)k);
  for (int j = 0; j < k; ++j) {
    idx[j] = all[j].id;
    asc[j] = all[j].id;
  }
  std::sort(asc.begin(), asc.end());
  if (mode == ROUTE_SOFTMAX) {
    /* shift by the largest selected logit: softmax is shift-invariant, and
     * with a bias the top-ranked expert need not hold the largest logit */
    float m = logits[idx[0]];
    for (int j = 1; j < k; ++j) m = std::max(m, logits[idx[j]]);
    float Z = 0.0f;
    for (int j = 0; j < k; ++j) Z = Z + routing_exp(logits[asc[j]] - m);
    for (int j = 0; j < k; ++j) wout[j] = routing_exp(logits[idx[j]] - m) / Z;
  } else {
    float Z = 0.0f;
    for (int j = 0; j < k; ++j) Z = Z + score[asc[j]];
    for (int j = 0; j < k; ++j) wout[j] = score[idx[j]] / Z;
  }
}

/* ---- MXFP8 activations for FP4 x FP8 expert GEMMs ----------------------- */
/* [DS] 6.2: FP4 (E2M1) expert weights feed an FP8 GEMM (FP4 -> FP8 is exact,
 * FP4 x FP8 matmul on newer hardware).  The page does not say how the
 * activations become FP8; this library's reading is OCP MX: E4M3 elements
 * with one E8M0 scale per 32 consecutive values along K.
 * E4M3 here is OCP FP8 E4M3 ("FN"): sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, exponent field 0 subnormal (m/8 * 2^-6), no infinities,
 * 0x7F / 0xFF NaN, largest finite 448. */
double e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return std::nan("");
  const double v = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* The E4M3 code nearest to v, ties to the even code (mantissa LSB 0);
 * magnitudes above 448 saturate to 448 (the MX conversion clamps to the
 * largest normal); NaN gives 0x7F.  The sign bit is v's, zero included.
 * Found by searching the finite non-negative codes, which increase with
 * their value. */
uint8_t e4m3_round(double v) {
  if (std::isnan(v)) return 0x7f;
  double a = std::fabs(v);
  if (a > 448.0) a = 448.0;
  int best = 0;
  double bd = a;
  for (int c = 1; c <= 0x7e; ++c) {
    const double d = std::fabs(a - e4m3_value((uint8_t)c));
    if (d < bd || (d == bd && (c & 1) == 0)) {
      best = c;
      bd = d;
    }
  }
  return (uint8_t)(best | (std::signbit(v) ? 0x80 : 0));
}

/* One block of 32 (OCP MX): X = floor(log2(amax)) - 8, 8 being the exponent
 * of E4M3's largest power of two, as the E8M0 byte X + 127 clamped to
 * [0, 254]; codes = e4m3_round(x / 2^X).  amax = 0 (no finite nonzero
 * value) gives the byte 0. */
void mx_e4m3_block(const double* x, uint8_t* codes, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i)
    if (std::isfinite(x[i]) && std::fabs(x[i]) > amax) amax = std::fabs(x[i]);
  int byte = 0;
  if (amax > 0.0) {
    int e;
    std::frexp(amax, &e);  // amax = f * 2^e, f in [0.5, 1): floor(log2(amax)) = e - 1
    byte = std::min(254, std::max(0, (e - 1) - 8 + 127));
  }
  *scale = (uint8_t)byte;
  for (int i = 0; i < 32; ++i) codes[i] = e4m3_round(std::ldexp(x[i], 127 - byte));
}

/* Row of n values (n % 32 == 0) quantised and dequantised: the values an
 * FP4 x FP8 GEMM sees. */
void mx_e4m3_dequantised_row(const double* x, int64_t n, double* out) {
  uint8_t codes[32], scale;
  for (int64_t b = 0; b < n; b += 32) {
    mx_e4m3_block(x + b, codes, &scale);
    for (int i = 0; i < 32; ++i) out[b + i] = std::ldexp(e4m3_value(codes[i]), (int)scale - 127);
  }
}

/* Gated activation a(g, u) of the expert FFN from the gate branch g = W_g x
 * and the up branch u = W_u x, in double:
 *  GLU_SWIGLU  SiLU(g) * u, SiLU(g) = g * sigmoid(g)        ([DS] 6.5; [LD] GLU branches)
 *  GLU_CLAMP   SiLU(min(g, 10)) * min(max(u, -10), 10)      ([DS] 6.5, the clamped SwiGLU:
 *              the gate branch is capped from above only, the up branch on both sides)
 *  GLU_SITU    [b1 tanh(g / b1) * sigmoid(g)] * [b2 tanh(u / b2)], b1 = 4 (gate), b2 = 25
 *              (up) ([LD] "SiTU-GLU": a scaled-tanh soft cap on each branch; the
 *              sigmoid takes the uncapped gate value)
 * A NaN branch value gives NaN (the comparisons below keep it). */
enum { GLU_SWIGLU = 0, GLU_CLAMP = 1, GLU_SITU = 2 };
const double kClampGate = 10.0, kClampUp = 10.0;
const double kSituGate = 4.0, kSituUp = 25.0;

double glu_value(double g, double u, int glu) {
  if (glu == GLU_CLAMP) {
    g = g > kClampGate ? kClampGate : g;
    u = u > kClampUp ? kClampUp : (u < -kClampUp ? -kClampUp : u);
    return g / (1.0 + std::exp(-g)) * u;
  }
  if (glu == GLU_SITU) {
    const double gate = kSituGate * std::tanh(g / kSituGate) * (1.0 / (1.0 + std::exp(-g)));
    return gate * (kSituUp * std::tanh(u / kSituUp));
  }
  return g / (1.0 + std::exp(-g)) * u;  // SiLU(g) * u
}

/* SwiGLU FFN of M rows with one expert's weights (double accumulation, the
 * method's rounding points).  x_rows [M,D] act; out [M,D] act; h_out [M,I] act. */
void expert_ffn(const void* x_rows, int act, int64_t M, int D, int I,
                const std::vector<double>& Wg, const std::vector<double>& Wu,
                const std::vector<double>& Wd, void* out, void* h_out,
                uint64_t* macs, int glu) {
  std::vector<double> h((size_t)(M * I));
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t ri = 0; ri < M * I; ++ri) {
    int64_t r = ri / I, i = ri % I;
    double g = 0.0, u = 0.0;
    for (int d = 0; d < D; ++d) {
      double xv = act_at(x_rows, act, r * D + d);
      g += xv * Wg[(size_t)(i * D + d)];
      u += xv * Wu[(size_t)(i * D + d)];
    }
    double a = glu_value(g, u, glu);
    double hv = (act == ACT_F32) ? (double)(float)a : (double)bf16_value(bf16_round(a));
    h[(size_t)ri] = hv;
    if (h_out) act_store(h_out, act, ri, hv);
  }
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t rn = 0; rn < M * D; ++rn) {
    int64_t r = rn / D, n = rn % D;
    double o = 0.0;
    for (int i = 0; i < I; ++i) o += h[(size_t)(r * I + i)] * Wd[(size_t)(n * I + i)];
    act_store(out, act, rn, o);
  }
  if (macs) *macs += (uint64_t)M * 3ull * (uint64_t)D * (uint64_t)I;
}

}  // namespace

extern "C" {

/* ---- scalar numerics, exposed for the pins ------------------------------- */
float orc_exp(float x) { return routing_exp(x); }
double orc_glu_value(double g, double u, int glu) { return glu_value(g, u, glu); }
float orc_sigmoid(float l) { return routing_sigmoid(l); }
uint16_t orc_bf16_from_f64(double d) { return bf16_round(d); }
uint16_t orc_bf16_from_f32(float f) { return bf16_round((double)f); }
double orc_mxfp4_value(uint8_t code, uint8_t scale) { return mxfp4_value(code, scale); }
uint32_t orc_fmix32(uint32_t h) { return fmix32(h); }

void orc_exp_array(const float* in, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = routing_exp(in[i]);
}
void orc_sigmoid_array(const float* in, float* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = routing_sigmoid(in[i]);
}
void orc_bf16_from_f64_array(const double* in, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(in[i]);
}

/* ---- router (DS 6.3 "scores = W h then top-k"; V4 2.2 linear router) ---- */
/* logits [T,E] fp32 in the pinned order. */
void orc_router_logits(const void* x, int act, const void* w_router, int64_t T, int D,
                       int E, float* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t te = 0; te < T * (int64_t)E; ++te) {
    int64_t t = te / E, e = te % E;
    logits[te] = router_logit(x, w_router, act, t * D, e * (int64_t)D, D);
  }
}

/* top-k + weights from logits (softmax / sigmoid) or token ids (hash).
 * keys [T,E] optional.  Returns 0, or -2 on a bad shape. */
int orc_route(const float* logits, const float* bias, const int32_t* token_ids, int64_t T,
              int E, int k, int mode, int32_t* topk_idx, float* topk_w, float* keys) {
  if (k < 1 || k > E) return -2;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    route_token(logits ? logits + t * E : nullptr, bias,
                token_ids ? token_ids[t] : 0, E, k, mode, topk_idx + t * k,
                topk_w + t * k, keys ? keys + t * E : nullptr);
  return 0;
}

/* ---- dispatch: stable counting sort of (token, slot) pairs by expert ---- */
int orc_permute(const int32_t* topk_idx, int64_t T, int k, int E, int32_t* counts,
                int32_t* offsets, int32_t* row_token, int32_t* pair_row) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < T * k; ++p) {
    int e = topk_idx[p];
    if (e < 0 || e >= E) return -2;
    counts[e]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> cursor(offsets, offsets + E);
  for (int64_t t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int e = topk_idx[t * k + j];
      int32_t r = cursor[e]++;
      row_token[r] = (int32_t)t;
      pair_row[t * k + j] = r;
    }
  return 0;
}

/* ---- MXFP8 helpers and the FP4 x FP8 expert FFN ------------------------- */
double orc_e4m3_value(uint8_t c) { return e4m3_value(c); }
uint8_t orc_e4m3_round(double v) { return e4m3_round(v); }
/* x [rows, n] (n % 32 == 0) -> codes [rows, n], scales [rows, n/32]. */
void orc_mx_e4m3_quantize(const double* x, int64_t rows, int64_t n, uint8_t* codes,
                          uint8_t* scales) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < n; b += 32)
      mx_e4m3_block(x + r * n + b, codes + r * n + b, scales + r * (n / 32) + b / 32);
}

/* One expert over M rows with MXFP4 weights and MXFP8 activations ([DS] 6.2
 * FP4 x FP8): x rows (bf16) are quantised per 32 along D before the gate/up
 * GEMM, and the rounded h rows per 32 along I before the down GEMM; the
 * GEMMs are exact (double) on the dequantised values; rounding points as in
 * expert_ffn (h and out bf16).  glu as in glu_value. */
void orc_expert_ffn_w4a8(const uint16_t* x_rows, int64_t M, int D, int I, const uint8_t* gate,
                         const uint8_t* up, const uint8_t* down, const uint8_t* gate_scale,
                         const uint8_t* up_scale, const uint8_t* down_scale, uint16_t* out,
                         uint16_t* h_out, int glu) {
  const std::vector<double> Wg = weight_matrix(gate, gate_scale, W_MXFP4, I, D);
  const std::vector<double> Wu = weight_matrix(up, up_scale, W_MXFP4, I, D);
  const std::vector<double> Wd = weight_matrix(down, down_scale, W_MXFP4, D, I);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < M; ++r) {
    std::vector<double> x((size_t)D), xq((size_t)D), h((size_t)I), hq((size_t)I);
    for (int d = 0; d < D; ++d) x[(size_t)d] = bf16_value(x_rows[r * D + d]);
    mx_e4m3_dequantised_row(x.data(), D, xq.data());
    for (int i = 0; i < I; ++i) {
      double g = 0.0, u = 0.0;
      for (int d = 0; d < D; ++d) {
        g += xq[(size_t)d] * Wg[(size_t)i * D + d];
        u += xq[(size_t)d] * Wu[(size_t)i * D + d];
      }
      h[(size_t)i] = bf16_value(bf16_round(glu_value(g, u, glu)));
      if (h_out) h_out[r * I + i] = bf16_round(h[(size_t)i]);
    }
    mx_e4m3_dequantised_row(h.data(), I, hq.data());
    for (int n = 0; n < D; ++n) {
      double o = 0.0;
      for (int i = 0; i < I; ++i) o += hq[(size_t)i] * Wd[(size_t)n * I + i];
      out[r * D + n] = bf16_round(o);
    }
  }
}

/* ---- one expert's SwiGLU FFN over M rows (DS 6.5 SwiGLU; LD GLU branches) */
/* wdtype: 0 fp32, 1 bf16, 2 mxfp4 (packed codes [.., cols/2] + scales [.., cols/32]).
 * glu: gated activation (GLU_SWIGLU, GLU_CLAMP or GLU_SITU, see glu_value). */
void orc_expert_ffn(const void* x_rows, int act, int64_t M, int D, int I, int wdtype,
                    const void* gate, const void* up, const void* down,
                    const uint8_t* gate_scale, const uint8_t* up_scale,
                    const uint8_t* down_scale, void* out, void* h_out, int glu) {
  std::vector<double> Wg = weight_matrix(gate, gate_scale, wdtype, I, D);
  std::vector<double> Wu = weight_matrix(up, up_scale, wdtype, I, D);
  std::vector<double> Wd = weight_matrix(down, down_scale, wdtype, D, I);
  expert_ffn(x_rows, act, M, D, I, Wg, Wu, Wd, out, h_out, nullptr, glu);
}

/* ---- combine (FW trap 3 + case study: fp32 sum, one final cast) --------- */
/* y[t] = round( (sum over the token's experts in ascending id of
 *                 fmaf(w, o[pair_row], acc)) + s[t] ) */
void orc_combine(const void* expert_out, const int32_t* topk_idx, const float* topk_w,
                 const int32_t* pair_row, const void* shared_out, int64_t T, int k, int D,
                 int act, void* y) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    std::vector<int> slot((size_t)k);
    for (int j = 0; j < k; ++j) slot[j] = j;
    std::sort(slot.begin(), slot.end(), [&](int a, int b) {
      return topk_idx[t * k + a] < topk_idx[t * k + b];
    });
    for (int d = 0; d < D; ++d) {
      float acc = 0.0f;
      for (int j : slot) {
        float o = act_at_f(expert_out, act, (int64_t)pair_row[t * k + j] * D + d);
        acc = std::fma(topk_w[t * k + j], o, acc);
      }
      if (shared_out) acc = acc + act_at_f(shared_out, act, t * D + d);
      act_store(y, act, t * D + d, (double)acc);
    }
  }
}

/* ---- residual add + RMSNorm (the next block's input norm) ---------------- */
/* The unfused MoE tail of [FW] trap 3 ends with rmsnorm(full_out + residual);
 * RMSNorm itself as in [LD] "RMSNorm before up-projection":
 *   RMSNorm(h) = g * h / sqrt(mean_d(h^2) + eps).
 * Readings (this library's definition): the residual stream is kept in the
 * activation type, so h = round(x + residual) is rounded before the norm sees
 * it (as the unfused kernels write it to memory), and the normalised value is
 * rounded once.  Everything between the two roundings is in double here.
 *   residual_out[t] = h[t] = round(x[t] + residual[t])
 *   normed[t, d] = round(g[d] * h[t, d] / sqrt(sum_d h[t, d]^2 / D + eps))
 * x, residual, gamma, residual_out, normed in the activation type. */
void orc_residual_rmsnorm(const void* x, const void* residual, const void* gamma, double eps,
                          int64_t T, int D, int act, void* residual_out, void* normed) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    std::vector<double> h((size_t)D);
    double ss = 0.0;
    for (int d = 0; d < D; ++d) {
      const int64_t i = t * D + d;
      const double sum = act_at(x, act, i) + act_at(residual, act, i);
      h[(size_t)d] = (act == ACT_F32) ? (double)(float)sum : (double)bf16_value(bf16_round(sum));
      ss += h[(size_t)d] * h[(size_t)d];
    }
    const double rms = std::sqrt(ss / D + eps);
    for (int d = 0; d < D; ++d) {
      act_store(residual_out, act, t * D + d, h[(size_t)d]);
      act_store(normed, act, t * D + d, act_at(gamma, act, d) * h[(size_t)d] / rms);
    }
  }
}

/* ---- the whole layer ------------------------------------------------------ */
/* Weights are given per expert (pointer arrays of length E, NULL allowed for
 * experts no token selects).  macs[3] (optional) receives the multiply-adds
 * the oracle executed: router, routed experts, shared expert.  glu: the gated
 * activation of every expert FFN of the layer (see glu_value). */
typedef struct {
  int wdtype;
  const void* const* gate;
  const void* const* up;
  const void* const* down;
  const uint8_t* const* gate_scale;
  const uint8_t* const* up_scale;
  const uint8_t* const* down_scale;
} orc_experts;

int orc_layer_forward(const void* x, int act, const int32_t* token_ids, const void* w_router,
                      const float* bias, const orc_experts* routed, const void* sh_gate,
                      const void* sh_up, const void* sh_down, int64_t T, int D, int E, int k,
                      int I, int I_shared, int mode, void* y, int32_t* topk_idx_out,
                      float* topk_w_out, uint64_t* macs, int glu) {
  if (k < 1 || k > E) return -2;
  const int64_t R = T * k;
  std::vector<float> logits;
  std::vector<int32_t> idx((size_t)R);
  std::vector<float> w((size_t)R);
  uint64_t mac_router = 0, mac_routed = 0, mac_shared = 0;
  if (mode != ROUTE_HASH) {
    logits.resize((size_t)(T * E));
    orc_router_logits(x, act, w_router, T, D, E, logits.data());
    mac_router = (uint64_t)T * (uint64_t)E * (uint64_t)D;
  }
  orc_route(mode != ROUTE_HASH ? logits.data() : nullptr, bias, token_ids, T, E, k, mode,
            idx.data(), w.data(), nullptr);
  std::vector<int32_t> counts((size_t)E), offsets((size_t)E + 1), row_token((size_t)R),
      pair_row((size_t)R);
  orc_permute(idx.data(), T, k, E, counts.data(), offsets.data(), row_token.data(),
              pair_row.data());
  const size_t esz = (act == ACT_F32) ? 4 : 2;
  std::vector<unsigned char> o((size_t)R * D * esz), xr, s;
  for (int e = 0; e < E; ++e) {
    int64_t M = counts[e];
    if (M == 0) continue;
    if (!routed->gate[e] || !routed->up[e] || !routed->down[e]) return -1;
    xr.resize((size_t)M * D * esz);
    for (int64_t r = 0; r < M; ++r)
      std::memcpy(&xr[(size_t)r * D * esz],
                  static_cast<const unsigned char*>(x) +
                      (size_t)row_token[offsets[e] + r] * D * esz,
                  (size_t)D * esz);
    std::vector<double> Wg = weight_matrix(routed->gate[e],
                                           routed->gate_scale ? routed->gate_scale[e] : nullptr,
                                           routed->wdtype, I, D);
    std::vector<double> Wu = weight_matrix(routed->up[e],
                                           routed->up_scale ? routed->up_scale[e] : nullptr,
                                           routed->wdtype, I, D);
    std::vector<double> Wd = weight_matrix(routed->down[e],
                                           routed->down_scale ? routed->down_scale[e] : nullptr,
                                           routed->wdtype, D, I);
    expert_ffn(xr.data(), act, M, D, I, Wg, Wu, Wd, &o[(size_t)offsets[e] * D * esz], nullptr,
               &mac_routed, glu);
  }
  if (I_shared > 0) {
    s.resize((size_t)T * D * esz);
    int sw = (act == ACT_F32) ? ACT_F32 : ACT_BF16;
    std::vector<double> Wg = weight_matrix(sh_gate, nullptr, sw, I_shared, D);
    std::vector<double> Wu = weight_matrix(sh_up, nullptr, sw, I_shared, D);
    std::vector<double> Wd = weight_matrix(sh_down, nullptr, sw, D, I_shared);
    expert_ffn(x, act, T, D, I_shared, Wg, Wu, Wd, s.data(), nullptr, &mac_shared, glu);
  }
  orc_combine(o.data(), idx.data(), w.data(), pair_row.data(), I_shared > 0 ? s.data() : nullptr,
              T, k, D, act, y);
  if (topk_idx_out) std::memcpy(topk_idx_out, idx.data(), (size_t)R * 4);
  if (topk_w_out) std::memcpy(topk_w_out, w.data(), (size_t)R * 4);
  if (macs) {
    macs[0] = mac_router;
    macs[1] = mac_routed;
    macs[2] = mac_shared;
  }
  return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads of later parallel regions (n >= 1); the arithmetic of every output
 * element is the same for any thread count. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

}  // extern "C"
