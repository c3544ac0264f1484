// Plain, slow CPU oracle of the fine-grained-quantized MoE experts forward.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
// this file; only the tests, the smoke check and the benchmark's CPU-baseline
// leg use it.  It shares no code, header, table or constant generator with the
// HIP library: its codecs, its sort and its arithmetic are written here from the
// definitions and nowhere else.
//
// What it follows (pages are cited by title and section):
//  * "grouped_mm experts dispatch does not support activation_scheme='static'",
//    section "Source": the grouped experts forward flattens the (token, slot)
//    pairs, sorts them by expert id, gathers each pair's token row, and ends
//    (shared contract with the batched path) by zeroing sentinel rows,
//    weighting each slot's output and summing the k slots of a token with a
//    deterministic reshape+sum before casting back to the input dtype.
//    Section "What it means": activations are quantized dynamically per block.
//  * "DeepGEMM Mega MoE requires a `process_group` for the EP group" (docstring
//    in the record's source): top_k_index holds global expert ids with -1 for a
//    skipped slot; gate_up_proj / down_proj are the L1 / L2 weights with their
//    scale factors; swiglu_limit is an optional SwiGLU clamp (absent means
//    unclamped).
//  * "DeepGEMM Mega MoE requires FP4-packed expert weights (dtype=int8)",
//    section "Source": FP4 weights arrive packed in int8 bytes.
//
// Readings of what the pages leave open (all listed in the design notes):
//  - sentinel slots (id -1, or any id outside the local expert range) sort
//    after every valid slot; ties inside one expert keep flat-slot order;
//  - FP8 is OCP e4m3fn; encoding is round-to-nearest-even on the magnitude,
//    saturating at 448, sign kept (negative values that round to zero give
//    0x80);
//  - FP8 block format: activation scale per 1x128 block s = max(amax,1e-4f)/448
//    in fp32, code = e4m3(x / s) with an IEEE fp32 division; weight scales are
//    fp32 per 128x128 block and multiply the decoded code;
//  - MX format: activation scale per 1x32 block is 2^e with
//    e = ceil(log2(max(amax,1e-4f)/448)) taken exactly from the fp32 bits,
//    stored as the byte e+127; code = e4m3(x * 2^-e); weights are e2m1 packed
//    two per byte along K (even k in the low nibble) with a UE8M0 byte per 1x32;
//  - gate rows are [0, I) of gate_up_proj, up rows are [I, 2I);
//    h = silu(g) * u; with a limit L: g <- min(g, L), u <- clamp(u, -L, L);
//  - the intermediate h is re-quantized with the same rule as the activations
//    (blocks along I), in fp32, before the down projection;
//  - the routing weight multiplies each slot's down-projection output; skipped
//    slots are never computed and contribute exactly zero (their weight is
//    never read); slots are summed in ascending j.
//
// Precision: dot products, SwiGLU and the weighted sum run in fp64.  Where a
// float decides an integer (activation and h codes and scales) the decision is
// taken in fp32, the precision of the GPU kernels.  The final value is rounded
// fp64 -> fp32 -> bf16 (round to nearest even each time).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

enum { FMT_FP8_B128 = 0, FMT_MX = 1, FMT_BF16 = 2 };
enum { OK = 0, ERR_NULL = 1, ERR_SHAPE = 2, ERR_FMT = 3 };

// ---------------------------------------------------------------- codecs --

// OCP 8-bit floating point, E4M3 ("fn" variant): 1 sign, 4 exponent (bias 7),
// 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is
// NaN; there is no infinity.  Largest finite magnitude 448.
double e4m3_value(uint8_t code) {
  const int sign = code >> 7;
  const int ex = (code >> 3) & 0xF;
  const int man = code & 0x7;
  double mag;
  if (ex == 0xF && man == 0x7) return NAN;
  if (ex == 0)
    mag = std::ldexp((double)man / 8.0, -6);
  else
    mag = std::ldexp(1.0 + (double)man / 8.0, ex - 7);
  return sign ? -mag : mag;
}

// OCP MX e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent field 0
// is subnormal (m/2 * 2^0).  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
double e2m1_value(uint8_t nib) {
  const int sign = (nib >> 3) & 1;
  const int ex = (nib >> 1) & 0x3;
  const int man = nib & 1;
  double mag = ex == 0 ? (double)man * 0.5 : std::ldexp(1.0 + (double)man / 2.0, ex - 1);
  return sign ? -mag : mag;
}

// Decode tables, built once from the definitions above (function-local
// statics are initialised exactly once, also under OpenMP).
const double* e4m3_table() {
  static const std::vector<double> t = [] {
    std::vector<double> v(256);
    for (int c = 0; c < 256; ++c) v[c] = e4m3_value((uint8_t)c);
    return v;
  }();
  return t.data();
}
const double* e2m1_table() {
  static const std::vector<double> t = [] {
    std::vector<double> v(16);
    for (int c = 0; c < 16; ++c) v[c] = e2m1_value((uint8_t)c);
    return v;
  }();
  return t.data();
}
// UE8M0 scale byte b -> 2^(b-127); 0xFF is NaN (OCP MX).
const double* e8m0_table() {
  static const std::vector<double> t = [] {
    std::vector<double> v(256);
    for (int b = 0; b < 255; ++b) v[b] = std::ldexp(1.0, b - 127);
    v[255] = NAN;
    return v;
  }();
  return t.data();
}

// Encode a value as e4m3: the representable magnitude nearest to |x|, ties
// going to the code with the even mantissa bit; magnitudes above 448 give 448.
// The candidates are the 127 finite non-negative codes, which increase with
// the code, searched directly.
uint8_t e4m3_encode(double x) {
  const double* table = e4m3_table();
  const uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  const double a = std::fabs(x);
  if (a >= 448.0) return sign | 0x7E;
  // first code whose value is >= a
  const int hi = (int)(std::lower_bound(table, table + 127, a) - table);
  int best;
  if (hi == 0) {
    best = 0;
  } else {
    const int lo = hi - 1;
    const double dlo = a - table[lo];
    const double dhi = table[hi] - a;
    if (dlo < dhi)
      best = lo;
    else if (dhi < dlo)
      best = hi;
    else
      best = (lo & 1) == 0 ? lo : hi;  // tie: even mantissa
  }
  return sign | (uint8_t)best;
}

float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// fp32 -> bf16, round to nearest even (NaN kept as a quiet NaN).
uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if (std::isnan(f)) return (uint16_t)((u >> 16) | 0x40);
  const uint32_t lsb = (u >> 16) & 1;
  u += 0x7FFF + lsb;
  return (uint16_t)(u >> 16);
}

// ceil(log2(r)) for a positive, normal fp32 r, read exactly from its bits:
// the unbiased exponent, plus one when any mantissa bit is set.
int ceil_log2_f32(float r) {
  uint32_t u;
  std::memcpy(&u, &r, 4);
  const int ex = (int)((u >> 23) & 0xFF) - 127;
  const uint32_t man = u & 0x7FFFFF;
  return ex + (man != 0 ? 1 : 0);
}

// -------------------------------------------------- activation quantization --
// Encoding of one block of B values once its scale is known.  FP8 format: the
// fp32 scale s, code = e4m3(x / s) with an IEEE fp32 division.  MX format: the
// UE8M0 byte b, code = e4m3(x * 2^-(b-127)) computed exactly in fp64.  e4m3()
// rounds to nearest even and saturates at 448, so values past 448 s give the
// largest code of their sign.
void encode_block(const float* x, int64_t B, int fmt, float s_f32, uint8_t s_u8, uint8_t* codes) {
  if (fmt == FMT_FP8_B128) {
    for (int64_t i = 0; i < B; ++i) {
      const float q = x[i] / s_f32;  // IEEE fp32 division
      codes[i] = e4m3_encode(q);
    }
  } else {
    const int e = (int)s_u8 - 127;
    for (int64_t i = 0; i < B; ++i) codes[i] = e4m3_encode(std::ldexp((double)x[i], -e));
  }
}

// Dynamic per-block quantization of one row of fp32 values (bf16 input is
// widened exactly first).  Block length 128 with an fp32 scale (FP8 format) or
// 32 with a UE8M0 byte (MX format).
void quant_row(const float* x, int64_t n, int fmt, uint8_t* codes, float* sc_f32, uint8_t* sc_u8) {
  const int64_t B = fmt == FMT_FP8_B128 ? 128 : 32;
  for (int64_t b = 0; b < n / B; ++b) {
    float amax = 0.0f;
    for (int64_t i = 0; i < B; ++i) amax = std::max(amax, std::fabs(x[b * B + i]));
    const float r = std::max(amax, 1e-4f) / 448.0f;
    if (fmt == FMT_FP8_B128) {
      sc_f32[b] = r;
      encode_block(x + b * B, B, fmt, r, 0, codes + b * B);
    } else {
      const int e = ceil_log2_f32(r);
      sc_u8[b] = (uint8_t)(e + 127);
      encode_block(x + b * B, B, fmt, 0.0f, sc_u8[b], codes + b * B);
    }
  }
}

// Static per-block quantization of one row: the caller's precomputed block
// scales (fp32 per 1x128 for the FP8 format, UE8M0 bytes per 1x32 for MX)
// replace the amax pass; the encoding is the dynamic rule's.
void quant_row_static(const float* x, int64_t n, int fmt, const void* row_scales, uint8_t* codes) {
  const int64_t B = fmt == FMT_FP8_B128 ? 128 : 32;
  for (int64_t b = 0; b < n / B; ++b) {
    if (fmt == FMT_FP8_B128)
      encode_block(x + b * B, B, fmt, ((const float*)row_scales)[b], 0, codes + b * B);
    else
      encode_block(x + b * B, B, fmt, 0.0f, ((const uint8_t*)row_scales)[b], codes + b * B);
  }
}

// Element size and row address of a caller's static scale array: token t's
// row of H/B scales starts `row_stride` elements after token t - 1's (0: the
// one row serves every token).
inline const void* static_row(int fmt, const void* scales, int64_t row_stride, int64_t t) {
  if (fmt == FMT_FP8_B128) return (const float*)scales + t * row_stride;
  return (const uint8_t*)scales + t * row_stride;
}

// Decoded (dequantized) activation element i of row `row` of a [rows, K]
// code array: code value times its block scale.
inline double act_value(int fmt, const uint8_t* codes, const void* scales, int64_t row, int64_t K,
                        int64_t i) {
  if (fmt == FMT_BF16) return (double)bf16_to_f32(((const uint16_t*)codes)[row * K + i]);
  const double q = e4m3_table()[codes[row * K + i]];
  if (fmt == FMT_FP8_B128) return q * (double)((const float*)scales)[row * (K / 128) + i / 128];
  return q * e8m0_table()[((const uint8_t*)scales)[row * (K / 32) + i / 32]];
}

// Decoded weight row n of expert e (N rows of K columns), written to out[K].
void weight_row(int fmt, const uint8_t* w, const void* ws, int64_t e, int64_t N, int64_t K, int64_t n,
                double* out) {
  if (fmt == FMT_BF16) {  // plain bf16 values, no scales
    const uint16_t* row = (const uint16_t*)w + (e * N + n) * K;
    for (int64_t i = 0; i < K; ++i) out[i] = (double)bf16_to_f32(row[i]);
    return;
  }
  if (fmt == FMT_FP8_B128) {
    const double* dec = e4m3_table();
    const uint8_t* code = w + (e * N + n) * K;
    const float* sc = (const float*)ws + (e * (N / 128) + n / 128) * (K / 128);
    for (int64_t i = 0; i < K; ++i) out[i] = dec[code[i]] * (double)sc[i / 128];
  } else {
    const double* dec = e2m1_table();
    const double* p2 = e8m0_table();
    const uint8_t* packed = w + (e * N + n) * (K / 2);
    const uint8_t* sc = (const uint8_t*)ws + (e * N + n) * (K / 32);
    for (int64_t i = 0; i < K; ++i) {
      const uint8_t byte = packed[i / 2];
      const uint8_t nib = (i & 1) ? (byte >> 4) : (byte & 0xF);  // even k in the low nibble
      out[i] = dec[nib] * p2[sc[i / 32]];
    }
  }
}

double dot(const double* a, const double* b, int64_t n) {
  double acc = 0.0;
  for (int64_t i = 0; i < n; ++i) acc += a[i] * b[i];
  return acc;
}

}  // namespace

extern "C" {

// Elementwise codecs, exported so the tests can pin them against the spec
// tables and torch's own float8 cast.
void oracle_e4m3_decode(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(c[i]);
}
void oracle_e2m1_decode(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e2m1_value(c[i] & 0xF);
}
void oracle_e8m0_decode(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e8m0_table()[c[i]];
}
void oracle_e4m3_encode(const float* x, int64_t n, uint8_t* out) {
  e4m3_table();
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(x[i]);
}

// Route sort.  key(s) = ids[s] - expert_begin when that lies in [0, E), else E
// (a sentinel).  sorted_slot lists flat slots s = t*k + j by (key, s);
// expert_offsets[e] counts the slots whose key is below e (e = 0..E);
// slot_pos is the inverse permutation; invalid_count counts ids that are
// neither -1 nor inside the local range.
int oracle_route_sort(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t expert_begin,
                      int32_t* sorted_slot, int32_t* expert_offsets, int32_t* slot_pos,
                      int32_t* invalid_count) {
  if (T < 0 || k < 1 || E < 1) return ERR_SHAPE;
  if ((T > 0 && (!ids || !sorted_slot || !slot_pos)) || !expert_offsets) return ERR_NULL;
  const int64_t S = (int64_t)T * k;
  std::vector<int32_t> key(S);
  int32_t invalid = 0;
  for (int64_t s = 0; s < S; ++s) {
    const int64_t local = (int64_t)ids[s] - expert_begin;
    if (local >= 0 && local < E) {
      key[s] = (int32_t)local;
    } else {
      key[s] = E;
      if (ids[s] != -1) ++invalid;
    }
  }
  std::vector<int32_t> order(S);
  for (int64_t s = 0; s < S; ++s) order[s] = (int32_t)s;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return key[a] < key[b]; });
  for (int64_t r = 0; r < S; ++r) {
    sorted_slot[r] = order[r];
    slot_pos[order[r]] = (int32_t)r;
  }
  for (int32_t e = 0; e <= E; ++e) {
    int64_t c = 0;
    for (int64_t s = 0; s < S; ++s) c += key[s] < e;
    expert_offsets[e] = (int32_t)c;
  }
  if (invalid_count) *invalid_count = invalid;
  return OK;
}

// Router top-k: the step just before the experts forward, which produces its
// top_k_index / top_k_weights.  The pages pass the router's output to the
// experts untouched, as global ids with unmasked weights (PR #49606, "How it
// runs" and the parallel-style table); the router of the layers the forward is
// shaped on (Mixtral, Qwen3-MoE) is: softmax over the E logits of a token, the
// k most probable experts, and (when `renormalize`) their probabilities divided
// by the sum of the k selected.
//  - Selection: softmax is strictly increasing in the logit, so the k most
//    probable experts are the k largest logits, compared as fp32 values;
//    among equal logits the lower id comes first.  ids[t][j] lists them in
//    that order (j = 0 is the largest).
//  - Weights in fp64: p_e = exp(l_e - m) / sum_e' exp(l_e' - m) with m the
//    row maximum; w_j = p_{ids[j]}, divided by sum_j p_{ids[j]} when
//    renormalizing; rounded once to fp32.
// Logits must be finite (not checked).
int oracle_router_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renormalize, int32_t* ids,
                       float* weights) {
  if (T < 0 || E < 1 || k < 1 || k > E) return ERR_SHAPE;
  if (T > 0 && (!logits || !ids || !weights)) return ERR_NULL;
  std::vector<int32_t> order(E);
  std::vector<double> p(E);
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    for (int32_t e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return l[a] > l[b]; });
    const double m = (double)l[order[0]];
    double z = 0.0;
    for (int32_t e = 0; e < E; ++e) {
      p[e] = std::exp((double)l[e] - m);
      z += p[e];
    }
    for (int32_t e = 0; e < E; ++e) p[e] /= z;
    double sel = 0.0;
    for (int32_t j = 0; j < k; ++j) sel += p[order[j]];
    for (int32_t j = 0; j < k; ++j) {
      ids[t * k + j] = order[j];
      weights[t * k + j] = (float)(renormalize ? p[order[j]] / sel : p[order[j]]);
    }
  }
  return OK;
}

// Dynamic per-block quantization of bf16 rows [rows, H].
int oracle_quant_rows_bf16(const uint16_t* x, int32_t rows, int32_t H, int32_t fmt, uint8_t* codes,
                           void* scales) {
  if (fmt != FMT_FP8_B128 && fmt != FMT_MX) return ERR_FMT;
  if (rows < 0 || H <= 0 || H % (fmt == FMT_FP8_B128 ? 128 : 32)) return ERR_SHAPE;
  if (rows > 0 && (!x || !codes || !scales)) return ERR_NULL;
  const int64_t B = fmt == FMT_FP8_B128 ? 128 : 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    std::vector<float> row(H);
    for (int64_t i = 0; i < H; ++i) row[i] = bf16_to_f32(x[r * H + i]);
    quant_row(row.data(), H, fmt, codes + r * H, fmt == FMT_FP8_B128 ? (float*)scales + r * (H / B) : nullptr,
              fmt == FMT_MX ? (uint8_t*)scales + r * (H / B) : nullptr);
  }
  return OK;
}

// Static quantization of bf16 rows [rows, H] with the caller's block scales:
// row t uses scales[t * row_stride ...] (fp32 [.., H/128] for the FP8 format,
// UE8M0 bytes [.., H/32] for MX); row_stride 0 broadcasts one row of scales.
// The scales are the static activation scheme's precomputed per-block scales
// ("grouped_mm experts dispatch does not support activation_scheme='static'",
// sections "What it means" and "Example fix": the eager path consumes them, the
// grouped one quantized dynamically instead).  FP8 scales must be finite and
// positive, MX bytes below 255.
int oracle_quant_rows_bf16_static(const uint16_t* x, int32_t rows, int32_t H, int32_t fmt, const void* scales,
                                  int32_t row_stride, uint8_t* codes) {
  if (fmt != FMT_FP8_B128 && fmt != FMT_MX) return ERR_FMT;
  const int32_t nb = H / (fmt == FMT_FP8_B128 ? 128 : 32);
  if (rows < 0 || H <= 0 || H % 128 || row_stride < 0 || (row_stride > 0 && row_stride < nb)) return ERR_SHAPE;
  if (rows > 0 && (!x || !codes || !scales)) return ERR_NULL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    std::vector<float> row(H);
    for (int64_t i = 0; i < H; ++i) row[i] = bf16_to_f32(x[r * H + i]);
    quant_row_static(row.data(), H, fmt, static_row(fmt, scales, row_stride, r), codes + r * H);
  }
  return OK;
}

// The same rule applied to fp32 rows (the rule the forward uses for h).
int oracle_quant_rows_f32(const float* x, int32_t rows, int32_t H, int32_t fmt, uint8_t* codes, void* scales) {
  if (fmt != FMT_FP8_B128 && fmt != FMT_MX) return ERR_FMT;
  if (rows < 0 || H <= 0 || H % (fmt == FMT_FP8_B128 ? 128 : 32)) return ERR_SHAPE;
  if (rows > 0 && (!x || !codes || !scales)) return ERR_NULL;
  const int64_t B = fmt == FMT_FP8_B128 ? 128 : 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    quant_row(x + r * H, H, fmt, codes + r * H, fmt == FMT_FP8_B128 ? (float*)scales + r * (H / B) : nullptr,
              fmt == FMT_MX ? (uint8_t*)scales + r * (H / B) : nullptr);
  return OK;
}

// Grouped GEMM over expert-sorted rows: for sorted row r in expert e's range
// [offsets[e], offsets[e+1]), C[r][n] = sum_i A[a_row(r)][i] * B[e][n][i] with
// both operands decoded to values (code times scale) and summed in fp64.
// a_row(r) = row_index[r] / row_div when row_index is given, else r.
// BF16 format: A and B hold bf16 bit patterns (uint16) and no scales.
int oracle_grouped_gemm(int32_t fmt, const uint8_t* a_codes, const void* a_scales, const int32_t* row_index,
                        int32_t row_div, const int32_t* offsets, int32_t E, const uint8_t* b_codes,
                        const void* b_scales, int32_t N, int32_t K, double* out) {
  if (fmt != FMT_FP8_B128 && fmt != FMT_MX && fmt != FMT_BF16) return ERR_FMT;
  if (E < 1 || N <= 0 || K <= 0 || K % 128 || N % (fmt == FMT_FP8_B128 ? 128 : 1)) return ERR_SHAPE;
  if (!a_codes || !offsets || !b_codes || !out) return ERR_NULL;
  if (fmt != FMT_BF16 && (!a_scales || !b_scales)) return ERR_NULL;
  const int64_t rows = offsets[E];
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    int64_t e = 0;
    while (!(offsets[e] <= r && r < offsets[e + 1])) ++e;
    const int64_t ar = row_index ? row_index[r] / row_div : r;
    std::vector<double> a(K), b(K);
    for (int64_t i = 0; i < K; ++i) a[i] = act_value(fmt, a_codes, a_scales, ar, K, i);
    for (int64_t n = 0; n < N; ++n) {
      weight_row(fmt, b_codes, b_scales, e, N, K, n, b.data());
      out[r * N + n] = dot(a.data(), b.data(), K);
    }
  }
  return OK;
}

// The experts forward, token by token and slot by slot.
//
// Weights (nt layout): FP8 format: w13 u8 [E, 2I, H] with fp32 scales
// [E, 2I/128, H/128]; w2 u8 [E, H, I] with fp32 scales [E, H/128, I/128].
// MX format: w13 packed [E, 2I, H/2] with u8 scales [E, 2I, H/32]; w2 packed
// [E, H, I/2] with u8 scales [E, H, I/32].
// BF16 format (the unquantized grouped_mm experts the pages fall back to, "DeepGEMM
// experts selected on a model spanning multiple CUDA devices", the record's
// source): w13 bf16 [E, 2I, H], w2 bf16 [E, H, I], no scales; activations are
// used as they are, and h is rounded once to bf16 (through fp32, the precision
// of the GPU's accumulators) to be the down projection's operand.
//
// Only the tokens listed in `tokens` (all tokens when NULL) are computed; their
// rows of `out` are written.  Optional per-slot debug outputs (indexed by the
// flat slot s = t*k + j, written for valid slots of computed tokens only):
// gu [S, 2I] fp32 (L1 result before the clamp), h_codes [S, I] with h_scales
// (fp32 [S, I/128] or u8 [S, I/32]), y [S, H] fp32 (down projection, before
// the routing weight).
int oracle_forward(int32_t fmt, int32_t E, int32_t H, int32_t I, const uint8_t* w13, const void* w13_scale,
                   const uint8_t* w2, const void* w2_scale, const uint16_t* x, const int32_t* ids,
                   const float* wts, int32_t T, int32_t k, int32_t expert_begin, int32_t has_limit, float limit,
                   const int32_t* tokens, int32_t n_tokens, uint16_t* out, float* dbg_gu, uint8_t* dbg_h_codes,
                   void* dbg_h_scales, float* dbg_y, const void* act_scales, int32_t act_row_stride) {
  if (fmt != FMT_FP8_B128 && fmt != FMT_MX && fmt != FMT_BF16) return ERR_FMT;
  if (E < 1 || T < 0 || k < 1 || H <= 0 || I <= 0 || H % 128 || I % 128) return ERR_SHAPE;
  // static activation scales (act_scales non-NULL): the layer input is
  // quantized with them instead of its own block amax; h stays dynamic (the
  // scheme names the input's scales only)
  if (act_scales && (fmt == FMT_BF16 || act_row_stride < 0 ||
                     (act_row_stride > 0 && act_row_stride < H / (fmt == FMT_FP8_B128 ? 128 : 32))))
    return ERR_SHAPE;
  if (has_limit && !(std::isfinite(limit) && limit > 0.0f)) return ERR_SHAPE;
  if (T == 0) return OK;
  if (!w13 || !w2 || !x || !ids || !wts || !out) return ERR_NULL;
  if (fmt != FMT_BF16 && (!w13_scale || !w2_scale)) return ERR_NULL;
  const bool bf = fmt == FMT_BF16;
  const int64_t n_list = tokens ? n_tokens : T;
  const int64_t Bh = fmt == FMT_FP8_B128 ? 128 : 32;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t li = 0; li < n_list; ++li) {
    const int64_t t = tokens ? tokens[li] : li;
    if (t < 0 || t >= T) continue;
    // Activation quantization of the token's row (dynamic, per block).
    std::vector<float> xr(H);
    for (int64_t i = 0; i < H; ++i) xr[i] = bf16_to_f32(x[t * H + i]);
    std::vector<double> a(H);
    if (bf) {
      for (int64_t i = 0; i < H; ++i) a[i] = (double)xr[i];
    } else {
      std::vector<uint8_t> xq(H);
      std::vector<float> xs_f(H / 128);
      std::vector<uint8_t> xs_u(H / 32);
      const void* xs;
      if (act_scales) {
        xs = static_row(fmt, act_scales, act_row_stride, t);
        quant_row_static(xr.data(), H, fmt, xs, xq.data());
      } else {
        quant_row(xr.data(), H, fmt, xq.data(), xs_f.data(), xs_u.data());
        xs = fmt == FMT_FP8_B128 ? (const void*)xs_f.data() : (const void*)xs_u.data();
      }
      for (int64_t i = 0; i < H; ++i) a[i] = act_value(fmt, xq.data(), xs, 0, H, i);
    }

    std::vector<double> acc(H, 0.0);
    std::vector<double> gu(2 * (int64_t)I);
    std::vector<float> h(I);
    std::vector<uint8_t> hq(I);
    std::vector<float> hs_f(I / 128);
    std::vector<uint8_t> hs_u(I / 32);
    std::vector<double> hd(I);
    std::vector<double> wrow(std::max<int64_t>(H, I));
    for (int64_t j = 0; j < k; ++j) {
      const int64_t s = t * k + j;
      const int64_t e = (int64_t)ids[s] - expert_begin;
      if (e < 0 || e >= E) continue;  // skipped slot: contributes nothing
      // L1: gate_up projection.
      for (int64_t n = 0; n < 2 * (int64_t)I; ++n) {
        weight_row(fmt, w13, w13_scale, e, 2 * (int64_t)I, H, n, wrow.data());
        gu[n] = dot(a.data(), wrow.data(), H);
      }
      if (dbg_gu)
        for (int64_t n = 0; n < 2 * (int64_t)I; ++n) dbg_gu[s * 2 * I + n] = (float)gu[n];
      // SwiGLU with the optional clamp.
      for (int64_t n = 0; n < I; ++n) {
        double g = gu[n], u = gu[I + n];
        if (has_limit) {
          g = std::min(g, (double)limit);
          u = std::min(std::max(u, -(double)limit), (double)limit);
        }
        h[n] = (float)(g / (1.0 + std::exp(-g)) * u);
      }
      if (bf) {
        // BF16: h rounded to bf16 is the down projection's operand.
        for (int64_t i = 0; i < I; ++i) hd[i] = (double)bf16_to_f32(f32_to_bf16(h[i]));
      } else {
      // Re-quantize h with the activation rule, blocks along I.
      quant_row(h.data(), I, fmt, hq.data(), hs_f.data(), hs_u.data());
      const void* hs = fmt == FMT_FP8_B128 ? (const void*)hs_f.data() : (const void*)hs_u.data();
      if (dbg_h_codes) std::memcpy(dbg_h_codes + s * I, hq.data(), I);
      if (dbg_h_scales) {
        if (fmt == FMT_FP8_B128)
          std::memcpy((float*)dbg_h_scales + s * (I / Bh), hs_f.data(), sizeof(float) * (I / Bh));
        else
          std::memcpy((uint8_t*)dbg_h_scales + s * (I / Bh), hs_u.data(), I / Bh);
      }
      for (int64_t i = 0; i < I; ++i) hd[i] = act_value(fmt, hq.data(), hs, 0, I, i);
      }
      // L2: down projection, then the routing weight, summed over ascending j.
      const double wj = (double)wts[s];
      for (int64_t c = 0; c < H; ++c) {
        weight_row(fmt, w2, w2_scale, e, H, I, c, wrow.data());
        const double y = dot(hd.data(), wrow.data(), I);
        if (dbg_y) dbg_y[s * H + c] = (float)y;
        acc[c] += wj * y;
      }
    }
    for (int64_t c = 0; c < H; ++c) out[t * H + c] = f32_to_bf16((float)acc[c]);
  }
  return OK;
}

}  // extern "C"
