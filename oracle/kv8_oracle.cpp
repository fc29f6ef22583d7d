// kv8 CPU oracle -- TEST INFRASTRUCTURE ONLY (see kv8_oracle.h).
//
// Plain C++17, no GPU headers, built with -ffp-contract=off and without
// fast-math so every float operation below is one IEEE f32 or f64 operation
// rounded to nearest-even, exactly as written.
//
// [colibri#299] = the page "KV8=1: fp8 e4m3 latent KV cache (CPU + CUDA) with
// .coli_kv v2" (colibri pull request #299).
// [OFP8 E4M3]   = the OCP 8-bit floating point format, E4M3 variant.
#include "kv8_oracle.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

int resolve_threads(int threads) {
    if (threads > 0) return threads;
    unsigned hc = std::thread::hardware_concurrency();
    return hc ? static_cast<int>(hc) : 1;
}

// Run body(i) for i in [0, n) on `threads` workers pulling from one counter.
template <class F>
void parallel_for(int64_t n, int threads, F body) {
    threads = resolve_threads(threads);
    if (threads <= 1 || n <= 1) {
        for (int64_t i = 0; i < n; ++i) body(i);
        return;
    }
    std::atomic<int64_t> next{0};
    auto worker = [&]() {
        for (;;) {
            int64_t i = next.fetch_add(1);
            if (i >= n) break;
            body(i);
        }
    };
    std::vector<std::thread> pool;
    int nt = static_cast<int>(std::min<int64_t>(threads, n));
    for (int k = 0; k < nt; ++k) pool.emplace_back(worker);
    for (auto& t : pool) t.join();
}

// The 127 non-negative finite e4m3 values, index = code (0x00..0x7E), built
// from orc_decode.  Used by the nearest-value search of the encoder and as the
// dequantization table of the attention ([colibri#299] commit message,
// kv_fp8.h item: a 256-entry decode table).
struct Tables {
    double pos[127];
    double all[256];
    Tables() {
        for (int c = 0; c < 127; ++c) pos[c] = orc_decode(static_cast<uint8_t>(c));
        for (int c = 0; c < 256; ++c) all[c] = orc_decode(static_cast<uint8_t>(c));
    }
};
const Tables& tables() {
    static const Tables t;
    return t;
}

float bf16_to_float(uint16_t bits) {
    uint32_t u = static_cast<uint32_t>(bits) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

}  // namespace

extern "C" {

// [OFP8 E4M3]: sign s, exponent field e (bias 7), mantissa field m (3 bits).
// e = 15 with m = 7 is NaN; e = 0 is subnormal m * 2^-9; otherwise the value
// is (1 + m/8) * 2^(e-7) = (8 + m) * 2^(e-10).
double orc_decode(uint8_t code) {
    const int s = code >> 7;
    const int e = (code >> 3) & 15;
    const int m = code & 7;
    if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
    double mag;
    if (e == 0)
        mag = std::ldexp(static_cast<double>(m), -9);
    else
        mag = std::ldexp(static_cast<double>(8 + m), e - 10);
    return s ? -mag : mag;
}

// [colibri#299] commit message, kv_fp8.h item: round to nearest even,
// saturate at +-448, keep the sign of zero, store NaN as an inert 0.
// Written as the definition: among the non-negative finite values pick the
// nearest to |q|; on an exact tie pick the code whose last bit is 0.
uint8_t orc_encode(float q) {
    if (std::isnan(q)) return 0x00;
    const uint8_t sign = std::signbit(q) ? 0x80 : 0x00;
    const double a = std::fabs(static_cast<double>(q));
    const Tables& T = tables();
    if (a >= T.pos[126]) return static_cast<uint8_t>(0x7E | sign);  // 448 and beyond
    // Largest index i with pos[i] <= a (binary search over the sorted values).
    int lo = 0, hi = 126;  // invariant: pos[lo] <= a < pos[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (T.pos[mid] <= a) lo = mid; else hi = mid;
    }
    // Compare 2a with pos[lo] + pos[hi]: both sides are exact in f64.
    const double twice = 2.0 * a;
    const double sum = T.pos[lo] + T.pos[hi];
    int code;
    if (twice < sum) code = lo;
    else if (twice > sum) code = hi;
    else code = (lo % 2 == 0) ? lo : hi;
    return static_cast<uint8_t>(code | sign);
}

void orc_encode_bits_range(uint64_t first, uint64_t count, uint8_t* out, int threads) {
    const int64_t chunk = 1 << 20;
    const int64_t nchunks = static_cast<int64_t>((count + chunk - 1) / chunk);
    parallel_for(nchunks, threads, [&](int64_t c) {
        uint64_t b = static_cast<uint64_t>(c) * chunk;
        uint64_t e = std::min<uint64_t>(count, b + chunk);
        for (uint64_t k = b; k < e; ++k) {
            uint32_t u = static_cast<uint32_t>(first + k);
            float f;
            std::memcpy(&f, &u, 4);
            out[k] = orc_encode(f);
        }
    });
}

void orc_encode_array(const float* in, int64_t n, uint8_t* out, int threads) {
    const int64_t chunk = 1 << 16;
    const int64_t nchunks = (n + chunk - 1) / chunk;
    parallel_for(nchunks, threads, [&](int64_t c) {
        int64_t b = c * chunk, e = std::min<int64_t>(n, b + chunk);
        for (int64_t k = b; k < e; ++k) out[k] = orc_encode(in[k]);
    });
}

// [colibri#299] commit message, kv_fp8.h item: per-row f32 amax/448 scale
// with a guard for amax so small that 448/amax overflows to +inf.
// amax runs over the finite entries only (NaN is stored as 0 and must not set
// the scale; +-inf saturates and must not set it either).
float orc_quantize_segment(const float* x, int32_t w, uint8_t* codes) {
    float amax = 0.0f;
    for (int32_t i = 0; i < w; ++i) {
        if (std::isfinite(x[i])) amax = std::max(amax, std::fabs(x[i]));
    }
    float inv = 448.0f / amax;  // f32 division, +inf when amax is 0 or tiny
    float scale;
    if (std::isinf(inv)) {       // the guard
        scale = 0.0f;
        inv = 0.0f;
    } else {
        scale = amax / 448.0f;
    }
    for (int32_t i = 0; i < w; ++i) {
        float q = x[i] * inv;    // one f32 multiply
        codes[i] = orc_encode(q);
    }
    return scale;
}

void orc_quantize_rows(const float* src, int64_t src_row_stride, int64_t n_rows,
                       int32_t kv_lora, int32_t rope, uint8_t* codes, float* scales,
                       const int64_t* dst_rows, int threads) {
    const int64_t D = static_cast<int64_t>(kv_lora) + rope;
    parallel_for(n_rows, threads, [&](int64_t i) {
        const float* x = src + i * src_row_stride;
        const int64_t d = dst_rows ? dst_rows[i] : i;
        uint8_t* c = codes + d * D;
        scales[2 * d + 0] = orc_quantize_segment(x, kv_lora, c);
        scales[2 * d + 1] = orc_quantize_segment(x + kv_lora, rope, c + kv_lora);
    });
}

}  // extern "C"

namespace {

// One output row of the absorbed decode: softmax over the visible tokens of
// s * (q . xhat_t), then the softmax-weighted sum of the Lc parts of xhat_t
// ([colibri#299] commit message, attention_rows item: absorbed score and
// context loops over the latent rows; the latent is both key and value).
// Row(t, j) returns xhat of visible token t, column j, as a double.
// num_splits > 1: split-T form -- per equal token range a partial (m, l, O),
// merged with log-sum-exp ([colibri#299] PR description, follow-up paragraph:
// split-T kernels).
template <class RowFn>
void attend_one(const double* q, int32_t D, int32_t kv_lora, double sigma,
                int64_t n_visible, int64_t seq_len, int32_t num_splits,
                RowFn row, double* out) {
    std::fill(out, out + kv_lora, 0.0);
    if (n_visible <= 0) return;
    std::vector<double> S(static_cast<size_t>(n_visible));
    for (int64_t t = 0; t < n_visible; ++t) {
        double acc = 0.0;
        for (int32_t j = 0; j < D; ++j) acc += q[j] * row(t, j);
        S[static_cast<size_t>(t)] = sigma * acc;
    }
    if (num_splits <= 1) {
        double m = -std::numeric_limits<double>::infinity();
        for (double s : S) m = std::max(m, s);
        double Z = 0.0;
        for (int64_t t = 0; t < n_visible; ++t) {
            double w = std::exp(S[static_cast<size_t>(t)] - m);
            Z += w;
            for (int32_t j = 0; j < kv_lora; ++j) out[j] += w * row(t, j);
        }
        for (int32_t j = 0; j < kv_lora; ++j) out[j] /= Z;
        return;
    }
    const int64_t chunk = (seq_len + num_splits - 1) / num_splits;
    std::vector<double> ms, ls;
    std::vector<std::vector<double>> Os;
    for (int32_t s = 0; s < num_splits; ++s) {
        int64_t b = static_cast<int64_t>(s) * chunk;
        int64_t e = std::min<int64_t>(n_visible, b + chunk);
        if (b >= e) continue;  // empty split contributes nothing
        double m = -std::numeric_limits<double>::infinity();
        for (int64_t t = b; t < e; ++t) m = std::max(m, S[static_cast<size_t>(t)]);
        double l = 0.0;
        std::vector<double> O(static_cast<size_t>(kv_lora), 0.0);
        for (int64_t t = b; t < e; ++t) {
            double w = std::exp(S[static_cast<size_t>(t)] - m);
            l += w;
            for (int32_t j = 0; j < kv_lora; ++j) O[static_cast<size_t>(j)] += w * row(t, j);
        }
        ms.push_back(m);
        ls.push_back(l);
        Os.push_back(std::move(O));
    }
    double M = -std::numeric_limits<double>::infinity();
    for (double m : ms) M = std::max(M, m);
    double L = 0.0;
    for (size_t k = 0; k < ms.size(); ++k) {
        double f = std::exp(ms[k] - M);
        L += f * ls[k];
        for (int32_t j = 0; j < kv_lora; ++j) out[j] += f * Os[k][static_cast<size_t>(j)];
    }
    for (int32_t j = 0; j < kv_lora; ++j) out[j] /= L;
}

bool bad_args(const void* q_lat, const void* q_rope, const void* rows,
              const int64_t* kv_start, const int32_t* kv_len, int32_t B, int32_t Q,
              int32_t H, int32_t kv_lora, int32_t rope, double* out) {
    return !q_lat || (rope > 0 && !q_rope) || !rows || !kv_start || !kv_len || !out ||
           B < 1 || Q < 1 || H < 1 || kv_lora < 1 || rope < 0;
}

// Shared driver: for every selected (b, i, h) build q in f64 and call
// attend_one with the row accessor made by make_row(b).
template <class MakeRow>
void run_attention(const uint16_t* q_lat, const uint16_t* q_rope,
                   const int32_t* kv_len, int32_t B, int32_t Q, int32_t H,
                   int32_t kv_lora, int32_t rope, float softmax_scale,
                   int32_t num_splits, const int64_t* sel, int64_t n_sel,
                   double* out, int threads, MakeRow make_row) {
    const int32_t D = kv_lora + rope;
    const int64_t n_items = sel ? n_sel : static_cast<int64_t>(B) * Q * H;
    const double sigma = static_cast<double>(softmax_scale);
    parallel_for(n_items, threads, [&](int64_t k) {
        const int64_t flat = sel ? sel[k] : k;  // (b*Q + i)*H + h
        const int64_t bi = flat / H;
        const int64_t i = bi % Q;
        const int64_t b = bi / Q;
        std::vector<double> q(static_cast<size_t>(D));
        const int64_t qoff = flat;
        for (int32_t j = 0; j < kv_lora; ++j)
            q[static_cast<size_t>(j)] = bf16_to_float(q_lat[qoff * kv_lora + j]);
        for (int32_t j = 0; j < rope; ++j)
            q[static_cast<size_t>(kv_lora + j)] = bf16_to_float(q_rope[qoff * rope + j]);
        const int64_t L = kv_len[b];
        const int64_t n_visible = std::min<int64_t>(L, L - (Q - 1) + i);
        attend_one(q.data(), D, kv_lora, sigma, n_visible, L, num_splits, make_row(b),
                   out + k * kv_lora);
    });
}

}  // namespace

extern "C" {

int orc_attention(const uint16_t* q_lat, const uint16_t* q_rope,
                  const uint8_t* codes, const float* scales,
                  const int64_t* kv_start, const int32_t* kv_len,
                  int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                  float softmax_scale, int32_t num_splits,
                  const int64_t* sel, int64_t n_sel, double* out, int threads) {
    if (bad_args(q_lat, q_rope, codes, kv_start, kv_len, B, Q, H, kv_lora, rope, out) ||
        !scales || (sel && n_sel < 0))
        return -1;
    const int64_t D = static_cast<int64_t>(kv_lora) + rope;
    const double* dec = tables().all;
    // xhat = decode(code) * (Lc scale for the first kv_lora columns, Rc scale
    // for the rest): [colibri#299] commit message -- the score and context
    // loops dequantize inline and apply the row scale.
    run_attention(q_lat, q_rope, kv_len, B, Q, H, kv_lora, rope, softmax_scale, num_splits,
                  sel, n_sel, out, threads, [&](int64_t b) {
                      const int64_t base = kv_start[b];
                      return [=](int64_t t, int32_t j) {
                          const int64_t r = base + t;
                          const double s = static_cast<double>(scales[2 * r + (j < kv_lora ? 0 : 1)]);
                          return dec[codes[r * D + j]] * s;
                      };
                  });
    return 0;
}

int orc_attention_f32rows(const uint16_t* q_lat, const uint16_t* q_rope,
                          const float* rows, int64_t row_stride,
                          const int64_t* kv_start, const int32_t* kv_len,
                          int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                          float softmax_scale, int32_t num_splits,
                          const int64_t* sel, int64_t n_sel, double* out, int threads) {
    if (bad_args(q_lat, q_rope, rows, kv_start, kv_len, B, Q, H, kv_lora, rope, out) ||
        row_stride < static_cast<int64_t>(kv_lora) + rope || (sel && n_sel < 0))
        return -1;
    run_attention(q_lat, q_rope, kv_len, B, Q, H, kv_lora, rope, softmax_scale, num_splits,
                  sel, n_sel, out, threads, [&](int64_t b) {
                      const int64_t base = kv_start[b];
                      return [=](int64_t t, int32_t j) {
                          return static_cast<double>(rows[(base + t) * row_stride + j]);
                      };
                  });
    return 0;
}

// [colibri#299] commit message, attention_rows item: the fresh row is
// normalised (Lc) and rotary-embedded (Rc) before it is quantized.  The
// forms follow the standard definitions stated in kv8_oracle.h: RMS
// normalisation with a weight, and rotation of interleaved pairs by position
// times a geometric frequency.
void orc_norm_rope_rows(const float* src, int64_t src_row_stride, int64_t n_rows,
                        int32_t kv_lora, int32_t rope, const float* norm_weight, float eps,
                        const int64_t* positions, float rope_theta, float* out, int threads) {
    const int64_t d = static_cast<int64_t>(kv_lora) + rope;
    std::vector<float> freq(static_cast<size_t>(rope / 2));
    for (int32_t i = 0; i < rope / 2; ++i)
        freq[static_cast<size_t>(i)] = static_cast<float>(
            std::pow(static_cast<double>(rope_theta), -2.0 * i / static_cast<double>(rope)));
    parallel_for(n_rows, threads, [&](int64_t r) {
        const float* x = src + r * src_row_stride;
        float* y = out + r * d;
        // Lc: y_j = w_j x_j / sqrt(mean x^2 + eps)
        double ss = 0.0;
        for (int32_t j = 0; j < kv_lora; ++j) ss += static_cast<double>(x[j]) * x[j];
        const double rms = std::sqrt(ss / kv_lora + static_cast<double>(eps));
        for (int32_t j = 0; j < kv_lora; ++j)
            y[j] = static_cast<float>(static_cast<double>(norm_weight[j]) * x[j] / rms);
        // Rc: pair (2i, 2i+1) rotated by a_i = fl32(fl32(pos) f_i)
        const float pos = static_cast<float>(positions[r]);
        for (int32_t i = 0; i < rope / 2; ++i) {
            const float a = pos * freq[static_cast<size_t>(i)];
            const double c = std::cos(static_cast<double>(a)), s = std::sin(static_cast<double>(a));
            const double x0 = x[kv_lora + 2 * i], x1 = x[kv_lora + 2 * i + 1];
            y[kv_lora + 2 * i] = static_cast<float>(x0 * c - x1 * s);
            y[kv_lora + 2 * i + 1] = static_cast<float>(x0 * s + x1 * c);
        }
    });
}

// [colibri#299] commit message, attention_rows item: the non-absorbed prefill
// dequantizes Lc (code value times the row's Lc scale) and multiplies it by the
// kv_b weight; Rc is read through the decode table.  The row scale is applied
// to each product here, as the dequantized staging row holds it.
void orc_project_rows(const uint8_t* codes, const float* scales, int64_t n_rows,
                      int32_t kv_lora, int32_t rope, const uint16_t* w_bf16, int32_t N,
                      double* out, double* rope_out, int threads) {
    const int64_t d = static_cast<int64_t>(kv_lora) + rope;
    std::vector<double> w(static_cast<size_t>(N) * kv_lora);
    for (size_t i = 0; i < w.size(); ++i) {
        const uint32_t bits = static_cast<uint32_t>(w_bf16[i]) << 16;
        float f;
        std::memcpy(&f, &bits, 4);
        w[i] = f;
    }
    const Tables& t = tables();
    parallel_for(n_rows, threads, [&](int64_t m) {
        const uint8_t* c = codes + m * d;
        std::vector<double> x(static_cast<size_t>(kv_lora));
        for (int32_t k = 0; k < kv_lora; ++k) x[static_cast<size_t>(k)] = t.all[c[k]] * scales[2 * m];
        for (int32_t n = 0; n < N; ++n) {
            const double* wn = w.data() + static_cast<size_t>(n) * kv_lora;
            double acc = 0.0;
            for (int32_t k = 0; k < kv_lora; ++k) acc += x[static_cast<size_t>(k)] * wn[k];
            out[m * N + n] = acc;
        }
        for (int32_t j = 0; j < rope; ++j) rope_out[m * rope + j] = t.all[c[kv_lora + j]] * scales[2 * m + 1];
    });
}

// Block-scaled variant (page "Phase 0 toward V4.1 on a 128 GB Mac: lossless
// mxfp8 residents and kill-test tooling", mxfp8 residents paragraph: e4m3
// bytes with a ue8m0 exponent per 32-wide group).  The exponent is found by
// counting: the smallest integer E with amax <= 448 * 2^E (compared exactly
// in f64), within the ue8m0 range.
static int mx_block_exponent(const float* x, int32_t w) {
    double amax = 0.0;
    for (int32_t i = 0; i < w; ++i)
        if (std::isfinite(x[i])) amax = std::max(amax, std::fabs(static_cast<double>(x[i])));
    int E = -127;
    while (E < 127 && amax > 448.0 * std::ldexp(1.0, E)) ++E;
    return E;
}

void orc_quantize_rows_mx(const float* src, int64_t src_row_stride, int64_t n_rows,
                          int32_t kv_lora, int32_t rope, uint8_t* codes, uint8_t* exps,
                          const int64_t* dst_rows, int threads) {
    const int32_t D = kv_lora + rope;
    const int32_t nb = D / 32;
    parallel_for(n_rows, threads, [&](int64_t i) {
        const float* x = src + i * src_row_stride;
        const int64_t d = dst_rows ? dst_rows[i] : i;
        for (int32_t b = 0; b < nb; ++b) {
            const float* xb = x + 32 * b;
            const int E = mx_block_exponent(xb, 32);
            exps[d * nb + b] = static_cast<uint8_t>(E + 127);
            for (int32_t j = 0; j < 32; ++j) {
                // x * 2^-E in f64 is exact; its f32 rounding only matters below
                // the smallest e4m3 step, where every value encodes to +-0
                const float q = static_cast<float>(std::ldexp(static_cast<double>(xb[j]), -E));
                codes[d * D + 32 * b + j] = orc_encode(q);
            }
        }
    });
}

int orc_attention_mx(const uint16_t* q_lat, const uint16_t* q_rope,
                     const uint8_t* codes, const uint8_t* exps,
                     const int64_t* kv_start, const int32_t* kv_len,
                     int32_t B, int32_t Q, int32_t H, int32_t kv_lora, int32_t rope,
                     float softmax_scale, int32_t num_splits,
                     const int64_t* sel, int64_t n_sel, double* out, int threads) {
    if (bad_args(q_lat, q_rope, codes, kv_start, kv_len, B, Q, H, kv_lora, rope, out) || !exps ||
        (sel && n_sel < 0) || (kv_lora + rope) % 32 != 0)
        return -1;
    const int64_t D = static_cast<int64_t>(kv_lora) + rope;
    const int64_t nb = D / 32;
    const double* dec = tables().all;
    run_attention(q_lat, q_rope, kv_len, B, Q, H, kv_lora, rope, softmax_scale, num_splits,
                  sel, n_sel, out, threads, [&](int64_t b) {
                      const int64_t base = kv_start[b];
                      return [=](int64_t t, int32_t j) {
                          const int64_t r = base + t;
                          return std::ldexp(dec[codes[r * D + j]], static_cast<int>(exps[r * nb + j / 32]) - 127);
                      };
                  });
    return 0;
}

int64_t orc_bytes_per_token_layer_mx(int32_t kv_lora, int32_t rope) {
    return static_cast<int64_t>(kv_lora) + rope + (static_cast<int64_t>(kv_lora) + rope) / 32;
}

int64_t orc_bytes_per_token_layer(int32_t kv_lora, int32_t rope) {
    return static_cast<int64_t>(kv_lora) + rope + 2 * static_cast<int64_t>(sizeof(float));
}

}  // extern "C"
