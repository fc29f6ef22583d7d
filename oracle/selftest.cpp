// Sanitizer self-test of the CPU oracle (test infrastructure only).  Built by
// oracle/build.py --selftest with -fsanitize=address,undefined; exercises the
// codec, the quantizer on special rows, the attention in all its modes, the
// producer step and the non-absorbed projection, so that an out-of-bounds
// access or undefined operation aborts the run.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kv8_oracle.h"

#define CHECK(c)                                                       \
    do {                                                               \
        if (!(c)) {                                                    \
            std::fprintf(stderr, "CHECK failed: %s (line %d)\n", #c, __LINE__); \
            std::exit(1);                                              \
        }                                                              \
    } while (0)

static uint16_t bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return static_cast<uint16_t>((u + 0x7FFF + ((u >> 16) & 1)) >> 16);
}

int main() {
    // codec round trip over every finite code
    for (int c = 0; c < 256; ++c) {
        if (c == 0x7F || c == 0xFF) continue;
        CHECK(orc_encode(static_cast<float>(orc_decode(static_cast<uint8_t>(c)))) == c);
    }
    CHECK(orc_encode(NAN) == 0 && orc_encode(INFINITY) == 0x7E && orc_encode(-INFINITY) == 0xFE);
    std::vector<uint8_t> sweep(1 << 20);
    orc_encode_bits_range(0x7F700000u, sweep.size(), sweep.data(), 4);

    // quantizer on special rows, scattered into a larger cache
    const int KL = 512, KR = 64, D = KL + KR, n = 9;
    std::vector<float> rows(static_cast<size_t>(n) * D);
    unsigned s = 12345;
    for (auto& v : rows) {
        s = s * 1103515245u + 12345u;
        v = static_cast<float>(static_cast<int>(s >> 8) % 2001 - 1000) / 250.0f;
    }
    for (int j = 0; j < D; ++j) rows[1 * D + j] = 0.0f;
    for (int j = 0; j < D; ++j) rows[2 * D + j] = 1e-40f;
    rows[3 * D + 5] = NAN;
    rows[4 * D + 7] = -INFINITY;
    for (int j = 0; j < D; ++j) rows[5 * D + j] = 1.3166e-36f;
    std::vector<uint8_t> codes(static_cast<size_t>(2 * n) * D, 0xAA);
    std::vector<float> scales(static_cast<size_t>(2 * n) * 2, -1.0f);
    std::vector<int64_t> dst(n);
    for (int i = 0; i < n; ++i) dst[i] = 2 * i + 1;
    orc_quantize_rows(rows.data(), D, n, KL, KR, codes.data(), scales.data(), dst.data(), 3);
    CHECK(scales[2 * 3 + 0] == 0.0f && scales[2 * 5 + 0] == 0.0f);  // rows 1, 2 guarded
    CHECK(scales[2 * 11 + 0] > 0.0f);                                // row 5 not guarded
    CHECK(codes[static_cast<size_t>(7) * D + 5] == 0);              // NaN -> 0
    CHECK(codes[static_cast<size_t>(9) * D + 7] == 0xFE);           // -inf saturates

    // attention: ragged, causal, split, selected rows, and the f32-row path
    const int B = 2, Q = 3, H = 2;
    int64_t kv_start[B] = {1, 9};
    int32_t kv_len[B] = {8, 2};
    std::vector<uint16_t> ql(static_cast<size_t>(B) * Q * H * KL), qr(static_cast<size_t>(B) * Q * H * KR);
    for (size_t i = 0; i < ql.size(); ++i) ql[i] = bf16(static_cast<float>((i * 7919) % 97) / 970.0f - 0.05f);
    for (size_t i = 0; i < qr.size(); ++i) qr[i] = bf16(static_cast<float>((i * 104729) % 89) / 890.0f - 0.05f);
    std::vector<double> o1(static_cast<size_t>(B) * Q * H * KL), o2(o1.size());
    CHECK(orc_attention(ql.data(), qr.data(), codes.data(), scales.data(), kv_start, kv_len, B, Q, H,
                        KL, KR, 1.0f / 24.0f, 1, nullptr, 0, o1.data(), 2) == 0);
    CHECK(orc_attention(ql.data(), qr.data(), codes.data(), scales.data(), kv_start, kv_len, B, Q, H,
                        KL, KR, 1.0f / 24.0f, 3, nullptr, 0, o2.data(), 2) == 0);
    for (size_t i = 0; i < o1.size(); ++i) CHECK(std::fabs(o1[i] - o2[i]) <= 1e-12 * (1 + std::fabs(o1[i])));
    int64_t sel[2] = {3, 11};
    std::vector<double> o3(2 * KL);
    CHECK(orc_attention(ql.data(), qr.data(), codes.data(), scales.data(), kv_start, kv_len, B, Q, H,
                        KL, KR, 1.0f / 24.0f, 1, sel, 2, o3.data(), 1) == 0);
    for (int j = 0; j < KL; ++j) CHECK(o3[j] == o1[3 * KL + j] && o3[KL + j] == o1[11 * KL + j]);
    int64_t f_start[1] = {0};
    int32_t f_len[1] = {n};
    std::vector<double> o4(static_cast<size_t>(Q) * H * KL);
    CHECK(orc_attention_f32rows(ql.data(), qr.data(), rows.data(), D, f_start, f_len, 1, Q, H, KL, KR,
                                1.0f / 24.0f, 2, nullptr, 0, o4.data(), 2) == 0);
    CHECK(orc_attention(nullptr, qr.data(), codes.data(), scales.data(), kv_start, kv_len, B, Q, H,
                        KL, KR, 1.0f, 1, nullptr, 0, o1.data(), 1) == -1);
    CHECK(orc_bytes_per_token_layer(KL, KR) == 584);

    // producer step: strided source rows, then the quantizer on its output
    const int64_t stride = D + 8;
    std::vector<float> src(static_cast<size_t>(n) * stride, 0.5f), y(static_cast<size_t>(n) * D);
    for (size_t i = 0; i < rows.size(); ++i) src[(i / D) * stride + i % D] = rows[i];
    std::vector<float> wnorm(KL);
    for (int j = 0; j < KL; ++j) wnorm[j] = 0.5f + static_cast<float>(j % 7) / 8.0f;
    std::vector<int64_t> pos(n);
    for (int i = 0; i < n; ++i) pos[i] = 1000 * i + 3;
    orc_norm_rope_rows(src.data(), stride, n, KL, KR, wnorm.data(), 1e-6f, pos.data(), 10000.0f,
                       y.data(), 3);
    CHECK(y[0] != 0.0f && std::isnan(y[static_cast<size_t>(3) * D + 5]));  // NaN propagates
    orc_quantize_rows(y.data(), D, n, KL, KR, codes.data(), scales.data(), nullptr, 2);

    // non-absorbed projection of the quantized rows by a bf16 weight
    const int N = 24;
    std::vector<uint16_t> wb(static_cast<size_t>(N) * KL);
    for (size_t i = 0; i < wb.size(); ++i) wb[i] = bf16(static_cast<float>((i * 31) % 13) / 13.0f - 0.5f);
    std::vector<double> po(static_cast<size_t>(n) * N), pr(static_cast<size_t>(n) * KR);
    orc_project_rows(codes.data(), scales.data(), n, KL, KR, wb.data(), N, po.data(), pr.data(), 3);
    CHECK(po[static_cast<size_t>(1) * N] == 0.0 && pr[static_cast<size_t>(1) * KR] == 0.0);  // zero row

    // block-scaled variant: the same special rows, scattered; attention over them
    const int NB = D / 32;
    std::vector<uint8_t> mcodes(static_cast<size_t>(2 * n) * D, 0xAA);
    std::vector<uint8_t> mexps(static_cast<size_t>(2 * n) * NB, 0xCD);
    orc_quantize_rows_mx(rows.data(), D, n, KL, KR, mcodes.data(), mexps.data(), dst.data(), 3);
    CHECK(mexps[static_cast<size_t>(3) * NB] == 0);                  // zero block: E = -127
    CHECK(mcodes[static_cast<size_t>(7) * D + 5] == 0);              // NaN -> 0
    CHECK(mcodes[static_cast<size_t>(9) * D + 7] == 0x7E + 0x80);    // -inf saturates
    std::vector<double> mout(static_cast<size_t>(2) * KL);
    const int64_t mstart[1] = {1};
    const int32_t mlen[1] = {2 * n - 1};
    CHECK(orc_attention_mx(ql.data(), qr.data(), mcodes.data(), mexps.data(), mstart, mlen, 1, 1, 2, KL, KR,
                           1.0f / 24.0f, 3, nullptr, 0, mout.data(), 2) == 0);
    for (double v : mout) CHECK(std::isfinite(v));
    CHECK(orc_bytes_per_token_layer_mx(KL, KR) == D + NB);

    std::printf("oracle selftest ok\n");
    return 0;
}
