// Host-side exercise of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: the codecs on many shapes and values, and
// every entry point's validation on good and bad arguments (fake, aligned
// device addresses; launches go to stubs). Exits non-zero on the first
// wrong result; the sanitizers abort on any memory or UB error.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <vector>

#include "qmv.h"

namespace qmv { extern int g_stub_launches; }

static int failures = 0;
#define EXPECT(cond, ...)                                      \
    do {                                                       \
        if (!(cond)) {                                         \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                      \
            fprintf(stderr, "\n");                             \
            ++failures;                                        \
        }                                                      \
    } while (0)

static uint64_t lcg = 0x2545F4914F6CDD1Dull;
static uint32_t rnd() {
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg >> 33);
}

static void codecs() {
    const int widths[] = {2, 3, 4, 5, 6, 8};
    for (int bits : widths) {
        for (int64_t K : {8, 16, 24, 32, 40, 64, 96, 200, 1056}) {
            if ((K * bits) % 8) continue;
            for (int64_t rows : {1, 3, 17}) {
                std::vector<uint8_t> codes((size_t)(rows * K)), back((size_t)(rows * K));
                for (auto& c : codes) c = (uint8_t)(rnd() & ((1u << bits) - 1u));
                const int64_t rb = qmv_packed_row_bytes(QMV_AFFINE, bits, K);
                EXPECT(rb == K * bits / 8, "row bytes %lld", (long long)rb);
                // exactly sized buffers, so ASan sees any overrun
                std::vector<uint8_t> packed((size_t)(rows * rb));
                EXPECT(qmv_pack_codes(codes.data(), rows, K, bits, packed.data()) == QMV_OK,
                       "pack bits=%d K=%lld", bits, (long long)K);
                EXPECT(qmv_unpack_codes(packed.data(), rows, K, bits, back.data()) == QMV_OK,
                       "unpack bits=%d", bits);
                EXPECT(codes == back, "round trip bits=%d K=%lld rows=%lld", bits, (long long)K,
                       (long long)rows);
            }
        }
        // a code that does not fit: rejected before anything is written
        std::vector<uint8_t> codes(32, 0), packed((size_t)(32 * bits / 8), 0xAB);
        codes[7] = (uint8_t)(1u << bits);
        if (bits < 8) {
            EXPECT(qmv_pack_codes(codes.data(), 1, 32, bits, packed.data()) ==
                       QMV_ERR_INVALID_ARGUMENT, "oversized code bits=%d", bits);
            for (uint8_t b : packed) EXPECT(b == 0xAB, "packed written on error");
        }
    }
    EXPECT(qmv_pack_codes(nullptr, 1, 32, 4, nullptr) == QMV_ERR_INVALID_ARGUMENT, "NULL pack");
    EXPECT(qmv_pack_codes(nullptr, 0, 32, 4, nullptr) == QMV_OK, "empty pack");
    EXPECT(qmv_pack_codes(nullptr, 1, 32, 7, nullptr) == QMV_ERR_UNSUPPORTED, "bits 7");
    EXPECT(qmv_packed_row_bytes(QMV_MXFP4, 4, 64) == 32, "mxfp4 row bytes");
    EXPECT(qmv_packed_row_bytes(QMV_MXFP8, 8, 64) == 64, "mxfp8 row bytes");
    EXPECT(qmv_packed_row_bytes((qmv_format_t)99, 4, 64) == -1, "bad format row bytes");

    // E4M3: every finite code decodes and re-encodes to itself; specials
    std::vector<float> v;
    for (int c = 0; c < 256; ++c) {
        const int e = (c >> 3) & 15, m = c & 7;
        if (e == 15 && m == 7) continue;
        float a = e == 0 ? std::ldexp((float)m, -9) : std::ldexp(1.0f + m / 8.0f, e - 7);
        v.push_back((c & 0x80) ? -a : a);
    }
    std::vector<uint8_t> out(v.size());
    EXPECT(qmv_encode_e4m3(v.data(), (int64_t)v.size(), out.data()) == QMV_OK, "encode");
    size_t i = 0;
    for (int c = 0; c < 256; ++c) {
        const int e = (c >> 3) & 15, m = c & 7;
        if (e == 15 && m == 7) continue;
        EXPECT(out[i] == c, "e4m3 code 0x%02x encodes to 0x%02x", c, out[i]);
        ++i;
    }
    const float sp[] = {NAN, INFINITY, -INFINITY, 1e9f, -500.0f, 449.0f, 1e-30f, -0.0f};
    const uint8_t want[] = {0x7F, 0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0x00, 0x80};
    uint8_t so[8];
    EXPECT(qmv_encode_e4m3(sp, 8, so) == QMV_OK, "encode specials");
    for (int j = 0; j < 8; ++j) EXPECT(so[j] == want[j], "special %d -> 0x%02x", j, so[j]);
    EXPECT(qmv_encode_e4m3(sp, -1, so) == QMV_ERR_INVALID_ARGUMENT, "n < 0");
}

#define D(a) reinterpret_cast<const void*>((uintptr_t)(a))
#define W8(a) reinterpret_cast<const uint8_t*>((uintptr_t)(a))
#define OUT(a) reinterpret_cast<void*>((uintptr_t)(a))

static void validation() {
    const int before = qmv::g_stub_launches;
    // good arguments reach the (stub) launch: QMV_ERR_HIP with its message
    EXPECT(qmv_affine(nullptr, QMV_BF16, 2, 4096, 300, D(0x10000), W8(0x100000), D(0x200000),
                      D(0x300000), 4, 64, OUT(0x400000)) == QMV_ERR_HIP, "affine good");
    EXPECT(strstr(qmv_last_error(), "stub launch") != nullptr, "msg %s", qmv_last_error());
    EXPECT(qmv_fp_mxfp4(nullptr, QMV_BF16, 1, 4096, 14336, D(0x10000), W8(0x100000),
                        W8(0x200000), OUT(0x400000)) == QMV_ERR_HIP, "mxfp4 good");
    EXPECT(qmv_fp_nvfp4(nullptr, QMV_F16, 8, 1024, 77, D(0x10000), W8(0x100000), W8(0x200000),
                        nullptr, OUT(0x400000)) == QMV_ERR_HIP, "nvfp4 good");
    EXPECT(qmv_fp_mxfp8(nullptr, QMV_F32, 3, 512, 5, D(0x10000), W8(0x100000), W8(0x200000),
                        OUT(0x400000)) == QMV_ERR_HIP, "mxfp8 good");
    EXPECT(qmv::g_stub_launches == before + 4, "launches %d", qmv::g_stub_launches - before);
    // bad arguments never launch
    const int mid = qmv::g_stub_launches;
    EXPECT(qmv_affine(nullptr, (qmv_dtype_t)7, 1, 64, 8, D(0x10000), W8(0x20000), D(0x30000),
                      D(0x40000), 4, 64, OUT(0x50000)) == QMV_ERR_INVALID_ARGUMENT, "dtype");
    EXPECT(qmv_affine(nullptr, QMV_BF16, 9, 64, 8, D(0x10000), W8(0x20000), D(0x30000),
                      D(0x40000), 4, 64, OUT(0x50000)) == QMV_ERR_UNSUPPORTED, "B=9");
    EXPECT(qmv_affine(nullptr, QMV_BF16, 1, 48, 8, D(0x10000), W8(0x20000), D(0x30000),
                      D(0x40000), 4, 32, OUT(0x50000)) == QMV_ERR_INVALID_ARGUMENT, "K=48");
    EXPECT(qmv_affine(nullptr, QMV_BF16, 1, 64, 8, D(0x10008), W8(0x20000), D(0x30000),
                      D(0x40000), 4, 64, OUT(0x50000)) == QMV_ERR_MISALIGNED, "x align");
    EXPECT(qmv_affine(nullptr, QMV_BF16, 1, 64, 8, D(0x10000), W8(0x20000), D(0x30000),
                      D(0x40000), 4, 64, OUT(0x10000)) == QMV_ERR_INVALID_ARGUMENT, "overlap");
    EXPECT(qmv_affine(nullptr, QMV_BF16, 1, ((int64_t)1 << 24) + 64, 8, D(0x10000),
                      W8(0x20000), D(0x30000), D(0x40000), 4, 64, OUT(0x50000)) ==
               QMV_ERR_UNSUPPORTED, "K too large");
    EXPECT(qmv_fp_block(nullptr, QMV_BF16, QMV_SB_F32, (qmv_element_t)99, 32, 1, 64, 8,
                        D(0x10000), W8(0x20000), D(0x30000), OUT(0x50000)) != QMV_OK &&
               qmv_fp_block(nullptr, QMV_BF16, QMV_SB_F32, (qmv_element_t)99, 32, 1, 64, 8,
                            D(0x10000), W8(0x20000), D(0x30000), OUT(0x50000)) != QMV_ERR_HIP,
           "bad element");
    EXPECT(qmv::g_stub_launches == mid, "a bad QMV call launched");
    // gather: one expert struct on the host, device pointers inside
    qmv_weights_t wt;
    memset(&wt, 0, sizeof wt);
    wt.format = QMV_MXFP4; wt.bits = 4; wt.group_size = 32;
    wt.n_experts = 8; wt.N = 96; wt.K = 1024;
    wt.w = W8(0x100000); wt.scales = D(0x200000);
    const uint32_t* lhs = reinterpret_cast<const uint32_t*>((uintptr_t)0x300000);
    const uint32_t* rhs = reinterpret_cast<const uint32_t*>((uintptr_t)0x310000);
    const int g0 = qmv::g_stub_launches;
    EXPECT(gather_qmv(nullptr, QMV_BF16, &wt, D(0x10000), 4, lhs, rhs, 12, OUT(0x400000)) ==
               QMV_ERR_HIP, "gather good");
    EXPECT(qmv::g_stub_launches > g0, "gather good did not launch");
    const int g1 = qmv::g_stub_launches;
    EXPECT(gather_qmv(nullptr, QMV_BF16, nullptr, D(0x10000), 4, lhs, rhs, 12, OUT(0x400000)) ==
               QMV_ERR_INVALID_ARGUMENT, "gather NULL weights");
    wt.n_experts = 1;
    EXPECT(qmv_qvm_noalloc(nullptr, QMV_BF16, &wt, 9, D(0x10000), OUT(0x400000)) ==
               QMV_ERR_UNSUPPORTED, "qvm B=9");
    qmv_weights_t big = wt;
    big.N = 32769; big.K = 16384;
    EXPECT(qmv_qvm_noalloc(nullptr, QMV_BF16, &big, 8, D(0x10000), OUT(0x10000000)) ==
               QMV_ERR_UNSUPPORTED, "qvm over the scratch");
    EXPECT(strstr(qmv_last_error(), "scratch") != nullptr, "scratch msg");
    EXPECT(qmv::g_stub_launches == g1, "a bad call launched");
    (void)mid;
    // long messages are truncated, never overrun
    for (int r = 0; r < 1000; ++r)
        qmv_affine(nullptr, QMV_BF16, 1, 64 + 32 * (r % 3), 8, D(0x10000), W8(0x20000),
                   D(0x30000), D(0x40000), 7, 64, OUT(0x50000));
    EXPECT(strlen(qmv_last_error()) > 0, "message kept");
}

int main() {
    codecs();
    validation();
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("HOST-SANITIZE-OK\n");
    return 0;
}
