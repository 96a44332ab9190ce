// sanitize_check.cpp -- drives every oracle entry point under AddressSanitizer
// and UndefinedBehaviorSanitizer (TEST INFRASTRUCTURE ONLY).
//
// Built together with oracle.cpp into one executable:
//     g++ -std=c++17 -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=all
//         -ffp-contract=off oracle.cpp sanitize_check.cpp -o <exe>
// and run by tests/test_oracle_sanitized.py.  Every call gets buffers of
// exactly the size the header documents, so a read or write past them, a
// use of freed memory, an out-of-range shift or a signed overflow aborts the
// run.  The outputs are also checked against each other: the counting-sort
// LSD and the one-bit split sort are independent algorithms of the same
// stable sort, so they must agree byte for byte.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "oracle.h"

namespace {

int g_failures = 0;

void fail(const char *what, size_t n, int b, int e) {
    std::fprintf(stderr, "mismatch: %s n=%zu bits=[%d,%d)\n", what, n, b, e);
    ++g_failures;
}

// Edge values mixed with random words: zeros, all ones, sign bits, NaN and
// infinity patterns of every width, denormals.
template <class T>
std::vector<T> make_keys(std::mt19937_64 &rng, size_t n) {
    static const uint64_t edges[] = {0x0ull,
                                     ~0ull,
                                     0x8000000000000000ull,
                                     0x7FFFFFFFFFFFFFFFull,
                                     0x7FF0000000000000ull,
                                     0xFFF8000000000001ull,
                                     0x000000007F800000ull,
                                     0x00000000FFC00000ull,
                                     0x0000000080000000ull,
                                     0x0000000000000001ull,
                                     0x0000000000007C00ull,
                                     0x000000000000FE00ull,
                                     0x0000000000008000ull};
    std::vector<T> k(n);
    for (size_t i = 0; i < n; ++i) {
        const uint64_t r = rng();
        k[i] = static_cast<T>((r & 3) == 0 ? edges[(r >> 2) % (sizeof(edges) / sizeof(edges[0]))] : (r >> 8));
    }
    return k;
}

std::vector<unsigned char> make_vals(std::mt19937_64 &rng, size_t n, int vb) {
    std::vector<unsigned char> v(n * static_cast<size_t>(vb));
    for (auto &x : v) x = static_cast<unsigned char>(rng());
    return v;
}

void check_any(std::mt19937_64 &rng, int kind, int kb, int vb, size_t n) {
    const int width = 8 * kb;
    const int b = static_cast<int>(rng() % (width + 1));
    const int e = b + static_cast<int>(rng() % (width - b + 1));
    const int radix = 1 + static_cast<int>(rng() % 16);
    std::vector<unsigned char> keys(n * kb);
    {
        std::vector<uint64_t> w = make_keys<uint64_t>(rng, n);
        for (size_t i = 0; i < n; ++i) std::memcpy(&keys[i * kb], &w[i], static_cast<size_t>(kb));
    }
    std::vector<unsigned char> vals = vb ? make_vals(rng, n, vb) : std::vector<unsigned char>();
    std::vector<unsigned char> ka(n * kb), kc(n * kb), va(n * vb), vc(n * vb);
    const void *vin = vb ? vals.data() : nullptr;
    if (oracle_lsd_sort_any(kind, keys.data(), vin, vb, n, b, e, radix, ka.data(), vb ? va.data() : nullptr) != 0 ||
        oracle_split_sort_any(kind, keys.data(), vin, vb, n, b, e, kc.data(), vb ? vc.data() : nullptr) != 0) {
        fail("oracle_*_sort_any returned an error", n, b, e);
        return;
    }
    if (ka != kc || va != vc) fail("oracle_lsd_sort_any vs oracle_split_sort_any", n, b, e);
}

void check_32(std::mt19937_64 &rng, int kind, bool pairs, size_t n) {
    const int b = static_cast<int>(rng() % 33);
    const int e = b + static_cast<int>(rng() % (33 - b));
    const int radix = 1 + static_cast<int>(rng() % 16);
    std::vector<uint32_t> keys = make_keys<uint32_t>(rng, n);
    std::vector<uint32_t> vals(n);
    for (size_t i = 0; i < n; ++i) vals[i] = static_cast<uint32_t>(i);
    std::vector<uint32_t> ka(n), kc(n), va(n), vc(n);
    const uint32_t *vin = pairs ? vals.data() : nullptr;
    if (oracle_lsd_sort(kind, keys.data(), vin, n, b, e, radix, ka.data(), pairs ? va.data() : nullptr) != 0 ||
        oracle_split_sort(kind, keys.data(), vin, n, b, e, kc.data(), pairs ? vc.data() : nullptr) != 0) {
        fail("oracle_lsd_sort / oracle_split_sort returned an error", n, b, e);
        return;
    }
    if (ka != kc || (pairs && va != vc)) fail("oracle_lsd_sort vs oracle_split_sort", n, b, e);
    for (size_t i = 0; i < n; ++i) (void)oracle_ordered_key(kind, keys[i]);
}

void check_64(std::mt19937_64 &rng, int kind, bool pairs, size_t n) {
    const int b = static_cast<int>(rng() % 65);
    const int e = b + static_cast<int>(rng() % (65 - b));
    const int radix = 1 + static_cast<int>(rng() % 16);
    std::vector<uint64_t> keys = make_keys<uint64_t>(rng, n);
    std::vector<uint32_t> vals(n);
    for (size_t i = 0; i < n; ++i) vals[i] = static_cast<uint32_t>(i);
    std::vector<uint64_t> ka(n), kc(n);
    std::vector<uint32_t> va(n), vc(n);
    const uint32_t *vin = pairs ? vals.data() : nullptr;
    if (oracle_lsd_sort64(kind, keys.data(), vin, n, b, e, radix, ka.data(), pairs ? va.data() : nullptr) != 0 ||
        oracle_split_sort64(kind, keys.data(), vin, n, b, e, kc.data(), pairs ? vc.data() : nullptr) != 0) {
        fail("oracle_lsd_sort64 / oracle_split_sort64 returned an error", n, b, e);
        return;
    }
    if (ka != kc || (pairs && va != vc)) fail("oracle_lsd_sort64 vs oracle_split_sort64", n, b, e);
    for (size_t i = 0; i < n; ++i) (void)oracle_ordered_key64(kind, keys[i]);
}

void check_decimal_and_morton(std::mt19937_64 &rng, size_t n) {
    std::vector<uint32_t> in(n), out(n);
    for (auto &x : in) x = static_cast<uint32_t>(rng());
    for (int place = 0; place <= 9; ++place) {
        if (oracle_decimal_pass(in.data(), n, place, out.data()) != 0) fail("oracle_decimal_pass", n, place, place);
    }
    std::vector<float> xyz(3 * n);
    std::uniform_real_distribution<float> u(-0.25f, 1.25f);
    for (auto &c : xyz) c = u(rng);
    if (n > 2) {
        xyz[0] = std::numeric_limits<float>::quiet_NaN();
        xyz[4] = std::numeric_limits<float>::infinity();
        xyz[8] = -std::numeric_limits<float>::infinity();
    }
    const float lo[3] = {0.0f, -1.0f, 0.125f}, hi[3] = {1.0f, 3.0f, 0.875f};
    std::vector<uint32_t> codes(n);
    if (oracle_morton30(xyz.data(), n, lo, hi, codes.data()) != 0) fail("oracle_morton30", n, 0, 30);
    for (uint32_t c : codes) {
        if (c >= (1u << 30)) fail("oracle_morton30 code above 30 bits", n, 0, 30);
    }
    (void)oracle_morton_scale(-3.0e38f, 3.0e38f);
}

}  // namespace

int main(int argc, char **argv) {
    const unsigned seed = argc > 1 ? static_cast<unsigned>(std::strtoul(argv[1], nullptr, 10)) : 1u;
    std::mt19937_64 rng(seed);
    const size_t sizes[] = {0, 1, 2, 3, 7, 64, 255, 256, 257, 1000, 4097};
    for (size_t n : sizes) {
        for (int rep = 0; rep < 3; ++rep) {
            for (int kind = ORACLE_KEY_U32; kind <= ORACLE_KEY_F32; ++kind) {
                check_32(rng, kind, false, n);
                check_32(rng, kind, true, n);
            }
            for (int kind = ORACLE_KEY_U64; kind <= ORACLE_KEY_F64; ++kind) {
                check_64(rng, kind, false, n);
                check_64(rng, kind, true, n);
            }
            const int kinds_any[][2] = {{ORACLE_KEY_U16, 2}, {ORACLE_KEY_I16, 2}, {ORACLE_KEY_F16, 2},
                                        {ORACLE_KEY_U32, 4}, {ORACLE_KEY_F32, 4}, {ORACLE_KEY_I64, 8},
                                        {ORACLE_KEY_F64, 8}};
            for (const auto &ka : kinds_any) {
                for (int vb : {0, 4, 8}) check_any(rng, ka[0], ka[1], vb, n);
            }
            check_decimal_and_morton(rng, n);
        }
    }
    // Invalid arguments must be rejected without touching the buffers.
    uint32_t dummy = 0;
    if (oracle_lsd_sort(ORACLE_KEY_U32, &dummy, nullptr, 1, 0, 33, 8, &dummy, nullptr) != -1) fail("bad bits", 1, 0, 33);
    if (oracle_lsd_sort(ORACLE_KEY_U32, &dummy, nullptr, 1, 0, 32, 17, &dummy, nullptr) != -1) fail("bad radix", 1, 0, 32);
    if (oracle_lsd_sort(99, &dummy, nullptr, 1, 0, 32, 8, &dummy, nullptr) != -1) fail("bad kind", 1, 0, 32);
    if (oracle_decimal_pass(&dummy, 1, 10, &dummy) != -1) fail("bad place", 1, 10, 10);
    if (g_failures != 0) {
        std::fprintf(stderr, "%d failure(s)\n", g_failures);
        return 1;
    }
    std::printf("sanitize_check ok (seed %u)\n", seed);
    return 0;
}
