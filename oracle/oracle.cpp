// oracle.cpp -- plain CPU reference for the stable LSD radix sort.
//
// TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
// benchmark's CPU-baseline leg, never by the product path.  Shares no code
// with the GPU library.  Build: g++ -std=c++17 -O2 -shared -fPIC (no
// -ffast-math: the float policy relies on std::isnan / std::isinf).
//
// Page abbreviations are those of oracle.h.
#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

namespace {

// One element as the sort moves it: the caller's original bit pattern and
// its payload.  The ordered key is recomputed from `bits` whenever a digit is
// needed, so nothing but the original pattern is ever stored or emitted.
template <class Bits>
struct ItemT {
    Bits bits;
    uint32_t val;
};
using Item = ItemT<uint32_t>;
using Item64 = ItemT<uint64_t>;

// [SS] "符号付型、浮動小数点型に対する radix sort": a float's bit pattern,
// read as an unsigned integer, orders like its value once the sign is
// handled; NaN and Inf are mapped to the maximum key (the page's stated
// choice: they sort last).
uint32_t float_key(uint32_t bits) {
    float value;
    std::memcpy(&value, &bits, sizeof value);
    if (std::isinf(value) || std::isnan(value)) {
        return 0xFFFFFFFFu;
    }
    if (bits & 0x80000000u) {
        return ~bits;  // negative: larger magnitude must come first
    }
    return bits ^ 0x80000000u;  // non-negative: above every negative
}

// [WA] "Claves con signo y en coma flotante": in two's complement the
// negatives have the sign bit set, so flipping that bit alone gives an
// unsigned key with the signed order.  (The int rule printed in [SS]
// inverts all bits of negatives, which orders -1 before -2; it is not used.)
uint32_t int_key(uint32_t bits) { return bits ^ 0x80000000u; }

uint32_t ordered_key(int kind, uint32_t bits) {
    switch (kind) {
        case ORACLE_KEY_U32: return bits;
        case ORACLE_KEY_I32: return int_key(bits);
        case ORACLE_KEY_F32: return float_key(bits);
        default: return 0u;
    }
}

bool valid_kind(int kind) {
    return kind == ORACLE_KEY_U32 || kind == ORACLE_KEY_I32 || kind == ORACLE_KEY_F32;
}

// 64-bit keys.  [SS] closes "符号付型、浮動小数点型に対する radix sort" by
// noting that 16- and 64-bit types follow the same procedure: the rules
// above with the sign in bit 63 and the double's exponent field.
uint64_t double_key(uint64_t bits) {
    double value;
    std::memcpy(&value, &bits, sizeof value);
    if (std::isinf(value) || std::isnan(value)) {
        return ~uint64_t{0};
    }
    if (bits >> 63) {
        return ~bits;
    }
    return bits ^ (uint64_t{1} << 63);
}

uint64_t int64_key(uint64_t bits) { return bits ^ (uint64_t{1} << 63); }

uint64_t ordered_key64(int kind, uint64_t bits) {
    switch (kind) {
        case ORACLE_KEY_U64: return bits;
        case ORACLE_KEY_I64: return int64_key(bits);
        case ORACLE_KEY_F64: return double_key(bits);
        default: return 0u;
    }
}

bool valid_kind64(int kind) {
    return kind == ORACLE_KEY_U64 || kind == ORACLE_KEY_I64 || kind == ORACLE_KEY_F64;
}

// One stable counting-sort pass ([WA] "Las tres fases de una pasada";
// [OH] "CPU上的基数排序"): count how many items fall in each bucket, turn the
// counts into bucket start positions with an exclusive prefix sum, then walk
// the input in index order and drop each item at the next free slot of its
// bucket.  Walking in index order is what makes the pass stable.
template <class It, class DigitFn>
void counting_pass(const It *in, It *out, size_t n, size_t buckets, DigitFn digit) {
    std::vector<size_t> count(buckets, 0);
    for (size_t i = 0; i < n; ++i) {
        count[digit(in[i])] += 1;
    }
    // Exclusive prefix sum, written as the serial recurrence of
    // [OH] "CPU上的扫描" shifted by one: start[d] = start[d-1] + count[d-1].
    std::vector<size_t> start(buckets, 0);
    for (size_t d = 1; d < buckets; ++d) {
        start[d] = start[d - 1] + count[d - 1];
    }
    for (size_t i = 0; i < n; ++i) {
        size_t d = digit(in[i]);
        out[start[d]] = in[i];
        start[d] += 1;
    }
}

bool valid_range(int begin_bit, int end_bit, int key_bits = 32) {
    return begin_bit >= 0 && end_bit <= key_bits && begin_bit <= end_bit;
}

template <class Bits>
int load_items(const Bits *keys_in, const uint32_t *vals_in, size_t n,
               std::vector<ItemT<Bits>> &items) {
    try {
        items.resize(n);
    } catch (const std::bad_alloc &) {
        return -2;
    }
    for (size_t i = 0; i < n; ++i) {
        items[i].bits = keys_in[i];
        items[i].val = vals_in ? vals_in[i] : 0u;
    }
    return 0;
}

template <class Bits>
void store_items(const std::vector<ItemT<Bits>> &items, Bits *keys_out, uint32_t *vals_out) {
    for (size_t i = 0; i < items.size(); ++i) {
        keys_out[i] = items[i].bits;
        if (vals_out) vals_out[i] = items[i].val;
    }
}

}  // namespace

extern "C" uint32_t oracle_ordered_key(int kind, uint32_t bits) {
    return ordered_key(kind, bits);
}

// LSD radix sort ([WA] "La idea y el requisito de estabilidad" and "Las tres
// fases de una pasada"): digits of radix_bits bits, least significant first,
// each sorted by one stable counting pass; the last digit is narrower when
// radix_bits does not divide end_bit - begin_bit.
extern "C" int oracle_lsd_sort(int kind, const uint32_t *keys_in, const uint32_t *vals_in,
                               size_t n, int begin_bit, int end_bit, int radix_bits,
                               uint32_t *keys_out, uint32_t *vals_out) {
    if (!valid_kind(kind) || !valid_range(begin_bit, end_bit)) return -1;
    if (radix_bits < 1 || radix_bits > 16) return -1;
    if (n > 0 && (!keys_in || !keys_out)) return -1;
    if (n > 0 && vals_in && !vals_out) return -1;

    std::vector<Item> a, b;
    int rc = load_items(keys_in, vals_in, n, a);
    if (rc) return rc;
    try {
        b.resize(n);
    } catch (const std::bad_alloc &) {
        return -2;
    }

    for (int shift = begin_bit; shift < end_bit; shift += radix_bits) {
        int width = end_bit - shift < radix_bits ? end_bit - shift : radix_bits;
        // 64-bit arithmetic so that a 32-bit-wide digit would not overflow.
        uint64_t mask = (uint64_t{1} << width) - 1;
        size_t buckets = size_t{1} << width;
        counting_pass(a.data(), b.data(), n, buckets, [&](const Item &it) {
            return static_cast<size_t>((uint64_t{ordered_key(kind, it.bits)} >> shift) & mask);
        });
        a.swap(b);
    }
    store_items(a, keys_out, vals_out);
    return 0;
}

// Bit-at-a-time sort with the two-bucket formula of [SS] "アルゴリズムの詳細":
// s_i = number of 0-bits strictly before i (an exclusive count), F = number of
// 0-bits in total; a 0 goes to s_i and a 1 to F + i - s_i (the ones before i
// number i - s_i and all come after the F zeros).  The page prints the second
// case as n - s_i + F in its display formula, but derives, and its code uses,
// F + i - s_i; the latter is the one that stays inside [0, n).
extern "C" int oracle_split_sort(int kind, const uint32_t *keys_in, const uint32_t *vals_in,
                                 size_t n, int begin_bit, int end_bit,
                                 uint32_t *keys_out, uint32_t *vals_out) {
    if (!valid_kind(kind) || !valid_range(begin_bit, end_bit)) return -1;
    if (n > 0 && (!keys_in || !keys_out)) return -1;
    if (n > 0 && vals_in && !vals_out) return -1;

    std::vector<Item> a, b;
    std::vector<size_t> zeros_before;
    int rc = load_items(keys_in, vals_in, n, a);
    if (rc) return rc;
    try {
        b.resize(n);
        zeros_before.resize(n);
    } catch (const std::bad_alloc &) {
        return -2;
    }

    for (int bit = begin_bit; bit < end_bit; ++bit) {
        size_t zeros = 0;
        for (size_t i = 0; i < n; ++i) {
            zeros_before[i] = zeros;
            if (((ordered_key(kind, a[i].bits) >> bit) & 1u) == 0u) zeros += 1;
        }
        const size_t F = zeros;
        for (size_t i = 0; i < n; ++i) {
            const size_t s = zeros_before[i];
            const bool one = ((ordered_key(kind, a[i].bits) >> bit) & 1u) != 0u;
            b[one ? F + i - s : s] = a[i];
        }
        a.swap(b);
    }
    store_items(a, keys_out, vals_out);
    return 0;
}

// One decimal-digit pass, as in the 170/045/075/... worked example of
// [WA] "La idea y el requisito de estabilidad": bucket = (x / 10^place) % 10.
extern "C" int oracle_decimal_pass(const uint32_t *in, size_t n, int place, uint32_t *out) {
    if (place < 0 || place > 9) return -1;
    if (n > 0 && (!in || !out)) return -1;
    std::vector<Item> a, b;
    int rc = load_items<uint32_t>(in, nullptr, n, a);
    if (rc) return rc;
    try {
        b.resize(n);
    } catch (const std::bad_alloc &) {
        return -2;
    }
    uint32_t divisor = 1;
    for (int p = 0; p < place; ++p) divisor *= 10u;
    counting_pass(a.data(), b.data(), n, 10, [&](const Item &it) {
        return static_cast<size_t>((it.bits / divisor) % 10u);
    });
    store_items(b, out, nullptr);
    return 0;
}

extern "C" uint64_t oracle_ordered_key64(int kind, uint64_t bits) {
    return ordered_key64(kind, bits);
}

// The LSD sort of oracle_lsd_sort for 64-bit keys: same passes, same
// counting pass, digits taken from the 64-bit ordered key.
extern "C" int oracle_lsd_sort64(int kind, const uint64_t *keys_in, const uint32_t *vals_in,
                                 size_t n, int begin_bit, int end_bit, int radix_bits,
                                 uint64_t *keys_out, uint32_t *vals_out) {
    if (!valid_kind64(kind) || !valid_range(begin_bit, end_bit, 64)) return -1;
    if (radix_bits < 1 || radix_bits > 16) return -1;
    if (n > 0 && (!keys_in || !keys_out)) return -1;
    if (n > 0 && vals_in && !vals_out) return -1;

    std::vector<Item64> a, b;
    int rc = load_items(keys_in, vals_in, n, a);
    if (rc) return rc;
    try {
        b.resize(n);
    } catch (const std::bad_alloc &) {
        return -2;
    }
    for (int shift = begin_bit; shift < end_bit; shift += radix_bits) {
        int width = end_bit - shift < radix_bits ? end_bit - shift : radix_bits;
        uint64_t mask = (uint64_t{1} << width) - 1;
        size_t buckets = size_t{1} << width;
        counting_pass(a.data(), b.data(), n, buckets, [&](const Item64 &it) {
            return static_cast<size_t>((ordered_key64(kind, it.bits) >> shift) & mask);
        });
        a.swap(b);
    }
    store_items(a, keys_out, vals_out);
    return 0;
}

// The one-bit two-bucket sort of oracle_split_sort for 64-bit keys.
extern "C" int oracle_split_sort64(int kind, const uint64_t *keys_in, const uint32_t *vals_in,
                                   size_t n, int begin_bit, int end_bit,
                                   uint64_t *keys_out, uint32_t *vals_out) {
    if (!valid_kind64(kind) || !valid_range(begin_bit, end_bit, 64)) return -1;
    if (n > 0 && (!keys_in || !keys_out)) return -1;
    if (n > 0 && vals_in && !vals_out) return -1;

    std::vector<Item64> a, b;
    std::vector<size_t> zeros_before;
    int rc = load_items(keys_in, vals_in, n, a);
    if (rc) return rc;
    try {
        b.resize(n);
        zeros_before.resize(n);
    } catch (const std::bad_alloc &) {
        return -2;
    }
    for (int bit = begin_bit; bit < end_bit; ++bit) {
        size_t zeros = 0;
        for (size_t i = 0; i < n; ++i) {
            zeros_before[i] = zeros;
            if (((ordered_key64(kind, a[i].bits) >> bit) & 1u) == 0u) zeros += 1;
        }
        const size_t F = zeros;
        for (size_t i = 0; i < n; ++i) {
            const size_t s = zeros_before[i];
            const bool one = ((ordered_key64(kind, a[i].bits) >> bit) & 1u) != 0u;
            b[one ? F + i - s : s] = a[i];
        }
        a.swap(b);
    }
    store_items(a, keys_out, vals_out);
    return 0;
}

// ---------------------------------------------------------------------------
// 30-bit Morton codes of 3-D points, the key an LBVH build sorts ([OH]
// "高性能计算：GPU上的基数排序": the sort is the step of a GPU BVH build; the
// page links its Morton-code post, whose text is not among the sources).
// Reading taken: each axis is quantised to 10 bits over the box [lo, hi),
// and the code interleaves them with x in the highest bit of each triple.
// The quantisation is carried out in IEEE single precision, step by step:
//   s = 1024 / (hi - lo);  t = (p - lo) * s;
//   q = 0 if t is NaN or t <= 0, 1023 if t >= 1023, else floor(t).
// ---------------------------------------------------------------------------
namespace {

uint32_t quantize10(float p, float lo, float s) {
    const float t = (p - lo) * s;
    if (!(t > 0.0f)) return 0u;
    if (t >= 1023.0f) return 1023u;
    return static_cast<uint32_t>(t);  // t in (0, 1023): truncation is floor
}

// Bit i of q moves to bit 3i.
uint32_t spread_bits3(uint32_t q) {
    uint32_t out = 0u;
    for (int i = 0; i < 10; ++i) out |= ((q >> i) & 1u) << (3 * i);
    return out;
}

}  // namespace

extern "C" float oracle_morton_scale(float lo, float hi) { return 1024.0f / (hi - lo); }

extern "C" int oracle_morton30(const float *xyz, size_t n, const float *lo, const float *hi, uint32_t *codes) {
    if (n > 0 && (!xyz || !codes)) return -1;
    if (!lo || !hi) return -1;
    float s[3];
    for (int a = 0; a < 3; ++a) {
        if (!std::isfinite(lo[a]) || !std::isfinite(hi[a]) || !(hi[a] > lo[a])) return -1;
        if (!std::isfinite(hi[a] - lo[a])) return -1;  // width overflows single precision
        s[a] = oracle_morton_scale(lo[a], hi[a]);
        if (!std::isfinite(s[a]) || !(s[a] > 0.0f)) return -1;
    }
    for (size_t i = 0; i < n; ++i) {
        const uint32_t qx = quantize10(xyz[3 * i + 0], lo[0], s[0]);
        const uint32_t qy = quantize10(xyz[3 * i + 1], lo[1], s[1]);
        const uint32_t qz = quantize10(xyz[3 * i + 2], lo[2], s[2]);
        codes[i] = (spread_bits3(qx) << 2) | (spread_bits3(qy) << 1) | spread_bits3(qz);
    }
    return 0;
}

// ---------------------------------------------------------------------------
// Every key width with 32- or 64-bit values.  [SS] closes "符号付型、浮動小数点
// 型に対する radix sort" by noting that 16- and 64-bit types follow the same
// procedure; the 16-bit kinds take the rules above with the sign in bit 15
// and IEEE binary16's exponent field.  The half is decoded to its value so
// that the NaN/Inf test is std::isnan / std::isinf on a number, as for f32.
// ---------------------------------------------------------------------------
namespace {

double half_value(uint16_t h) {
    const int sign = h >> 15;
    const int exponent = (h >> 10) & 0x1F;
    const int mantissa = h & 0x3FF;
    double v;
    if (exponent == 0x1F) {
        v = mantissa ? std::nan("") : INFINITY;
    } else if (exponent == 0) {
        v = std::ldexp(static_cast<double>(mantissa), -24);  // subnormal: m * 2^-24
    } else {
        v = std::ldexp(static_cast<double>(mantissa + 1024), exponent - 25);  // (1 + m/1024) * 2^(e-15)
    }
    return sign ? -v : v;
}

uint16_t half_key(uint16_t bits) {
    const double value = half_value(bits);
    if (std::isinf(value) || std::isnan(value)) return 0xFFFFu;
    if (bits & 0x8000u) return static_cast<uint16_t>(~bits);
    return static_cast<uint16_t>(bits ^ 0x8000u);
}

int key_bits_of(int kind) {
    switch (kind) {
        case ORACLE_KEY_U16: case ORACLE_KEY_I16: case ORACLE_KEY_F16: return 16;
        case ORACLE_KEY_U32: case ORACLE_KEY_I32: case ORACLE_KEY_F32: return 32;
        case ORACLE_KEY_U64: case ORACLE_KEY_I64: case ORACLE_KEY_F64: return 64;
        default: return 0;
    }
}

uint64_t ordered_key_any(int kind, uint64_t bits) {
    switch (kind) {
        case ORACLE_KEY_U16: return bits & 0xFFFFu;
        case ORACLE_KEY_I16: return (bits & 0xFFFFu) ^ 0x8000u;
        case ORACLE_KEY_F16: return half_key(static_cast<uint16_t>(bits));
        case ORACLE_KEY_U32: case ORACLE_KEY_I32: case ORACLE_KEY_F32:
            return ordered_key(kind, static_cast<uint32_t>(bits));
        default: return ordered_key64(kind, bits);
    }
}

template <class Bits, class Val>
struct Elem {
    Bits bits;
    Val val;
};

template <class Bits, class Val>
int sort_any(int kind, const void *keys_in, const void *vals_in, size_t n, int begin_bit, int end_bit,
             int radix_bits, void *keys_out, void *vals_out) {
    using E = Elem<Bits, Val>;
    std::vector<E> a, b;
    std::vector<size_t> zeros_before;
    try {
        a.resize(n);
        b.resize(n);
        if (radix_bits == 0) zeros_before.resize(n);
    } catch (const std::bad_alloc &) {
        return -2;
    }
    const Bits *kin = static_cast<const Bits *>(keys_in);
    const Val *vin = static_cast<const Val *>(vals_in);
    for (size_t i = 0; i < n; ++i) {
        a[i].bits = kin[i];
        a[i].val = vin ? vin[i] : Val(0);
    }
    auto key = [&](const E &e) { return ordered_key_any(kind, static_cast<uint64_t>(e.bits)); };
    if (radix_bits > 0) {
        // Counting-sort passes, as in oracle_lsd_sort.
        for (int shift = begin_bit; shift < end_bit; shift += radix_bits) {
            const int width = end_bit - shift < radix_bits ? end_bit - shift : radix_bits;
            const uint64_t mask = (uint64_t{1} << width) - 1;
            counting_pass(a.data(), b.data(), n, size_t{1} << width,
                          [&](const E &e) { return static_cast<size_t>((key(e) >> shift) & mask); });
            a.swap(b);
        }
    } else {
        // One-bit two-bucket splits, as in oracle_split_sort.
        for (int bit = begin_bit; bit < end_bit; ++bit) {
            size_t zeros = 0;
            for (size_t i = 0; i < n; ++i) {
                zeros_before[i] = zeros;
                if (((key(a[i]) >> bit) & 1u) == 0u) zeros += 1;
            }
            const size_t F = zeros;
            for (size_t i = 0; i < n; ++i) {
                const size_t s = zeros_before[i];
                const bool one = ((key(a[i]) >> bit) & 1u) != 0u;
                b[one ? F + i - s : s] = a[i];
            }
            a.swap(b);
        }
    }
    Bits *kout = static_cast<Bits *>(keys_out);
    Val *vout = static_cast<Val *>(vals_out);
    for (size_t i = 0; i < n; ++i) {
        kout[i] = a[i].bits;
        if (vout) vout[i] = a[i].val;
    }
    return 0;
}

template <class Bits>
int sort_any_vals(int kind, const void *keys_in, const void *vals_in, int val_bytes, size_t n, int begin_bit,
                  int end_bit, int radix_bits, void *keys_out, void *vals_out) {
    if (val_bytes == 8) return sort_any<Bits, uint64_t>(kind, keys_in, vals_in, n, begin_bit, end_bit, radix_bits, keys_out, vals_out);
    return sort_any<Bits, uint32_t>(kind, keys_in, vals_in, n, begin_bit, end_bit, radix_bits, keys_out, vals_out);
}

int sort_dispatch(int kind, const void *keys_in, const void *vals_in, int val_bytes, size_t n, int begin_bit,
                  int end_bit, int radix_bits, void *keys_out, void *vals_out) {
    const int kbits = key_bits_of(kind);
    if (kbits == 0 || !valid_range(begin_bit, end_bit, kbits)) return -1;
    if (radix_bits < 0 || radix_bits > 16) return -1;
    if (vals_in && val_bytes != 4 && val_bytes != 8) return -1;
    if (n > 0 && (!keys_in || !keys_out)) return -1;
    if (n > 0 && vals_in && !vals_out) return -1;
    if (kbits == 16) return sort_any_vals<uint16_t>(kind, keys_in, vals_in, val_bytes, n, begin_bit, end_bit, radix_bits, keys_out, vals_out);
    if (kbits == 32) return sort_any_vals<uint32_t>(kind, keys_in, vals_in, val_bytes, n, begin_bit, end_bit, radix_bits, keys_out, vals_out);
    return sort_any_vals<uint64_t>(kind, keys_in, vals_in, val_bytes, n, begin_bit, end_bit, radix_bits, keys_out, vals_out);
}

}  // namespace

extern "C" uint64_t oracle_ordered_key_any(int kind, uint64_t bits) {
    return key_bits_of(kind) ? ordered_key_any(kind, bits) : 0u;
}

extern "C" int oracle_lsd_sort_any(int kind, const void *keys_in, const void *vals_in, int val_bytes, size_t n,
                                   int begin_bit, int end_bit, int radix_bits, void *keys_out, void *vals_out) {
    if (radix_bits < 1) return -1;
    return sort_dispatch(kind, keys_in, vals_in, val_bytes, n, begin_bit, end_bit, radix_bits, keys_out, vals_out);
}

extern "C" int oracle_split_sort_any(int kind, const void *keys_in, const void *vals_in, int val_bytes, size_t n,
                                     int begin_bit, int end_bit, void *keys_out, void *vals_out) {
    return sort_dispatch(kind, keys_in, vals_in, val_bytes, n, begin_bit, end_bit, 0, keys_out, vals_out);
}

// CPU context for the benchmark (not part of the oracle's checks): the
// standard library's comparison sorts on the native order of 32-bit
// integers, as [SS] "測定" timed std::sort beside its radix sorts.
extern "C" int oracle_std_sort(int kind, void *keys, size_t n, int stable) {
    if (n > 0 && !keys) return -1;
    if (kind == ORACLE_KEY_U32) {
        uint32_t *k = static_cast<uint32_t *>(keys);
        if (stable) std::stable_sort(k, k + n); else std::sort(k, k + n);
        return 0;
    }
    if (kind == ORACLE_KEY_I32) {
        int32_t *k = static_cast<int32_t *>(keys);
        if (stable) std::stable_sort(k, k + n); else std::sort(k, k + n);
        return 0;
    }
    return -1;
}
