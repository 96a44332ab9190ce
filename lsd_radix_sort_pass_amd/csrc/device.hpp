// device.hpp -- gfx950 device primitives of the LSD radix sort: ordered keys,
// digits, wave scans and the status words of the chained (decoupled
// look-back) digit scan.
//
// Page abbreviations used in comments:
//   [SS] Silicon Studio blog, "Radix sort を実装 & 測定してみた"
//   [WA] wandres.dev WebGPU guide, "Radix sort paralelo sobre el scan"
//   [PM] PMPP notes ch. 13, "정렬: 라딕스와 머지소트"
//   [OH] onikatahoshio, "高性能计算：GPU上的基数排序"
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rs {

constexpr int kWave = 64;  // CDNA wavefront width

// M30: 30-bit Morton codes computed from float32 points (xyz interleaved)
// where the keys are first read; stored and moved as uint32 codes.
// U16/I16/F16: 16-bit keys (F16: IEEE binary16 bit patterns).
enum class KeyKind : int { U32 = 0, I32 = 1, F32 = 2, U64 = 3, I64 = 4, F64 = 5, M30 = 6, U16 = 7, I16 = 8, F16 = 9 };

// Storage type of a key kind: 32-bit kinds move uint32_t patterns, 64-bit
// kinds uint64_t patterns ([SS] "符号付型、浮動小数点型に対する radix sort"
// notes that 64-bit types take the same procedure as 32-bit ones).
template <KeyKind KIND>
struct KeyBits {
    using type = uint32_t;
};
template <>
struct KeyBits<KeyKind::U64> {
    using type = uint64_t;
};
template <>
struct KeyBits<KeyKind::I64> {
    using type = uint64_t;
};
template <>
struct KeyBits<KeyKind::F64> {
    using type = uint64_t;
};
template <>
struct KeyBits<KeyKind::U16> {
    using type = uint16_t;
};
template <>
struct KeyBits<KeyKind::I16> {
    using type = uint16_t;
};
template <>
struct KeyBits<KeyKind::F16> {
    using type = uint16_t;
};
template <KeyKind KIND>
using key_t = typename KeyBits<KIND>::type;

// Order-preserving unsigned key.  Integer operations only: a key never goes
// through floating-point arithmetic, so NaN payloads and denormals are never
// touched (the sort moves the original bits; this value only feeds digits).
//   i32/i64: flip the sign bit ([WA] "Claves con signo y en coma flotante").
//   f32/f64: exponent field all ones (NaN or +-Inf) -> all ones, the maximum
//        ([SS] "符号付型、浮動小数点型に対する radix sort"); otherwise invert
//        every bit of a negative and only the sign bit of a non-negative.
template <KeyKind KIND>
__device__ __forceinline__ key_t<KIND> ordered_key(key_t<KIND> bits) {
    if constexpr (KIND == KeyKind::U32 || KIND == KeyKind::U64 || KIND == KeyKind::M30 || KIND == KeyKind::U16) {
        return bits;
    } else if constexpr (KIND == KeyKind::I16) {
        return static_cast<uint16_t>(bits ^ 0x8000u);
    } else if constexpr (KIND == KeyKind::F16) {
        const bool special = (bits & 0x7C00u) == 0x7C00u;
        const uint32_t flip = (bits & 0x8000u) ? 0xFFFFu : 0x8000u;
        return special ? static_cast<uint16_t>(0xFFFFu) : static_cast<uint16_t>(bits ^ flip);
    } else if constexpr (KIND == KeyKind::I32) {
        return bits ^ 0x80000000u;
    } else if constexpr (KIND == KeyKind::I64) {
        return bits ^ 0x8000000000000000ull;
    } else if constexpr (KIND == KeyKind::F32) {
        const bool special = (bits & 0x7F800000u) == 0x7F800000u;
        const uint32_t flip = static_cast<uint32_t>(static_cast<int32_t>(bits) >> 31) | 0x80000000u;
        return special ? 0xFFFFFFFFu : (bits ^ flip);
    } else {
        const bool special = (bits & 0x7FF0000000000000ull) == 0x7FF0000000000000ull;
        const uint64_t flip = static_cast<uint64_t>(static_cast<int64_t>(bits) >> 63) | 0x8000000000000000ull;
        return special ? ~0ull : (bits ^ flip);
    }
}

// 30-bit Morton code of a point: each coordinate quantised to 10 bits over
// the box [lo, lo + 1024 / scale), the three spread to every third bit, x
// highest.  The quantisation runs in single precision as written (one
// subtraction, one multiplication, each rounded; no contraction):
// q = 0 for NaN or t <= 0, 1023 for t >= 1023, else floor(t).
struct MortonBox {
    float lo[3];
    float scale[3];  // 1024 / (hi - lo), computed in single precision
};

// Branch-free form: max(t, 0) is 0 for NaN and t <= 0, min(., 1023) clamps,
// and truncation of a value in [0, 1023] is its floor.
__device__ __forceinline__ uint32_t quantize10(float p, float lo, float scale) {
#pragma clang fp contract(off)
    const float t = (p - lo) * scale;
    return static_cast<uint32_t>(__builtin_fminf(__builtin_fmaxf(t, 0.0f), 1023.0f));
}

// Bit i of a 10-bit value to bit 3i: four shift-or-mask steps that move
// the bits apart by 16, 8, 4 and 2 places.
__device__ __forceinline__ uint32_t spread3(uint32_t q) {
    q = (q | (q << 16)) & 0x030000FFu;
    q = (q | (q << 8)) & 0x0300F00Fu;
    q = (q | (q << 4)) & 0x030C30C3u;
    q = (q | (q << 2)) & 0x09249249u;
    return q;
}

__device__ __forceinline__ uint32_t morton30(float x, float y, float z, const MortonBox &b) {
    return (spread3(quantize10(x, b.lo[0], b.scale[0])) << 2) | (spread3(quantize10(y, b.lo[1], b.scale[1])) << 1) |
           spread3(quantize10(z, b.lo[2], b.scale[2]));
}

// Digit of one key for a pass: `mask` has the pass's digit width (the last
// pass of a bit range may be narrower than the radix).
template <KeyKind KIND>
__device__ __forceinline__ uint32_t digit_of(key_t<KIND> bits, uint32_t shift, uint32_t mask) {
    return static_cast<uint32_t>(ordered_key<KIND>(bits) >> shift) & mask;
}

// The same digit given its width (bits) instead of its mask: one bit-field
// extract for keys of up to 32 bits.
template <KeyKind KIND>
__device__ __forceinline__ uint32_t digit_field(key_t<KIND> bits, uint32_t shift, uint32_t width, uint32_t mask) {
    if constexpr (sizeof(key_t<KIND>) <= 4) {
        return __builtin_amdgcn_ubfe(static_cast<uint32_t>(ordered_key<KIND>(bits)), shift, width);
    } else {
        return static_cast<uint32_t>(ordered_key<KIND>(bits) >> shift) & mask;
    }
}

// A compile-time key kind as a value, to instantiate a generic lambda.
template <KeyKind K>
struct KindC {
    static constexpr KeyKind value = K;
};

// A compile-time bool as a value, to instantiate a generic lambda twice.
template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// Raw buffer resource (gfx9 family word 3: 32-bit data, no swizzle) over
// `bytes` bytes: buffer accesses at offsets >= bytes are dropped by hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}

// Raw buffer accesses of one key (32 or 64 bits) at a byte offset.
typedef uint32_t u32x2_t __attribute__((__vector_size__(8)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
template <class T>
__device__ __forceinline__ T buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (sizeof(T) == 2) {
        return static_cast<T>(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, 0));
    } else if constexpr (sizeof(T) == 4) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0);
    } else {
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, 0));
    }
}
template <class T>
__device__ __forceinline__ void buffer_store(T v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (sizeof(T) == 2) {
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(v), r, static_cast<int>(off), 0, 0);
    } else if constexpr (sizeof(T) == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, static_cast<int>(off), 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, static_cast<int>(off), 0, 0);
    }
}

// Inclusive prefix sum across the 64 lanes of a fully active wave, with DPP
// lane moves (no LDS traffic): a Hillis-Steele scan inside each row of 16
// lanes (row_shr 1, 2, 4, 8; lanes shifted in from outside the row read 0),
// then row 15's total broadcast into rows 1 and 3 and row 31's into rows 2
// and 3.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
    constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr1, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr2, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr4, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr8, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowBcast15, 0xA, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowBcast31, 0xC, 0xF, false));
    return x;
}

// Bitwise OR (AND = false) or AND (AND = true) of x over the 64 lanes of a
// fully active wave, returned to every lane: the same DPP steps as
// wave_inclusive_sum, with lanes that have no source lane taking the
// operation's identity (0 for OR, all ones for AND); lane 63 ends with the
// whole wave's result.
template <bool AND, int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t wave_bits_step(uint32_t x) {
    constexpr int kId = AND ? -1 : 0;
    const uint32_t y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(kId, static_cast<int>(x), CTRL, ROW_MASK, 0xF, false));
    return AND ? (x & y) : (x | y);
}
template <bool AND>
__device__ __forceinline__ uint32_t wave_bits(uint32_t x) {
    x = wave_bits_step<AND, 0x111, 0xF>(x);
    x = wave_bits_step<AND, 0x112, 0xF>(x);
    x = wave_bits_step<AND, 0x114, 0xF>(x);
    x = wave_bits_step<AND, 0x118, 0xF>(x);
    x = wave_bits_step<AND, 0x142, 0xA>(x);
    x = wave_bits_step<AND, 0x143, 0xC>(x);
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}
template <bool AND, class T>
__device__ __forceinline__ T wave_bits_of(T x) {
    if constexpr (sizeof(T) == 8) {
        return (static_cast<T>(wave_bits<AND>(static_cast<uint32_t>(x >> 32))) << 32) |
               wave_bits<AND>(static_cast<uint32_t>(x));
    } else {
        return static_cast<T>(wave_bits<AND>(static_cast<uint32_t>(x)));
    }
}

// The value of the next lane (lane + 1) of a fully active wave, by a DPP
// wave shift; the last lane gets 0.
__device__ __forceinline__ uint32_t next_lane(uint32_t x) {
    constexpr int kWaveShl1 = 0x130;
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kWaveShl1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint16_t next_lane(uint16_t x) {
    return static_cast<uint16_t>(next_lane(static_cast<uint32_t>(x)));
}
__device__ __forceinline__ uint64_t next_lane(uint64_t x) {
    return (static_cast<uint64_t>(next_lane(static_cast<uint32_t>(x >> 32))) << 32) | next_lane(static_cast<uint32_t>(x));
}

// The value lane `l` (a constant) holds, for every lane.
__device__ __forceinline__ uint32_t lane_value(uint32_t x, int l) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), l));
}
__device__ __forceinline__ uint16_t lane_value(uint16_t x, int l) {
    return static_cast<uint16_t>(lane_value(static_cast<uint32_t>(x), l));
}
__device__ __forceinline__ uint64_t lane_value(uint64_t x, int l) {
    return (static_cast<uint64_t>(lane_value(static_cast<uint32_t>(x >> 32), l)) << 32) |
           lane_value(static_cast<uint32_t>(x), l);
}

// Local rank by digit matching within a wave64 (the ballot/popcount ranker):
// the lanes holding the same digit as this lane are found with one ballot
// per digit bit, so every lane learns its peer set without any LDS traffic.
// The lowest lane of each peer set adds the set's size (times `unit`) to the
// wave's counter of that digit and passes the old value to its peers; a
// lane's rank is that value plus `unit` times the number of peers in lower
// lanes (mbcnt).  Within one instruction the adding lanes hold distinct
// digits, so no two adds share an address and the rank never depends on the
// order in which the LDS serves same-address atomics.  `valid` lanes take
// part; the others return an unspecified value.  Must be called with every
// lane of the wave active.
template <int RBITS>
__device__ __forceinline__ uint32_t match_rank(uint32_t digit, bool valid, uint32_t *wave_counters, uint32_t unit) {
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < RBITS; ++b) {
        const bool bit = (digit >> b) & 1u;
        const unsigned long long m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(peers >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(peers), 0u));
    uint32_t base = 0u;
    if (valid && below == 0u) {
        base = __hip_atomic_fetch_add(wave_counters + digit, static_cast<uint32_t>(__popcll(peers)) * unit,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    const int leader = valid ? __builtin_ctzll(peers) : 0;
    base = static_cast<uint32_t>(__shfl(static_cast<int>(base), leader, 64));
    return base + below * unit;
}

// ---------------------------------------------------------------------------
// Status words of the chained digit scan.  One word per (tile, digit): a
// 2-bit flag on top of the count it publishes.  The word carries all the
// information the reader needs, so relaxed device-scope atomic loads/stores
// suffice (no fences): a reader either sees EMPTY and retries, or a complete
// (flag, value) pair.  32-bit words hold counts below 2^30; 64-bit words are
// used for larger inputs.
// ---------------------------------------------------------------------------
constexpr uint32_t kFlagEmpty = 0u;
constexpr uint32_t kFlagAggregate = 1u;   // count of this tile only
constexpr uint32_t kFlagInclusive = 2u;   // count of this tile and all before
constexpr uint32_t kFlagError = 3u;       // a wait gave up; value meaningless

template <class T>
struct StatusWord;

template <>
struct StatusWord<uint32_t> {
    static constexpr int kShift = 30;
    static constexpr uint32_t kValueMask = (1u << 30) - 1u;
};

template <>
struct StatusWord<uint64_t> {
    static constexpr int kShift = 62;
    static constexpr uint64_t kValueMask = 0xFFFFFFFFull;
};

template <class T>
__device__ __forceinline__ T make_status(uint32_t flag, uint32_t value) {
    return (static_cast<T>(flag) << StatusWord<T>::kShift) | static_cast<T>(value);
}

template <class T>
__device__ __forceinline__ T status_load(T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A cheaper read of a status word that may be served by this XCD's L2 and
// so may return an OLDER value of the word.  A word only ever moves
// EMPTY -> AGGREGATE -> INCLUSIVE (or ERROR) within a pass, so an older value
// is still a true statement (an aggregate is a correct count, just less
// informative than the inclusive prefix it became); only EMPTY has to be
// re-read with status_load.
template <class T>
__device__ __forceinline__ T status_load_near(T *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Index of the accelerator complex die (XCD) this wave runs on; each XCD has
// its own L2.
__device__ __forceinline__ uint32_t xcd_id() {
    uint32_t v;
    __asm__ volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    return v & 0xFu;
}

template <class T>
__device__ __forceinline__ void status_store(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace rs
