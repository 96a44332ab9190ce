// kernels.hpp -- gfx950 kernels of the stable LSD radix sort.
//
// One sort = fill (zero the scan state) -> all-pass digit histogram (one read
// of the keys) -> per-pass starting offsets -> one fused rank-and-scatter
// kernel per digit pass.  Page abbreviations as in device.hpp.
#pragma once

#include "device.hpp"

namespace rs {

// ---------------------------------------------------------------------------
// Zero fill and copy (plain streaming kernels).
// ---------------------------------------------------------------------------

// Zero `n16` 16-byte words at a 16-byte-aligned address.
__global__ void fill_zero_kernel(uint4 *p, size_t n16) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
        p[i] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// Copy n 32-bit words (any 4-byte alignment).
__global__ void copy_u32_kernel(const uint32_t *__restrict__ in, uint32_t *__restrict__ out, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        out[i] = in[i];
    }
}

// Copy n 16-bit halves (16-bit keys whose buffers are not 4-byte aligned,
// or an odd count).
__global__ void copy_u16_kernel(const uint16_t *__restrict__ in, uint16_t *__restrict__ out, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        out[i] = in[i];
    }
}

// Copy n4 16-byte words (both pointers 16-byte aligned).  Copies run one
// 1024-thread workgroup per compute unit, each thread with kCopyUnroll
// 16-byte words in flight per step.  Measured on MI355X, 2^28 words each
// way: 256-thread blocks, up to eight per compute unit, four words in
// flight 408 us, one word 442 us; 1024-thread blocks, one per compute unit,
// one word 375-379 us (two per compute unit 429 us).  The pass kernel's
// copy of already-sorted keys (the same shape) went from 431 us with four
// words in flight to 362 us with one (eight: 510 us, sixteen: 582 us).
constexpr int kCopyBlock = 1024;
constexpr int kCopyUnroll = 1;
__global__ __launch_bounds__(kCopyBlock) void copy_u128_kernel(const uint4 *__restrict__ in, uint4 *__restrict__ out,
                                                               size_t n4) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kCopyBlock * kCopyUnroll;
    for (size_t base = static_cast<size_t>(blockIdx.x) * kCopyBlock * kCopyUnroll + threadIdx.x; base < n4;
         base += stride) {
        uint4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t i = base + static_cast<size_t>(u) * kCopyBlock;
            if (i < n4) v[u] = in[i];
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const size_t i = base + static_cast<size_t>(u) * kCopyBlock;
            if (i < n4) out[i] = v[u];
        }
    }
}

// ---------------------------------------------------------------------------
// Segments.
//
// The input of every pass is cut into kSegments contiguous key ranges, one
// per XCD (each XCD has its own L2).  A workgroup takes its tiles from the
// segment of the XCD it runs on, so the chained scan between consecutive
// tiles of a segment mostly stays inside one L2; every segment has its own
// chain, started from offsets known before the pass runs.
//
// Those offsets need each segment's digit histogram, taken in the single
// histogram read of the ORIGINAL keys, so segment membership must be a
// function of the key, not of where the key sits at that pass:
//   pass 0:  the input is the original array; segment s = the s-th
//            eighth of its tiles (by position);
//   pass p:  the input is sorted by the digit of pass p-1, so the keys whose
//            pass-(p-1) digit has top bits s (digits [32s, 32s+32) for 8-bit
//            digits) form one contiguous range -- that range is segment s.
// ---------------------------------------------------------------------------
#ifndef RS_SEGMENT_BITS
#define RS_SEGMENT_BITS 3
#endif
constexpr int kSegmentBits = RS_SEGMENT_BITS;
constexpr int kSegments = 1 << kSegmentBits;
constexpr int kXcds = 8;  // XCDs of an MI355X
static_assert(kSegments % kXcds == 0, "whole segments per XCD");

// First tile of pass-0 segment s (s = kSegments gives `tiles`).
__host__ __device__ __forceinline__ uint32_t pass0_segment_first_tile(uint32_t s, uint32_t tiles) {
    return static_cast<uint32_t>((static_cast<uint64_t>(s) * tiles) / kSegments);
}

// Where one segment of one pass lies, in keys and in tiles.
struct SegmentInfo {
    uint32_t key_begin;
    uint32_t key_end;
    uint32_t tile_first;  // index of its first tile in the pass's status array
    uint32_t tiles;
};

// ---------------------------------------------------------------------------
// Segments balanced by position.
//
// Segment s of pass p >= 1 is normally the keys whose pass-(p-1) digit has
// top bits s.  When a few digit values hold most keys (duplicate-heavy keys,
// a constant byte below a varying one) one segment then holds most tiles,
// workgroups of every XCD crowd into its chain, and its look-backs wait on
// predecessors across XCDs (2^26 duplicate-heavy pairs: 268 against 217 us
// per pass).  Pass p's input is ordered by the bits below its digit,
// L_p = (K >> begin_bit) mod 2^b_p with b_p = shift_p - begin_bit, and then
// by original index (each earlier pass is a stable sort).  The 32-bit
// position key X = L_p * 2^(32 - b_p) + (index >> s_p), with s_p the
// smallest shift that fits every index of the input into 32 - b_p bits but
// at least kPositionMinShift, never decreases along that order, so cutting
// X at any boundaries cuts pass p's input into contiguous ranges.  (Keys of
// up to 32 bits only, so b_p <= 24; indexes sharing their top bits and L_p
// share one X and stay in one range.  The shift of at least 3 lets the
// histogram kernel take the index part once for the up to 8 consecutive
// keys a lane loads at once.)  A sampling step takes kSamples keys at evenly spaced
// positions and, for each pass whose digit-group segments would be
// unbalanced, keeps the X of every (kSamples / kSegments)-th sample in X
// order as the boundaries; the histogram kernel then counts each key in
// the segment its X falls into, and the digit-base kernel takes the
// segment ranges from those counts.
// ---------------------------------------------------------------------------
constexpr int kMaxPasses = 8;
constexpr uint32_t kPositionMinShift = 3;
// 512 samples, 64 per segment: the sort of their X takes 45 bitonic stages
// of one compare-exchange per thread (2048 samples took the launch from 10
// to 42 us on duplicate-heavy keys).
constexpr int kSamples = 512;
constexpr int kPrepareBlock = 256;
static_assert(kSamples == 2 * kPrepareBlock, "one compare-exchange per thread and stage");

struct SampleArgs {
    const void *keys;
    size_t n;
    int passes;
    uint32_t shift[kMaxPasses];
    uint32_t mask[kMaxPasses];
    uint32_t seg_shift;
    uint32_t begin_bit;
    uint32_t *seg_mode;                 // [kMaxPasses] 1: pass p takes the boundaries, else 0
    uint32_t *bounds;                   // [kMaxPasses][kSegments - 1] boundaries per pass
};

// s_p of the position key for b_p = `below` bits under the digit and n keys.
__device__ __forceinline__ uint32_t position_index_shift(uint32_t below, size_t n) {
    const uint32_t index_bits = n > 1 ? 64u - static_cast<uint32_t>(__builtin_clzll(n - 1)) : 0u;
    const uint32_t room = 32u - below;
    const uint32_t need = index_bits > room ? index_bits - room : 0u;
    return need > kPositionMinShift ? need : kPositionMinShift;
}

// X of a key for pass p from its bits below pass p's digit and the top bits
// of its index, ipart = index >> position_index_shift(shift_p - begin_bit, n).
template <class KT>
__device__ __forceinline__ uint32_t position_key(KT k, uint32_t shift_p, uint32_t begin_bit, uint32_t ipart) {
    const uint32_t below = shift_p - begin_bit;  // 8 to 24 for keys of up to 32 bits
    const uint32_t low = __builtin_amdgcn_ubfe(static_cast<uint32_t>(k), begin_bit, below);
    return (low << (32u - below)) | ipart;
}

// Offset of sample k inside its stratum of the input: a multiplicative hash
// of k (so that a period in the data cannot line up with the strata).
__device__ __forceinline__ size_t sample_offset(uint32_t k, size_t stratum) {
    uint32_t h = k * 0x9E3779B1u;
    h ^= h >> 15;
    return static_cast<size_t>(h) % stratum;
}

// The sampling step for pass p >= 1, run by one workgroup of kPrepareBlock
// threads.  Sample k is one key at a hashed position inside the k-th of
// kSamples equal strata of the input.  Independent keys matter: keys next
// to each other in sorted or clustered input share their upper digits, and
// runs of them would count as one sample many times over, tripping the
// balance test below on input whose digit groups are even.  A tie of X
// between samples cannot happen (the index is part of it).
template <KeyKind KIND>
__device__ void sample_pass(const SampleArgs &a, int p, uint32_t *s_x, uint32_t *s_group) {
    using KT = key_t<KIND>;
    const int tid = threadIdx.x;
    if (tid <= kSegments) s_group[tid] = 0u;  // [kSegments]: pass p's own digit varies
    __syncthreads();
    const size_t stratum = a.n / kSamples;  // the sampling step runs for n >= 2^22 only
    const uint32_t ishift = position_index_shift(a.shift[p] - a.begin_bit, a.n);
    const uint32_t digit0 =
        static_cast<uint32_t>(ordered_key<KIND>(static_cast<const KT *>(a.keys)[sample_offset(0u, stratum)]) >>
                              a.shift[p]) & a.mask[p];
    for (int k = tid; k < kSamples; k += kPrepareBlock) {
        const size_t index = static_cast<size_t>(k) * stratum + sample_offset(static_cast<uint32_t>(k), stratum);
        const KT key = ordered_key<KIND>(static_cast<const KT *>(a.keys)[index]);
        s_x[k] = position_key(key, a.shift[p], a.begin_bit, static_cast<uint32_t>(index >> ishift));
        const uint32_t prev = static_cast<uint32_t>(key >> a.shift[p - 1]) & a.mask[p - 1];
        atomicAdd(&s_group[prev >> a.seg_shift], 1u);
        if ((static_cast<uint32_t>(key >> a.shift[p]) & a.mask[p]) != digit0) s_group[kSegments] = 1u;
    }
    __syncthreads();
    uint32_t largest = 0u;
#pragma unroll
    for (int g = 0; g < kSegments; ++g) largest = s_group[g] > largest ? s_group[g] : largest;
    // Unbalanced: one digit group holds more than 3/16 of the samples
    // (1.5 times its share).  A pass whose own digit is the same in every
    // sample is left whole: it is most likely trivial and skipped, and its
    // keys then keep the histogram's shared-bin shortcut.
    const bool cut = largest * 16u > 3u * kSamples && s_group[kSegments] != 0u;
    if (cut) {
        // Bitonic sort of the samples' X.
        for (int size = 2; size <= kSamples; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int t = tid; t < kSamples / 2; t += kPrepareBlock) {
                    const int i = 2 * t - (t & (stride - 1));
                    const int l = i + stride;
                    const bool up = (i & size) == 0;
                    const uint32_t x = s_x[i], y = s_x[l];
                    if ((x > y) == up) {
                        s_x[i] = y;
                        s_x[l] = x;
                    }
                }
                __syncthreads();
            }
        }
        if (tid < kSegments - 1) a.bounds[p * (kSegments - 1) + tid] = s_x[(tid + 1) * (kSamples / kSegments)];
    }
    if (tid == 0) a.seg_mode[p] = cut ? 1u : 0u;
}

// The first kernel of a sort whose keys are sampled: workgroups below
// `sample_groups` run the sampling step of pass blockIdx.x + 1; the others
// zero the scan state (two ranges: the sampling step's words lie between
// them and are written, not zeroed).
struct PrepareArgs {
    uint4 *zero[2];
    size_t zero16[2];
    int sample_groups;
    SampleArgs s;
};

template <KeyKind KIND>
__global__ __launch_bounds__(kPrepareBlock) void prepare_kernel(PrepareArgs a) {
    __shared__ uint32_t s_x[kSamples];
    __shared__ uint32_t s_group[kSegments + 1];
    if (static_cast<int>(blockIdx.x) < a.sample_groups) {
        sample_pass<KIND>(a.s, static_cast<int>(blockIdx.x) + 1, s_x, s_group);
        return;
    }
    const size_t groups = gridDim.x - static_cast<size_t>(a.sample_groups);
    const size_t stride = groups * kPrepareBlock;
    const size_t first = (blockIdx.x - static_cast<size_t>(a.sample_groups)) * kPrepareBlock + threadIdx.x;
    for (int r = 0; r < 2; ++r) {
        for (size_t i = first; i < a.zero16[r]; i += stride) a.zero[r][i] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// ---------------------------------------------------------------------------
// All-pass digit histogram, per segment.
//
// [WA] "Las tres fases de una pasada" counts each block's digits into a
// workgroup-shared atomic histogram.  A digit histogram does not depend on
// the order of the keys, so the histograms of every pass are taken here from
// the ORIGINAL keys in a single read, into LDS-privatised counters
// [pass][segment][digit] that are folded into the global array at the end.
// ---------------------------------------------------------------------------
struct HistArgs {
    const void *keys;        // 32- or 64-bit keys (the kernel's key kind); M30: float xyz points
    MortonBox box;           // M30 only
    uint32_t *hist;          // [passes][kSegments][radix], zeroed beforehand
    size_t n;
    uint32_t tiles0;         // tiles of pass 0 (n / tile_keys rounded up)
    uint32_t tile_keys;
    uint32_t groups_per_seg; // workgroups per pass-0 segment
    size_t chunk;            // keys per workgroup, multiple of 64*ITEMS
    int passes;
    uint32_t shift[kMaxPasses];
    uint32_t mask[kMaxPasses];
    uint32_t seg_shift;      // pass p >= 1: segment = digit(p-1) >> seg_shift
    uint32_t begin_bit;      // sub-key = (ordered key >> begin_bit) & sub_mask
    unsigned long long sub_mask;
    uint32_t *unsorted;      // set to 1 when some key's sub-key exceeds the next key's
    const uint32_t *seg_mode;             // [kMaxPasses] 1: pass p's segments come from `bounds` (or null)
    const uint32_t *bounds;               // [kMaxPasses][kSegments - 1] (see SampleArgs)
};

// REPL copies of every counter, interleaved: lane l adds into copy
// l % REPL, so lanes of a wave that share a digit (frequent with skewed or
// duplicate-heavy keys) mostly update different words instead of
// serialising on one.
template <int BLOCK, int ITEMS, int RBITS, int REPL, KeyKind KIND>
__global__ __launch_bounds__(BLOCK) void hist_kernel(HistArgs a) {
    using KT = key_t<KIND>;
    constexpr int RADIX = 1 << RBITS;
    constexpr int MAXP = (8 * static_cast<int>(sizeof(KT)) + RBITS - 1) / RBITS;
    static_assert(MAXP <= kMaxPasses, "too many passes");
    static_assert((REPL & (REPL - 1)) == 0, "power-of-two replication");
    // Pass 0 counts only this workgroup's own segment (its keys all lie in
    // one pass-0 segment); passes >= 1 count every segment.  Bin of
    // (pass 0, digit d): d.  Bin of (pass p >= 1, segment s, digit d):
    // RADIX + (p-1)*S*RADIX + d*S + s when pass p's segments are groups of
    // the previous digit -- d*S + s is then the key's bits from the segment
    // bits of the previous digit to the top of its own digit, so one bit
    // field extract gives it, and a wave's adds to one digit spread over
    // the LDS banks by segment -- or + s*RADIX + d when they are position
    // ranges (a wave's keys then mostly share one segment, and the digit
    // spreads the banks).  The flush writes the global histogram segment
    // major.
    constexpr int BINS = RADIX + (MAXP - 1) * kSegments * RADIX;
    // Pass 0's RADIX bins have P0C copies each, lane l adding into copy
    // l % 32: a half-wave's 32 lanes then add into 32 different banks
    // whatever their digits (with REPL copies, the lanes of one copy
    // collide on the banks that their random bins share).  Uniform 2^28
    // uint32 keys 240.5 -> 225 us (16 copies: 228 us), duplicate-heavy
    // 137.8 -> 128.4 us; the 2048 bins of a later pass have no room for
    // as many copies.
    constexpr int P0C = 32;
    static_assert((P0C & (P0C - 1)) == 0 && P0C <= kWave, "power-of-two pass-0 copies");
    constexpr int WORDS = RADIX * P0C + (BINS - RADIX) * REPL;
    __shared__ uint32_t s_hist[WORDS];
    static_assert(BINS + BINS / 32 <= WORDS, "the flush's padded copy fits in the bins");

    const int tid = threadIdx.x;
    __shared__ uint32_t s_next_unit;  // number of the next unit of keys to count
    const uint32_t copy = static_cast<uint32_t>(tid) & (REPL - 1);
    for (int i = tid; i < WORDS; i += BLOCK) s_hist[i] = 0u;
    if (tid == 0) s_next_unit = 0u;
    __syncthreads();

    const uint32_t seg0 = blockIdx.x / a.groups_per_seg;
    const uint32_t group = blockIdx.x % a.groups_per_seg;
    const size_t seg_begin = static_cast<size_t>(pass0_segment_first_tile(seg0, a.tiles0)) * a.tile_keys;
    size_t seg_end = static_cast<size_t>(pass0_segment_first_tile(seg0 + 1, a.tiles0)) * a.tile_keys;
    if (seg_end > a.n) seg_end = a.n;
    const size_t begin = seg_begin + group * a.chunk;
    const size_t end = begin + a.chunk < seg_end ? begin + a.chunk : seg_end;
    // The key of element i: stored, or (M30) computed from point i.  Points
    // are read through a buffer resource over this workgroup's chunk, one
    // 96-bit load per point (three strided 4-byte loads took 2^24 points
    // 85 us); the order check, which reads past the chunk, never runs for
    // them.
    const bool m30 = KIND == KeyKind::M30;
    const __amdgpu_buffer_rsrc_t pts_rsrc =
        buffer_rsrc(const_cast<float *>(static_cast<const float *>(a.keys)) + (m30 ? 3 * begin : 0),
                    m30 ? static_cast<uint32_t>((end > begin ? end - begin : 0) * 12u) : 0u);
    auto key_at = [&](size_t i) -> KT {
        if constexpr (KIND == KeyKind::M30) {
            const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(pts_rsrc, static_cast<int>((i - begin) * 12u), 0, 0);
            // Components copied to scalars before the bit casts.
            const uint32_t xb = v.x, yb = v.y, zb = v.z;
            return morton30(__uint_as_float(xb), __uint_as_float(yb), __uint_as_float(zb), a.box);
        } else {
            return static_cast<const KT *>(a.keys)[i];
        }
    };
    // Bit p: pass p's segments are position ranges cut at sampled
    // boundaries (see sample_pass); otherwise groups of the previous digit.
    // (Only keys of up to 32 bits are sampled.)
    constexpr bool kCanSample = sizeof(KT) <= 4 && KIND != KeyKind::M30;
    uint32_t seg_mode = 0u;
    if (kCanSample && a.seg_mode != nullptr) {
        for (int q = 1; q < a.passes; ++q) seg_mode |= (__builtin_amdgcn_readfirstlane(a.seg_mode[q]) != 0u ? 1u : 0u) << q;
    }
    // Bits [low[p], low[p] + width[p]) of the ordered key choose pass p's
    // bin: its digit and, for passes >= 1, the top kSegmentBits bits of the
    // previous digit (every pass but the last is RBITS wide, so those bits
    // lie right below pass p's digit).
    uint32_t low[MAXP], width[MAXP];
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        const uint32_t dbits = static_cast<uint32_t>(__builtin_popcount(a.mask[p]));
        low[p] = p == 0 ? a.shift[0] : a.shift[p - 1] + a.seg_shift;
        width[p] = a.shift[p] + dbits - low[p];
    }
    auto bits_at = [&](KT k, uint32_t off, uint32_t w) -> uint32_t {
        if constexpr (sizeof(KT) <= 4) {
            return __builtin_amdgcn_ubfe(static_cast<uint32_t>(k), off, w);
        } else {
            return static_cast<uint32_t>(k >> off) & ((1u << w) - 1u);
        }
    };
    auto pass_bin0 = [](int p) { return p == 0 ? 0 : RADIX + (p - 1) * kSegments * RADIX; };
    // LDS word of pass p's bin `bin` in copy `cp` (lane 0's adds of a
    // shared bin's whole count go to copy 0), and this lane's copy.
    auto word_of = [&](int p, uint32_t bin, uint32_t cp) -> int {
        return p == 0 ? static_cast<int>(bin) * P0C + static_cast<int>(cp)
                      : RADIX * P0C + (pass_bin0(p) - RADIX + static_cast<int>(bin)) * REPL + static_cast<int>(cp);
    };
    auto copy_of = [&](int p) -> uint32_t { return p == 0 ? static_cast<uint32_t>(tid) & (P0C - 1) : copy; };
    auto is_cut = [&](int p) { return kCanSample && p > 0 && ((seg_mode >> p) & 1u) != 0u; };
    // The position-cut passes' boundaries, loaded once, with vector loads
    // (from a lane-varying zero offset) so they stay in VGPRs: as scalar
    // values the compiler reloaded them for every key, and each scalar
    // load's wait also waited for every LDS add in flight (both count on
    // one wait counter).
    constexpr int CUTP = kCanSample ? MAXP : 1;
    uint32_t bq[CUTP][kSegments - 1];
    uint32_t ishift[CUTP];
#pragma unroll
    for (int p = 0; p < CUTP; ++p) {
        ishift[p] = 0u;
#pragma unroll
        for (int t = 0; t < kSegments - 1; ++t) bq[p][t] = 0u;
    }
    if (kCanSample && seg_mode != 0u) {
        int z = 0;
        __asm__ volatile("" : "+v"(z));
#pragma unroll
        for (int p = 1; p < CUTP; ++p) {
            if ((seg_mode >> p) & 1u) {
                ishift[p] = position_index_shift(a.shift[p] - a.begin_bit, a.n);
#pragma unroll
                for (int t = 0; t < kSegments - 1; ++t) bq[p][t] = a.bounds[p * (kSegments - 1) + t + z];
            }
        }
    }
    // Bin of ordered key k (element `index`) in position-cut pass p, and in
    // pass p otherwise, relative to pass_bin0(p).
    // ipart: the key's index >> ishift[p] (shared by the V keys of a run).
    // (A binary search over the boundaries made the compiler index them
    // dynamically and keep them in scratch memory: slower than 7 compares.)
    auto cut_bin_at = [&](int p, KT k, uint32_t ipart) -> uint32_t {
        const uint32_t x = position_key(k, a.shift[p], a.begin_bit, ipart);
        uint32_t seg = 0u;
#pragma unroll
        for (int t = 0; t < kSegments - 1; ++t) seg += x >= bq[kCanSample ? p : 0][t] ? 1u : 0u;
        return (seg << RBITS) | bits_at(k, a.shift[p], width[p] - kSegmentBits);
    };
    auto cut_bin = [&](int p, KT k, size_t index) -> uint32_t {
        return cut_bin_at(p, k, static_cast<uint32_t>(index >> ishift[kCanSample ? p : 0]));
    };
    auto bin_of = [&](int p, KT k, size_t index) -> uint32_t {
        return is_cut(p) ? cut_bin(p, k, index) : bits_at(k, low[p], width[p]);
    };
    // ALL: the sort runs every pass of the key width (the usual case), so
    // no per-pass test is compiled.
    auto count_key = [&](KT bits, size_t index, auto all_c) {
        const KT k = ordered_key<KIND>(bits);
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            if (decltype(all_c)::value || p < a.passes) {
                atomicAdd(&s_hist[word_of(p, bin_of(p, k, index), copy_of(p))], 1u);
            }
        }
    };
    // Units: a wave counts UNIT = 64*ITEMS consecutive keys at a time, and
    // the whole units of the workgroup's chunk are handed out one at a time
    // from an LDS counter, so a wave that is served faster takes more of
    // them.  (With shares fixed in advance a quarter of the waves' time was
    // idle: the LDS does not serve a workgroup's waves evenly, the first of
    // 16 equal shares finished in about half the time of the last, and the
    // last few waves left alone could not keep the LDS busy.)  Key j of a
    // lane is element unit + (j / V)*64*V + V*lane + j % V: row r = j / V
    // is 64*V consecutive keys, and a lane's V of them come from one
    // 16-byte load (Morton keys, computed point by point: V = 1).  (One
    // 4-byte load per key: 2^28 uint32 keys 260 -> 256 us, int32 265 -> 255
    // us.)  Keys at an address that is not 16-byte aligned are loaded one by
    // one in the same layout.  The chunk's last, partial unit, counted by
    // the wave that draws the first number past the whole units, is read one
    // key per lane and row: element unit + j*64 + lane.
    constexpr int V = KIND == KeyKind::M30 ? 1 : static_cast<int>(16 / sizeof(KT));
    static_assert(ITEMS % V == 0, "whole rows of 16-byte loads");
    constexpr int ROWS = ITEMS / V;
    constexpr size_t UNIT = static_cast<size_t>(kWave) * ITEMS;
    const int lane = tid & (kWave - 1);
    auto whole_index = [&](size_t unit, int j) {
        return unit + static_cast<size_t>(j / V) * V * kWave + static_cast<size_t>(V) * lane + static_cast<size_t>(j % V);
    };
    const bool keys16 = (reinterpret_cast<uintptr_t>(a.keys) & 15u) == 0u;
    auto load_whole = [&](KT (&raw)[ITEMS], size_t unit) {
        if constexpr (V > 1) {
            if (keys16) {
#pragma unroll
                for (int r = 0; r < ROWS; ++r) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(static_cast<const KT *>(a.keys) + whole_index(unit, r * V));
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int c = 0; c < V; ++c) {
                        if constexpr (sizeof(KT) == 2) {
                            raw[r * V + c] = static_cast<KT>(w4[c / 2] >> (16 * (c % 2)));
                        } else if constexpr (sizeof(KT) == 4) {
                            raw[r * V + c] = static_cast<KT>(w4[c]);
                        } else {
                            raw[r * V + c] = static_cast<KT>((static_cast<uint64_t>(w4[2 * c + 1]) << 32) | w4[2 * c]);
                        }
                    }
                }
                return;
            }
        }
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) raw[j] = key_at(whole_index(unit, j));
    };
    // Already-sorted check ([OH] "GPU上的基数排序" closes with the early exit
    // of its reference paper that first verifies whether the input is
    // already ordered): a stable sort of keys whose sub-keys never decrease
    // is the identity, so every pass can be skipped.  Each key is compared
    // with the next one.  In a whole unit a lane holds runs of V consecutive
    // keys, compared in registers; the key after a run is the next lane's
    // first of the row (a DPP lane move), after the last lane's run the
    // first lane's first of the next row (a lane read), and after the unit
    // element unit + UNIT, which the last lane loads with the unit's keys
    // while no descent has been seen.  In the partial unit every lane whose
    // successor is not the next lane's key of the same row loads it itself.
    // A wave stops checking at its first descent (random input: in its
    // first unit).
    const KT sub_mask = static_cast<KT>(a.sub_mask);
    auto sub_key = [&](KT bits) { return static_cast<KT>(static_cast<KT>(ordered_key<KIND>(bits) >> a.begin_bit) & sub_mask); };
    bool descent = KIND == KeyKind::M30;  // Morton keys: their first pass always runs (it writes the codes)
    auto check_order = [&](const KT (&raw)[ITEMS], size_t unit, bool whole, KT succ) {
        KT sk[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) sk[j] = sub_key(raw[j]);
        bool d = false;
        if (whole) {
            // Lane moves and reads need every lane active: all of them
            // before any test.
            KT nl[ROWS], first[ROWS];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                nl[r] = next_lane(sk[r * V]);
                first[r] = lane_value(sk[r * V], 0);
            }
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                if (j % V != V - 1) d = d | (sk[j + 1] < sk[j]);
            }
            const bool last_lane = lane == kWave - 1;
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const KT after = !last_lane ? nl[r] : (r + 1 < ROWS ? first[r + 1 < ROWS ? r + 1 : 0] : sub_key(succ));
                const bool known = !last_lane || r + 1 < ROWS || unit + UNIT < a.n;
                d = d | (known & (after < sk[r * V + V - 1]));
            }
            descent = __any(d);
            return;
        }
        KT nl[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) nl[j] = next_lane(sk[j]);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const size_t idx = unit + static_cast<size_t>(j) * kWave + lane;
            d = d | ((lane != kWave - 1) & (idx + 1 < end) & (nl[j] < sk[j]));
        }
        if (__any(d)) {
            descent = true;
            return;
        }
        KT nx[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const size_t idx = unit + static_cast<size_t>(j) * kWave + lane;
            const bool edge = (lane == kWave - 1 || idx + 1 == end) && idx < end && idx + 1 < a.n;
            nx[j] = key_at(edge ? idx + 1 : (idx < a.n ? idx : size_t{0}));
        }
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const size_t idx = unit + static_cast<size_t>(j) * kWave + lane;
            const bool edge = (lane == kWave - 1 || idx + 1 == end) && idx < end && idx + 1 < a.n;
            d = d | (edge & (sub_key(nx[j]) < sk[j]));
        }
        descent = __any(d);
    };
    // Bins shared by a whole wave.  With keys whose high bytes are constant
    // (small integers in wide keys) or sorted keys, every lane of a wave
    // often adds to the same counter, and those adds serialise on one LDS
    // word.  A pass whose bin (its digit and, for passes >= 1, the top bits
    // of the previous digit that choose the segment) lies in bits equal for
    // every key of the wave's unit (OR and AND over the wave) gets one add
    // of the whole count from lane 0.  After a unit without such a pass the
    // check waits 1, 2, 4, ... (at most 16) units before it looks again, so
    // varied keys check about one unit in 16, while keys whose high bytes
    // stay constant, apart from a boundary crossed now and then, keep the
    // shortcut.  (The kernel lasts as long as its slowest workgroup, so a
    // check that stopped for good at a miss lost the gain whenever one
    // chunk's first keys crossed a boundary.)  (A per-slot form of the
    // check for sorted keys, comparing the first and last of each 64 keys,
    // was measured slower: its scalar work per slot and pass made sorted
    // 2^28 keys 661 -> 752 us.)
    auto field = [&](int p) -> KT {
        const uint32_t top = low[p] + width[p];
        const KT hi = top >= 8 * sizeof(KT) ? static_cast<KT>(~KT(0)) : static_cast<KT>((KT(1) << top) - 1);
        return static_cast<KT>(hi & ~static_cast<KT>((KT(1) << low[p]) - 1));
    };
    // Morton keys are computed per key and never checked.
    uint32_t const_wait = KIND == KeyKind::M30 ? 0xFFFFFFFFu : 0u;  // units before the next check
    uint32_t const_gap = 1u;                                         // wait after the next miss
    // One unit counted pass by pass; bit p of `whole_const`: pass p's bin
    // is shared by the wave's whole unit.
    uint32_t row_wait = 0u;  // units before the next row check
    uint32_t row_gap = 1u;   // wait after the next miss
    // Bit p of row_const[r]: pass p's bin is shared by row r (64*V
    // consecutive keys), which then gets one add of 64*V from lane 0.  Looked
    // for by OR and AND only in units where some pass's bin is shared by the
    // whole unit: in sorted keys a lower pass's bin stays the same over a
    // row long before it does over a unit (2^28 keys: pass 2's bin field,
    // bits 13-23, changes every ~512 keys).  After a unit whose rows share
    // nothing more, the row check waits 1, 2, 4, ... (at most 16) units, as
    // the unit check does (keys below 2^16 share their top pass's bin in
    // every unit and nothing in rows: 254 -> 274 us without the wait).
    auto rows_by_bits = [&](const KT (&raw)[ITEMS], uint32_t whole_const, auto all_c, uint32_t (&row_const)[ROWS],
                            uint32_t &any_row) {
        if constexpr (V > 1) {
            if (whole_const != 0u && row_wait != 0u) {
                --row_wait;
            } else if (whole_const != 0u) {
#pragma unroll
                for (int r = 0; r < ROWS; ++r) {
                    KT o = KT(0), n = static_cast<KT>(~KT(0));
#pragma unroll
                    for (int c = 0; c < V; ++c) {
                        const KT k = ordered_key<KIND>(raw[r * V + c]);
                        o = static_cast<KT>(o | k);
                        n = static_cast<KT>(n & k);
                    }
                    const KT differ = static_cast<KT>(wave_bits_of<false>(o) ^ wave_bits_of<true>(n));
#pragma unroll
                    for (int p = 0; p < MAXP; ++p) {
                        if ((decltype(all_c)::value || p < a.passes) && ((whole_const >> p) & 1u) == 0u && !is_cut(p) &&
                            (differ & field(p)) == KT(0)) {
                            row_const[r] |= 1u << p;
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < ROWS; ++r) any_row |= row_const[r];
                if (any_row != 0u) {
                    row_gap = 1u;
                } else {
                    row_wait = row_gap;
                    row_gap = row_gap < 16u ? 2u * row_gap : 16u;
                }
            }
        }
    };
    // Keys in sub-key order (the order check found no descent in the unit)
    // share pass p's bin over a run exactly when the run's first and last
    // sub-keys agree on every bit from the bin's lowest up: the keys between
    // them agree there too.  Two lane reads per run instead of an OR and an
    // AND over the wave (sorted 2^28 keys: histogram 241 -> 227 us).  Bit p
    // of the result: pass p shares (not those in `done`, nor passes cut by
    // position).
    auto shared_by_ends = [&](KT first, KT last, uint32_t done, auto all_c) -> uint32_t {
        const KT x = static_cast<KT>(first ^ last);
        uint32_t m = 0u;
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            const uint32_t rel = low[p] - a.begin_bit;
            const bool agree = rel >= 8 * sizeof(KT) || (x >> rel) == KT(0);
            if ((decltype(all_c)::value || p < a.passes) && ((done >> p) & 1u) == 0u && !is_cut(p) && agree) m |= 1u << p;
        }
        return m;
    };
    auto count_unit = [&](const KT (&raw)[ITEMS], size_t unit, uint32_t whole_const, const uint32_t (&row_const)[ROWS],
                          uint32_t any_row, auto all_c) {
#pragma unroll
        for (int p = 0; p < MAXP; ++p) {
            if (decltype(all_c)::value || p < a.passes) {
                if ((whole_const >> p) & 1u) {
                    if (lane == 0) {
                        atomicAdd(&s_hist[word_of(p, bin_of(p, ordered_key<KIND>(raw[0]), whole_index(unit, 0)), 0u)],
                                  static_cast<uint32_t>(ITEMS * kWave));
                    }
                } else {
                    // The pass's rule is tested once per unit, not per key.
                    uint32_t bin[ITEMS];
                    if (is_cut(p)) {
                        // A run's V consecutive indexes (starting at a
                        // multiple of V <= 2^kPositionMinShift) share
                        // index >> ishift.
                        static_assert(V <= (1 << kPositionMinShift), "a run shares its index part");
#pragma unroll
                        for (int r = 0; r < ROWS; ++r) {
                            const uint32_t ipart =
                                static_cast<uint32_t>(whole_index(unit, r * V) >> ishift[kCanSample ? p : 0]);
#pragma unroll
                            for (int c = 0; c < V; ++c) bin[r * V + c] = cut_bin_at(p, ordered_key<KIND>(raw[r * V + c]), ipart);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < ITEMS; ++j) bin[j] = bits_at(ordered_key<KIND>(raw[j]), low[p], width[p]);
                    }
                    if (((any_row >> p) & 1u) == 0u) {
#pragma unroll
                        for (int j = 0; j < ITEMS; ++j) atomicAdd(&s_hist[word_of(p, bin[j], copy_of(p))], 1u);
                    } else {
#pragma unroll
                        for (int r = 0; r < ROWS; ++r) {
                            if ((row_const[r] >> p) & 1u) {
                                if (lane == 0) atomicAdd(&s_hist[word_of(p, bin[r * V], 0u)], static_cast<uint32_t>(V * kWave));
                            } else {
#pragma unroll
                                for (int c = 0; c < V; ++c) atomicAdd(&s_hist[word_of(p, bin[r * V + c], copy_of(p))], 1u);
                            }
                        }
                    }
                }
            }
        }
    };
    // Whole units, while the counter hands them out: every load in range,
    // all issued before any is used.  The next unit's number is drawn
    // before this one is counted, so its LDS round trip overlaps the count.
    const size_t units = end > begin ? (end - begin) / UNIT : 0;
    auto draw = [&]() -> uint32_t {
        uint32_t u = 0u;
        if (lane == 0) u = atomicAdd(&s_next_unit, 1u);
        return u;
    };
    auto whole_units = [&](auto all_c) -> uint32_t {
        uint32_t u = __builtin_amdgcn_readfirstlane(draw());
        // A wave checks its first unit after counting it, as random keys
        // then stop checking without waiting for the check; later units,
        // while in order, are checked first and share bins by their ends.
        bool later = false;
        for (; u < units;) {
            const size_t unit = begin + static_cast<size_t>(u) * UNIT;
            KT raw[ITEMS];
            load_whole(raw, unit);
            // While no descent is seen, the key after the unit is loaded
            // with the unit's keys (loaded at the check, its latency stalled
            // every unit of sorted input).
            KT succ = KT(0);
            if (!descent && lane == kWave - 1 && unit + UNIT < a.n) succ = key_at(unit + UNIT);
            const uint32_t next = draw();
            uint32_t whole_const = 0u, any_row = 0u;  // any_row bit p: some row shares pass p's bin
            uint32_t row_const[ROWS];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) row_const[r] = 0u;
            bool in_order = false;
            if (!descent && later) {
                check_order(raw, unit, true, succ);
                in_order = !descent;
            }
            if (in_order) {
                whole_const = shared_by_ends(lane_value(sub_key(raw[0]), 0), lane_value(sub_key(raw[ITEMS - 1]), kWave - 1),
                                             0u, all_c);
                if constexpr (V > 1) {
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) {
                        row_const[r] = shared_by_ends(lane_value(sub_key(raw[r * V]), 0),
                                                      lane_value(sub_key(raw[r * V + V - 1]), kWave - 1), whole_const, all_c);
                        any_row |= row_const[r];
                    }
                }
            } else if (const_wait != 0u) {
                if (const_wait != 0xFFFFFFFFu) --const_wait;
            } else {
                KT o = KT(0), n = static_cast<KT>(~KT(0));
#pragma unroll
                for (int j = 0; j < ITEMS; ++j) {
                    const KT k = ordered_key<KIND>(raw[j]);
                    o = static_cast<KT>(o | k);
                    n = static_cast<KT>(n & k);
                }
                const KT differ = static_cast<KT>(wave_bits_of<false>(o) ^ wave_bits_of<true>(n));
#pragma unroll
                for (int p = 0; p < MAXP; ++p) {
                    // A pass cut by position has bins that also depend on
                    // the index; it never shares one across the wave.
                    if ((decltype(all_c)::value || p < a.passes) && ((seg_mode >> p) & 1u) == 0u &&
                        (differ & field(p)) == KT(0)) {
                        whole_const |= 1u << p;
                    }
                }
                if (whole_const != 0u) {
                    const_gap = 1u;
                } else {
                    const_wait = const_gap;
                    const_gap = const_gap < 16u ? 2u * const_gap : 16u;
                }
            }
            if (!in_order) rows_by_bits(raw, whole_const, all_c, row_const, any_row);
            if (whole_const != 0u || any_row != 0u || seg_mode != 0u) {
                count_unit(raw, unit, whole_const, row_const, any_row, all_c);
            } else {
#pragma unroll
                for (int j = 0; j < ITEMS; ++j) count_key(raw[j], whole_index(unit, j), all_c);
            }
            if (!descent && !later) check_order(raw, unit, true, succ);
            later = true;
            u = __builtin_amdgcn_readfirstlane(next);
        }
        return u;
    };
    const uint32_t drawn = a.passes == MAXP ? whole_units(BoolC<true>{}) : whole_units(BoolC<false>{});
    // The partial unit: one wave draws exactly the number `units`.
    const size_t tail = begin + units * UNIT;
    if (drawn == units && tail < end) {
        KT raw[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const size_t idx = tail + static_cast<size_t>(j) * kWave + lane;
            raw[j] = idx < end ? key_at(idx) : KT(0);
        }
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const size_t index = tail + static_cast<size_t>(j) * kWave + lane;
            if (index < end) count_key(raw[j], index, BoolC<false>{});
        }
        if (!descent) check_order(raw, tail, false, KT(0));
    }
    // One plain store per workgroup that saw a descent.  Every writer
    // stores the same 1, so no read-modify-write is needed: device-scope
    // atomics on one word from every wave serialise (about 25 us for 4096
    // of them).
    if (__syncthreads_or(descent) && tid == 0) {
        __hip_atomic_store(a.unsorted, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Flush.  The copies' sums are read in bin order (consecutive threads,
    // consecutive words), then written back into the start of s_hist in
    // segment-major order, one pad word per 32, and read from there in
    // that order, so a wave's device atomics cover consecutive words.
    constexpr int FLUSH = (BINS + BLOCK - 1) / BLOCK;
    const int used = RADIX + (a.passes - 1) * kSegments * RADIX;
    uint32_t sum[FLUSH];
    int at[FLUSH];
#pragma unroll
    for (int f = 0; f < FLUSH; ++f) {
        const int i = f * BLOCK + tid;
        sum[f] = 0u;
        at[f] = i;
        if (i < used) {
            if (i < RADIX) {
#pragma unroll
                for (int r = 0; r < P0C; ++r) sum[f] += s_hist[i * P0C + ((r + tid) & (P0C - 1))];
            } else {
#pragma unroll
                for (int r = 0; r < REPL; ++r) sum[f] += s_hist[RADIX * P0C + (i - RADIX) * REPL + r];
            }
            if (i >= RADIX) {
                const int r = i - RADIX;
                const int w = r % (kSegments * RADIX);
                const int q = r / (kSegments * RADIX) + 1;
                if (!(kCanSample && ((seg_mode >> q) & 1u))) {
                    at[f] = RADIX + (r - w) + (w & (kSegments - 1)) * RADIX + (w >> kSegmentBits);
                }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int f = 0; f < FLUSH; ++f) {
        if (f * BLOCK + tid < used) s_hist[at[f] + (at[f] >> 5)] = sum[f];
    }
    __syncthreads();
    for (int i = tid; i < used; i += BLOCK) {
        const uint32_t c = s_hist[i + (i >> 5)];
        // Global layout [pass][segment][digit]: pass 0 goes to this
        // workgroup's segment, the rest follows pass 0's block.
        const int g = i < RADIX ? static_cast<int>(seg0) * RADIX + i : kSegments * RADIX + (i - RADIX);
        if (c != 0u) atomicAdd(&a.hist[g], c);
    }
}

// ---------------------------------------------------------------------------
// Per-pass starting offsets and segment layout.  For pass p (one workgroup,
// one thread per digit):
//   base[p][s][d] = (keys whose pass-p digit is below d)
//                 + (digit-d keys in segments before s)
// i.e. where segment s starts writing digit d in the output of pass p -- the
// digit-major exclusive scan of [WA] "Las tres fases", at segment
// granularity -- plus each segment's key range and tile numbering.
// ---------------------------------------------------------------------------
struct BaseArgs {
    const uint32_t *hist;    // [passes][kSegments][radix]
    uint32_t *base;          // [passes][kSegments][radix]
    SegmentInfo *segs;       // [passes][kSegments]
    uint32_t n;
    uint32_t tiles0;
    uint32_t tile_keys;
    uint32_t seg_shift;      // pass p >= 1: segment s = pass-(p-1) digits [s << seg_shift, ...)
    uint32_t *trivial;       // [passes] set to 1 when one digit holds all n keys
    const uint32_t *unsorted; // 0 when the keys are already in sub-key order
    int keep_first;          // pass 0 is never skipped (it computes the keys)
    const uint32_t *seg_mode; // [kMaxPasses] 1: pass p's segments are position ranges (sample_pass), or null
};

// Exclusive prefix sum over the threads of a workgroup of RADIX threads.
template <int RADIX>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t *s_wave_total) {
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const uint32_t incl = wave_inclusive_sum(v);
    if ((tid & (kWave - 1)) == kWave - 1) s_wave_total[wave] = incl;
    __syncthreads();
    uint32_t before = incl - v;
    for (int w = 0; w < wave; ++w) before += s_wave_total[w];
    __syncthreads();
    return before;
}

template <int RADIX>
__global__ __launch_bounds__(RADIX) void digit_base_kernel(BaseArgs a) {
    static_assert(RADIX % kWave == 0 && RADIX > kSegments, "radix must fill whole waves");
    __shared__ uint32_t s_wave_total[RADIX / kWave];
    __shared__ uint32_t s_bound[kSegments + 1];
    const int tid = threadIdx.x;
    const int p = blockIdx.x;

    const uint32_t *h = a.hist + p * kSegments * RADIX;
    uint32_t c[kSegments];
    uint32_t total = 0u;
#pragma unroll
    for (int s = 0; s < kSegments; ++s) {
        c[s] = h[s * RADIX + tid];
        total += c[s];
    }
    // A pass in which one digit holds every key is the identity permutation
    // (a stable counting sort of equal digits); the pass kernels skip it.
    // Keys already in sub-key order need no pass at all (the passes
    // together are the identity).  a.trivial[p] is zero on entry.
    if ((total == a.n || *a.unsorted == 0u) && !(a.keep_first && p == 0)) a.trivial[p] = 1u;
    uint32_t run = block_exclusive_sum<RADIX>(total, s_wave_total);
    uint32_t *b = a.base + p * kSegments * RADIX;
#pragma unroll
    for (int s = 0; s < kSegments; ++s) {
        b[s * RADIX + tid] = run;
        run += c[s];
    }

    // Segment boundaries of this pass's input.
    const bool by_position = p > 0 && a.seg_mode != nullptr && a.seg_mode[p] != 0u;
    if (by_position) {
        // Segments cut at sampled boundaries: their sizes are the counts
        // (summed per wave with lane moves, then over the waves).
        __shared__ uint32_t s_wave_seg[RADIX / kWave][kSegments];
#pragma unroll
        for (int s = 0; s < kSegments; ++s) {
            const uint32_t w = wave_inclusive_sum(c[s]);
            if ((tid & (kWave - 1)) == kWave - 1) s_wave_seg[tid / kWave][s] = w;
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t at = 0u;
            for (int s = 0; s < kSegments; ++s) {
                s_bound[s] = at;
                for (int w = 0; w < RADIX / kWave; ++w) at += s_wave_seg[w][s];
            }
            s_bound[kSegments] = a.n;
        }
    } else if (p == 0) {
        if (tid <= kSegments) {
            const size_t k = static_cast<size_t>(pass0_segment_first_tile(tid, a.tiles0)) * a.tile_keys;
            s_bound[tid] = static_cast<uint32_t>(k < a.n ? k : a.n);
        }
    } else {
        // Start of each group of pass-(p-1) digits in pass p-1's output.
        const uint32_t *hp = a.hist + (p - 1) * kSegments * RADIX;
        uint32_t prev_total = 0u;
#pragma unroll
        for (int s = 0; s < kSegments; ++s) prev_total += hp[s * RADIX + tid];
        const uint32_t prev_start = block_exclusive_sum<RADIX>(prev_total, s_wave_total);
        if ((static_cast<uint32_t>(tid) & ((1u << a.seg_shift) - 1u)) == 0u) {
            const uint32_t s = static_cast<uint32_t>(tid) >> a.seg_shift;
            if (s < kSegments) s_bound[s] = prev_start;
        }
        if (tid == 0) s_bound[kSegments] = a.n;
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t first = 0u;
        for (int s = 0; s < kSegments; ++s) {
            SegmentInfo info;
            info.key_begin = s_bound[s];
            info.key_end = s_bound[s + 1];
            info.tile_first = first;
            info.tiles = (info.key_end - info.key_begin + a.tile_keys - 1u) / a.tile_keys;
            first += info.tiles;
            a.segs[p * kSegments + s] = info;
        }
    }
}

// ---------------------------------------------------------------------------
// One digit pass: load a tile, rank, chained digit scan, LDS shuffle, stable
// scatter -- fused in one kernel.
//
// Global position of an element ([OH] "GPU上的基数排序": position = scanned
// block sum of its digit + its local rank; [WA] "Las tres fases": the
// digit-major exclusive scan of counts gives, at (d, b), where block b starts
// writing digit d):
//     dst = base[segment][d] + (digit-d count of earlier tiles of the
//           segment) + rank in tile.
// The middle term is the digit-major scan across tiles.  Here it is computed
// by a chained scan with decoupled look-back: each tile publishes its digit
// counts as soon as it has ranked, then sums the published counts of earlier
// tiles of its segment back to the first one that already holds an
// inclusive prefix.  A workgroup claims the next tile of its own XCD's
// segment from an atomic counter (another segment's once its own is used
// up), so every tile a tile waits for was claimed earlier by a running
// workgroup: the chains always drain.
//
// Local rank (what the 1-bit splits of [WA] "El ranking local..." and the
// one-hot Blelloch scans of [OH] Pass1 compute): rank(i) = number of earlier
// elements of the tile with the same digit.  Each wave holds its keys
// wave-striped (slot j of lane l is tile element wave_base + 64*j + l), so
// element order is (wave, slot, lane) order.  Ranking uses one counter per
// (wave, digit) in LDS:
//   * every element adds 1 to its (wave, digit) counter, slot by slot; the
//     value the add returns is the number of the wave's earlier elements
//     with that digit (its rank within the wave);
//   * after a barrier the counters hold each wave's digit counts, which give
//     the tile's digit counts (published at once) and are overwritten with
//     where each wave's run of each digit starts in the tile-sorted order;
//   * tile-sorted position = rank within the wave + that start (an LDS
//     read).
// The rank is stable because a wave issues its slots' adds in slot order
// and the LDS of gfx950 applies same-address atomic adds of one wave64
// instruction in ascending lane order, so each add returns the count of the
// elements before it in element order.  (That lane order is a measured
// property of the hardware, not a documented one; the GPU tests check
// stability with heavily duplicated keys.)
//
// Scatter ([PM] §13.4: stage the tile in shared memory, then write contiguous
// runs): keys are written to LDS at their tile-sorted position, then read
// back in order, so consecutive lanes write consecutive addresses of the
// same digit run.
//
// The last tile of a segment may be partial.  Its missing elements (pads)
// take no part in counting or ranking: the real elements fill tile
// positions [0, valid) and positions >= valid are never written out.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Which buffer each pass reads and writes once trivial passes are skipped.
// Buffers: 0 = the caller's input, 1 = the caller's output, 2 = temp.  The
// executed passes alternate between output and temp so that, out of place,
// the last one writes the caller's output; in place (input == output) the
// first reads the output, and an odd number of executed passes ends in temp
// (one copy back).  With no executed pass, out of place, the input is copied.
// ---------------------------------------------------------------------------
struct PassRoute {
    bool skip;
    int src;
    int dst;
};

__device__ __forceinline__ int executed_passes(const uint32_t *trivial, int passes) {
    int e = 0;
    for (int q = 0; q < passes; ++q) e += trivial[q] == 0u ? 1 : 0;
    return e;
}

__device__ __forceinline__ PassRoute pass_route(const uint32_t *trivial, int passes, int pass, bool in_place) {
    const int e = executed_passes(trivial, passes);
    int k = 0;  // executed passes before this one
    for (int q = 0; q < pass; ++q) k += trivial[q] == 0u ? 1 : 0;
    if (trivial[pass] != 0u) return {true, 0, 0};
    auto dst = [&](int kk) { return in_place ? (kk % 2 == 0 ? 2 : 1) : ((e - 1 - kk) % 2 == 0 ? 1 : 2); };
    return {false, k == 0 ? (in_place ? 1 : 0) : dst(k - 1), dst(k)};
}

// Buffer to copy into the caller's output after the passes, or -1.
__device__ __forceinline__ int final_copy_source(const uint32_t *trivial, int passes, bool in_place) {
    const int e = executed_passes(trivial, passes);
    if (in_place) return e % 2 == 1 ? 2 : -1;
    return e == 0 ? 0 : -1;
}

// Grid-stride copy of n elements of T by the whole launch, with
// kCopyUnroll loads in flight per thread before their stores.  16-byte
// accesses when both pointers are 16-byte aligned, the remaining elements
// one by one.
template <class V>
__device__ __forceinline__ void grid_copy_unrolled(const V *in, V *out, size_t n) {
    const size_t threads = static_cast<size_t>(gridDim.x) * blockDim.x;
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + (kCopyUnroll - 1) * threads < n; i += kCopyUnroll * threads) {
        V v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) v[u] = in[i + u * threads];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) out[i + u * threads] = v[u];
    }
    for (; i < n; i += threads) out[i] = in[i];
}

template <class T>
__device__ __forceinline__ void grid_copy(const T *in, T *out, size_t n) {
    constexpr size_t PER = sizeof(uint4) / sizeof(T);
    if (((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & (sizeof(uint4) - 1)) == 0) {
        const size_t n16 = n / PER;
        grid_copy_unrolled(reinterpret_cast<const uint4 *>(in), reinterpret_cast<uint4 *>(out), n16);
        const size_t done = n16 * PER;
        grid_copy_unrolled(in + done, out + done, n - done);
    } else {
        grid_copy_unrolled(in, out, n);
    }
}

// n elements of `bytes` bytes each (2, 4 or 8).
__device__ __forceinline__ void grid_copy_elems(const void *in, void *out, size_t n, int bytes) {
    if (bytes == 2) {
        grid_copy(static_cast<const uint16_t *>(in), static_cast<uint16_t *>(out), n);
    } else if (bytes == 8) {
        grid_copy(static_cast<const uint64_t *>(in), static_cast<uint64_t *>(out), n);
    } else {
        grid_copy(static_cast<const uint32_t *>(in), static_cast<uint32_t *>(out), n);
    }
}

struct CopyArgs {
    void *kbuf[3];
    void *vbuf[3];
    const uint32_t *trivial;
    int passes;
    int keys_in_place;
    int vals_in_place;
    size_t n;          // elements
    int key_bytes;     // 2, 4 or 8
    int val_bytes;     // 4 or 8
};

// Copies temp back into the caller's output after an in-place sort whose
// executed pass count is odd; nothing otherwise.
__global__ __launch_bounds__(kCopyBlock) void route_copy_kernel(CopyArgs a) {
    const int ks = final_copy_source(a.trivial, a.passes, a.keys_in_place != 0);
    if (ks == 2 && a.keys_in_place) grid_copy_elems(a.kbuf[2], a.kbuf[1], a.n, a.key_bytes);
    if (a.vbuf[1] != nullptr) {
        const int vs = final_copy_source(a.trivial, a.passes, a.vals_in_place != 0);
        if (vs == 2 && a.vals_in_place) grid_copy_elems(a.vbuf[2], a.vbuf[1], a.n, a.val_bytes);
    }
}

template <class StatusT>
struct PassArgs {
    void *kbuf[3];               // keys: caller input, caller output, temp
    void *vbuf[3];               // values (pairs only)
    const uint32_t *trivial;     // [passes] 1 if that pass is skipped
    int pass;
    int passes;
    int keys_in_place;
    int vals_in_place;
    const uint32_t *seg_base;    // [kSegments][RADIX] this pass's starting offsets
    const SegmentInfo *segs;     // [kSegments] this pass's segments
    StatusT *status;             // [tiles_max][RADIX] this pass, zero on entry
    StatusT *status_next;        // [tiles_max][RADIX] next pass's words to zero, or null
    uint32_t *seg_counter;       // [kSegments] tiles claimed per segment, zero on entry
    uint32_t *error_word;
    uint32_t tiles_max;          // status words per pass = grid size
    uint32_t n;
    uint32_t shift;
    uint32_t mask;
    MortonBox box;               // M30 (first pass from points) only
    uint32_t spin_limit;         // bound on look-back polls of one status word (kSpinLimit)
    uint32_t withhold_tile;      // tile whose status words are never published (test hook), or 0xFFFFFFFF
};

// Bound on look-back polls of one status word (each poll is a device-scope
// load of ~1 us plus a short sleep): a few seconds, far beyond any real wait.
constexpr uint32_t kSpinLimit = 1u << 22;
// Predecessor status words fetched per look-back step.  The first window,
// fetched while the tile is ranked, holds 2 in the kernels of 32-bit keys
// and values (2^28 keys 446.6 -> 443.6 us per pass against 4; 6 or 8 were
// slower), 4 in those with smaller tiles; later windows hold 4.
constexpr int kLookbackWindow = 4;
#ifndef LOOKBACK_FIRST
#define LOOKBACK_FIRST 2
#endif
constexpr int kLookbackFirst = LOOKBACK_FIRST;


// A window of look-back status words: w[i] belongs to tile k - i.  Tiles
// before the segment's first tile read as an inclusive prefix of 0.  `far`
// selects device-scope reads; otherwise reads may be served by this XCD's L2
// (status_load_near).
template <class StatusT, int RADIX, int W>
struct LookbackWindow {
    StatusT w[W];

    __device__ __forceinline__ void fetch(StatusT *status, uint32_t k, uint32_t first, uint32_t digit,
                                          bool far) {
#pragma unroll
        for (int i = 0; i < W; ++i) {
            StatusT *p = status + static_cast<size_t>(k - i) * RADIX + digit;
            if (k < first + static_cast<uint32_t>(i)) {
                w[i] = make_status<StatusT>(kFlagInclusive, 0u);
            } else {
                w[i] = far ? status_load(p) : status_load_near(p);
            }
        }
    }

    // Adds the window's counts (tiles k, k-1, ...) to `before` up to and
    // including the first inclusive prefix.  Sets `consumed` to the number of
    // words used, `done` when an inclusive prefix was reached, `empty` when
    // a word was still empty (nothing after it is used) and `failed` on an
    // error word.
    __device__ __forceinline__ void consume(uint32_t &before, int &consumed, bool &done, bool &empty,
                                            bool &failed) const {
        using SW = StatusWord<StatusT>;
        consumed = 0;
        done = empty = false;
#pragma unroll
        for (int i = 0; i < W; ++i) {
            if (!done && !empty && !failed) {
                const uint32_t flag = static_cast<uint32_t>(w[i] >> SW::kShift);
                if (flag == kFlagEmpty) {
                    empty = true;
                } else if (flag == kFlagError) {
                    failed = true;
                } else {
                    before += static_cast<uint32_t>(w[i] & SW::kValueMask);
                    consumed = i + 1;
                    done = (flag == kFlagInclusive);
                }
            }
        }
    }
};

// Decoupled look-back of one digit: the count of that digit in the tiles of
// the segment before `tile` (seg_first < tile).  `first` holds the window of
// tiles tile-1, tile-2, ... fetched earlier; later windows hold W1 words.
// Returns false if a wait gave up or the segment's chain is inconsistent.
template <int W1, class StatusT, int RADIX, int W0>
__device__ __forceinline__ bool lookback_sum(StatusT *status, uint32_t tile, uint32_t seg_first, uint32_t digit,
                                             const LookbackWindow<StatusT, RADIX, W0> &first, uint32_t &before,
                                             uint32_t spin_limit = kSpinLimit) {
    before = 0u;
    bool failed = false, done = false, empty = false, far = false;
    uint32_t spins = 0u;
    uint32_t k = tile - 1u;  // tile of the window's first word
    int consumed = 0;
    first.consume(before, consumed, done, empty, failed);
    LookbackWindow<StatusT, RADIX, W1> lb;
    for (;;) {
        if (consumed < 0) lb.consume(before, consumed, done, empty, failed);
        if (done) return true;
        if (failed) return false;
        if (empty) {
            // The near read may be stale; from now on read device-wide.
            if (far) {
                if (++spins > spin_limit) return false;
                __builtin_amdgcn_s_sleep(1);
            }
            far = true;
        } else if (k < seg_first + static_cast<uint32_t>(consumed)) {
            return false;  // ran past the segment's first tile, which is always inclusive
        }
        k -= static_cast<uint32_t>(consumed);
        lb.fetch(status, k, seg_first, digit, far);
        consumed = -1;
    }
}

// RANK selects the local ranker: kRankAtomic (each element's LDS atomic add
// on its (wave, digit) counter; relies on same-address adds of one wave64
// instruction being served in ascending lane order, a measured property of
// the gfx950 LDS) or kRankMatch (match_rank: ballots per digit bit, one add
// per distinct digit, no reliance on that order).
constexpr int kRankAtomic = 0;
constexpr int kRankMatch = 1;

template <int BLOCK, int ITEMS, int RBITS, KeyKind KIND, bool PAIRS, class StatusT, class VT = uint32_t,
          int RANK = kRankAtomic>
__global__ __launch_bounds__(BLOCK) void onesweep_kernel(PassArgs<StatusT> a) {
    constexpr int RADIX = 1 << RBITS;
    constexpr int WAVES = BLOCK / kWave;
    constexpr int TILE = BLOCK * ITEMS;
    constexpr int WAVE_KEYS = kWave * ITEMS;
    // 64-bit status words come with inputs of 2^30 keys or more; those also
    // need 64-bit addressing (buffer offsets are 32-bit).
    constexpr bool WIDE = sizeof(StatusT) == 8;
    static_assert(BLOCK % kWave == 0, "block must be whole waves");
    static_assert(BLOCK >= RADIX && RADIX % kWave == 0, "one thread per digit");
    constexpr uint32_t kNone = 0xFFFFFFFFu;

    using KT = key_t<KIND>;
    constexpr uint32_t KB = sizeof(KT);               // bytes per key
    __shared__ KT s_tile[TILE];                       // keys in tile-sorted order
    constexpr uint32_t VB = sizeof(VT);               // bytes per value
    __shared__ VT s_vals[PAIRS ? TILE : 1];           // values in the same order
    __shared__ uint32_t s_cnt[WAVES * RADIX];         // (wave, digit) counters
    __shared__ uint32_t s_goff[RADIX];                // global start - tile start, per digit
    __shared__ uint32_t s_wave_total[RADIX / kWave];
    __shared__ SegmentInfo s_segs[kSegments];
    __shared__ uint32_t s_claim[2][4];                // per claim: tile, segment, key start, valid
    __shared__ uint32_t s_claim_seq;                  // claims published so far

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint32_t width = static_cast<uint32_t>(__builtin_popcount(a.mask));  // digit bits of this pass

    // The next pass's status words are cleared by this launch, spread over
    // the grid (the pass that last used them has completed): by a
    // workgroup that has no tile work at once, by the others after their
    // last tile, where the stores neither delay their first loads nor add
    // to the pass (workgroups finish a tile apart).
    auto clear_next_status = [&]() {
        if (a.status_next != nullptr) {
            const size_t words = static_cast<size_t>(a.tiles_max) * RADIX;
            for (size_t i = static_cast<size_t>(blockIdx.x) * BLOCK + tid; i < words;
                 i += static_cast<size_t>(gridDim.x) * BLOCK) {
                a.status_next[i] = StatusT(0);
            }
        }
    };

    // ---- tile claims (the last wave) -------------------------------------
    // A workgroup takes tiles from its home segment (first the one of its
    // XCD) and moves to another segment with tiles left once that one is
    // used up.  The next tile is claimed while the current one is ranked
    // (its counter increment issued after the scan in keys-only sorts, after
    // ranking with values), shortly before it is worked on, so tiles are
    // published in about the order they are claimed.  The claiming wave is
    // the last one, which has no status traffic to wait behind.
    const bool claim_wave = wave == WAVES - 1;
    // Home segment: one of this XCD's kSegments / kXcds segments (workgroups
    // of an XCD alternate between them).
    uint32_t home = (xcd_id() % kXcds) * (kSegments / kXcds) + (blockIdx.x / kXcds) % (kSegments / kXcds);
    auto publish_claim = [&](uint32_t idx, uint32_t *dst) {
        const SegmentInfo info = s_segs[home];
        const uint32_t start = info.key_begin + idx * static_cast<uint32_t>(TILE);
        const uint32_t left = info.key_end - start;
        dst[0] = info.tile_first + idx;
        dst[1] = home;
        dst[2] = start;
        dst[3] = left < static_cast<uint32_t>(TILE) ? left : static_cast<uint32_t>(TILE);
    };
    // Called by every lane of the claiming wave; lane 0 writes `dst`.  One
    // counter increment on the home segment; once that segment is used up,
    // one read of all counters finds the segments with tiles left.  Every
    // failed increment leaves a segment used up for good, so the loop ends.
    // The home segment's counter increment is issued by claim_issue well
    // before claim needs its result: a device-scope atomic takes ~2.5 us
    // under the bulk traffic, longer than a tile's look-back.
    auto claim_issue = [&]() -> uint32_t {
        uint32_t idx = 0u;
        if (lane == 0) idx = atomicAdd(a.seg_counter + home, 1u);
        return idx;
    };
    auto claim = [&](uint32_t *dst, uint32_t ticket) {
        uint32_t idx = __builtin_amdgcn_readfirstlane(ticket);
        while (idx >= s_segs[home].tiles) {
            const uint32_t taken = lane < kSegments
                ? __hip_atomic_load(a.seg_counter + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
            const bool open = lane < kSegments && taken < s_segs[lane < kSegments ? lane : 0].tiles;
            const uint32_t mask = static_cast<uint32_t>(__ballot(open)) & ((1u << kSegments) - 1u);
            if (mask == 0u) {
                if (lane == 0) dst[0] = kNone;
                return;
            }
            // First open segment at or after home, cyclically.
            const uint32_t rot = ((mask >> home) | (mask << (kSegments - home))) & ((1u << kSegments) - 1u);
            home = (home + static_cast<uint32_t>(__builtin_ctz(rot))) % kSegments;
            if (lane == 0) idx = atomicAdd(a.seg_counter + home, 1u);
            idx = __builtin_amdgcn_readfirstlane(idx);
        }
        if (lane == 0) publish_claim(idx, dst);
    };

    // The first claim's counter increment and the segment table's load are
    // issued before the pass's route is read, so the three round trips
    // overlap: 2^24 float keys 40.95 -> 40.25 us per pass, Morton-code
    // pairs 59.9 -> 58.3 us.  A skipped pass leaves the increment unused
    // and returns ~1 us later, and a last pass that copies the whole input
    // (no pass ran) takes ~7 us longer with it in flight: already-sorted
    // 2^28 keys 417.7 -> 409.0 Gkeys/s.  (Issued early in every pass but the
    // last, the gains and the loss were both about halved.)
    const uint32_t first_ticket = claim_wave ? claim_issue() : 0u;
    if (tid < kSegments) s_segs[tid] = a.segs[tid];
    // Route of this pass through the buffers; a trivial pass does nothing,
    // except that the last pass kernel copies the input when no pass runs.
    const PassRoute kroute = pass_route(a.trivial, a.passes, a.pass, a.keys_in_place != 0);
    if (kroute.skip) {
        clear_next_status();
        if (a.pass == a.passes - 1) {
            if (final_copy_source(a.trivial, a.passes, a.keys_in_place != 0) == 0) {
                grid_copy(static_cast<const KT *>(a.kbuf[0]), static_cast<KT *>(a.kbuf[1]), static_cast<size_t>(a.n));
            }
            if (PAIRS && final_copy_source(a.trivial, a.passes, a.vals_in_place != 0) == 0) {
                grid_copy(static_cast<const VT *>(a.vbuf[0]), static_cast<VT *>(a.vbuf[1]), static_cast<size_t>(a.n));
            }
        }
        return;
    }
    const PassRoute vroute = PAIRS ? pass_route(a.trivial, a.passes, a.pass, a.vals_in_place != 0) : kroute;
    const KT *const keys_in = static_cast<const KT *>(a.kbuf[kroute.src]);
    KT *const keys_out = static_cast<KT *>(a.kbuf[kroute.dst]);
    const VT *const vals_in = PAIRS ? static_cast<const VT *>(a.vbuf[vroute.src]) : nullptr;
    VT *const vals_out = PAIRS ? static_cast<VT *>(a.vbuf[vroute.dst]) : nullptr;

    uint32_t *const wave_cnt = s_cnt + wave * RADIX;
#pragma unroll
    for (int i = lane; i < RADIX; i += kWave) wave_cnt[i] = 0u;
    __syncthreads();  // s_segs
    if (claim_wave) {
        claim(s_claim[0], first_ticket);
        if (lane == 0) s_claim_seq = 1u;
    }
    __syncthreads();
    if (s_claim[0][0] == kNone) {  // more workgroups than tiles
        clear_next_status();
        return;
    }

    KT key[ITEMS];
    VT val[PAIRS ? ITEMS : 1];
    // Per-element offsets are derived from an opaque copy of the thread
    // index in every tile, so the compiler recomputes them instead of holding
    // one register per element across the tile loop.
    auto opaque_tid = [&]() {
        int t = tid;
        __asm__ volatile("" : "+v"(t));
        return t;
    };
    // Wave-striped load of a tile: slot j of lane l is tile element
    // wave_base + 64*j + l.  The loads go through a buffer resource covering
    // exactly the tile's valid keys, so a pad reads 0 from an out-of-range
    // offset and every thread issues the same loads for every tile (the
    // compiler can then count them exactly when it waits for them).
    auto load_tile = [&](uint32_t start_v, uint32_t valid_v) {
        // Workgroup-uniform values read from LDS: move them to scalar
        // registers so the buffer resource is scalar.
        const uint32_t start = __builtin_amdgcn_readfirstlane(start_v);
        const uint32_t valid = __builtin_amdgcn_readfirstlane(valid_v);
        const int t = opaque_tid();
        const uint32_t elem = static_cast<uint32_t>(t / kWave) * WAVE_KEYS + static_cast<uint32_t>(t & (kWave - 1));
        if constexpr (KIND == KeyKind::M30) {
            // Point i of the tile: 12 bytes at 12 i of a buffer over the
            // tile's points; the key is its code, the value its index.
            const float *pts = reinterpret_cast<const float *>(keys_in) + 3 * static_cast<size_t>(start);
            const __amdgpu_buffer_rsrc_t pr = buffer_rsrc(const_cast<float *>(pts), valid * 12u);
            u32x3_t p[ITEMS];
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) p[j] = __builtin_amdgcn_raw_buffer_load_b96(pr, (elem + j * kWave) * 12u, 0, 0);
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                // Components reinterpreted one by one from scalar copies (a
                // bit cast applied to a vector component directly was
                // compiled as a read of the vector's first component).
                const uint32_t xb = p[j].x, yb = p[j].y, zb = p[j].z;
                key[j] = morton30(__uint_as_float(xb), __uint_as_float(yb), __uint_as_float(zb), a.box);
            }
            if constexpr (PAIRS) {
#pragma unroll
                for (int j = 0; j < ITEMS; ++j) val[j] = static_cast<VT>(start + elem + static_cast<uint32_t>(j * kWave));
            }
            return;
        }
        const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(const_cast<KT *>(keys_in) + start, valid * KB);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) key[j] = buffer_load<KT>(kr, (elem + j * kWave) * KB);
        if constexpr (PAIRS) {
            const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(const_cast<VT *>(vals_in) + start, valid * VB);
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) val[j] = buffer_load<VT>(vr, (elem + j * kWave) * VB);
        }
    };
    load_tile(s_claim[0][2], s_claim[0][3]);

    // The claiming wave finishes the next tile's claim after its share of
    // the scatter, not before the third barrier, in every instance but the
    // 28-keys-per-thread keys-only kernels: there the extra live register
    // spills and the pass got 3-4% slower, while pairs (250.7 -> 231.9 us
    // per pass at 2^26) and the 16384-key keys-only tiles (2^24 keys
    // 44.4 -> 38.1 us) gain.
    constexpr bool DEFER_CLAIM = PAIRS || ITEMS != 28;
    uint32_t it = 0u;  // tiles worked on so far
    for (int cur = 0;; cur ^= 1, ++it) {
        const uint32_t tile = s_claim[cur][0];
        const uint32_t seg = s_claim[cur][1];
        const uint32_t seg_first = s_segs[seg].tile_first;
        const uint32_t valid = s_claim[cur][3];
        const bool full = valid == static_cast<uint32_t>(TILE);
        const int t_o = opaque_tid();
        const uint32_t elem0 = static_cast<uint32_t>(t_o / kWave) * WAVE_KEYS + static_cast<uint32_t>(t_o & (kWave - 1));
        auto real = [&](int j) { return full || elem0 + static_cast<uint32_t>(j * kWave) < valid; };
        auto digit = [&](int j) { return digit_field<KIND>(key[j], a.shift, width, a.mask); };

        // ---- rank within the wave ---------------------------------------------
        // The add returns how many of the wave's earlier elements have this
        // digit; afterwards the counters hold the wave's digit counts.
        // A wave in which many keys share one digit (the NaN/Inf block a
        // float sort gathers at its end, a dominant top byte, runs of equal
        // keys) would serialise those adds on one counter.  Such a wave
        // (half its lanes share lane 0's digit in slot 0; with a quarter,
        // duplicate-heavy keys whose digit is 0 a third of the time got 1-2%
        // slower) lets lane 0 add the number of lanes with lane 0's slot-0
        // digit once per slot; those lanes take the result plus the count of
        // such lanes below them (lane order is element order within a slot).
        // The other lanes add one by one, and other waves pay one compare
        // per tile.  Partial tiles take the same path with their missing
        // elements left out (a segment's last tile can be all NaN/Inf keys:
        // 2^24 float keys with 0.2% of them, 46.4 -> 42.7 us in the pass
        // that gathers them there).  Peeling the two most frequent digits of
        // a skewed pass (from its histogram) in every wave was slower:
        // duplicate-heavy pairs 256 -> 281 us per pass, float keys' top-byte
        // pass 55 -> 58 us.
        // Float keys keep each key's digit in bits 16-23 of its rank (ranks
        // are below 2^16): their digit takes a handful of operations, which
        // the LDS shuffle then need not repeat.
        // With 4-byte keys (and values) the wave counters count bytes, so a
        // rank plus its run start is directly the key's LDS byte offset.
        constexpr uint32_t UNIT = (KB == 4 && (!PAIRS || VB == 4)) ? 4u : 1u;
        constexpr uint32_t UNIT_SHIFT = UNIT == 4u ? 2u : 0u;
        constexpr bool KEEP_DIGIT = KIND == KeyKind::F32 || KIND == KeyKind::F64 || KIND == KeyKind::F16;
        // A wave rank counts at most WAVE_KEYS elements of UNIT each.
        static_assert(!KEEP_DIGIT || WAVE_KEYS * UNIT <= 65536, "rank and digit share a word");
        auto with_digit = [&](uint32_t r, uint32_t d) { return KEEP_DIGIT ? (r | (d << 16)) : r; };
        uint32_t wrank[ITEMS];
        bool dominant = false;
        uint32_t lead = 0u;
        if constexpr (RANK == kRankAtomic) {
            const uint32_t d0 = digit(0);
            lead = __builtin_amdgcn_readfirstlane(d0);
#ifndef RS_DOMINANT_LANES
#define RS_DOMINANT_LANES 32
#endif
            dominant = __popcll(__ballot(real(0) && d0 == lead)) >= RS_DOMINANT_LANES;
        }
        if constexpr (RANK == kRankMatch) {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const uint32_t dj = digit(j);
                wrank[j] = with_digit(match_rank<RBITS>(dj, real(j), wave_cnt, UNIT), dj);
            }
        } else if (dominant) {
            // Every slot issues one add per lane, except that of the lanes
            // holding `lead` only the lowest adds, for all of them; its
            // result reaches the others afterwards (readlane), so the slots'
            // adds stay back to back.
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const bool rj = real(j);
                const uint32_t dj = digit(j);
                const unsigned long long m = __ballot(rj && dj == lead);
                const uint32_t first = m != 0ull ? static_cast<uint32_t>(__builtin_ctzll(m)) : 0u;
                const bool group = rj && dj == lead;
                const uint32_t add = group ? static_cast<uint32_t>(__popcll(m)) * UNIT : UNIT;
                if (rj && (!group || static_cast<uint32_t>(lane) == first)) {
                    wrank[j] = __hip_atomic_fetch_add(wave_cnt + dj, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const bool rj = real(j);
                const uint32_t dj = digit(j);
                const unsigned long long m = __ballot(rj && dj == lead);
                const uint32_t first = m != 0ull ? static_cast<uint32_t>(__builtin_ctzll(m)) : 0u;
                const uint32_t base = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wrank[j]), first));
                const uint32_t below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
                if (rj && dj == lead) wrank[j] = base + below * UNIT;
                if (rj) wrank[j] = with_digit(wrank[j], dj);
            }
        } else {
            // Full tiles (all but at most one per segment) skip the
            // per-element range test: no masked block per element.
            auto count_all = [&](auto full_c) {
#pragma unroll
                for (int j = 0; j < ITEMS; ++j) {
                    if (decltype(full_c)::value || real(j)) {
                        const uint32_t dj = digit(j);
                        wrank[j] = with_digit(__hip_atomic_fetch_add(wave_cnt + dj, UNIT, __ATOMIC_RELAXED,
                                                                     __HIP_MEMORY_SCOPE_WORKGROUP), dj);
                    }
                }
            };
            if (full) {
                count_all(BoolC<true>{});
            } else {
                count_all(BoolC<false>{});
            }
        }
        __syncthreads();

        // ---- tile digit counts, publish, tile-sorted starts ----------------
        StatusT *const my_status = a.status + static_cast<size_t>(tile) * RADIX + tid;
        uint32_t tile_count = 0u;
        uint32_t incl = 0u;
        uint32_t wave_start[WAVES];
        if (tid < RADIX) {
            uint32_t run = 0u;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                wave_start[w] = run;
                run += s_cnt[w * RADIX + tid];
            }
            tile_count = run >> UNIT_SHIFT;
            if (tile != a.withhold_tile) {
                status_store(my_status, make_status<StatusT>(tile == seg_first ? kFlagInclusive : kFlagAggregate,
                                                             tile_count));
            }
            incl = wave_inclusive_sum(run);
            if (lane == kWave - 1) s_wave_total[wave] = incl;
        }
        __syncthreads();

        // The short first window is for the kernels of keys of up to 32 bits
        // with no values or 32-bit values (the largest tiles); those with
        // 64-bit keys or values keep kLookbackWindow.  16-bit keys were
        // measured both ways: 2^28 uint16 keys 331 us per pass with 2 words,
        // 337 us with 4.
        constexpr int LB_FIRST = (KB <= 4 && (!PAIRS || VB == 4)) ? kLookbackFirst : kLookbackWindow;
        LookbackWindow<StatusT, RADIX, LB_FIRST> lb;
        uint32_t local_start = 0u;
        if (tid < RADIX) {
            local_start = incl - (tile_count << UNIT_SHIFT);
            for (int w = 0; w < wave; ++w) local_start += s_wave_total[w];
#pragma unroll
            for (int w = 0; w < WAVES; ++w) s_cnt[w * RADIX + tid] = local_start + wave_start[w];
            local_start >>= UNIT_SHIFT;
            // First look-back window in flight while the tile is ranked.
            if (tile > seg_first) lb.fetch(a.status, tile - 1u, seg_first, tid, false);
        }
        __syncthreads();
        // Keys-only sorts start the next tile's claim here, while the tile
        // is ranked (2^28 uint32 keys 456 -> 449 us per pass).  Key-value
        // sorts start it after ranking: claimed earlier, duplicate-heavy
        // pairs got 3% slower (claim order drifts further from the order
        // tiles are worked on).
        uint32_t ticket = 0u;
        if (!PAIRS && claim_wave) ticket = claim_issue();

        // ---- tile-sorted position: wave rank + where the wave's run starts --
        auto rank_round = [&](auto full_c) {
            constexpr bool F = decltype(full_c)::value;
            uint32_t pos[ITEMS];
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                if (F || real(j)) {
                    if constexpr (KEEP_DIGIT) {
                        pos[j] = (wrank[j] & 0xFFFFu) + wave_cnt[wrank[j] >> 16];
                    } else {
                        pos[j] = wrank[j] + wave_cnt[digit(j)];
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                if (F || real(j)) {
                    if constexpr (UNIT == 4u) {
                        *reinterpret_cast<KT *>(reinterpret_cast<char *>(s_tile) + pos[j]) = key[j];
                        if constexpr (PAIRS) *reinterpret_cast<VT *>(reinterpret_cast<char *>(s_vals) + pos[j]) = val[j];
                    } else {
                        s_tile[pos[j]] = key[j];
                        if constexpr (PAIRS) s_vals[pos[j]] = val[j];
                    }
                }
            }
            // This wave's counters are not read again for this tile (its own
            // LDS operations complete in order): clear them for the next one.
#pragma unroll
            for (int i = lane; i < RADIX; i += kWave) wave_cnt[i] = 0u;
        };

        // ---- decoupled look-back over earlier tiles of the segment ----------
        auto look_back = [&]() {
            uint32_t before = 0u;
            if (tile > seg_first) {
                if (lookback_sum<kLookbackWindow>(a.status, tile, seg_first, static_cast<uint32_t>(tid), lb, before,
                                                  a.spin_limit)) {
                    if (tile != a.withhold_tile) {
                        status_store(my_status, make_status<StatusT>(kFlagInclusive, before + tile_count));
                    }
                } else {
                    atomicOr(a.error_word, 1u);
                    status_store(my_status, make_status<StatusT>(kFlagError, 0u));
                }
            }
            s_goff[tid] = a.seg_base[seg * RADIX + tid] + before - local_start;
        };

        // Digit waves rank their keys, then run the look-back (its first
        // window arrived meanwhile); the claiming wave finishes the next
        // tile's claim after ranking.
        if (full) {
            rank_round(BoolC<true>{});
        } else {
            rank_round(BoolC<false>{});
        }
        if (tid < RADIX) {
            look_back();
        } else if (claim_wave) {
            if constexpr (PAIRS) ticket = claim_issue();
            if constexpr (!DEFER_CLAIM) claim(s_claim[cur ^ 1], ticket);
        }
        __syncthreads();

        // ---- scatter digit runs --------------------------------------------
        // Tile position i holds the i-th key of the tile in sorted order.
        // Positions >= valid hold no key and are not written: their store
        // gets an offset past the end of the output, which the hardware
        // drops, so every thread issues the same stores for every tile.
        if constexpr (!WIDE) {
            const __amdgpu_buffer_rsrc_t kout = buffer_rsrc(keys_out, a.n * KB);
            __amdgpu_buffer_rsrc_t vout;
            if constexpr (PAIRS) vout = buffer_rsrc(vals_out, a.n * VB);
            const uint32_t t_w = static_cast<uint32_t>(opaque_tid());
            // Each element's store is kept in place by a scheduling barrier:
            // otherwise the compiler gathers the loop's LDS reads ahead of
            // the stores (467 -> 490 us per pass without the range test).
            // Keys-only sorts compile full tiles without the per-element
            // range test (16-bit keys 353 -> 338 us per pass, 32-bit keys
            // within 1%); with values that was 5% slower and is not done.
            auto scatter_all = [&](auto full_c) {
#pragma unroll
                for (int j = 0; j < ITEMS; ++j) {
                    const uint32_t i = static_cast<uint32_t>(j) * BLOCK + t_w;
                    const KT k = s_tile[i];
                    // Element index; past the end of the output for pads.
                    const uint32_t o = (decltype(full_c)::value || full || i < valid)
                        ? s_goff[digit_field<KIND>(k, a.shift, width, a.mask)] + i : 0x3FFFFFFFu;
                    buffer_store<KT>(k, kout, o * KB);
                    if constexpr (PAIRS) buffer_store<VT>(s_vals[i], vout, o * VB);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            if (!PAIRS && full) {
                scatter_all(BoolC<true>{});
            } else {
                scatter_all(BoolC<false>{});
            }
        } else {
            const uint32_t t_w = static_cast<uint32_t>(opaque_tid());
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const uint32_t i = static_cast<uint32_t>(j) * BLOCK + t_w;
                if (i < valid) {
                    const KT k = s_tile[i];
                    const size_t o = static_cast<size_t>(s_goff[digit_field<KIND>(k, a.shift, width, a.mask)]) + i;
                    if (o < a.n) {
                        keys_out[o] = k;
                        if constexpr (PAIRS) vals_out[o] = s_vals[i];
                    }
                }
            }
        }
        // ---- next tile's claim and loads -------------------------------------
        // With DEFER_CLAIM the claiming wave finishes the next tile's claim
        // after its share of the scatter (the counter increment has long
        // returned) and publishes it; the other waves wait for that in LDS.
        // Finishing it before the third barrier made that barrier wait for
        // the atomic.  The wait is bounded: past the bound the error word is
        // set and the workgroup stops.
        bool stop = false;
        if constexpr (DEFER_CLAIM) {
            const uint32_t want = it + 2u;
            if (claim_wave) {
                claim(s_claim[cur ^ 1], ticket);
                if (lane == 0) __hip_atomic_store(&s_claim_seq, want, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                uint32_t spins = 0u;
                while (__hip_atomic_load(&s_claim_seq, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < want) {
                    if (++spins > kSpinLimit) {
                        if (lane == 0) atomicOr(a.error_word, 1u);
                        stop = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
        }
        // Loads issued after this tile's stores: a wave's memory operations go
        // through the memory pipeline in order, and stores queued behind a
        // tile of loads would wait for those loads.
        const uint32_t next = s_claim[cur ^ 1][0];
        if (stop || next == kNone) break;
        load_tile(s_claim[cur ^ 1][2], s_claim[cur ^ 1][3]);
        // No barrier here: until the next tile's first barrier a wave only
        // touches its own counters, and the LDS this tile's scatter reads
        // (s_tile, s_vals, s_goff) is next written after the next tile's
        // third barrier.  Waves that finish early start counting.
    }
    clear_next_status();
}

// ---------------------------------------------------------------------------
// Probe of the LDS property the local rank relies on (a measurement hook,
// not part of the sort): every wave of every workgroup holds SLOTS digits
// per lane, slot j of lane l being element 64 j + l of the wave, and adds
// `unit` per element to its own (wave, digit) counter, all slots issued back
// to back as the pass kernel issues them.  What each add returns is stored,
// so the host can check that it equals `unit` times the number of the
// wave's earlier elements (in slot, then lane order) with the same digit.
// digits and ranks hold gridDim.x * BLOCK * SLOTS words.
// ---------------------------------------------------------------------------
template <int BLOCK, int SLOTS>
__global__ __launch_bounds__(BLOCK) void lds_rank_probe_kernel(const uint32_t *digits, uint32_t *ranks,
                                                               uint32_t unit) {
    constexpr int RADIX = 256;
    constexpr int WAVES = BLOCK / kWave;
    __shared__ uint32_t s_cnt[WAVES * RADIX];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    for (int i = tid; i < WAVES * RADIX; i += BLOCK) s_cnt[i] = 0u;
    __syncthreads();
    uint32_t *const wave_cnt = s_cnt + wave * RADIX;
    const size_t base = (static_cast<size_t>(blockIdx.x) * WAVES + wave) * SLOTS * kWave + lane;
    uint32_t d[SLOTS], r[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) d[j] = digits[base + static_cast<size_t>(j) * kWave] & (RADIX - 1);
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
        r[j] = __hip_atomic_fetch_add(wave_cnt + d[j], unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) ranks[base + static_cast<size_t>(j) * kWave] = r[j];
}

// ---------------------------------------------------------------------------
// Small inputs: the whole sort in one launch.  For a few tiles the fixed
// cost of a launch per step (fill, histogram, base, one per pass) dominates,
// so here one launch runs every step as phases: phase 0 counts the digits
// of every pass over the input (the totals give each digit's start), phase
// 1 + p runs pass p tile by tile (count, publish, look back over the earlier
// tiles -- the pass kernel's chained scan, one chain -- rank, scatter).
// Workgroups claim the tiles of each phase from a counter in order and a
// phase starts once every tile of the one before is done, so the launch
// needs no more than one resident workgroup to finish: a look-back only
// waits for tiles claimed earlier, and a phase wait only for claimed tiles
// or tiles any running workgroup will claim.  A workgroup claims its first
// tile of the next phase in the same step as its last claim of the current
// one, before it waits.
// ---------------------------------------------------------------------------
// Status words per look-back window of the small path.
constexpr int kSmallLookback = 8;
constexpr int kSmallPhases = kMaxPasses + 1;

struct SmallArgs {
    const void *keys_in;         // caller input
    const void *vals_in;         // caller input values (pairs)
    void *kbuf[2];               // [0] caller output, [1] temp; pass p writes kbuf[(passes-1-p) & 1]
    void *vbuf[2];
    uint32_t *hist;              // [passes][RADIX] digit totals, zero on entry
    uint32_t *status;            // [passes][tiles][RADIX] chained-scan words, zero on entry
    uint32_t *claimed;           // [kSmallPhases] tiles claimed per phase, zero on entry
    uint32_t *done;              // [kSmallPhases] tiles finished per phase, zero on entry
    uint32_t *error_word;
    uint32_t n;
    uint32_t tiles;
    int passes;
    // An in-place sort with an odd number of passes has pass 0 write the
    // caller's buffer, which other tiles of pass 0 may not have read yet:
    // phase 0 then copies the keys (values) to temp, and pass 0 reads there.
    int copy_keys;
    int copy_vals;
    uint32_t shift[kMaxPasses];
    uint32_t mask[kMaxPasses];
};

template <int BLOCK, int ITEMS, int RBITS, KeyKind KIND, bool PAIRS, class VT = uint32_t, int RANK = kRankAtomic>
__global__ __launch_bounds__(BLOCK) void small_sort_kernel(SmallArgs a) {
    using KT = key_t<KIND>;
    constexpr int RADIX = 1 << RBITS;
    constexpr int WAVES = BLOCK / kWave;
    constexpr int TILE = BLOCK * ITEMS;
    constexpr int WAVE_KEYS = kWave * ITEMS;
    constexpr int MAXP = (8 * static_cast<int>(sizeof(KT)) + RBITS - 1) / RBITS;
    constexpr uint32_t KB = sizeof(KT);
    static_assert(BLOCK >= RADIX && RADIX % kWave == 0, "one thread per digit");
    static_assert(MAXP <= kMaxPasses, "too many passes");
    __shared__ KT s_tile[TILE];
    constexpr uint32_t VB = sizeof(VT);
    __shared__ VT s_vals[PAIRS ? TILE : 1];
    __shared__ uint32_t s_cnt[WAVES * RADIX];
    __shared__ uint32_t s_hist[MAXP * RADIX];
    __shared__ uint32_t s_goff[RADIX];
    __shared__ uint32_t s_tile_total[RADIX / kWave];
    __shared__ uint32_t s_digit_total[RADIX / kWave];
    __shared__ uint32_t s_claim[2];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const uint32_t tiles = a.tiles;
    // Slot j of lane l of wave w: tile element w * WAVE_KEYS + 64 j + l.
    const uint32_t elem0 = static_cast<uint32_t>(wave) * WAVE_KEYS + static_cast<uint32_t>(lane);
    uint32_t *const wave_cnt = s_cnt + wave * RADIX;

    // ---- claims and phase waits ------------------------------------------
    // Claims a tile of `phase` and, if `also` >= 0, the first of phase `also`
    // in the same round trip.  (Issued before the tile's scatter, so that
    // the round trip overlaps it, the claims made 2^16 keys 4% slower.)
    auto claim = [&](int phase, int also) {
        if (tid == 0) {
            const uint32_t t = atomicAdd(a.claimed + phase, 1u);
            const uint32_t u = also >= 0 ? atomicAdd(a.claimed + also, 1u) : 0u;
            s_claim[0] = t;
            s_claim[1] = u;
        }
        __syncthreads();
        const uint32_t t = s_claim[0], u = s_claim[1];
        __syncthreads();  // s_claim is written again by the next claim
        return uint2{t, u};
    };
    // `count` finished tiles of `phase`: every wave's stores are complete,
    // then released device-wide before they are counted.
    auto finish = [&](int phase, uint32_t count) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt 0
        __syncthreads();
        if (tid == 0 && count != 0u) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            atomicAdd(a.done + phase, count);
        }
    };
    // Waits (bounded) until every tile of `phase` is finished, then acquires.
    // Only the waiting thread runs the acquire fence: the other waves issue
    // no load until the barrier after it, and the caches it invalidates are
    // the ones their loads go through (a fence in every wave: 2^16 keys
    // 1.70 -> 1.84 Gkeys/s without it).
    auto wait_phase = [&](int phase) {
        if (tid == 0) {
            uint32_t spins = 0u;
            while (__hip_atomic_load(a.done + phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < tiles) {
                if (__hip_atomic_load(a.error_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
                if (++spins > kSpinLimit) {
                    atomicOr(a.error_word, 1u);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
    };

    KT key[ITEMS];
    VT val[PAIRS ? ITEMS : 1];
    auto load_tile = [&](const void *kin, const void *vin, uint32_t start, uint32_t valid, bool with_values) {
        const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(const_cast<KT *>(static_cast<const KT *>(kin)) + start, valid * KB);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) key[j] = buffer_load<KT>(kr, (elem0 + j * kWave) * KB);
        if constexpr (PAIRS) {
            if (with_values) {
                const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(const_cast<VT *>(static_cast<const VT *>(vin)) + start, valid * VB);
#pragma unroll
                for (int j = 0; j < ITEMS; ++j) val[j] = buffer_load<VT>(vr, (elem0 + j * kWave) * VB);
            }
        }
    };
    auto tile_valid = [&](uint32_t t) {
        const uint32_t left = a.n - t * static_cast<uint32_t>(TILE);
        return left < static_cast<uint32_t>(TILE) ? left : static_cast<uint32_t>(TILE);
    };

    // ---- phase 0: histograms of every pass, from the input ------------------
    for (int i = tid; i < MAXP * RADIX; i += BLOCK) s_hist[i] = 0u;
    for (int i = tid; i < WAVES * RADIX; i += BLOCK) s_cnt[i] = 0u;
    uint2 c = claim(0, -1);
    uint32_t counted = 0u;
    uint32_t next = 0u;
    bool have_next = false;
    while (c.x < tiles) {
        const uint32_t valid = tile_valid(c.x);
        const uint32_t start = c.x * static_cast<uint32_t>(TILE);
        load_tile(a.keys_in, a.vals_in, start, valid, a.copy_vals != 0);
        if (a.copy_keys) {
            KT *const to = static_cast<KT *>(a.kbuf[1]) + start;
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                if (elem0 + static_cast<uint32_t>(j * kWave) < valid) to[elem0 + j * kWave] = key[j];
            }
        }
        if constexpr (PAIRS) {
            if (a.copy_vals) {
                VT *const to = static_cast<VT *>(a.vbuf[1]) + start;
#pragma unroll
                for (int j = 0; j < ITEMS; ++j) {
                    if (elem0 + static_cast<uint32_t>(j * kWave) < valid) to[elem0 + j * kWave] = val[j];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            if (elem0 + static_cast<uint32_t>(j * kWave) < valid) {
                const KT k = ordered_key<KIND>(key[j]);
#pragma unroll
                for (int p = 0; p < MAXP; ++p) {
                    if (p < a.passes) atomicAdd(&s_hist[p * RADIX + (static_cast<uint32_t>(k >> a.shift[p]) & a.mask[p])], 1u);
                }
            }
        }
        ++counted;
        c = claim(0, have_next ? -1 : 1);
        if (!have_next) {
            next = c.y;
            have_next = true;
        }
    }
    if (!have_next) next = claim(1, -1).x;
    __syncthreads();
    if (counted != 0u) {
        for (int i = tid; i < a.passes * RADIX; i += BLOCK) {
            if (s_hist[i] != 0u) atomicAdd(&a.hist[i], s_hist[i]);
        }
    }
    finish(0, counted);
    wait_phase(0);
    // Digit totals of every pass, kept in LDS for the passes.
    for (int i = tid; i < a.passes * RADIX; i += BLOCK) s_hist[i] = a.hist[i];
    __syncthreads();

    // ---- phases 1 + p: the passes ------------------------------------------
    for (int p = 0; p < a.passes; ++p) {
        const int phase = 1 + p;
        const int dst = (a.passes - 1 - p) & 1;
        const int src = (a.passes - p) & 1;  // where pass p - 1 wrote
        const uint32_t shift = a.shift[p], mask = a.mask[p];
        auto digit = [&](KT k) { return digit_of<KIND>(k, shift, mask); };
        uint32_t *const status = a.status + static_cast<size_t>(p) * tiles * RADIX;
        const bool last = p + 1 == a.passes;
        uint32_t tile = next;
        have_next = last;  // no phase after the last pass
        while (tile < tiles) {
            const uint32_t start = tile * static_cast<uint32_t>(TILE);
            const uint32_t valid = tile_valid(tile);
            auto real = [&](int j) { return elem0 + static_cast<uint32_t>(j * kWave) < valid; };
            if (p == 0) {
                load_tile(a.copy_keys ? a.kbuf[1] : a.keys_in, a.copy_vals ? a.vbuf[1] : a.vals_in, start, valid, true);
            } else {
                load_tile(a.kbuf[src], a.vbuf[src], start, valid, true);
            }

            // Rank within the wave (the counters then hold the wave's counts).
            uint32_t wrank[ITEMS];
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                if constexpr (RANK == kRankMatch) {
                    wrank[j] = match_rank<RBITS>(digit(key[j]), real(j), wave_cnt, 1u);
                } else if (real(j)) {
                    wrank[j] = __hip_atomic_fetch_add(wave_cnt + digit(key[j]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
            __syncthreads();

            // Tile counts: publish, then wave scans of the tile counts and
            // of the digit totals.
            uint32_t wave_start[WAVES];
            uint32_t tile_count = 0u, tile_incl = 0u, total = 0u, total_incl = 0u;
            LookbackWindow<uint32_t, RADIX, kSmallLookback> lb;
            if (tid < RADIX) {
                uint32_t run = 0u;
#pragma unroll
                for (int w = 0; w < WAVES; ++w) {
                    wave_start[w] = run;
                    run += s_cnt[w * RADIX + tid];
                }
                tile_count = run;
                status_store(status + static_cast<size_t>(tile) * RADIX + tid,
                             make_status<uint32_t>(tile == 0u ? kFlagInclusive : kFlagAggregate, tile_count));
                if (tile > 0u) lb.fetch(status, tile - 1u, 0u, static_cast<uint32_t>(tid), true);
                total = s_hist[p * RADIX + tid];
                tile_incl = wave_inclusive_sum(tile_count);
                total_incl = wave_inclusive_sum(total);
                if (lane == kWave - 1) {
                    s_tile_total[wave] = tile_incl;
                    s_digit_total[wave] = total_incl;
                }
            }
            __syncthreads();
            uint32_t local_start = 0u, digit_start = 0u;
            if (tid < RADIX) {
                local_start = tile_incl - tile_count;
                digit_start = total_incl - total;
                for (int w = 0; w < wave; ++w) {
                    local_start += s_tile_total[w];
                    digit_start += s_digit_total[w];
                }
#pragma unroll
                for (int w = 0; w < WAVES; ++w) s_cnt[w * RADIX + tid] = local_start + wave_start[w];
            }
            __syncthreads();

            // Tile-sorted position: wave rank + the wave's run start (while
            // the first look-back window is in flight).
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                if (real(j)) {
                    const uint32_t pos = wrank[j] + wave_cnt[digit(key[j])];
                    s_tile[pos] = key[j];
                    if constexpr (PAIRS) s_vals[pos] = val[j];
                }
            }
#pragma unroll
            for (int i = lane; i < RADIX; i += kWave) wave_cnt[i] = 0u;
            // Look-back over the earlier tiles (one chain over the input).
            if (tid < RADIX) {
                uint32_t before = 0u;
                if (tile > 0u) {
                    if (lookback_sum<kSmallLookback>(status, tile, 0u, static_cast<uint32_t>(tid), lb, before)) {
                        status_store(status + static_cast<size_t>(tile) * RADIX + tid,
                                     make_status<uint32_t>(kFlagInclusive, before + tile_count));
                    } else {
                        atomicOr(a.error_word, 1u);
                        status_store(status + static_cast<size_t>(tile) * RADIX + tid, make_status<uint32_t>(kFlagError, 0u));
                    }
                }
                s_goff[tid] = digit_start + before - local_start;
            }
            __syncthreads();

            // Scatter the tile's digit runs.
            KT *const kout = static_cast<KT *>(a.kbuf[dst]);
            VT *const vout = static_cast<VT *>(a.vbuf[dst]);
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const uint32_t i = static_cast<uint32_t>(j) * BLOCK + static_cast<uint32_t>(tid);
                if (i < valid) {
                    const KT k = s_tile[i];
                    const uint32_t o = s_goff[digit(k)] + i;
                    if (o < a.n) {  // always, unless a wait gave up (error word set)
                        kout[o] = k;
                        if constexpr (PAIRS) vout[o] = s_vals[i];
                    }
                }
            }
            finish(phase, 1u);
            const uint2 cc = claim(phase, have_next ? -1 : phase + 1);
            tile = cc.x;
            if (!have_next) {
                next = cc.y;
                have_next = true;
            }
        }
        if (!last) {
            if (!have_next) next = claim(phase + 1, -1).x;
            wait_phase(phase);
        }
    }
}

}  // namespace rs
