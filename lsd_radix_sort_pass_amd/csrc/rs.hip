// rs.hip -- host planner and C ABI of the gfx950 stable LSD radix sort.
//
// Plan of one sort of n keys over [begin_bit, end_bit) with RADIX_BITS-wide
// digits ([WA] "La idea y el requisito de estabilidad": one pass per digit,
// least significant first; [WA] "Claves con signo...": fewer significant
// bits means fewer passes):
//     P = ceil((end_bit - begin_bit) / RADIX_BITS) passes, pass p on digit
//     shift = begin_bit + p*RADIX_BITS, width min(RADIX_BITS, end_bit - shift).
// Launch sequence on the caller's stream:
//     fill (zero scan state) -> hist (all P histograms, one read of the keys)
//     -> digit_base (exclusive scan per pass) -> P x onesweep pass
//     [-> copy, only for an in-place sort with odd P].
// Passes ping-pong between the output buffer and a temp buffer
// ([WA] "Las tres fases": source and destination swap every pass), arranged
// so that the last pass writes the caller's output.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <type_traits>
#include <vector>

#include "kernels.hpp"
#include "rs.h"
#include "rs_prof.h"

namespace {

using rs::KeyKind;

constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kPassBlock = 1024;
constexpr int kMaxPasses = 64 / kRadixBits;  // 64-bit keys
constexpr int key_bytes(KeyKind k) {
    return (k == KeyKind::U64 || k == KeyKind::I64 || k == KeyKind::F64) ? 8
         : (k == KeyKind::U16 || k == KeyKind::I16 || k == KeyKind::F16) ? 2 : 4;
}
// Keys per thread of a pass tile (kb key bytes, vb value bytes, 0 for keys
// only): keys-only tiles are larger (fewer tiles, fewer look-back steps);
// with values the tile's keys and values must both fit in LDS, and 64-bit
// keys or values take more registers and LDS.
//   16/32-bit keys: 28672-key tiles, 17408 with 32-bit values, 11264 with 64-bit;
//   64-bit keys: 14336-key tiles, 11264 with 32-bit values, 8192 with 64-bit.
// The key-value tiles are the most that fit in LDS beside the wave counters
// (17408 pairs of 4-byte keys and values: 153 KiB in all): 16384-pair tiles
// took duplicate-heavy 2^26 pairs 229.9 us per pass against 226.4,
// Morton-code pairs at 2^24 59.6 against 58.6; 10240-pair tiles of 32-bit
// keys and 64-bit values 334.1 against 330.9 at 2^26.
constexpr int pass_items(int vb, int kb) {
    return kb == 8 ? (vb == 0 ? 14 : vb == 4 ? 11 : 8) : (vb == 0 ? 28 : vb == 4 ? 17 : 11);
}
// Keys-only sorts of 32-bit keys below 2^30 may instead take tiles of
// kShortItems keys per thread: a pass costs about (rounds of tiles over the
// resident workgroups) x (time of one tile), and a short tile takes ~0.70 of
// a long one.  When the long tiles' last round is mostly empty (2^24 keys:
// 2.3 rounds of 28672-key tiles, exactly 4 of 16384-key ones) the short
// tiles finish first.
constexpr int kShortItems = 16;
constexpr bool short_tiles_allowed(int vb, int kb) { return vb == 0 && kb == 4; }
int g_tile_items = 0;  // rs_prof_tile_items: 0 automatic, else forced keys per thread

constexpr int kHistBlock = 1024;
constexpr int hist_items(int kb) { return kb == 8 ? 8 : 16; }
constexpr int kHistMaxGrid = 256;
constexpr unsigned kHistMinUnits = 16;
// LDS counter copies per histogram bin: as many as fit in LDS (the
// histogram kernel counts every segment of passes >= 1; 64-bit keys have
// twice the passes).
#ifndef HIST_REPL
#define HIST_REPL (rs::kSegments > 8 ? 2 : 4)
#endif
constexpr int hist_repl(int kb) { return kb == 8 ? 2 : HIST_REPL; }
constexpr size_t kTempAlign = 256;
// Header words: 0 error flag; 1 + p*kSegments + s tile counters; from
// kTrivialWord one flag per pass (1 = the pass moves nothing, skipped);
// kUnsortedWord 1 once two adjacent keys are out of sub-key order; from
// kSegModeWord one word per pass, 1 when its segments are position ranges
// cut at the sampled boundaries at byte kBoundsByte ([kMaxPasses][kSegments
// - 1] u32).  Those words are written by the sampling step, never zeroed.
constexpr int kTrivialWord = 1 + kMaxPasses * rs::kSegments;
constexpr int kUnsortedWord = kTrivialWord + kMaxPasses;
constexpr int kSegModeWord = (kUnsortedWord + 1 + 3) / 4 * 4;  // 16-byte aligned: zeroing stops exactly there
constexpr size_t kBoundsByte = 4 * (kSegModeWord + kMaxPasses);
constexpr size_t kHeaderBytes =
    ((kBoundsByte + 4 * kMaxPasses * (rs::kSegments - 1) + 255) / 256) * 256;
// Inputs from this size on (keys of up to 32 bits) take the sampling step
// that balances skewed passes' segments by position.
constexpr size_t kSampleMinKeys = size_t{1} << 22;
// Inputs from this size on use 64-bit status words (counts beyond the
// 30-bit field of a 32-bit word) and 64-bit store addresses (32-bit buffer
// offsets cover 2^32 bytes of keys or values).  The limit sits 2^16
// elements below 2^30 (2^29 for 8-byte keys or values) so that the byte
// offset the pass kernel gives a pad's dropped store (element 2^30 - 1,
// truncated to 32 bits) always lies at least 2^17 bytes past the end of the
// output buffer, never exactly at its end.
constexpr size_t wide_limit(int kb, int vb) {
    return ((kb == 8 || vb == 8) ? size_t{1} << 29 : size_t{1} << 30) - (size_t{1} << 16);
}

size_t align_up(size_t x) { return (x + kTempAlign - 1) & ~(kTempAlign - 1); }

struct Layout {
    int passes = 0;
    uint32_t tile = 0;         // keys per pass tile
    uint32_t tiles0 = 0;       // tiles of pass 0 (tile-aligned segments)
    uint32_t tiles_max = 0;    // upper bound on any pass's tiles: segments end in partial tiles
    bool wide_status = false;
    size_t off_header = 0;     // word 0: error flag; words 1 + p*kSegments + s: tile counters
    size_t off_hist = 0;       // [passes][kSegments][radix] u32
    size_t off_base = 0;       // [passes][kSegments][radix] u32
    size_t off_segs = 0;       // [passes][kSegments] rs::SegmentInfo
    size_t off_status[2] = {0, 0};
    size_t zero_bytes = 0;     // [0, zero_bytes) is zeroed before each sort
    size_t off_alt_keys = 0;
    size_t off_alt_vals = 0;
    size_t total = 0;
};

// Small inputs, at most kSmallMaxTiles tiles of kSmallTile keys, are sorted
// in one launch (small_sort_kernel).  Temp: header (word 0 the error word,
// then the per-phase claim and finish counters), digit totals
// [passes][radix], chained-scan words [passes][tiles][radix], alternate keys
// and values.
#ifndef RS_SMALL_BLOCK
#define RS_SMALL_BLOCK 512
#endif
#ifndef RS_SMALL_MAX_TILES
#define RS_SMALL_MAX_TILES 16
#endif
constexpr int kSmallBlock = RS_SMALL_BLOCK;
constexpr int kSmallItems = 8;
constexpr uint32_t kSmallTile = kSmallBlock * kSmallItems;
constexpr uint32_t kSmallMaxTiles = RS_SMALL_MAX_TILES;

struct SmallLayout {
    int passes = 0;
    uint32_t tiles = 0;
    size_t off_hist = 0;
    size_t off_status = 0;
    size_t zero_bytes = 0;
    size_t off_alt_keys = 0;
    size_t off_alt_vals = 0;
    size_t total = 0;
};

int g_small_path = 1;  // rs_prof_small_path: 0 off, 1 on, 2 on with one workgroup
// rs_prof_force_giveup: pass 0 never publishes the status words of its tile
// 0, and every look-back gives up after kGiveupSpins polls of an empty word.
bool g_force_giveup = false;
// rs_prof_ranker: 0 the LDS-atomic local rank, 1 the ballot match ranker (for
// the kinds match_ranker_kind accepts).
int g_ranker = 0;
constexpr bool match_ranker_kind(KeyKind k, int vb) {
    return (k == KeyKind::U32 || k == KeyKind::I32 || k == KeyKind::F32) && (vb == 0 || vb == 4);
}
constexpr uint32_t kGiveupSpins = 64;

bool small_input(size_t n) { return n >= 2 && n <= size_t{kSmallMaxTiles} * kSmallTile; }

bool valid_bits(int begin_bit, int end_bit, int kb) {
    return begin_bit >= 0 && end_bit <= 8 * kb && begin_bit <= end_bit;
}

bool trivial(size_t n, int begin_bit, int end_bit) { return n <= 1 || begin_bit == end_bit; }

// kb key bytes; vb value bytes (0 without values).
// items: keys per thread of a pass tile (0: the default for the widths).
Layout make_layout(size_t n, int vb, int begin_bit, int end_bit, int kb, int items = 0) {
    Layout L;
    L.passes = (end_bit - begin_bit + kRadixBits - 1) / kRadixBits;
    L.tile = static_cast<uint32_t>(kPassBlock * (items > 0 ? items : pass_items(vb, kb)));
    L.tiles0 = static_cast<uint32_t>((n + L.tile - 1) / L.tile);
    L.tiles_max = L.tiles0 + rs::kSegments;
    L.wide_status = n >= wide_limit(kb, vb);
    const size_t status_bytes = align_up(size_t{L.tiles_max} * kRadix * (L.wide_status ? 8 : 4));
    size_t off = 0;
    L.off_header = off;
    off += kHeaderBytes;
    L.off_hist = off;
    off += align_up(size_t(L.passes) * rs::kSegments * kRadix * 4);
    L.off_status[0] = off;
    off += status_bytes;
    L.zero_bytes = off;
    L.off_status[1] = off;
    off += L.passes > 1 ? status_bytes : 0;
    L.off_base = off;
    off += align_up(size_t(L.passes) * rs::kSegments * kRadix * 4);
    L.off_segs = off;
    off += align_up(size_t(L.passes) * rs::kSegments * sizeof(rs::SegmentInfo));
    L.off_alt_keys = off;
    off += align_up(n * kb);
    L.off_alt_vals = off;
    off += align_up(n * vb);
    L.total = off;
    return L;
}

SmallLayout make_small_layout(size_t n, int vb, int begin_bit, int end_bit, int kb) {
    SmallLayout S;
    S.passes = (end_bit - begin_bit + kRadixBits - 1) / kRadixBits;
    S.tiles = static_cast<uint32_t>((n + kSmallTile - 1) / kSmallTile);
    size_t off = kTempAlign;  // header
    S.off_hist = off;
    off += align_up(size_t(S.passes) * kRadix * 4);
    S.off_status = off;
    off += align_up(size_t(S.passes) * S.tiles * kRadix * 4);
    S.zero_bytes = off;
    S.off_alt_keys = off;
    off += align_up(n * kb);
    S.off_alt_vals = off;
    off += align_up(n * vb);
    S.total = off;
    return S;
}

// Temp bytes a non-trivial sort needs: enough for the multi-launch path,
// and for the one-launch path when the input is small.
size_t temp_need(size_t n, int vb, int begin_bit, int end_bit, int kb) {
    size_t need = make_layout(n, vb, begin_bit, end_bit, kb).total;
    if (short_tiles_allowed(vb, kb)) {
        // Either tile size may be chosen at sort time (more, smaller tiles
        // need more status words).
        const size_t short_need = make_layout(n, vb, begin_bit, end_bit, kb, kShortItems).total;
        if (short_need > need) need = short_need;
    }
    if (small_input(n)) {
        const size_t small = make_small_layout(n, vb, begin_bit, end_bit, kb).total;
        if (small > need) need = small;
    }
    return need;
}

// ---------------------------------------------------------------------------
// Per-kernel event timing (rs_prof.h).
// ---------------------------------------------------------------------------
struct ProfRecord {
    int kind;
    int sub;  // pass index of a pass launch, else -1
    hipEvent_t start;
    hipEvent_t stop;
};

struct ProfSample {
    int sub;
    double ms;
};

struct Prof {
    bool on = false;
    std::mutex mu;
    std::vector<ProfRecord> pending;
    std::vector<hipEvent_t> spare;
    uint64_t launches[RS_KERNEL_KINDS] = {};
    double ms[RS_KERNEL_KINDS] = {};
    std::vector<ProfSample> samples[RS_KERNEL_KINDS];
};

Prof &prof() {
    static Prof p;
    return p;
}

hipEvent_t take_event(Prof &p) {
    if (!p.spare.empty()) {
        hipEvent_t e = p.spare.back();
        p.spare.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Timing events of the launch under way (set by launch_kernel while timing
// is on, else null).
thread_local hipEvent_t t_launch_start = nullptr;
thread_local hipEvent_t t_launch_stop = nullptr;

// Enqueues kernel<<<grid, block, 0, stream>>>(args...); while a launch is
// timed, the timing events are attached to the dispatch itself.
template <class... KArgs, class... Args>
void run_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream, Args... args) {
    if (t_launch_start != nullptr) {
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, t_launch_start, t_launch_stop, 0,
                              static_cast<KArgs>(args)...);
    } else {
        kernel<<<grid, block, 0, stream>>>(static_cast<KArgs>(args)...);
    }
}

// Runs `launch` (which enqueues one kernel on `stream` with run_kernel) and
// reports whether the launch succeeded; times it while timing is on.  `sub`
// tags the record (the pass index of a pass launch).
template <class F>
bool launch_kernel(int kind, hipStream_t stream, F &&launch, int sub = -1) {
    Prof &p = prof();
    if (!p.on) {
        launch();
        return hipGetLastError() == hipSuccess;
    }
    std::lock_guard<std::mutex> lock(p.mu);
    hipEvent_t a = take_event(p);
    hipEvent_t b = take_event(p);
    // The launch attaches the pair to the kernel's dispatch (run_kernel):
    // they stamp the kernel's own start and end, as a profiler's trace does.
    // (A pair recorded around the launch added ~3.5 us per launch at 2^28.)
    if (a && b) {
        t_launch_start = a;
        t_launch_stop = b;
    }
    launch();
    t_launch_start = nullptr;
    t_launch_stop = nullptr;
    const bool ok = hipGetLastError() == hipSuccess;
    if (a && b) {
        p.pending.push_back({kind, sub, a, b});
    } else {
        if (a) p.spare.push_back(a);
        if (b) p.spare.push_back(b);
    }
    return ok;
}

unsigned grid_for(size_t work, unsigned per_block, unsigned max_grid) {
    size_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > max_grid) g = max_grid;
    return static_cast<unsigned>(g);
}

bool launch_copy(const uint32_t *in, uint32_t *out, size_t n, hipStream_t stream);

// n elements of elem_bytes bytes (2, 4 or 8): whole 32-bit words where the
// buffers allow, else 16-bit halves.
bool launch_copy_elems(const void *in, void *out, size_t n, int elem_bytes, hipStream_t stream) {
    const size_t bytes = n * static_cast<size_t>(elem_bytes);
    const bool words = bytes % 4 == 0 && reinterpret_cast<uintptr_t>(in) % 4 == 0 &&
                       reinterpret_cast<uintptr_t>(out) % 4 == 0;
    if (words) return launch_copy(static_cast<const uint32_t *>(in), static_cast<uint32_t *>(out), bytes / 4, stream);
    if (n == 0 || in == out) return true;
    const size_t halves = bytes / 2;
    const unsigned grid = grid_for(halves, 256, 8192);
    return launch_kernel(RS_KERNEL_COPY, stream, [&] {
        run_kernel(rs::copy_u16_kernel, grid, 256, stream, static_cast<const uint16_t *>(in), static_cast<uint16_t *>(out), halves);
    });
}

// Compute units of the current device (256 when the query fails).
unsigned device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        return 256u;
    }
    return static_cast<unsigned>(cus);
}

bool launch_copy(const uint32_t *in, uint32_t *out, size_t n, hipStream_t stream) {
    if (n == 0 || in == out) return true;
    const bool vec = (reinterpret_cast<uintptr_t>(in) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(out) % 16 == 0) && (n % 4 == 0);
    if (vec) {
        const size_t n4 = n / 4;
        const unsigned grid = grid_for(n4, rs::kCopyBlock * rs::kCopyUnroll, device_cus());
        return launch_kernel(RS_KERNEL_COPY, stream, [&] {
            run_kernel(rs::copy_u128_kernel, grid, rs::kCopyBlock, stream, reinterpret_cast<const uint4 *>(in),
                                                                     reinterpret_cast<uint4 *>(out), n4);
        });
    }
    const unsigned grid = grid_for(n, 256, 8192);
    return launch_kernel(RS_KERNEL_COPY, stream, [&] {
        run_kernel(rs::copy_u32_kernel, grid, 256, stream, in, out, n);
    });
}

// ---------------------------------------------------------------------------
// Validation (host only, before any HIP call).
// ---------------------------------------------------------------------------
struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

Span span_of(const void *p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + bytes};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

// In/out pair: identical start (in place) or disjoint.
bool same_or_disjoint(Span a, Span b) { return a.lo == b.lo || !overlap(a, b); }

// vb: value bytes (0 for keys only), kb: key bytes.  own_scratch: temp is
// the library's fixed scratch of temp_bytes bytes, whose address is not yet
// looked up; only its size is checked.
rs_status validate(const void *kin, const void *kout, const void *vin, const void *vout, int vb,
                   size_t n, int begin_bit, int end_bit, const void *temp, size_t temp_bytes, int kb,
                   bool own_scratch = false) {
    const bool pairs = vb != 0;
    if (!valid_bits(begin_bit, end_bit, kb)) return RS_ERROR_INVALID_VALUE;
    if (n > RS_MAX_ELEMENTS) return RS_ERROR_INVALID_VALUE;
    if (n == 0) return RS_SUCCESS;
    if (!kin || !kout) return RS_ERROR_INVALID_VALUE;
    if (pairs && (!vin || !vout)) return RS_ERROR_INVALID_VALUE;
    const auto misaligned = [](const void *p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; };
    if (misaligned(kin, kb) || misaligned(kout, kb)) return RS_ERROR_INVALID_VALUE;
    if (pairs && (misaligned(vin, vb) || misaligned(vout, vb))) return RS_ERROR_INVALID_VALUE;
    const size_t bytes = n * static_cast<size_t>(vb);  // values
    const size_t kbytes = n * kb;     // keys
    const Span ki = span_of(kin, kbytes), ko = span_of(kout, kbytes);
    if (!same_or_disjoint(ki, ko)) return RS_ERROR_INVALID_VALUE;
    if (pairs) {
        const Span vi = span_of(vin, bytes), vo = span_of(vout, bytes);
        if (!same_or_disjoint(vi, vo)) return RS_ERROR_INVALID_VALUE;
        if (overlap(ki, vi) || overlap(ki, vo) || overlap(ko, vi) || overlap(ko, vo)) {
            return RS_ERROR_INVALID_VALUE;
        }
    }
    if (trivial(n, begin_bit, end_bit)) return RS_SUCCESS;
    const size_t need = temp_need(n, vb, begin_bit, end_bit, kb);
    if (own_scratch) return temp_bytes < need ? RS_ERROR_SCRATCH_LIMIT : RS_SUCCESS;
    if (!temp) return RS_ERROR_INVALID_VALUE;
    if (reinterpret_cast<uintptr_t>(temp) % kTempAlign != 0) return RS_ERROR_INVALID_VALUE;
    if (temp_bytes < need) return RS_ERROR_INSUFFICIENT_TEMP;
    const Span t = span_of(temp, need);
    if (overlap(t, ki) || overlap(t, ko)) return RS_ERROR_INVALID_VALUE;
    if (pairs && (overlap(t, span_of(vin, bytes)) || overlap(t, span_of(vout, bytes)))) {
        return RS_ERROR_INVALID_VALUE;
    }
    return RS_SUCCESS;
}

// ---------------------------------------------------------------------------
// The sort.
// ---------------------------------------------------------------------------

// Workgroups of a pass launch: as many as the device holds at once (the
// kernel loops over tiles), at most one per tile.  0 on a query failure.
unsigned pass_grid(const void *kernel, uint32_t tiles) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kPassBlock, 0) != hipSuccess) return 0;
    const uint64_t resident = static_cast<uint64_t>(cus) * static_cast<uint64_t>(per_cu > 0 ? per_cu : 1);
    return static_cast<unsigned>(resident < tiles ? resident : tiles);
}

// Keys per thread of the pass tiles for n keys: the long default, or
// kShortItems when its rounds of tiles over the compute units cost less
// (rounds x relative tile time, 0.70 for a short tile).  Both tiles hold one
// workgroup per compute unit.
int choose_items(size_t n, int vb, int kb) {
    const int items = pass_items(vb, kb);
    if (!short_tiles_allowed(vb, kb) || n >= wide_limit(kb, vb)) return items;
    if (g_tile_items == items || g_tile_items == kShortItems) return g_tile_items;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        return items;
    }
    auto rounds = [&](int k) {
        const size_t tiles = (n + size_t{kPassBlock} * k - 1) / (size_t{kPassBlock} * k);
        return (tiles + static_cast<size_t>(cus) - 1) / static_cast<size_t>(cus);
    };
    return rounds(kShortItems) * 7 < rounds(items) * 10 ? kShortItems : items;
}

// KIND is the key kind of the input.  Morton keys (M30) are computed from
// points by the histogram kernel and the first pass; the later passes sort
// the uint32 codes that pass wrote.
template <KeyKind KIND, bool PAIRS, class StatusT, class VT>
bool launch_passes(const Layout &L, const void *kin, void *kout, const void *vin,
                   void *vout, size_t n, int begin_bit, int end_bit, char *temp, hipStream_t stream,
                   const rs::MortonBox *box = nullptr) {
    constexpr int KB = key_bytes(KIND);
    constexpr int VB = PAIRS ? static_cast<int>(sizeof(VT)) : 0;
    constexpr KeyKind LATER = KIND == KeyKind::M30 ? KeyKind::U32 : KIND;
    const int P = L.passes;
    uint32_t *header = reinterpret_cast<uint32_t *>(temp + L.off_header);
    uint32_t *hist = reinterpret_cast<uint32_t *>(temp + L.off_hist);
    uint32_t *base = reinterpret_cast<uint32_t *>(temp + L.off_base);
    rs::SegmentInfo *segs = reinterpret_cast<rs::SegmentInfo *>(temp + L.off_segs);
    void *alt_k = temp + L.off_alt_keys;
    void *alt_v = temp + L.off_alt_vals;
    StatusT *status[2] = {reinterpret_cast<StatusT *>(temp + L.off_status[0]),
                          reinterpret_cast<StatusT *>(temp + L.off_status[1])};

    // 1. zero the error word, tile counters, histograms and pass-0 status;
    //    for keys of up to 32 bits and large inputs, the same launch samples
    //    the keys for position-balanced segments of skewed passes.
    uint32_t *seg_mode = nullptr;
    uint32_t *bounds = nullptr;
    constexpr bool kSampled = KB <= 4 && KIND != KeyKind::M30;
    if (kSampled && P >= 2 && n >= kSampleMinKeys) {
        seg_mode = header + kSegModeWord;
        bounds = reinterpret_cast<uint32_t *>(temp + L.off_header + kBoundsByte);
        rs::PrepareArgs pa{};
        pa.zero[0] = reinterpret_cast<uint4 *>(temp);
        // the header words before the sampling words, then everything from
        // the histograms on
        pa.zero16[0] = (sizeof(uint32_t) * kSegModeWord) / 16;
        static_assert((sizeof(uint32_t) * kSegModeWord) % 16 == 0, "sampling words start a 16-byte unit");
        pa.zero[1] = reinterpret_cast<uint4 *>(temp + L.off_hist);
        pa.zero16[1] = (L.zero_bytes - L.off_hist) / 16;
        pa.sample_groups = P - 1;
        rs::SampleArgs &sa = pa.s;
        sa.keys = kin;
        sa.n = n;
        sa.passes = P;
        for (int p = 0; p < P; ++p) {
            const int shift = begin_bit + p * kRadixBits;
            const int width = end_bit - shift < kRadixBits ? end_bit - shift : kRadixBits;
            sa.shift[p] = static_cast<uint32_t>(shift);
            sa.mask[p] = (1u << width) - 1u;
        }
        sa.seg_shift = kRadixBits - rs::kSegmentBits;
        sa.begin_bit = static_cast<uint32_t>(begin_bit);
        sa.seg_mode = seg_mode;
        sa.bounds = bounds;
        const unsigned fill_groups = grid_for(pa.zero16[1], rs::kPrepareBlock, 4096);
        if (!launch_kernel(RS_KERNEL_FILL, stream, [&] {
                if constexpr (kSampled) {
                    run_kernel(rs::prepare_kernel<KIND>, fill_groups + (P - 1), rs::kPrepareBlock, stream, pa);
                }
            })) {
            return false;
        }
    } else {
        const size_t n16 = L.zero_bytes / 16;
        const unsigned grid = grid_for(n16, 256, 4096);
        uint4 *p = reinterpret_cast<uint4 *>(temp);
        if (!launch_kernel(RS_KERNEL_FILL, stream, [&] {
                run_kernel(rs::fill_zero_kernel, grid, 256, stream, p, n16);
            })) {
            return false;
        }
    }

    // 3. all-pass histogram of the original keys.
    rs::HistArgs h{};
    h.keys = kin;
    h.hist = hist;
    h.n = n;
    h.tiles0 = L.tiles0;
    h.tile_keys = L.tile;
    h.passes = P;
    h.seg_shift = kRadixBits - rs::kSegmentBits;
    h.begin_bit = static_cast<uint32_t>(begin_bit);
    h.sub_mask = (end_bit - begin_bit >= 64) ? ~0ull : ((1ull << (end_bit - begin_bit)) - 1ull);
    h.unsorted = header + kUnsortedWord;
    h.seg_mode = seg_mode;
    h.bounds = bounds;
    if (box) h.box = *box;
    for (int p = 0; p < P; ++p) {
        const int shift = begin_bit + p * kRadixBits;
        const int width = end_bit - shift < kRadixBits ? end_bit - shift : kRadixBits;
        h.shift[p] = static_cast<uint32_t>(shift);
        h.mask[p] = (width >= 32) ? 0xFFFFFFFFu : ((1u << width) - 1u);
    }
    {
        // Workgroups per segment: enough to cover the largest segment in
        // chunks of whole units (the keys one wave counts at a time), at
        // least kHistMinUnits units each, at most kHistMaxGrid workgroups in
        // total.  (Chunks of whole 16-unit steps left up to a fifth of the
        // workgroups without keys at 2^24 keys, and made the others count
        // one step more than the average at 2^26.)
        const size_t unit = size_t{rs::kWave} * hist_items(KB);
        size_t seg_keys = 0;
        for (uint32_t s = 0; s < static_cast<uint32_t>(rs::kSegments); ++s) {
            const size_t b = size_t{rs::pass0_segment_first_tile(s, L.tiles0)} * L.tile;
            size_t e = size_t{rs::pass0_segment_first_tile(s + 1, L.tiles0)} * L.tile;
            if (e > n) e = n;
            if (e > b && e - b > seg_keys) seg_keys = e - b;
        }
        const size_t units = (seg_keys + unit - 1) / unit;
        const unsigned per_seg = grid_for(units, kHistMinUnits, kHistMaxGrid / rs::kSegments);
        h.groups_per_seg = per_seg;
        h.chunk = ((units + per_seg - 1) / per_seg) * unit;
        const unsigned grid = per_seg * rs::kSegments;
        if (!launch_kernel(RS_KERNEL_HIST, stream, [&] {
                run_kernel(rs::hist_kernel<kHistBlock, hist_items(KB), kRadixBits, hist_repl(KB), KIND>, grid,
                           kHistBlock, stream, h);
            })) {
            return false;
        }
    }

    // 4. per-pass starting offsets and segment layout.
    rs::BaseArgs ba{};
    ba.hist = hist;
    ba.base = base;
    ba.segs = segs;
    ba.n = static_cast<uint32_t>(n);
    ba.tiles0 = L.tiles0;
    ba.tile_keys = L.tile;
    ba.seg_shift = kRadixBits - rs::kSegmentBits;
    ba.trivial = header + kTrivialWord;
    ba.unsorted = header + kUnsortedWord;
    ba.keep_first = KIND == KeyKind::M30 ? 1 : 0;
    ba.seg_mode = seg_mode;
    if (!launch_kernel(RS_KERNEL_SCAN, stream, [&] {
            run_kernel(rs::digit_base_kernel<kRadix>, P, kRadix, stream, ba);
        })) {
        return false;
    }

    // 5. the digit passes.
    // Each pass kernel finds its source and destination from the flags of
    // the trivial passes (known only on the device); see pass_route.
    const bool k_in_place = (kin == kout);
    const bool v_in_place = PAIRS && (vin == vout);
    for (int p = 0; p < P; ++p) {
        rs::PassArgs<StatusT> a{};
        a.kbuf[0] = const_cast<void *>(kin);
        a.kbuf[1] = kout;
        a.kbuf[2] = alt_k;
        if (PAIRS) {
            a.vbuf[0] = const_cast<void *>(vin);
            a.vbuf[1] = vout;
            a.vbuf[2] = alt_v;
        }
        a.trivial = header + kTrivialWord;
        a.pass = p;
        a.passes = P;
        a.keys_in_place = k_in_place ? 1 : 0;
        a.vals_in_place = v_in_place ? 1 : 0;
        a.seg_base = base + p * rs::kSegments * kRadix;
        a.segs = segs + p * rs::kSegments;
        a.status = status[p % 2];
        a.status_next = (p + 1 < P) ? status[(p + 1) % 2] : nullptr;
        a.seg_counter = header + 1 + p * rs::kSegments;
        a.error_word = header;
        a.tiles_max = L.tiles_max;
        a.n = static_cast<uint32_t>(n);
        a.shift = h.shift[p];
        a.mask = h.mask[p];
        if (box) a.box = *box;
        a.spin_limit = g_force_giveup ? kGiveupSpins : rs::kSpinLimit;
        a.withhold_tile = (g_force_giveup && p == 0) ? 0u : 0xFFFFFFFFu;
        auto launch = [&](auto kernel) {
            const unsigned grid = pass_grid(reinterpret_cast<const void *>(kernel), L.tiles_max);
            return grid != 0 && launch_kernel(RS_KERNEL_PASS, stream, [&] {
                       run_kernel(kernel, grid, kPassBlock, stream, a);
                   }, p);
        };
        bool ok;
        constexpr bool kMatchOk = match_ranker_kind(KIND, VB) && std::is_same<StatusT, uint32_t>::value;
        constexpr int kMatch = rs::kRankMatch;
        if (kMatchOk && g_ranker == 1) {
            if constexpr (kMatchOk) {
                constexpr int LONG = pass_items(VB, KB);
                if constexpr (short_tiles_allowed(VB, KB)) {
                    ok = L.tile == static_cast<uint32_t>(kPassBlock * kShortItems)
                        ? launch(&rs::onesweep_kernel<kPassBlock, kShortItems, kRadixBits, KIND, PAIRS, StatusT, VT, kMatch>)
                        : launch(&rs::onesweep_kernel<kPassBlock, LONG, kRadixBits, KIND, PAIRS, StatusT, VT, kMatch>);
                } else {
                    ok = launch(&rs::onesweep_kernel<kPassBlock, LONG, kRadixBits, KIND, PAIRS, StatusT, VT, kMatch>);
                }
            }
        } else {
            // A pass of the kernel instantiated for key kind K.
            auto launch_as = [&](auto kind_c) -> bool {
                constexpr KeyKind K = decltype(kind_c)::value;
                if constexpr (short_tiles_allowed(VB, KB) && K != KeyKind::M30 && std::is_same<StatusT, uint32_t>::value) {
                    return L.tile == static_cast<uint32_t>(kPassBlock * kShortItems)
                        ? launch(&rs::onesweep_kernel<kPassBlock, kShortItems, kRadixBits, K, PAIRS, StatusT, VT>)
                        : launch(&rs::onesweep_kernel<kPassBlock, pass_items(VB, KB), kRadixBits, K, PAIRS, StatusT, VT>);
                } else {
                    return launch(&rs::onesweep_kernel<kPassBlock, pass_items(VB, KB), kRadixBits, K, PAIRS, StatusT, VT>);
                }
            };
            // The signed transform flips only the sign bit, so a pass whose
            // digit lies below it is the unsigned kind's pass (one operation
            // less per digit).
            constexpr KeyKind UNSIGNED = KIND == KeyKind::I32 ? KeyKind::U32
                                       : KIND == KeyKind::I64 ? KeyKind::U64
                                       : KIND == KeyKind::I16 ? KeyKind::U16 : KIND;
            const int width = __builtin_popcount(h.mask[p]);
            const bool below_sign = static_cast<int>(h.shift[p]) + width <= 8 * KB - 1;
            if (KIND != LATER && p == 0) {
                ok = launch_as(rs::KindC<KIND>{});
            } else if (UNSIGNED != KIND && below_sign) {
                ok = launch_as(rs::KindC<UNSIGNED>{});
            } else {
                ok = launch_as(rs::KindC<LATER>{});
            }
        }
        if (!ok) return false;
    }

    // 6. an in-place sort whose executed pass count is odd ends in temp.
    if (k_in_place || v_in_place) {
        rs::CopyArgs c{};
        c.kbuf[1] = kout;
        c.kbuf[2] = alt_k;
        if (PAIRS) {
            c.vbuf[1] = vout;
            c.vbuf[2] = alt_v;
        }
        c.trivial = header + kTrivialWord;
        c.passes = P;
        c.keys_in_place = k_in_place ? 1 : 0;
        c.vals_in_place = v_in_place ? 1 : 0;
        c.n = n;
        c.key_bytes = KB;
        c.val_bytes = VB;
        const unsigned grid = grid_for(n, rs::kCopyBlock, device_cus());
        if (!launch_kernel(RS_KERNEL_COPY, stream, [&] { run_kernel(rs::route_copy_kernel, grid, rs::kCopyBlock, stream, c); })) {
            return false;
        }
    }
    return true;
}

// The one-launch sort of a small input.  Returns false when a launch failed.
template <KeyKind KIND, bool PAIRS, class VT>
bool launch_small(const void *kin, void *kout, const void *vin, void *vout, size_t n, int begin_bit,
                  int end_bit, char *temp, hipStream_t stream) {
    constexpr int KB = key_bytes(KIND);
    constexpr int VB = PAIRS ? static_cast<int>(sizeof(VT)) : 0;
    const SmallLayout S = make_small_layout(n, VB, begin_bit, end_bit, KB);
    uint32_t *header = reinterpret_cast<uint32_t *>(temp);
    {
        const size_t n16 = S.zero_bytes / 16;
        const unsigned grid = grid_for(n16, 256, 4096);
        uint4 *p = reinterpret_cast<uint4 *>(temp);
        if (!launch_kernel(RS_KERNEL_FILL, stream, [&] { run_kernel(rs::fill_zero_kernel, grid, 256, stream, p, n16); })) {
            return false;
        }
    }
    rs::SmallArgs a{};
    a.keys_in = kin;
    a.vals_in = vin;
    a.kbuf[0] = kout;
    a.kbuf[1] = temp + S.off_alt_keys;
    if (PAIRS) {
        a.vbuf[0] = vout;
        a.vbuf[1] = temp + S.off_alt_vals;
    }
    a.hist = reinterpret_cast<uint32_t *>(temp + S.off_hist);
    a.status = reinterpret_cast<uint32_t *>(temp + S.off_status);
    a.error_word = header;
    a.claimed = header + 1;
    a.done = header + 1 + rs::kSmallPhases;
    a.n = static_cast<uint32_t>(n);
    a.tiles = S.tiles;
    a.copy_keys = (kin == kout && S.passes % 2 == 1) ? 1 : 0;
    a.copy_vals = (PAIRS && vin == vout && S.passes % 2 == 1) ? 1 : 0;
    a.passes = S.passes;
    for (int p = 0; p < S.passes; ++p) {
        const int shift = begin_bit + p * kRadixBits;
        const int width = end_bit - shift < kRadixBits ? end_bit - shift : kRadixBits;
        a.shift[p] = static_cast<uint32_t>(shift);
        a.mask[p] = (1u << width) - 1u;
    }
    return launch_kernel(RS_KERNEL_SMALL, stream, [&] {
        const unsigned grid = g_small_path == 2 ? 1u : S.tiles;
        if constexpr (match_ranker_kind(KIND, VB)) {
            if (g_ranker == 1) {
                run_kernel(rs::small_sort_kernel<kSmallBlock, kSmallItems, kRadixBits, KIND, PAIRS, VT, rs::kRankMatch>,
                           grid, kSmallBlock, stream, a);
                return;
            }
        }
        run_kernel(rs::small_sort_kernel<kSmallBlock, kSmallItems, kRadixBits, KIND, PAIRS, VT>, grid, kSmallBlock, stream, a);
    });
}

template <KeyKind KIND, bool PAIRS, class VT = uint32_t>
rs_status sort_impl(const void *kin, void *kout, const void *vin, void *vout, size_t n,
                    int begin_bit, int end_bit, void *temp, size_t temp_bytes, hipStream_t stream) {
    constexpr int KB = key_bytes(KIND);
    constexpr int VB = PAIRS ? static_cast<int>(sizeof(VT)) : 0;
    const rs_status st = validate(kin, kout, vin, vout, VB, n, begin_bit, end_bit, temp, temp_bytes, KB);
    if (st != RS_SUCCESS) return st;
    if (n == 0) return RS_SUCCESS;
    if (trivial(n, begin_bit, end_bit)) {
        bool ok = launch_copy_elems(kin, kout, n, KB, stream);
        if (PAIRS) ok = ok && launch_copy_elems(vin, vout, n, VB, stream);
        return ok ? RS_SUCCESS : RS_ERROR_LAUNCH;
    }
    char *t = static_cast<char *>(temp);
    if (g_small_path != 0 && small_input(n)) {
        return launch_small<KIND, PAIRS, VT>(kin, kout, vin, vout, n, begin_bit, end_bit, t, stream) ? RS_SUCCESS
                                                                                                    : RS_ERROR_LAUNCH;
    }
    const Layout L = make_layout(n, VB, begin_bit, end_bit, KB, choose_items(n, VB, KB));
    const bool ok = L.wide_status
        ? launch_passes<KIND, PAIRS, uint64_t, VT>(L, kin, kout, vin, vout, n, begin_bit, end_bit, t, stream)
        : launch_passes<KIND, PAIRS, uint32_t, VT>(L, kin, kout, vin, vout, n, begin_bit, end_bit, t, stream);
    return ok ? RS_SUCCESS : RS_ERROR_LAUNCH;
}

// Morton-code sort of points: validation, then the key-value passes with
// Morton keys over bits [0, 30).
constexpr int kMortonBits = 30;

size_t morton_temp_bytes(size_t n) {
    if (n == 0 || n > RS_MAX_ELEMENTS) return 0;
    return make_layout(n, 4, 0, kMortonBits, 4).total;
}

rs_status morton_box(const float *lo, const float *hi, rs::MortonBox &box) {
    if (!lo || !hi) return RS_ERROR_INVALID_VALUE;
    for (int a = 0; a < 3; ++a) {
        if (!std::isfinite(lo[a]) || !std::isfinite(hi[a]) || !(hi[a] > lo[a])) return RS_ERROR_INVALID_VALUE;
        const float width = hi[a] - lo[a];
        const float scale = 1024.0f / width;
        if (!std::isfinite(width) || !std::isfinite(scale) || !(scale > 0.0f)) return RS_ERROR_INVALID_VALUE;
        box.lo[a] = lo[a];
        box.scale[a] = scale;
    }
    return RS_SUCCESS;
}

rs_status sort_morton(const float *xyz, size_t n, const float *lo, const float *hi, uint32_t *codes,
                      uint32_t *index, void *temp, size_t temp_bytes, hipStream_t stream) {
    rs::MortonBox box;
    const rs_status bs = morton_box(lo, hi, box);
    if (bs != RS_SUCCESS) return bs;
    if (n > RS_MAX_ELEMENTS) return RS_ERROR_INVALID_VALUE;
    if (n == 0) return RS_SUCCESS;
    if (!xyz || !codes || !index) return RS_ERROR_INVALID_VALUE;
    const auto misaligned = [](const void *p) { return reinterpret_cast<uintptr_t>(p) % 4 != 0; };
    if (misaligned(xyz) || misaligned(codes) || misaligned(index)) return RS_ERROR_INVALID_VALUE;
    const Span pts = span_of(xyz, n * 12), cs = span_of(codes, n * 4), is = span_of(index, n * 4);
    if (overlap(pts, cs) || overlap(pts, is) || overlap(cs, is)) return RS_ERROR_INVALID_VALUE;
    if (!temp || reinterpret_cast<uintptr_t>(temp) % kTempAlign != 0) return RS_ERROR_INVALID_VALUE;
    const size_t need = morton_temp_bytes(n);
    if (temp_bytes < need) return RS_ERROR_INSUFFICIENT_TEMP;
    const Span t = span_of(temp, need);
    if (overlap(t, pts) || overlap(t, cs) || overlap(t, is)) return RS_ERROR_INVALID_VALUE;
    const Layout L = make_layout(n, 4, 0, kMortonBits, 4);
    char *tp = static_cast<char *>(temp);
    const bool ok = L.wide_status
        ? launch_passes<KeyKind::M30, true, uint64_t, uint32_t>(L, xyz, codes, nullptr, index, n, 0, kMortonBits, tp, stream, &box)
        : launch_passes<KeyKind::M30, true, uint32_t, uint32_t>(L, xyz, codes, nullptr, index, n, 0, kMortonBits, tp, stream, &box);
    return ok ? RS_SUCCESS : RS_ERROR_LAUNCH;
}

}  // namespace

// ---------------------------------------------------------------------------
// Fixed scratch of the allocation-free entry point (rs_sort_keys_u32_noalloc).
// Each GPU the library is loaded on holds its own copy until the process
// ends.  Host code never uses the array's name as an address: the name
// stands for a host-side shadow, and a kernel handed it would fault.  The
// device address of the current device's copy comes from
// hipGetSymbolAddress, looked up once per device and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[RS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch, or nullptr if it cannot
// be found.  Looked up with that device current, once per device.
void *scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        if (reinterpret_cast<uintptr_t>(p) % kTempAlign != 0) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI (include/rs.h, include/rs_prof.h)
// ---------------------------------------------------------------------------
extern "C" {

size_t rs_temp_bytes(size_t n, int with_values, int begin_bit, int end_bit) {
    if (!valid_bits(begin_bit, end_bit, 4) || n > RS_MAX_ELEMENTS) return 0;
    if (trivial(n, begin_bit, end_bit)) return 0;
    return temp_need(n, with_values != 0 ? 4 : 0, begin_bit, end_bit, 4);
}

size_t rs_temp_bytes_morton30(size_t n) { return morton_temp_bytes(n); }

rs_status rs_sort_morton30(const float *xyz, size_t n, const float *box_lo, const float *box_hi,
                           uint32_t *codes_out, uint32_t *index_out, void *temp, size_t temp_bytes,
                           hipStream_t stream) {
    return sort_morton(xyz, n, box_lo, box_hi, codes_out, index_out, temp, temp_bytes, stream);
}

size_t rs_temp_bytes64(size_t n, int with_values, int begin_bit, int end_bit) {
    if (!valid_bits(begin_bit, end_bit, 8) || n > RS_MAX_ELEMENTS) return 0;
    if (trivial(n, begin_bit, end_bit)) return 0;
    return temp_need(n, with_values != 0 ? 4 : 0, begin_bit, end_bit, 8);
}

rs_status rs_sort_keys_u32(const uint32_t *keys_in, uint32_t *keys_out, size_t n, int begin_bit,
                           int end_bit, void *temp, size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::U32, false>(keys_in, keys_out, nullptr, nullptr, n, begin_bit, end_bit,
                                          temp, temp_bytes, stream);
}

rs_status rs_sort_keys_u32_noalloc(const uint32_t *keys_in, uint32_t *keys_out, size_t n, int begin_bit,
                                   int end_bit, hipStream_t stream) {
    if (n > RS_NOALLOC_MAX_KEYS) return RS_ERROR_SCRATCH_LIMIT;
    // Every argument check runs on the host before the scratch address is
    // looked up (the first HIP call); trivial calls need no scratch.
    const rs_status st = validate(keys_in, keys_out, nullptr, nullptr, 0, n, begin_bit, end_bit, nullptr,
                                  RS_NOALLOC_SCRATCH_BYTES, 4, true);
    if (st != RS_SUCCESS) return st;
    if (n == 0 || trivial(n, begin_bit, end_bit)) {
        return sort_impl<KeyKind::U32, false>(keys_in, keys_out, nullptr, nullptr, n, begin_bit, end_bit, nullptr,
                                              0, stream);
    }
    void *s = scratch_address();
    if (s == nullptr) return RS_ERROR_LAUNCH;
    return sort_impl<KeyKind::U32, false>(keys_in, keys_out, nullptr, nullptr, n, begin_bit, end_bit, s,
                                          RS_NOALLOC_SCRATCH_BYTES, stream);
}

rs_status rs_sort_keys_i32(const int32_t *keys_in, int32_t *keys_out, size_t n, int begin_bit,
                           int end_bit, void *temp, size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::I32, false>(reinterpret_cast<const uint32_t *>(keys_in),
                                          reinterpret_cast<uint32_t *>(keys_out), nullptr, nullptr, n,
                                          begin_bit, end_bit, temp, temp_bytes, stream);
}

rs_status rs_sort_keys_f32(const float *keys_in, float *keys_out, size_t n, int begin_bit, int end_bit,
                           void *temp, size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::F32, false>(reinterpret_cast<const uint32_t *>(keys_in),
                                          reinterpret_cast<uint32_t *>(keys_out), nullptr, nullptr, n,
                                          begin_bit, end_bit, temp, temp_bytes, stream);
}

rs_status rs_sort_pairs_u32(const uint32_t *keys_in, uint32_t *keys_out, const uint32_t *vals_in,
                            uint32_t *vals_out, size_t n, int begin_bit, int end_bit, void *temp,
                            size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::U32, true>(keys_in, keys_out, vals_in, vals_out, n, begin_bit, end_bit,
                                         temp, temp_bytes, stream);
}

rs_status rs_sort_pairs_i32(const int32_t *keys_in, int32_t *keys_out, const uint32_t *vals_in,
                            uint32_t *vals_out, size_t n, int begin_bit, int end_bit, void *temp,
                            size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::I32, true>(reinterpret_cast<const uint32_t *>(keys_in),
                                         reinterpret_cast<uint32_t *>(keys_out), vals_in, vals_out, n,
                                         begin_bit, end_bit, temp, temp_bytes, stream);
}

rs_status rs_sort_pairs_f32(const float *keys_in, float *keys_out, const uint32_t *vals_in,
                            uint32_t *vals_out, size_t n, int begin_bit, int end_bit, void *temp,
                            size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::F32, true>(reinterpret_cast<const uint32_t *>(keys_in),
                                         reinterpret_cast<uint32_t *>(keys_out), vals_in, vals_out, n,
                                         begin_bit, end_bit, temp, temp_bytes, stream);
}

rs_status rs_sort_keys_u64(const uint64_t *keys_in, uint64_t *keys_out, size_t n, int begin_bit,
                           int end_bit, void *temp, size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::U64, false>(keys_in, keys_out, nullptr, nullptr, n, begin_bit, end_bit, temp,
                                          temp_bytes, stream);
}

rs_status rs_sort_keys_i64(const int64_t *keys_in, int64_t *keys_out, size_t n, int begin_bit,
                           int end_bit, void *temp, size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::I64, false>(keys_in, keys_out, nullptr, nullptr, n, begin_bit, end_bit, temp,
                                          temp_bytes, stream);
}

rs_status rs_sort_keys_f64(const double *keys_in, double *keys_out, size_t n, int begin_bit, int end_bit,
                           void *temp, size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::F64, false>(keys_in, keys_out, nullptr, nullptr, n, begin_bit, end_bit, temp,
                                          temp_bytes, stream);
}

rs_status rs_sort_pairs_u64(const uint64_t *keys_in, uint64_t *keys_out, const uint32_t *vals_in,
                            uint32_t *vals_out, size_t n, int begin_bit, int end_bit, void *temp,
                            size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::U64, true>(keys_in, keys_out, vals_in, vals_out, n, begin_bit, end_bit, temp,
                                         temp_bytes, stream);
}

rs_status rs_sort_pairs_i64(const int64_t *keys_in, int64_t *keys_out, const uint32_t *vals_in,
                            uint32_t *vals_out, size_t n, int begin_bit, int end_bit, void *temp,
                            size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::I64, true>(keys_in, keys_out, vals_in, vals_out, n, begin_bit, end_bit, temp,
                                         temp_bytes, stream);
}

rs_status rs_sort_pairs_f64(const double *keys_in, double *keys_out, const uint32_t *vals_in,
                            uint32_t *vals_out, size_t n, int begin_bit, int end_bit, void *temp,
                            size_t temp_bytes, hipStream_t stream) {
    return sort_impl<KeyKind::F64, true>(keys_in, keys_out, vals_in, vals_out, n, begin_bit, end_bit, temp,
                                         temp_bytes, stream);
}

// 16-bit keys (F16: IEEE binary16 bit patterns), and key-value sorts with
// 64-bit values for every key type.
#define RS_KEYS_ENTRY(NAME, KTYPE, KIND)                                                                       \
    rs_status rs_sort_keys_##NAME(const KTYPE *keys_in, KTYPE *keys_out, size_t n, int begin_bit, int end_bit, \
                                  void *temp, size_t temp_bytes, hipStream_t stream) {                         \
        return sort_impl<KIND, false>(keys_in, keys_out, nullptr, nullptr, n, begin_bit, end_bit, temp,        \
                                      temp_bytes, stream);                                                     \
    }
#define RS_PAIRS_ENTRY(NAME, KTYPE, VTYPE, KIND)                                                                 \
    rs_status rs_sort_pairs_##NAME(const KTYPE *keys_in, KTYPE *keys_out, const VTYPE *vals_in, VTYPE *vals_out, \
                                   size_t n, int begin_bit, int end_bit, void *temp, size_t temp_bytes,          \
                                   hipStream_t stream) {                                                         \
        return sort_impl<KIND, true, VTYPE>(keys_in, keys_out, vals_in, vals_out, n, begin_bit, end_bit, temp,    \
                                            temp_bytes, stream);                                                 \
    }

RS_KEYS_ENTRY(u16, uint16_t, KeyKind::U16)
RS_KEYS_ENTRY(i16, int16_t, KeyKind::I16)
RS_KEYS_ENTRY(f16, uint16_t, KeyKind::F16)
RS_PAIRS_ENTRY(u16, uint16_t, uint32_t, KeyKind::U16)
RS_PAIRS_ENTRY(i16, int16_t, uint32_t, KeyKind::I16)
RS_PAIRS_ENTRY(f16, uint16_t, uint32_t, KeyKind::F16)
RS_PAIRS_ENTRY(u16_v64, uint16_t, uint64_t, KeyKind::U16)
RS_PAIRS_ENTRY(i16_v64, int16_t, uint64_t, KeyKind::I16)
RS_PAIRS_ENTRY(f16_v64, uint16_t, uint64_t, KeyKind::F16)
RS_PAIRS_ENTRY(u32_v64, uint32_t, uint64_t, KeyKind::U32)
RS_PAIRS_ENTRY(i32_v64, int32_t, uint64_t, KeyKind::I32)
RS_PAIRS_ENTRY(f32_v64, float, uint64_t, KeyKind::F32)
RS_PAIRS_ENTRY(u64_v64, uint64_t, uint64_t, KeyKind::U64)
RS_PAIRS_ENTRY(i64_v64, int64_t, uint64_t, KeyKind::I64)
RS_PAIRS_ENTRY(f64_v64, double, uint64_t, KeyKind::F64)

#undef RS_KEYS_ENTRY
#undef RS_PAIRS_ENTRY

size_t rs_temp_bytes_ex(size_t n, int key_bytes, int value_bytes, int begin_bit, int end_bit) {
    if (key_bytes != 2 && key_bytes != 4 && key_bytes != 8) return 0;
    if (value_bytes != 0 && value_bytes != 4 && value_bytes != 8) return 0;
    if (!valid_bits(begin_bit, end_bit, key_bytes) || n > RS_MAX_ELEMENTS) return 0;
    if (trivial(n, begin_bit, end_bit)) return 0;
    return temp_need(n, value_bytes, begin_bit, end_bit, key_bytes);
}

const char *rs_status_string(rs_status status) {
    switch (status) {
        case RS_SUCCESS: return "success";
        case RS_ERROR_INVALID_VALUE: return "invalid argument";
        case RS_ERROR_INSUFFICIENT_TEMP: return "temp buffer smaller than rs_temp_bytes()";
        case RS_ERROR_LAUNCH: return "kernel launch failed";
        case RS_ERROR_SCRATCH_LIMIT: return "input larger than the fixed scratch of the allocation-free sort";
        default: return "unknown rs_status";
    }
}

int rs_prof_enable(int on) {
    Prof &p = prof();
    std::lock_guard<std::mutex> lock(p.mu);
    const int prev = p.on ? 1 : 0;
    p.on = on != 0;
    return prev;
}

void rs_prof_reset(void) {
    Prof &p = prof();
    std::lock_guard<std::mutex> lock(p.mu);
    for (auto &r : p.pending) {
        (void)hipEventSynchronize(r.stop);  // drop: a failed wait only loses a timing
        p.spare.push_back(r.start);
        p.spare.push_back(r.stop);
    }
    p.pending.clear();
    for (int k = 0; k < RS_KERNEL_KINDS; ++k) {
        p.launches[k] = 0;
        p.ms[k] = 0.0;
        p.samples[k].clear();
    }
}

size_t rs_prof_samples(int kind, int sub, double *ms, size_t cap) {
    if (kind < 0 || kind >= RS_KERNEL_KINDS) return 0;
    Prof &p = prof();
    uint64_t launches = 0;
    double total = 0.0;
    (void)rs_prof_summary(kind, &launches, &total);  // folds the pending events into the samples
    std::lock_guard<std::mutex> lock(p.mu);
    size_t count = 0;
    for (const ProfSample &x : p.samples[kind]) {
        if (sub >= 0 && x.sub != sub) continue;
        if (ms != nullptr && count < cap) ms[count] = x.ms;
        ++count;
    }
    return count;
}

int rs_prof_ranker(int mode) {
    const int prev = g_ranker;
    g_ranker = mode == 1 ? 1 : 0;
    return prev;
}

int rs_prof_force_giveup(int on) {
    const int prev = g_force_giveup ? 1 : 0;
    g_force_giveup = on != 0;
    return prev;
}

rs_status rs_prof_lds_rank_probe(const uint32_t *digits, uint32_t *ranks, int blocks, int slots, int unit,
                                 hipStream_t stream) {
    constexpr int kProbeBlock = 1024;
    if (!digits || !ranks || blocks < 1 || blocks > 65535 || (unit != 1 && unit != 4)) return RS_ERROR_INVALID_VALUE;
    if (slots != 8 && slots != 16 && slots != 28) return RS_ERROR_INVALID_VALUE;
    const size_t words = static_cast<size_t>(blocks) * kProbeBlock * static_cast<size_t>(slots);
    if (overlap(span_of(digits, words * 4), span_of(ranks, words * 4))) return RS_ERROR_INVALID_VALUE;
    const uint32_t u = static_cast<uint32_t>(unit);
    auto go = [&](auto kernel) {
        run_kernel(kernel, blocks, kProbeBlock, stream, digits, ranks, u);
        return hipGetLastError() == hipSuccess ? RS_SUCCESS : RS_ERROR_LAUNCH;
    };
    switch (slots) {
        case 8: return go(rs::lds_rank_probe_kernel<kProbeBlock, 8>);
        case 16: return go(rs::lds_rank_probe_kernel<kProbeBlock, 16>);
        case 28: return go(rs::lds_rank_probe_kernel<kProbeBlock, 28>);
        default: return RS_ERROR_INVALID_VALUE;
    }
}

int rs_prof_tile_items(int items) {
    const int prev = g_tile_items;
    g_tile_items = (items == kShortItems || items == pass_items(0, 4)) ? items : 0;
    return prev;
}

size_t rs_prof_header_offset(int which) {
    switch (which) {
        case 0: return 0;
        case 1: return sizeof(uint32_t) * kTrivialWord;
        case 2: return sizeof(uint32_t) * kUnsortedWord;
        case 3: return kHeaderBytes;
        case 4: return sizeof(uint32_t) * kSegModeWord;
        case 5: return kBoundsByte;
        default: return static_cast<size_t>(-1);
    }
}

int rs_prof_small_path(int mode) {
    const int prev = g_small_path;
    g_small_path = (mode == 0 || mode == 2) ? mode : 1;
    return prev;
}

rs_status rs_prof_summary(int kind, uint64_t *launches, double *total_ms) {
    if (kind < 0 || kind >= RS_KERNEL_KINDS || !launches || !total_ms) return RS_ERROR_INVALID_VALUE;
    Prof &p = prof();
    std::lock_guard<std::mutex> lock(p.mu);
    bool ok = true;
    for (auto &r : p.pending) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
            ok = false;
        } else {
            p.launches[r.kind] += 1;
            p.ms[r.kind] += ms;
            p.samples[r.kind].push_back({r.sub, static_cast<double>(ms)});
        }
        p.spare.push_back(r.start);
        p.spare.push_back(r.stop);
    }
    p.pending.clear();
    *launches = p.launches[kind];
    *total_ms = p.ms[kind];
    return ok ? RS_SUCCESS : RS_ERROR_LAUNCH;
}

rs_status rs_copy_u32(const uint32_t *in, uint32_t *out, size_t n, hipStream_t stream) {
    if (n == 0) return RS_SUCCESS;
    if (!in || !out || n > RS_MAX_ELEMENTS) return RS_ERROR_INVALID_VALUE;
    if (overlap(span_of(in, n * 4), span_of(out, n * 4))) return RS_ERROR_INVALID_VALUE;
    return launch_copy(in, out, n, stream) ? RS_SUCCESS : RS_ERROR_LAUNCH;
}

}  // extern "C"
