// kernels.hpp -- gfx950 kernels of the stable LSD radix sort.
//
// One sort = fill (zero the scan state) -> all-pass digit histogram (one read
// of the keys) -> exclusive scan of each pass's histogram -> one fused
// rank-and-scatter kernel per digit pass.  Page abbreviations as in
// device.hpp.
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

// Copy n4 16-byte words (both pointers 16-byte aligned).
__global__ void copy_u128_kernel(const uint4 *__restrict__ in, uint4 *__restrict__ out, size_t n4) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride) {
        out[i] = in[i];
    }
}

// ---------------------------------------------------------------------------
// All-pass digit histogram.
//
// [WA] "Las tres fases de una pasada" counts each block's digits into a
// workgroup-shared atomic histogram.  A digit histogram does not depend on
// the order of the keys, so the histograms of every pass are taken here from
// the ORIGINAL keys in a single read, into LDS-privatised counters that are
// folded into the global [pass][digit] array at the end.
// ---------------------------------------------------------------------------
constexpr int kMaxPasses = 8;

struct HistArgs {
    const uint32_t *keys;
    uint32_t *hist;          // [passes][radix], zeroed beforehand
    size_t n;
    size_t chunk;            // keys per workgroup, multiple of BLOCK*ITEMS
    int passes;
    uint32_t shift[kMaxPasses];
    uint32_t mask[kMaxPasses];
};

template <int BLOCK, int ITEMS, int RBITS, KeyKind KIND>
__global__ __launch_bounds__(BLOCK) void hist_kernel(HistArgs a) {
    constexpr int RADIX = 1 << RBITS;
    constexpr int MAXP = (32 + RBITS - 1) / RBITS;
    static_assert(MAXP <= kMaxPasses, "too many passes");
    __shared__ uint32_t s_hist[MAXP * RADIX];

    const int tid = threadIdx.x;
    for (int i = tid; i < MAXP * RADIX; i += BLOCK) s_hist[i] = 0u;
    __syncthreads();

    const size_t begin = static_cast<size_t>(blockIdx.x) * a.chunk;
    const size_t end = begin + a.chunk < a.n ? begin + a.chunk : a.n;
    for (size_t base = begin; base < end; base += static_cast<size_t>(BLOCK) * ITEMS) {
        uint32_t k[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const size_t idx = base + static_cast<size_t>(j) * BLOCK + tid;
            k[j] = idx < end ? ordered_key<KIND>(a.keys[idx]) : 0u;
        }
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const size_t idx = base + static_cast<size_t>(j) * BLOCK + tid;
            if (idx < end) {
#pragma unroll
                for (int p = 0; p < MAXP; ++p) {
                    if (p < a.passes) atomicAdd(&s_hist[p * RADIX + ((k[j] >> a.shift[p]) & a.mask[p])], 1u);
                }
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < a.passes * RADIX; i += BLOCK) {
        const uint32_t c = s_hist[i];
        if (c != 0u) atomicAdd(&a.hist[i], c);
    }
}

// ---------------------------------------------------------------------------
// Exclusive scan of each pass's digit histogram: base[p][d] = number of keys
// whose pass-p digit is below d, i.e. where digit d's run starts in the
// output of pass p.  One workgroup per pass.
// ---------------------------------------------------------------------------
template <int RADIX>
__global__ __launch_bounds__(RADIX) void digit_base_kernel(const uint32_t *__restrict__ hist,
                                                           uint32_t *__restrict__ base) {
    static_assert(RADIX % kWave == 0, "radix must fill whole waves");
    __shared__ uint32_t s_wave_total[RADIX / kWave];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const uint32_t v = hist[blockIdx.x * RADIX + tid];
    const uint32_t incl = wave_inclusive_sum(v);
    if ((tid & (kWave - 1)) == kWave - 1) s_wave_total[wave] = incl;
    __syncthreads();
    uint32_t before = 0u;
    for (int w = 0; w < wave; ++w) before += s_wave_total[w];
    base[blockIdx.x * RADIX + tid] = before + incl - v;
}

// ---------------------------------------------------------------------------
// One digit pass: load a tile, rank, chained digit scan, LDS shuffle, stable
// scatter -- fused in one kernel.
//
// Global position of an element ([OH] "GPU上的基数排序": position = scanned
// block sum of its digit + its local rank; [WA] "Las tres fases": the
// digit-major exclusive scan of counts gives, at (d, b), where block b starts
// writing digit d):
//     dst = base[d] + (digit-d count of all earlier tiles) + rank in tile.
// The middle term is the digit-major scan across tiles.  Here it is computed
// by a chained scan with decoupled look-back: each tile publishes its digit
// counts as soon as it has ranked, then sums the published counts of earlier
// tiles back to the first one that already holds an inclusive prefix.  Tiles
// take their index from an atomic counter in launch order, so every tile a
// tile waits for has already started: the chain always drains.
//
// Local rank (what the 1-bit splits of [WA] "El ranking local..." and the
// one-hot Blelloch scans of [OH] Pass1 compute): rank(i) = number of earlier
// elements of the tile with the same digit.  Each wave holds its keys
// wave-striped (slot j of lane l is tile element wave_base + 64*j + l) and
// ranks slot by slot:
//   * the lanes of a slot sharing a digit are found through LDS: every lane
//     ORs its lane bit into a per-wave 64-bit word of its digit, reads the
//     word back and clears it.  The word is the same whatever order the ORs
//     land in, so the result is deterministic;
//   * rank = (count of the digit in earlier slots, a per-wave LDS counter
//     read before this slot's increments) + (matching lanes below this one).
// Slots are ranked in slot order and lanes in lane order, which is element
// order: the ranking is stable.
//
// Scatter ([PM] §13.4: stage the tile in shared memory, then write contiguous
// runs): keys are written to LDS at their tile-sorted position, then read
// back in order, so consecutive lanes write consecutive addresses of the
// same digit run.
//
// The final partial tile pads its missing elements with the largest digit
// slot (RADIX-1).  Pads come after every real element in element order and
// the largest digit's run is last in the tile, so they rank after every real
// element, occupy tile positions >= the real count and are never written.
// ---------------------------------------------------------------------------
template <class StatusT>
struct PassArgs {
    const uint32_t *keys_in;
    uint32_t *keys_out;
    const uint32_t *vals_in;
    uint32_t *vals_out;
    const uint32_t *digit_base;  // [RADIX] this pass's exclusive digit scan
    StatusT *status;             // [tiles][RADIX] this pass, zero on entry
    StatusT *status_next;        // [tiles][RADIX] next pass's words to zero, or null
    uint32_t *tile_counter;      // zero on entry
    uint32_t *error_word;
    uint32_t n;
    uint32_t shift;
    uint32_t mask;
};

// Bound on look-back polls of one status word (each poll is a device-scope
// load of ~1 us plus a short sleep): a few seconds, far beyond any real wait.
constexpr uint32_t kSpinLimit = 1u << 22;
// Predecessor status words fetched per look-back step.
constexpr int kLookbackWindow = 4;

// Raw buffer resource (gfx9 family word 3: 32-bit data, no swizzle) over
// `bytes` bytes: buffer accesses at offsets >= bytes are dropped by hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}

// A window of look-back status words: w[i] belongs to tile k - i.  Tiles
// before tile 0 read as an inclusive prefix of 0.
template <class StatusT, int RADIX>
struct LookbackWindow {
    StatusT w[kLookbackWindow];

    __device__ __forceinline__ void fetch(StatusT *status, uint32_t k, uint32_t digit) {
#pragma unroll
        for (int i = 0; i < kLookbackWindow; ++i) {
            w[i] = (k >= static_cast<uint32_t>(i))
                       ? status_load(status + static_cast<size_t>(k - i) * RADIX + digit)
                       : make_status<StatusT>(kFlagInclusive, 0u);
        }
    }
};

template <int BLOCK, int ITEMS, int RBITS, KeyKind KIND, bool PAIRS, class StatusT>
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
    static_assert(WAVES * RADIX * 2 <= TILE, "match words must fit in the tile buffer");
    using SW = StatusWord<StatusT>;

    // The tile buffer doubles as the per-wave match words during ranking.
    __shared__ uint64_t s_buf[TILE / 2];
    __shared__ uint32_t s_cnt[WAVES * RADIX];     // per-wave digit counts (bytes) -> offsets
    __shared__ uint32_t s_goff[RADIX];            // global start - local start, per digit
    __shared__ uint32_t s_wave_total[RADIX / kWave];
    __shared__ uint32_t s_tile_id;
    uint32_t *const s_tile = reinterpret_cast<uint32_t *>(s_buf);
    char *const s_tile_bytes = reinterpret_cast<char *>(s_buf);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    if (tid == 0) s_tile_id = atomicAdd(a.tile_counter, 1u);
    uint64_t *const wave_match = s_buf + wave * RADIX;
    uint32_t *const wave_cnt = s_cnt + wave * RADIX;
#pragma unroll
    for (int i = lane; i < RADIX; i += kWave) {
        wave_match[i] = 0ull;
        wave_cnt[i] = 0u;
    }
    __syncthreads();

    const uint32_t tile = s_tile_id;
    const size_t tile_start = static_cast<size_t>(tile) * TILE;
    const size_t left = static_cast<size_t>(a.n) - tile_start;
    const bool full = left >= static_cast<size_t>(TILE);
    const uint32_t valid = full ? static_cast<uint32_t>(TILE) : static_cast<uint32_t>(left);

    // The next pass uses the other status region; its words for this tile
    // are cleared here (the pass that last used them has completed).
    if (a.status_next != nullptr && tid < RADIX) {
        a.status_next[static_cast<size_t>(tile) * RADIX + tid] = StatusT(0);
    }

    // ---- load (wave-striped) --------------------------------------------
    const uint32_t wave_base = static_cast<uint32_t>(wave) * WAVE_KEYS;
    const uint32_t *kin = a.keys_in + tile_start + wave_base + lane;
    uint32_t key[ITEMS];
    uint32_t dig[ITEMS];
    uint32_t val[PAIRS ? ITEMS : 1];
    if (full) {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) key[j] = kin[j * kWave];
        if constexpr (PAIRS) {
            const uint32_t *vin = a.vals_in + tile_start + wave_base + lane;
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) val[j] = vin[j * kWave];
        }
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) dig[j] = digit_of<KIND>(key[j], a.shift, a.mask);
    } else {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const bool ok = wave_base + j * kWave + lane < valid;
            key[j] = ok ? kin[j * kWave] : 0u;
            if constexpr (PAIRS) val[j] = ok ? a.vals_in[tile_start + wave_base + j * kWave + lane] : 0u;
            dig[j] = ok ? digit_of<KIND>(key[j], a.shift, a.mask) : static_cast<uint32_t>(RADIX - 1);
        }
    }

    // ---- rank within the wave (byte offsets: 4 * rank) --------------------
    const uint64_t lane_bit = 1ull << lane;
    uint32_t rank4[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        uint64_t *const word = wave_match + dig[j];
        uint32_t *const counter = wave_cnt + dig[j];
        __hip_atomic_fetch_or(word, lane_bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        const uint64_t same = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        const uint32_t before = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        __hip_atomic_fetch_add(counter, 4u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        rank4[j] = before + 4u * lanes_below(same);
    }
    __syncthreads();

    // ---- tile digit counts, publish, local starts ---------------------
    StatusT *const my_status = a.status + static_cast<size_t>(tile) * RADIX + tid;
    uint32_t tile_count = 0u;
    uint32_t incl = 0u;
    if (tid < RADIX) {
        uint32_t run = 0u;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const uint32_t c = s_cnt[w * RADIX + tid];
            s_cnt[w * RADIX + tid] = run;  // exclusive over waves, bytes
            run += c;
        }
        tile_count = run >> 2;
        status_store(my_status, make_status<StatusT>(tile == 0u ? kFlagInclusive : kFlagAggregate,
                                                     tile_count));
        incl = wave_inclusive_sum(tile_count);
        if (lane == kWave - 1) s_wave_total[wave] = incl;
    }
    __syncthreads();

    LookbackWindow<StatusT, RADIX> lb;
    uint32_t local_start = 0u;
    if (tid < RADIX) {
        local_start = incl - tile_count;
        for (int w = 0; w < wave; ++w) local_start += s_wave_total[w];
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s_cnt[w * RADIX + tid] += 4u * local_start;
        // First look-back window in flight while the tile is shuffled.
        if (tile > 0u) lb.fetch(a.status, tile - 1u, tid);
    }
    __syncthreads();

    // ---- shuffle keys into tile-sorted order in LDS ---------------------
    uint32_t pos4[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        pos4[j] = wave_cnt[dig[j]] + rank4[j];
        *reinterpret_cast<uint32_t *>(s_tile_bytes + pos4[j]) = key[j];
    }

    // ---- decoupled look-back over earlier tiles -----------------------
    if (tid < RADIX) {
        uint32_t before = 0u;
        if (tile > 0u) {
            bool failed = false;
            uint32_t spins = 0u;
            uint32_t k = tile - 1u;  // tile of lb.w[0]
            for (;;) {
                int consumed = 0;
                bool done = false, empty = false;
#pragma unroll
                for (int i = 0; i < kLookbackWindow; ++i) {
                    if (!done && !empty && !failed) {
                        const uint32_t flag = static_cast<uint32_t>(lb.w[i] >> SW::kShift);
                        if (flag == kFlagEmpty) {
                            empty = true;
                        } else if (flag == kFlagError) {
                            failed = true;
                        } else {
                            before += static_cast<uint32_t>(lb.w[i] & SW::kValueMask);
                            consumed = i + 1;
                            done = (flag == kFlagInclusive);
                        }
                    }
                }
                if (done || failed) break;
                if (empty) {
                    if (++spins > kSpinLimit) { failed = true; break; }
                    __builtin_amdgcn_s_sleep(1);
                } else if (k < static_cast<uint32_t>(consumed)) {
                    failed = true;  // tile 0 is always inclusive
                    break;
                }
                k -= static_cast<uint32_t>(consumed);
                lb.fetch(a.status, k, tid);
            }
            if (failed) {
                atomicOr(a.error_word, 1u);
                status_store(my_status, make_status<StatusT>(kFlagError, 0u));
            } else {
                status_store(my_status, make_status<StatusT>(kFlagInclusive, before + tile_count));
            }
        }
        s_goff[tid] = a.digit_base[tid] + before - local_start;
    }
    __syncthreads();

    // ---- scatter digit runs ------------------------------------------------
    uint32_t dst[PAIRS ? ITEMS : 1];
    if constexpr (!WIDE) {
        const __amdgpu_buffer_rsrc_t kout = buffer_rsrc(a.keys_out, a.n * 4u);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t i = static_cast<uint32_t>(j) * BLOCK + tid;
            const uint32_t k = s_tile[i];
            const uint32_t o = s_goff[digit_of<KIND>(k, a.shift, a.mask)] + i;
            if (full || i < valid) __builtin_amdgcn_raw_buffer_store_b32(k, kout, static_cast<int>(o * 4u), 0, 0);
            if constexpr (PAIRS) dst[j] = (full || i < valid) ? o : 0xFFFFFFFFu;
        }
    } else {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t i = static_cast<uint32_t>(j) * BLOCK + tid;
            uint32_t o = 0xFFFFFFFFu;
            if (i < valid) {
                const uint32_t k = s_tile[i];
                o = s_goff[digit_of<KIND>(k, a.shift, a.mask)] + i;
                if (o < a.n) a.keys_out[o] = k;
            }
            if constexpr (PAIRS) dst[j] = o;
        }
    }

    if constexpr (PAIRS) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) *reinterpret_cast<uint32_t *>(s_tile_bytes + pos4[j]) = val[j];
        __syncthreads();
        if constexpr (!WIDE) {
            const __amdgpu_buffer_rsrc_t vout = buffer_rsrc(a.vals_out, a.n * 4u);
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const uint32_t i = static_cast<uint32_t>(j) * BLOCK + tid;
                if (full || i < valid) {
                    __builtin_amdgcn_raw_buffer_store_b32(s_tile[i], vout, static_cast<int>(dst[j] * 4u), 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) {
                const uint32_t i = static_cast<uint32_t>(j) * BLOCK + tid;
                if (i < valid && dst[j] < a.n) a.vals_out[dst[j]] = s_tile[i];
            }
        }
    }
}

}  // namespace rs
