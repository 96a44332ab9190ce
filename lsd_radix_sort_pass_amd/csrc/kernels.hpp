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
// Local rank (replaces the 1-bit splits of [WA] "El ranking local..." and the
// one-hot Blelloch scans of [OH] Pass1): each wave ranks its keys with
// 64-lane ballots -- the lanes holding the same digit are found by RBITS
// ballots, a lane's rank among them is the popcount of those below it, and
// a per-wave LDS counter per digit carries the count across the wave's
// key slots.  Keys are held "wave-striped" (slot j of lane l is tile element
// wave_base + 64*j + l), so ranking slot by slot, lane by lane follows the
// element order exactly: the ranking is stable.
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

template <int BLOCK, int ITEMS, int RBITS, KeyKind KIND, bool PAIRS, class StatusT>
__global__ __launch_bounds__(BLOCK) void onesweep_kernel(PassArgs<StatusT> a) {
    constexpr int RADIX = 1 << RBITS;
    constexpr int WAVES = BLOCK / kWave;
    constexpr int TILE = BLOCK * ITEMS;
    constexpr int WAVE_KEYS = kWave * ITEMS;
    static_assert(BLOCK % kWave == 0, "block must be whole waves");
    static_assert(BLOCK >= RADIX && RADIX % kWave == 0, "one thread per digit");
    using SW = StatusWord<StatusT>;

    __shared__ uint32_t s_tile[TILE];             // tile in sorted order (keys, then values)
    __shared__ uint32_t s_cnt[WAVES * RADIX];     // per-wave digit counters -> tile offsets
    __shared__ uint32_t s_goff[RADIX];            // global start - local start, per digit
    __shared__ uint32_t s_wave_total[RADIX / kWave];
    __shared__ uint32_t s_tile_id;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    if (tid == 0) s_tile_id = atomicAdd(a.tile_counter, 1u);
    for (int i = lane; i < RADIX; i += kWave) s_cnt[wave * RADIX + i] = 0u;
    __syncthreads();

    const uint32_t tile = s_tile_id;
    const size_t tile_start = static_cast<size_t>(tile) * TILE;
    const size_t left = static_cast<size_t>(a.n) - tile_start;
    const uint32_t valid = left < static_cast<size_t>(TILE) ? static_cast<uint32_t>(left) : TILE;

    // The next pass uses the other status region; its words for this tile
    // are cleared here (the pass that last used them has completed).
    if (a.status_next != nullptr && tid < RADIX) {
        a.status_next[static_cast<size_t>(tile) * RADIX + tid] = StatusT(0);
    }

    // ---- load (wave-striped) --------------------------------------------
    const uint32_t wave_base = static_cast<uint32_t>(wave) * WAVE_KEYS;
    const uint32_t *kin = a.keys_in + tile_start;
    uint32_t key[ITEMS];
    uint32_t dig[ITEMS];
    uint32_t val[PAIRS ? ITEMS : 1];
    if (valid == TILE) {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) key[j] = kin[wave_base + j * kWave + lane];
        if constexpr (PAIRS) {
            const uint32_t *vin = a.vals_in + tile_start;
#pragma unroll
            for (int j = 0; j < ITEMS; ++j) val[j] = vin[wave_base + j * kWave + lane];
        }
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) dig[j] = digit_of<KIND>(key[j], a.shift, a.mask);
    } else {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t idx = wave_base + j * kWave + lane;
            const bool ok = idx < valid;
            key[j] = ok ? kin[idx] : 0u;
            if constexpr (PAIRS) val[j] = ok ? a.vals_in[tile_start + idx] : 0u;
            dig[j] = ok ? digit_of<KIND>(key[j], a.shift, a.mask) : static_cast<uint32_t>(RADIX - 1);
        }
    }

    // ---- rank within the wave --------------------------------------------
    uint32_t *wave_cnt = s_cnt + wave * RADIX;
    uint32_t rank[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const uint64_t same = match_digit<RBITS>(dig[j]);
        const uint32_t below = lanes_below(same);
        const uint32_t count = static_cast<uint32_t>(__popcll(same));
        const uint32_t before = wave_cnt[dig[j]];
        __builtin_amdgcn_wave_barrier();
        // Lowest lane of each digit group advances the counter; LDS requests
        // of one wave complete in order, so every lane read the old value.
        if (below == 0u) wave_cnt[dig[j]] = before + count;
        __builtin_amdgcn_wave_barrier();
        rank[j] = before + below;
    }
    __syncthreads();

    // ---- tile digit counts, publish, local starts ---------------------
    StatusT *my_status = a.status + static_cast<size_t>(tile) * RADIX + tid;
    uint32_t tile_count = 0u;
    uint32_t incl = 0u;
    if (tid < RADIX) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const uint32_t c = s_cnt[w * RADIX + tid];
            s_cnt[w * RADIX + tid] = tile_count;  // exclusive over waves
            tile_count += c;
        }
        status_store(my_status, make_status<StatusT>(tile == 0u ? kFlagInclusive : kFlagAggregate,
                                                     tile_count));
        incl = wave_inclusive_sum(tile_count);
        if (lane == kWave - 1) s_wave_total[wave] = incl;
    }
    __syncthreads();

    if (tid < RADIX) {
        uint32_t local_start = incl - tile_count;
        for (int w = 0; w < wave; ++w) local_start += s_wave_total[w];

        // ---- decoupled look-back over earlier tiles -------------------
        uint32_t before = 0u;
        if (tile > 0u) {
            bool failed = false;
            uint32_t spins = 0u;
            uint32_t k = tile - 1u;
            for (;;) {
                const StatusT s = status_load(a.status + static_cast<size_t>(k) * RADIX + tid);
                const uint32_t flag = static_cast<uint32_t>(s >> SW::kShift);
                if (flag == kFlagEmpty) {
                    if (++spins > kSpinLimit) { failed = true; break; }
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                if (flag == kFlagError) { failed = true; break; }
                before += static_cast<uint32_t>(s & SW::kValueMask);
                if (flag == kFlagInclusive) break;
                if (k == 0u) { failed = true; break; }  // tile 0 is always inclusive
                --k;
            }
            if (failed) {
                atomicOr(a.error_word, 1u);
                status_store(my_status, make_status<StatusT>(kFlagError, 0u));
            } else {
                status_store(my_status, make_status<StatusT>(kFlagInclusive, before + tile_count));
            }
        }
        s_goff[tid] = a.digit_base[tid] + before - local_start;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s_cnt[w * RADIX + tid] += local_start;
    }
    __syncthreads();

    // ---- shuffle keys into tile-sorted order in LDS ---------------------
    uint32_t pos[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        pos[j] = wave_cnt[dig[j]] + rank[j];
        s_tile[pos[j]] = key[j];
    }
    __syncthreads();

    // ---- scatter digit runs ------------------------------------------------
    uint32_t dst[PAIRS ? ITEMS : 1];
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

    if constexpr (PAIRS) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) s_tile[pos[j]] = val[j];
        __syncthreads();
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t i = static_cast<uint32_t>(j) * BLOCK + tid;
            if (i < valid && dst[j] < a.n) a.vals_out[dst[j]] = s_tile[i];
        }
    }
}

}  // namespace rs
