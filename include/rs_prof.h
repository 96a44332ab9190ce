/*
 * rs_prof.h -- measurement hooks of the radix sort library (not part of the
 * sort's interface; used by the benchmark).
 *
 *  - Per-kernel timing: while enabled, every kernel the rs_sort_* calls
 *    launch is bracketed by two hipEvents recorded on the caller's stream;
 *    rs_prof_summary() waits for the recorded events and reports, per kernel
 *    kind, the number of launches and their summed duration.  Enabling adds
 *    two event records per launch, so time the headline number with it off.
 *  - A plain device copy (read n words, write n words) whose byte counts are
 *    known exactly; the benchmark runs it to calibrate hardware byte counters
 *    (FETCH_SIZE / WRITE_SIZE) against algorithmic bytes.
 */
#ifndef RS_PROF_H
#define RS_PROF_H

#include <stddef.h>
#include <stdint.h>

#include "rs.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rs_kernel_kind {
    RS_KERNEL_FILL = 0,   /* zeroes the scan state in temp (and samples the keys of large inputs) */
    RS_KERNEL_HIST = 1,   /* one read of the keys: digit histograms of all passes */
    RS_KERNEL_SCAN = 2,   /* exclusive scan of each pass's digit histogram */
    RS_KERNEL_PASS = 3,   /* one digit pass: rank + chained scan + scatter */
    RS_KERNEL_COPY = 4,   /* plain copies (trivial calls, odd in-place passes) */
    RS_KERNEL_SMALL = 5,  /* a whole sort of a small input in one launch */
    RS_KERNEL_KINDS = 6
} rs_kernel_kind;

/* Turn per-kernel event timing on (non-zero) or off: while on, every kernel
 * the library enqueues is launched with a start and a stop event attached to
 * its dispatch (hipExtLaunchKernel), so each pair spans the kernel's own
 * execution.  Returns the previous setting.  Not thread-safe against
 * concurrent sort calls. */
int rs_prof_enable(int on);

/* Drop every recorded event and zero the accumulated totals. */
void rs_prof_reset(void);

/* Wait for all recorded events, fold them into the totals, and return the
 * totals for `kind`: launches and summed milliseconds.  Returns RS_SUCCESS,
 * or RS_ERROR_INVALID_VALUE for a bad kind or NULL outputs, or
 * RS_ERROR_LAUNCH if an event query failed. */
rs_status rs_prof_summary(int kind, uint64_t *launches, double *total_ms);

/* The one-launch path for small inputs: mode 0 forbids it (every sort takes
 * the multi-launch path), 1 allows it (the default; one workgroup per tile),
 * 2 allows it with a single workgroup that claims every tile of every phase
 * itself.  Any other mode means 1.  Returns the previous mode.  Tests use 0
 * and 2 to cover the multi-launch path at small sizes and the one-launch
 * path's tile claiming.  Not thread-safe against concurrent sort calls. */
int rs_prof_small_path(int mode);

/* Keys per thread of the pass tiles of keys-only sorts of 32-bit keys below
 * 2^30 keys: 0 lets the library choose per size (28, or 16 when fewer
 * rounds of smaller tiles over the compute units cost less), 16 or 28
 * forces that size; other values mean 0.  Returns the previous setting.
 * Tests force each size to cover both at every input size.  Not
 * thread-safe against concurrent sort calls. */
int rs_prof_tile_items(int items);

/* Byte offset in temp of a header word that a multi-launch sort (more than
 * 65536 keys) leaves behind for inspection: which = 0 the error word (0 after
 * success), 1 the first of the per-pass skip flags (one 32-bit word per
 * pass, 1 = the pass moved nothing and was skipped), 2 the order flag (0 =
 * the keys were already in sub-key order, so every pass was skipped), 3 the
 * digit counts of every pass, [passes][8][256] uint32 (pass 0 by segment of
 * position, each segment a run of whole pass tiles, segment s starting at
 * tile floor(s * tiles / 8); pass p >= 1 by segment = top 3 bits of the
 * pass-(p-1) digit, or, for a pass p whose word is 1 in the [8] uint32
 * words at `which` = 4 (written only for inputs of 2^22 keys or more of up
 * to 32 bits), by position: the segment of a key is the number of
 * boundaries at `which` = 5 ([8][7] uint32, row p) at or below the 32-bit
 * X = L * 2^(32 - w) + (index >> s), L being the w = shift_p - begin_bit
 * bits of the ordered key from begin_bit up to pass p's digit, index the
 * key's input index and s the smallest shift, but at least 3, that fits
 * index n - 1 into 32 - w bits).
 * Returns (size_t)-1 for any other `which`.  The one-launch path for small
 * inputs keeps none of these but the error word. */
size_t rs_prof_header_offset(int which);

/* Per-launch durations recorded while timing was on (after folding the
 * pending events as rs_prof_summary does): the milliseconds of every launch
 * of `kind` whose tag equals `sub` (pass launches are tagged with their pass
 * index 0..7, every other launch with -1; sub < 0 selects every launch of
 * the kind), in launch order.  Copies up to `cap` of them into `ms` (which
 * may be NULL) and returns how many there are (0 for a bad kind). */
size_t rs_prof_samples(int kind, int sub, double *ms, size_t cap);

/* Test hook for the device-side guard: while on, the pass-0 kernel of every
 * multi-launch sort never publishes the status words of its tile 0, and
 * every look-back gives up after 64 polls of a status word that is still
 * empty (instead of 2^22).  The tile after tile 0 then gives up through the
 * ordinary bounded wait, publishes an error status and sets the error word;
 * every kernel still runs to its end, and the output is invalid.  Returns
 * the previous setting.  Not thread-safe against concurrent sort calls. */
int rs_prof_force_giveup(int on);

/* Local ranker of the digit passes (and of the one-launch path): mode 0
 * (the default) gives each element one LDS atomic add on its (wave, digit)
 * counter, whose returned value is its rank among the wave's earlier
 * elements with that digit -- stable because the gfx950 LDS serves
 * same-address adds of one wave64 instruction in ascending lane order, a
 * measured property (rs_prof_lds_rank_probe checks it); mode 1 selects the
 * ballot match ranker, which finds each lane's peers with one ballot per
 * digit bit and issues one add per distinct digit, so it never depends on
 * that order (slower: about 60 vector instructions per element).  Mode 1
 * applies to uint32/int32/float32 keys with no values or 32-bit values
 * below 2^30 - 2^16 keys (the 64-bit-status kernels, other key widths,
 * 64-bit values and the Morton sort keep mode 0).  Any other mode means 0.
 * Returns the previous mode.  Not thread-safe against concurrent sort
 * calls. */
int rs_prof_ranker(int mode);

/* Probe of the LDS property the pass kernel's local rank relies on: same-
 * address atomic adds of one wave64 instruction return lane-ascending
 * prefix counts.  `blocks` workgroups of 1024 threads (16 waves); each wave
 * holds `slots` (8, 16 or 28) digits per lane, slot j of lane l being
 * element 64 j + l of the wave's run of 64 * slots words of `digits` (the
 * low 8 bits are the digit), and adds `unit` (1 or 4) per element to its
 * own counter of that digit in LDS, all slots back to back; `ranks` (same
 * shape, DEVICE) receives what each add returned.  The property holds when
 * every returned value is `unit` times the number of the wave's earlier
 * elements (slot, then lane order) with the same digit.  Returns
 * RS_ERROR_INVALID_VALUE for NULL or overlapping arrays, blocks outside
 * [1, 65535], or another slots/unit value; RS_ERROR_LAUNCH if the launch
 * failed. */
rs_status rs_prof_lds_rank_probe(const uint32_t *digits, uint32_t *ranks, int blocks, int slots, int unit,
                                 hipStream_t stream);

/* Copy n 32-bit words from in to out (device pointers, 4-byte aligned, not
 * overlapping) on `stream`.  Uses 16-byte accesses when both pointers are
 * 16-byte aligned and n is a multiple of 4. */
rs_status rs_copy_u32(const uint32_t *in, uint32_t *out, size_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RS_PROF_H */
