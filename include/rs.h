/*
 * rs.h -- C ABI of the MI355X (gfx950) stable LSD radix sort.
 *
 * The operation.  A stable, ascending least-significant-digit radix sort of
 * 32-bit keys, optionally carrying 32-bit values.  Each pass takes one digit
 * of the key, counts the digits per tile, turns the digit-major count array
 * into global start positions with an exclusive scan, ranks every element
 * among the equal digits of its tile and scatters it stably; passes run from
 * the least significant digit up.  Sources:
 *   - wandres.dev WebGPU guide "Radix sort paralelo sobre el scan",
 *     sections "La idea y el requisito de estabilidad" (LSD order, stability
 *     as the condition of correctness) and "Las tres fases de una pasada"
 *     (histogram, digit-major scan, scatter; ping-pong between passes);
 *   - onikatahoshio "高性能计算：GPU上的基数排序", section "GPU上的基数排序"
 *     (global position = scanned block sum of the digit + local rank);
 *   - PMPP notes "정렬: 라딕스와 머지소트" §13.4 (stage the tile in shared
 *     memory so the scatter writes contiguous runs) and §13.5 (digit width).
 *
 * Result.  keys_out receives the caller's ORIGINAL bit patterns ordered by the
 * sub-key  S(x) = (K(x) >> begin_bit) & (2^(end_bit - begin_bit) - 1),
 * ascending, equal sub-keys in input order (stable).  K is the
 * order-preserving unsigned key of the key type:
 *   u32: K(x) = x;
 *   i32: K(x) = bits(x) ^ 0x80000000  (wandres.dev, "Claves con signo y en
 *        coma flotante": flip the sign bit of a two's complement value);
 *   f32: K(x) = 0xFFFFFFFF if x is NaN or +-Inf, else ~bits(x) if the sign
 *        bit is set, else bits(x) ^ 0x80000000  (Silicon Studio blog "Radix
 *        sort を実装 & 測定してみた", section "符号付型、浮動小数点型に対する
 *        radix sort": NaN and Inf treated as the maximum).  Consequences:
 *        every NaN and both infinities sort last, in input order; -0.0 sorts
 *        before +0.0; denormals keep their value order.  The bit range indexes
 *        K, not the raw pattern.  Keys never pass through floating-point
 *        arithmetic, so NaN payloads and denormals come out unchanged.
 * Values (pairs) move with their keys.
 *
 * Layout.  All key/value pointers are DEVICE pointers to n contiguous 32-bit
 * elements, 4-byte aligned (a misaligned pointer is RS_ERROR_INVALID_VALUE).  temp is a DEVICE pointer, 256-byte aligned, of at
 * least rs_temp_bytes(...) bytes.  The caller owns every buffer; the library
 * allocates nothing, keeps no state between calls, and is reentrant for
 * calls that use distinct temp buffers.
 *
 * Aliasing.  keys_in == keys_out (in place) is allowed, likewise
 * vals_in == vals_out.  Any other overlap between inputs, outputs and temp is
 * invalid.  Inputs that are not written in place are never modified.
 *
 * Asynchrony.  Every call only enqueues work on `stream` (0 = the null
 * stream) and returns; results are ready when the stream is.  A device fault
 * surfaces at the caller's next synchronisation.  Calls that share a temp
 * buffer must be ordered (same stream, or synchronised).
 *
 * Errors.  Arguments are validated on the host before any HIP call:
 *   RS_ERROR_INVALID_VALUE     NULL pointer with n > 0; begin_bit < 0,
 *                              end_bit > 32 or begin_bit > end_bit;
 *                              n > RS_MAX_ELEMENTS; temp not 256-byte
 *                              aligned; forbidden overlap; stream handle of a
 *                              wrong device is NOT detected.
 *   RS_ERROR_INSUFFICIENT_TEMP temp_bytes < rs_temp_bytes(...).
 *   RS_ERROR_LAUNCH            a kernel launch failed (hipGetLastError).
 * Trivial calls (n <= 1 or begin_bit == end_bit) copy input to output (no-op
 * in place) and need no temp (temp may be NULL).
 *
 * Device-side guard.  The chained scan between tiles waits on a bounded spin.
 * If a wait ever exceeds its bound the pass gives up instead of hanging, the
 * output is then invalid, and the 32-bit word at temp offset 0 is non-zero
 * once the stream has completed (it is zero after every successful sort).
 */
#ifndef RS_H
#define RS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rs_status {
    RS_SUCCESS = 0,
    RS_ERROR_INVALID_VALUE = 1,
    RS_ERROR_INSUFFICIENT_TEMP = 2,
    RS_ERROR_LAUNCH = 3,
    RS_ERROR_SCRATCH_LIMIT = 4  /* n exceeds the fixed scratch of rs_sort_keys_u32_noalloc */
} rs_status;

/* Largest supported element count (n must be <= this). */
#define RS_MAX_ELEMENTS ((size_t)0xFFFFFFFFu)

/* Bytes of temp storage a sort of n elements over [begin_bit, end_bit)
 * needs; with_values != 0 for the rs_sort_pairs_* calls.  Pure host function, no HIP
 * call.  Returns 0 for trivial calls (n <= 1 or begin_bit == end_bit) and for
 * invalid arguments (which the sort calls then reject). */
size_t rs_temp_bytes(size_t n, int with_values, int begin_bit, int end_bit);

/* Keys-only sorts; see the header comment for the result, layout, aliasing
 * and errors. */
rs_status rs_sort_keys_u32(const uint32_t *keys_in, uint32_t *keys_out, size_t n,
                           int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                           hipStream_t stream);
rs_status rs_sort_keys_i32(const int32_t *keys_in, int32_t *keys_out, size_t n,
                           int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                           hipStream_t stream);
rs_status rs_sort_keys_f32(const float *keys_in, float *keys_out, size_t n,
                           int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                           hipStream_t stream);

/* Key-value sorts: keys of the named type ordered as above, 32-bit values
 * (any bit pattern) moved with their keys.  With values = 0..n-1 the output
 * values are the stable sorting permutation.  Same layout, aliasing, temp
 * (rs_temp_bytes with with_values != 0) and errors as the keys-only sorts. */
rs_status rs_sort_pairs_u32(const uint32_t *keys_in, uint32_t *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, size_t n,
                            int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                            hipStream_t stream);
rs_status rs_sort_pairs_i32(const int32_t *keys_in, int32_t *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, size_t n,
                            int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                            hipStream_t stream);
rs_status rs_sort_pairs_f32(const float *keys_in, float *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, size_t n,
                            int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                            hipStream_t stream);

/* 64-bit keys.  Silicon Studio blog "Radix sort を実装 & 測定してみた",
 * section "符号付型、浮動小数点型に対する radix sort", closes by noting that
 * 16- and 64-bit types are sorted by the same procedure; these calls apply it
 * to 64-bit keys with the same order-preserving transforms, widened:
 *   u64: K(x) = x;
 *   i64: K(x) = bits(x) ^ 0x8000000000000000;
 *   f64: K(x) = 0xFFFFFFFFFFFFFFFF if the exponent field is all ones (NaN or
 *        +-Inf), else ~bits(x) if the sign bit is set, else
 *        bits(x) ^ 0x8000000000000000.
 * Bit ranges satisfy 0 <= begin_bit <= end_bit <= 64.  Keys are n contiguous
 * 8-byte elements, 8-byte aligned; values (pairs) stay 32-bit.  temp must hold
 * rs_temp_bytes64(...) bytes.  Everything else (result, stability, aliasing,
 * asynchrony, errors, device-side guard) is as for the 32-bit calls. */
size_t rs_temp_bytes64(size_t n, int with_values, int begin_bit, int end_bit);
rs_status rs_sort_keys_u64(const uint64_t *keys_in, uint64_t *keys_out, size_t n,
                           int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                           hipStream_t stream);
rs_status rs_sort_keys_i64(const int64_t *keys_in, int64_t *keys_out, size_t n,
                           int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                           hipStream_t stream);
rs_status rs_sort_keys_f64(const double *keys_in, double *keys_out, size_t n,
                           int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                           hipStream_t stream);
rs_status rs_sort_pairs_u64(const uint64_t *keys_in, uint64_t *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, size_t n,
                            int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                            hipStream_t stream);
rs_status rs_sort_pairs_i64(const int64_t *keys_in, int64_t *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, size_t n,
                            int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                            hipStream_t stream);
rs_status rs_sort_pairs_f64(const double *keys_in, double *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, size_t n,
                            int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                            hipStream_t stream);

/* 16-bit keys and 64-bit values.  The same page section notes that 16-bit
 * types take the same procedure as well; these calls apply the 32-bit rules
 * at bit 15:
 *   u16: K(x) = x;
 *   i16: K(x) = bits(x) ^ 0x8000;
 *   f16 (IEEE binary16 bit patterns, passed as uint16_t): K(x) = 0xFFFF if
 *        the exponent field (bits 10-14) is all ones (NaN or +-Inf), else
 *        ~bits(x) & 0xFFFF if the sign bit is set, else bits(x) ^ 0x8000.
 * Bit ranges satisfy 0 <= begin_bit <= end_bit <= 16; keys are 2-byte
 * aligned.  The *_v64 calls carry 64-bit values (any bit pattern, 8-byte
 * aligned) with keys of the named type.  temp must hold
 * rs_temp_bytes_ex(n, key bytes, value bytes (0, 4 or 8), begin_bit,
 * end_bit) bytes; it returns 0 for trivial calls and invalid arguments.
 * Everything else is as for the 32-bit calls. */
size_t rs_temp_bytes_ex(size_t n, int key_bytes, int value_bytes, int begin_bit, int end_bit);
rs_status rs_sort_keys_u16(const uint16_t *keys_in, uint16_t *keys_out, size_t n,
                           int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                           hipStream_t stream);
rs_status rs_sort_keys_i16(const int16_t *keys_in, int16_t *keys_out, size_t n,
                           int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                           hipStream_t stream);
rs_status rs_sort_keys_f16(const uint16_t *keys_in, uint16_t *keys_out, size_t n,
                           int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                           hipStream_t stream);
rs_status rs_sort_pairs_u16(const uint16_t *keys_in, uint16_t *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, size_t n,
                            int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                            hipStream_t stream);
rs_status rs_sort_pairs_i16(const int16_t *keys_in, int16_t *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, size_t n,
                            int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                            hipStream_t stream);
rs_status rs_sort_pairs_f16(const uint16_t *keys_in, uint16_t *keys_out,
                            const uint32_t *vals_in, uint32_t *vals_out, size_t n,
                            int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                            hipStream_t stream);
rs_status rs_sort_pairs_u16_v64(const uint16_t *keys_in, uint16_t *keys_out,
                                const uint64_t *vals_in, uint64_t *vals_out, size_t n,
                                int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                                hipStream_t stream);
rs_status rs_sort_pairs_i16_v64(const int16_t *keys_in, int16_t *keys_out,
                                const uint64_t *vals_in, uint64_t *vals_out, size_t n,
                                int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                                hipStream_t stream);
rs_status rs_sort_pairs_f16_v64(const uint16_t *keys_in, uint16_t *keys_out,
                                const uint64_t *vals_in, uint64_t *vals_out, size_t n,
                                int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                                hipStream_t stream);
rs_status rs_sort_pairs_u32_v64(const uint32_t *keys_in, uint32_t *keys_out,
                                const uint64_t *vals_in, uint64_t *vals_out, size_t n,
                                int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                                hipStream_t stream);
rs_status rs_sort_pairs_i32_v64(const int32_t *keys_in, int32_t *keys_out,
                                const uint64_t *vals_in, uint64_t *vals_out, size_t n,
                                int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                                hipStream_t stream);
rs_status rs_sort_pairs_f32_v64(const float *keys_in, float *keys_out,
                                const uint64_t *vals_in, uint64_t *vals_out, size_t n,
                                int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                                hipStream_t stream);
rs_status rs_sort_pairs_u64_v64(const uint64_t *keys_in, uint64_t *keys_out,
                                const uint64_t *vals_in, uint64_t *vals_out, size_t n,
                                int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                                hipStream_t stream);
rs_status rs_sort_pairs_i64_v64(const int64_t *keys_in, int64_t *keys_out,
                                const uint64_t *vals_in, uint64_t *vals_out, size_t n,
                                int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                                hipStream_t stream);
rs_status rs_sort_pairs_f64_v64(const double *keys_in, double *keys_out,
                                const uint64_t *vals_in, uint64_t *vals_out, size_t n,
                                int begin_bit, int end_bit, void *temp, size_t temp_bytes,
                                hipStream_t stream);

/* Morton-code sort of points, the sort step of an LBVH build
 * (onikatahoshio "高性能计算：GPU上的基数排序" introduces the radix sort as a
 * step of building a BVH on the GPU, and avoiding a host round trip as the
 * reason to sort there).  The codes are computed where the points are first
 * read (the histogram read and the first pass) and are never written unsorted.
 *
 * xyz: DEVICE pointer to n points of three float32 coordinates (x, y, z
 * interleaved, 12 bytes per point, 4-byte aligned).  box_lo, box_hi: HOST
 * pointers to three floats each, the box the codes cover; finite, with
 * box_hi[a] > box_lo[a], a finite single-precision width
 * box_hi[a] - box_lo[a] and a finite, positive scale 1024 / width.
 * Code of a point: per axis, in single precision, t = (p - lo) * scale and
 * q = 0 if t is NaN or t <= 0, 1023 if t >= 1023, else floor(t) (points
 * outside the box clamp to its faces); code = spread(qx) << 2 |
 * spread(qy) << 1 | spread(qz), bit i of q at bit 3i (30 bits).
 * Result: codes_out (n uint32, DEVICE) holds the codes ascending, index_out
 * (n uint32, DEVICE) the index of each code's point; equal codes keep
 * increasing index order (stable).  The three device arrays and temp must
 * not overlap.  temp: DEVICE, 256-byte aligned, at least
 * rs_temp_bytes_morton30(n) bytes (nonzero for every n >= 1).
 * Errors as for the other sorts; a bad box is RS_ERROR_INVALID_VALUE. */
size_t rs_temp_bytes_morton30(size_t n);
rs_status rs_sort_morton30(const float *xyz, size_t n, const float *box_lo, const float *box_hi,
                           uint32_t *codes_out, uint32_t *index_out, void *temp, size_t temp_bytes,
                           hipStream_t stream);

/* Allocation-free keys-only sort of uint32 keys, for callers that cannot
 * allocate device memory or hand in a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 *
 * Operation, result, layout, aliasing and asynchrony are those of
 * rs_sort_keys_u32, with the temp storage replaced by a fixed scratch array
 * inside the library: RS_NOALLOC_SCRATCH_BYTES bytes of device memory on each
 * GPU the library runs on, held until the process ends.  The call makes no
 * device allocation of its own.  It uses the scratch of the CURRENT device
 * (hipGetDevice); `stream` must belong to that device.
 *
 * Limits and errors.  n <= RS_NOALLOC_MAX_KEYS; a larger n returns
 * RS_ERROR_SCRATCH_LIMIT before any HIP call.  Every other argument error is
 * reported as by rs_sort_keys_u32 (RS_ERROR_INVALID_VALUE, RS_ERROR_LAUNCH;
 * a failed lookup of the scratch address is RS_ERROR_LAUNCH).
 *
 * Sharing.  Every call on one GPU uses that GPU's one scratch array, which
 * keeps the previous call's contents (each call clears the part that must
 * start at zero).  Calls that overlap in time on one GPU -- on different
 * streams, or from different host threads without ordering -- race on the
 * scratch and give wrong results: order them on one stream or synchronise.
 * The device-side guard word of these calls lives in the scratch and is not
 * visible to the caller. */
#define RS_NOALLOC_MAX_KEYS ((size_t)1 << 22)
#define RS_NOALLOC_SCRATCH_BYTES ((size_t)17 << 20)
rs_status rs_sort_keys_u32_noalloc(const uint32_t *keys_in, uint32_t *keys_out, size_t n,
                                   int begin_bit, int end_bit, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *rs_status_string(rs_status status);

#ifdef __cplusplus
}
#endif

#endif /* RS_H */
