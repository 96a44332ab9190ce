/*
 * oracle.h -- plain, slow, CPU-only reference for the stable LSD radix sort.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists so that the tests, the
 * smoke check and the benchmark's CPU-baseline leg can check and time the GPU
 * library.  Nothing in the product path may include, link or call it, and it
 * shares no source, header, table or helper with the GPU library.
 *
 * Sources (the web pages this method is taken from):
 *   [SS] Silicon Studio blog, "Radix sort を実装 & 測定してみた"
 *   [WA] wandres.dev WebGPU guide, "Radix sort paralelo sobre el scan"
 *   [PM] PMPP study notes ch. 13, "정렬: 라딕스와 머지소트"
 *   [OH] onikatahoshio blog, "高性能计算：GPU上的基数排序"
 *
 * Every function here is pinned by CPU tests against facts the pages or plain
 * mathematics fix (worked example, native comparators, brute force, closed
 * form transform values, stability invariant).
 */
#ifndef LSD_ORACLE_H
#define LSD_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Key kinds.  The sort always moves the caller's original 32-bit patterns;
 * the kind only selects the order-preserving unsigned key the digits are
 * taken from. */
enum oracle_key_kind {
    ORACLE_KEY_U32 = 0,
    ORACLE_KEY_I32 = 1,
    ORACLE_KEY_F32 = 2,
    ORACLE_KEY_U64 = 3,
    ORACLE_KEY_I64 = 4,
    ORACLE_KEY_F64 = 5,
    ORACLE_KEY_U16 = 6,
    ORACLE_KEY_I16 = 7,
    ORACLE_KEY_F16 = 8
};

/* Order-preserving unsigned key of one 32-bit pattern.
 *   u32: the value itself.
 *   i32: sign bit flipped ([WA] "Claves con signo y en coma flotante").
 *   f32: NaN and +-Inf -> 0xFFFFFFFF (the maximum); negative -> all bits
 *        inverted; otherwise sign bit set ([SS] "符号付型、浮動小数点型に対する
 *        radix sort", FloatToOrderedUint policy).
 * Returns 0 for an unknown kind. */
uint32_t oracle_ordered_key(int kind, uint32_t bits);

/* Stable ascending LSD radix sort by the sub-key
 *   S(x) = (K(x) >> begin_bit) & (2^(end_bit-begin_bit) - 1),  K = ordered key,
 * one counting-sort pass per radix_bits-wide digit from the least significant
 * digit up ([WA] "Las tres fases de una pasada"; [OH] "CPU上的基数排序").
 * keys_out receives the caller's original bit patterns, permuted; when
 * vals_in is non-NULL, vals_out receives the values under the same
 * permutation.  Buffers must not overlap.  radix_bits in [1,16].
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure. */
int oracle_lsd_sort(int kind, const uint32_t *keys_in, const uint32_t *vals_in,
                    size_t n, int begin_bit, int end_bit, int radix_bits,
                    uint32_t *keys_out, uint32_t *vals_out);

/* The same sort done one bit at a time with the two-bucket index formula of
 * [SS] "アルゴリズムの詳細": with s_i the number of 0-bits strictly before i
 * and F the total number of 0-bits, item i goes to s_i if its bit is 0 and to
 * F + i - s_i if it is 1.  An independent algorithm used as a cross-check.
 * Same arguments and return values as oracle_lsd_sort (no radix_bits). */
int oracle_split_sort(int kind, const uint32_t *keys_in, const uint32_t *vals_in,
                      size_t n, int begin_bit, int end_bit,
                      uint32_t *keys_out, uint32_t *vals_out);

/* One stable counting-sort pass on decimal digit (x / 10^place) % 10, the
 * pass of the worked example in [WA] "La idea y el requisito de estabilidad".
 * Shares the counting pass with oracle_lsd_sort.  place in [0,9].
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure. */
int oracle_decimal_pass(const uint32_t *in, size_t n, int place, uint32_t *out);

/* 64-bit keys ([SS] "符号付型、浮動小数点型に対する radix sort" ends by noting
 * that 16- and 64-bit types take the same procedure): the kinds
 * ORACLE_KEY_U64/I64/F64 with the rules above, sign bit 63 and the double's
 * exponent field (NaN and +-Inf -> 0xFFFFFFFFFFFFFFFF).  Bit ranges are
 * within [0, 64); values stay 32-bit.  Same returns as the 32-bit calls. */
uint64_t oracle_ordered_key64(int kind, uint64_t bits);
int oracle_lsd_sort64(int kind, const uint64_t *keys_in, const uint32_t *vals_in,
                      size_t n, int begin_bit, int end_bit, int radix_bits,
                      uint64_t *keys_out, uint32_t *vals_out);
int oracle_split_sort64(int kind, const uint64_t *keys_in, const uint32_t *vals_in,
                        size_t n, int begin_bit, int end_bit,
                        uint64_t *keys_out, uint32_t *vals_out);

/* Any key width with 32- or 64-bit values ([SS] "符号付型、浮動小数点型に対する
 * radix sort" ends by noting that 16- and 64-bit types take the same
 * procedure).  kind: any ORACLE_KEY_* (16-bit kinds: sign bit 15, IEEE
 * binary16 exponent field, NaN and +-Inf -> 0xFFFF); keys are arrays of that
 * width; vals_in NULL or val_bytes 4 or 8.  oracle_lsd_sort_any takes
 * counting passes of radix_bits bits, oracle_split_sort_any one-bit splits.
 * Same returns as the 32-bit calls. */
uint64_t oracle_ordered_key_any(int kind, uint64_t bits);
int oracle_lsd_sort_any(int kind, const void *keys_in, const void *vals_in, int val_bytes, size_t n,
                        int begin_bit, int end_bit, int radix_bits, void *keys_out, void *vals_out);
int oracle_split_sort_any(int kind, const void *keys_in, const void *vals_in, int val_bytes, size_t n,
                          int begin_bit, int end_bit, void *keys_out, void *vals_out);

/* 30-bit Morton codes of n points (xyz interleaved, float32), the sort key
 * of an LBVH build ([OH] "高性能计算：GPU上的基数排序" introduces the sort as
 * a step of a GPU BVH build).  Readings (the Morton post itself is not among
 * the sources): per axis, in IEEE single precision, s = 1024 / (hi - lo),
 * t = (p - lo) * s, q = 0 if t is NaN or t <= 0, 1023 if t >= 1023, else
 * floor(t); code = spread(qx) << 2 | spread(qy) << 1 | spread(qz) with bit i
 * of q at bit 3i.  Returns 0, or -1 for NULL pointers or a box with
 * hi <= lo, a non-finite bound, a width hi - lo that overflows single
 * precision, or a scale that is not finite and positive. */
float oracle_morton_scale(float lo, float hi);
int oracle_morton30(const float *xyz, size_t n, const float *lo, const float *hi, uint32_t *codes);

/* CPU context for the benchmark, not a reference: std::sort (stable = 0) or
 * std::stable_sort (stable != 0) of n keys in place, in the native order of
 * the kind; only ORACLE_KEY_U32 and ORACLE_KEY_I32 ([SS] "測定" times
 * std::sort beside its radix sorts).  Returns 0, or -1 for another kind or
 * a NULL pointer with n > 0. */
int oracle_std_sort(int kind, void *keys, size_t n, int stable);

#ifdef __cplusplus
}
#endif

#endif /* LSD_ORACLE_H */
