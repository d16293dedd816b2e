/*
 * Exhaustive check of the oracle's fp32 -> fp16 / bf16 rounding against a second,
 * independent conversion: the host compiler's own _Float16 and __bf16 types (clang,
 * x86-64), whose casts round to nearest even.  Build with clang (gcc 11 has neither
 * type) and link against the oracle library.
 *
 * usage: cast_check <dtype 1=f16 2=bf16> <lo> <hi>   checks fp32 bit patterns [lo, hi)
 * prints "<mismatches> <first mismatching input bits>"
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t orc_float_to_half(int32_t dtype, float x);

static int is_nan_bits(int dtype, uint16_t b) {
    if (dtype == 1) return (b & 0x7C00u) == 0x7C00u && (b & 0x03FFu) != 0;
    return (b & 0x7F80u) == 0x7F80u && (b & 0x007Fu) != 0;
}

int main(int argc, char** argv) {
    if (argc != 4) return 2;
    int dtype = atoi(argv[1]);
    uint64_t lo = strtoull(argv[2], NULL, 0), hi = strtoull(argv[3], NULL, 0);
    uint64_t bad = 0, first = 0;
    for (uint64_t b = lo; b < hi; ++b) {
        uint32_t u = (uint32_t)b;
        float x;
        memcpy(&x, &u, 4);
        uint16_t want;
        if (dtype == 1) { _Float16 h = (_Float16)x; memcpy(&want, &h, 2); }
        else            { __bf16 h = (__bf16)x;     memcpy(&want, &h, 2); }
        uint16_t got = orc_float_to_half(dtype, x);
        int ok = (x != x) ? (is_nan_bits(dtype, got) && is_nan_bits(dtype, want)) : (got == want);
        if (!ok) {
            if (!bad) first = b;
            ++bad;
        }
    }
    printf("%llu %llu\n", (unsigned long long)bad, (unsigned long long)first);
    return 0;
}
