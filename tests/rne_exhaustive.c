/* Exhaustive check of the oracle's fp32 -> bf16 rounding over all 2^32 fp32
 * bit patterns (tests only).  The expected value comes from the definition of
 * round-to-nearest-even, evaluated in double: of the two bf16 neighbours of f
 * (truncation and the next value up in magnitude) take the nearer one, and on
 * a tie the one with an even last mantissa bit; NaN maps to the canonical
 * quiet NaN 0x7fc0.  Usage: rne_exhaustive <path to liboracle.so>.  Exit 0 on
 * success. */
#include <dlfcn.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef void (*round_fn)(const float*, float*, int64_t);

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

static uint32_t expected(uint32_t b) {
    float f = from_bits(b);
    if (isnan(f)) return 0x7fc00000u;
    uint32_t lo = b & 0xffff0000u;              /* toward zero */
    if (lo == b) return b;                       /* already a bf16 value (incl. inf, 0) */
    uint32_t hi = lo + 0x10000u;                 /* next bf16 away from zero; may carry into exponent / inf */
    double dlo = fabs((double)from_bits(lo));
    double dhi = fabs((double)from_bits(hi));    /* inf when hi is the infinity pattern */
    double af = fabs((double)f);
    if ((hi & 0x7fffffffu) == 0x7f800000u) {
        /* above the largest finite bf16: the rounding boundary is the midpoint
         * between max-finite and 2^128 (which is what inf stands for). */
        dhi = ldexp(1.0, 128);
    }
    double down = af - dlo, up = dhi - af;
    if (down < up) return lo;
    if (up < down) return hi;
    return ((lo >> 16) & 1u) ? hi : lo;          /* tie: even */
}

int main(int argc, char** argv) {
    if (argc < 2) { fprintf(stderr, "usage: %s liboracle.so\n", argv[0]); return 2; }
    void* h = dlopen(argv[1], RTLD_NOW);
    if (!h) { fprintf(stderr, "dlopen: %s\n", dlerror()); return 2; }
    round_fn fn = (round_fn)dlsym(h, "oracle_round_bf16");
    if (!fn) { fprintf(stderr, "missing oracle_round_bf16\n"); return 2; }
    const int64_t chunk = 1 << 22;
    float* in = (float*)malloc(sizeof(float) * chunk);
    float* out = (float*)malloc(sizeof(float) * chunk);
    uint64_t bad = 0;
    for (uint64_t base = 0; base < (1ull << 32); base += (uint64_t)chunk) {
        for (int64_t i = 0; i < chunk; ++i) in[i] = from_bits((uint32_t)(base + (uint64_t)i));
        fn(in, out, chunk);
        for (int64_t i = 0; i < chunk; ++i) {
            uint32_t b = (uint32_t)(base + (uint64_t)i);
            uint32_t got = to_bits(out[i]);
            uint32_t want = expected(b);
            if (got != want) {
                if (bad < 10) fprintf(stderr, "mismatch in=%08x got=%08x want=%08x\n", b, got, want);
                ++bad;
            }
        }
    }
    printf("checked 2^32 patterns, mismatches=%llu\n", (unsigned long long)bad);
    return bad ? 1 : 0;
}
