// Host check of the prefill launches' division by a launch-invariant
// divisor (FastDiv in kda_launch.h): every quotient against the plain
// integer division, exhaustively for small divisors and dividends and at
// random and boundary values up to 2^31 - 1.  Prints "ok" and exits 0.
#include "kda_launch.h"
#include <stdint.h>
#include <stdio.h>

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next31() {
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return uint32_t(rng >> 33);
}

static int check(uint32_t d, uint32_t n) {
    const kda::FastDiv f = kda::make_fastdiv(d);
    const int q = kda::fdiv(int(n), f);
    if (uint32_t(q) != n / d) {
        printf("mismatch: %u / %u = %u, got %d\n", n, d, n / d, q);
        return 1;
    }
    return 0;
}

int main() {
    int bad = 0;
    for (uint32_t d = 1; d <= 4096 && !bad; ++d)
        for (uint32_t n = 0; n <= 20000 && !bad; ++n) bad |= check(d, n);
    const uint32_t edge[] = {0u, 1u, 2u, 3u, 0x7FFFFFFEu, 0x7FFFFFFFu, 0x40000000u, 0x3FFFFFFFu, 0x40000001u};
    for (int i = 0; i < 200000 && !bad; ++i) {
        const uint32_t d = (i & 1) ? (next31() % 100000u) + 1u : next31() | 1u;
        bad |= check(d, next31());
        for (uint32_t e : edge) bad |= check(d, e);
        for (uint32_t j = 0; j < 3; ++j) {  // around multiples of d
            const uint32_t k = next31() / d;
            const uint64_t base = uint64_t(k) * d;
            for (int64_t delta = -1; delta <= 1; ++delta) {
                const int64_t n = int64_t(base) + delta;
                if (n >= 0 && n <= 0x7FFFFFFF) bad |= check(d, uint32_t(n));
            }
        }
    }
    for (uint32_t s = 1; s < 31 && !bad; ++s) {  // powers of two and their neighbours
        for (int64_t dd = -1; dd <= 1; ++dd) {
            const uint32_t d = uint32_t((int64_t(1) << s) + dd);
            for (int i = 0; i < 2000; ++i) bad |= check(d, next31());
            for (uint32_t e : edge) bad |= check(d, e);
        }
    }
    if (!bad) printf("ok\n");
    return bad;
}
