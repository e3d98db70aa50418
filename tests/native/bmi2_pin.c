/*
 * Pins the oracle's bit-serial extract/deposit and its single-block codec to
 * the x86 BMI2 instructions PEXT/PDEP (a hardware library routine).  Built by
 * the test suite with gcc -mbmi2 and linked against the oracle's shared
 * object; prints one line per failed group and exits non-zero on any
 * mismatch.
 *
 * Checks:
 *  1. orc_pext / orc_pdep == _pext_u64 / _pdep_u64 on every 16-bit mask
 *     with random words, and on 10^7 random 64-bit (word, mask) pairs.
 *  2. Width 8, every (Mask, Bitval subset of Mask) pair (3^8 = 6561) and
 *     every byte x, one-block rows (S = 1): the compressed row must be
 *        C    = 1 + (match ? 8 - p : 8)
 *        flag = C < 8
 *        slot = flag ? 1 | PEXT(x, ~Mask) << 1 : x
 *     with bits above C zero, and decompression must give x back.
 *  3. Width 8, rows of four blocks (S = 4), random: the stream is the four
 *     participation bits, then the four payloads, LSB first, no padding.
 */
#include <immintrin.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint64_t orc_pext(uint64_t x, uint64_t m);
uint64_t orc_pdep(uint64_t v, uint64_t m);
int orc_compress_row(const uint8_t *row, uint64_t row_bytes, unsigned w,
                     uint64_t mask, uint64_t bitval, uint8_t *slot,
                     uint64_t *c_bits, int *flag);
int orc_decompress_row(const uint8_t *slot, uint64_t row_bytes, unsigned w,
                       uint64_t mask, uint64_t bitval, int flag, uint8_t *row);

static uint64_t s = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void)
{ /* splitmix64 */
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main(void)
{
    long bad = 0;

    /* 1. extract / deposit */
    long b1 = 0;
    for (uint64_t m = 0; m < 65536; ++m)
        for (int i = 0; i < 64; ++i) {
            uint64_t x = rnd() & 0xFFFF;
            if (orc_pext(x, m) != _pext_u64(x, m)) ++b1;
            if (orc_pdep(x, m) != _pdep_u64(x, m)) ++b1;
        }
    for (long i = 0; i < 10000000; ++i) {
        uint64_t x = rnd(), m = rnd();
        if (i & 1) m &= rnd(); /* vary the mask density */
        if (orc_pext(x, m) != _pext_u64(x, m)) ++b1;
        if (orc_pdep(x, m) != _pdep_u64(x, m)) ++b1;
    }
    if (b1) printf("pext/pdep mismatches: %ld\n", b1);
    bad += b1;

    /* 2. exhaustive one-block rows at width 8 */
    long b2 = 0, pairs = 0;
    for (unsigned m = 0; m < 256; ++m) {
        for (unsigned bv = 0; bv < 256; ++bv) {
            if (bv & ~m) continue;
            ++pairs;
            unsigned p = (unsigned)__builtin_popcount(m);
            for (unsigned x = 0; x < 256; ++x) {
                uint8_t row = (uint8_t)x, slot = 0xAA, back = 0x55;
                uint64_t c = 0;
                int flag = -1;
                if (orc_compress_row(&row, 1, 8, m, bv, &slot, &c, &flag)) { ++b2; continue; }
                int match = (x & m) == bv;
                uint64_t want_c = 1 + (match ? 8 - p : 8);
                int want_flag = want_c < 8;
                uint8_t want_slot = want_flag
                    ? (uint8_t)(1u | (unsigned)_pext_u32(x, ~m & 0xFFu) << 1)
                    : (uint8_t)x;
                if (c != want_c || flag != want_flag || slot != want_slot) ++b2;
                if (orc_decompress_row(&slot, 1, 8, m, bv, flag, &back) || back != x) ++b2;
            }
        }
    }
    if (pairs != 6561) { printf("pair count %ld\n", pairs); ++bad; }
    if (b2) printf("one-block codec mismatches: %ld\n", b2);
    bad += b2;

    /* 3. four-block rows at width 8 */
    long b3 = 0;
    for (int it = 0; it < 200000; ++it) {
        unsigned m = (unsigned)(rnd() & 0xFF), bv = (unsigned)(rnd() & m);
        unsigned p = (unsigned)__builtin_popcount(m);
        uint8_t row[4], slot[4], back[4];
        for (int k = 0; k < 4; ++k) {
            uint64_t r = rnd();
            /* half the blocks forced to match */
            row[k] = (r & 1) ? (uint8_t)((((unsigned)(r >> 8)) & ~m) | bv) : (uint8_t)(r >> 16);
        }
        uint64_t want = 0, c = 0;
        unsigned cur = 0;
        for (int k = 0; k < 4; ++k)
            want |= (uint64_t)(((row[k] & m) == bv) ? 1 : 0) << cur++;
        for (int k = 0; k < 4; ++k) {
            if ((row[k] & m) == bv) {
                want |= (uint64_t)_pext_u32(row[k], ~m & 0xFFu) << cur;
                cur += 8 - p;
            } else {
                want |= (uint64_t)row[k] << cur;
                cur += 8;
            }
        }
        int flag;
        if (orc_compress_row(row, 4, 8, m, bv, slot, &c, &flag)) { ++b3; continue; }
        int want_flag = cur < 32;
        uint32_t got;
        memcpy(&got, slot, 4);
        if (c != cur || flag != want_flag) ++b3;
        else if (flag && got != (uint32_t)want) ++b3;
        else if (!flag && memcmp(slot, row, 4)) ++b3;
        if (orc_decompress_row(slot, 4, 8, m, bv, flag, back) || memcmp(back, row, 4)) ++b3;
    }
    if (b3) printf("four-block stream mismatches: %ld\n", b3);
    bad += b3;

    printf("bmi2 pin: %s (%ld mismatches)\n", bad ? "FAIL" : "ok", bad);
    return bad ? 1 : 0;
}
