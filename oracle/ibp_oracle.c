/*
 * ibp_oracle.c -- plain, slow, bit-serial CPU oracle for Invariant Bit Packing.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the test suite, the smoke check and the CPU
 * baseline of the benchmark load it.  It shares no code, header, table or
 * helper with the HIP library: everything here is written out one bit at a
 * time so that it can be checked against the method's description by eye.
 *
 * Source of the method (cited below as [IBP]): the explainer page
 * "Reducing the GPU Memory Bottleneck with Lossless Compression for ML --
 * Extended" (Kamath, Krishnamurthy, Canini, Peter), section "Methodology:
 * Invariant Bit Packing (IBP)", core algorithm in three phases
 * (Preprocessing / Compression / Decompression), and section
 * "System integration" (fixed-size buffers plus a GPU bitmask).
 *
 * The page gives no byte layout, so the following readings are fixed here
 * (each one is also listed, with its reason, in the design notes):
 *   - a row of S bytes is a bit string, bit i = bit (i mod 8) of byte i/8;
 *     block k is bits [kW, kW+W) of that string (little-endian words);
 *   - one W-bit Mask/Bitval pair for the whole data set;
 *   - bit b is invariant when its majority value covers at least a fraction
 *     T of the sample blocks; T is carried as parts per million and compared
 *     in exact integers; a tie between 0 and 1 picks 0;
 *   - the participation bits of a row (1 = stripped) form an n-bit header in
 *     front of all the payloads; payloads follow in block order, each written
 *     least significant bit first, without alignment;
 *   - a stripped payload keeps the non-invariant bits in ascending position
 *     order (parallel bit extract by ~Mask);
 *   - a row is stored compressed only if its stream is shorter than the raw
 *     row (C < 8S); otherwise the slot holds the raw bytes;
 *   - the stream is zero padded to a 32-bit word (never beyond the slot);
 *     slot bytes past that are not part of the image (the oracle zeroes them).
 *
 * Every function returns 0 on success and a negative value on bad input.
 */
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_EWIDTH (-2)
#define ORC_ELAYOUT (-3)
#define ORC_EEMPTY (-4)

/* ---------------------------------------------------------------- bits -- */

static unsigned get_bit(const uint8_t *buf, uint64_t i)
{
    return (buf[i >> 3] >> (i & 7)) & 1u;
}

static void put_bit(uint8_t *buf, uint64_t i, unsigned v)
{
    if (v)
        buf[i >> 3] = (uint8_t)(buf[i >> 3] | (1u << (i & 7)));
    else
        buf[i >> 3] = (uint8_t)(buf[i >> 3] & ~(1u << (i & 7)));
}

/* Read W bits starting at bit position pos, bit 0 of the result first. */
static uint64_t read_bits(const uint8_t *buf, uint64_t pos, unsigned w)
{
    uint64_t v = 0;
    for (unsigned b = 0; b < w; ++b)
        v |= (uint64_t)get_bit(buf, pos + b) << b;
    return v;
}

static void write_bits(uint8_t *buf, uint64_t pos, unsigned w, uint64_t v)
{
    for (unsigned b = 0; b < w; ++b)
        put_bit(buf, pos + b, (unsigned)((v >> b) & 1u));
}

static uint64_t width_mask(unsigned w)
{
    return w >= 64 ? ~(uint64_t)0 : (((uint64_t)1 << w) - 1);
}

static int width_ok(unsigned w)
{
    return w == 4 || w == 8 || w == 16 || w == 32 || w == 64;
}

static unsigned popcount64(uint64_t x)
{
    unsigned c = 0;
    for (unsigned b = 0; b < 64; ++b)
        c += (unsigned)((x >> b) & 1u);
    return c;
}

/*
 * Parallel bit extract: walk the positions of m from bit 0 upward and copy
 * each selected bit of x to the next free low bit of the result.  This is
 * the "remove the invariant bits and close the gaps" step of [IBP]
 * Compression when called with m = ~Mask.
 */
uint64_t orc_pext(uint64_t x, uint64_t m)
{
    uint64_t r = 0;
    unsigned k = 0;
    for (unsigned b = 0; b < 64; ++b) {
        if ((m >> b) & 1u) {
            r |= ((x >> b) & 1u) << k;
            ++k;
        }
    }
    return r;
}

/*
 * Parallel bit deposit, the inverse: the low bits of v go, in order, to the
 * set positions of m.  Used by [IBP] Decompression to put the stored bits
 * back around the invariant positions.
 */
uint64_t orc_pdep(uint64_t v, uint64_t m)
{
    uint64_t r = 0;
    unsigned k = 0;
    for (unsigned b = 0; b < 64; ++b) {
        if ((m >> b) & 1u) {
            r |= ((v >> k) & 1u) << b;
            ++k;
        }
    }
    return r;
}

/* ------------------------------------------------------------ metadata -- */

/*
 * [IBP] Preprocessing: look at a batch of input blocks and mark the bit
 * positions that keep one value in at least a fraction T of them.
 *
 * ones[b]  = number of sample blocks whose bit b is 1       (b < W)
 * zeros_b  = n_blocks - ones[b]
 * majority = 1 if ones > zeros, else 0 (a tie picks 0)
 * count    = max(ones, zeros)
 * invariant  <=>  1e6 * count >= t_ppm * n_blocks   (exact, 128-bit)
 * Mask bit b = invariant, Bitval bit b = invariant and majority.
 *
 * ones_out may be NULL; otherwise it receives W counters.
 */
int orc_build_metadata(const uint8_t *sample, uint64_t n_blocks, unsigned w,
                       uint32_t t_ppm, uint64_t *ones_out, uint64_t *mask_out,
                       uint64_t *bitval_out)
{
    if (!width_ok(w))
        return ORC_EWIDTH;
    if (!sample || !mask_out || !bitval_out || t_ppm > 1000000u)
        return ORC_EINVAL;
    if (n_blocks == 0)
        return ORC_EEMPTY;

    uint64_t ones[64];
    for (unsigned b = 0; b < 64; ++b)
        ones[b] = 0;
    for (uint64_t i = 0; i < n_blocks; ++i) {
        for (unsigned b = 0; b < w; ++b)
            ones[b] += get_bit(sample, i * w + b);
    }

    uint64_t mask = 0, bitval = 0;
    for (unsigned b = 0; b < w; ++b) {
        uint64_t zeros = n_blocks - ones[b];
        unsigned majority = ones[b] > zeros ? 1u : 0u;
        uint64_t count = majority ? ones[b] : zeros;
        unsigned __int128 lhs = (unsigned __int128)count * 1000000u;
        unsigned __int128 rhs = (unsigned __int128)n_blocks * t_ppm;
        if (lhs >= rhs) {
            mask |= (uint64_t)1 << b;
            if (majority)
                bitval |= (uint64_t)1 << b;
        }
    }
    if (ones_out)
        for (unsigned b = 0; b < w; ++b)
            ones_out[b] = ones[b];
    *mask_out = mask;
    *bitval_out = bitval;
    return ORC_OK;
}

/* --------------------------------------------------------- row codec ---- */

static int row_args_ok(uint64_t row_bytes, unsigned w, uint64_t mask,
                       uint64_t bitval)
{
    if (!width_ok(w))
        return ORC_EWIDTH;
    if (row_bytes == 0 || (row_bytes * 8) % w != 0)
        return ORC_ELAYOUT;
    if ((mask & ~width_mask(w)) != 0 || (bitval & ~mask) != 0)
        return ORC_EINVAL;
    return ORC_OK;
}

/* Bytes of a slot that belong to the image: the stream padded to a 32-bit
 * word for a compressed row, the whole slot for a raw one. */
uint64_t orc_stored_bytes(uint64_t row_bytes, uint64_t c_bits, int flag)
{
    if (!flag)
        return row_bytes;
    uint64_t b = ((c_bits + 31) / 32) * 4;
    return b < row_bytes ? b : row_bytes;
}

/*
 * [IBP] Compression of one row ("tensor") of S bytes into its slot of S
 * bytes.  Steps, in the page's order:
 *   1. split into n = 8S/W blocks;
 *   2. a block matches when its invariant positions equal Bitval;
 *   3. a matching block loses its invariant bits (extract by ~Mask), the
 *      others are kept whole;
 *   4. each block gets a participation bit (1 = stripped); the n bits lead
 *      the stream, then the payloads in block order;
 *   5. with a fixed-size buffer per row ([IBP] System integration), a row
 *      whose stream would not be shorter than the raw row is stored raw.
 * *c_bits receives C = n + sum of payload lengths, *flag = (C < 8S).
 */
int orc_compress_row(const uint8_t *row, uint64_t row_bytes, unsigned w,
                     uint64_t mask, uint64_t bitval, uint8_t *slot,
                     uint64_t *c_bits, int *flag)
{
    int rc = row_args_ok(row_bytes, w, mask, bitval);
    if (rc)
        return rc;
    if (!row || !slot || !c_bits || !flag)
        return ORC_EINVAL;

    const uint64_t n = row_bytes * 8 / w;
    const uint64_t keep = ~mask & width_mask(w);
    const unsigned p = popcount64(mask);

    uint64_t c = n;
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t x = read_bits(row, k * w, w);
        int match = (x & mask) == bitval;
        c += match ? (uint64_t)(w - p) : (uint64_t)w;
    }
    int f = c < row_bytes * 8;
    *c_bits = c;
    *flag = f;

    if (!f) {
        memcpy(slot, row, row_bytes);
        return ORC_OK;
    }

    memset(slot, 0, row_bytes);
    uint64_t cursor = 0;
    for (uint64_t k = 0; k < n; ++k) { /* participation header */
        uint64_t x = read_bits(row, k * w, w);
        put_bit(slot, cursor++, (x & mask) == bitval);
    }
    for (uint64_t k = 0; k < n; ++k) { /* payloads */
        uint64_t x = read_bits(row, k * w, w);
        if ((x & mask) == bitval) {
            write_bits(slot, cursor, w - p, orc_pext(x, keep));
            cursor += w - p;
        } else {
            write_bits(slot, cursor, w, x);
            cursor += w;
        }
    }
    return cursor == c ? ORC_OK : ORC_EINVAL;
}

/*
 * [IBP] Decompression of one slot back into S raw bytes: read the n
 * participation bits, then walk the payloads; a stripped block gets its
 * invariant bits back from Bitval (deposit by ~Mask, then OR Bitval).
 */
int orc_decompress_row(const uint8_t *slot, uint64_t row_bytes, unsigned w,
                       uint64_t mask, uint64_t bitval, int flag, uint8_t *row)
{
    int rc = row_args_ok(row_bytes, w, mask, bitval);
    if (rc)
        return rc;
    if (!slot || !row)
        return ORC_EINVAL;
    if (!flag) {
        memcpy(row, slot, row_bytes);
        return ORC_OK;
    }
    const uint64_t n = row_bytes * 8 / w;
    const uint64_t keep = ~mask & width_mask(w);
    const unsigned p = popcount64(mask);
    const uint64_t limit = row_bytes * 8;

    uint64_t cursor = n;
    for (uint64_t k = 0; k < n; ++k) {
        int stripped = (int)get_bit(slot, k);
        unsigned len = stripped ? w - p : w;
        if (cursor + len > limit)
            return ORC_ELAYOUT; /* stream runs past the slot: corrupt */
        uint64_t v = read_bits(slot, cursor, len);
        cursor += len;
        uint64_t x = stripped ? (orc_pdep(v, keep) | bitval) : v;
        write_bits(row, k * w, w, x);
    }
    return ORC_OK;
}

/* ---------------------------------------------------------- tables ------ */

/*
 * Compress n_rows rows laid out back to back (row r at src + r*S) into the
 * slotted image: slot r at slots + r*S, flag of row r in bit (r & 63) of
 * flags[r >> 6] (unused high bits of the last word are 0), and optionally
 * row_bits[r] = C of row r ([IBP] System integration: fixed-size buffers
 * and a bitmask of compressed rows).
 */
int orc_compress_table(const uint8_t *src, uint64_t n_rows, uint64_t row_bytes,
                       unsigned w, uint64_t mask, uint64_t bitval,
                       uint8_t *slots, uint64_t *flags, uint64_t *row_bits)
{
    int rc = row_args_ok(row_bytes, w, mask, bitval);
    if (rc)
        return rc;
    if ((n_rows && (!src || !slots)) || !flags)
        return ORC_EINVAL;
    for (uint64_t i = 0; i < (n_rows + 63) / 64; ++i)
        flags[i] = 0;
    for (uint64_t r = 0; r < n_rows; ++r) {
        uint64_t c;
        int f;
        rc = orc_compress_row(src + r * row_bytes, row_bytes, w, mask, bitval,
                              slots + r * row_bytes, &c, &f);
        if (rc)
            return rc;
        if (f)
            flags[r >> 6] |= (uint64_t)1 << (r & 63);
        if (row_bits)
            row_bits[r] = c;
    }
    return ORC_OK;
}

/*
 * Gather: out row i = decompressed row ids[i], in id order, duplicates
 * allowed.  Ids must lie in [0, n_rows).
 */
int orc_gather_decompress(const uint8_t *slots, const uint64_t *flags,
                          uint64_t n_rows, uint64_t row_bytes, unsigned w,
                          uint64_t mask, uint64_t bitval, const int64_t *ids,
                          uint64_t n_ids, uint8_t *out)
{
    int rc = row_args_ok(row_bytes, w, mask, bitval);
    if (rc)
        return rc;
    if (n_ids && (!slots || !flags || !ids || !out))
        return ORC_EINVAL;
    for (uint64_t i = 0; i < n_ids; ++i) {
        int64_t id = ids[i];
        if (id < 0 || (uint64_t)id >= n_rows)
            return ORC_EINVAL;
        int f = (int)((flags[(uint64_t)id >> 6] >> ((uint64_t)id & 63)) & 1u);
        rc = orc_decompress_row(slots + (uint64_t)id * row_bytes, row_bytes, w,
                                mask, bitval, f, out + i * row_bytes);
        if (rc)
            return rc;
    }
    return ORC_OK;
}

/* ------------------------------------------------ per-position metadata -- */
/*
 * The kilobyte-sized reading of [IBP] Preprocessing ("fixed-size" metadata
 * of a few kilobytes): one Mask/Bitval pair per block position k of a row
 * (k < n), each obtained by the rule of orc_build_metadata from the k-th
 * blocks of the sample rows.  Compression and decompression are the ones
 * above with Mask, Bitval and p taken at each block's own position.
 */
int orc_build_metadata_positional(const uint8_t *sample, uint64_t n_sample_rows,
                                  uint64_t row_bytes, unsigned w, uint32_t t_ppm,
                                  uint64_t *mask_out, uint64_t *bitval_out)
{
    if (!width_ok(w))
        return ORC_EWIDTH;
    if (row_bytes == 0 || (row_bytes * 8) % w != 0)
        return ORC_ELAYOUT;
    if (!sample || !mask_out || !bitval_out)
        return ORC_EINVAL;
    if (n_sample_rows == 0)
        return ORC_EEMPTY;
    const uint64_t n = row_bytes * 8 / w;
    uint8_t *column = (uint8_t *)calloc(n_sample_rows * w / 8 + 8, 1);
    if (!column)
        return ORC_EINVAL;
    int rc = ORC_OK;
    for (uint64_t k = 0; k < n && rc == ORC_OK; ++k) {
        memset(column, 0, n_sample_rows * w / 8 + 8);
        for (uint64_t r = 0; r < n_sample_rows; ++r)
            write_bits(column, r * w, w, read_bits(sample + r * row_bytes, k * w, w));
        rc = orc_build_metadata(column, n_sample_rows, w, t_ppm, NULL, &mask_out[k],
                                &bitval_out[k]);
    }
    free(column);
    return rc;
}

static int positional_args_ok(uint64_t row_bytes, unsigned w, const uint64_t *mask,
                              const uint64_t *bitval)
{
    if (!width_ok(w))
        return ORC_EWIDTH;
    if (row_bytes == 0 || (row_bytes * 8) % w != 0)
        return ORC_ELAYOUT;
    if (!mask || !bitval)
        return ORC_EINVAL;
    for (uint64_t k = 0; k < row_bytes * 8 / w; ++k)
        if ((mask[k] & ~width_mask(w)) != 0 || (bitval[k] & ~mask[k]) != 0)
            return ORC_EINVAL;
    return ORC_OK;
}

/* Compression of one row with per-position metadata: block k matches when
 * its bits under mask[k] equal bitval[k]; a match keeps W - popcount(mask[k])
 * bits (extract by ~mask[k]); header, order, fallback as in orc_compress_row. */
int orc_compress_row_positional(const uint8_t *row, uint64_t row_bytes, unsigned w,
                                const uint64_t *mask, const uint64_t *bitval,
                                uint8_t *slot, uint64_t *c_bits, int *flag)
{
    int rc = positional_args_ok(row_bytes, w, mask, bitval);
    if (rc)
        return rc;
    if (!row || !slot || !c_bits || !flag)
        return ORC_EINVAL;
    const uint64_t n = row_bytes * 8 / w;

    uint64_t c = n;
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t x = read_bits(row, k * w, w);
        int match = (x & mask[k]) == bitval[k];
        c += match ? (uint64_t)(w - popcount64(mask[k])) : (uint64_t)w;
    }
    int shorter = c < row_bytes * 8;
    *c_bits = c;
    *flag = shorter;
    if (!shorter) {
        memcpy(slot, row, row_bytes);
        return ORC_OK;
    }
    memset(slot, 0, row_bytes);
    uint64_t cursor = 0;
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t x = read_bits(row, k * w, w);
        put_bit(slot, cursor++, (x & mask[k]) == bitval[k]);
    }
    for (uint64_t k = 0; k < n; ++k) {
        uint64_t x = read_bits(row, k * w, w);
        if ((x & mask[k]) == bitval[k]) {
            unsigned len = w - popcount64(mask[k]);
            write_bits(slot, cursor, len, orc_pext(x, ~mask[k] & width_mask(w)));
            cursor += len;
        } else {
            write_bits(slot, cursor, w, x);
            cursor += w;
        }
    }
    return cursor == c ? ORC_OK : ORC_EINVAL;
}

int orc_decompress_row_positional(const uint8_t *slot, uint64_t row_bytes, unsigned w,
                                  const uint64_t *mask, const uint64_t *bitval, int flag,
                                  uint8_t *row)
{
    int rc = positional_args_ok(row_bytes, w, mask, bitval);
    if (rc)
        return rc;
    if (!slot || !row)
        return ORC_EINVAL;
    if (!flag) {
        memcpy(row, slot, row_bytes);
        return ORC_OK;
    }
    const uint64_t n = row_bytes * 8 / w;
    const uint64_t limit = row_bytes * 8;
    uint64_t cursor = n;
    for (uint64_t k = 0; k < n; ++k) {
        int stripped = (int)get_bit(slot, k);
        unsigned len = stripped ? w - popcount64(mask[k]) : w;
        if (cursor + len > limit)
            return ORC_ELAYOUT;
        uint64_t v = read_bits(slot, cursor, len);
        cursor += len;
        uint64_t x = stripped ? (orc_pdep(v, ~mask[k] & width_mask(w)) | bitval[k]) : v;
        write_bits(row, k * w, w, x);
    }
    return ORC_OK;
}

int orc_compress_table_positional(const uint8_t *src, uint64_t n_rows, uint64_t row_bytes,
                                  unsigned w, const uint64_t *mask, const uint64_t *bitval,
                                  uint8_t *slots, uint64_t *flags, uint64_t *row_bits)
{
    int rc = positional_args_ok(row_bytes, w, mask, bitval);
    if (rc)
        return rc;
    if ((n_rows && (!src || !slots)) || !flags)
        return ORC_EINVAL;
    for (uint64_t i = 0; i < (n_rows + 63) / 64; ++i)
        flags[i] = 0;
    for (uint64_t r = 0; r < n_rows; ++r) {
        uint64_t c;
        int compressed;
        rc = orc_compress_row_positional(src + r * row_bytes, row_bytes, w, mask, bitval,
                                         slots + r * row_bytes, &c, &compressed);
        if (rc)
            return rc;
        if (compressed)
            flags[r >> 6] |= (uint64_t)1 << (r & 63);
        if (row_bits)
            row_bits[r] = c;
    }
    return ORC_OK;
}

int orc_gather_decompress_positional(const uint8_t *slots, const uint64_t *flags,
                                     uint64_t n_rows, uint64_t row_bytes, unsigned w,
                                     const uint64_t *mask, const uint64_t *bitval,
                                     const int64_t *ids, uint64_t n_ids, uint8_t *out)
{
    int rc = positional_args_ok(row_bytes, w, mask, bitval);
    if (rc)
        return rc;
    if (n_ids && (!slots || !flags || !ids || !out))
        return ORC_EINVAL;
    for (uint64_t i = 0; i < n_ids; ++i) {
        int64_t id = ids[i];
        if (id < 0 || (uint64_t)id >= n_rows)
            return ORC_EINVAL;
        int compressed = (int)((flags[(uint64_t)id >> 6] >> ((uint64_t)id & 63)) & 1u);
        rc = orc_decompress_row_positional(slots + (uint64_t)id * row_bytes, row_bytes, w,
                                           mask, bitval, compressed, out + i * row_bytes);
        if (rc)
            return rc;
    }
    return ORC_OK;
}
