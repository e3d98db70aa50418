/*
 * ibp.h -- C ABI of libibp, Invariant Bit Packing on AMD Instinct MI355X
 * (gfx950).
 *
 * Method source, cited as [IBP]: the explainer page "Reducing the GPU Memory
 * Bottleneck with Lossless Compression for ML -- Extended" (Kamath,
 * Krishnamurthy, Canini, Peter), section "Methodology: Invariant Bit Packing
 * (IBP)" with its three phases Preprocessing, Compression and Decompression,
 * and section "System integration".
 *
 * Data model
 * ----------
 * A table is n_rows rows of row_bytes (= S) bytes, row r at byte r*S.  The
 * unit the page calls a tensor is a row here.  A row is cut into n = 8S/W
 * blocks of W bits, W = 16, 32 or 64 (block k = little-endian W-bit word k:
 * with W = 32 a bf16 row packs two elements per block, with W = 16 one, with
 * W = 64 four, or one fp64).  S is a multiple of 4, and of 8 when W = 64.
 * One ibp_metadata (Mask/Bitval) covers the whole table.
 *
 * Compressed image
 * ----------------
 * slots: n_rows slots of S bytes each (the fixed-size buffers of [IBP]
 * System integration), slot r at byte r*S.  flags: ceil(n_rows/64) uint64
 * words, bit (r & 63) of word r >> 6 set when row r is stored compressed
 * (the GPU-side bitmask of [IBP] System integration); unused high bits of
 * the last word are 0.
 *   flag 0: the slot holds the S raw bytes.
 *   flag 1: the slot's first ceil(C/32) little-endian 32-bit words hold the
 *           row stream of C bits, zero padded; later slot bytes are not part
 *           of the image and are neither written nor read.
 * Row stream: bits [0, n) are the participation bits, bit k = 1 when block
 * k was stripped ([IBP] Compression); then the payloads of blocks 0..n-1 in
 * order, each least significant bit first at the running bit cursor, no
 * alignment.  A stripped payload is the block's non-invariant bits in
 * ascending position order (W - p bits, p = popcount(Mask)); any other
 * payload is the whole block (W bits).  So C = n + n*W - p*m for a row with
 * m stripped blocks, and payload k starts at bit n + k*W - p*(number of
 * stripped blocks before k).  A row is stored compressed iff C < n*W.
 *
 * Memory, ownership, streams
 * --------------------------
 * The caller allocates and owns every buffer.  Device pointers are HIP
 * device memory; `sample` and `slots` may also be pinned host memory mapped
 * for the device (pass the pointer ibp_host_device_pointer returns), which
 * the kernels then read across the host link without a staging copy
 * ([IBP] Compression and Decompression use zero-copy access to host memory).
 * row_bytes must be a multiple of 4 and every buffer 4-byte aligned (flags and
 * row ids 8-byte aligned; with W = 64 src, slots and dst 8-byte aligned too);
 * 16-byte aligned slots/src/dst with row_bytes a multiple of 16 enable
 * 16-byte memory operations (W = 32).
 * ibp_compress, ibp_decompress, ibp_decompress_batch and the gathers only
 * enqueue work on `stream` (a hipStream_t, NULL = the null stream) and
 * return at once; they allocate nothing, copy nothing on the host and never
 * synchronise.  The W = 32 decodes ask HIP (hipPointerGetAttributes) whether
 * `slots` is host memory, and then cut rows of 1024 or more blocks into
 * smaller tasks, which suits the host link; the result is the same.
 * The same holds for ibp_compress_batch and the per-position compress and
 * decompress calls; none of these clears memory with a memset (the flag
 * words are written by the compression kernels), so a caller may capture
 * them in a HIP graph and replay it.
 * ibp_build_metadata is synchronous.  The library keeps no state between
 * calls apart from the last HIP error code of the calling thread, the
 * compute-unit count of each device (read once per device, to size
 * launches) and, for ibp_build_metadata_noalloc only, one static scratch
 * array per device.
 *
 * Errors
 * ------
 * Every entry point validates its arguments on the host before it enqueues
 * anything; a negative status means nothing was enqueued.  IBP_ERR_HIP means
 * a HIP call or launch failed; ibp_last_hip_error() gives its hipError_t.
 * A HIP error already pending on the calling thread when an entry point is
 * called (hipPeekAtLastError) is returned as IBP_ERR_HIP before any work is
 * enqueued and is left pending for its owner.
 * A row id outside [0, n_rows) (negative ids included) yields an all-zero
 * output row; the kernels never read outside the image for it.
 */
#ifndef IBP_H_
#define IBP_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IBP_OK 0
#define IBP_ERR_INVALID_ARGUMENT (-1) /* null pointer, overflow, t_ppm > 1e6, bad metadata */
#define IBP_ERR_UNSUPPORTED (-2)      /* block width not 16, 32 or 64; row too long */
#define IBP_ERR_LAYOUT (-3)           /* row_bytes not a multiple of 4, misaligned pointer */
#define IBP_ERR_EMPTY (-4)            /* empty sample */
#define IBP_ERR_HIP (-5)              /* HIP API or launch failure */

/* Largest row ibp_compress accepts (the row's stream is assembled in LDS). */
#define IBP_MAX_COMPRESS_ROW_BYTES 98304u

/* The fixed-size global metadata of [IBP] Preprocessing: one Mask/Bitval
 * pair for every block of the data set, 32 bytes, built once and reused. */
typedef struct ibp_metadata {
    uint32_t width_bits;     /* W: 16, 32 or 64 */
    uint32_t invariant_bits; /* p = popcount(mask) */
    uint64_t mask;           /* bit b set <=> block bit b is invariant; bits >= W are 0 */
    uint64_t bitval;         /* values of the invariant bits; (bitval & ~mask) == 0 */
    uint32_t t_ppm;          /* threshold T in parts per million (0.9 -> 900000) */
    uint32_t reserved;       /* 0 */
} ibp_metadata;

/*
 * [IBP] Preprocessing, host half.  From per-bit one-counts over n_blocks
 * sample blocks: for each bit b < width_bits, the majority value (ties give
 * 0) is invariant when 1e6 * majority_count >= t_ppm * n_blocks, compared in
 * exact integers.  ones: width_bits host counters.  Pure host code; lets
 * counts from several devices or passes be summed before thresholding.
 * Errors: INVALID_ARGUMENT (null, ones[b] > n_blocks, t_ppm > 1e6),
 * UNSUPPORTED (width not 16, 32 or 64), EMPTY (n_blocks == 0).
 */
int ibp_metadata_from_counts(const uint64_t *ones, uint64_t n_blocks,
                             uint32_t width_bits, uint32_t t_ppm,
                             ibp_metadata *out);

/*
 * [IBP] Preprocessing.  Counts the ones of every bit position over the
 * n_blocks W-bit blocks at `sample` (device memory or mapped pinned host
 * memory, 4-byte aligned) on the GPU, then applies the threshold rule of
 * ibp_metadata_from_counts.  out: host struct.  out_ones: optional host
 * array of width_bits counters.  SYNCHRONOUS: waits for `stream`.  Allocates
 * (hipMalloc) and frees a device buffer of partial counts, 256 bytes per
 * workgroup of the count kernel (two per compute unit, plus one, for
 * samples below 2^40 blocks), for the duration of the call.
 */
int ibp_build_metadata(const void *sample, uint64_t n_blocks,
                       uint32_t width_bits, uint32_t t_ppm, ibp_metadata *out,
                       uint64_t *out_ones, void *stream);

/*
 * ibp_build_metadata for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, result and synchronisation, but the
 * partial counts live in a static device array of the library
 * ((IBP_NOALLOC_COUNT_GRID + 1) * 64 uint64 counters, 513 KiB, one copy per
 * device, held until the process ends) instead of a per-call hipMalloc.  It
 * calls no hipMalloc or hipFree.  Samples of up to IBP_NOALLOC_MAX_WORDS
 * 32-bit words (n_blocks / 2 words for W = 16, n_blocks for W = 32,
 * 2 * n_blocks for W = 64); a larger sample returns IBP_ERR_UNSUPPORTED.
 * Every call on a device uses that device's one array (every counter it
 * reads is written by the same call first): calls that overlap on one
 * device, from several threads or streams, race and must be serialised by
 * the caller.
 */
#define IBP_NOALLOC_COUNT_GRID 1024u
#define IBP_NOALLOC_MAX_WORDS (1024ull * 4ull * 524287ull * 2048ull)
int ibp_build_metadata_noalloc(const void *sample, uint64_t n_blocks,
                               uint32_t width_bits, uint32_t t_ppm,
                               ibp_metadata *out, uint64_t *out_ones,
                               void *stream);

/*
 * [IBP] Compression.  src: the n_rows x row_bytes table.  Writes the image
 * (slots, flags) described above and, when row_bits is not NULL,
 * row_bits[r] = C of row r (also for rows stored raw).  src and slots may be
 * device memory or mapped pinned host memory (zero-copy).  src == slots
 * compresses in place, each row into its own fixed-size buffer ([IBP] System
 * integration: in-place compression of host tensors before transfer).  Slot
 * bytes past a compressed row's stream are not part of the image: on device
 * memory the kernels may write zeros there up to the next 64-byte boundary
 * (a write ending inside a 64-byte unit costs HBM a read-modify-write); the
 * rest is not written (in place it keeps raw bytes).  Any other overlap of
 * src and slots is
 * INVALID_ARGUMENT.  Asynchronous on `stream`.  row_bytes <=
 * IBP_MAX_COMPRESS_ROW_BYTES.  Equal inputs give equal bytes.
 */
int ibp_compress(const ibp_metadata *md, uint64_t n_rows, uint64_t row_bytes,
                 const void *src, void *slots, uint64_t *flags,
                 uint32_t *row_bits, void *stream);

/*
 * One tensor of a batched compression: its n_rows x row_bytes table `src`,
 * its image (slots, flags) and optional row_bits, with the meaning, memory
 * classes and alignment of ibp_compress's arguments.
 */
typedef struct ibp_compress_tensor {
  uint64_t n_rows;
  uint64_t row_bytes;
  const void *src;
  void *slots;
  uint64_t *flags;
  uint32_t *row_bits;
} ibp_compress_tensor;

/*
 * [IBP] Compression of n_tensors tensors that share the metadata `md` (the
 * weight matrices of a model layer): each tensor's image exactly as
 * ibp_compress would write it.  With W = 32 or 16, the tensors whose rows
 * are 8, 16, 28 or 32 KiB are compressed in one launch per row length and 16
 * tensors; any other tensor is compressed as by ibp_compress.  The descriptor array is host memory and is read before the
 * call returns.  Every tensor is checked first (the rules of ibp_compress);
 * on an error nothing is enqueued.  n_tensors == 0 is a no-op.  Tensors must
 * not overlap each other's buffers (each may compress in place).
 * Asynchronous on `stream`.
 */
int ibp_compress_batch(const ibp_metadata *md, const ibp_compress_tensor *tensors,
                       uint64_t n_tensors, void *stream);

/*
 * [IBP] Decompression of the whole table: dst row r = row r restored.
 * slots: device memory or mapped pinned host memory; flags, dst: device.
 * Asynchronous on `stream`.
 */
int ibp_decompress(const ibp_metadata *md, uint64_t n_rows, uint64_t row_bytes,
                   const void *slots, const uint64_t *flags, void *dst,
                   void *stream);

/*
 * One tensor of a batched decompression: its image (slots, flags) and the
 * device buffer its rows are restored into (n_rows x row_bytes bytes), with
 * the same memory classes and alignment as ibp_decompress.
 */
typedef struct ibp_tensor {
  uint64_t n_rows;
  uint64_t row_bytes;
  const void *slots;
  const uint64_t *flags;
  void *dst;
} ibp_tensor;

/*
 * [IBP] Decompression of n_tensors whole tensors that share the metadata
 * `md` (the weight matrices of a model layer, loaded layer by layer):
 * tensors[t].dst = tensor t restored, as ibp_decompress would give it, in
 * one launch per 16 tensors instead of one per tensor.  The descriptor array
 * is host memory and is read before the call returns.  Every tensor is
 * validated first; on an error nothing is enqueued.  n_tensors == 0 is a
 * no-op.  Tensors must not overlap each other's outputs.  Every width in
 * one launch per 16 tensors, except W = 64 batches that hold a tensor of
 * 512-byte to 2 KiB rows (those rows decode faster through their own
 * kernel), which decode tensor by tensor.  Asynchronous on `stream`.
 */
int ibp_decompress_batch(const ibp_metadata *md, const ibp_tensor *tensors,
                         uint64_t n_tensors, void *stream);

/*
 * Gather-decompress: dst row i = row row_ids[i] restored, for i < n_ids, in
 * id order; duplicate ids are allowed; an id outside [0, n_rows) gives a
 * zero row.  The fetch of a feature / embedding /
 * KV page by index that the page's GNN, DLRM and LLM integrations perform
 * ([IBP] Decompression; System integration).  row_ids: device int64 array.
 * n_ids == 0 is a no-op.  Asynchronous on `stream`.
 */
int ibp_gather_decompress(const ibp_metadata *md, uint64_t n_rows,
                          uint64_t row_bytes, const void *slots,
                          const uint64_t *flags, const int64_t *row_ids,
                          uint64_t n_ids, void *dst, void *stream);

/*
 * Compressed row cache in GPU memory ([IBP] System integration: tensors kept
 * in a GPU software cache are stored compressed, so the same memory holds
 * more of them).
 *
 * Packed arena: a device buffer holding the stored form of selected rows of
 * an image back to back, each entry starting at a 16-byte boundary: entry e
 * is the first `words` 32-bit words of the row's slot (the stream of a
 * compressed row, the S raw bytes of a raw row), zero padded to a multiple
 * of 4 words.
 *
 * Locator (uint64): where a table row lives in the arena.
 *   bit 63       IBP_LOC_RESIDENT: the row is in the arena (0: it is not; a
 *                locator of 0 means "not cached")
 *   bit 62       IBP_LOC_COMPRESSED: the entry is a compressed stream (the
 *                row's flag in the image)
 *   bits 36..61  words: 32-bit words stored (ceil(C/32), or S/4 when raw)
 *   bits 0..35   offset of the entry in the arena, in 16-byte units
 */
#define IBP_LOC_RESIDENT (1ull << 63)
#define IBP_LOC_COMPRESSED (1ull << 62)
#define IBP_LOC_WORDS_SHIFT 36
#define IBP_LOC_WORDS_MASK ((1ull << 26) - 1)
#define IBP_LOC_OFFSET_MASK ((1ull << 36) - 1)

/*
 * Plans a packed arena for the rows row_ids[0..n_ids) of an image (slots,
 * flags as ibp_compress wrote them; slots may be mapped pinned host memory).
 * entry_loc (device, n_ids uint64): the locator of entry e = row row_ids[e],
 * entries laid out in id order; an id outside [0, n_rows) gets locator 0 and
 * no space.  *arena_bytes (host): bytes the arena needs.  SYNCHRONOUS: waits
 * for `stream`.  Allocates (hipMalloc) and frees a scratch buffer of 8 bytes
 * per 4096 ids, plus 8, for the duration of the call.  Errors as for
 * ibp_gather_decompress; UNSUPPORTED when the arena would exceed 2^40 bytes.
 */
int ibp_cache_plan(const ibp_metadata *md, uint64_t n_rows, uint64_t row_bytes,
                   const void *slots, const uint64_t *flags, const int64_t *row_ids,
                   uint64_t n_ids, uint64_t *entry_loc, uint64_t *arena_bytes,
                   void *stream);

/*
 * Fills the arena planned by ibp_cache_plan (same row_ids and entry_loc) and
 * the table's locators: cache_loc (device, n_rows uint64) is cleared to 0,
 * then cache_loc[row_ids[e]] = entry_loc[e] for every resident entry.  A row
 * listed twice gets two entries, and cache_loc points at one of them.
 * arena: device, 16-byte aligned, arena_bytes long; an entry that would end
 * past arena_bytes is skipped (its row stays uncached).  Asynchronous on
 * `stream`.
 */
int ibp_cache_fill(const ibp_metadata *md, uint64_t n_rows, uint64_t row_bytes,
                   const void *slots, const uint64_t *flags, const int64_t *row_ids,
                   uint64_t n_ids, const uint64_t *entry_loc, void *arena,
                   uint64_t arena_bytes, uint64_t *cache_loc, void *stream);

/*
 * Gather-decompress through the cache: dst row i = row row_ids[i] restored,
 * decoded from the arena when cache_loc[row_ids[i]] is resident (a hit),
 * else from the image (slots, flags) (a miss; with slots in mapped pinned
 * host memory that is the zero-copy fetch over the host link).  Same id rules
 * and output as ibp_gather_decompress.  arena, cache_loc: as ibp_cache_fill
 * left them (device).  Asynchronous on `stream`.
 */
int ibp_gather_decompress_cached(const ibp_metadata *md, uint64_t n_rows,
                                 uint64_t row_bytes, const void *arena,
                                 const uint64_t *cache_loc, const void *slots,
                                 const uint64_t *flags, const int64_t *row_ids,
                                 uint64_t n_ids, void *dst, void *stream);

/*
 * Per-position metadata: the reading of [IBP] Preprocessing in which the
 * fixed-size metadata of a few kilobytes holds one Mask/Bitval pair per block
 * position k of a row (k < n = S/4), each chosen by the threshold rule from
 * the k-th blocks of the sample rows.  The stream format is the one above
 * with Mask, Bitval and p taken at each block's own position: payload k has
 * 32 - p_k bits when stripped, so C = n + sum over k of (stripped ? 32 - p_k
 * : 32), and payload k starts at bit n + 32k - (sum of p_j over stripped
 * j < k).  W = 32 only.
 *
 * Position table (device memory, 16-byte aligned,
 * ibp_positional_table_bytes(n) bytes): for each position k a 32-byte entry
 * {Mask_k, Bitval_k, p_k, five 32-bit masks derived from ~Mask_k that drive
 * the bit extract and deposit (the parallel suffix method of Hacker's
 * Delight)}, then for each 64-position chunk c six 64-bit planes of the p
 * values (bit L of plane t = bit t of p at position 64c + L) and two zero
 * words.  Built by ibp_positional_table or ibp_build_metadata_positional;
 * the other calls take it as it is and assume it was built for n = S/4.
 */
uint64_t ibp_positional_table_bytes(uint64_t n_positions);

/* Host: fills `table` (host memory, ibp_positional_table_bytes(n) bytes)
 * from the n pairs mask[k], bitval[k].  INVALID_ARGUMENT when a bitval has
 * bits outside its mask, or on null pointers with n > 0. */
int ibp_positional_table(const uint32_t *mask, const uint32_t *bitval,
                         uint64_t n_positions, void *table);

/*
 * Per-position [IBP] Preprocessing on the GPU: counts the ones of every bit
 * at every position over the n_sample_rows rows of S bytes at `sample`
 * (device or mapped pinned host memory, 4-byte aligned), applies the rule of
 * ibp_metadata_from_counts position by position, and writes the table to
 * `table` (device).  mask_out / bitval_out: optional host arrays of n.
 * SYNCHRONOUS.  Allocates (hipMalloc) and frees 128 bytes of counters per
 * position for the duration of the call.
 */
int ibp_build_metadata_positional(const void *sample, uint64_t n_sample_rows,
                                  uint64_t row_bytes, uint32_t t_ppm, void *table,
                                  uint32_t *mask_out, uint32_t *bitval_out,
                                  void *stream);

/* ibp_compress with per-position metadata (same image layout, flags and
 * row_bits; in place allowed).  row_bytes <= IBP_MAX_COMPRESS_ROW_BYTES. */
int ibp_compress_positional(const void *table, uint64_t n_rows, uint64_t row_bytes,
                            const void *src, void *slots, uint64_t *flags,
                            uint32_t *row_bits, void *stream);

/* ibp_decompress with per-position metadata. */
int ibp_decompress_positional(const void *table, uint64_t n_rows, uint64_t row_bytes,
                              const void *slots, const uint64_t *flags, void *dst,
                              void *stream);

/* ibp_gather_decompress with per-position metadata (same id rules). */
int ibp_gather_decompress_positional(const void *table, uint64_t n_rows,
                                     uint64_t row_bytes, const void *slots,
                                     const uint64_t *flags, const int64_t *row_ids,
                                     uint64_t n_ids, void *dst, void *stream);

/* (n_rows + 63) / 64: the number of uint64 words of a flag bitmap. */
uint64_t ibp_flag_words(uint64_t n_rows);

/*
 * Device-visible address of pinned host memory (hipHostMalloc'd, e.g. a
 * torch pin_memory tensor), for zero-copy sample/slots arguments.
 * Errors: INVALID_ARGUMENT on null, IBP_ERR_HIP when the memory is not
 * mapped for the current device (the failed query's HIP error is cleared;
 * ibp_last_hip_error() keeps it).
 */
int ibp_host_device_pointer(const void *host_ptr, void **device_ptr);

/* Static description of a status code. */
const char *ibp_status_string(int status);

/* hipError_t behind the calling thread's last IBP_ERR_HIP (0 if none). */
int ibp_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IBP_H_ */
