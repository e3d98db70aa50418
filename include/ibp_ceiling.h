/*
 * ibp_ceiling.h -- C ABI of libibp_ceiling, a measuring instrument for
 * libibp on AMD Instinct MI355X (gfx950): a plain gather-copy kernel that
 * moves exactly the bytes a decompression moves, with none of its work.
 *
 * The explainer page "Reducing the GPU Memory Bottleneck with Lossless
 * Compression for ML -- Extended" (Kamath, Krishnamurthy, Canini, Peter)
 * judges its decompressor against the ideal rate of the same transfer
 * without decoding (section "Results": throughput above 95% of the ideal
 * uncompressed rate), and its decompression reads only the compressed part
 * of each fixed-size buffer (section "System integration").  This copy is
 * that ideal for the library's device and host images: for each output row
 * it reads the stored bytes of the requested slot and writes the whole row,
 * so that its time is the floor of the access pattern (random slot reads of
 * the stored length, streaming row writes) on the machine at hand.
 *
 * It is not part of the compression method: the benchmark times it beside
 * the decompression on the same ids, images and outputs.  A plain contiguous
 * copy (ibp_ceiling_copy) gives the practical rate of a streaming read/write
 * mix on the GPU, against which the nominal HBM peak is put in context.
 */
#ifndef IBP_CEILING_H_
#define IBP_CEILING_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest number of tensors one ibp_ceiling_gather_copy call takes. */
#define IBP_CEILING_MAX_TENSORS 16u

/* Flags of ibp_ceiling_gather_copy. */
#define IBP_CEILING_PACK 1u         /* several short rows per 4 KiB task */
#define IBP_CEILING_STREAM_LOADS 2u /* non-temporal slot loads */

/*
 * One tensor of a gather copy.
 *   n_rows     rows of the source table (slots)
 *   row_bytes  S, bytes of a slot and of an output row; a multiple of 16
 *   src        the slots, row r at byte r*S: device memory or pinned host
 *              memory mapped for the device (its device address); 16-byte
 *              aligned
 *   src_bytes  device, n_out uint32: how many leading bytes of the slot of
 *              output row i to copy (the stored length of row ids[i]); values
 *              above S count as S; each is rounded up to a multiple of 16
 *              (16-byte loads)
 *   ids        device, n_out int64 row ids; NULL: row i of the output is
 *              row i of the table (then n_out <= n_rows)
 *   n_out      output rows
 *   dst        device, n_out x S bytes, 16-byte aligned
 * Output row i = the first src_bytes[i] bytes (rounded up to 16) of slot
 * ids[i], then zeros to S; an id outside [0, n_rows) gives a zero row.  The
 * byte counts are indexed by the output row so that they load alongside the
 * ids: a floor must not wait for a lookup the decompression does not pay.
 */
typedef struct ibp_copy_tensor {
  uint64_t n_rows;
  uint64_t row_bytes;
  const void *src;
  const uint32_t *src_bytes;
  const int64_t *ids;
  uint64_t n_out;
  void *dst;
} ibp_copy_tensor;

/*
 * Enqueues one launch on `stream` (a hipStream_t; NULL = the null stream)
 * that copies every tensor as described above, n_tensors <=
 * IBP_CEILING_MAX_TENSORS.  A task is 4 KiB of output: a row or a 4 KiB
 * chunk of a longer row; with IBP_CEILING_PACK in flags, rows shorter than
 * 4 KiB whose size is a power of two times 16 bytes go 4 KiB / S to a task
 * instead.  With IBP_CEILING_STREAM_LOADS the slot loads are non-temporal
 * (the cache policy libibp's decoders give the image reads), otherwise they
 * take the default policy.
 * max_workgroups caps the grid (workgroups of 256 threads; each wave loops
 * over its share of the tasks), 0 = one wave per task.  The result is the
 * same either way.  Asynchronous; allocates nothing.  Returns 0, or -1 (null
 * or misaligned pointer, row_bytes not a multiple of 16 or above 2^26,
 * n_out > n_rows without ids, too many tensors, an unknown flag; nothing
 * enqueued) or -5
 * (launch failure).  Tensors with n_out == 0 are skipped.
 */
int ibp_ceiling_gather_copy(const ibp_copy_tensor *tensors, uint64_t n_tensors,
                            uint32_t max_workgroups, uint32_t flags, void *stream);

/*
 * Enqueues one launch on `stream` that copies n_bytes from src to dst (both
 * device memory, 16-byte aligned, not overlapping; n_bytes a multiple of 16):
 * workgroups of 256 threads stride over 16 KiB tiles, every load and store
 * 16 bytes and non-temporal.  max_workgroups caps the grid, 0 = one
 * workgroup per tile (at most 2^20).  Asynchronous; allocates nothing.
 * Returns 0 (n_bytes == 0: nothing enqueued), -1 (null or misaligned
 * pointer, n_bytes not a multiple of 16; nothing enqueued) or -5 (launch
 * failure).
 */
int ibp_ceiling_copy(const void *src, void *dst, uint64_t n_bytes, uint32_t max_workgroups,
                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* IBP_CEILING_H_ */
