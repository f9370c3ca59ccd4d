/*
 * planezip.h — C ABI of the MI355X (gfx950) PlaneZip block codec.
 *
 * The codec is the one of "PlaneZip: Lossless Bit-Plane Compression of
 * Training Activations Offloaded over PCIe" (arXiv:2610.25033), §III-A
 * "Codec" and its "Stream format" paragraph, and Fig. 2: a tensor is cut into
 * 128-byte blocks of N w-bit symbols; each block is coded with whichever of
 * ZVC, DBX, BX, ZBX or a verbatim copy is shortest, marked by a 3-bit tag;
 * every 4 KB (32 blocks) is a chunk with a 16-bit length header, and a chunk
 * whose coded form is not shorter than its raw bytes is kept uncompressed.
 * The exact bit layout (which the paper leaves partly open) is the
 * repository's FORMAT.md, version 1.
 *
 * Conventions for every entry point:
 *   - All data pointers are device pointers (hipMalloc'd memory or a torch
 *     CUDA/HIP tensor's data_ptr()), owned by the caller, and must be 16-byte
 *     aligned.
 *   - Device scratch (look-back words, tile counters, per-call offsets) is
 *     kept by the library, one buffer per (device, stream), and reused by the
 *     calls on that stream, so a call normally allocates and clears nothing.
 *     A buffer grows, with hipFreeAsync / hipMallocAsync on its stream, when a
 *     call needs more; buffers live until the process ends (a few tens of
 *     bytes per 4 KB chunk of the largest tensor seen on the stream). A
 *     stream handle that is destroyed and handed out again is taken for the
 *     same stream: finish the PlaneZip work of a stream before destroying it.
 *   - `stream` is a hipStream_t (NULL means the null stream). Every call only
 *     enqueues work and returns; results written to device memory are valid
 *     once the stream has been synchronized.
 *   - Because that scratch is found by the stream handle and the look-back
 *     bookkeeping is fixed when a call is enqueued, the compress and
 *     decompress calls (single and batched) refuse, with
 *     PZ_ERROR_INVALID_VALUE and nothing enqueued, hipStreamPerThread (one
 *     handle for a different stream in every host thread) and a stream that
 *     is being captured into a HIP graph (replays would reuse the captured
 *     bookkeeping). Code under graph capture uses pz_compress_noalloc.
 *   - Argument errors are returned synchronously, before anything is
 *     enqueued. A call that needs several launches (a batch of more than 8
 *     tensors, or empty tensors whose sizes are set by a small kernel) may
 *     have enqueued its earlier launches when a later HIP call fails with
 *     PZ_ERROR_HIP. Errors that depend on the data (a corrupt stream) are
 *     written to device memory.
 *   - Calls on different streams are independent (each stream has its own
 *     scratch); apart from that scratch, the library keeps no state between
 *     calls. Calls on different streams may be made from several host
 *     threads; calls that share a stream are ordered by it.
 */
#ifndef PLANEZIP_H
#define PLANEZIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the tensor. In the paper the copy descriptor carries it to
 * the engine (§III-A). */
typedef enum {
    PZ_DTYPE_BF16 = 0,
    PZ_DTYPE_FP32 = 1,
    PZ_DTYPE_OTHER = 2
} pz_dtype_t;

typedef enum {
    PZ_SUCCESS = 0,
    PZ_ERROR_INVALID_VALUE = 1,      /* bad pointer, size, dtype/width pair or alignment */
    PZ_ERROR_INSUFFICIENT_BUFFER = 2, /* destination capacity below the worst case */
    PZ_ERROR_CORRUPT_STREAM = 3,     /* stream fails the decoder's checks */
    PZ_ERROR_HIP = 4                 /* a HIP runtime call or launch failed */
} pz_status_t;

#define PZ_BLOCK_BYTES 128
#define PZ_CHUNK_BYTES 4096
#define PZ_NUM_CHUNKS(n) (((n) + 4095) / 4096)
/* Worst case stream size: every chunk stored raw, plus its 2-byte header. */
#define PZ_MAX_COMPRESSED_BYTES(n) (2 * PZ_NUM_CHUNKS(n) + (n))
/* Largest raw tensor any call takes (512 GiB, above one GPU's memory): the
 * device-wide prefix sums of chunk offsets carry 40-bit values. A larger
 * raw_bytes (raw_bytes[i] in the batched calls) returns
 * PZ_ERROR_INVALID_VALUE. */
#define PZ_MAX_RAW_BYTES ((size_t)1 << 39)

/* Allowed (dtype, elem_bits) pairs; elem_bits is the symbol width w:
 *   BF16 with 16 (the paper's w for BF16) or 32 (BPC's original width, the
 *   §V-A ablation); FP32 with 32; OTHER with 32 (§III-A codes every
 *   type other than BF16 and FP32 as 32-bit symbols).
 * Any other pair returns PZ_ERROR_INVALID_VALUE. */

/* Exact size in bytes of the stream pz_compress would write for the same
 * input, computed without writing a stream — the paper's profiling-iteration
 * measurement (§III-B: during profiling the engine codes each saved tensor
 * only to learn its size, whose value is the sum of the chunk headers).
 *   d_src        raw tensor bytes, raw_bytes long (any length, including 0)
 *   d_out_bytes  one uint64: 2*chunks + sum of chunk payload lengths
 *   d_chunk_lens nullable; PZ_NUM_CHUNKS(raw_bytes) uint16 header values */
pz_status_t pz_compressed_size(const void *d_src, size_t raw_bytes, int dtype,
                               int elem_bits, uint64_t *d_out_bytes,
                               uint16_t *d_chunk_lens, void *stream);

/* Compress raw_bytes bytes of d_src into d_dst (FORMAT.md §5: the uint16
 * header table H[0..C-1], then the chunk payloads). dst_capacity must be at
 * least PZ_MAX_COMPRESSED_BYTES(raw_bytes); d_out_bytes receives the stream
 * length. The stream is a pure function of (bytes, dtype, elem_bits): d_src
 * is read in 16-byte units, so the bytes of its last unit past raw_bytes
 * may be read (d_src is 16-byte aligned, so that unit lies in the same page
 * as the tensor's last byte), and they do not change the stream. */
pz_status_t pz_compress(const void *d_src, size_t raw_bytes, int dtype,
                        int elem_bits, void *d_dst, size_t dst_capacity,
                        uint64_t *d_out_bytes, void *stream);

/* Decompress a stream of comp_bytes bytes into raw_bytes bytes at d_dst.
 * raw_bytes, dtype and elem_bits must be those given to pz_compress; they are
 * not stored in the stream. d_status (nullable, one int32) receives
 * PZ_SUCCESS or PZ_ERROR_CORRUPT_STREAM (FORMAT.md §6); on a corrupt stream
 * the contents of d_dst are unspecified but nothing outside
 * [d_dst, d_dst + raw_bytes) is written and nothing outside
 * [d_src, d_src + comp_bytes) is read. A comp_bytes below 2*chunks is
 * reported synchronously as PZ_ERROR_CORRUPT_STREAM. */
pz_status_t pz_decompress(const void *d_src, size_t comp_bytes, int dtype,
                          int elem_bits, void *d_dst, size_t raw_bytes,
                          int32_t *d_status, void *stream);

/* Codec variants (the single-codec columns the paper compares PlaneZip with,
 * §V-A and Fig. 3: ZVC as in cDMA, BPC's DBX on every block, BX or ZBX
 * alone; and PlaneZip with a subset of its candidates). codec_mask allows
 * candidate t when bit t is set (tags in Fig. 2 order). With tagged = 1 every
 * block carries the 3-bit tag and takes the smallest allowed candidate, equal
 * sizes to the lowest tag; with tagged = 0 the mask must hold exactly one
 * candidate, which every block uses, and no tag is written. In every mode a
 * chunk that does not shrink is kept raw (FORMAT.md §4). A stream must be
 * decompressed with the (codec_mask, tagged) pair it was compressed with;
 * a tagged decoder accepts any tag 0..4 whatever the mask. An empty mask,
 * bits above PZ_CODEC_ALL, or an untagged mask with more than one candidate
 * return PZ_ERROR_INVALID_VALUE. The plain calls above are the same calls
 * with (PZ_CODEC_ALL, 1). */
#define PZ_CODEC_ZVC (1u << 0)
#define PZ_CODEC_DBX (1u << 1)
#define PZ_CODEC_BX (1u << 2)
#define PZ_CODEC_ZBX (1u << 3)
#define PZ_CODEC_RAW (1u << 4)
#define PZ_CODEC_ALL 0x1Fu

pz_status_t pz_compressed_size_ex(const void *d_src, size_t raw_bytes, int dtype,
                                  int elem_bits, uint32_t codec_mask, int tagged,
                                  uint64_t *d_out_bytes, uint16_t *d_chunk_lens,
                                  void *stream);

pz_status_t pz_compress_ex(const void *d_src, size_t raw_bytes, int dtype,
                           int elem_bits, uint32_t codec_mask, int tagged,
                           void *d_dst, size_t dst_capacity,
                           uint64_t *d_out_bytes, void *stream);

pz_status_t pz_decompress_ex(const void *d_src, size_t comp_bytes, int dtype,
                             int elem_bits, uint32_t codec_mask, int tagged,
                             void *d_dst, size_t raw_bytes, int32_t *d_status,
                             void *stream);

/* Batched calls: pz_compress / pz_decompress on `count` separate tensors of
 * one (dtype, elem_bits) in as few launches as possible (up to 8 tensors per
 * launch), for callers that code several tensors at once — the swaps waiting
 * on a copy queue, or every saved tensor measured in the profiling iteration
 * (PlaneZip paper, §III-B and §III-C). Tensor i gets exactly the stream (or
 * output and status) that the single call would give it; streams are not
 * concatenated.
 *   count            >= 0 (0: nothing is enqueued)
 *   d_srcs, d_dsts   host arrays of count device pointers (16-byte aligned;
 *                    a tensor's pointers may be null when its size is 0)
 *   raw_bytes,       host arrays of count sizes, as in the single calls
 *   comp_bytes,
 *   dst_capacities
 *   d_out_bytes      device array of count uint64 (compress)
 *   d_status         nullable device array of count int32 (decompress)
 * Every tensor is checked before anything is enqueued: the first failing
 * check's status is returned (PZ_ERROR_INVALID_VALUE,
 * PZ_ERROR_INSUFFICIENT_BUFFER, or PZ_ERROR_CORRUPT_STREAM for a comp_bytes
 * below 2*chunks) and no tensor is coded. The host arrays are read before
 * the call returns; device buffers follow the single calls' rules, and the
 * tensors of one call must not overlap one another's outputs. */
pz_status_t pz_compress_batch(int count, const void *const *d_srcs,
                              const size_t *raw_bytes, int dtype, int elem_bits,
                              void *const *d_dsts, const size_t *dst_capacities,
                              uint64_t *d_out_bytes, void *stream);

/* pz_compressed_size on `count` tensors of one (dtype, elem_bits) in as few
 * launches as possible (up to 8 tensors per launch): the profiling
 * iteration's measurement of every saved tensor (PlaneZip paper, §III-B).
 *   d_srcs, raw_bytes  host arrays of count device pointers (16-byte aligned)
 *                      and sizes
 *   d_out_bytes        device array of count uint64: tensor i's stream bytes
 *   d_chunk_lens       nullable host array of count nullable device pointers:
 *                      tensor i's PZ_NUM_CHUNKS(raw_bytes[i]) header values
 * Every tensor is checked before anything is enqueued. */
pz_status_t pz_compressed_size_batch(int count, const void *const *d_srcs,
                                     const size_t *raw_bytes, int dtype,
                                     int elem_bits, uint64_t *d_out_bytes,
                                     uint16_t *const *d_chunk_lens, void *stream);

pz_status_t pz_decompress_batch(int count, const void *const *d_srcs,
                                const size_t *comp_bytes, int dtype,
                                int elem_bits, void *const *d_dsts,
                                const size_t *raw_bytes, int32_t *d_status,
                                void *stream);

/* Compression that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. Same arguments, checks and stream as
 * pz_compress (PlaneZip with all five candidates, tagged), but its scratch
 * (a tile counter and one look-back word per 32 KB tile) lives in a fixed
 * 2 MiB device array that the library holds on each GPU it runs on until
 * the process ends; the call allocates and frees nothing (no hipMalloc,
 * hipMallocAsync, hipFree or allocating library routine) and clears the
 * array with a kernel, not a memset.
 *   raw_bytes  at most PZ_NOALLOC_MAX_BYTES; larger sizes return
 *              PZ_ERROR_INVALID_VALUE with nothing enqueued
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (two streams, two host threads)
 * race and must be serialized by the caller. The first call with a device
 * current looks the array's device address up once (hipGetSymbolAddress). */
#define PZ_NOALLOC_MAX_BYTES ((size_t)1073545216) /* 32762 tiles of 32 KB */
pz_status_t pz_compress_noalloc(const void *d_src, size_t raw_bytes, int dtype,
                                int elem_bits, void *d_dst, size_t dst_capacity,
                                uint64_t *d_out_bytes, void *stream);

/* Sampled size: the pz_compressed_size measurement over chunks 0, stride,
 * 2*stride, ... only (the paper's methodology sizes tensors above 32 MB on
 * every fourth 4 KB chunk, §IV "Tensor capture"), at 1/stride of the work.
 *   chunk_stride  >= 1; 1 sizes every chunk
 *   d_sample      two uint64: [0] the stream bytes of the sampled chunks
 *                 (2 header bytes + payload each), [1] their raw bytes; the
 *                 estimated stream size of the tensor is
 *                 raw_bytes * d_sample[0] / d_sample[1] (exact for stride 1)
 *   d_sample_lens nullable; ceil(PZ_NUM_CHUNKS(raw_bytes) / chunk_stride)
 *                 uint16 header values of the sampled chunks, in order
 * A stride of 0 or a misaligned d_sample return PZ_ERROR_INVALID_VALUE. */
pz_status_t pz_compressed_size_sampled(const void *d_src, size_t raw_bytes,
                                       int dtype, int elem_bits,
                                       uint32_t chunk_stride, uint64_t *d_sample,
                                       uint16_t *d_sample_lens, void *stream);

/* Per-tensor compressibility predictor (§III-B "Compressibility Predictor",
 * accuracy in §V-B and Table IV). Host memory only; no device work. A saved
 * tensor is named by a 64-bit signature, normally PZ_SIGNATURE(position of
 * its producing operator in the iteration's operator sequence, output slot).
 * The table keeps one measurement (raw bytes, compressed bytes) per
 * signature: the size the engine reported for a swap (d_out_bytes of
 * pz_compress), or a profiling measurement (pz_compressed_size, or the two
 * words of pz_compressed_size_sampled). A new measurement overwrites the
 * previous one. Every call is safe from several host threads. */
typedef struct pz_predictor pz_predictor_t;

#define PZ_SIGNATURE(op_index, output_slot) \
    ((((uint64_t)(op_index)) << 16) | ((uint64_t)(output_slot) & 0xFFFFu))

/* A table for up to `capacity` signatures (§III-B sizes it at a few hundred
 * entries); NULL for a capacity of 0 or above 2^40, or when host memory runs
 * out. */
pz_predictor_t *pz_predictor_create(size_t capacity);
void pz_predictor_destroy(pz_predictor_t *pred);

/* Records that a tensor of this signature took comp_bytes for raw_bytes.
 * raw_bytes and comp_bytes must be >= 1 and comp_bytes at most
 * PZ_MAX_COMPRESSED_BYTES(raw_bytes) (else PZ_ERROR_INVALID_VALUE); a new
 * signature in a full table returns PZ_ERROR_INSUFFICIENT_BUFFER and changes
 * nothing. */
pz_status_t pz_predictor_update(pz_predictor_t *pred, uint64_t signature,
                                uint64_t raw_bytes, uint64_t comp_bytes);

/* Predicted compressed bytes of a tensor of this signature and raw_bytes:
 * ceil(raw_bytes * comp / raw) of the signature's last measurement, or
 * raw_bytes (a ratio of 1) while it has none. *measured (nullable) is set to
 * 1 or 0 accordingly. A prediction above 2^64-1 returns
 * PZ_ERROR_INVALID_VALUE. */
pz_status_t pz_predictor_predict(pz_predictor_t *pred, uint64_t signature,
                                 uint64_t raw_bytes, uint64_t *pred_bytes,
                                 int *measured);

/* Signatures held, and forgetting them all (e.g. when the operator sequence
 * changes and signatures are renumbered). */
size_t pz_predictor_entries(pz_predictor_t *pred);
void pz_predictor_clear(pz_predictor_t *pred);

/* Time in seconds that one swap of a tensor occupies a copy queue, the
 * planner's cost model (§III-C, Eq. 2): x = min(m / g, max(m / (c g), m / B))
 * with m = raw_bytes, c = ratio (raw over compressed bytes, as the predictor
 * gives it), g = link_bytes_per_s (the copy link, per direction) and
 * B = engine_bytes_per_s (the codec's rate in raw bytes per second, e.g. the
 * measured pz_compress rate). A compressed transfer is bound by the slower of
 * link and engine; the engine is bypassed (m / g) when that is not shorter.
 * Returns -1 if ratio, link_bytes_per_s or engine_bytes_per_s is not a
 * positive finite number. Pure host arithmetic. */
double pz_transfer_time(uint64_t raw_bytes, double ratio, double link_bytes_per_s,
                        double engine_bytes_per_s);

/* Swap engine: the copy path of §III and Fig. 2. A swapped-out tensor is
 * compressed on the GPU into a device staging slot and its stream's exact
 * bytes are copied by DMA into equal-sized pieces of a pinned host pool (the
 * host-side layout of §III-A); swapping in copies the pieces back and
 * decompresses them. The
 * stream's length is known only after the compression has run, so a worker
 * thread of the engine waits for each compression, takes pool chunks and
 * issues the copies on the engine's device-to-host stream; pz_swap_out
 * returns once the compression is enqueued. The engine belongs to the device
 * that is current at creation; all its calls are safe from several host
 * threads. Streams are the callers' (compression and decompression run on
 * them) plus two copy streams of the engine's own (default priority). */
typedef struct pz_swapper pz_swapper_t;

/* pool_chunk_bytes (a multiple of 16) x pool_chunks of pinned host memory,
 * and staging_slots (1..64) device buffers of staging_bytes, which bound the
 * tensors it takes: PZ_MAX_COMPRESSED_BYTES(raw_bytes) <= staging_bytes.
 * More slots let more compressions run ahead of the copies. NULL on bad
 * sizes or when an allocation fails (or there is no device). */
pz_swapper_t *pz_swapper_create(size_t pool_chunk_bytes, size_t pool_chunks,
                                size_t staging_bytes, int staging_slots);
/* Waits for all pending work and frees the pool, the slots and the streams. */
void pz_swapper_destroy(pz_swapper_t *swapper);
/* Pool chunks not held by a swapped-out tensor. */
size_t pz_swapper_free_chunks(pz_swapper_t *swapper);

/* Enqueues the compression of d_src (raw_bytes >= 1, device memory, 16-byte
 * aligned) on `stream`, after the work already there, and returns a ticket
 * (>= 1). d_src may be reused once `stream` has passed this point. Blocks
 * while every staging slot is in use. A tensor above the staging size returns
 * PZ_ERROR_INSUFFICIENT_BUFFER; argument errors are those of pz_compress. */
pz_status_t pz_swap_out(pz_swapper_t *swapper, const void *d_src, size_t raw_bytes,
                        int dtype, int elem_bits, void *stream, uint64_t *ticket);

/* Blocks until the ticket's stream is in the pool. *comp_bytes (nullable):
 * its length. PZ_ERROR_INSUFFICIENT_BUFFER if the pool had too few free
 * chunks (the tensor was not swapped; release the ticket), PZ_ERROR_HIP if a
 * copy failed, PZ_ERROR_INVALID_VALUE for an unknown ticket. */
pz_status_t pz_swap_wait(pz_swapper_t *swapper, uint64_t ticket, uint64_t *comp_bytes);

/* Enqueues the host-to-device copy of the ticket's chunks (after its
 * device-to-host copies) into a staging slot and their decompression into
 * d_dst (raw_bytes of the swap-out) on `stream`; d_status as pz_decompress.
 * Blocks until the worker has handled the swap-out and while every staging
 * slot is in use. The chunks stay held: a ticket can be swapped in again. */
pz_status_t pz_swap_in(pz_swapper_t *swapper, uint64_t ticket, void *d_dst,
                       int32_t *d_status, void *stream);

/* Returns the ticket's pool chunks, after any copy still reading or writing
 * them, and forgets the ticket. */
pz_status_t pz_swap_release(pz_swapper_t *swapper, uint64_t ticket);

/* Copies the ticket's stream (FORMAT.md §5) into h_dst (capacity bytes),
 * after waiting as pz_swap_wait; *comp_bytes (nullable) its length. */
pz_status_t pz_swap_read(pz_swapper_t *swapper, uint64_t ticket, void *h_dst,
                         size_t capacity, uint64_t *comp_bytes);

/* Diagnostics of the size pass, per 128-byte block (nblocks =
 * ceil(raw_bytes/128)): d_sizes (nullable) receives the five candidate sizes
 * in bits (ZVC, DBX, BX, ZBX, RAW; payload only, no tag) as 5*nblocks
 * uint16; d_tags (nullable) receives the chosen tag per block. */
pz_status_t pz_block_sizes(const void *d_src, size_t raw_bytes, int dtype,
                           int elem_bits, uint16_t *d_sizes, uint8_t *d_tags,
                           void *stream);

/* Human-readable name of a status code (static storage). */
const char *pz_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PLANEZIP_H */
