/*
 * pzref — plain CPU oracle of the PlaneZip block codec.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline of the benchmark may load this library. The product path (the HIP
 * library and its Python binding) never calls it and shares no code with it.
 *
 * Method: "PlaneZip: Lossless Bit-Plane Compression of Training Activations
 * Offloaded over PCIe", §III-A (Codec, Stream format), Fig. 2, and §II-B for
 * BPC's delta/bit-plane/XOR transform. The bit layout follows the repository's
 * FORMAT.md, version 1.
 */
#ifndef PZREF_H
#define PZREF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { PZREF_ZVC = 0, PZREF_DBX = 1, PZREF_BX = 2, PZREF_ZBX = 3, PZREF_RAW = 4 };
enum { PZREF_OK = 0, PZREF_EINVAL = 1, PZREF_ENOSPC = 2, PZREF_ECORRUPT = 3 };

#define PZREF_ALL_CODECS 0x1Fu

/* Symbol width for (dtype, elem_bits): dtype 0 = BF16, 1 = FP32, 2 = other.
 * Returns 16 or 32, or -1 for an unsupported pair. */
int pzref_width(int dtype, int elem_bits);

/* Number of chunks and the worst-case stream size (every chunk raw). */
size_t pzref_num_chunks(size_t raw_bytes);
size_t pzref_max_compressed(size_t raw_bytes);

/* Encode one 128-byte block with one candidate (no tag). The payload goes to
 * `out` (zeroed by the call, cap_bytes long); *nbits receives its length. */
int pzref_encode_candidate(const uint8_t *block, int w, int cand, uint8_t *out,
                           size_t cap_bytes, int64_t *nbits);

/* Decode one candidate payload of `in` (in_bits long) into a 128-byte block.
 * *consumed receives the bits read. */
int pzref_decode_candidate(const uint8_t *in, int64_t in_bits, int w, int cand,
                           uint8_t *block, int64_t *consumed);

/* Bit counts of the five candidates of one block (payload only, no tag). */
int pzref_block_sizes(const uint8_t *block, int w, int32_t sizes[5]);

/* Plane coder on its own: K planes of L bits (P[0] least significant) and the
 * zero-run field width R. */
int pzref_code_planes(const uint64_t *P, int K, int L, int R, uint8_t *out,
                      size_t cap_bytes, int64_t *nbits);
int pzref_decode_planes(const uint8_t *in, int64_t in_bits, int K, int L, int R,
                        uint64_t *P, int64_t *consumed);

/* One chunk of raw_len (1..4096) bytes. `payload` must hold raw_len bytes.
 * codec_mask selects the allowed candidates (bit t = tag t); tagged = 0 means
 * a single-codec variant (exactly one bit in codec_mask, no tag written).
 * tags / block_bits (nullable) receive, per block, the chosen candidate and
 * the coded bits including the tag. Returns the header value H (>0) or a
 * negative error. */
int64_t pzref_compress_chunk(const uint8_t *src, size_t raw_len, int w,
                             uint32_t codec_mask, int tagged, uint8_t *payload,
                             uint8_t *tags, int32_t *block_bits);

/* Whole tensor. Returns the stream size in bytes, or a negative error.
 * tags / block_bits (nullable) are per block of the tensor. */
int64_t pzref_compress(const uint8_t *src, size_t raw_bytes, int w,
                       uint32_t codec_mask, int tagged, uint8_t *dst,
                       size_t dst_capacity, uint8_t *tags, int32_t *block_bits);

/* Whole tensor. Returns PZREF_OK or an error; on PZREF_ECORRUPT the output is
 * unspecified. */
int pzref_decompress(const uint8_t *src, size_t comp_bytes, int w,
                     uint32_t codec_mask, int tagged, uint8_t *dst,
                     size_t raw_bytes);

/* The same two calls spread over `threads` POSIX threads, chunk by chunk.
 * They return exactly what the single-threaded calls return. */
int64_t pzref_compress_mt(const uint8_t *src, size_t raw_bytes, int w,
                          uint32_t codec_mask, int tagged, uint8_t *dst,
                          size_t dst_capacity, int threads);
int pzref_decompress_mt(const uint8_t *src, size_t comp_bytes, int w,
                        uint32_t codec_mask, int tagged, uint8_t *dst,
                        size_t raw_bytes, int threads);

#ifdef __cplusplus
}
#endif

#endif
