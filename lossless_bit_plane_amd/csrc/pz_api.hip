// C ABI of the PlaneZip codec: argument checks and dispatch to the HIP
// kernels. Declarations and the meaning of every argument: include/planezip.h.
#include "../../include/planezip.h"

#include <hip/hip_runtime.h>

#include "pz_launch.h"

namespace {

// Symbol width w for (dtype, elem_bits), or -1. PlaneZip paper §III-A: w is
// 16 for BF16 and 32 for FP32 and every other type; BF16 may also use w = 32
// (BPC's original width, §V-A).
int symbol_width(int dtype, int elem_bits) {
  if (dtype == PZ_DTYPE_BF16 && (elem_bits == 16 || elem_bits == 32)) return elem_bits;
  if ((dtype == PZ_DTYPE_FP32 || dtype == PZ_DTYPE_OTHER) && elem_bits == 32) return 32;
  return -1;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A codec mode: a non-empty subset of the five candidates; an untagged mode
// has exactly one.
bool valid_mode(uint32_t codec_mask, int tagged) {
  if (codec_mask == 0 || (codec_mask & ~(uint32_t)PZ_CODEC_ALL)) return false;
  if (tagged != 0 && tagged != 1) return false;
  return tagged || (codec_mask & (codec_mask - 1)) == 0;
}

pz_status_t from_hip(hipError_t e) { return e == hipSuccess ? PZ_SUCCESS : PZ_ERROR_HIP; }

}  // namespace

extern "C" {

const char *pz_status_string(int status) {
  switch (status) {
    case PZ_SUCCESS: return "success";
    case PZ_ERROR_INVALID_VALUE: return "invalid value";
    case PZ_ERROR_INSUFFICIENT_BUFFER: return "insufficient buffer";
    case PZ_ERROR_CORRUPT_STREAM: return "corrupt stream";
    case PZ_ERROR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

pz_status_t pz_compressed_size_ex(const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                                  uint32_t codec_mask, int tagged, uint64_t *d_out_bytes,
                                  uint16_t *d_chunk_lens, void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || !valid_mode(codec_mask, tagged) || !d_out_bytes || (raw_bytes && !d_src))
    return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u) ||
      (reinterpret_cast<uintptr_t>(d_chunk_lens) & 1u))
    return PZ_ERROR_INVALID_VALUE;
  return from_hip(pz::launch_size(w, static_cast<const uint8_t *>(d_src), raw_bytes, codec_mask, tagged,
                                  d_out_bytes, d_chunk_lens, nullptr, nullptr,
                                  static_cast<hipStream_t>(stream)));
}

pz_status_t pz_compressed_size(const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                               uint64_t *d_out_bytes, uint16_t *d_chunk_lens, void *stream) {
  return pz_compressed_size_ex(d_src, raw_bytes, dtype, elem_bits, PZ_CODEC_ALL, 1, d_out_bytes,
                               d_chunk_lens, stream);
}

pz_status_t pz_block_sizes(const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                           uint16_t *d_sizes, uint8_t *d_tags, void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || (raw_bytes && !d_src)) return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || (reinterpret_cast<uintptr_t>(d_sizes) & 1u)) return PZ_ERROR_INVALID_VALUE;
  return from_hip(pz::launch_size(w, static_cast<const uint8_t *>(d_src), raw_bytes, PZ_CODEC_ALL, 1,
                                  nullptr, nullptr, d_sizes, d_tags, static_cast<hipStream_t>(stream)));
}

pz_status_t pz_compress_ex(const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                           uint32_t codec_mask, int tagged, void *d_dst, size_t dst_capacity,
                           uint64_t *d_out_bytes, void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || !valid_mode(codec_mask, tagged) || !d_out_bytes || (raw_bytes && (!d_src || !d_dst)))
    return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || !aligned16(d_dst) || (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u))
    return PZ_ERROR_INVALID_VALUE;
  if (dst_capacity < PZ_MAX_COMPRESSED_BYTES(raw_bytes)) return PZ_ERROR_INSUFFICIENT_BUFFER;
  return from_hip(pz::launch_compress(w, static_cast<const uint8_t *>(d_src), raw_bytes, codec_mask,
                                      tagged, static_cast<uint8_t *>(d_dst), d_out_bytes,
                                      static_cast<hipStream_t>(stream)));
}

pz_status_t pz_compress(const void *d_src, size_t raw_bytes, int dtype, int elem_bits, void *d_dst,
                        size_t dst_capacity, uint64_t *d_out_bytes, void *stream) {
  return pz_compress_ex(d_src, raw_bytes, dtype, elem_bits, PZ_CODEC_ALL, 1, d_dst, dst_capacity,
                        d_out_bytes, stream);
}

pz_status_t pz_decompress_ex(const void *d_src, size_t comp_bytes, int dtype, int elem_bits,
                             uint32_t codec_mask, int tagged, void *d_dst, size_t raw_bytes,
                             int32_t *d_status, void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || !valid_mode(codec_mask, tagged) || (comp_bytes && !d_src) || (raw_bytes && !d_dst))
    return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || !aligned16(d_dst) || (reinterpret_cast<uintptr_t>(d_status) & 3u))
    return PZ_ERROR_INVALID_VALUE;
  if (comp_bytes < 2 * PZ_NUM_CHUNKS(raw_bytes)) return PZ_ERROR_CORRUPT_STREAM;
  return from_hip(pz::launch_decompress(w, static_cast<const uint8_t *>(d_src), comp_bytes, codec_mask,
                                        tagged, static_cast<uint8_t *>(d_dst), raw_bytes, d_status,
                                        static_cast<hipStream_t>(stream)));
}

pz_status_t pz_decompress(const void *d_src, size_t comp_bytes, int dtype, int elem_bits,
                          void *d_dst, size_t raw_bytes, int32_t *d_status, void *stream) {
  return pz_decompress_ex(d_src, comp_bytes, dtype, elem_bits, PZ_CODEC_ALL, 1, d_dst, raw_bytes,
                          d_status, stream);
}

}  // extern "C"
