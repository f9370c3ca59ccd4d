// Host-side launchers of the PlaneZip kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pz {

hipError_t fill_u64(uint64_t *p, uint64_t n, uint64_t value, hipStream_t stream);

hipError_t launch_size(int w, const uint8_t *src, uint64_t raw_bytes, uint32_t codec_mask, int tagged,
                       uint64_t *out_bytes, uint16_t *chunk_lens, uint16_t *block_sizes,
                       uint8_t *block_tags, hipStream_t stream);

hipError_t launch_compress(int w, const uint8_t *src, uint64_t raw_bytes, uint32_t codec_mask,
                           int tagged, uint8_t *dst, uint64_t *out_bytes, hipStream_t stream);

hipError_t launch_decompress(int w, const uint8_t *src, uint64_t comp_bytes, uint32_t codec_mask,
                             int tagged, uint8_t *dst, uint64_t raw_bytes, int32_t *status,
                             hipStream_t stream);

}  // namespace pz
