// Host-side launchers of the PlaneZip kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pz {

// The device scratch of one compress or decompress call: a buffer reused by
// the calls on one (device, stream) (see the scratch cache of pz_api.hip).
// Its look-back words carry the call's epoch, and its tile counter is never
// reset: a call's tiles are counted from counter_base, so no call clears it.
struct Scratch {
  uint64_t *words;        // look-back status words
  uint32_t *counter;      // tile counter
  uint32_t *err;          // epoch of the last decompress call that found a corrupt stream
  uint8_t *extra;         // per-call buffers (decompress: chunk and block offsets)
  uint32_t epoch;         // this call's epoch, 1..kEpochMax
  uint32_t counter_base;  // tile counter at the start of this call
};

// What a call needs of the scratch: look-back words, per-call bytes, and the
// workgroups that take a tile from the counter (the counter's advance).
struct ScratchNeed {
  size_t words;
  size_t extra;
  uint32_t counted;
};

ScratchNeed compress_scratch_need(uint64_t raw_bytes);
ScratchNeed decompress_scratch_need(uint64_t raw_bytes);

hipError_t fill_u64(uint64_t *p, uint64_t n, uint64_t value, hipStream_t stream);

// Size pass over chunks 0, stride, 2*stride, ...: out_bytes receives their
// stream bytes (2 + payload each), out_raw their raw bytes, chunk_lens their
// header values. Every output is nullable.
hipError_t launch_size(int w, const uint8_t *src, uint64_t raw_bytes, uint32_t codec_mask, int tagged,
                       uint64_t stride, uint64_t *out_bytes, uint64_t *out_raw, uint16_t *chunk_lens,
                       hipStream_t stream);
// Per-block candidate sizes and tags (PlaneZip candidates, tagged).
hipError_t launch_block_sizes(int w, const uint8_t *src, uint64_t raw_bytes, uint16_t *block_sizes,
                              uint8_t *block_tags, hipStream_t stream);

hipError_t launch_compress(int w, const uint8_t *src, uint64_t raw_bytes, uint32_t codec_mask,
                           int tagged, uint8_t *dst, uint64_t *out_bytes, const Scratch &scratch,
                           hipStream_t stream);

hipError_t launch_decompress(int w, const uint8_t *src, uint64_t comp_bytes, uint32_t codec_mask,
                             int tagged, uint8_t *dst, uint64_t raw_bytes, int32_t *status,
                             const Scratch &scratch, hipStream_t stream);

}  // namespace pz
