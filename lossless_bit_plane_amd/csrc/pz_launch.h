// Host-side launchers of the PlaneZip kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pz {

// Tensors coded by one launch (a batch call is split into launches of at
// most this many).
constexpr int kMaxBatch = 8;

// The device scratch of one compress or decompress launch: a buffer reused by
// the calls on one (device, stream) (see the scratch cache of pz_api.hip).
// Its look-back words carry the call's epoch, and its tile counter is never
// reset: a call's tiles are counted from counter_base, so no call clears it.
struct Scratch {
  uint64_t *words;        // look-back status words
  uint32_t *counter;      // tile counter
  uint32_t *err;          // per tensor of a launch (kMaxBatch words): the epoch of
                          // the last decompress launch that found its stream corrupt
  uint8_t *extra;         // per-call buffers (decompress: chunk and block offsets)
  uint32_t *done;         // decompress: count of located tiles, never reset
  uint32_t epoch;         // this call's epoch, 1..kEpochMax
  uint32_t counter_base;  // tile counter at the start of this call
  uint32_t done_base;     // located-tile count at the start of this call
};

// What a call needs of the scratch: look-back words, per-call bytes, and the
// workgroups that take a tile from the counter (the counter's advance).
struct ScratchNeed {
  size_t words;
  size_t extra;
  uint32_t counted;
  uint32_t done;  // advance of the located-tile count
};

// The tensors of one compress launch. The launch numbers its tiles across the
// tensors (tensor k holds tiles tile_begin .. tile_begin + ntiles - 1, in
// increasing order of k) and takes them from the tile counter in that order;
// tensor k's look-back words are words[tile_begin ..].
struct CTensor {
  const uint8_t *src;
  uint8_t *dst;
  uint64_t *out_bytes;
  uint64_t raw_bytes;
  uint64_t nchunks;
  uint32_t tile_begin;
  uint32_t ntiles;
};
struct CBatch {
  uint32_t n;
  uint32_t total_tiles;
  CTensor t[kMaxBatch];
};

// The tensors of one decompress launch: locate tiles numbered across the
// tensors as in CBatch, decode groups likewise; tensor k reports corruption
// in error word k.
struct DTensor {
  const uint8_t *src;
  uint8_t *dst;
  int32_t *status;
  uint64_t *chunk_off;
  uint16_t *block_off;
  uint64_t comp_bytes;
  uint64_t raw_bytes;
  uint64_t nchunks;
  uint32_t tile_begin;
  uint32_t ntiles;
  uint32_t group_begin;
  uint32_t ngroups;
};
struct DBatch {
  uint32_t n;
  uint32_t total_tiles;
  uint32_t total_groups;
  uint32_t fused;         // 1: one kernel locates and decodes; 0: locate, then decode
  uint32_t locate_lanes;  // lanes per chunk in locate (chunks per tile: 256 / locate_lanes)
  DTensor t[kMaxBatch];
};

// Compress: tiles of the tensors (CTensor::ntiles). Decompress: decode groups
// of a tensor, and its per-call bytes (16-byte multiple).
uint32_t compress_tiles(uint64_t raw_bytes);
uint32_t decode_groups(uint64_t raw_bytes);
size_t decompress_extra(uint64_t raw_bytes);

hipError_t fill_u64(uint64_t *p, uint64_t n, uint64_t value, hipStream_t stream);

// The tensors of one size launch. The size pass of tensor k covers its
// chunks 0, stride, 2*stride, ... (nsampled of them, 16 per workgroup, the
// launch's groups group_begin .. group_begin + ngroups - 1): out_bytes
// receives their stream bytes (2 + payload each), out_raw their raw bytes,
// chunk_lens their header values. Every output is nullable; a tensor with no
// chunks has no groups and gets zeros.
struct STensor {
  const uint8_t *src;
  uint64_t *out_bytes;
  uint64_t *out_raw;
  uint16_t *chunk_lens;
  uint64_t raw_bytes;
  uint64_t nchunks;
  uint64_t stride;
  uint64_t nsampled;
  uint32_t group_begin;
  uint32_t ngroups;
};
struct SBatch {
  uint32_t n;
  uint32_t total_groups;
  STensor t[kMaxBatch];
};

// Fills in nchunks, nsampled and ngroups of a tensor from raw_bytes and stride.
void size_plan(STensor &x);
hipError_t launch_size(int w, const SBatch &batch, uint32_t codec_mask, int tagged, hipStream_t stream);
// Per-block candidate sizes and tags (PlaneZip candidates, tagged).
hipError_t launch_block_sizes(int w, const uint8_t *src, uint64_t raw_bytes, uint16_t *block_sizes,
                              uint8_t *block_tags, hipStream_t stream);

// One launch per kernel for the batch's tensors (each with at least one
// chunk; the batch has at least one tile). Decompress points each tensor's
// chunk_off and block_off into scratch.extra itself.
hipError_t launch_compress(int w, const CBatch &batch, uint32_t codec_mask, int tagged,
                           const Scratch &scratch, hipStream_t stream);
hipError_t launch_decompress(int w, DBatch &batch, uint32_t codec_mask, int tagged,
                             const Scratch &scratch, hipStream_t stream);
// Chooses a decompress batch's launch form from the symbol width and its
// chunk count (fused, locate_lanes) and numbers its locate tiles (tile_begin,
// ntiles, total_tiles); nchunks of every tensor must be set.
void plan_decompress(int w, DBatch &batch);
// The scratch a decompress launch of the batch needs (plan_decompress done, groups filled in).
ScratchNeed decompress_need(const DBatch &batch, size_t extra);
// Status of a decompress call with no chunks: corrupt unless comp_bytes is 0.
hipError_t launch_empty_status(int32_t *status, uint64_t comp_bytes, hipStream_t stream);

}  // namespace pz
