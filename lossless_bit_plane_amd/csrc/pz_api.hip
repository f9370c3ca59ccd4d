// C ABI of the PlaneZip codec: argument checks and dispatch to the HIP
// kernels. Declarations and the meaning of every argument: include/planezip.h.
#include "../../include/planezip.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "pz_device.h"
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

// ---------------------------------------------------------------------------
// Scratch cache. Compress and decompress calls need device scratch (look-back
// words, a tile counter, per-call offsets). Each (device, stream) keeps one
// buffer, reused by the calls on that stream (which the stream orders), so a
// call allocates and clears nothing: look-back words carry the call's epoch
// and the tile counter keeps counting (a call counts its tiles from where the
// previous one left it). The buffer grows (stream-ordered free and
// allocation, then one clearing) when a call needs more, and is cleared again
// when the epoch wraps. Buffer layout: the tile counter and the error word
// (16 bytes), the look-back words, the per-call bytes.
// ---------------------------------------------------------------------------
struct ScratchEntry {
  int device;
  hipStream_t stream;
  uint8_t *base;
  size_t words;       // look-back words held
  size_t extra;       // per-call bytes held
  uint32_t epoch;     // of the last call
  uint32_t counter;   // tile counter after the last call
  bool clear;         // the header and words must be cleared before the next call
};

constexpr size_t kScratchHeader = 16;

std::mutex g_scratch_mu;
std::vector<ScratchEntry> g_scratch;

// Runs `launch(scratch)` with this stream's scratch, under the cache lock (so
// that the epochs and counter bases follow the order in which the calls are
// enqueued).
template <typename F>
hipError_t with_scratch(hipStream_t stream, const pz::ScratchNeed &need, F launch) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchEntry *ent = nullptr;
  for (ScratchEntry &x : g_scratch)
    if (x.device == device && x.stream == stream) ent = &x;
  if (!ent) {
    g_scratch.push_back(ScratchEntry{device, stream, nullptr, 0, 0, 0, 0, true});
    ent = &g_scratch.back();
  }
  if (ent->words < need.words || ent->extra < need.extra || !ent->base) {
    const size_t words = need.words > ent->words ? need.words + need.words / 4 + 64 : ent->words;
    const size_t extra = ((need.extra > ent->extra ? need.extra + need.extra / 4 : ent->extra) + 15) & ~size_t(15);
    if (ent->base) {
      e = hipFreeAsync(ent->base, stream);
      ent->base = nullptr;
      if (e != hipSuccess) return e;
    }
    e = hipMallocAsync(reinterpret_cast<void **>(&ent->base), kScratchHeader + 8 * words + extra, stream);
    if (e != hipSuccess) {
      ent->base = nullptr;
      ent->words = ent->extra = 0;
      return e;
    }
    ent->words = words;
    ent->extra = extra;
    ent->clear = true;
  }
  if (ent->clear || ent->epoch >= pz::kEpochMax) {
    e = pz::fill_u64(reinterpret_cast<uint64_t *>(ent->base), kScratchHeader / 8 + ent->words, 0, stream);
    if (e != hipSuccess) return e;
    ent->epoch = 0;
    ent->counter = 0;
    ent->clear = false;
  }
  pz::Scratch sc;
  sc.counter = reinterpret_cast<uint32_t *>(ent->base);
  sc.err = reinterpret_cast<uint32_t *>(ent->base) + 1;
  sc.words = reinterpret_cast<uint64_t *>(ent->base + kScratchHeader);
  sc.extra = ent->base + kScratchHeader + 8 * ent->words;
  sc.epoch = ++ent->epoch;
  sc.counter_base = ent->counter;
  e = launch(sc);
  if (e == hipSuccess)
    ent->counter += need.counted;  // every workgroup of the call takes one tile
  else
    ent->clear = true;
  return e;
}

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
  return from_hip(pz::launch_size(w, static_cast<const uint8_t *>(d_src), raw_bytes, codec_mask, tagged, 1,
                                  d_out_bytes, nullptr, d_chunk_lens, static_cast<hipStream_t>(stream)));
}

pz_status_t pz_compressed_size(const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                               uint64_t *d_out_bytes, uint16_t *d_chunk_lens, void *stream) {
  return pz_compressed_size_ex(d_src, raw_bytes, dtype, elem_bits, PZ_CODEC_ALL, 1, d_out_bytes,
                               d_chunk_lens, stream);
}

pz_status_t pz_compressed_size_sampled(const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                                       uint32_t chunk_stride, uint64_t *d_sample, uint16_t *d_sample_lens,
                                       void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || chunk_stride == 0 || !d_sample || (raw_bytes && !d_src)) return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || (reinterpret_cast<uintptr_t>(d_sample) & 7u) ||
      (reinterpret_cast<uintptr_t>(d_sample_lens) & 1u))
    return PZ_ERROR_INVALID_VALUE;
  return from_hip(pz::launch_size(w, static_cast<const uint8_t *>(d_src), raw_bytes, PZ_CODEC_ALL, 1,
                                  chunk_stride, d_sample, d_sample + 1, d_sample_lens,
                                  static_cast<hipStream_t>(stream)));
}

pz_status_t pz_block_sizes(const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                           uint16_t *d_sizes, uint8_t *d_tags, void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || (raw_bytes && !d_src)) return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || (reinterpret_cast<uintptr_t>(d_sizes) & 1u)) return PZ_ERROR_INVALID_VALUE;
  return from_hip(pz::launch_block_sizes(w, static_cast<const uint8_t *>(d_src), raw_bytes, d_sizes, d_tags,
                                         static_cast<hipStream_t>(stream)));
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(with_scratch(s, pz::compress_scratch_need(raw_bytes), [&](const pz::Scratch &sc) {
    return pz::launch_compress(w, static_cast<const uint8_t *>(d_src), raw_bytes, codec_mask, tagged,
                               static_cast<uint8_t *>(d_dst), d_out_bytes, sc, s);
  }));
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  return from_hip(with_scratch(s, pz::decompress_scratch_need(raw_bytes), [&](const pz::Scratch &sc) {
    return pz::launch_decompress(w, static_cast<const uint8_t *>(d_src), comp_bytes, codec_mask, tagged,
                                 static_cast<uint8_t *>(d_dst), raw_bytes, d_status, sc, s);
  }));
}

pz_status_t pz_decompress(const void *d_src, size_t comp_bytes, int dtype, int elem_bits,
                          void *d_dst, size_t raw_bytes, int32_t *d_status, void *stream) {
  return pz_decompress_ex(d_src, comp_bytes, dtype, elem_bits, PZ_CODEC_ALL, 1, d_dst, raw_bytes,
                          d_status, stream);
}

}  // extern "C"
