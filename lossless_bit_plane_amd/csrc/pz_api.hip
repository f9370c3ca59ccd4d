// C ABI of the PlaneZip codec: argument checks and dispatch to the HIP
// kernels. Declarations and the meaning of every argument: include/planezip.h.
#include "../../include/planezip.h"

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "pz_device.h"
#include "pz_launch.h"

namespace {

// Symbol width w for (dtype, elem_bits), or -1. PlaneZip paper §III-A: BF16
// uses 16-bit symbols, FP32 and all other element types 32-bit ones; BF16 may
// also be coded as 32-bit symbols (BPC's own width, §V-A).
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
// when the epoch wraps. Buffer layout: the tile counter and the error words
// of a launch's tensors (48 bytes), the look-back words, the per-call bytes.
// ---------------------------------------------------------------------------
struct ScratchEntry {
  int device;
  hipStream_t stream;
  uint8_t *base;
  size_t words;       // look-back words held
  size_t extra;       // per-call bytes held
  uint32_t epoch;     // of the last call
  uint32_t counter;   // tile counter after the last call
  uint32_t done;      // located-tile count after the last call
  bool clear;         // the header and words must be cleared before the next call
};

constexpr size_t kScratchHeader = 48;
static_assert(4 + 4 * pz::kMaxBatch + 4 <= kScratchHeader, "counter, error words and located-tile count");

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
    g_scratch.push_back(ScratchEntry{device, stream, nullptr, 0, 0, 0, 0, 0, true});
    ent = &g_scratch.back();
  }
  if (ent->words < need.words || ent->extra < need.extra || !ent->base) {
    // An even word count keeps the per-call bytes 16-byte aligned (locate
    // stores block offsets in 16-byte units).
    const size_t words = need.words > ent->words ? (need.words + need.words / 4 + 64 + 1) & ~size_t(1) : ent->words;
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
    ent->done = 0;
    ent->clear = false;
  }
  pz::Scratch sc;
  sc.counter = reinterpret_cast<uint32_t *>(ent->base);
  sc.err = reinterpret_cast<uint32_t *>(ent->base) + 1;
  sc.done = reinterpret_cast<uint32_t *>(ent->base) + 1 + pz::kMaxBatch;
  sc.words = reinterpret_cast<uint64_t *>(ent->base + kScratchHeader);
  sc.extra = ent->base + kScratchHeader + 8 * ent->words;
  sc.epoch = ++ent->epoch;
  sc.counter_base = ent->counter;
  sc.done_base = ent->done;
  e = launch(sc);
  if (e == hipSuccess) {
    ent->counter += need.counted;  // every workgroup of the call takes one tile
    ent->done += need.done;
  } else {
    ent->clear = true;
  }
  return e;
}

// The scratch cache identifies a stream by its handle, and its look-back
// epochs and tile-counter bases are host values fixed when a call is
// enqueued. So it serves only streams whose calls the stream itself orders
// and that run once as enqueued: not hipStreamPerThread (one handle, a
// different stream in every host thread), and not a stream under graph
// capture (a replay would reuse the captured epoch and counter base).
pz_status_t check_stream(hipStream_t s) {
  if (s == hipStreamPerThread) return PZ_ERROR_INVALID_VALUE;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return PZ_ERROR_HIP;
  return cs == hipStreamCaptureStatusNone ? PZ_SUCCESS : PZ_ERROR_INVALID_VALUE;
}

// Compress calls: every tensor is checked first (nothing is enqueued if one
// fails); then tensors with chunks go out in launches of up to kMaxBatch,
// and an empty tensor's size is set to 0.
pz_status_t compress_many(int dtype, int elem_bits, uint32_t codec_mask, int tagged, int count,
                          const void *const *srcs, const size_t *raw, void *const *dsts, const size_t *caps,
                          uint64_t *d_out_bytes, void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || !valid_mode(codec_mask, tagged) || count < 0 || (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u))
    return PZ_ERROR_INVALID_VALUE;
  if (count > 0 && (!srcs || !raw || !dsts || !caps || !d_out_bytes)) return PZ_ERROR_INVALID_VALUE;
  for (int i = 0; i < count; ++i) {
    if ((raw[i] && (!srcs[i] || !dsts[i])) || raw[i] > PZ_MAX_RAW_BYTES) return PZ_ERROR_INVALID_VALUE;
    if (!aligned16(srcs[i]) || !aligned16(dsts[i])) return PZ_ERROR_INVALID_VALUE;
  }
  for (int i = 0; i < count; ++i)
    if (caps[i] < PZ_MAX_COMPRESSED_BYTES(raw[i])) return PZ_ERROR_INSUFFICIENT_BUFFER;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (count > 0) {
    const pz_status_t st = check_stream(s);
    if (st != PZ_SUCCESS) return st;
  }
  int i = 0;
  while (i < count) {
    pz::CBatch b{};
    while (i < count && b.n < (uint32_t)pz::kMaxBatch) {
      if (raw[i] == 0) {
        const hipError_t e = pz::fill_u64(d_out_bytes + i, 1, 0, s);
        if (e != hipSuccess) return from_hip(e);
        ++i;
        continue;
      }
      pz::CTensor &x = b.t[b.n++];
      x.src = static_cast<const uint8_t *>(srcs[i]);
      x.dst = static_cast<uint8_t *>(dsts[i]);
      x.out_bytes = d_out_bytes + i;
      x.raw_bytes = raw[i];
      x.nchunks = PZ_NUM_CHUNKS(raw[i]);
      x.tile_begin = b.total_tiles;
      x.ntiles = pz::compress_tiles(raw[i]);
      b.total_tiles += x.ntiles;
      ++i;
    }
    if (b.n == 0) continue;
    const pz::ScratchNeed need{b.total_tiles * pz::kLookbackStride, 0, b.total_tiles};
    const hipError_t e = with_scratch(s, need, [&](const pz::Scratch &sc) {
      return pz::launch_compress(w, b, codec_mask, tagged, sc, s);
    });
    if (e != hipSuccess) return from_hip(e);
  }
  return PZ_SUCCESS;
}

// Decompress calls, checked and launched as compress_many; an empty tensor
// gets its status from comp_bytes alone. Within a launch the densest streams
// (most stream bytes per raw byte) come first, so that the longest chunk
// walks start first.
pz_status_t decompress_many(int dtype, int elem_bits, uint32_t codec_mask, int tagged, int count,
                            const void *const *srcs, const size_t *comp, void *const *dsts, const size_t *raw,
                            int32_t *d_status, void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || !valid_mode(codec_mask, tagged) || count < 0 || (reinterpret_cast<uintptr_t>(d_status) & 3u))
    return PZ_ERROR_INVALID_VALUE;
  if (count > 0 && (!srcs || !comp || !dsts || !raw)) return PZ_ERROR_INVALID_VALUE;
  for (int i = 0; i < count; ++i) {
    if ((comp[i] && !srcs[i]) || (raw[i] && !dsts[i]) || raw[i] > PZ_MAX_RAW_BYTES) return PZ_ERROR_INVALID_VALUE;
    if (!aligned16(srcs[i]) || !aligned16(dsts[i])) return PZ_ERROR_INVALID_VALUE;
  }
  for (int i = 0; i < count; ++i)
    if (comp[i] < 2 * PZ_NUM_CHUNKS(raw[i])) return PZ_ERROR_CORRUPT_STREAM;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (count > 0) {
    const pz_status_t st = check_stream(s);
    if (st != PZ_SUCCESS) return st;
  }
  int i = 0;
  while (i < count) {
    int idx[pz::kMaxBatch];
    int n = 0;
    while (i < count && n < pz::kMaxBatch) {
      if (raw[i] == 0) {
        const hipError_t e = pz::launch_empty_status(d_status ? d_status + i : nullptr, comp[i], s);
        if (e != hipSuccess) return from_hip(e);
      } else {
        idx[n++] = i;
      }
      ++i;
    }
    if (n == 0) continue;
    // Densest first (insertion sort on comp / raw, compared as products).
    for (int a = 1; a < n; ++a)
      for (int c = a; c > 0; --c) {
        const unsigned __int128 l = (unsigned __int128)comp[idx[c]] * raw[idx[c - 1]];
        const unsigned __int128 r = (unsigned __int128)comp[idx[c - 1]] * raw[idx[c]];
        if (l <= r) break;
        const int tmp = idx[c];
        idx[c] = idx[c - 1];
        idx[c - 1] = tmp;
      }
    pz::DBatch b{};
    size_t extra = 0;
    for (int a = 0; a < n; ++a) {
      const int j = idx[a];
      pz::DTensor &x = b.t[b.n++];
      x.src = static_cast<const uint8_t *>(srcs[j]);
      x.dst = static_cast<uint8_t *>(dsts[j]);
      x.status = d_status ? d_status + j : nullptr;
      x.comp_bytes = comp[j];
      x.raw_bytes = raw[j];
      x.nchunks = PZ_NUM_CHUNKS(raw[j]);
      x.group_begin = b.total_groups;
      x.ngroups = pz::decode_groups(raw[j]);
      b.total_groups += x.ngroups;
      extra += pz::decompress_extra(raw[j]);
    }
    pz::plan_decompress(w, b);
    const pz::ScratchNeed need = pz::decompress_need(b, extra);
    const hipError_t e = with_scratch(s, need, [&](const pz::Scratch &sc) {
      return pz::launch_decompress(w, b, codec_mask, tagged, sc, s);
    });
    if (e != hipSuccess) return from_hip(e);
  }
  return PZ_SUCCESS;
}

// ---------------------------------------------------------------------------
// Compression without allocation (pz_compress_noalloc). Its scratch (the tile
// counter and one look-back word per tile) is a fixed array in device
// memory, one copy per GPU, that lives until the process ends. Host code
// never passes the array's name to a kernel: its name is a host-side stand-in,
// not a device address. The device address comes from hipGetSymbolAddress,
// once per device, on the first call made with that device current, and is
// kept per device.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocWords = 262144;  // 2 MiB: header + look-back words (one per 64-byte line)
constexpr size_t kNoAllocHeaderWords = kScratchHeader / 8;
static __device__ __align__(256) uint64_t scratch[kNoAllocWords];

std::mutex g_noalloc_mu;
uint64_t *g_noalloc_ptr[64];

hipError_t noalloc_scratch(uint64_t **out) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[device]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_noalloc_ptr[device] = static_cast<uint64_t *>(ptr);
  }
  *out = g_noalloc_ptr[device];
  return hipSuccess;
}

}  // namespace

extern "C" {

pz_status_t pz_compress_noalloc(const void *d_src, size_t raw_bytes, int dtype, int elem_bits, void *d_dst,
                                size_t dst_capacity, uint64_t *d_out_bytes, void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || !d_out_bytes || (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u)) return PZ_ERROR_INVALID_VALUE;
  if (raw_bytes && (!d_src || !d_dst)) return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || !aligned16(d_dst)) return PZ_ERROR_INVALID_VALUE;
  if (dst_capacity < PZ_MAX_COMPRESSED_BYTES(raw_bytes)) return PZ_ERROR_INSUFFICIENT_BUFFER;
  if (raw_bytes > PZ_NOALLOC_MAX_BYTES ||
      pz::compress_tiles(raw_bytes) * pz::kLookbackStride > kNoAllocWords - kNoAllocHeaderWords)
    return PZ_ERROR_INVALID_VALUE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (raw_bytes == 0) return from_hip(pz::fill_u64(d_out_bytes, 1, 0, s));
  uint64_t *base = nullptr;
  hipError_t e = noalloc_scratch(&base);
  if (e != hipSuccess) return from_hip(e);
  pz::CBatch b{};
  b.n = 1;
  pz::CTensor &x = b.t[0];
  x.src = static_cast<const uint8_t *>(d_src);
  x.dst = static_cast<uint8_t *>(d_dst);
  x.out_bytes = d_out_bytes;
  x.raw_bytes = raw_bytes;
  x.nchunks = PZ_NUM_CHUNKS(raw_bytes);
  x.tile_begin = 0;
  x.ntiles = pz::compress_tiles(raw_bytes);
  b.total_tiles = x.ntiles;
  // The previous call's counter and look-back words are still there: clear
  // them (a kernel, not a memset) and count this call's tiles from 0 under
  // epoch 1.
  e = pz::fill_u64(base, kNoAllocHeaderWords + (uint64_t)x.ntiles * pz::kLookbackStride, 0, s);
  if (e != hipSuccess) return from_hip(e);
  pz::Scratch sc;
  sc.counter = reinterpret_cast<uint32_t *>(base);
  sc.err = reinterpret_cast<uint32_t *>(base) + 1;
  sc.words = base + kNoAllocHeaderWords;
  sc.extra = nullptr;
  sc.done = nullptr;
  sc.epoch = 1;
  sc.counter_base = 0;
  sc.done_base = 0;
  return from_hip(pz::launch_compress(w, b, PZ_CODEC_ALL, 1, sc, s));
}


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
  if (w < 0 || !valid_mode(codec_mask, tagged) || !d_out_bytes || (raw_bytes && !d_src) ||
      raw_bytes > PZ_MAX_RAW_BYTES)
    return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u) ||
      (reinterpret_cast<uintptr_t>(d_chunk_lens) & 1u))
    return PZ_ERROR_INVALID_VALUE;
  pz::SBatch b{};
  b.n = 1;
  pz::STensor &x = b.t[0];
  x.src = static_cast<const uint8_t *>(d_src);
  x.out_bytes = d_out_bytes;
  x.chunk_lens = d_chunk_lens;
  x.raw_bytes = raw_bytes;
  x.stride = 1;
  pz::size_plan(x);
  b.total_groups = x.ngroups;
  return from_hip(pz::launch_size(w, b, codec_mask, tagged, static_cast<hipStream_t>(stream)));
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
  if (w < 0 || chunk_stride == 0 || !d_sample || (raw_bytes && !d_src) || raw_bytes > PZ_MAX_RAW_BYTES)
    return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || (reinterpret_cast<uintptr_t>(d_sample) & 7u) ||
      (reinterpret_cast<uintptr_t>(d_sample_lens) & 1u))
    return PZ_ERROR_INVALID_VALUE;
  pz::SBatch b{};
  b.n = 1;
  pz::STensor &x = b.t[0];
  x.src = static_cast<const uint8_t *>(d_src);
  x.out_bytes = d_sample;
  x.out_raw = d_sample + 1;
  x.chunk_lens = d_sample_lens;
  x.raw_bytes = raw_bytes;
  x.stride = chunk_stride;
  pz::size_plan(x);
  b.total_groups = x.ngroups;
  return from_hip(pz::launch_size(w, b, PZ_CODEC_ALL, 1, static_cast<hipStream_t>(stream)));
}

pz_status_t pz_compressed_size_batch(int count, const void *const *d_srcs, const size_t *raw_bytes, int dtype,
                                     int elem_bits, uint64_t *d_out_bytes, uint16_t *const *d_chunk_lens,
                                     void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || count < 0 || (reinterpret_cast<uintptr_t>(d_out_bytes) & 7u)) return PZ_ERROR_INVALID_VALUE;
  if (count > 0 && (!d_srcs || !raw_bytes || !d_out_bytes)) return PZ_ERROR_INVALID_VALUE;
  for (int i = 0; i < count; ++i) {
    if ((raw_bytes[i] && !d_srcs[i]) || !aligned16(d_srcs[i]) || raw_bytes[i] > PZ_MAX_RAW_BYTES)
      return PZ_ERROR_INVALID_VALUE;
    if (d_chunk_lens && (reinterpret_cast<uintptr_t>(d_chunk_lens[i]) & 1u)) return PZ_ERROR_INVALID_VALUE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < count;) {
    pz::SBatch b{};
    for (; i < count && b.n < (uint32_t)pz::kMaxBatch; ++i) {
      pz::STensor &x = b.t[b.n++];
      x.src = static_cast<const uint8_t *>(d_srcs[i]);
      x.out_bytes = d_out_bytes + i;
      x.chunk_lens = d_chunk_lens ? d_chunk_lens[i] : nullptr;
      x.raw_bytes = raw_bytes[i];
      x.stride = 1;
      pz::size_plan(x);
      x.group_begin = b.total_groups;
      b.total_groups += x.ngroups;
    }
    const hipError_t e = pz::launch_size(w, b, PZ_CODEC_ALL, 1, s);
    if (e != hipSuccess) return from_hip(e);
  }
  return PZ_SUCCESS;
}

pz_status_t pz_block_sizes(const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                           uint16_t *d_sizes, uint8_t *d_tags, void *stream) {
  const int w = symbol_width(dtype, elem_bits);
  if (w < 0 || (raw_bytes && !d_src) || raw_bytes > PZ_MAX_RAW_BYTES) return PZ_ERROR_INVALID_VALUE;
  if (!aligned16(d_src) || (reinterpret_cast<uintptr_t>(d_sizes) & 1u)) return PZ_ERROR_INVALID_VALUE;
  return from_hip(pz::launch_block_sizes(w, static_cast<const uint8_t *>(d_src), raw_bytes, d_sizes, d_tags,
                                         static_cast<hipStream_t>(stream)));
}

pz_status_t pz_compress_ex(const void *d_src, size_t raw_bytes, int dtype, int elem_bits,
                           uint32_t codec_mask, int tagged, void *d_dst, size_t dst_capacity,
                           uint64_t *d_out_bytes, void *stream) {
  return compress_many(dtype, elem_bits, codec_mask, tagged, 1, &d_src, &raw_bytes, &d_dst, &dst_capacity,
                       d_out_bytes, stream);
}

pz_status_t pz_compress(const void *d_src, size_t raw_bytes, int dtype, int elem_bits, void *d_dst,
                        size_t dst_capacity, uint64_t *d_out_bytes, void *stream) {
  return pz_compress_ex(d_src, raw_bytes, dtype, elem_bits, PZ_CODEC_ALL, 1, d_dst, dst_capacity,
                        d_out_bytes, stream);
}

pz_status_t pz_compress_batch(int count, const void *const *d_srcs, const size_t *raw_bytes, int dtype,
                              int elem_bits, void *const *d_dsts, const size_t *dst_capacities,
                              uint64_t *d_out_bytes, void *stream) {
  return compress_many(dtype, elem_bits, PZ_CODEC_ALL, 1, count, d_srcs, raw_bytes, d_dsts, dst_capacities,
                       d_out_bytes, stream);
}

pz_status_t pz_decompress_ex(const void *d_src, size_t comp_bytes, int dtype, int elem_bits,
                             uint32_t codec_mask, int tagged, void *d_dst, size_t raw_bytes,
                             int32_t *d_status, void *stream) {
  return decompress_many(dtype, elem_bits, codec_mask, tagged, 1, &d_src, &comp_bytes, &d_dst, &raw_bytes,
                         d_status, stream);
}

pz_status_t pz_decompress(const void *d_src, size_t comp_bytes, int dtype, int elem_bits,
                          void *d_dst, size_t raw_bytes, int32_t *d_status, void *stream) {
  return pz_decompress_ex(d_src, comp_bytes, dtype, elem_bits, PZ_CODEC_ALL, 1, d_dst, raw_bytes,
                          d_status, stream);
}

pz_status_t pz_decompress_batch(int count, const void *const *d_srcs, const size_t *comp_bytes, int dtype,
                                int elem_bits, void *const *d_dsts, const size_t *raw_bytes,
                                int32_t *d_status, void *stream) {
  return decompress_many(dtype, elem_bits, PZ_CODEC_ALL, 1, count, d_srcs, comp_bytes, d_dsts, raw_bytes,
                         d_status, stream);
}

}  // extern "C"
