// PlaneZip decompression on gfx950.
//
// Method: PlaneZip paper, §III-A "Stream format": a prefix sum over the
// 16-bit chunk headers locates every chunk, so chunks decode in parallel; the
// decoder reproduces every block exactly (§III-A "Validation"). Bit layout and
// decoder checks: FORMAT.md version 1, §5 and §6.
//
// A chunk's blocks carry no offsets, so the blocks of one chunk must be
// parsed in order. The work is split in two kernels:
//   locate: one lane per chunk. Scans the headers (decoupled look-back across
//           waves), validates them, and walks each chunk's codes without
//           decoding them to record the bit offset of every block.
//   decode: one lane per block. The wave stages its two chunks' payloads in
//           LDS with coalesced loads, then every lane decodes its block from
//           its known bit offset: codes -> XORed planes -> planes -> inverse
//           32x32 bit transpose -> symbols (delta prefix sum for DBX, scatter
//           by the zero mask for ZVC/ZBX), and stores 128 bytes.
#include <type_traits>

#include "pz_device.h"
#include "pz_launch.h"

namespace pz {

constexpr int32_t kStatusCorrupt = 3;

// Bits of the stream in global memory, read through dword loads that never
// touch a byte at or past `limit`.
struct GlobalBits {
  const uint8_t *src;
  uint64_t limit;     // comp_bytes
  uint64_t base_bit;  // bit offset of the chunk payload in the stream

  PZ_DEV uint32_t dword(uint64_t q) const {
    const uint64_t b = q * 4;
    if (b + 4 <= limit) return *reinterpret_cast<const uint32_t *>(src + b);
    uint32_t v = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (b + k < limit) v |= (uint32_t)src[b + k] << (8 * k);
    return v;
  }
  // 32 stream bits starting at payload bit `pos`; bit 0 is the first.
  PZ_DEV uint32_t peek(uint32_t pos) const {
    const uint64_t a = base_bit + pos;
    const uint64_t q = a >> 5;
    return funnel(dword(q + 1), dword(q), (uint32_t)(a & 31));
  }
};

// Walks the codes of one coded chunk, recording each block's bit offset.
// Returns false when the chunk fails a decoder check (FORMAT.md §6).
template <int W>
PZ_DEV bool parse_chunk(const GlobalBits &in, uint32_t H, uint32_t raw_len, uint16_t *boff) {
  constexpr int N = 1024 / W;
  constexpr int R = W == 16 ? 4 : 5;
  const uint32_t end = H * 8;
  const int nb = (int)((raw_len + kBlockBytes - 1) / kBlockBytes);
  uint32_t pos = 0;
  for (int b = 0; b < nb; ++b) {
    boff[b] = (uint16_t)pos;
    const uint32_t tag = in.peek(pos) & 7u;
    pos += 3;
    if (tag > 4) return false;
    int K = 0, L = 0;
    if (tag == kRAW) {
      pos += 1024;
    } else if (tag == kZVC || tag == kZBX) {
      int n = popc32(in.peek(pos));
      if (W == 16) n += popc32(in.peek(pos + 32));
      pos += N;
      if (tag == kZVC) {
        pos += (uint32_t)(W * n);
      } else {
        K = W;
        L = n;
      }
    } else if (tag == kDBX) {
      pos += W;
      K = W + 1;
      L = N - 1;
    } else {
      K = W;
      L = N;
    }
    if (K) {
      const uint32_t pw = (uint32_t)position_bits(L);
      int left = K;
      while (left > 0) {
        const uint32_t win = in.peek(pos);
        const uint32_t tz = win ? (uint32_t)__builtin_ctz(win) : 32u;
        if (tz == 0) {
          pos += 1 + (uint32_t)L;
          --left;
        } else if (tz == 1) {
          const int k = (int)((win >> 2) & ((1u << R) - 1u)) + 2;
          if (k > left) return false;
          pos += 2 + R;
          left -= k;
        } else if (tz == 2) {
          pos += 3;
          --left;
        } else if (tz == 3) {
          const int p = (int)((win >> 5) & ((1u << pw) - 1u));
          const bool single = (win >> 4) & 1u;
          if (p > L - (single ? 1 : 2)) return false;
          pos += 5 + pw;
          --left;
        } else {
          pos += 5;
          --left;
        }
      }
    }
    if (pos > end) return false;
  }
  if ((pos + 7) / 8 != H) return false;
  if (pos & 7u) {
    const uint32_t rest = in.peek(pos) & ((1u << (8 - (pos & 7u))) - 1u);
    if (rest) return false;
  }
  return true;
}

template <int W>
__global__ __launch_bounds__(kGroupThreads) void locate_kernel(
    const uint8_t *__restrict__ src, uint64_t comp_bytes, uint64_t raw_bytes, uint64_t nchunks,
    uint64_t ntiles, uint64_t *__restrict__ chunk_off, uint16_t *__restrict__ block_off,
    int32_t *status_out, uint64_t *lb_status, uint32_t *tile_counter) {
  const uint32_t lane = lane_id();
  const uint32_t tile = acquire_tile(tile_counter);
  if (tile >= ntiles) return;
  const uint64_t c = (uint64_t)tile * kWave + lane;
  const uint32_t H = c < nchunks ? reinterpret_cast<const uint16_t *>(src)[c] : 0u;
  const uint64_t agg = wave_sum_u64(H);
  const uint64_t before = lookback(lb_status, tile, agg);
  const uint64_t excl = wave_inclusive_scan_u64(H) - H;
  const uint64_t off = 2 * nchunks + before + excl;
  bool bad = false;
  if (tile == ntiles - 1 && lane == 0 && 2 * nchunks + before + agg != comp_bytes) bad = true;
  if (c < nchunks) {
    const uint32_t raw_len = (uint32_t)min<uint64_t>(kChunkBytes, raw_bytes - c * kChunkBytes);
    bool chunk_bad = H > raw_len || off + H > comp_bytes;
    if (!chunk_bad && H < raw_len) {
      GlobalBits in{src, comp_bytes, off * 8};
      chunk_bad = !parse_chunk<W>(in, H, raw_len, block_off + c * kBlocksPerChunk);
    }
    chunk_off[c] = chunk_bad ? kBadChunk : off;
    bad |= chunk_bad;
  }
  if (bad) *status_out = kStatusCorrupt;
}

// Bits of a chunk payload staged in LDS; bit `pos` of the payload is bit
// (lead + pos) of the buffer.
struct LdsBits {
  const uint32_t *buf;
  uint32_t lead;

  PZ_DEV uint32_t peek(uint32_t pos) const {
    uint32_t a = lead + pos;
    uint32_t q = a >> 5;
    q = q > (uint32_t)kChunkBufDwords - 2 ? (uint32_t)kChunkBufDwords - 2 : q;
    return funnel(buf[q + 1], buf[q], a & 31u);
  }
  PZ_DEV uint64_t peek64(uint32_t pos) const {
    return (uint64_t)peek(pos) | ((uint64_t)peek(pos + 32) << 32);
  }
};

// Reads the plane code of K <= KMAX planes (top plane first) into P[0..K-1];
// planes at or above K are zero.
template <typename PT, int KMAX>
PZ_DEV void read_plane_code(const LdsBits &in, uint32_t &pos, PT (&P)[KMAX], int K, int L, int R,
                            bool active) {
  const uint32_t pw = (uint32_t)position_bits(L);
  const PT ones = (PT)all_ones64(L);
  const uint32_t rmask = (1u << R) - 1u;
  PT above = 0;
  uint32_t run = 0;
#pragma unroll
  for (int j = KMAX - 1; j >= 0; --j) {
    const bool live = active && j < K;
    PT x = 0;
    if (live) {
      if (run) {
        --run;
      } else {
        const uint32_t win = in.peek(pos);
        const uint32_t tz = win ? (uint32_t)__builtin_ctz(win) : 32u;
        if (tz == 0) {
          if constexpr (sizeof(PT) == 8)
            x = (PT)in.peek64(pos + 1) & ones;
          else
            x = (PT)in.peek(pos + 1) & ones;
          pos += 1 + (uint32_t)L;
        } else if (tz == 1) {
          run = ((win >> 2) & rmask) + 1u;
          pos += 2 + (uint32_t)R;
        } else if (tz == 2) {
          pos += 3;
        } else if (tz == 3) {
          const uint32_t p = (win >> 5) & ((1u << pw) - 1u);
          x = (((win >> 4) & 1u) ? (PT)1 : (PT)3) << p;
          pos += 5 + pw;
        } else if (tz == 4) {
          x = above;  // the plane before the XOR is zero
          pos += 5;
        } else {
          x = ones;
          pos += 5;
        }
      }
    }
    const PT p = x ^ above;
    P[j] = live ? p : (PT)0;
    if (live) above = p;
  }
}

// Inverse of the w = 16 plane construction: 16 planes of 64 bits to packed
// symbols d[i] = sym 2i | sym 2i+1 << 16.
PZ_DEV void symbols_from_planes16(const uint64_t (&P)[17], uint32_t (&d)[32]) {
  uint32_t e[32];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    e[j] = (uint32_t)P[j];
    e[j + 16] = (uint32_t)(P[j] >> 32);
  }
  transpose32(e);  // e[r] = sym r | sym r+32 << 16
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if (i < 16)
      d[i] = (e[2 * i] & 0xFFFFu) | (e[2 * i + 1] << 16);
    else
      d[i] = (e[2 * i - 32] >> 16) | (e[2 * i - 31] & 0xFFFF0000u);
  }
}

template <int W>
__global__ __launch_bounds__(kGroupThreads) void decode_kernel(
    const uint8_t *__restrict__ src, uint64_t comp_bytes, uint64_t raw_bytes, uint64_t nchunks,
    const uint64_t *__restrict__ chunk_off, const uint16_t *__restrict__ block_off,
    uint8_t *__restrict__ dst) {
  constexpr int N = 1024 / W;
  constexpr int R = W == 16 ? 4 : 5;
  constexpr int KMAX = W + 1;
  constexpr uint32_t WMASK = W == 16 ? 0xFFFFu : 0xFFFFFFFFu;
  using PT = typename std::conditional<W == 16, uint64_t, uint32_t>::type;
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[kWavesPerGroup * kWaveLdsDwords];
  uint32_t *lds = lds_all + (threadIdx.x >> 6) * kWaveLdsDwords;

  const uint32_t lane = lane_id();
  const uint64_t tile = (uint64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  if (tile * 2 >= nchunks) return;
  const uint32_t half = lane >> 5;
  const uint64_t block = tile * kWave + lane;
  const uint64_t chunk = block >> 5;
  const uint64_t off = block * kBlockBytes;
  const bool valid = off < raw_bytes;

  // Stage both chunk payloads (dword-aligned copies) in LDS.
  const uint16_t *hdr = reinterpret_cast<const uint16_t *>(src);
  uint64_t my_off = kBadChunk;
  uint32_t my_H = 0, my_raw = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint64_t c = tile * 2 + h;
    uint64_t coff = kBadChunk;
    uint32_t H = 0;
    if (c < nchunks) {
      coff = chunk_off[c];
      H = hdr[c];
    }
    if (half == (uint32_t)h) {
      my_off = coff;
      my_H = H;
      my_raw = c < nchunks ? (uint32_t)min<uint64_t>(kChunkBytes, raw_bytes - c * kChunkBytes) : 0u;
    }
    if (coff == kBadChunk) continue;
    const uint32_t sh = (uint32_t)(coff & 3);
    const uint64_t q0 = coff >> 2;
    const uint32_t ndw = (sh + H + 3) / 4;
    uint32_t *buf = lds + h * kChunkBufDwords;
    GlobalBits g{src, comp_bytes, 0};
    for (uint32_t i = lane; i < (uint32_t)kChunkBufDwords; i += kWave) buf[i] = i < ndw ? g.dword(q0 + i) : 0u;
  }
  wave_lds_fence();

  const bool ok = valid && my_off != kBadChunk;
  const bool raw_chunk = ok && my_H == my_raw;
  const bool coded = ok && !raw_chunk;
  LdsBits in{lds + half * kChunkBufDwords, 8u * (uint32_t)(my_off & 3)};

  uint32_t pos = 0;
  uint32_t tag = 0;
  if (raw_chunk) pos = 1024u * (lane & 31);
  if (coded) {
    pos = block_off[block];
    tag = in.peek(pos) & 7u;
    pos += 3;
  }

  uint32_t d[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) d[i] = 0;

  const bool want_raw = raw_chunk || (coded && tag == kRAW);
  if (__ballot(want_raw)) {
    if (want_raw) {
#pragma unroll
      for (int i = 0; i < 32; ++i) d[i] = in.peek(pos + 32 * i);
    }
  }

  // Zero mask of ZVC and ZBX.
  const bool want_zvc = coded && tag == kZVC;
  const bool want_zbx = coded && tag == kZBX;
  uint64_t nzmask = 0;
  if (want_zvc || want_zbx) {
    nzmask = W == 16 ? in.peek64(pos) : (uint64_t)in.peek(pos);
    pos += N;
  }
  if (__ballot(want_zvc)) {
    if (want_zvc) {
#pragma unroll
      for (int k = 0; k < N; ++k) {
        if ((nzmask >> k) & 1u) {
          const uint32_t v = in.peek(pos) & WMASK;
          pos += W;
          if constexpr (W == 16)
            d[k >> 1] |= v << (16 * (k & 1));
          else
            d[k] = v;
        }
      }
    }
  }

  const bool want_dbx = coded && tag == kDBX;
  const bool want_planes = coded && (tag == kDBX || tag == kBX || tag == kZBX);
  if (__ballot(want_planes)) {
    uint32_t base = 0;
    if (want_dbx) {
      base = in.peek(pos) & WMASK;
      pos += W;
    }
    int K = W, L = N;
    if (want_dbx) {
      K = W + 1;
      L = N - 1;
    } else if (want_zbx) {
      L = popc64(nzmask);
    }
    PT P[KMAX];
    read_plane_code<PT, KMAX>(in, pos, P, K, L, R, want_planes);
    if (want_dbx) {
      // Plane element k-1 is delta k: move delta k to bit k (delta 0 := 0).
#pragma unroll
      for (int j = 0; j < W; ++j) P[j] <<= 1;
    }
    uint32_t e[32];
    if constexpr (W == 16) {
      symbols_from_planes16(P, e);
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) e[j] = P[j];
      transpose32(e);
    }
    // DBX: running sum of the deltas from the base symbol, modulo 2^w.
    if (want_dbx) {
      if constexpr (W == 16) {
        uint32_t carry = base;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t v = e[i];
          const uint32_t pair = v + (v << 16);  // (lo, lo + hi)
          const uint32_t outv = pk_add_u16(pair, carry | (carry << 16));
          e[i] = outv;
          carry = outv >> 16;
        }
      } else {
        uint32_t acc = base;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          acc += e[i];
          e[i] = acc;
        }
      }
    }
    if (want_planes && !want_zbx) {
#pragma unroll
      for (int i = 0; i < 32; ++i) d[i] = e[i];
    }
    // ZBX: the compacted symbols go back to the non-zero positions.
    if (__ballot(want_zbx)) {
      wave_lds_fence();  // all lanes are done reading the staged payloads
      uint32_t *region = lds + lane * kLaneStride;
      if (want_zbx) {
#pragma unroll
        for (int i = 0; i < 32; ++i) region[i] = e[i];
      }
      wave_lds_fence();
      if (want_zbx) {
        uint32_t rank = 0;
        if constexpr (W == 16) {
          const uint16_t *r16 = reinterpret_cast<const uint16_t *>(region);
#pragma unroll
          for (int k = 0; k < 64; ++k) {
            if ((nzmask >> k) & 1u) {
              d[k >> 1] |= (uint32_t)r16[rank] << (16 * (k & 1));
              ++rank;
            }
          }
        } else {
#pragma unroll
          for (int k = 0; k < 32; ++k) {
            if ((nzmask >> k) & 1u) {
              d[k] = region[rank];
              ++rank;
            }
          }
        }
      }
    }
  }

  // Store the block (the tail block only up to raw_bytes).
  if (ok) {
    if (off + kBlockBytes <= raw_bytes) {
      uint4 *p = reinterpret_cast<uint4 *>(dst + off);
#pragma unroll
      for (int q = 0; q < 8; ++q) p[q] = make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);
    } else {
      const uint32_t n = (uint32_t)(raw_bytes - off);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t k = 4 * i + b;
          if (k < n) dst[off + k] = (uint8_t)(d[i] >> (8 * b));
        }
      }
    }
  }
}

__global__ void fill_u32_kernel(uint32_t *p, uint64_t n, uint32_t value) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

hipError_t fill_u32(uint32_t *p, uint64_t n, uint32_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const uint64_t groups = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)groups), dim3(256), 0, stream, p, n, value);
  return hipGetLastError();
}

hipError_t launch_decompress(int w, const uint8_t *src, uint64_t comp_bytes, uint8_t *dst,
                             uint64_t raw_bytes, int32_t *status, hipStream_t stream) {
  const uint64_t nchunks = (raw_bytes + kChunkBytes - 1) / kChunkBytes;
  const uint64_t ntiles_a = (nchunks + kWave - 1) / kWave;
  // Scratch (8-byte words): chunk offsets, block offsets, look-back status,
  // tile counter, and a status word when the caller passes none.
  const uint64_t w_off = nchunks;
  const uint64_t w_boff = (nchunks * kBlocksPerChunk * 2 + 7) / 8;
  const uint64_t w_lb = ntiles_a;
  const size_t words = (size_t)(w_off + w_boff + w_lb + 2);
  uint64_t *scratch = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void **>(&scratch), words * sizeof(uint64_t), stream);
  if (e != hipSuccess) return e;
  uint64_t *chunk_off = scratch;
  uint16_t *block_off = reinterpret_cast<uint16_t *>(scratch + w_off);
  uint64_t *lb_status = scratch + w_off + w_boff;
  uint32_t *counter = reinterpret_cast<uint32_t *>(lb_status + w_lb);
  int32_t *own_status = reinterpret_cast<int32_t *>(lb_status + w_lb + 1);
  int32_t *st = status ? status : own_status;

  e = fill_u64(lb_status, w_lb + 1, 0, stream);
  if (e == hipSuccess) e = fill_u32(reinterpret_cast<uint32_t *>(st), 1, 0u, stream);
  if (e == hipSuccess && nchunks == 0) {
    if (comp_bytes != 0) e = fill_u32(reinterpret_cast<uint32_t *>(st), 1, (uint32_t)kStatusCorrupt, stream);
  } else if (e == hipSuccess) {
    const uint64_t groups_a = (ntiles_a + kWavesPerGroup - 1) / kWavesPerGroup;
    if (w == 16)
      hipLaunchKernelGGL(locate_kernel<16>, dim3((unsigned)groups_a), dim3(kGroupThreads), 0, stream,
                         src, comp_bytes, raw_bytes, nchunks, ntiles_a, chunk_off, block_off, st,
                         lb_status, counter);
    else
      hipLaunchKernelGGL(locate_kernel<32>, dim3((unsigned)groups_a), dim3(kGroupThreads), 0, stream,
                         src, comp_bytes, raw_bytes, nchunks, ntiles_a, chunk_off, block_off, st,
                         lb_status, counter);
    e = hipGetLastError();
    if (e == hipSuccess) {
      const uint64_t ntiles_b = (nchunks + 1) / 2;
      const uint64_t groups_b = (ntiles_b + kWavesPerGroup - 1) / kWavesPerGroup;
      if (w == 16)
        hipLaunchKernelGGL(decode_kernel<16>, dim3((unsigned)groups_b), dim3(kGroupThreads), 0,
                           stream, src, comp_bytes, raw_bytes, nchunks, chunk_off, block_off, dst);
      else
        hipLaunchKernelGGL(decode_kernel<32>, dim3((unsigned)groups_b), dim3(kGroupThreads), 0,
                           stream, src, comp_bytes, raw_bytes, nchunks, chunk_off, block_off, dst);
      e = hipGetLastError();
    }
  }
  hipError_t f = hipFreeAsync(scratch, stream);
  return e != hipSuccess ? e : f;
}

}  // namespace pz
