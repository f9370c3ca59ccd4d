// Device helpers shared by the PlaneZip compress and decompress kernels
// (gfx950, wave64).
//
// Codec: PlaneZip paper, §III-A and Fig. 2 (128-byte blocks of N w-bit
// symbols; ZVC, DBX, BX, ZBX and raw candidates; BPC's plane prefix code;
// 4 KB chunks with 16-bit headers). Bit layout: FORMAT.md version 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define PZ_DEV __device__ __forceinline__

namespace pz {

constexpr int kBlockBytes = 128;
constexpr int kChunkBytes = 4096;
constexpr int kBlocksPerChunk = 32;
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kGroupThreads = kWave * kWavesPerGroup;

// Candidate tags (Fig. 2 order).
constexpr int kZVC = 0, kDBX = 1, kBX = 2, kZBX = 3, kRAW = 4;

// Per-wave LDS: two chunk buffers of kChunkBufDwords, or 64 per-lane regions
// of kLaneStride dwords (stride 33 keeps lane-strided reads conflict free).
constexpr int kChunkBufDwords = 1032;
constexpr int kLaneStride = 33;
constexpr int kWaveLdsDwords = 2 * kChunkBufDwords > kWave * kLaneStride
                                   ? 2 * kChunkBufDwords
                                   : kWave * kLaneStride;

// Look-back status words: a flag in the top two bits, then the epoch of the
// call that wrote the word (22 bits), then the value (40 bits: streams of up
// to 1 TiB). A word of another epoch reads as not ready, so the words that a
// reused scratch buffer keeps from earlier calls need no clearing.
constexpr uint64_t kFlagAggregate = 1ull << 62;
constexpr uint64_t kFlagPrefix = 2ull << 62;
constexpr int kEpochShift = 40;
constexpr uint64_t kEpochBits = (1ull << 22) - 1;
constexpr uint64_t kValueMask = (1ull << kEpochShift) - 1;
constexpr uint32_t kEpochMax = (uint32_t)kEpochBits;

constexpr uint64_t kBadChunk = ~0ull;

// A tile's look-back word sits alone in its 64-byte line (tile t at word
// t * kLookbackStride): each word is read at device scope by the hundreds of
// successors whose walks pass it, and words sharing a line share those
// reads' queue (8 words per line measured 4% slower compression).
constexpr uint64_t kLookbackStride = 8;

// Codec mode (§III-A; the single-codec columns of §V-A and Table III):
// the candidates a block may use (bit t = tag t) and whether each block
// carries the 3-bit tag. PlaneZip itself is {all five, tagged}; an untagged
// mode has exactly one candidate and writes no tags. In every mode a chunk
// that does not shrink is kept raw.
constexpr uint32_t kAllCodecs = 0x1Fu;
struct Mode {
  uint32_t mask;    // allowed candidates
  uint32_t tagged;  // 1: a 3-bit tag per block
  uint32_t fixed;   // the candidate of an untagged mode
  uint32_t zc;      // the candidate this mode picks for an all-zero block
};

// Size in bits (payload, no tag) of an all-zero block under candidate c: a
// zero mask for ZVC and ZBX, a zero base for DBX, all planes in one zero run
// for the plane encodings (W planes, W+1 for DBX), 1024 bits for RAW.
__host__ __device__ inline uint32_t zero_block_size(int W, uint32_t c) {
  const uint32_t N = 1024u / W, R = W == 16 ? 4u : 5u;
  switch (c) {
    case 0: return N;
    case 1: return W + 2 + R;
    case 2: return 2 + R;
    case 3: return N + 2 + R;
    default: return 1024;
  }
}

// The mode for (mask, tagged): the all-zero block's candidate is the
// smallest allowed one, ties to the lowest tag, as for any block.
__host__ __device__ inline Mode make_mode(int W, uint32_t mask, int tagged) {
  Mode m{mask, tagged ? 1u : 0u, 0u, 0u};
  uint32_t best = 0xFFFFFFFFu;
  for (uint32_t t = 0; t < 5; ++t) {
    if (!((mask >> t) & 1u)) continue;
    if (!tagged) m.fixed = t;
    const uint32_t z = zero_block_size(W, t);
    if (z < best) {
      best = z;
      m.zc = t;
    }
  }
  return m;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

PZ_DEV uint32_t pk_sub_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) - __builtin_bit_cast(u16x2, b));
}
PZ_DEV uint32_t pk_add_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) + __builtin_bit_cast(u16x2, b));
}
// One v_pk_min_u16. (Written as an elementwise min, a min with 1 is turned
// into two 16-bit compares, two selects and a byte permute per call.)
PZ_DEV uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

PZ_DEV uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t shift) {
  // Low 32 bits of ((hi:lo) >> shift), shift in [0, 31].
  return __builtin_amdgcn_alignbit(hi, lo, shift);
}

PZ_DEV int popc64(uint64_t x) { return __popcll(x); }
PZ_DEV int popc32(uint32_t x) { return __popc(x); }

PZ_DEV uint32_t lane_id() { return __lane_id(); }

// Number of set bits of a wave mask below this lane.
PZ_DEV uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Integer minimum of two 64-bit values (HIP's templated min goes through
// floating point for 64-bit integers).
__host__ __device__ inline uint64_t min_u64(uint64_t a, uint64_t b) { return a < b ? a : b; }

PZ_DEV uint64_t all_ones64(int L) { return L >= 64 ? ~0ull : ((1ull << L) - 1ull); }

// ceil(log2 L) for L >= 2, else 0: width of the position field.
PZ_DEV int position_bits(int L) { return L >= 2 ? 32 - __clz(L - 1) : 0; }

// ---------------------------------------------------------------------------
// 32x32 bit-matrix transpose in registers: afterwards a[c] bit r equals the
// old a[r] bit c. Five butterfly stages: byte permutes for the 16- and 8-bit
// stages, a shift and a bitwise select per output for the others.
// ---------------------------------------------------------------------------
// Bitwise m ? a : b as one v_bitop3_b32 (the function's truth table over
// m = 0xF0, a = 0xCC, b = 0xAA). Written with & | ~, the stages below took
// six instructions per pair of outputs instead of four.
PZ_DEV uint32_t bit_select(uint32_t m, uint32_t a, uint32_t b) {
  return __builtin_amdgcn_bitop3_b32(m, a, b, 0xCA);
}

template <int J>
PZ_DEV void transpose_stage(uint32_t (&a)[32], uint32_t m) {
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if (k & J) continue;
    const uint32_t x = a[k], y = a[k + J];
    a[k] = bit_select(m, x, y << J);
    a[k + J] = bit_select(m, x >> J, y);
  }
}

// The byte stages as one byte permute per output (left to the compiler, the
// 8-bit stage became two to four instructions per output).
template <int J>
PZ_DEV void transpose_bytes(uint32_t (&a)[32], uint32_t sel_lo, uint32_t sel_hi) {
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if (k & J) continue;
    const uint32_t x = a[k], y = a[k + J];
    a[k] = __builtin_amdgcn_perm(y, x, sel_lo);
    a[k + J] = __builtin_amdgcn_perm(y, x, sel_hi);
  }
}

PZ_DEV void transpose32(uint32_t (&a)[32]) {
  // Selector byte i names the source byte of output byte i: 0..3 are x's
  // bytes, 4..7 y's. 16-bit stage: (x.lo, y.lo) and (x.hi, y.hi); 8-bit
  // stage: (x.b0, y.b0, x.b2, y.b2) and (x.b1, y.b1, x.b3, y.b3).
  transpose_bytes<16>(a, 0x05040100u, 0x07060302u);
  transpose_bytes<8>(a, 0x06020400u, 0x07030501u);
  transpose_stage<4>(a, 0x0F0F0F0Fu);
  transpose_stage<2>(a, 0x33333333u);
  transpose_stage<1>(a, 0x55555555u);
}

// ---------------------------------------------------------------------------
// Wave-wide helpers.
// ---------------------------------------------------------------------------
PZ_DEV uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Inclusive scan of a 32-bit value within each 32-lane half of the wave.
PZ_DEV uint32_t half_inclusive_scan(uint32_t v) {
  const uint32_t l = lane_id() & 31;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    uint32_t t = __shfl_up(v, off, 32);
    if (l >= (uint32_t)off) v += t;
  }
  return v;
}

PZ_DEV uint64_t wave_inclusive_scan_u64(uint64_t v) {
  const uint32_t l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint64_t t = __shfl_up(v, off, 64);
    if (l >= (uint32_t)off) v += t;
  }
  return v;
}

PZ_DEV uint64_t atomic_load_agent(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
PZ_DEV void atomic_store_agent(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Next tile index for this wave, from a device-wide counter, so that every
// tile a wave waits on in the look-back belongs to a wave that is already
// running (tiles are handed out in the order waves start).
PZ_DEV uint32_t acquire_tile(uint32_t *counter) {
  uint32_t t = 0;
  if (lane_id() == 0) t = atomicAdd(counter, 1u);
  return __shfl(t, 0, 64);
}

// Decoupled look-back (Merrill & Garland, "Single-pass Parallel Prefix Scan
// with Decoupled Look-back"), in two halves so that a tile can do other work
// between them. lookback_publish makes this tile's aggregate visible (tile 0
// publishes its inclusive prefix); lookback_resolve walks back over the
// predecessors 64 at a time until it meets an inclusive prefix, publishes this
// tile's inclusive prefix and returns the exclusive prefix of `agg`.
PZ_DEV void lookback_publish(uint64_t *status, uint32_t tile, uint64_t agg, uint32_t epoch) {
  if (lane_id() == 0)
    atomic_store_agent(&status[(uint64_t)tile * kLookbackStride],
                       (tile == 0 ? kFlagPrefix : kFlagAggregate) | ((uint64_t)epoch << kEpochShift) | agg);
}

PZ_DEV uint64_t lookback_resolve(uint64_t *status, uint32_t tile, uint64_t agg, uint32_t epoch) {
  if (tile == 0) return 0;
  const uint32_t lane = lane_id();
  const uint64_t stamp = (uint64_t)epoch << kEpochShift;
  uint64_t excl = 0;
  int64_t base = (int64_t)tile - 1;
  while (true) {
    const int64_t idx = base - (int64_t)lane;
    const uint64_t st = idx >= 0 ? atomic_load_agent(&status[(uint64_t)idx * kLookbackStride]) : (kFlagPrefix | stamp);
    const bool current = ((st >> kEpochShift) & kEpochBits) == epoch;
    const uint64_t flag = current ? st >> 62 : 0;
    const uint64_t not_ready = __ballot(flag == 0);
    const uint64_t prefix = __ballot(flag == 2);
    const uint64_t first = prefix & (~prefix + 1);         // nearest inclusive prefix
    const uint64_t need = prefix ? (first << 1) - 1 : ~0ull;  // lanes up to it
    if (not_ready & need) {
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    const uint64_t mine = ((need >> lane) & 1ull) ? (st & kValueMask) : 0;
    excl += wave_sum_u64(mine);
    if (prefix) break;
    base -= 64;
  }
  if (lane == 0) atomic_store_agent(&status[(uint64_t)tile * kLookbackStride], kFlagPrefix | stamp | (excl + agg));
  return excl;
}

PZ_DEV uint64_t lookback(uint64_t *status, uint32_t tile, uint64_t agg, uint32_t epoch) {
  lookback_publish(status, tile, agg, epoch);
  return lookback_resolve(status, tile, agg, epoch);
}

// Orders this wave's LDS accesses before and after (all lanes of a wave run
// the same instruction stream; this keeps the compiler from moving LDS
// accesses across phases that hand data between lanes).
PZ_DEV void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// Plane-code size from per-plane class masks (bit j describes plane j):
// nz: XORed plane non-zero; ones: XORed plane all ones; pz: plane before the
// XOR is zero; pair: exactly two adjacent ones; single: exactly one one.
// Codes of §III-A: a lone zero plane 3 bits, a run of zero planes 2+R bits,
// all-ones and pre-XOR-zero planes 5 bits, pair and single 5 + PW bits, any
// other plane 1 + L bits; the first matching class wins, in that order.
// ---------------------------------------------------------------------------
PZ_DEV int plane_code_bits(uint64_t nz, uint64_t ones, uint64_t pz, uint64_t pair,
                           uint64_t single, int K, int L, int R) {
  const uint64_t kmask = (K >= 64) ? ~0ull : ((1ull << K) - 1ull);
  nz &= kmask;
  const uint64_t a = nz & ones;
  const uint64_t b = nz & ~a & pz;
  const uint64_t rest = nz & ~a & ~b;
  const uint64_t cd = rest & (pair | single);
  const uint64_t e = rest & ~cd;
  const uint64_t z = ~nz & kmask;
  const uint64_t starts = z & ~(z >> 1);
  const uint64_t lone = starts & ~(z << 1);
  const int runs = popc64(starts), lones = popc64(lone);
  const int pw = position_bits(L);
  return 5 * popc64(a | b) + (5 + pw) * popc64(cd) + (1 + L) * popc64(e) + 3 * lones +
         (2 + R) * (runs - lones);
}

}  // namespace pz
