// PlaneZip compression on gfx950.
//
// Method: PlaneZip paper, §III-A "Codec" and "Stream format", Fig. 2. Every
// 128-byte block is read as N symbols of w bits (N = 64 for w = 16, 32 for
// w = 32) and sized under ZVC, DBX, BX, ZBX and raw; the smallest is kept
// under a 3-bit tag; 32 blocks form a chunk with a 16-bit header and a chunk
// that would grow is stored raw. Bit layout: FORMAT.md version 1.
//
// Mapping to the hardware: one lane owns one 128-byte block, so a wave holds
// two 4 KB chunks. A lane sizes the four plane encodings without transposing:
// the XORed planes of BX are the bit-planes of s ^ (s >> 1), so "plane j is
// zero / all ones / holds one 1 / holds two 1s" are OR, AND and saturating
// count reductions over the block's symbols, evaluated bit-parallel on all
// planes at once (two BF16 symbols per 32-bit register). Only the chosen
// encoding is transposed (a 32x32 bit-matrix butterfly in registers) and
// emitted: every code is OR-ed into a per-chunk LDS buffer at its bit offset,
// with no branches on the bit position. Chunk offsets come from a single-pass
// decoupled look-back over per-wave chunk-length sums, so the input is read
// once and the stream written once.
#include <type_traits>

#include "pz_device.h"
#include "pz_launch.h"

namespace pz {

// ---------------------------------------------------------------------------
// Loading a block: 32 little-endian dwords, zero-padded past the tensor end.
// ---------------------------------------------------------------------------
PZ_DEV void load_block(const uint8_t *__restrict__ src, uint64_t raw_bytes, uint64_t off,
                       uint32_t (&d)[32]) {
  if (off + kBlockBytes <= raw_bytes) {
    const uint4 *p = reinterpret_cast<const uint4 *>(src + off);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = p[q];
      d[4 * q + 0] = v.x;
      d[4 * q + 1] = v.y;
      d[4 * q + 2] = v.z;
      d[4 * q + 3] = v.w;
    }
  } else {
    // The tensor's last block: whole dwords, then the 1..3 trailing bytes.
    const uint64_t n = off < raw_bytes ? raw_bytes - off : 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint64_t b = 4 * (uint64_t)i;
      uint32_t v = 0;
      if (b + 4 <= n) {
        v = *reinterpret_cast<const uint32_t *>(src + off + b);
      } else if (b < n) {
        for (uint64_t k = b; k < n; ++k) v |= (uint32_t)src[off + k] << (8 * (k - b));
      }
      d[i] = v;
    }
  }
}

// Makes the compiler treat the block's registers as new values, so that
// expressions of one phase are recomputed in the next instead of being kept
// alive across it (which would double the register footprint).
PZ_DEV void launder_regs(uint32_t (&d)[32]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) asm volatile("" : "+v"(d[i]));
}

PZ_DEV uint32_t lo16(uint32_t x) { return x & 0xFFFFu; }
PZ_DEV uint32_t hi16(uint32_t x) { return x >> 16; }

struct Sizes {
  int sz[5];
  int n;         // non-zero symbols
  uint32_t b0;   // DBX borrow bits (layout: candidate_sizes16 / 32)
  uint32_t b1;
};

// Merges per-half saturating counters (>=1, >=2, >=3 ones) of the two halves.
PZ_DEV void fold_counts16(uint32_t t1, uint32_t t2, uint32_t t3, uint32_t &c1, uint32_t &c2,
                          uint32_t &c3) {
  c1 = lo16(t1) | hi16(t1);
  c2 = lo16(t2) | hi16(t2) | (lo16(t1) & hi16(t1));
  c3 = lo16(t3) | hi16(t3) | (lo16(t2) & hi16(t1)) | (lo16(t1) & hi16(t2));
}

// Number of non-zero symbols of a block (w = 16: two per dword).
template <int W>
PZ_DEV uint32_t count_nonzero(const uint32_t (&d)[32]) {
  if constexpr (W == 16) {
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) cnt = pk_add_u16(cnt, pk_min_u16(d[i], 0x00010001u));
    return lo16(cnt) + hi16(cnt);
  } else {
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) cnt += d[i] != 0 ? 1u : 0u;
    return cnt;
  }
}

// ---------------------------------------------------------------------------
// Candidate sizes, w = 16. d[i] holds symbols 2i (low half) and 2i+1 (high);
// n is the block's number of non-zero symbols. zbx (wave-uniform) is false
// when no lane of the wave holds a block with 0 < n < 64: then ZBX compacts
// nothing away and its size is the mask plus the BX size.
// ---------------------------------------------------------------------------
PZ_DEV void candidate_sizes16(uint32_t (&d)[32], int n, bool zbx, Sizes &out) {
  uint32_t bx_or_s = 0, bx_or = 0, bx_and = ~0u, bx_t2 = 0, bx_t3 = 0, bx_adj = 0, gh_prev = 0;
  uint32_t db_or_s = 0, db_or = 0, db_and = ~0u, db_t2 = 0, db_t3 = 0, db_adj = 0, dgh_prev = 0;
  uint32_t b0 = 0, b1 = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t s = d[i];
    // BX: the XORed planes are the bit-planes of s ^ (s >> 1) per symbol.
    const uint32_t g = s ^ ((s >> 1) & 0x7FFF7FFFu);
    const uint32_t gh = g >> 16;
    bx_or_s |= s;
    bx_t3 |= bx_t2 & g;
    bx_t2 |= bx_or & g;
    bx_or |= g;
    bx_and &= g;
    bx_adj |= g & (gh | gh_prev);  // pairs (2i, 2i+1) and (2i-1, 2i), low half
    gh_prev = gh;

    // DBX: deltas s[k] - s[k-1] as 17-bit two's complement; the low 16 bits
    // come from a packed subtract, bit 16 is the borrow (bits 15 and 31 of
    // bo). The XORed planes are the bits of D ^ (D >> 1).
    const uint32_t prevp = i == 0 ? (s << 16) : funnel(s, d[i - 1], 16);
    uint32_t ld = pk_sub_u16(s, prevp);
    uint32_t bo = (~s & prevp) | (~(s ^ prevp) & ld);
    uint32_t gd = ld ^ (((ld >> 1) & 0x7FFF7FFFu) | (bo & 0x80008000u));
    if (i == 0) {  // symbol 0 is the base, not a delta
      ld &= 0xFFFF0000u;
      gd &= 0xFFFF0000u;
      bo &= 0x80000000u;
    }
    const uint32_t dgh = gd >> 16;
    db_or_s |= ld;
    db_t3 |= db_t2 & gd;
    db_t2 |= db_or & gd;
    db_or |= gd;
    db_and &= (i == 0) ? (gd | 0xFFFFu) : gd;
    db_adj |= gd & (dgh | dgh_prev);
    dgh_prev = dgh;
    // Borrow bits, shifted in from the top: b0 bit i = borrow of delta 2i,
    // bit 16+i = borrow of delta 2i+1 (i < 16); b1 likewise for deltas 32+.
    if (i < 16)
      b0 = (b0 >> 1) | (bo & 0x80008000u);
    else
      b1 = (b1 >> 1) | (bo & 0x80008000u);
  }

  uint32_t c1, c2, c3;

  // BX: 16 planes of 64 bits.
  fold_counts16(bx_or, bx_t2, bx_t3, c1, c2, c3);
  const uint32_t nz = c1;
  const uint32_t pz = ~(lo16(bx_or_s) | hi16(bx_or_s)) & 0xFFFFu;
  const uint32_t single = c1 & ~c2;
  const uint32_t exactly2 = c2 & ~c3;
  out.sz[kBX] = plane_code_bits(nz, lo16(bx_and) & hi16(bx_and), pz, exactly2 & lo16(bx_adj), single,
                                16, 64, 4);

  // DBX: base, then 17 planes of 63 bits; plane 16 is the borrow plane.
  fold_counts16(db_or, db_t2, db_t3, c1, c2, c3);
  uint64_t dnz = c1;
  uint64_t dones = lo16(db_and) & hi16(db_and);
  const uint64_t dpz = ~(lo16(db_or_s) | hi16(db_or_s)) & 0xFFFFu;
  uint64_t dsingle = c1 & ~c2;
  uint64_t dpair = c2 & ~c3 & lo16(db_adj);
  const int bc = popc32(b0) + popc32(b1);
  // Adjacent borrows: deltas (2i, 2i+1), (2i+1, 2i+2), and (31, 32).
  const uint32_t badj = ((b0 & (b0 >> 16)) & 0xFFFFu) | (((b0 >> 16) & (b0 >> 1)) & 0x7FFFu) |
                        ((b1 & (b1 >> 16)) & 0xFFFFu) | (((b1 >> 16) & (b1 >> 1)) & 0x7FFFu) |
                        ((b0 >> 31) & b1 & 1u);
  dnz |= (uint64_t)(bc != 0) << 16;
  dones |= (uint64_t)(bc == 63) << 16;
  dsingle |= (uint64_t)(bc == 1) << 16;
  dpair |= (uint64_t)(bc == 2 && badj != 0) << 16;
  out.sz[kDBX] = 16 + plane_code_bits(dnz, dones, dpz, dpair, dsingle, 17, 63, 4);

  // ZBX: the zero, count and pre-XOR masks are those of BX (zero symbols add
  // nothing); "all ones" and adjacency run over the non-zero symbols only.
  if (zbx) {
    launder_regs(d);
    uint32_t zb_and = ~0u, zb_adj = 0, zprev = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t s = d[i];
      const uint32_t g = s ^ ((s >> 1) & 0x7FFF7FFFu);
      const uint32_t gh = g >> 16;
      const uint32_t zfill = pk_sub_u16(pk_min_u16(s, 0x00010001u), 0x00010001u);  // 0xFFFF if zero
      zb_and &= g | zfill;
      const uint32_t q = g | (zprev & zfill);  // low half: last non-zero g up to symbol 2i
      zb_adj |= (zprev & g) | (q & gh);
      zprev = gh | (q & (zfill >> 16));
    }
    out.sz[kZBX] = 64 + plane_code_bits(nz, lo16(zb_and) & hi16(zb_and), pz, exactly2 & lo16(zb_adj),
                                        single, 16, n, 4);
  } else {
    out.sz[kZBX] = 64 + out.sz[kBX];
  }

  out.sz[kZVC] = 64 + 16 * n;
  out.sz[kRAW] = 1024;
  out.n = n;
  out.b0 = b0;
  out.b1 = b1;
}

// ---------------------------------------------------------------------------
// Candidate sizes, w = 32. d[i] is symbol i.
// ---------------------------------------------------------------------------
PZ_DEV void candidate_sizes32(uint32_t (&d)[32], int n, bool zbx, Sizes &out) {
  uint32_t bx_or_s = 0, bx_or = 0, bx_and = ~0u, t2 = 0, t3 = 0, adj = 0, gprev = 0;
  uint32_t db_or_s = 0, db_or = 0, db_and = ~0u, u2 = 0, u3 = 0, dadj = 0, dgprev = 0;
  uint32_t bacc = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t s = d[i];
    const uint32_t g = s ^ (s >> 1);
    bx_or_s |= s;
    t3 |= t2 & g;
    t2 |= bx_or & g;
    bx_or |= g;
    bx_and &= g;
    adj |= g & gprev;
    gprev = g;
    if (i > 0) {
      const uint32_t p = d[i - 1];
      const uint32_t ld = s - p;
      const uint32_t bo = (~s & p) | (~(s ^ p) & ld);  // borrow in bit 31
      const uint32_t gd = ld ^ ((ld >> 1) | (bo & 0x80000000u));
      db_or_s |= ld;
      u3 |= u2 & gd;
      u2 |= db_or & gd;
      db_or |= gd;
      db_and &= gd;
      dadj |= gd & dgprev;
      dgprev = gd;
      bacc = (bacc >> 1) | (bo & 0x80000000u);  // ends with delta i's borrow at bit i
    }
  }
  const uint32_t bm = bacc >> 1;  // plane element k = borrow of delta k+1
  const uint32_t single = bx_or & ~t2;
  const uint32_t exactly2 = t2 & ~t3;
  out.sz[kBX] = plane_code_bits(bx_or, bx_and, ~bx_or_s, exactly2 & adj, single, 32, 32, 5);

  uint32_t zand = bx_and, zadj = adj;
  if (zbx) {
    launder_regs(d);
    uint32_t za = ~0u, zj = 0, zprev = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t s = d[i];
      const uint32_t g = s ^ (s >> 1);
      za &= s != 0 ? g : ~0u;
      zj |= zprev & g;
      zprev = s != 0 ? g : zprev;
    }
    zand = za;
    zadj = zj;
  }
  out.sz[kZBX] = 32 + plane_code_bits(bx_or, zand, ~bx_or_s, exactly2 & zadj, single, 32, n, 5);

  const int bc = popc32(bm);
  const uint64_t dnz = (uint64_t)db_or | ((uint64_t)(bm != 0) << 32);
  const uint64_t dones = (uint64_t)db_and | ((uint64_t)(bm == 0x7FFFFFFFu) << 32);
  const uint64_t dpz = (uint64_t)(~db_or_s);
  const uint64_t dsingle = (uint64_t)(db_or & ~u2) | ((uint64_t)(bc == 1) << 32);
  const uint64_t dpair =
      (uint64_t)(u2 & ~u3 & dadj) | ((uint64_t)(bc == 2 && (bm & (bm >> 1)) != 0) << 32);
  out.sz[kDBX] = 32 + plane_code_bits(dnz, dones, dpz, dpair, dsingle, 33, 31, 5);

  out.sz[kZVC] = 32 + 32 * n;
  out.sz[kRAW] = 1024;
  out.n = n;
  out.b0 = bm;
  out.b1 = 0;
}

template <int W>
PZ_DEV void candidate_sizes(uint32_t (&d)[32], int n, bool zbx, Sizes &out) {
  if constexpr (W == 16)
    candidate_sizes16(d, n, zbx, out);
  else
    candidate_sizes32(d, n, zbx, out);
}

// Smallest allowed candidate (mask bit t = tag t); equal sizes go to the
// lowest tag. Returns the tag and its size (no indexing of the size array by
// a lane-varying tag).
PZ_DEV int select_tag(const Sizes &s, int &best_size, uint32_t mask) {
  int best = 0, bsz = 0x7FFFFFFF;
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    if (((mask >> t) & 1u) && s.sz[t] < bsz) {
      best = t;
      bsz = s.sz[t];
    }
  }
  best_size = bsz;
  return best;
}

// ---------------------------------------------------------------------------
// Per-block diagnostics (pz_block_sizes): every block's five candidate sizes
// and its tag, one lane per block.
// ---------------------------------------------------------------------------
template <int W>
__global__ __launch_bounds__(kGroupThreads, 4) void block_sizes_kernel(
    const uint8_t *__restrict__ src, uint64_t raw_bytes, uint64_t nblocks,
    uint16_t *__restrict__ block_sizes, uint8_t *__restrict__ block_tags) {
  const uint64_t block = (uint64_t)blockIdx.x * kGroupThreads + threadIdx.x;
  if ((uint64_t)blockIdx.x * kGroupThreads >= nblocks) return;
  uint32_t d[32];
  load_block(src, raw_bytes, block * kBlockBytes, d);
  const int n = (int)count_nonzero<W>(d);
  Sizes s;
  candidate_sizes<W>(d, n, __ballot(n > 0 && n < 1024 / W) != 0, s);
  int best_size;
  const int tag = select_tag(s, best_size, 0x1Fu);
  if (block < nblocks) {
    if (block_sizes) {
#pragma unroll
      for (int t = 0; t < 5; ++t) block_sizes[block * 5 + t] = (uint16_t)s.sz[t];
    }
    if (block_tags) block_tags[block] = (uint8_t)tag;
  }
}

// ---------------------------------------------------------------------------
// Emission helpers: fields are OR-ed into the zeroed LDS chunk buffer at an
// explicit bit offset (stream bit t = bit t%32 of dword t/32).
// ---------------------------------------------------------------------------
struct BitSink {
  uint32_t *buf;
  uint32_t off;  // next bit

  // n <= 32 bits of v (v < 2^n).
  PZ_DEV void put(uint32_t v, uint32_t n) {
    const uint32_t q = off >> 5, sh = off & 31u;
    atomicOr(&buf[q], v << sh);
    atomicOr(&buf[q + 1], (v >> 1) >> (31u - sh));  // v >> (32 - sh); 0 when sh == 0
    off += n;
  }
  // n <= 64 bits of v (v < 2^n).
  PZ_DEV void put64(uint64_t v, uint32_t n) {
    const uint32_t q = off >> 5, sh = off & 31u;
    const uint64_t lowpart = v << sh;
    atomicOr(&buf[q], (uint32_t)lowpart);
    atomicOr(&buf[q + 1], (uint32_t)(lowpart >> 32));
    atomicOr(&buf[q + 2], ((uint32_t)(v >> 32) >> 1) >> (31u - sh));
    off += n;
  }
};

// Morton spread: bit i of the low 16 bits goes to bit 2i.
PZ_DEV uint32_t spread16(uint32_t v) {
  v &= 0xFFFFu;
  v = (v | (v << 8)) & 0x00FF00FFu;
  v = (v | (v << 4)) & 0x0F0F0F0Fu;
  v = (v | (v << 2)) & 0x33333333u;
  v = (v | (v << 1)) & 0x55555555u;
  return v;
}

// One plane's code: the pending zero run (if any) and this plane's code in one
// field, then the verbatim payload. x is the XORed plane, p the plane itself.
template <typename PT>
PZ_DEV void emit_plane(BitSink &bs, PT x, PT p, PT ones, uint32_t L, uint32_t pw, uint32_t R,
                       uint32_t &run) {
  if (x == 0) {
    ++run;
    return;
  }
  uint32_t rcode = 0, rlen = 0;
  if (run) {
    rlen = run == 1 ? 3u : 2u + R;
    rcode = run == 1 ? 4u : (2u | ((run - 2u) << 2));
  }
  run = 0;
  int cnt;
  uint32_t low;
  if constexpr (sizeof(PT) == 8) {
    cnt = popc64((uint64_t)x);
    low = (uint32_t)__builtin_ctzll((uint64_t)x);
  } else {
    cnt = popc32((uint32_t)x);
    low = (uint32_t)__builtin_ctz((uint32_t)x);
  }
  const bool is_ones = x == ones;
  const bool is_pz = p == 0;
  const bool is_pair = cnt == 2 && (x >> low) == (PT)3;
  const bool is_single = cnt == 1;
  uint32_t code, clen;
  if (is_ones || is_pz) {
    code = is_ones ? 0u : 16u;
    clen = 5;
  } else if (is_pair || is_single) {
    code = (is_pair ? 8u : 24u) | (low << 5);
    clen = 5 + pw;
  } else {
    code = 1u;
    clen = 1;
  }
  bs.put(rcode | (code << rlen), rlen + clen);
  if (!(is_ones || is_pz || is_pair || is_single)) {
    if constexpr (sizeof(PT) == 8)
      bs.put64((uint64_t)x, L);
    else
      bs.put((uint32_t)x, L);
  }
}

PZ_DEV void emit_run(BitSink &bs, uint32_t run, uint32_t R) {
  if (run) bs.put(run == 1 ? 4u : (2u | ((run - 2u) << 2)), run == 1 ? 3u : 2u + R);
}

// ---------------------------------------------------------------------------
// Single-pass compression, one workgroup per tile of 16 chunks (512 blocks,
// eight waves: two such workgroups fill a CU's LDS; tiles of 8 chunks, with
// twice the workgroups and tile tickets, were 4% slower and tiles of 32
// slower still).
//
// Softmax-like activations hold many all-zero blocks, and a wave runs the
// candidate statistics and the emission for all its lanes at the cost of
// the slowest. So the group first loads its 512 blocks one per thread,
// gives every all-zero block its fixed code (below), and packs the non-zero
// blocks through LDS into the lowest slots: only ceil(nnz / 64) waves then
// run the statistics and the emission. Chunk offsets come from one decoupled
// look-back per group.
// ---------------------------------------------------------------------------
constexpr int kCWaves = 8;  // waves per compress / size workgroup
constexpr int kCThreads = kWave * kCWaves;
constexpr int kGroupChunks = kCThreads / kBlocksPerChunk;
constexpr int kStageDwords = kCThreads * kLaneStride;
constexpr int kGroupBufDwords = kGroupChunks * kChunkBufDwords;
constexpr int kGroupLdsDwords = kStageDwords > kGroupBufDwords ? kStageDwords : kGroupBufDwords;

// An all-zero block under the mode's candidate for it (the smallest allowed;
// BX in PlaneZip): the tag, a zero mask / base / raw block of zero bits
// (already present in the cleared buffer), and for the plane encodings one
// zero run over all planes.
template <int W>
PZ_DEV void emit_zero_block(uint32_t *buf, uint32_t off, const Mode &m) {
  constexpr uint32_t N = 1024 / W, R = W == 16 ? 4 : 5;
  const uint32_t c = m.zc;
  BitSink z;
  z.buf = buf;
  z.off = off;
  if (m.tagged) z.put(c, 3);
  z.off += c == 0 ? N : (c == 1 ? (uint32_t)W : (c == 3 ? N : (c == 4 ? 1024u : 0u)));
  const uint32_t planes = c == 1 ? W + 1 : ((c == 2 || c == 3) ? (uint32_t)W : 0u);
  if (planes) z.put(2u | ((planes - 2u) << 2), 2 + R);
}

template <int W>
__global__ __launch_bounds__(kCThreads, 2) void compress_kernel(const CBatch batch, uint64_t *lb_words,
                                                                 uint32_t *tile_counter, uint32_t counter_base,
                                                                 uint32_t epoch, Mode mode) {
  constexpr int N = 1024 / W;
  constexpr uint32_t R = W == 16 ? 4 : 5;
  using PT = typename std::conditional<W == 16, uint64_t, uint32_t>::type;
  // Staging slots / ZBX compaction regions (stride kLaneStride), later the
  // eight chunk buffers.
  __shared__ __attribute__((aligned(16))) uint32_t lds[kGroupLdsDwords];
  __shared__ uint16_t blk_bits[kCThreads];  // per block: its cost, then its bit offset
  __shared__ uint16_t slot_block[kCThreads];  // compacted slot -> block of the group
  __shared__ uint8_t slot_n[kCThreads];      // compacted slot -> its non-zero symbols
  __shared__ uint32_t wave_full[kCWaves];
  __shared__ uint32_t wave_part[kCWaves];
  __shared__ uint32_t chunk_len[kGroupChunks];
  __shared__ uint64_t chunk_pay[kGroupChunks];
  __shared__ uint32_t group_tile;

  const uint32_t t = threadIdx.x, lane = lane_id();
  const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: a scalar
  if (t == 0) group_tile = atomicAdd(tile_counter, 1u) - counter_base;
  __syncthreads();
  // The launch's tile -> the tensor it belongs to and the tile within it.
  const uint32_t gtile = __builtin_amdgcn_readfirstlane(group_tile);
  if (gtile >= batch.total_tiles) return;
  uint32_t k = 0;
  if (batch.n > 1) {  // a single tensor's fields load at once
#pragma unroll
    for (uint32_t i = 1; i < (uint32_t)kMaxBatch; ++i) k += i < batch.n && gtile >= batch.t[i].tile_begin ? 1u : 0u;
  }
  const uint8_t *__restrict__ src = batch.t[k].src;
  uint8_t *__restrict__ dst = batch.t[k].dst;
  const uint64_t raw_bytes = batch.t[k].raw_bytes, nchunks = batch.t[k].nchunks;
  const uint32_t ntiles = batch.t[k].ntiles;
  const uint32_t tile = gtile - batch.t[k].tile_begin;
  uint64_t *status = lb_words + batch.t[k].tile_begin;

  // --- 1. Load block t; count its non-zero symbols. ---
  // (Block and chunk indices are recomputed where needed rather than kept
  // live through the statistics, which use every register.)
  const uint64_t block = (uint64_t)tile * kCThreads + t;
  const bool valid = block * kBlockBytes < raw_bytes;
  uint32_t d[32];
  load_block(src, raw_bytes, block * kBlockBytes, d);
  uint32_t sn = count_nonzero<W>(d);  // blocks past the end load as zeros
  const bool nonzero = sn != 0;
  const bool partial = nonzero && sn < (uint32_t)N;
  const uint64_t mfull = __ballot(nonzero && !partial), mpart = __ballot(partial);
  if (lane == 0) {
    wave_full[wave] = (uint32_t)popc64(mfull);
    wave_part[wave] = (uint32_t)popc64(mpart);
  }
  if (!nonzero) blk_bits[t] = (uint16_t)(valid ? 3u * mode.tagged + zero_block_size(W, mode.zc) : 0u);
  __syncthreads();

  // --- 2. Slots: the non-zero blocks are packed through LDS into slots
  // 0..nnz-1, those without a zero symbol first, so that the ZBX statistics
  // (needed only when 0 < n < N) run on as few waves as possible. ---
  uint32_t nfull = 0, npart = 0, ffirst = 0, pfirst = 0;
#pragma unroll
  for (int k = 0; k < kCWaves; ++k) {
    const uint32_t f = wave_full[k], q = wave_part[k];
    ffirst += (uint32_t)k < wave ? f : 0u;
    pfirst += (uint32_t)k < wave ? q : 0u;
    nfull += f;
    npart += q;
  }
  const uint32_t nnz = nfull + npart;
  if (nonzero) {
    const uint32_t idx = partial ? nfull + pfirst + lanes_below(mpart) : ffirst + lanes_below(mfull);
    uint32_t *slot = lds + idx * kLaneStride;
#pragma unroll
    for (int i = 0; i < 32; ++i) slot[i] = d[i];
    slot_block[idx] = (uint16_t)t;
    slot_n[idx] = (uint8_t)sn;
  }
  __syncthreads();

  // Waves take the slots in an order rotated per tile, so that the busy
  // waves of successive groups fall on different SIMDs.
  const uint32_t slot = (t + kCThreads - 64u * (tile & (kCWaves - 1u))) & (kCThreads - 1);
  const bool active = slot < nnz;
  const bool wave_active = __ballot(active) != 0;

  // --- 3. Sizes, selection and the transform input of the packed blocks. ---
  Sizes s;
  s.n = 0;
  s.b0 = s.b1 = 0;
  int tag = kRAW;
  uint64_t nzmask = 0;
  uint32_t base = 0;
  uint32_t e[32];
  if (wave_active) {
    uint32_t *region = lds + slot * kLaneStride;
    sn = active ? (uint32_t)slot_n[slot] : 0u;
    if (active) {
#pragma unroll
      for (int i = 0; i < 32; ++i) d[i] = region[i];
    }
    const bool zbx = __ballot(active && sn < (uint32_t)N) != 0;  // active blocks are non-zero
    candidate_sizes<W>(d, (int)sn, zbx, s);
    s.n = (int)sn;
    launder_regs(d);
    int best_size;
    tag = select_tag(s, best_size, mode.mask);
    if (active) blk_bits[slot_block[slot]] = (uint16_t)(3u * mode.tagged + best_size);

    const bool want_zvc = active && tag == kZVC;
    const bool want_dbx = active && tag == kDBX;
    const bool want_zbx = active && tag == kZBX;
    // Non-zero mask (ZVC and ZBX prefix), bit i = symbol i non-zero.
    if (__ballot(want_zvc || want_zbx)) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if constexpr (W == 16) {
          nzmask |= (uint64_t)((d[i] & 0xFFFFu) != 0) << (2 * i);
          nzmask |= (uint64_t)((d[i] >> 16) != 0) << (2 * i + 1);
        } else {
          nzmask |= (uint64_t)(d[i] != 0) << i;
        }
      }
    }
    base = W == 16 ? (d[0] & 0xFFFFu) : d[0];

    // ZBX and ZVC: move the non-zero symbols to the front of this slot's
    // region (the slot was read above; no other thread touches it).
    const bool want_cmp = want_zbx || want_zvc;
    const bool any_cmp = __ballot(want_cmp) != 0;
    if (any_cmp) {
      if (want_cmp) {
#pragma unroll
        for (int i = 0; i < 32; ++i) region[i] = 0;
      }
      wave_lds_fence();
      if (want_cmp) {
        // Every symbol is written at the current rank, which advances only
        // past non-zero ones: a zero symbol writes 0 where the next non-zero
        // symbol (or nothing) goes, so there are no branches.
        uint32_t k = 0;
        if constexpr (W == 16) {
          uint16_t *r16 = reinterpret_cast<uint16_t *>(region);
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const uint32_t a = d[i] & 0xFFFFu, b = d[i] >> 16;
            r16[k] = (uint16_t)a;
            k += a ? 1u : 0u;
            r16[k] = (uint16_t)b;
            k += b ? 1u : 0u;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            region[k] = d[i];
            k += d[i] ? 1u : 0u;
          }
        }
      }
      wave_lds_fence();
    }

    // Transform input: the symbols, the deltas (DBX, arranged so that plane
    // element k is delta k+1) or the compacted symbols (ZBX).
#pragma unroll
    for (int i = 0; i < 32; ++i) e[i] = d[i];
    if (__ballot(want_dbx)) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        uint32_t v;
        if constexpr (W == 16) {
          // dword i = (delta 2i+1, delta 2i+2); the last slot is empty.
          const uint32_t cur = funnel(i < 31 ? d[i + 1] : 0u, d[i], 16);  // (s 2i+1, s 2i+2)
          v = pk_sub_u16(cur, d[i]);
          if (i == 31) v &= 0xFFFFu;
        } else {
          v = i < 31 ? d[i + 1] - d[i] : 0u;
        }
        e[i] = want_dbx ? v : e[i];
      }
    }
    if (any_cmp) {
#pragma unroll
      for (int i = 0; i < 32; ++i) e[i] = want_cmp ? region[i] : e[i];
    }
  }
  __syncthreads();  // costs complete; staging and regions free

  // --- 4. Chunk assembly in block order: bit offsets, lengths, headers. ---
  const uint32_t cost = blk_bits[t];
  const uint32_t incl = half_inclusive_scan(cost);
  const uint32_t excl = incl - cost;
  const uint32_t bits = __shfl(incl, (int)((lane & 32) | 31), 64);
  uint32_t raw_len = 0, len = 0;
  const uint64_t chunk = (uint64_t)tile * kGroupChunks + (t >> 5);
  if (chunk < nchunks) {
    raw_len = (uint32_t)min_u64(kChunkBytes, raw_bytes - chunk * kChunkBytes);
    len = (bits + 7) / 8;
    if (len >= raw_len) len = raw_len;
  }
  const bool raw_chunk = len == raw_len;
  blk_bits[t] = (uint16_t)excl;
  if ((lane & 31) == 0) {
    chunk_len[t >> 5] = len;
    if (chunk < nchunks) reinterpret_cast<uint16_t *>(dst)[chunk] = (uint16_t)len;
  }
  {
    uint4 *z = reinterpret_cast<uint4 *>(lds);
    for (uint32_t i = t; i < (uint32_t)kGroupBufDwords / 4; i += kCThreads)
      z[i] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  // The group's aggregate goes out now; the device-wide offsets are resolved
  // after the emission (which works at byte alignment 0), so that waiting on
  // the predecessors overlaps with it.
  uint32_t l = 0, inc = 0, agg = 0;
  if (wave == 0) {
    l = lane < (uint32_t)kGroupChunks ? chunk_len[lane] : 0u;
    inc = l;
#pragma unroll
    for (int o = 1; o < kGroupChunks; o <<= 1) {
      const uint32_t v = __shfl_up(inc, o, 64);
      if (lane >= (uint32_t)o) inc += v;
    }
    agg = __shfl(inc, kGroupChunks - 1, 64);
    lookback_publish(status, tile, agg, epoch);
  }

  // --- 5. Emission into the chunk buffers (payload bit i at buffer bit i). ---
  // All-zero blocks of coded chunks: their one code. (In a raw chunk their
  // bytes are zeros, which the cleared buffer already holds.)
  if (((uint64_t)tile * kCThreads + t) * kBlockBytes < raw_bytes && !nonzero && !raw_chunk) {
    emit_zero_block<W>(lds + (t >> 5) * kChunkBufDwords, excl, mode);
  }

  if (wave_active) {
    const uint32_t sb = active ? (uint32_t)slot_block[slot] : 0u;  // the slot's block in the group
    const uint32_t ch = sb >> 5;
    const uint64_t cchunk = (uint64_t)tile * kGroupChunks + ch;
    const uint32_t craw_len =
        cchunk < nchunks ? (uint32_t)min_u64(kChunkBytes, raw_bytes - cchunk * kChunkBytes) : 0u;
    const bool craw = chunk_len[ch] == craw_len;
    const bool coded = active && !craw;
    const bool want_raw = active && (craw || tag == kRAW);
    const bool want_zvc = coded && tag == kZVC;
    const bool want_dbx = coded && tag == kDBX;
    const bool want_zbx = coded && tag == kZBX;
    const bool want_planes = coded && (tag == kDBX || tag == kBX || tag == kZBX);

    BitSink bs;
    bs.buf = lds + ch * kChunkBufDwords;
    bs.off = craw ? 1024u * (sb & 31) : (uint32_t)blk_bits[sb];
    if (coded && mode.tagged) bs.put((uint32_t)tag, 3);

    if (__ballot(want_raw)) {
      // A raw chunk needs the symbols themselves back where e holds a transform.
      const bool reload = want_raw && (tag == kDBX || tag == kZBX || tag == kZVC);
      if (__ballot(reload)) {
        if (reload) load_block(src, raw_bytes, ((uint64_t)tile * kCThreads + sb) * kBlockBytes, e);
      }
      if (want_raw) {
        // 1024 bits: the first and last dwords are shared with neighbours
        // (OR), the 31 between belong to this block alone.
        const uint32_t q = bs.off >> 5, sh = bs.off & 31u;
        atomicOr(&bs.buf[q], e[0] << sh);
#pragma unroll
        for (int i = 1; i < 32; ++i) bs.buf[q + i] = (e[i] << sh) | ((e[i - 1] >> 1) >> (31u - sh));
        atomicOr(&bs.buf[q + 32], (e[31] >> 1) >> (31u - sh));
        bs.off += 1024;
      }
    }

    if (__ballot(want_zvc)) {
      // The mask, then the n non-zero symbols: the compacted symbols in e,
      // 32 bits (two symbols) at a time, until no lane has any left.
      if (want_zvc) bs.put64(nzmask, N);
      const uint32_t bits = want_zvc ? (uint32_t)W * (uint32_t)s.n : 0u;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        if (!__ballot(32u * q < bits)) break;
        if (32u * q < bits) {
          const uint32_t len = bits - 32u * q < 32u ? bits - 32u * q : 32u;
          bs.put(e[q], len);
        }
      }
    }

    if (__ballot(want_planes)) {
      if (want_dbx) bs.put(base, W);
      if (want_zbx) bs.put64(nzmask, N);
      const uint32_t L = want_dbx ? (uint32_t)(N - 1) : (want_zbx ? (uint32_t)s.n : (uint32_t)N);
      const uint32_t pw = (uint32_t)position_bits((int)L);
      const PT ones = (PT)all_ones64((int)L);
      uint32_t run = 0;
      PT above = 0;
      // DBX's top plane: the borrow bits of the deltas.
      if (__ballot(want_dbx)) {
        PT bm;
        if constexpr (W == 16) {
          const uint32_t m0 = spread16(s.b0) | (spread16(s.b0 >> 16) << 1);  // bit m: delta m
          const uint32_t m1 = spread16(s.b1) | (spread16(s.b1 >> 16) << 1);  // bit m: delta 32+m
          bm = (((uint64_t)m1 << 32) | m0) >> 1;
        } else {
          bm = s.b0;
        }
        if (want_dbx) {
          emit_plane<PT>(bs, bm, bm, ones, L, pw, R, run);
          above = bm;
        }
      }
      if constexpr (W == 16) {
        uint64_t P[16];
        {
          // Symbols k and k+32 share a dword, so one 32x32 transpose yields
          // the low and high halves of every 64-bit plane.
          uint32_t tr[32];
#pragma unroll
          for (int r = 0; r < 32; ++r) {
            const uint32_t a = e[r >> 1], b = e[16 + (r >> 1)];
            tr[r] = ((r & 1) ? (a >> 16) : (a & 0xFFFFu)) | ((r & 1) ? (b & 0xFFFF0000u) : (b << 16));
          }
          transpose32(tr);
#pragma unroll
          for (int j = 0; j < 16; ++j) P[j] = (uint64_t)tr[j] | ((uint64_t)tr[j + 16] << 32);
        }
#pragma unroll
        for (int j = 15; j >= 0; --j) {
          if (want_planes) {
            const uint64_t p = P[j];
            emit_plane<uint64_t>(bs, p ^ above, p, ones, L, pw, R, run);
            above = p;
          }
        }
      } else {
        transpose32(e);
#pragma unroll
        for (int j = 31; j >= 0; --j) {
          if (want_planes) {
            const uint32_t p = e[j];
            emit_plane<uint32_t>(bs, p ^ above, p, ones, L, pw, R, run);
            above = p;
          }
        }
      }
      if (want_planes) emit_run(bs, run, R);
    }
  }

  // Device-wide payload offsets of the group's chunks.
  if (wave == 0) {
    const uint64_t before = lookback_resolve(status, tile, agg, epoch);
    if (lane < (uint32_t)kGroupChunks) chunk_pay[lane] = 2 * nchunks + before + (inc - l);
    if (tile == ntiles - 1 && lane == 0) *batch.t[k].out_bytes = 2 * nchunks + before + agg;
  }
  __syncthreads();

  // --- 6. Store: wave w writes chunks 2w and 2w+1 in 16-byte units.
  // Payload byte i goes to dst byte poff + i. With sh = poff & 15 =
  // 4 dsh + bsh, dst dword o of the 16-byte aligned span holds payload bytes
  // 4o - sh .. 4o - sh + 3: buffer dwords o - dsh - 1 and o - dsh joined by
  // a funnel shift. Unit u of the span therefore needs buffer dwords
  // 4u - dsh - 1 .. 4u - dsh + 3, which lie in the aligned quads u - 1 and u
  // (two conflict-free 16-byte LDS reads; dsh is uniform over the chunk).
  // Only the first and last units (shared with the neighbouring chunks) are
  // written piecewise. ---
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t c = 2 * wave + (uint32_t)h;
    const uint32_t plen = chunk_len[c];
    if (plen == 0) continue;
    const uint64_t poff = chunk_pay[c];
    const uint32_t sh = (uint32_t)(poff & 15);
    const uint32_t dsh = sh >> 2, rs = 32u - 8u * (sh & 3u);
    uint8_t *span = dst + (poff - sh);
    const uint32_t total = sh + plen;
    const uint32_t nun = (total + 15) / 16;
    const uint4 *quad = reinterpret_cast<const uint4 *>(lds + c * kChunkBufDwords);
    for (uint32_t u = lane; u < nun; u += kWave) {
      const uint4 p = u > 0 ? quad[u - 1] : make_uint4(0, 0, 0, 0);
      const uint4 q = quad[u];
      uint32_t w0, w1, w2, w3, w4;  // buffer dwords 4u - dsh - 1 .. 4u - dsh + 3
      if (dsh == 0) {
        w0 = p.w; w1 = q.x; w2 = q.y; w3 = q.z; w4 = q.w;
      } else if (dsh == 1) {
        w0 = p.z; w1 = p.w; w2 = q.x; w3 = q.y; w4 = q.z;
      } else if (dsh == 2) {
        w0 = p.y; w1 = p.z; w2 = p.w; w3 = q.x; w4 = q.y;
      } else {
        w0 = p.x; w1 = p.y; w2 = p.z; w3 = p.w; w4 = q.x;
      }
      uint32_t v[4];
      if (rs == 32) {
        v[0] = w1; v[1] = w2; v[2] = w3; v[3] = w4;
      } else {
        v[0] = funnel(w1, w0, rs); v[1] = funnel(w2, w1, rs); v[2] = funnel(w3, w2, rs); v[3] = funnel(w4, w3, rs);
      }
      const uint32_t b0 = 16 * u;
      if (b0 >= sh && b0 + 16 <= total) {
        *reinterpret_cast<uint4 *>(span + b0) = make_uint4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (uint32_t k = 0; k < 4; ++k) {
          const uint32_t d0 = b0 + 4 * k;
          if (d0 >= sh && d0 + 4 <= total) {
            *reinterpret_cast<uint32_t *>(span + d0) = v[k];
          } else {
#pragma unroll
            for (uint32_t b = 0; b < 4; ++b)
              if (d0 + b >= sh && d0 + b < total) span[d0 + b] = (uint8_t)(v[k] >> (8 * b));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Size pass (pz_compressed_size, pz_compressed_size_sampled): the first four
// phases of compress_kernel with nothing emitted. A workgroup takes 16 sampled
// chunks (chunk = sample * stride; stride 1 samples every chunk), loads their
// 512 blocks one per thread, gives all-zero blocks their fixed cost, packs the
// other blocks onto the fewest waves for the candidate sizes, and scans each
// chunk's block costs to its length. Lengths go to chunk_lens; their sum to
// out_bytes (which holds the headers' bytes beforehand).
// ---------------------------------------------------------------------------
template <int W>
__global__ __launch_bounds__(kCThreads, 2) void size_kernel(const SBatch batch, Mode mode) {
  constexpr int N = 1024 / W;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kStageDwords];
  __shared__ uint16_t blk_bits[kCThreads];
  __shared__ uint16_t slot_block[kCThreads];
  __shared__ uint8_t slot_n[kCThreads];
  __shared__ uint32_t wave_full[kCWaves];
  __shared__ uint32_t wave_part[kCWaves];
  __shared__ uint32_t chunk_len[kGroupChunks];

  const uint32_t t = threadIdx.x, lane = lane_id();
  const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // The launch's group -> the tensor it belongs to (the last one starting at
  // or before it: a tensor without chunks has no groups).
  uint32_t k = 0;
  if (batch.n > 1) {  // a single tensor's fields load at once
#pragma unroll
    for (uint32_t i = 1; i < (uint32_t)kMaxBatch; ++i) k += i < batch.n && blockIdx.x >= batch.t[i].group_begin ? 1u : 0u;
  }
  const uint8_t *__restrict__ src = batch.t[k].src;
  const uint64_t raw_bytes = batch.t[k].raw_bytes, nchunks = batch.t[k].nchunks;
  const uint64_t stride = batch.t[k].stride, nsampled = batch.t[k].nsampled;
  uint64_t *__restrict__ out_bytes = batch.t[k].out_bytes;
  uint16_t *__restrict__ chunk_lens = batch.t[k].chunk_lens;
  const uint64_t sample = (uint64_t)(blockIdx.x - batch.t[k].group_begin) * kGroupChunks + (t >> 5);
  // Samples past the last one read as zeros (their chunk is past the end).
  const uint64_t chunk = sample < nsampled ? sample * stride : nchunks;
  const uint64_t block = chunk * kBlocksPerChunk + (t & 31);
  const bool valid = block * kBlockBytes < raw_bytes;

  uint32_t d[32];
  load_block(src, raw_bytes, block * kBlockBytes, d);
  uint32_t sn = count_nonzero<W>(d);
  const bool nonzero = sn != 0;
  const bool partial = nonzero && sn < (uint32_t)N;
  const uint64_t mfull = __ballot(nonzero && !partial), mpart = __ballot(partial);
  if (lane == 0) {
    wave_full[wave] = (uint32_t)popc64(mfull);
    wave_part[wave] = (uint32_t)popc64(mpart);
  }
  if (!nonzero) blk_bits[t] = (uint16_t)(valid ? 3u * mode.tagged + zero_block_size(W, mode.zc) : 0u);
  __syncthreads();

  uint32_t nfull = 0, npart = 0, ffirst = 0, pfirst = 0;
#pragma unroll
  for (int k = 0; k < kCWaves; ++k) {
    const uint32_t f = wave_full[k], q = wave_part[k];
    ffirst += (uint32_t)k < wave ? f : 0u;
    pfirst += (uint32_t)k < wave ? q : 0u;
    nfull += f;
    npart += q;
  }
  const uint32_t nnz = nfull + npart;
  if (nonzero) {
    const uint32_t idx = partial ? nfull + pfirst + lanes_below(mpart) : ffirst + lanes_below(mfull);
    uint32_t *slot = lds + idx * kLaneStride;
#pragma unroll
    for (int i = 0; i < 32; ++i) slot[i] = d[i];
    slot_block[idx] = (uint16_t)t;
    slot_n[idx] = (uint8_t)sn;
  }
  __syncthreads();

  const uint32_t slot = (t + kCThreads - 64u * (blockIdx.x & (kCWaves - 1u))) & (kCThreads - 1);
  const bool active = slot < nnz;
  if (__ballot(active) != 0) {
    const uint32_t *region = lds + slot * kLaneStride;
    sn = active ? (uint32_t)slot_n[slot] : 0u;
    if (active) {
#pragma unroll
      for (int i = 0; i < 32; ++i) d[i] = region[i];
    }
    Sizes s;
    candidate_sizes<W>(d, (int)sn, __ballot(active && sn < (uint32_t)N) != 0, s);
    int best_size;
    select_tag(s, best_size, mode.mask);
    if (active) blk_bits[slot_block[slot]] = (uint16_t)(3u * mode.tagged + best_size);
  }
  __syncthreads();

  const uint32_t cost = blk_bits[t];
  const uint32_t bits = __shfl(half_inclusive_scan(cost), (int)((lane & 32) | 31), 64);
  if ((lane & 31) == 0) {
    uint32_t len = 0;
    if (chunk < nchunks) {
      const uint32_t raw_len = (uint32_t)min_u64(kChunkBytes, raw_bytes - chunk * kChunkBytes);
      len = (bits + 7) / 8;
      if (len >= raw_len) len = raw_len;
      if (chunk_lens) chunk_lens[sample] = (uint16_t)len;
    }
    chunk_len[t >> 5] = len;
  }
  __syncthreads();
  if (t == 0 && out_bytes) {
    uint64_t sum = 0;
#pragma unroll
    for (int c = 0; c < kGroupChunks; ++c) sum += chunk_len[c];
    atomicAdd((unsigned long long *)out_bytes, (unsigned long long)sum);
  }
}

__global__ void fill_u64_kernel(uint64_t *p, uint64_t n, uint64_t value) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

hipError_t fill_u64(uint64_t *p, uint64_t n, uint64_t value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const uint64_t groups = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(fill_u64_kernel, dim3((unsigned)groups), dim3(256), 0, stream, p, n, value);
  return hipGetLastError();
}

// Starting values of a size launch's outputs: the sampled chunks' headers
// (2 bytes each) and their raw bytes (whole chunks except the tensor's last
// chunk when it is sampled); thread k sets tensor k's.
__global__ void store_size_init_kernel(const SBatch batch) {
  const uint32_t k = threadIdx.x;
  if (k >= batch.n) return;
  const STensor &x = batch.t[k];
  const uint64_t last = x.nsampled ? (x.nsampled - 1) * x.stride : 0;
  const uint64_t sampled_raw =
      x.nsampled ? (x.nsampled - 1) * kChunkBytes + min_u64(kChunkBytes, x.raw_bytes - last * kChunkBytes) : 0;
  if (x.out_bytes) *x.out_bytes = 2 * x.nsampled;
  if (x.out_raw) *x.out_raw = sampled_raw;
}

void size_plan(STensor &x) {
  x.nchunks = (x.raw_bytes + kChunkBytes - 1) / kChunkBytes;
  x.nsampled = (x.nchunks + x.stride - 1) / x.stride;
  x.ngroups = (uint32_t)((x.nsampled + kGroupChunks - 1) / kGroupChunks);
}

hipError_t launch_size(int w, const SBatch &batch, uint32_t codec_mask, int tagged, hipStream_t stream) {
  hipLaunchKernelGGL(store_size_init_kernel, dim3(1), dim3(64), 0, stream, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || batch.total_groups == 0) return e;
  const Mode mode = make_mode(w, codec_mask, tagged);
  if (w == 16)
    hipLaunchKernelGGL(size_kernel<16>, dim3(batch.total_groups), dim3(kCThreads), 0, stream, batch, mode);
  else
    hipLaunchKernelGGL(size_kernel<32>, dim3(batch.total_groups), dim3(kCThreads), 0, stream, batch, mode);
  return hipGetLastError();
}

hipError_t launch_block_sizes(int w, const uint8_t *src, uint64_t raw_bytes, uint16_t *block_sizes,
                              uint8_t *block_tags, hipStream_t stream) {
  const uint64_t nblocks = (raw_bytes + kBlockBytes - 1) / kBlockBytes;
  if (nblocks == 0) return hipSuccess;
  const uint64_t groups = (nblocks + kGroupThreads - 1) / kGroupThreads;
  if (w == 16)
    hipLaunchKernelGGL(block_sizes_kernel<16>, dim3((unsigned)groups), dim3(kGroupThreads), 0, stream, src,
                       raw_bytes, nblocks, block_sizes, block_tags);
  else
    hipLaunchKernelGGL(block_sizes_kernel<32>, dim3((unsigned)groups), dim3(kGroupThreads), 0, stream, src,
                       raw_bytes, nblocks, block_sizes, block_tags);
  return hipGetLastError();
}

uint32_t compress_tiles(uint64_t raw_bytes) {
  const uint64_t nchunks = (raw_bytes + kChunkBytes - 1) / kChunkBytes;
  return (uint32_t)((nchunks + kGroupChunks - 1) / kGroupChunks);
}

hipError_t launch_compress(int w, const CBatch &batch, uint32_t codec_mask, int tagged,
                           const Scratch &scratch, hipStream_t stream) {
  const Mode mode = make_mode(w, codec_mask, tagged);
  if (w == 16)
    hipLaunchKernelGGL(compress_kernel<16>, dim3(batch.total_tiles), dim3(kCThreads), 0, stream, batch,
                       scratch.words, scratch.counter, scratch.counter_base, scratch.epoch, mode);
  else
    hipLaunchKernelGGL(compress_kernel<32>, dim3(batch.total_tiles), dim3(kCThreads), 0, stream, batch,
                       scratch.words, scratch.counter, scratch.counter_base, scratch.epoch, mode);
  return hipGetLastError();
}

}  // namespace pz
