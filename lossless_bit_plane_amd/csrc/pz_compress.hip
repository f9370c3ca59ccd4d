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
// emitted, bit by bit-field, into a per-chunk LDS buffer. Chunk offsets come
// from a single-pass decoupled look-back over per-wave chunk-length sums, so
// the input is read once and the stream written once.
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
#pragma unroll
    for (int i = 0; i < 32; ++i) d[i] = 0;
    if (off < raw_bytes) {
      const uint32_t n = (uint32_t)(raw_bytes - off);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t k = 4 * i + b;
          if (k < n) v |= (uint32_t)src[off + k] << (8 * b);
        }
        d[i] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Candidate sizes, w = 16. d[i] holds symbols 2i (low half) and 2i+1 (high).
// ---------------------------------------------------------------------------
struct Sizes {
  int sz[5];
  int n;          // non-zero symbols
  uint64_t bm;    // DBX top plane: borrow bits of the deltas
};

PZ_DEV uint32_t lo16(uint32_t x) { return x & 0xFFFFu; }
PZ_DEV uint32_t hi16(uint32_t x) { return x >> 16; }

// Merges per-half saturating counters (>=1, >=2, >=3 ones) of the two halves.
PZ_DEV void fold_counts16(uint32_t t1, uint32_t t2, uint32_t t3, uint32_t &c1, uint32_t &c2,
                          uint32_t &c3) {
  c1 = lo16(t1) | hi16(t1);
  c2 = lo16(t2) | hi16(t2) | (lo16(t1) & hi16(t1));
  c3 = lo16(t3) | hi16(t3) | (lo16(t2) & hi16(t1)) | (lo16(t1) & hi16(t2));
}

PZ_DEV void candidate_sizes16(const uint32_t (&d)[32], Sizes &out) {
  uint32_t bx_or_s = 0, bx_or = 0, bx_and = ~0u, bx_t1 = 0, bx_t2 = 0, bx_t3 = 0, bx_adj = 0;
  uint32_t db_or_s = 0, db_or = 0, db_and = ~0u, db_t1 = 0, db_t2 = 0, db_t3 = 0, db_adj = 0;
  uint32_t zb_and = ~0u, zb_adj = 0, zb_prev = 0;
  uint32_t cnt = 0, gh_prev = 0, dgh_prev = 0;
  uint64_t bm = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t s = d[i];
    // BX: the XORed planes are the bit-planes of s ^ (s >> 1) per symbol.
    const uint32_t g = s ^ ((s >> 1) & 0x7FFF7FFFu);
    const uint32_t gh = g >> 16;
    bx_or_s |= s;
    bx_or |= g;
    bx_and &= g;
    bx_t3 |= bx_t2 & g;
    bx_t2 |= bx_t1 & g;
    bx_t1 |= g;
    bx_adj |= g & (gh | gh_prev);  // pairs (2i, 2i+1) and (2i-1, 2i), in the low half
    gh_prev = gh;

    // Zero symbols: zfill is 0xFFFF in a half whose symbol is zero.
    const uint32_t nzh = pk_min_u16(s, 0x00010001u);
    const uint32_t zfill = pk_sub_u16(nzh, 0x00010001u);
    cnt = pk_add_u16(cnt, nzh);

    // ZBX: AND over the non-zero symbols only; adjacency in compacted order
    // (zb_prev is the last non-zero symbol's g, in the low half).
    zb_and &= g | zfill;
    const uint32_t q = g | (zb_prev & zfill);
    zb_adj |= (zb_prev & g) | (q & gh);
    zb_prev = gh | (q & (zfill >> 16));

    // DBX: deltas s[k] - s[k-1] as 17-bit two's complement; the low 16 bits
    // come from a packed subtract, bit 16 is the borrow. The XORed planes are
    // the bits of D ^ (D >> 1), whose bit 15 mixes in the borrow.
    const uint32_t prevp = i == 0 ? (s << 16) : funnel(s, d[i - 1], 16);
    uint32_t ld = pk_sub_u16(s, prevp);
    uint32_t bo = ((~s & prevp) | (~(s ^ prevp) & ld)) & 0x80008000u;
    uint32_t gd = ld ^ (((ld >> 1) & 0x7FFF7FFFu) | bo);
    if (i == 0) {  // symbol 0 is the base, not a delta
      ld &= 0xFFFF0000u;
      gd &= 0xFFFF0000u;
      bo &= 0x80000000u;
    }
    const uint32_t dgh = gd >> 16;
    db_or_s |= ld;
    db_or |= gd;
    db_and &= (i == 0) ? (gd | 0xFFFFu) : gd;
    db_t3 |= db_t2 & gd;
    db_t2 |= db_t1 & gd;
    db_t1 |= gd;
    db_adj |= gd & (dgh | dgh_prev);
    dgh_prev = dgh;
    // Delta 2i (low half) is plane element 2i-1; delta 2i+1 is element 2i.
    if (i > 0) bm |= (uint64_t)((bo >> 15) & 1u) << (2 * i - 1);
    bm |= (uint64_t)(bo >> 31) << (2 * i);
  }

  const int n = (int)(lo16(cnt) + hi16(cnt));
  uint32_t c1, c2, c3;

  // BX: 16 planes of 64 bits.
  fold_counts16(bx_t1, bx_t2, bx_t3, c1, c2, c3);
  const uint32_t nz = lo16(bx_or) | hi16(bx_or);
  const uint32_t pz = ~(lo16(bx_or_s) | hi16(bx_or_s)) & 0xFFFFu;
  const uint32_t single = c1 & ~c2;
  const uint32_t adj = lo16(bx_adj);
  out.sz[kBX] = plane_code_bits(nz, lo16(bx_and) & hi16(bx_and), pz, c2 & ~c3 & adj, single, 16, 64, 4);

  // ZBX: mask, then 16 planes of n bits (same zero, count and pre-XOR masks).
  const uint32_t zadj = lo16(zb_adj);
  out.sz[kZBX] = 64 + plane_code_bits(nz, lo16(zb_and) & hi16(zb_and), pz, c2 & ~c3 & zadj, single,
                                      16, n, 4);

  // DBX: base, then 17 planes of 63 bits; plane 16 is the borrow plane.
  fold_counts16(db_t1, db_t2, db_t3, c1, c2, c3);
  uint64_t dnz = lo16(db_or) | hi16(db_or);
  uint64_t dones = lo16(db_and) & hi16(db_and);
  const uint64_t dpz = ~(lo16(db_or_s) | hi16(db_or_s)) & 0xFFFFu;
  uint64_t dsingle = c1 & ~c2;
  uint64_t dpair = c2 & ~c3 & lo16(db_adj);
  const int bc = popc64(bm);
  dnz |= (uint64_t)(bm != 0) << 16;
  dones |= (uint64_t)(bm == 0x7FFFFFFFFFFFFFFFull) << 16;
  dsingle |= (uint64_t)(bc == 1) << 16;
  dpair |= (uint64_t)(bc == 2 && (bm & (bm >> 1)) != 0) << 16;
  out.sz[kDBX] = 16 + plane_code_bits(dnz, dones, dpz, dpair, dsingle, 17, 63, 4);

  out.sz[kZVC] = 64 + 16 * n;
  out.sz[kRAW] = 1024;
  out.n = n;
  out.bm = bm;
}

// ---------------------------------------------------------------------------
// Candidate sizes, w = 32. d[i] is symbol i.
// ---------------------------------------------------------------------------
PZ_DEV void candidate_sizes32(const uint32_t (&d)[32], Sizes &out) {
  uint32_t bx_or_s = 0, bx_or = 0, bx_and = ~0u, t1 = 0, t2 = 0, t3 = 0, adj = 0, gprev = 0;
  uint32_t db_or_s = 0, db_or = 0, db_and = ~0u, u1 = 0, u2 = 0, u3 = 0, dadj = 0, dgprev = 0;
  uint32_t zand = ~0u, zadj = 0, zprev = 0, bm = 0;
  int n = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t s = d[i];
    const uint32_t g = s ^ (s >> 1);
    bx_or_s |= s;
    bx_or |= g;
    bx_and &= g;
    t3 |= t2 & g;
    t2 |= t1 & g;
    t1 |= g;
    adj |= g & gprev;
    gprev = g;

    const bool nzs = s != 0;
    n += nzs ? 1 : 0;
    zand &= nzs ? g : ~0u;
    zadj |= zprev & g;
    zprev = nzs ? g : zprev;

    if (i > 0) {
      const uint32_t p = d[i - 1];
      const uint32_t ld = s - p;
      const uint32_t bo = ((~s & p) | (~(s ^ p) & ld)) & 0x80000000u;
      const uint32_t gd = ld ^ ((ld >> 1) | bo);
      db_or_s |= ld;
      db_or |= gd;
      db_and &= gd;
      u3 |= u2 & gd;
      u2 |= u1 & gd;
      u1 |= gd;
      dadj |= gd & dgprev;
      dgprev = gd;
      bm |= (bo >> 31) << (i - 1);
    }
  }
  const uint32_t single = t1 & ~t2;
  out.sz[kBX] = plane_code_bits(bx_or, bx_and, ~bx_or_s, t2 & ~t3 & adj, single, 32, 32, 5);
  out.sz[kZBX] = 32 + plane_code_bits(bx_or, zand, ~bx_or_s, t2 & ~t3 & zadj, single, 32, n, 5);

  const int bc = popc32(bm);
  const uint64_t dnz = (uint64_t)db_or | ((uint64_t)(bm != 0) << 32);
  const uint64_t dones = (uint64_t)db_and | ((uint64_t)(bm == 0x7FFFFFFFu) << 32);
  const uint64_t dpz = (uint64_t)(~db_or_s);
  const uint64_t dsingle = (uint64_t)(u1 & ~u2) | ((uint64_t)(bc == 1) << 32);
  const uint64_t dpair =
      (uint64_t)(u2 & ~u3 & dadj) | ((uint64_t)(bc == 2 && (bm & (bm >> 1)) != 0) << 32);
  out.sz[kDBX] = 32 + plane_code_bits(dnz, dones, dpz, dpair, dsingle, 33, 31, 5);

  out.sz[kZVC] = 32 + 32 * n;
  out.sz[kRAW] = 1024;
  out.n = n;
  out.bm = bm;
}

template <int W>
PZ_DEV void candidate_sizes(const uint32_t (&d)[32], Sizes &out) {
  if constexpr (W == 16)
    candidate_sizes16(d, out);
  else
    candidate_sizes32(d, out);
}

// Smallest candidate; equal sizes go to the lowest tag.
PZ_DEV int select_tag(const Sizes &s) {
  int best = 0, bsz = s.sz[0];
#pragma unroll
  for (int t = 1; t < 5; ++t) {
    if (s.sz[t] < bsz) {
      best = t;
      bsz = s.sz[t];
    }
  }
  return best;
}

// ---------------------------------------------------------------------------
// Size pass: chunk lengths (pz_compressed_size) and per-block diagnostics.
// ---------------------------------------------------------------------------
template <int W>
__global__ __launch_bounds__(kGroupThreads) void size_kernel(
    const uint8_t *__restrict__ src, uint64_t raw_bytes, uint64_t nchunks,
    uint64_t *__restrict__ out_bytes, uint16_t *__restrict__ chunk_lens,
    uint16_t *__restrict__ block_sizes, uint8_t *__restrict__ block_tags) {
  const uint32_t lane = lane_id();
  const uint64_t tile = (uint64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  if (tile * 2 >= nchunks) return;
  const uint64_t block = tile * kWave + lane;
  const uint64_t off = block * kBlockBytes;
  const bool valid = off < raw_bytes;
  uint32_t d[32];
  load_block(src, raw_bytes, off, d);
  Sizes s;
  candidate_sizes<W>(d, s);
  const int tag = select_tag(s);
  const uint32_t cost = valid ? 3u + (uint32_t)s.sz[tag] : 0u;
  if (valid && block_sizes) {
#pragma unroll
    for (int t = 0; t < 5; ++t) block_sizes[block * 5 + t] = (uint16_t)s.sz[t];
  }
  if (valid && block_tags) block_tags[block] = (uint8_t)tag;

  const uint32_t incl = half_inclusive_scan(cost);
  const uint32_t bits = __shfl(incl, (int)((lane & 32) | 31), 64);
  const uint64_t chunk = block >> 5;
  uint32_t len = 0;
  if (chunk < nchunks) {
    const uint64_t start = chunk * kChunkBytes;
    const uint32_t raw_len = (uint32_t)min<uint64_t>(kChunkBytes, raw_bytes - start);
    len = (bits + 7) / 8;
    if (len >= raw_len) len = raw_len;
  }
  if ((lane & 31) == 0 && chunk < nchunks && chunk_lens) chunk_lens[chunk] = (uint16_t)len;
  const uint64_t sum = (uint64_t)__shfl(len, 0, 64) + (uint64_t)__shfl(len, 32, 64);
  if (lane == 0 && out_bytes) atomicAdd((unsigned long long *)out_bytes, (unsigned long long)sum);
}

// ---------------------------------------------------------------------------
// Plane construction for the chosen encoding.
// ---------------------------------------------------------------------------

// w = 16: from packed symbols (d[i] = sym 2i | sym 2i+1 << 16) to 16 planes of
// 64 bits (bit k of plane j = bit j of symbol k). Symbols k and k+32 are
// paired in one dword first, so that one 32x32 transpose yields the low and
// high halves of every plane.
PZ_DEV void planes_from_symbols16(const uint32_t (&d)[32], uint64_t (&P)[17]) {
  uint32_t e[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const uint32_t a = d[r >> 1], b = d[16 + (r >> 1)];
    const uint32_t lo = (r & 1) ? (a >> 16) : (a & 0xFFFFu);
    const uint32_t hi = (r & 1) ? (b & 0xFFFF0000u) : (b << 16);
    e[r] = lo | hi;
  }
  transpose32(e);
#pragma unroll
  for (int j = 0; j < 16; ++j) P[j] = (uint64_t)e[j] | ((uint64_t)e[j + 16] << 32);
}

// Emits the plane code of P[0..K-1] (K <= KMAX, P[K] treated as zero), top
// plane first: zero runs, all-ones, pre-XOR-zero, pair, single, verbatim.
template <typename PT, int KMAX>
PZ_DEV void emit_plane_code(LdsBitWriter &bw, const PT (&P)[KMAX], int K, int L, int R,
                            bool active) {
  const uint32_t pw = (uint32_t)position_bits(L);
  const PT ones = (PT)all_ones64(L);
  uint32_t run = 0;
  PT above = 0;
#pragma unroll
  for (int j = KMAX - 1; j >= 0; --j) {
    const bool live = active && j < K;
    const PT p = live ? P[j] : (PT)0;
    const PT x = p ^ above;
    above = p;
    if (!live) continue;
    if (x == 0) {
      ++run;
      continue;
    }
    // Pending zero run first, then this plane's code, in one field.
    uint32_t field = 0, flen = 0;
    if (run) {
      if (run == 1) {
        field = 4u;
        flen = 3;
      } else {
        field = 2u | ((run - 2u) << 2);
        flen = 2 + (uint32_t)R;
      }
      run = 0;
    }
    uint32_t code, clen;
    bool verbatim = false;
    const int cnt = sizeof(PT) == 8 ? popc64((uint64_t)x) : popc32((uint32_t)x);
    const uint32_t low = sizeof(PT) == 8 ? (uint32_t)__builtin_ctzll((uint64_t)x)
                                         : (uint32_t)__builtin_ctz((uint32_t)x);
    if (x == ones) {
      code = 0u;
      clen = 5;
    } else if (p == 0) {
      code = 16u;
      clen = 5;
    } else if (cnt == 2 && (x >> low) == (PT)3) {
      code = 8u | (low << 5);
      clen = 5 + pw;
    } else if (cnt == 1) {
      code = 24u | (low << 5);
      clen = 5 + pw;
    } else {
      code = 1u;
      clen = 1;
      verbatim = true;
    }
    bw.put(field | (code << flen), flen + clen);
    if (verbatim) bw.put64((uint64_t)x, (uint32_t)L);
  }
  if (active && run) {
    if (run == 1)
      bw.put(4u, 3);
    else
      bw.put(2u | ((run - 2u) << 2), 2 + (uint32_t)R);
  }
}

// ---------------------------------------------------------------------------
// Single-pass compression.
// ---------------------------------------------------------------------------
template <int W>
__global__ __launch_bounds__(kGroupThreads) void compress_kernel(
    const uint8_t *__restrict__ src, uint64_t raw_bytes, uint64_t nchunks, uint64_t ntiles,
    uint8_t *__restrict__ dst, uint64_t *__restrict__ out_bytes, uint64_t *status,
    uint32_t *tile_counter) {
  constexpr int N = 1024 / W;
  constexpr int R = W == 16 ? 4 : 5;
  constexpr int KMAX = W + 1;
  using PT = typename std::conditional<W == 16, uint64_t, uint32_t>::type;
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[kWavesPerGroup * kWaveLdsDwords];
  uint32_t *lds = lds_all + (threadIdx.x >> 6) * kWaveLdsDwords;

  const uint32_t lane = lane_id();
  const uint32_t tile = acquire_tile(tile_counter);
  if (tile >= ntiles) return;

  const uint32_t half = lane >> 5;
  const uint64_t block = (uint64_t)tile * kWave + lane;
  const uint64_t chunk = block >> 5;
  const uint64_t off = block * kBlockBytes;
  const bool valid = off < raw_bytes;

  uint32_t d[32];
  load_block(src, raw_bytes, off, d);
  Sizes s;
  candidate_sizes<W>(d, s);
  const int tag = select_tag(s);
  const uint32_t cost = valid ? 3u + (uint32_t)s.sz[tag] : 0u;

  // Chunk assembly: bit offsets of the blocks, chunk length, raw decision.
  const uint32_t incl = half_inclusive_scan(cost);
  const uint32_t excl = incl - cost;
  const uint32_t bits = __shfl(incl, (int)((lane & 32) | 31), 64);
  uint32_t raw_len = 0, len = 0;
  if (chunk < nchunks) {
    raw_len = (uint32_t)min<uint64_t>(kChunkBytes, raw_bytes - chunk * kChunkBytes);
    len = (bits + 7) / 8;
    if (len >= raw_len) len = raw_len;
  }
  const bool raw_chunk = len == raw_len;
  const uint32_t len0 = __shfl(len, 0, 64), len1 = __shfl(len, 32, 64);

  // Device-wide offsets of this wave's two payloads.
  const uint64_t before = lookback(status, tile, (uint64_t)len0 + len1);
  const uint64_t pay_off = 2 * nchunks + before + (half ? len0 : 0);
  if ((lane & 31) == 0 && chunk < nchunks) reinterpret_cast<uint16_t *>(dst)[chunk] = (uint16_t)len;
  if (tile == ntiles - 1 && lane == 0) *out_bytes = 2 * nchunks + before + len0 + len1;

  // --- ZBX: move the non-zero symbols to the front (through LDS). ---
  const bool coded = valid && !raw_chunk;
  const bool want_planes = coded && (tag == kDBX || tag == kBX || tag == kZBX);
  const bool want_zbx = coded && tag == kZBX;
  uint32_t cd[32];
  if (__ballot(want_zbx)) {
    uint32_t *region = lds + lane * kLaneStride;
    if (want_zbx) {
#pragma unroll
      for (int i = 0; i < 32; ++i) region[i] = 0;
    }
    wave_lds_fence();
    if (want_zbx) {
      uint32_t k = 0;
      if constexpr (W == 16) {
        uint16_t *r16 = reinterpret_cast<uint16_t *>(region);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t a = d[i] & 0xFFFFu, b = d[i] >> 16;
          if (a) r16[k++] = (uint16_t)a;
          if (b) r16[k++] = (uint16_t)b;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if (d[i]) region[k++] = d[i];
      }
    }
    wave_lds_fence();
#pragma unroll
    for (int i = 0; i < 32; ++i) cd[i] = want_zbx ? region[i] : 0u;
    wave_lds_fence();
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) cd[i] = 0;
  }

  // --- Zero the two chunk buffers. ---
  {
    uint4 *z = reinterpret_cast<uint4 *>(lds);
    for (int i = (int)lane; i < (2 * kChunkBufDwords) / 4; i += kWave) z[i] = make_uint4(0, 0, 0, 0);
  }
  wave_lds_fence();

  // --- Emit this lane's block into its chunk buffer. ---
  uint32_t *cbuf = lds + half * kChunkBufDwords;
  const uint32_t lead = 8u * (uint32_t)(pay_off & 3);
  LdsBitWriter bw;
  bw.init(cbuf, lead + (raw_chunk ? 1024u * (lane & 31) : excl));
  if (coded) bw.put((uint32_t)tag, 3);

  const bool want_raw = valid && (raw_chunk || tag == kRAW);
  if (__ballot(want_raw)) {
    if (want_raw) {
#pragma unroll
      for (int i = 0; i < 32; ++i) bw.put(d[i], 32);
    }
  }

  // Non-zero mask (ZVC and ZBX prefix), bit i = symbol i non-zero.
  const bool want_zvc = coded && tag == kZVC;
  uint64_t nzmask = 0;
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
  if (__ballot(want_zvc)) {
    if (want_zvc) {
      bw.put64(nzmask, N);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if constexpr (W == 16) {
          const uint32_t a = d[i] & 0xFFFFu, b = d[i] >> 16;
          if (a) bw.put(a, 16);
          if (b) bw.put(b, 16);
        } else {
          if (d[i]) bw.put(d[i], 32);
        }
      }
    }
  }

  if (__ballot(want_planes)) {
    // Prefix fields.
    if (want_planes && tag == kDBX) bw.put(W == 16 ? (d[0] & 0xFFFFu) : d[0], W);
    if (want_zbx) bw.put64(nzmask, N);
    // Transpose input: symbols (BX), compacted symbols (ZBX) or deltas (DBX).
    uint32_t e[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      uint32_t delta;
      if constexpr (W == 16) {
        const uint32_t prevp = i == 0 ? (d[0] << 16) : funnel(d[i], d[i - 1], 16);
        delta = pk_sub_u16(d[i], prevp);
        if (i == 0) delta &= 0xFFFF0000u;
      } else {
        delta = i == 0 ? 0u : d[i] - d[i - 1];
      }
      e[i] = tag == kDBX ? delta : (tag == kZBX ? cd[i] : d[i]);
    }
    PT P[KMAX];
    if constexpr (W == 16) {
      planes_from_symbols16(e, P);
    } else {
      transpose32(e);
#pragma unroll
      for (int j = 0; j < 32; ++j) P[j] = e[j];
    }
    int K = W, L = N;
    if (tag == kDBX) {
      // Delta k sits at bit k; plane element k-1 is delta k.
#pragma unroll
      for (int j = 0; j < W; ++j) P[j] >>= 1;
      P[W] = (PT)s.bm;
      K = W + 1;
      L = N - 1;
    } else {
      P[W] = 0;
      if (tag == kZBX) L = s.n;
    }
    emit_plane_code<PT, KMAX>(bw, P, K, L, R, want_planes);
  }
  if (valid) bw.flush();
  wave_lds_fence();

  // --- Store both payloads: LDS byte i goes to dst byte (pay_off & ~3) + i. ---
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint64_t poff = __shfl(pay_off, h * 32, 64);
    const uint32_t plen = h ? len1 : len0;
    if (plen == 0) continue;
    const uint32_t sh = (uint32_t)(poff & 3);
    const uint64_t gbase = poff - sh;
    const uint32_t total = sh + plen;
    const uint32_t ndw = (total + 3) / 4;
    const uint32_t *buf = lds + h * kChunkBufDwords;
    for (uint32_t i = lane; i < ndw; i += kWave) {
      const uint32_t v = buf[i];
      const uint32_t b0 = 4 * i, b1 = 4 * i + 4;
      if (b0 >= sh && b1 <= total) {
        *reinterpret_cast<uint32_t *>(dst + gbase + b0) = v;
      } else {
#pragma unroll
        for (uint32_t b = 0; b < 4; ++b) {
          const uint32_t k = b0 + b;
          if (k >= sh && k < total) dst[gbase + k] = (uint8_t)(v >> (8 * b));
        }
      }
    }
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

hipError_t launch_size(int w, const uint8_t *src, uint64_t raw_bytes, uint64_t *out_bytes,
                       uint16_t *chunk_lens, uint16_t *block_sizes, uint8_t *block_tags,
                       hipStream_t stream) {
  const uint64_t nchunks = (raw_bytes + kChunkBytes - 1) / kChunkBytes;
  if (out_bytes) {
    hipError_t e = fill_u64(out_bytes, 1, 2 * nchunks, stream);
    if (e != hipSuccess) return e;
  }
  if (nchunks == 0) return hipSuccess;
  const uint64_t ntiles = (nchunks + 1) / 2;
  const uint64_t groups = (ntiles + kWavesPerGroup - 1) / kWavesPerGroup;
  if (w == 16)
    hipLaunchKernelGGL(size_kernel<16>, dim3((unsigned)groups), dim3(kGroupThreads), 0, stream,
                       src, raw_bytes, nchunks, out_bytes, chunk_lens, block_sizes, block_tags);
  else
    hipLaunchKernelGGL(size_kernel<32>, dim3((unsigned)groups), dim3(kGroupThreads), 0, stream,
                       src, raw_bytes, nchunks, out_bytes, chunk_lens, block_sizes, block_tags);
  return hipGetLastError();
}

hipError_t launch_compress(int w, const uint8_t *src, uint64_t raw_bytes, uint8_t *dst,
                           uint64_t *out_bytes, hipStream_t stream) {
  const uint64_t nchunks = (raw_bytes + kChunkBytes - 1) / kChunkBytes;
  if (nchunks == 0) return fill_u64(out_bytes, 1, 0, stream);
  const uint64_t ntiles = (nchunks + 1) / 2;
  const uint64_t groups = (ntiles + kWavesPerGroup - 1) / kWavesPerGroup;
  // Scratch: one look-back status word per tile, then the tile counter.
  const size_t words = (size_t)ntiles + 1;
  uint64_t *scratch = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void **>(&scratch), words * sizeof(uint64_t), stream);
  if (e != hipSuccess) return e;
  e = fill_u64(scratch, words, 0, stream);
  if (e == hipSuccess) {
    uint32_t *counter = reinterpret_cast<uint32_t *>(scratch + ntiles);
    if (w == 16)
      hipLaunchKernelGGL(compress_kernel<16>, dim3((unsigned)groups), dim3(kGroupThreads), 0,
                         stream, src, raw_bytes, nchunks, ntiles, dst, out_bytes, scratch, counter);
    else
      hipLaunchKernelGGL(compress_kernel<32>, dim3((unsigned)groups), dim3(kGroupThreads), 0,
                         stream, src, raw_bytes, nchunks, ntiles, dst, out_bytes, scratch, counter);
    e = hipGetLastError();
  }
  hipError_t f = hipFreeAsync(scratch, stream);
  return e != hipSuccess ? e : f;
}

}  // namespace pz
