// PlaneZip compression on gfx950.
//
// Method: PlaneZip paper, §III-A "Codec" and "Stream format", Fig. 2. A
// 128-byte block holds N w-bit symbols (N = 64 for w = 16, 32 for w = 32);
// its ZVC, DBX, BX, ZBX and verbatim encodings are sized and the shortest is
// kept behind a 3-bit tag; each 32 blocks make a chunk with a 16-bit length
// header, and a chunk that does not shrink is kept raw. Bit layout:
// FORMAT.md version 1.
//
// Mapping to the hardware: one lane owns one 128-byte block, so a wave holds
// two 4 KB chunks. A lane sizes the four plane encodings without transposing:
// the XORed planes of BX are the bit-planes of s ^ (s >> 1), so "plane j is
// zero / all ones / holds one 1 / holds two adjacent 1s" are OR, AND, a
// saturating per-bit population count and an adjacency OR over the block's
// symbols, evaluated on all planes at once. For w = 16 a register holds
// symbols i and i + 32 (the "split" layout), so that neighbouring symbols sit
// in neighbouring registers at the same bit positions and one packed 16-bit
// subtraction yields two of DBX's deltas. Only the chosen encoding is
// transposed (a 32x32 bit-matrix butterfly in registers) and emitted: each
// code is OR-ed into a per-chunk LDS buffer at its bit offset. Planes that
// every lane of a wave codes verbatim, or that are zero in every lane, take
// short uniform paths; the others go through a branch-free classifier. Chunk
// offsets come from a single-pass decoupled look-back over per-workgroup
// stream lengths, so the input is read once and the stream written once.
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
    // The tensor's last block: the 16-byte units that hold some of its n
    // bytes, with the bytes past n cleared. (A 16-byte aligned unit never
    // crosses a page, so a unit holding a byte of the tensor can be read.)
    const uint32_t n = off < raw_bytes ? (uint32_t)(raw_bytes - off) : 0u;
    const uint4 *p = reinterpret_cast<const uint4 *>(src + off);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (16u * q < n) v = p[q];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t b = 16u * q + 4u * j;  // first byte of the dword
        const uint32_t keep = n > b ? n - b : 0u;
        d[4 * q + j] = keep >= 4u ? w[j] : w[j] & ((1u << (8u * keep)) - 1u);
      }
    }
  }
}

PZ_DEV uint32_t lo16(uint32_t x) { return x & 0xFFFFu; }
PZ_DEV uint32_t hi16(uint32_t x) { return x >> 16; }

// Both 16-bit halves shifted right by one (bits 15 and 31 become zero).
PZ_DEV uint32_t pk_shr1(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, x) >> (unsigned short)1);
}

// One v_bitop3_b32: bit i of the result is IMM's bit (4 a_i + 2 b_i + c_i),
// so an IMM is written as the function applied to a = 0xF0, b = 0xCC,
// c = 0xAA. (Spelled out, some of the statistics below were compiled into
// two or three instructions each.)
template <uint32_t IMM>
PZ_DEV uint32_t b3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, IMM);
}
constexpr uint32_t kAnd3 = 0xF0 & 0xCC & 0xAA;            // a & b & c
constexpr uint32_t kOrAnd = 0xF0 | (0xCC & 0xAA);         // a | (b & c)
constexpr uint32_t kCount0 = (0xF0 ^ 0xCC) | (0xF0 & 0xAA);  // (a ^ b) | (a & c)
constexpr uint32_t kCount1 = (0xF0 & 0xCC) | 0xAA;        // (a & b) | c
constexpr uint32_t kBorrow = (~0xF0 & 0xCC) | (~(0xF0 ^ 0xCC) & 0xAA);  // borrow out of a - b = c
constexpr uint32_t kSelect = (0xF0 & 0xCC) | (~0xF0 & 0xAA);  // a ? b : c, bitwise

// w = 16: the natural layout holds symbols 2q and 2q+1 in dword q; the split
// layout holds symbol i in the low half of dword i and symbol i + 32 in its
// high half.
PZ_DEV void to_split16(uint32_t (&d)[32]) {
  uint32_t s[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    s[i] = __builtin_amdgcn_perm(d[16 + (i >> 1)], d[i >> 1], (i & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
  for (int i = 0; i < 32; ++i) d[i] = s[i];
}

// Number of non-zero symbols of a block (either layout).
template <int W>
PZ_DEV uint32_t count_nonzero(const uint32_t (&d)[32]) {
  if constexpr (W == 16) {
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 32; i += 2)
      cnt = cnt + pk_min_u16(d[i], 0x00010001u) + pk_min_u16(d[i + 1], 0x00010001u);
    return lo16(cnt) + hi16(cnt);
  } else {
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) cnt += d[i] != 0 ? 1u : 0u;
    return cnt;
  }
}

// Per-bit population count saturating at 3, over the values fed to it: the
// pair (c0, c1) reads 0 = (0,0), 1 = (1,0), 2 = (0,1), 3 or more = (1,1).
PZ_DEV void count4(uint32_t &c0, uint32_t &c1, uint32_t g) {
  const uint32_t n0 = b3<kCount0 & 0xFF>(c0, g, c1);  // (c0 ^ g) | (c0 & c1)
  c1 = b3<kCount1 & 0xFF>(c0, g, c1);                 // (c0 & g) | c1
  c0 = n0;
}

// Per-plane "at least 1 / 2 / 3 ones" of a w = 16 counter whose two halves
// count symbols 0..31 and 32..63 of the same plane.
PZ_DEV void fold4_16(uint32_t c0, uint32_t c1, uint32_t &ge1, uint32_t &ge2, uint32_t &ge3) {
  const uint32_t a = c0 | c1, b = c1, c = c0 & c1;
  ge1 = lo16(a) | hi16(a);
  ge2 = lo16(b) | hi16(b) | (lo16(a) & hi16(a));
  ge3 = lo16(c) | hi16(c) | (lo16(b) & hi16(a)) | (lo16(a) & hi16(b));
}

// ---------------------------------------------------------------------------
// Plane-code size from per-plane class masks (bit j describes plane j):
// nz: XORed plane non-zero; ones: XORed plane all ones; pz: plane before the
// XOR is zero; pair: exactly two adjacent ones; single: exactly one one.
// Codes of §III-A: a lone zero plane 3 bits, a run of zero planes 2+R bits,
// all-ones and pre-XOR-zero planes 5 bits, pair and single 5 + PW bits, any
// other plane 1 + L bits; the first matching class wins, in that order. Also
// returns the masks of the verbatim and of the zero planes.
// ---------------------------------------------------------------------------
PZ_DEV int plane_code_bits(uint64_t nz, uint64_t ones, uint64_t pz, uint64_t pair, uint64_t single, int K,
                           int L, int R, uint64_t &verb, uint64_t &zero) {
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
  verb = e;
  zero = z;
  return 5 * popc64(a | b) + (5 + pw) * popc64(cd) + (1 + L) * popc64(e) + 3 * lones + (2 + R) * (runs - lones);
}

// What the statistics of a block give the selection and the emission: the
// five candidate sizes (payload bits, no tag), and for the plane encodings
// (index 0 DBX, 1 BX, 2 ZBX) the masks of their verbatim and zero planes;
// and DBX's top plane (the borrows of the deltas).
struct Stats {
  int sz[5];
  uint64_t verb[3];
  uint64_t zero[3];
  uint32_t bm_lo, bm_hi;
};

// ---------------------------------------------------------------------------
// Candidate sizes, w = 16, split layout: d[i] holds symbols i (low half) and
// i + 32 (high half). DBX's deltas are taken as delta[k] = s[k] - s[k-1] in
// the arrangement (delta[i+1], delta[i+33]) = d[i+1] - d[i], so that the
// register of delta k+1 is the one the transpose turns into plane bit k.
// zbx (wave-uniform) is false when no lane of the wave holds a block with
// 0 < n < 64: then ZBX compacts nothing away and its size is the mask plus
// the BX size.
// ---------------------------------------------------------------------------
PZ_DEV void candidate_sizes16(const uint32_t (&d)[32], int n, bool zbx, Stats &o) {
  uint32_t os = 0, an = ~0u, c0 = 0, c1 = 0, aj = 0, gp = 0, g0 = 0;
  uint32_t dos = 0, dan = ~0u, e0 = 0, e1 = 0, daj = 0, dp = 0, dg0 = 0, bw0 = 0, bw1 = 0;
  const uint32_t s32 = hi16(d[0]);
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    uint32_t g[2], gd[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = i + h;
      const uint32_t s = d[k];
      // BX: the XORed planes are the bit-planes of s ^ (s >> 1) per symbol.
      g[h] = s ^ pk_shr1(s);
      count4(c0, c1, g[h]);
      if (k == 0)
        g0 = g[h];
      else
        aj = b3<kOrAnd & 0xFF>(aj, g[h], gp);  // symbols (k-1, k) and (k+31, k+32)
      gp = g[h];
      // DBX: deltas (k+1, k+33) as 17-bit two's complement; the low 16 bits
      // come from a packed subtraction, bit 16 is the borrow (bits 15 and
      // 31 of bo). The XORed planes are the bits of D ^ (D >> 1). The last
      // register holds delta 32 (symbol 32 - symbol 31) alone.
      const uint32_t cur = k < 31 ? d[k + 1] : s32;
      const uint32_t prv = k < 31 ? s : lo16(s);
      const uint32_t ld = pk_sub_u16(cur, prv);
      const uint32_t bo = b3<kBorrow & 0xFF>(cur, prv, ld);
      gd[h] = ld ^ b3<kSelect & 0xFF>(0x80008000u, bo, pk_shr1(ld));
      count4(e0, e1, gd[h]);
      if (k == 0)
        dg0 = gd[h];
      else
        daj = b3<kOrAnd & 0xFF>(daj, gd[h], dp);
      dp = gd[h];
      dos |= ld;
      // Borrow bits, shifted in from the top: bw0 bit k = borrow of delta
      // k+1, bit 16+k = borrow of delta k+33 (k < 16); bw1 likewise for 16..31.
      if (k < 16)
        bw0 = b3<kOrAnd & 0xFF>(bw0 >> 1, bo, 0x80008000u);
      else
        bw1 = b3<kOrAnd & 0xFF>(bw1 >> 1, bo, 0x80008000u);
    }
    os = os | d[i] | d[i + 1];
    an = b3<kAnd3 & 0xFF>(an, g[0], g[1]);
    // The high half of the last register holds no delta: all ones for the AND.
    dan = b3<kAnd3 & 0xFF>(dan, gd[0], i + 1 == 31 ? (gd[1] | 0xFFFF0000u) : gd[1]);
  }
  aj |= gp & (g0 >> 16);    // symbols 31 and 32 (low half of gp, high half of g0)
  daj |= dp & (dg0 >> 16);  // deltas 32 and 33

  uint32_t ge1, ge2, bge3;
  // BX: 16 planes of 64 bits.
  fold4_16(c0, c1, ge1, ge2, bge3);
  const uint32_t nz = ge1, single = ge1 & ~ge2;
  const uint32_t pair = (lo16(aj) | hi16(aj)) & ~bge3;
  const uint32_t ones = lo16(an) & hi16(an);
  const uint32_t pz = ~(lo16(os) | hi16(os)) & 0xFFFFu;
  o.sz[kBX] = plane_code_bits(nz, ones, pz, pair, single, 16, 64, 4, o.verb[1], o.zero[1]);

  // DBX: base, then 17 planes of 63 bits; plane 16 is the borrow plane.
  uint32_t dge1, dge2, dge3;
  fold4_16(e0, e1, dge1, dge2, dge3);
  uint64_t dnz = dge1, dsingle = dge1 & ~dge2;
  uint64_t dpair = (lo16(daj) | hi16(daj)) & ~dge3;
  uint64_t dones = lo16(dan) & hi16(dan);
  const uint64_t dpz = ~(lo16(dos) | hi16(dos)) & 0xFFFFu;
  const uint32_t bl = __builtin_amdgcn_perm(bw1, bw0, 0x05040100u);  // plane bits 0..31
  const uint32_t bh = __builtin_amdgcn_perm(bw1, bw0, 0x07060302u);  // plane bits 32..63
  const int bc = popc32(bl) + popc32(bh);
  const bool badj = ((bl & (bl >> 1)) | (bh & (bh >> 1)) | ((bl >> 31) & bh & 1u)) != 0;
  dnz |= (uint64_t)(bc != 0) << 16;
  dones |= (uint64_t)(bc == 63) << 16;
  dsingle |= (uint64_t)(bc == 1) << 16;
  dpair |= (uint64_t)(bc == 2 && badj) << 16;
  o.sz[kDBX] = 16 + plane_code_bits(dnz, dones, dpz, dpair, dsingle, 17, 63, 4, o.verb[0], o.zero[0]);
  o.bm_lo = bl;
  o.bm_hi = bh;

  // ZBX: the zero, count and pre-XOR masks are those of BX (zero symbols add
  // nothing); "all ones" and adjacency run over the non-zero symbols only,
  // in order: symbols 0..31 (low halves), then 32..63 (high halves).
  if (zbx) {
    uint32_t zan = ~0u, zaj = 0, zp = 0, zf = 0, seen = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t s = d[i];
      const uint32_t g = s ^ pk_shr1(s);
      const uint32_t zfill = pk_sub_u16(pk_min_u16(s, 0x00010001u), 0x00010001u);  // 0xFFFF if zero
      zan &= g | zfill;
      zaj |= zp & g;                      // last non-zero symbol before this one
      zp = (zp & zfill) | g;
      zf |= g & ~seen;                    // first non-zero symbol of each half
      seen |= ~zfill;
    }
    zaj |= zp & (zf >> 16);  // last non-zero of 0..31 and first of 32..63
    const uint32_t zpair = (lo16(zaj) | hi16(zaj)) & ~bge3;
    o.sz[kZBX] = 64 + plane_code_bits(nz, lo16(zan) & hi16(zan), pz, zpair, single, 16, n, 4, o.verb[2],
                                      o.zero[2]);
  } else {
    o.sz[kZBX] = 64 + o.sz[kBX];
    o.verb[2] = o.verb[1];
    o.zero[2] = o.zero[1];
  }

  o.sz[kZVC] = 64 + 16 * n;
  o.sz[kRAW] = 1024;
}

// ---------------------------------------------------------------------------
// Candidate sizes, w = 32. d[i] is symbol i; delta k+1 = d[k+1] - d[k] is
// plane bit k.
// ---------------------------------------------------------------------------
PZ_DEV void candidate_sizes32(const uint32_t (&d)[32], int n, bool zbx, Stats &o) {
  uint32_t os = 0, an = ~0u, c0 = 0, c1 = 0, aj = 0, gp = 0;
  uint32_t dos = 0, dan = ~0u, e0 = 0, e1 = 0, daj = 0, dp = 0, bacc = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t s = d[i];
    const uint32_t g = s ^ (s >> 1);
    os |= s;
    an &= g;
    count4(c0, c1, g);
    if (i > 0) aj |= g & gp;
    gp = g;
    if (i < 31) {
      const uint32_t cur = d[i + 1];
      const uint32_t ld = cur - s;
      const uint32_t bo = (~cur & s) | (~(cur ^ s) & ld);  // borrow in bit 31
      const uint32_t gd = ld ^ ((ld >> 1) | (bo & 0x80000000u));
      dos |= ld;
      dan &= gd;
      count4(e0, e1, gd);
      if (i > 0) daj |= gd & dp;
      dp = gd;
      bacc = (bacc >> 1) | (bo & 0x80000000u);  // ends with delta k+1's borrow at bit k+1
    }
  }
  const uint32_t bm = bacc >> 1;  // plane bit k = borrow of delta k+1
  const uint32_t ge1 = c0 | c1, ge3 = c0 & c1;
  const uint32_t single = ge1 & ~c1;
  o.sz[kBX] = plane_code_bits(ge1, an, ~os, aj & ~ge3, single, 32, 32, 5, o.verb[1], o.zero[1]);

  if (zbx) {
    uint32_t za = ~0u, zj = 0, zprev = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t s = d[i];
      const uint32_t g = s ^ (s >> 1);
      za &= s != 0 ? g : ~0u;
      zj |= zprev & g;
      zprev = s != 0 ? g : zprev;
    }
    o.sz[kZBX] = 32 + plane_code_bits(ge1, za, ~os, zj & ~ge3, single, 32, n, 5, o.verb[2], o.zero[2]);
  } else {
    o.sz[kZBX] = 32 + o.sz[kBX];
    o.verb[2] = o.verb[1];
    o.zero[2] = o.zero[1];
  }

  const uint32_t dge1 = e0 | e1, dge3 = e0 & e1;
  const int bc = popc32(bm);
  const uint64_t dnz = (uint64_t)dge1 | ((uint64_t)(bm != 0) << 32);
  const uint64_t dones = (uint64_t)dan | ((uint64_t)(bm == 0x7FFFFFFFu) << 32);
  const uint64_t dpz = (uint64_t)(~dos);
  const uint64_t dsingle = (uint64_t)(dge1 & ~e1) | ((uint64_t)(bc == 1) << 32);
  const uint64_t dpair = (uint64_t)(daj & ~dge3) | ((uint64_t)(bc == 2 && (bm & (bm >> 1)) != 0) << 32);
  o.sz[kDBX] = 32 + plane_code_bits(dnz, dones, dpz, dpair, dsingle, 33, 31, 5, o.verb[0], o.zero[0]);
  o.bm_lo = bm;
  o.bm_hi = 0;

  o.sz[kZVC] = 32 + 32 * n;
  o.sz[kRAW] = 1024;
}

template <int W>
PZ_DEV void candidate_sizes(const uint32_t (&d)[32], int n, bool zbx, Stats &out) {
  if constexpr (W == 16)
    candidate_sizes16(d, n, zbx, out);
  else
    candidate_sizes32(d, n, zbx, out);
}

// Smallest allowed candidate (mask bit t = tag t); equal sizes go to the
// lowest tag. Returns the tag and its size (no indexing of the size array by
// a lane-varying tag).
PZ_DEV int select_tag(const Stats &s, int &best_size, uint32_t mask) {
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

// AND of a value over the 64 lanes of the wave (every lane must be active).
PZ_DEV uint32_t wave_and32(uint32_t v) {
  v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad: lanes 1,0,3,2
  v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad: lanes 2,3,0,1
  v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // half-row mirror
  v &= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);  // row mirror
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) & (uint32_t)__builtin_amdgcn_readlane((int)v, 16) &
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) & (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
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
  if constexpr (W == 16) to_split16(d);
  Stats s;
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
// Emission: fields are OR-ed into the zeroed LDS chunk buffer at an explicit
// bit offset (stream bit t = bit t%32 of dword t/32). A write may touch a
// dword past its last bit with a zero value.
// ---------------------------------------------------------------------------
// v (below 2^32) at bit off: dwords off/32 and off/32 + 1.
PZ_DEV void or32(uint32_t *buf, uint32_t off, uint32_t v) {
  uint32_t *p = buf + (off >> 5);
  const uint32_t sh = off & 31u;
  atomicOr(p, v << sh);
  atomicOr(p + 1, (v >> 1) >> (31u - sh));  // v >> (32 - sh); 0 when sh == 0
}

// 64 bits (hi:lo) at bit off: dwords off/32 .. off/32 + 2.
PZ_DEV void or64(uint32_t *buf, uint32_t off, uint32_t lo, uint32_t hi) {
  uint32_t *p = buf + (off >> 5);
  const uint32_t sh = off & 31u;
  const uint64_t v = (((uint64_t)hi << 32) | lo) << sh;
  atomicOr(p, (uint32_t)v);
  atomicOr(p + 1, (uint32_t)(v >> 32));
  atomicOr(p + 2, (hi >> 1) >> (31u - sh));
}

// A verbatim plane code: the bit 1, then the plane (hi:lo) at bit off + 1.
PZ_DEV void or_verbatim(uint32_t *buf, uint32_t off, uint32_t lo, uint32_t hi) {
  uint32_t *p = buf + (off >> 5);
  const uint32_t sh = off & 31u, nsh = 31u - sh;
  atomicOr(p, ((lo << 1) | 1u) << sh);
  atomicOr(p + 1, funnel(hi, lo, nsh));  // bits 32..63 of (plane << (sh + 1))
  atomicOr(p + 2, hi >> nsh);            // bits 64..95
}
PZ_DEV void or_verbatim(uint32_t *buf, uint32_t off, uint32_t x) {
  uint32_t *p = buf + (off >> 5);
  const uint32_t sh = off & 31u;
  atomicOr(p, ((x << 1) | 1u) << sh);
  atomicOr(p + 1, x >> (31u - sh));
}

// Code of a run of `run` zero planes (0: none) and its length: '001' for one
// plane, '01' and run - 2 in R bits for more. Written as arithmetic on
// min(run, 2): as selects on run, the compiler turned it into branches.
template <uint32_t R>
PZ_DEV void run_code(uint32_t run, uint32_t &code, uint32_t &len) {
  const uint32_t m = run < 2u ? run : 2u;  // 0, 1, 2
  const uint32_t two = m >> 1;            // run >= 2
  len = 3u * m + (R - 4u) * two;          // 0, 3, 2 + R
  code = (run << 2) - 6u * two;           // 0, 4, 2 | (run - 2) << 2
}

// One plane, any class, without branches: x is the XORed plane, pz whether
// the plane before the XOR is zero, ones the all-ones value of the plane
// width L, cs = 5 + PW the length of a pair or single code. A zero plane
// extends the pending run; a non-zero one writes the pending run's code and
// its own code, and, if verbatim, the plane itself.
template <typename PT, uint32_t R>
PZ_DEV void emit_plane(uint32_t *buf, uint32_t &off, uint32_t &run, PT x, bool pz, PT ones, uint32_t L,
                       uint32_t cs) {
  uint32_t xlo, xhi;
  if constexpr (sizeof(PT) == 8) {
    xlo = (uint32_t)x;
    xhi = (uint32_t)((uint64_t)x >> 32);
  } else {
    xlo = (uint32_t)x;
    xhi = 0;
  }
  const bool nz = (xlo | xhi) != 0;
  const uint32_t cnt = (uint32_t)popc32(xlo) + (uint32_t)popc32(xhi);
  // Lowest set bit (a zero half gives ffbl = ~0, which min ignores).
  const uint32_t flo = (uint32_t)__ffs(xlo) - 1u, fhi = (uint32_t)__ffs(xhi) - 1u;
  const uint32_t low = sizeof(PT) == 8 ? min(flo, 32u + fhi) : flo;
  const uint32_t tl = (uint32_t)(x >> (low & (8 * sizeof(PT) - 1)));
  // One 1, or two adjacent 1s: cnt minus "bit low+1 set" is then 1.
  const bool shortc = cnt - ((tl >> 1) & 1u) == 1u;
  const bool is_ones = x == ones;
  // Code and length by the first matching class (all ones, pre-XOR zero,
  // pair or single, verbatim).
  uint32_t code = shortc ? ((24u - ((tl & 2u) << 3)) | (low << 5)) : 1u;
  uint32_t clen = shortc ? cs : 1u;
  code = pz ? 16u : code;
  clen = pz ? 5u : clen;
  code = is_ones ? 0u : code;
  clen = is_ones ? 5u : clen;
  uint32_t rcode, rlen;
  run_code<R>(run, rcode, rlen);
  const uint32_t item = nz ? rcode | (code << rlen) : 0u;
  or32(buf, off, item);
  off += nz ? rlen + clen : 0u;
  run = nz ? 0u : run + 1u;
  const bool verb = nz && !(shortc || pz || is_ones);
  if (verb) {
    if constexpr (sizeof(PT) == 8)
      or64(buf, off, xlo, xhi);
    else
      or32(buf, off, xlo);
    off += L;
  }
}

// ---------------------------------------------------------------------------
// Single-pass compression, one workgroup per tile of 8 chunks (256 blocks,
// four waves: four such workgroups fill a CU, whose phases interleave better
// than those of two groups of eight waves).
//
// Softmax-like activations hold many all-zero blocks, and a wave runs the
// candidate statistics and the emission for all its lanes at the cost of
// the slowest. So the group first loads its 256 blocks one per thread,
// gives every all-zero block its fixed code (below), and, when some block is
// all zero, packs the non-zero blocks through LDS into the lowest slots: only
// ceil(nnz / 64) waves then run the statistics and the emission. Chunk
// offsets come from one decoupled look-back per group.
// ---------------------------------------------------------------------------
constexpr int kCWaves = 4;  // waves per compress workgroup
// The second launch bound is the minimum number of waves per SIMD: four caps
// a lane at 128 VGPRs, so that a CU holds the 16 waves above.
constexpr int kCWavesPerSimd = 4;
constexpr int kCThreads = kWave * kCWaves;
constexpr int kGroupChunks = kCThreads / kBlocksPerChunk;
constexpr int kStageDwords = kCThreads * kLaneStride;
constexpr int kGroupBufDwords = kGroupChunks * kChunkBufDwords;
// Load staging: a wave's 64 blocks at stride 36 dwords (16-byte aligned
// slots; lane reads of 16 bytes at that stride cover all 64 banks).
constexpr int kLoadStride = 36;
constexpr int kLoadDwords = kCThreads * kLoadStride;
// LDS of a workgroup: the slots of the packing, the chunk buffers and, for
// 16-bit symbols, the load staging, one after another in time.
constexpr int kGroupLdsDwords = kStageDwords > kGroupBufDwords ? kStageDwords : kGroupBufDwords;
template <int W>
constexpr int group_lds_dwords() {
  return W == 16 && kLoadDwords > kGroupLdsDwords ? kLoadDwords : kGroupLdsDwords;
}

// The 64 blocks of a wave (the 8 KB at byte wave_off of src): lane l loads
// 16-byte units l, l + 64, ..., l + 448 (each load instruction reads 1 KB
// contiguous), stores them into the wave's staging slots, and reads back
// its own block (block l of the wave). Bytes at or past raw_bytes load as
// zeros; a 16-byte aligned unit holding a byte of the tensor is read whole
// (it never crosses a page).
PZ_DEV void load_wave_blocks(const uint8_t *__restrict__ src, uint64_t raw_bytes, uint64_t wave_off,
                             uint32_t *slots, uint32_t lane, uint32_t (&d)[32]) {
  uint4 v[8];
  const uint4 *p = reinterpret_cast<const uint4 *>(src + wave_off);
  if (wave_off + 64 * kBlockBytes <= raw_bytes) {
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = p[lane + 64 * q];
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t u = lane + 64 * q;
      const uint64_t o = wave_off + 16ull * u;
      const uint32_t n = o < raw_bytes ? (uint32_t)min_u64(raw_bytes - o, 16) : 0u;
      uint4 x = make_uint4(0, 0, 0, 0);
      if (n > 0) x = p[u];
      uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t keep = n > 4u * j ? n - 4u * j : 0u;
        w[j] = keep >= 4 ? w[j] : w[j] & ((1u << (8u * keep)) - 1u);
      }
      v[q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t u = lane + 64 * q;
    *reinterpret_cast<uint4 *>(slots + (u >> 3) * kLoadStride + 4 * (u & 7)) = v[q];
  }
  wave_lds_fence();
  const uint4 *mine = reinterpret_cast<const uint4 *>(slots + lane * kLoadStride);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 x = mine[q];
    d[4 * q + 0] = x.x;
    d[4 * q + 1] = x.y;
    d[4 * q + 2] = x.z;
    d[4 * q + 3] = x.w;
  }
}


// An all-zero block under the mode's candidate for it (the smallest allowed;
// BX in PlaneZip): the tag, a zero mask / base / raw block of zero bits
// (already present in the cleared buffer), and for the plane encodings one
// zero run over all planes.
template <int W>
PZ_DEV void emit_zero_block(uint32_t *buf, uint32_t off, const Mode &m) {
  constexpr uint32_t N = 1024 / W, R = W == 16 ? 4 : 5;
  const uint32_t c = m.zc;
  uint32_t v = 0, len = 0;
  if (m.tagged) {
    v = c;
    len = 3;
  }
  len += c == 0 ? N : (c == 1 ? (uint32_t)W : (c == 3 ? N : (c == 4 ? 1024u : 0u)));
  const uint32_t planes = c == 1 ? W + 1 : ((c == 2 || c == 3) ? (uint32_t)W : 0u);
  if (m.tagged) or32(buf, off, v);
  if (planes) or32(buf, off + len, 2u | ((planes - 2u) << 2));
}

// The (ZVC / ZBX) mask of a block: bit k = symbol k non-zero.
template <int W>
PZ_DEV void nonzero_mask(const uint32_t (&d)[32], uint32_t &mlo, uint32_t &mhi) {
  mlo = mhi = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if constexpr (W == 16) {
      const uint32_t z = pk_min_u16(d[i], 0x00010001u);
      mlo |= (z & 1u) << i;
      mhi |= (z >> 16) << i;
    } else {
      mlo |= (uint32_t)(d[i] != 0) << i;
    }
  }
}

// The tensor of a launch's tile (the last one whose first tile is at or
// before it: a tensor without chunks has no tiles).
PZ_DEV uint32_t tensor_of(const CBatch &batch, uint32_t gtile) {
  uint32_t k = 0;
  if (batch.n > 1) {  // a single tensor's fields load at once
#pragma unroll
    for (uint32_t i = 1; i < (uint32_t)kMaxBatch; ++i) k += i < batch.n && gtile >= batch.t[i].tile_begin ? 1u : 0u;
  }
  return k;
}

// Block t of the launch's tile gtile, into registers.
PZ_DEV void load_tile_block(const CBatch &batch, uint32_t gtile, uint32_t t, uint32_t (&d)[32]) {
  const uint32_t k = tensor_of(batch, gtile);
  const uint64_t block = (uint64_t)(gtile - batch.t[k].tile_begin) * kCThreads + t;
  load_block(batch.t[k].src, batch.t[k].raw_bytes, block * kBlockBytes, d);
}

template <int W>
__global__ __launch_bounds__(kCThreads, kCWavesPerSimd) void compress_kernel(const CBatch batch, uint64_t *lb_words,
                                                                 uint32_t *tile_counter, uint32_t counter_base,
                                                                 uint32_t epoch, Mode mode) {
  constexpr int N = 1024 / W;
  constexpr uint32_t R = W == 16 ? 4 : 5;
  constexpr int KT = W;  // index of DBX's top plane (the borrow plane) in the plane masks
  using PT = typename std::conditional<W == 16, uint64_t, uint32_t>::type;
  // Staging slots / compaction regions (stride kLaneStride), later the
  // chunk buffers.
  __shared__ __attribute__((aligned(16))) uint32_t lds[group_lds_dwords<W>()];
  __shared__ uint16_t blk_bits[kCThreads];    // per block: its cost, then its bit offset
  __shared__ uint16_t slot_block[kCThreads];  // compacted slot -> block of the group
  __shared__ uint8_t slot_n[kCThreads];       // compacted slot -> its non-zero symbols
  __shared__ uint32_t wave_full[kCWaves];
  __shared__ uint32_t wave_part[kCWaves];
  __shared__ uint32_t chunk_len[kGroupChunks];
  __shared__ uint64_t chunk_pay[kGroupChunks];
  __shared__ uint32_t group_tile;
  __shared__ uint32_t done_waves;  // waves done with the emission

  const uint32_t t = threadIdx.x, lane = lane_id();
  const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: a scalar
  if (t == 0) group_tile = atomicAdd(tile_counter, 1u) - counter_base;
  __syncthreads();
  // The launch's tile -> the tensor it belongs to and the tile within it.
  const uint32_t gtile = __builtin_amdgcn_readfirstlane(group_tile);
  if (gtile >= batch.total_tiles) return;
  const uint32_t k = tensor_of(batch, gtile);
  const uint8_t *__restrict__ src = batch.t[k].src;
  uint8_t *__restrict__ dst = batch.t[k].dst;
  const uint64_t raw_bytes = batch.t[k].raw_bytes, nchunks = batch.t[k].nchunks;
  const uint32_t ntiles = batch.t[k].ntiles;
  const uint32_t tile = gtile - batch.t[k].tile_begin;
  uint64_t *status = lb_words + (uint64_t)batch.t[k].tile_begin * kLookbackStride;
  uint32_t d[32];
  // 16-bit symbols: coalesced loads staged through LDS (a lane's own
  // 128-byte block, read directly, puts 64 cache lines behind every load
  // instruction and stalls the address path: this made compress 2% faster
  // on the GPT-2 tensors). 32-bit symbols keep the direct loads (the staged
  // form took two more VGPRs and was 2% slower on the FP32 CNN tensor).
  if constexpr (W == 16)
    load_wave_blocks(src, raw_bytes, ((uint64_t)tile * kCThreads + 64u * wave) * kBlockBytes,
                     lds + wave * 64u * kLoadStride, lane, d);
  else
    load_tile_block(batch, gtile, t, d);

  // --- 1. Count block t's non-zero symbols (loaded before). ---
  const uint64_t block = (uint64_t)tile * kCThreads + t;
  const bool valid = block * kBlockBytes < raw_bytes;
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

  // --- 2. Slots. When some block is all zero, or full and partial blocks
  // (those with a zero symbol) are mixed, the non-zero blocks are packed
  // through LDS into slots 0..nnz-1, full blocks first, so that the
  // statistics (and ZBX's, needed only when 0 < n < N) run on as few waves
  // as possible. Otherwise every thread keeps its own block. ---
  uint32_t nfull = 0, npart = 0, ffirst = 0, pfirst = 0;
#pragma unroll
  for (int q = 0; q < kCWaves; ++q) {
    const uint32_t f = wave_full[q], p = wave_part[q];
    ffirst += (uint32_t)q < wave ? f : 0u;
    pfirst += (uint32_t)q < wave ? p : 0u;
    nfull += f;
    npart += p;
  }
  const uint32_t nnz = nfull + npart;
  const bool staged = !(nnz == (uint32_t)kCThreads && (npart == 0 || nfull == 0));
  if (staged) {
    if (nonzero) {
      const uint32_t idx = partial ? nfull + pfirst + lanes_below(mpart) : ffirst + lanes_below(mfull);
      uint32_t *slotp = lds + idx * kLaneStride;
#pragma unroll
      for (int i = 0; i < 32; ++i) slotp[i] = d[i];
      slot_block[idx] = (uint16_t)t;
      slot_n[idx] = (uint8_t)sn;
    }
    __syncthreads();
  }

  // Waves take the slots in an order rotated per tile, so that the busy
  // waves of successive groups fall on different SIMDs.
  const uint32_t slot = staged ? (t + kCThreads - 64u * (tile & (kCWaves - 1u))) & (kCThreads - 1) : t;
  const bool active = slot < nnz;
  const bool wave_active = __ballot(active) != 0;
  const uint32_t sblock = staged ? (active ? (uint32_t)slot_block[slot] : 0u) : t;  // the slot's block

  // --- 3. Sizes, selection and the transform input of the slot's block. ---
  int tag = kRAW;
  uint32_t bm_lo = 0, bm_hi = 0, mlo = 0, mhi = 0, base = 0;
  uint64_t fv = ~0ull, zr = ~0ull;  // this lane's fast-verbatim and zero plane masks
  uint32_t e[32];
  if (wave_active) {
    uint32_t *region = lds + slot * kLaneStride;
    if (staged) {
      sn = active ? (uint32_t)slot_n[slot] : 0u;
      if (active) {
#pragma unroll
        for (int i = 0; i < 32; ++i) d[i] = region[i];
      }
    }
    if constexpr (W == 16) to_split16(d);
    const bool zbx = __ballot(active && sn < (uint32_t)N) != 0;  // active blocks are non-zero
    Stats s;
    candidate_sizes<W>(d, (int)sn, zbx, s);
    int best_size;
    tag = select_tag(s, best_size, mode.mask);
    if (active) blk_bits[sblock] = (uint16_t)(3u * mode.tagged + best_size);
    if (!active) tag = kRAW;  // inactive lanes code nothing
    bm_lo = s.bm_lo;
    bm_hi = s.bm_hi;

    // Fast-path masks: plane j (bit j; bit KT = DBX's top plane) is verbatim
    // with no zero run pending above it, or zero.
    if (active && (tag == kDBX || tag == kBX || tag == kZBX)) {
      const int ci = tag == kDBX ? 0 : (tag == kBX ? 1 : 2);
      const uint64_t vb = ci == 0 ? s.verb[0] : (ci == 1 ? s.verb[1] : s.verb[2]);
      const uint64_t zo = ci == 0 ? s.zero[0] : (ci == 1 ? s.zero[1] : s.zero[2]);
      fv = vb & ~(zo >> 1);
      zr = zo;
      if (tag != kDBX) {
        fv |= 1ull << KT;
        zr |= 1ull << KT;
      }
    }

    const bool want_zvc = active && tag == kZVC;
    const bool want_dbx = active && tag == kDBX;
    const bool want_zbx = active && tag == kZBX;
    const bool want_cmp = want_zbx || want_zvc;
    if (__ballot(want_cmp)) {
      if (want_cmp) nonzero_mask<W>(d, mlo, mhi);
    }
    base = W == 16 ? lo16(d[0]) : d[0];

    // ZBX and ZVC: the non-zero symbols, in order, at the front of this
    // slot's region (the slot was read above; no other thread touches it).
    const bool any_cmp = __ballot(want_cmp) != 0;
    if (any_cmp) {
      if (want_cmp) {
#pragma unroll
        for (int i = 0; i < 33; ++i) region[i] = 0;
      }
      wave_lds_fence();
      if (want_cmp) {
        // Every symbol is written at the current rank, which advances only
        // past non-zero ones: a zero symbol writes 0 where the next non-zero
        // symbol (or nothing) goes, so there are no branches.
        uint32_t r = 0;
        if constexpr (W == 16) {
          uint16_t *r16 = reinterpret_cast<uint16_t *>(region);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
              const uint32_t a = h ? hi16(d[i]) : lo16(d[i]);
              r16[r] = (uint16_t)a;
              r += a ? 1u : 0u;
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            region[r] = d[i];
            r += d[i] ? 1u : 0u;
          }
        }
      }
      wave_lds_fence();
    }

    // Transform input, in place: the symbols (BX), the deltas (DBX), the
    // compacted symbols (ZBX: split layout for w = 16; ZVC: in order).
    if (__ballot(want_dbx)) {
      const uint32_t s32 = hi16(d[0]);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        uint32_t v;
        if constexpr (W == 16)
          v = i < 31 ? pk_sub_u16(d[i + 1], d[i]) : lo16(s32 - lo16(d[31]));
        else
          v = i < 31 ? d[i + 1] - d[i] : 0u;
        d[i] = want_dbx ? v : d[i];
      }
    }
    if (any_cmp) {
#pragma unroll
      for (int i = 0; i < 32; ++i) e[i] = region[i];
      if constexpr (W == 16) {
        if (__ballot(want_zbx)) {
          uint32_t sp[32];
#pragma unroll
          for (int i = 0; i < 32; ++i) sp[i] = e[i];
          to_split16(sp);
#pragma unroll
          for (int i = 0; i < 32; ++i) e[i] = want_zbx ? sp[i] : e[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) d[i] = want_cmp ? e[i] : d[i];
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) e[i] = d[i];
  }
  const uint64_t FV = W == 16 ? (uint64_t)wave_and32((uint32_t)fv)
                              : ((uint64_t)wave_and32((uint32_t)(fv >> 32)) << 32) | wave_and32((uint32_t)fv);
  const uint64_t ZR = W == 16 ? (uint64_t)wave_and32((uint32_t)zr)
                              : ((uint64_t)wave_and32((uint32_t)(zr >> 32)) << 32) | wave_and32((uint32_t)zr);
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
  if (t == 0) done_waves = 0;
  if ((lane & 31) == 0) {
    chunk_len[t >> 5] = len;
    if (chunk < nchunks) reinterpret_cast<uint16_t *>(dst)[chunk] = (uint16_t)len;
  }
  {
    uint4 *z = reinterpret_cast<uint4 *>(lds);
    for (uint32_t i = t; i < (uint32_t)kGroupBufDwords / 4; i += kCThreads) z[i] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  // The group's aggregate goes out now; the device-wide offsets are resolved
  // after the emission (which works at byte alignment 0), so that waiting on
  // the predecessors overlaps with the other waves' emission.
  if (wave == 0) {
    uint32_t inc = lane < (uint32_t)kGroupChunks ? chunk_len[lane] : 0u;
#pragma unroll
    for (int o = 1; o < kGroupChunks; o <<= 1) {
      const uint32_t v = __shfl_up(inc, o, 64);
      if (lane >= (uint32_t)o) inc += v;
    }
    lookback_publish(status, tile, __shfl(inc, kGroupChunks - 1, 64), epoch);
  }

  // --- 5. Emission into the chunk buffers (payload bit i at buffer bit i). ---
  // All-zero blocks of coded chunks: their one code. (In a raw chunk their
  // bytes are zeros, which the cleared buffer already holds.)
  if (valid && !nonzero && !raw_chunk) emit_zero_block<W>(lds + (t >> 5) * kChunkBufDwords, excl, mode);

  if (wave_active) {
    const uint32_t ch = sblock >> 5;
    const uint64_t cchunk = (uint64_t)tile * kGroupChunks + ch;
    const uint32_t craw_len =
        cchunk < nchunks ? (uint32_t)min_u64(kChunkBytes, raw_bytes - cchunk * kChunkBytes) : 0u;
    const bool craw = chunk_len[ch] == craw_len;
    const bool coded = active && !craw;
    const bool want_zvc = coded && tag == kZVC;
    const bool want_dbx = coded && tag == kDBX;
    const bool want_zbx = coded && tag == kZBX;
    const bool want_planes = coded && (tag == kDBX || tag == kBX || tag == kZBX);
    uint32_t *buf = lds + ch * kChunkBufDwords;

    // Raw chunks: the block's bytes at its place (dword aligned).
    if (__ballot(active && craw)) {
      if (active && craw) {
        uint32_t r[32];
        load_block(src, raw_bytes, ((uint64_t)tile * kCThreads + sblock) * kBlockBytes, r);
        uint4 *q = reinterpret_cast<uint4 *>(buf + 32 * (sblock & 31));
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = make_uint4(r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]);
      }
    }

    uint32_t off = coded ? (uint32_t)blk_bits[sblock] : 0u;
    // Tag, then the DBX base or the ZVC / ZBX mask.
    if (coded) {
      uint32_t hv = 0, hl = 0;
      if (mode.tagged) {
        hv = (uint32_t)tag;
        hl = 3;
      }
      if (W == 16 && want_dbx) {
        hv |= base << hl;
        hl += 16;
      }
      or32(buf, off, hv);
      off += hl;
      if (W == 32 && want_dbx) {
        or32(buf, off, base);
        off += 32;
      }
    }
    if (__ballot(want_zvc || want_zbx)) {
      if (want_zvc || want_zbx) {
        if constexpr (W == 16)
          or64(buf, off, mlo, mhi);
        else
          or32(buf, off, mlo);
        off += N;
      }
    }

    // RAW blocks of coded chunks: 1024 bits at an arbitrary bit offset.
    const bool want_rawblk = coded && tag == kRAW;
    if (__ballot(want_rawblk)) {
      if (want_rawblk) {
        uint32_t r[32];
        load_block(src, raw_bytes, ((uint64_t)tile * kCThreads + sblock) * kBlockBytes, r);
        const uint32_t q = off >> 5, sh = off & 31u;
        atomicOr(&buf[q], r[0] << sh);
#pragma unroll
        for (int i = 1; i < 32; ++i) buf[q + i] = (r[i] << sh) | ((r[i - 1] >> 1) >> (31u - sh));
        atomicOr(&buf[q + 32], (r[31] >> 1) >> (31u - sh));
      }
    }

    // ZVC: the n non-zero symbols, in order, 32 bits (two w = 16 symbols) at
    // a time, until no lane has any left.
    if (__ballot(want_zvc)) {
      const uint32_t zbits = want_zvc ? (uint32_t)W * sn : 0u;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        if (!__ballot(32u * q < zbits)) break;
        if (32u * q < zbits) or32(buf, off + 32u * q, e[q]);  // words past n hold zeros
      }
    }

    // Plane encodings: DBX's top plane (the borrows), then planes W-1..0 of
    // the transposed input; each plane takes the zero path, the verbatim
    // path or the general classifier, as the whole wave allows.
    if (__ballot(want_planes)) {
      const uint32_t L = want_dbx ? (uint32_t)(N - 1) : (want_zbx ? sn : (uint32_t)N);
      const uint32_t L1 = L + 1;
      const uint32_t cs = 5u + (uint32_t)position_bits((int)L);
      const PT ones = (PT)all_ones64((int)L);
      uint32_t run = 0;
      PT above = 0;
      if (__ballot(want_dbx)) {
        PT bm;
        if constexpr (W == 16)
          bm = ((uint64_t)bm_hi << 32) | bm_lo;
        else
          bm = bm_lo;
        if ((ZR >> KT) & 1u) {
          if (want_dbx) run = 1;
        } else if ((FV >> KT) & 1u) {
          if (want_dbx) {
            if constexpr (W == 16)
              or_verbatim(buf, off, bm_lo, bm_hi);
            else
              or_verbatim(buf, off, bm_lo);
            off += L1;
          }
        } else {
          if (want_dbx) emit_plane<PT, R>(buf, off, run, bm, false, ones, L, cs);
        }
        above = want_dbx ? bm : (PT)0;
      }
      transpose32(e);
#pragma unroll
      for (int j = W - 1; j >= 0; --j) {
        PT pj;
        if constexpr (W == 16)
          pj = ((uint64_t)e[16 + j] << 32) | e[j];
        else
          pj = e[j];
        const PT x = pj ^ above;
        above = pj;
        if ((ZR >> j) & 1u) {
          if (want_planes) ++run;
        } else if ((FV >> j) & 1u) {
          if (want_planes) {
            if constexpr (W == 16)
              or_verbatim(buf, off, (uint32_t)x, (uint32_t)((uint64_t)x >> 32));
            else
              or_verbatim(buf, off, (uint32_t)x);
            off += L1;
          }
        } else {
          if (want_planes) emit_plane<PT, R>(buf, off, run, x, pj == 0, ones, L, cs);
        }
      }
      if (want_planes && run) {
        uint32_t rcode, rlen;
        run_code<R>(run, rcode, rlen);
        or32(buf, off, rcode);
      }
    }
  }

  // Device-wide payload offsets of the group's chunks: the first wave done
  // with its emission resolves the look-back (waves with little or no
  // emission, as in a tile of mostly zero blocks, start waiting at once).
  uint32_t first = 0;
  if (lane == 0) first = atomicAdd(&done_waves, 1u);
  if (__builtin_amdgcn_readfirstlane(__shfl(first, 0, 64)) == 0) {
    const uint32_t cl = lane < (uint32_t)kGroupChunks ? chunk_len[lane] : 0u;
    uint32_t cinc = cl;
#pragma unroll
    for (int o = 1; o < kGroupChunks; o <<= 1) {
      const uint32_t v = __shfl_up(cinc, o, 64);
      if (lane >= (uint32_t)o) cinc += v;
    }
    const uint32_t total = __shfl(cinc, kGroupChunks - 1, 64);
    const uint64_t before = lookback_resolve(status, tile, total, epoch);
    if (lane < (uint32_t)kGroupChunks) chunk_pay[lane] = 2 * nchunks + before + (cinc - cl);
    if (tile == ntiles - 1 && lane == 0) *batch.t[k].out_bytes = 2 * nchunks + before + total;
  }
  __syncthreads();

  // --- 6. Store: wave w writes chunks 2w and 2w+1 in 16-byte units.
  // Payload byte i goes to dst byte poff + i. With sh = poff & 15 =
  // 4 dsh + bsh, dst dword o of the 16-byte aligned span holds payload bytes
  // 4o - sh .. 4o - sh + 3: buffer dwords o - dsh - 1 and o - dsh joined by
  // a funnel shift. Unit u of the span therefore needs buffer dwords
  // 4u - dsh - 1 .. 4u - dsh + 3, which lie in the aligned quads u - 1 and u
  // (two conflict-free 16-byte LDS reads; dsh is uniform over the chunk).
  // A lane's units are u = lane + 64 m (a chunk spans at most 257), one
  // per iteration (issuing all of a chunk's LDS reads before its first
  // store measured the same: the other waves hide these waits). Only the
  // first and last units (shared with the neighbouring chunks) are written
  // piecewise. ---
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
        for (uint32_t kk = 0; kk < 4; ++kk) {
          const uint32_t d0 = b0 + 4 * kk;
          if (d0 >= sh && d0 + 4 <= total) {
            *reinterpret_cast<uint32_t *>(span + d0) = v[kk];
          } else {
#pragma unroll
            for (uint32_t bb = 0; bb < 4; ++bb)
              if (d0 + bb >= sh && d0 + bb < total) span[d0 + bb] = (uint8_t)(v[kk] >> (8 * bb));
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
// The size pass keeps tiles of 16 chunks (eight waves): it adds each
// workgroup's bytes to the tensor's total with one atomic on a single
// address, and such atomics complete one after another (about 6 ns each), so
// twice the workgroups cost about 50 us more on the GPT-2-XL workload.
constexpr int kSWaves = 8;
constexpr int kSThreads = kWave * kSWaves;
constexpr int kSGroupChunks = kSThreads / kBlocksPerChunk;
constexpr int kSStageDwords = kSThreads * kLaneStride;

template <int W>
__global__ __launch_bounds__(kSThreads, kCWavesPerSimd) void size_kernel(const SBatch batch, Mode mode) {
  constexpr int N = 1024 / W;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kSStageDwords];
  __shared__ uint16_t blk_bits[kSThreads];
  __shared__ uint16_t slot_block[kSThreads];
  __shared__ uint8_t slot_n[kSThreads];
  __shared__ uint32_t wave_full[kSWaves];
  __shared__ uint32_t wave_part[kSWaves];
  __shared__ uint32_t chunk_len[kSGroupChunks];

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
  const uint64_t sample = (uint64_t)(blockIdx.x - batch.t[k].group_begin) * kSGroupChunks + (t >> 5);
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
  for (int q = 0; q < kSWaves; ++q) {
    const uint32_t f = wave_full[q], p = wave_part[q];
    ffirst += (uint32_t)q < wave ? f : 0u;
    pfirst += (uint32_t)q < wave ? p : 0u;
    nfull += f;
    npart += p;
  }
  const uint32_t nnz = nfull + npart;
  const bool staged = !(nnz == (uint32_t)kSThreads && (npart == 0 || nfull == 0));
  if (staged) {
    if (nonzero) {
      const uint32_t idx = partial ? nfull + pfirst + lanes_below(mpart) : ffirst + lanes_below(mfull);
      uint32_t *slotp = lds + idx * kLaneStride;
#pragma unroll
      for (int i = 0; i < 32; ++i) slotp[i] = d[i];
      slot_block[idx] = (uint16_t)t;
      slot_n[idx] = (uint8_t)sn;
    }
    __syncthreads();
  }

  const uint32_t slot = staged ? (t + kSThreads - 64u * (blockIdx.x & (kSWaves - 1u))) & (kSThreads - 1) : t;
  const bool active = slot < nnz;
  if (__ballot(active) != 0) {
    if (staged) {
      const uint32_t *region = lds + slot * kLaneStride;
      sn = active ? (uint32_t)slot_n[slot] : 0u;
      if (active) {
#pragma unroll
        for (int i = 0; i < 32; ++i) d[i] = region[i];
      }
    }
    if constexpr (W == 16) to_split16(d);
    Stats s;
    candidate_sizes<W>(d, (int)sn, __ballot(active && sn < (uint32_t)N) != 0, s);
    int best_size;
    select_tag(s, best_size, mode.mask);
    const uint32_t sb = staged ? (uint32_t)slot_block[slot] : t;
    if (active) blk_bits[sb] = (uint16_t)(3u * mode.tagged + best_size);
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
    for (int c = 0; c < kSGroupChunks; ++c) sum += chunk_len[c];
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
  x.ngroups = (uint32_t)((x.nsampled + kSGroupChunks - 1) / kSGroupChunks);
}

hipError_t launch_size(int w, const SBatch &batch, uint32_t codec_mask, int tagged, hipStream_t stream) {
  hipLaunchKernelGGL(store_size_init_kernel, dim3(1), dim3(64), 0, stream, batch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || batch.total_groups == 0) return e;
  const Mode mode = make_mode(w, codec_mask, tagged);
  if (w == 16)
    hipLaunchKernelGGL(size_kernel<16>, dim3(batch.total_groups), dim3(kSThreads), 0, stream, batch, mode);
  else
    hipLaunchKernelGGL(size_kernel<32>, dim3(batch.total_groups), dim3(kSThreads), 0, stream, batch, mode);
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
    hipLaunchKernelGGL(compress_kernel<16>, dim3(batch.total_tiles), dim3(kCThreads), 0, stream, batch, scratch.words,
                       scratch.counter, scratch.counter_base, scratch.epoch, mode);
  else
    hipLaunchKernelGGL(compress_kernel<32>, dim3(batch.total_tiles), dim3(kCThreads), 0, stream, batch, scratch.words,
                       scratch.counter, scratch.counter_base, scratch.epoch, mode);
  return hipGetLastError();
}

}  // namespace pz
