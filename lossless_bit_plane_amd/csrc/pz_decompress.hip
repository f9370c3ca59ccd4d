// PlaneZip decompression on gfx950.
//
// Method: PlaneZip paper, §III-A "Stream format": a prefix sum over the
// 16-bit chunk headers locates every chunk, so chunks decode in parallel; the
// decoder reproduces every block exactly (§III-A "Validation"). Bit layout and
// decoder checks: FORMAT.md version 1, §5 and §6.
//
// A chunk's blocks carry no offsets, so the blocks of one chunk must be
// parsed in order. The work is split in two halves, two kernels for small
// launches and one ticketed kernel for large ones (decompress_kernel):
//   locate: one quad of lanes per chunk, 64 chunks per workgroup. Scans the
//           headers (decoupled look-back across workgroups), validates them,
//           and walks each chunk's codes without decoding them to record the
//           bit offset of every block; the quad settles up to 16 verbatim
//           plane codes per step by speculation.
//   decode: 8 chunks per workgroup. The payloads are staged in LDS with
//           coalesced loads; all-zero blocks are recognised by their code and
//           the other blocks packed onto the fewest waves, where a lane decodes
//           a block from its known bit offset: codes -> XORed planes -> planes
//           -> inverse 32x32 bit transpose -> symbols (delta prefix sum for
//           DBX, scatter by the zero mask for ZVC/ZBX). The decoded blocks
//           are gathered in LDS and leave in coalesced stores.
#include <type_traits>

#include "pz_device.h"
#include "pz_launch.h"

namespace pz {

constexpr int32_t kStatusCorrupt = 3;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // for non-temporal 16-byte stores

// What the decoder needs of a codec mode: whether blocks carry a tag (else
// every block is the fixed candidate), and the code of an all-zero block it
// can settle at once: BX with all planes in one zero run, behind a BX tag or
// alone in the untagged BX mode, as it appears in the stream's low bits at a
// block start (zmask = 0: no such shortcut). Any other block, and any stream
// a tagged decoder is given whatever mask the encoder used, is decoded by
// its codes.
struct DMode {
  uint32_t tagged, fixed;
  uint32_t zmask, zcode, zbits;
};

inline DMode make_dmode(int W, uint32_t mask, int tagged) {
  const uint32_t R = W == 16 ? 4 : 5;
  const uint32_t run = 2u | ((uint32_t)(W - 2) << 2);  // one zero run over all W planes
  DMode m{tagged ? 1u : 0u, 0u, 0u, 1u, 0u};
  for (uint32_t t = 0; t < 5; ++t)
    if (mask == (1u << t)) m.fixed = t;
  if (tagged) {
    m.zbits = 3 + 2 + R;
    m.zcode = (uint32_t)kBX | (run << 3);
  } else if (m.fixed == (uint32_t)kBX) {
    m.zbits = 2 + R;
    m.zcode = run;
  }
  if (m.zbits) m.zmask = (1u << m.zbits) - 1u;
  return m;
}

// ---------------------------------------------------------------------------
// Locate. A workgroup takes a tile of 256 / G chunks (64); each chunk is
// walked by a group of G = 4 lanes. Walking is sequential by nature (a block starts where
// the previous one ends), and a wave's time is mostly the length of its
// dependent instruction chain, so each step speculates: lane q of the group
// reads the windows at pos + (4q + s)(1+L), s = 0..3, i.e. where codes 4q+s
// would start if all codes before them were verbatim (their length 1+L is
// fixed within a block). One step thus settles a run of up to 16 verbatim
// planes, then decodes up to two short codes from the window at the first
// non-verbatim code. (One lane per chunk does a quarter of the instructions
// but walks four times as many steps per wave; it measured slower on every
// tensor of the bench workload.)
// ---------------------------------------------------------------------------
// Lanes per chunk. The kernel takes 4, 8 or 16: 4 in the single decompress
// kernel and for 16-bit symbols, 8 for 32-bit symbols in launches of locate
// and decode (32 speculated codes settle a block's 32 planes in fewer steps;
// 8 lanes made the GPT-2 tensors 20% slower, 16 lanes were slower
// everywhere: a step's latency, not its width, sets a small tensor's walk).
constexpr int kLocateLanes = 4;
constexpr int kLocateLanesWide = 8;
constexpr int kLocateThreads = 256;            // four waves per workgroup
template <int G>
constexpr int locate_chunks() { return kLocateThreads / G; }  // chunks per tile (per workgroup)
constexpr int kLocateChunks = locate_chunks<kLocateLanes>();
// Per-chunk LDS region: a ring of kRingDwords dwords of the chunk's stream, one
// mirror dword (slot kRingDwords = slot 0, so a peek at the last slot reads two
// dwords), then the chunk's 32 block offsets (16-bit). 145 dwords: odd, spreads
// chunks over banks. (A 64-dword ring with 16-dword refills fits twice the
// chunks per compute unit but measured slower on every workload: the walk then
// waits on its refills.)
constexpr int kRingDwords = 128;
constexpr int kRingRegion = kRingDwords + 1 + 16;
constexpr uint32_t kBlockAhead = 38;   // dwords one block (and its look-ahead) can touch

// One of four values by the two low bits of k, as bit-tested selects (an
// equality chain would be turned into branches).
PZ_DEV uint32_t select4(uint32_t k, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
  const bool odd = (k & 1u) != 0;
  const uint32_t lo = odd ? a1 : a0, hi = odd ? a3 : a2;
  return (k & 2u) ? hi : lo;
}

// Value of `v` in lane k of this lane's group of G (DPP quad broadcast for
// quads, a lane permute otherwise).
template <int G>
PZ_DEV uint32_t group_lane(uint32_t v, uint32_t k) {
  if constexpr (G == 4) {
    const uint32_t b0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, true);
    const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, true);
    const uint32_t b2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, true);
    const uint32_t b3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, true);
    return select4(k, b0, b1, b2, b3);
  } else if constexpr (G == 8) {
    // Lane k & 3 of each quad, then the other quad's copy by a half-row mirror
    // (lane i of the 8 reads lane 7 - i, which lies in the other quad).
    const uint32_t b = group_lane<4>(v, k & 3u);
    const uint32_t m = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x141, 0xF, 0xF, true);
    return ((lane_id() >> 2) & 1u) == (k >> 2) ? b : m;
  } else {
    return (uint32_t)__shfl((int)v, (int)((lane_id() & ~(uint32_t)(G - 1)) | k), 64);
  }
}

// OR of `v` over this lane's group of G (4, 8 or 16 lanes of one DPP row).
template <int G>
PZ_DEV uint32_t group_or32(uint32_t v) {
  static_assert(G == 4 || G == 8 || G == 16, "groups of 4, 8 or 16 lanes");
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // lanes 1,0,3,2
  v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // lanes 2,3,0,1
  if constexpr (G >= 8) v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true);  // half-row mirror
  if constexpr (G >= 16) v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true);  // row mirror
  return v;
}
template <int G>
PZ_DEV uint64_t group_or(uint64_t v) {
  if constexpr (4 * G <= 32) {
    return group_or32<G>((uint32_t)v);
  } else {
    return (uint64_t)group_or32<G>((uint32_t)v) | ((uint64_t)group_or32<G>((uint32_t)(v >> 32)) << 32);
  }
}

// A chunk's stream, read by the chunk's group through the LDS ring. The ring
// is topped up only at block starts, and only when some group of the wave has
// fewer than one block's worth of dwords buffered: then every group stores the
// 32 dwords it requested at the last such round and requests the next 32 if
// the ring will have room for them, and a group still short waits for a load
// on the spot. Each of the G lanes holds and stores 32/G of the 32 dwords.
template <int G>
struct ChunkRing {
  // Refill unit: 32 dwords (4G for 16 lanes), split over the G lanes (at
  // least one 16-byte load each).
  static constexpr uint32_t kGroupDwords = 4 * G > 32 ? 4 * G : 32;
  static constexpr int kStartGroups = (int)((kBlockAhead + kGroupDwords - 1) / kGroupDwords);
  // A refill made while a group is short (fill < cur + kBlockAhead) and the
  // request made after the first groups must not overwrite dwords at or above cur.
  static_assert(kBlockAhead - 1 + kGroupDwords <= (uint32_t)kRingDwords, "refill fits in the ring");
  static_assert((kStartGroups + 1) * kGroupDwords <= (uint32_t)kRingDwords, "start fits in the ring");
  static constexpr int kPart = kGroupDwords / G;  // dwords per lane per refill
  uint32_t *ring;
  const uint8_t *src;
  uint64_t limit;   // comp_bytes: nothing at or past it is read
  uint64_t q0;      // absolute dword index of relative dword 0 (16-byte aligned)
  uint32_t lead;    // bit offset of the chunk payload within relative dword 0
  uint32_t ql;      // lane within the group
  uint32_t fill;    // relative dwords below fill have been stored (the last kRingDwords are kept)
  bool pending;     // g holds relative dwords [fill + kPart ql, +kPart)
  uint4 g[kPart / 4];

  PZ_DEV uint4 load4(uint32_t r) const {
    const uint64_t b = (q0 + r) * 4;
    if (b + 16 <= limit) return *reinterpret_cast<const uint4 *>(src + b);
    return load4_tail(b);
  }
  // The stream's last bytes: byte loads below limit, zeros above (a plain
  // loop: it runs at most once per chunk near the end of the stream).
  PZ_DEV uint4 load4_tail(uint64_t b) const {
    uint32_t v[4] = {0, 0, 0, 0};
#pragma unroll 1
    for (uint32_t k = 0; k < 16 && b + k < limit; ++k) {
      const uint32_t x = (uint32_t)src[b + k] << (8 * (k & 3));
      if (k < 4) v[0] |= x; else if (k < 8) v[1] |= x; else if (k < 12) v[2] |= x; else v[3] |= x;
    }
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  PZ_DEV void issue() {
#pragma unroll
    for (int k = 0; k < kPart / 4; ++k) g[k] = load4(fill + kPart * ql + 4 * k);
    pending = true;
  }
  // Stores the in-flight group at fill (slots fill % kRingDwords, + kGroupDwords: never wraps).
  PZ_DEV void commit() {
    uint32_t *r = ring + (fill & (kRingDwords - 1)) + kPart * ql;
#pragma unroll
    for (int k = 0; k < kPart / 4; ++k) {
      r[4 * k + 0] = g[k].x;
      r[4 * k + 1] = g[k].y;
      r[4 * k + 2] = g[k].z;
      r[4 * k + 3] = g[k].w;
    }
    if ((fill & (kRingDwords - 1)) == 0 && ql == 0) ring[kRingDwords] = g[0].x;  // mirror
    fill += kGroupDwords;
    pending = false;
  }
  PZ_DEV void start(uint32_t *r, const uint8_t *s, uint64_t lim, uint64_t payload_off, uint32_t lane_in_group) {
    ring = r;
    src = s;
    limit = lim;
    ql = lane_in_group;
    q0 = (payload_off >> 2) & ~3ull;
    lead = (uint32_t)(8 * (payload_off - 4 * q0));
    // The groups one block needs in one round trip, then the next requested.
    uint4 first[kStartGroups][kPart / 4];
#pragma unroll
    for (int s = 0; s < kStartGroups; ++s)
#pragma unroll
      for (int k = 0; k < kPart / 4; ++k) first[s][k] = load4(s * kGroupDwords + kPart * ql + 4 * k);
#pragma unroll
    for (int s = 0; s < kStartGroups; ++s) {
      uint32_t *w = ring + s * kGroupDwords + kPart * ql;
#pragma unroll
      for (int k = 0; k < kPart / 4; ++k) {
        w[4 * k + 0] = first[s][k].x;
        w[4 * k + 1] = first[s][k].y;
        w[4 * k + 2] = first[s][k].z;
        w[4 * k + 3] = first[s][k].w;
      }
    }
    if (ql == 0) ring[kRingDwords] = first[0][0].x;  // mirror of slot 0
    fill = kStartGroups * kGroupDwords;
    issue();
  }
  // At a block start whose first bit is pos (group-uniform): makes relative
  // dwords [dword of pos, +kBlockAhead) available and requests the next group.
  PZ_DEV void step(uint32_t pos) {
    const uint32_t cur = (lead + pos) >> 5;
    // A wave waits for all its loads at once, so the groups of a wave store
    // and request in common rounds, and a round is held only when some group
    // is short of buffered dwords: the loads of the last round have then had
    // every step since to arrive.
    if (__ballot(fill < cur + kBlockAhead)) {
      if (pending) commit();
      while (fill < cur + kBlockAhead) {
        issue();
        commit();
      }
      // Stored dwords at or above cur stay in the ring until the group passes them.
      if (fill + kGroupDwords <= cur + kRingDwords) issue();
      wave_lds_fence();  // the group's stores before its reads
    }
  }
  PZ_DEV uint32_t peek(uint32_t pos) const {
    const uint32_t a = lead + pos;
    const uint32_t slot = (a >> 5) & (kRingDwords - 1);
    return funnel(ring[slot + 1], ring[slot], a & 31u);
  }
};

// Walks the codes of a coded chunk (group-uniform: the G lanes compute the
// same positions), recording each block's bit offset in boff (LDS, written by
// group lane 0). Returns false for a chunk that fails a decoder check
// (FORMAT.md §6). Blocks are taken in wave-uniform steps: all groups read a
// block header together (tag, then the base or the zero mask), then the
// block's plane codes, whose class is the trailing-zero count of the next
// bits and whose length comes from a per-block table.
template <int W, int G>
PZ_DEV bool parse_chunk(ChunkRing<G> &in, bool coded, uint32_t H, uint32_t raw_len, uint16_t *boff,
                        const DMode &mode) {
  constexpr uint32_t N = 1024 / W;
  constexpr uint32_t R = W == 16 ? 4 : 5;
  constexpr uint32_t kSpec = 4 * G;  // codes tried per step
  const uint32_t end = H * 8;
  const uint32_t nb = (raw_len + kBlockBytes - 1) / kBlockBytes;
  const uint32_t ql = in.ql;
  uint32_t pos = 0;
  bool bad = false;
  for (uint32_t b = 0; b < (uint32_t)kBlocksPerChunk; ++b) {
    const bool live = coded && !bad && b < nb;
    if (!__ballot(live)) break;
    int left = 0;
    uint32_t L = N, pmask = 0, V = 0;
    uint32_t lut = 0;  // short-code lengths by class: byte tz - 1 for tz = 1..4
    if (live) {
      in.step(pos);
      if (ql == 0) boff[b] = (uint16_t)pos;
      const uint32_t head = in.peek(pos);
      const uint32_t tag = mode.tagged ? head & 7u : mode.fixed;
      const uint32_t hb = 3u * mode.tagged;  // tag bits
      if ((head & mode.zmask) == mode.zcode) {
        pos += mode.zbits;  // an all-zero block: one run over all planes
      } else {
        const bool masked = tag == kZVC || tag == kZBX;
        // The zero mask's count, read only when some chunk of the wave needs it.
        uint32_t n = 0;
        if (__ballot(masked)) {
          n = (uint32_t)popc32(in.peek(pos + hb));
          if (W == 16) n += (uint32_t)popc32(in.peek(pos + hb + 32));
        }
        pos += hb + (tag == kDBX ? W : 0u) + (masked ? N : 0u) + (tag == kZVC ? W * n : 0u) +
               (tag == kRAW ? 1024u : 0u);
        bad |= tag > 4;
        L = tag == kDBX ? N - 1 : (tag == kZBX ? n : N);
        left = (tag == kBX || tag == kZBX) ? (int)W : (tag == kDBX ? (int)W + 1 : 0);
        // Code length by class (trailing zeros of the next bits, capped at 4):
        // verbatim 1+L, run 2+R, lone zero 3, pair/single 5+PW, other 5.
        const uint32_t pw = (uint32_t)position_bits((int)L);
        pmask = (1u << pw) - 1u;
        V = 1 + L;
        lut = (2 + R) | (3u << 8) | ((5 + pw) << 16) | (5u << 24);
      }
    }
    const uint32_t spec = 4 * ql * V;  // this lane tries codes 4 ql .. 4 ql + 3
    const uint32_t runf = (1u << R) - 1u;
    // Straight-line steps (selects, no branches): a lone wave pays for every
    // instruction, and exec-mask branches cost more than the selects.
    while (left > 0) {
      const uint32_t a = pos + spec;
      const uint32_t w0 = in.peek(a), w1 = in.peek(a + V), w2 = in.peek(a + 2 * V),
                     w3 = in.peek(a + 3 * V);
      using VM = typename std::conditional<(4 * G > 32), uint64_t, uint32_t>::type;
      const VM mine = (VM)((w0 & 1u) | ((w1 & 1u) << 1) | ((w2 & 1u) << 2) | ((w3 & 1u) << 3));
      const VM vmask = (VM)group_or<G>((uint64_t)(mine << (4 * ql)));  // bit k: code k would be verbatim
      // Leading verbatim codes (at most 4G: for 4G < 32 bit 4G of ~vmask is set).
      uint32_t lead;
      if constexpr (4 * G >= 64)
        lead = vmask == ~0ull ? 64u : (uint32_t)__builtin_ctzll(~vmask);
      else if constexpr (4 * G == 32)
        lead = vmask == ~0u ? 32u : (uint32_t)__builtin_ctz(~vmask);
      else
        lead = (uint32_t)__builtin_ctz(~vmask);
      const uint32_t j = min(lead, (uint32_t)left);
      pos += j * V;
      left -= (int)j;
      // The window of code j: lane j/4 of the group read it as its w[j%4].
      uint32_t win = group_lane<G>(select4(j, w0, w1, w2, w3), j >> 2);
      bool take = j < kSpec;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        take = take && left > 0 && (win & 1u) == 0u;  // a short code (at most 11 bits)
        const uint32_t tz = (uint32_t)__builtin_ctz(win | 16u);  // trailing zeros, capped at 4
        const uint32_t len = __builtin_amdgcn_ubfe(lut, 8u * tz - 8u, 8u);  // tz = 0 is never taken
        const int planes = tz == 1 ? (int)((win >> 2) & runf) + 2 : 1;  // a run past the end: left < 0
        // A position must lie inside the plane: p <= L-1 (single), L-2 (pair).
        const bool badpos = tz == 3 && ((win >> 5) & pmask) + 2 > L + ((win >> 4) & 1u);
        pos += take ? len : 0u;
        left -= take ? planes : 0;
        bad |= take && badpos;
        win >>= len;
      }
    }
    if (live) bad |= left < 0 || pos > end;
  }
  if (coded && !bad) {
    // The last block must end in the payload's last byte, padded with zeros.
    bad |= (pos + 7) / 8 != H;
    in.step(pos);
    if ((pos & 7u) && (in.peek(pos) & ((1u << (8 - (pos & 7u))) - 1u))) bad = true;
  }
  return !bad;
}

// The tensor a launch's tile belongs to (tiles are numbered across the
// tensors, in increasing order of the tensor).
PZ_DEV uint32_t tensor_of_tile(const DBatch &batch, uint32_t gtile) {
  uint32_t k = 0;
  if (batch.n > 1) {  // a single tensor's fields load at once
#pragma unroll
    for (uint32_t i = 1; i < (uint32_t)kMaxBatch; ++i) k += i < batch.n && gtile >= batch.t[i].tile_begin ? 1u : 0u;
  }
  return k;
}

template <int G>
struct LocateShared {
  uint32_t lds[locate_chunks<G>() * kRingRegion];
  uint64_t wave_sum[kLocateThreads / kWave];
  uint64_t tile_before;
};

// Locates tile gtile of the launch (tensor k): chunk offsets and block
// offsets of its chunks, corruption in error word k. kShared: the offsets
// go to decode groups of the same launch, so they are stored at device
// scope (decompress_kernel).
template <int W, int G, bool kShared>
PZ_DEV void locate_tile(const DBatch &batch, uint32_t k, uint32_t gtile, uint32_t *err_words, uint32_t epoch,
                        uint64_t *lb_words, const DMode &mode, LocateShared<G> &sh) {
  constexpr int kWaves = kLocateThreads / kWave;  // 256 / G chunks x G lanes
  uint32_t *lds = sh.lds;
  uint64_t *wave_sum = sh.wave_sum;
  uint64_t &tile_before = sh.tile_before;
  const uint32_t t = threadIdx.x, lane = lane_id(), ql = t & (G - 1);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint8_t *__restrict__ src = batch.t[k].src;
  const uint64_t comp_bytes = batch.t[k].comp_bytes, raw_bytes = batch.t[k].raw_bytes;
  const uint64_t nchunks = batch.t[k].nchunks;
  const uint32_t ntiles = batch.t[k].ntiles;
  uint64_t *__restrict__ chunk_off = batch.t[k].chunk_off;
  uint16_t *__restrict__ block_off = batch.t[k].block_off;
  uint32_t *err = err_words + k;
  const uint32_t tile = gtile - batch.t[k].tile_begin;
  uint64_t *lb_status = lb_words + (uint64_t)batch.t[k].tile_begin * kLookbackStride;

  // Chunk offsets: a scan of the 16-bit headers over the tile, and one
  // look-back per tile for the headers before it.
  const uint32_t ci = t / G;  // chunk within the tile
  const uint64_t c = (uint64_t)tile * locate_chunks<G>() + ci;
  const uint32_t H = c < nchunks ? reinterpret_cast<const uint16_t *>(src)[c] : 0u;
  const uint64_t incl = wave_inclusive_scan_u64(ql == 0 ? H : 0u);  // equal over the group
  if (lane == kWave - 1) wave_sum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint64_t agg = 0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) agg += wave_sum[k];
    const uint64_t before = lookback(lb_status, tile, agg, epoch);
    if (lane == 0) {
      tile_before = before;
      if (tile == ntiles - 1 && 2 * nchunks + before + agg != comp_bytes) atomicMax(err, epoch);
    }
  }
  __syncthreads();
  uint64_t wave_before = tile_before;
  for (uint32_t k = 0; k < wave; ++k) wave_before += wave_sum[k];
  const uint64_t off = 2 * nchunks + wave_before + incl - H;

  const uint32_t raw_len =
      c < nchunks ? (uint32_t)min_u64(kChunkBytes, raw_bytes - c * kChunkBytes) : 0u;
  const bool header_bad = c < nchunks && (H > raw_len || off + H > comp_bytes);
  const bool coded = c < nchunks && !header_bad && H < raw_len;
  uint32_t *region = lds + ci * kRingRegion;
  uint16_t *boff = reinterpret_cast<uint16_t *>(region + kRingDwords + 1);
  ChunkRing<G> in;
  in.start(region, src, comp_bytes, coded ? off : 0, ql);
  const bool parsed = parse_chunk<W, G>(in, coded, H, raw_len, boff, mode);  // whole wave
  wave_lds_fence();
  if (coded) {
    // The chunk's block offsets: 64 bytes, 64/G per group lane.
    const uint32_t *b32 = region + kRingDwords + 1 + (16 / G) * ql;
    if constexpr (kShared) {
      uint64_t *o64 = reinterpret_cast<uint64_t *>(block_off + c * kBlocksPerChunk) + (8 / G) * ql;
#pragma unroll
      for (int k = 0; k < 8 / G; ++k)
        __hip_atomic_store(o64 + k, (uint64_t)b32[2 * k] | ((uint64_t)b32[2 * k + 1] << 32), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else if constexpr (G == 4) {
      *(reinterpret_cast<uint4 *>(block_off + c * kBlocksPerChunk) + ql) = make_uint4(b32[0], b32[1], b32[2], b32[3]);
    } else {
      uint32_t *outd = reinterpret_cast<uint32_t *>(block_off + c * kBlocksPerChunk) + (16 / G) * ql;
#pragma unroll
      for (int k = 0; k < 16 / G; ++k) outd[k] = b32[k];
    }
  }
  if (c < nchunks && ql == 0) {
    const bool chunk_bad = header_bad || (coded && !parsed);
    if constexpr (kShared)
      __hip_atomic_store(chunk_off + c, chunk_bad ? kBadChunk : off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      chunk_off[c] = chunk_bad ? kBadChunk : off;
    if (chunk_bad) atomicMax(err, epoch);
  }
}

template <int W, int G>
__global__ __launch_bounds__(kLocateThreads) void locate_kernel(const DBatch batch, uint32_t *err_words,
                                                                    uint32_t epoch, uint64_t *lb_words,
                                                                    uint32_t *tile_counter,
                                                                    uint32_t counter_base, DMode mode) {
  __shared__ LocateShared<G> sh;
  __shared__ uint32_t group_tile;
  if (threadIdx.x == 0) group_tile = atomicAdd(tile_counter, 1u) - counter_base;
  __syncthreads();
  const uint32_t gtile = __builtin_amdgcn_readfirstlane(group_tile);
  if (gtile >= batch.total_tiles) return;
  locate_tile<W, G, false>(batch, tensor_of_tile(batch, gtile), gtile, err_words, epoch, lb_words, mode, sh);
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
  // A plane code's window and the 64 bits after its first bit (the payload
  // of a verbatim code), from one read of three dwords.
  PZ_DEV void peek_code(uint32_t pos, uint32_t &win, uint64_t &after) const {
    const uint32_t a = lead + pos;
    uint32_t q = a >> 5;
    q = q > (uint32_t)kChunkBufDwords - 3 ? (uint32_t)kChunkBufDwords - 3 : q;
    const uint32_t d0 = buf[q], d1 = buf[q + 1], d2 = buf[q + 2];
    const uint32_t sh = (a & 31u) + 1u;  // 1..32
    win = funnel(d1, d0, a & 31u);
    const uint32_t lo = (uint32_t)((((uint64_t)d1 << 32) | d0) >> sh);
    const uint32_t hi = (uint32_t)((((uint64_t)d2 << 32) | d1) >> sh);
    after = (uint64_t)lo | ((uint64_t)hi << 32);
  }
};

// Reads the plane code of K planes (top plane first) and leaves the planes in
// the transpose layout: w = 16: plane j = t[j] | t[j+16] << 32; w = 32: plane
// j = t[j]. DBX planes are stored shifted up by one (delta k at bit k, delta
// 0 := 0); DBX's top plane (the borrow plane) only feeds the XOR chain. Every
// plane is decoded with selects rather than branches: the class comes from the
// trailing-zero count of the next 32 bits, and a pending zero run yields X = 0.
// A lane with `active` false keeps its pos; its planes are unspecified.
template <int W>
PZ_DEV void read_planes(const LdsBits &in, uint32_t &pos, uint32_t (&t)[32], int K, uint32_t L,
                        bool dbx, bool active) {
  using PT = typename std::conditional<W == 16, uint64_t, uint32_t>::type;
  constexpr uint32_t R = W == 16 ? 4 : 5;
  const uint32_t pw = (uint32_t)position_bits((int)L);
  const uint32_t pmask = (1u << pw) - 1u;
  const PT ones = (PT)all_ones64((int)L);
  // Code length by class: verbatim, run, lone zero, pair/single, pre-zero, ones.
  const uint64_t lut = (uint64_t)(1 + L) | ((uint64_t)(2 + R) << 8) | (3ull << 16) |
                       ((uint64_t)(5 + pw) << 24) | (5ull << 32) | (5ull << 40);
  PT above = 0;
  uint32_t run = 0;
#pragma unroll
  for (int j = W; j >= 0; --j) {
    // Only the top plane can be absent (K is W or W + 1). Below it every
    // plane of a decoding lane is live, and the other lanes' planes are
    // never used, so those planes need no liveness selects (only their
    // position must not move).
    const bool live = j < W || (active && j < K);
    const bool fresh = live && run == 0;
    uint32_t win;
    uint64_t after;
    in.peek_code(pos, win, after);
    // A plane that every decoding lane codes verbatim (the low mantissa
    // planes of dense data, in most waves): the plane is the code's payload.
    if (!__ballot(active && live && !(fresh && (win & 1u)))) {
      const PT p = live ? (((PT)after & ones) ^ above) : (PT)0;
      above = live ? p : above;
      pos += active && live ? 1u + L : 0u;
      if (j < W) {
        const PT ps = dbx ? (PT)(p << 1) : p;
        if constexpr (W == 16) {
          t[j] = (uint32_t)ps;
          t[j + 16] = (uint32_t)((uint64_t)ps >> 32);
        } else {
          t[j] = (uint32_t)ps;
        }
      }
      continue;
    }
    const uint32_t tz = (uint32_t)__builtin_ctz(win | 32u);  // 5: five or more zeros
    const PT verb = (PT)after & ones;
    // Single (bit 4 set): one 1; pair: two adjacent 1s.
    const PT one_or_pair = (PT)(3u - 2u * ((win >> 4) & 1u)) << ((win >> 5) & pmask);
    // Within a zero run (not fresh) the class reads as a run (X = 0).
    const uint32_t cls = fresh ? tz : 1u;
    PT x = cls >= 5 ? ones : (PT)0;
    x = cls == 0 ? verb : x;
    x = cls == 3 ? one_or_pair : x;
    x = cls == 4 ? above : x;  // the plane before the XOR is zero
    const uint32_t len = (uint32_t)(lut >> (8 * tz)) & 0xFFu;
    // Planes left in a zero run: a fresh run code sets them, every live
    // plane uses one (as arithmetic on masks: written as selects, the
    // update is compiled into exec-mask branches).
    const uint32_t fm = 0u - (uint32_t)(fresh && active);  // other lanes keep their position
    const uint32_t newrun = (tz == 1 ? ((win >> 2) & ((1u << R) - 1u)) + 1u : 0u) & fm;
    pos += len & fm;
    run = newrun | ((run - (uint32_t)live) & ~fm);
    const PT p = live ? (x ^ above) : (PT)0;
    above = live ? p : above;
    if (j < W) {
      const PT ps = dbx ? (PT)(p << 1) : p;
      if constexpr (W == 16) {
        t[j] = (uint32_t)ps;
        t[j + 16] = (uint32_t)((uint64_t)ps >> 32);
      } else {
        t[j] = (uint32_t)ps;
      }
    }
  }
}

// Decode: one workgroup per tile of 8 chunks (256 blocks). The chunk
// payloads are staged in LDS; every block's own thread recognises an
// all-zero block (coded as one zero run over all planes) and the rest are
// packed into the lowest slots, so that only ceil(n / 64) waves run the
// decoders. Decoded blocks are gathered in LDS rows (stride 33 dwords, which
// keeps lane-strided row access conflict free) over the dead payloads, and
// the group's 32 KB of output leaves in coalesced 16-byte stores.
constexpr int kDecWaves = 4;  // waves per workgroup
constexpr int kDecThreads = kWave * kDecWaves;
constexpr int kDecodeChunks = kDecThreads / kBlocksPerChunk;  // 8
constexpr int kDecodeBufDwords = kDecodeChunks * kChunkBufDwords;
constexpr int kDecodeRowDwords = kDecThreads * kLaneStride;
constexpr int kDecodeLdsDwords =
    kDecodeBufDwords > kDecodeRowDwords ? kDecodeBufDwords : kDecodeRowDwords;

struct __attribute__((aligned(16))) DecodeShared {
  uint32_t lds[kDecodeLdsDwords];
  uint32_t blk_info[kDecThreads];      // per packed block: bit position | tag << 16 | raw << 19
  uint8_t slot_block[kDecThreads];     // packed slot -> block of the group
  uint32_t chunk_lead[kDecodeChunks];  // bit offset of each payload in its buffer
  uint32_t wave_busy[kDecWaves];
};

// Decodes groups gtile0 .. gtile0 + NG - 1 (of 8 chunks each) of tensor k,
// one after another. The metadata and payload loads of all NG groups are
// issued at the start, so that the later groups' staging is not waited for.
// With set_status, group 0 writes the call's status from the error word
// (locate must be complete). kShared: the offsets come from locate tiles of
// the same launch and are read at device scope (decompress_kernel).
template <int W, bool kShared, int NG>
PZ_DEV void decode_group(const DBatch &batch, uint32_t k, uint64_t gtile0, const uint32_t *err_words, uint32_t epoch,
                         const DMode &mode, bool set_status, DecodeShared &sh) {
  constexpr int N = 1024 / W;
  constexpr uint32_t WMASK = W == 16 ? 0xFFFFu : 0xFFFFFFFFu;
  uint32_t *lds = sh.lds;
  uint32_t *blk_info = sh.blk_info;
  uint8_t *slot_block = sh.slot_block;
  uint32_t *chunk_lead = sh.chunk_lead;
  uint32_t *wave_busy = sh.wave_busy;

  const uint32_t t = threadIdx.x, lane = lane_id();
  const uint32_t wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint8_t *__restrict__ src = batch.t[k].src;
  uint8_t *__restrict__ dst = batch.t[k].dst;
  const uint64_t comp_bytes = batch.t[k].comp_bytes, raw_bytes = batch.t[k].raw_bytes;
  const uint64_t nchunks = batch.t[k].nchunks;
  const uint64_t *__restrict__ chunk_off = batch.t[k].chunk_off;
  const uint16_t *__restrict__ block_off = batch.t[k].block_off;
  const uint32_t *err = err_words + k;
  int32_t *status = batch.t[k].status;
  if (gtile0 * kDecodeChunks >= nchunks) return;
  // The call's status: locate, complete before this group, marked a corrupt
  // stream with the call's epoch.
  if (set_status && gtile0 == 0 && t == 0 && status)
    *status = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch ? kStatusCorrupt : 0;

  // Every thread's metadata at once: its chunk's payload offset and header
  // and its block's bit offset, so that the staging below waits for one
  // round trip before its payload loads, and the classification none.
  const uint16_t *hdr = reinterpret_cast<const uint16_t *>(src);
  uint64_t gm_coff[NG];
  uint32_t gm_H[NG], gm_boff[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint64_t block = (gtile0 + g) * kDecThreads + t;
    const uint64_t chunk = block >> 5;
    gm_coff[g] = kBadChunk;
    gm_H[g] = 0;
    gm_boff[g] = 0;
    if (chunk < nchunks) {
      if constexpr (kShared) {
        gm_coff[g] = __hip_atomic_load(chunk_off + chunk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        gm_boff[g] = __hip_atomic_load(block_off + block, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        gm_coff[g] = chunk_off[chunk];
        gm_boff[g] = block_off[block];
      }
      gm_H[g] = hdr[chunk];
    }
  }

  // --- 1. Payload loads: wave w takes chunks 2w and 2w+1 of every group
  // (whose metadata its lanes 0 and 32 hold). A payload is at most 258
  // 16-byte units, five per lane: every load is issued before any is
  // stored, so that the wave waits for memory once. ---
  constexpr int kStageUnits = (kChunkBufDwords / 4 + kWave - 1) / kWave;
  uint4 sv[NG][2][kStageUnits];
  uint32_t snq[NG][2], sfull[NG][2], slead[NG][2];
  uint64_t sq0[NG][2];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // Both halves zero-extended: readlane returns an int, and a sign-extended
      // low half would corrupt every offset with bit 31 set.
      const uint64_t coff =
          (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)gm_coff[g], 32 * h) |
          ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(gm_coff[g] >> 32), 32 * h) << 32);
      const uint32_t H = (uint32_t)__builtin_amdgcn_readlane((int)gm_H[g], 32 * h);
      const uint64_t q0 = (coff >> 2) & ~3ull;
      slead[g][h] = coff == kBadChunk ? 0u : (uint32_t)(8 * (coff - 4 * q0));
      const uint32_t nq = coff == kBadChunk ? 0u : ((uint32_t)(coff - 4 * q0) + H + 15) / 16;
      // Units wholly inside the stream (the others, at its very end, are read
      // byte by byte below); the loads are unconditional, clamped to the last
      // such unit, so that none waits for another.
      const uint64_t inside = comp_bytes > 4 * q0 ? (comp_bytes - 4 * q0) / 16 : 0;
      const uint32_t nfull = nq < inside ? nq : (uint32_t)inside;
      snq[g][h] = nq;
      sfull[g][h] = nfull;
      sq0[g][h] = q0;
      const uint4 *gp = reinterpret_cast<const uint4 *>(src + 4 * q0);
      if (nfull > 0) {  // wave-uniform
#pragma unroll
        for (int kk = 0; kk < kStageUnits; ++kk) {
          const uint32_t u = lane + (uint32_t)kWave * kk;
          sv[g][h][kk] = gp[u < nfull ? u : nfull - 1];
        }
      }
    }
  }

#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint64_t gtile = gtile0 + g;
    if (gtile * kDecodeChunks >= nchunks) break;
    if (g > 0) __syncthreads();  // the previous group's rows are stored: LDS is free
    const uint64_t gblock0 = gtile * kDecThreads;  // first block of the group
    const uint64_t block = gblock0 + t;
    const uint64_t chunk = block >> 5;
    const uint64_t my_coff = gm_coff[g];
    const uint32_t my_H = gm_H[g], my_boff = gm_boff[g];
    // Stage the group's 8 payloads (dword-aligned copies).
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (lane == 0) chunk_lead[2 * wave + (uint32_t)h] = slead[g][h];
      uint4 *buf4 = reinterpret_cast<uint4 *>(lds + (2 * wave + (uint32_t)h) * kChunkBufDwords);
#pragma unroll
      for (int kk = 0; kk < kStageUnits; ++kk) {
        const uint32_t u = lane + (uint32_t)kWave * kk;
        if (u >= snq[g][h]) continue;
        const uint64_t b = 4 * sq0[g][h] + 16ull * u;
        if (u >= sfull[g][h]) {
          // The stream's last bytes: byte loads below comp_bytes, zeros above.
          uint32_t tv[4] = {0, 0, 0, 0};
#pragma unroll 1
          for (uint32_t q = 0; q < 16 && b + q < comp_bytes; ++q) {
            const uint32_t x = (uint32_t)src[b + q] << (8 * (q & 3));
            if (q < 4) tv[0] |= x; else if (q < 8) tv[1] |= x; else if (q < 12) tv[2] |= x; else tv[3] |= x;
          }
          sv[g][h][kk] = make_uint4(tv[0], tv[1], tv[2], tv[3]);
        }
        buf4[u] = sv[g][h][kk];
      }
    }
    __syncthreads();

    // --- 2. Block t: all-zero blocks stay here, the rest go to the slot list. ---
    bool busy = false;
    {
      const uint32_t ci = t >> 5;
      const uint64_t coff = my_coff;
      const uint32_t H = my_H;
      const uint32_t raw_len = chunk < nchunks ? (uint32_t)min_u64(kChunkBytes, raw_bytes - chunk * kChunkBytes) : 0u;
      const bool ok = block * kBlockBytes < raw_bytes && coff != kBadChunk;
      const bool raw_chunk = ok && H == raw_len;
      const bool coded = ok && !raw_chunk;
      // Bit positions from here on count from the start of the chunk's
      // buffer (its lead added once; at most 31 * 1024 + 1024 + 120 bits, so
      // they fit the 16-bit field below).
      const uint32_t lead = chunk_lead[ci];
      uint32_t pos = lead + 1024u * (t & 31), head = 0;
      if (coded) {
        const LdsBits in{lds + ci * kChunkBufDwords, 0u};
        pos = lead + my_boff;
        head = in.peek(pos);
        pos += 3u * mode.tagged;
      }
      const bool zero = coded && (head & mode.zmask) == mode.zcode;
      const uint32_t tag = mode.tagged ? head & 7u : mode.fixed;
      busy = raw_chunk || (coded && !zero);
      if (busy) blk_info[t] = pos | (tag << 16) | ((uint32_t)raw_chunk << 19);
    }
    const uint64_t bmask = __ballot(busy);
    if (lane == 0) wave_busy[wave] = (uint32_t)popc64(bmask);
    __syncthreads();
    uint32_t nbusy = 0, first = 0;
#pragma unroll
    for (int k = 0; k < kDecWaves; ++k) {
      const uint32_t c = wave_busy[k];
      first += (uint32_t)k < wave ? c : 0u;
      nbusy += c;
    }
    if (busy) slot_block[first + lanes_below(bmask)] = (uint8_t)t;
    __syncthreads();

    // --- 3. Packed slots: raw copy, ZVC or plane decoding into d. Waves take the
    // slots in an order rotated per tile, so that the busy waves of successive
    // groups fall on different SIMDs. ---
    const uint32_t slot = (t + kDecThreads - 64u * (uint32_t)(gtile % kDecWaves)) % kDecThreads;
    const bool active = slot < nbusy;
    const bool wave_active = __ballot(active) != 0;
    uint32_t sb = 0;
    uint64_t nzmask = 0;
    bool want_spread = false;  // ZVC or ZBX: symbols in order of the non-zero positions
    uint32_t d[32];
    if (wave_active) {
      uint32_t pos = 0, tag = kBX;
      bool raw_chunk = false;
      if (active) {
        sb = slot_block[slot];
        const uint32_t info = blk_info[sb];
        pos = info & 0xFFFFu;
        tag = (info >> 16) & 7u;
        raw_chunk = (info >> 19) & 1u;
      }
      const LdsBits in{lds + (sb >> 5) * kChunkBufDwords, 0u};  // positions include the lead

      const bool coded = active && !raw_chunk;
      const bool want_raw = active && (raw_chunk || tag == kRAW);
      const bool want_zvc = coded && tag == kZVC;
      const bool want_dbx = coded && tag == kDBX;
      const bool want_planes = coded && (tag == kDBX || tag == kBX || tag == kZBX);
      const bool want_zbx = coded && tag == kZBX;
      // Zero mask of ZVC and ZBX (bit i = symbol i non-zero).
      if (want_zvc || want_zbx) {
        nzmask = W == 16 ? in.peek64(pos) : (uint64_t)in.peek(pos);
        pos += N;
      }

      // Plane decoding first (it needs the most registers, and d is not yet
      // holding anything), then the raw and ZVC blocks fill d.
      if (__ballot(want_planes)) {
        uint32_t base = 0;
        if (want_dbx) {
          base = in.peek(pos) & WMASK;
          pos += W;
        }
        int K = W;
        uint32_t L = N;
        if (want_dbx) {
          K = W + 1;
          L = N - 1;
        } else if (want_zbx) {
          L = (uint32_t)popc64(nzmask);
        }
        uint32_t tp[32];
        read_planes<W>(in, pos, tp, K, L, want_dbx, want_planes);
        transpose32(tp);
        if constexpr (W == 16) {
          // tp[r] = symbol r | symbol r+32 << 16 -> d[i] = symbol 2i | symbol 2i+1 << 16.
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            if (i < 16)
              d[i] = (tp[2 * i] & 0xFFFFu) | (tp[2 * i + 1] << 16);
            else
              d[i] = (tp[2 * i - 32] >> 16) | (tp[2 * i - 31] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 32; ++i) d[i] = tp[i];
        }
        // DBX: running sum of the deltas from the base symbol, modulo 2^w.
        if (__ballot(want_dbx)) {
          if constexpr (W == 16) {
            uint32_t carry = base;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
              const uint32_t v = d[i];
              const uint32_t pair = v + (v << 16);  // (lo, lo + hi)
              const uint32_t outv = pk_add_u16(pair, carry | (carry << 16));
              d[i] = want_dbx ? outv : v;
              carry = outv >> 16;
            }
          } else {
            uint32_t acc = base;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
              acc += d[i];
              d[i] = want_dbx ? acc : d[i];
            }
          }
        }
      }

      // Raw chunks and RAW blocks: 1024 bits verbatim. ZVC: its payload, the
      // non-zero symbols in order (the same layout as ZBX's compacted
      // symbols), spread to their positions below.
      const bool want_copy = want_raw || want_zvc;
      if (__ballot(want_copy)) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t v = in.peek(pos + 32 * i);
          d[i] = want_copy ? v : d[i];
        }
      }
      want_spread = want_zvc || want_zbx;
    }
    __syncthreads();  // payloads dead: LDS becomes the output rows

    // --- 4. Output rows. All-zero (and unusable) blocks: zeros. Packed blocks:
    // their symbols; ZVC and ZBX spread the non-zero symbols to their
    // positions in place. ---
    if (!busy) {
      uint32_t *row = lds + t * kLaneStride;
#pragma unroll
      for (int i = 0; i < 32; ++i) row[i] = 0;
    }
    if (wave_active) {
      uint32_t *row = lds + sb * kLaneStride;
      if (active) {
#pragma unroll
        for (int i = 0; i < 32; ++i) row[i] = d[i];
      }
      if (__ballot(want_spread)) {
        wave_lds_fence();
        if (want_spread) {
          // Symbol i takes compacted symbol rank(i) = number of non-zero symbols
          // before it. Every read is issued (rank <= N stays inside the padded
          // row) and the zero positions are selected away, so the reads need no
          // branches and no wait between them.
          uint32_t rank = 0;
          if constexpr (W == 16) {
            const uint16_t *r16 = reinterpret_cast<const uint16_t *>(row);
#pragma unroll
            for (int i = 0; i < 32; ++i) {
              const bool n0 = (nzmask >> (2 * i)) & 1u, n1 = (nzmask >> (2 * i + 1)) & 1u;
              const uint32_t a = r16[rank];
              rank += n0 ? 1u : 0u;
              const uint32_t b = r16[rank];
              rank += n1 ? 1u : 0u;
              d[i] = (n0 ? a : 0u) | ((n1 ? b : 0u) << 16);
            }
          } else {
#pragma unroll
            for (int k = 0; k < 32; ++k) {
              const bool n0 = (nzmask >> k) & 1u;
              const uint32_t a = row[rank];
              rank += n0 ? 1u : 0u;
              d[k] = n0 ? a : 0u;
            }
          }
        }
        wave_lds_fence();
        if (want_spread) {
#pragma unroll
          for (int i = 0; i < 32; ++i) row[i] = d[i];
        }
      }
    }
    __syncthreads();

    // --- 5. Coalesced store of the group's output span (bytes past raw_bytes
    // are not written). (Each lane storing its own block's 128 bytes from
    // registers, eight 16-byte stores 128 bytes apart across the lanes, made
    // decompression 2.8 times slower.) ---
    const uint64_t span0 = gblock0 * kBlockBytes;
    const uint64_t span_end = min_u64(raw_bytes, span0 + (uint64_t)kDecThreads * kBlockBytes);
    const uint32_t span = (uint32_t)(span_end - span0);
#pragma unroll
    for (int k = 0; k < kBlocksPerChunk / 4; ++k) {
      const uint32_t u = t + (uint32_t)k * kDecThreads;  // 16-byte unit of the span
      const uint32_t b0 = 16 * u;
      if (b0 >= span) continue;
      const uint32_t *row = lds + (u >> 3) * kLaneStride + 4 * (u & 7);
      const uint4 v = make_uint4(row[0], row[1], row[2], row[3]);
      if (b0 + 16 <= span) {
        // Non-temporal: the codec never reads its output back (1-2% faster).
        const u32x4 q = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(dst + span0 + b0));
      } else {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        for (uint32_t bb = b0; bb < span; ++bb)
          dst[span0 + bb] = (uint8_t)(w4[(bb - b0) >> 2] >> (8 * ((bb - b0) & 3)));
      }
    }
  }
}

template <int W>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DBatch batch, const uint32_t *err_words,
                                                               uint32_t epoch, DMode mode) {
  __shared__ DecodeShared sh;
  // The launch's group -> the tensor it belongs to and the group within it.
  uint32_t k = 0;
  if (batch.n > 1) {  // a single tensor's fields load at once
#pragma unroll
    for (uint32_t i = 1; i < (uint32_t)kMaxBatch; ++i) k += i < batch.n && blockIdx.x >= batch.t[i].group_begin ? 1u : 0u;
  }
  decode_group<W, false, 1>(batch, k, blockIdx.x - batch.t[k].group_begin, err_words, epoch, mode, true, sh);
}

// Both halves in one launch, for launches of many tiles. Workgroups take
// tickets in the order they start: tickets 0 .. T-1 locate tiles 0 .. T-1,
// ticket T + j decodes groups 2j and 2j + 1, numbered by tile (tile u holds
// groups 8u .. 8u+7 of its tensor; those past the tensor's last chunk are
// skipped). A decode ticket waits for its tile's flag, and that tile always
// has an earlier ticket, so every wait is on a workgroup that is running or
// done. The decode groups of the first tiles thus run beside the last
// walks, where two launches would leave the GPU partly idle at the end of
// the walks and between the kernels.
//
// Hand-over without cache maintenance: locate stores the offsets at device
// scope (written through to the coherence point, as relaxed atomics), and
// each wave waits until its stores and its error-word update are performed
// before the tile's flag is set; decode reads the flag and then the offsets
// with device-scope loads (served from the coherence point). These are the
// steps the gfx9 memory model takes for atomics; a release/acquire pair at
// device scope would add an L2 write-back per locate wave and an L2
// invalidation per decode group, which measured 60% slower.
static_assert(kLocateChunks == 8 * kDecodeChunks, "a locate tile is eight decode groups");
// Decode groups per ticket of the single kernel (the second group's loads
// are issued with the first's: measured on the GPT-2-XL batch, 2 groups per
// ticket decompressed 3% faster than 1, and 4 or 8, with the next group
// prefetched while one is decoded, 7% and 12% slower), and decode tickets per
// tile.
constexpr uint32_t kFusedGroups = 2;
constexpr uint32_t kDecodeTickets = 8 / kFusedGroups;
static_assert(kDecodeTickets * kFusedGroups == 8, "a tile's groups split evenly over its tickets");
static_assert(kLocateThreads == kDecThreads, "one workgroup size for both halves");

// (The second launch bound, four waves per SIMD, caps a lane at 128 VGPRs:
// the two staged groups of a decode ticket take 124.)
template <int W, int G>
__global__ __launch_bounds__(kDecThreads, 4) void decompress_kernel(const DBatch batch, uint32_t *err_words,
                                                                   uint32_t epoch, uint64_t *lb_words,
                                                                   uint32_t *tile_counter, uint32_t counter_base,
                                                                   uint32_t *done, uint32_t done_base, DMode mode) {
  __shared__ union {
    LocateShared<G> l;
    DecodeShared d;
  } sh;
  __shared__ uint32_t ticket_s;
  static_assert(locate_chunks<G>() == 8 * kDecodeChunks, "a locate tile is eight decode groups");
  const uint32_t t = threadIdx.x;
  if (t == 0) ticket_s = atomicAdd(tile_counter, 1u) - counter_base;
  __syncthreads();
  const uint32_t ticket = __builtin_amdgcn_readfirstlane(ticket_s);
  const uint32_t T = batch.total_tiles;
  const bool loc = ticket < T;
  const uint32_t tile = loc ? ticket : (ticket - T) / kDecodeTickets;
  if (tile >= T) return;
  const uint32_t k = tensor_of_tile(batch, tile);
  uint64_t *flag = lb_words + (uint64_t)tile * kLookbackStride + 1;  // beside the tile's look-back word
  if (loc) {
    locate_tile<W, G, true>(batch, k, tile, err_words, epoch, lb_words, mode, sh.l);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's offset stores and error update performed
    __syncthreads();
    if (t == 0) {
      __hip_atomic_store(flag, (uint64_t)epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t before = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (before - done_base == T - 1u) {
        // The launch's last tile located: every error word is final.
        for (uint32_t m = 0; m < batch.n; ++m)
          if (batch.t[m].status)
            *batch.t[m].status =
                __hip_atomic_load(err_words + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch ? kStatusCorrupt : 0;
      }
    }
  } else {
    const uint64_t g =
        (uint64_t)(tile - batch.t[k].tile_begin) * 8u + ((ticket - T) % kDecodeTickets) * kFusedGroups;
    if (g * kDecodeChunks >= batch.t[k].nchunks) return;
    if (t == 0) {
      while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (uint64_t)epoch)
        __builtin_amdgcn_s_sleep(16);
    }
    __syncthreads();
    decode_group<W, true, kFusedGroups>(batch, k, g, err_words, epoch, mode, false, sh.d);
  }
}

// Sets a decompress call's status when it launches no kernel (an empty
// tensor).
__global__ void set_status_kernel(int32_t *status, int32_t value) { *status = value; }

hipError_t launch_empty_status(int32_t *status, uint64_t comp_bytes, hipStream_t stream) {
  if (!status) return hipSuccess;
  hipLaunchKernelGGL(set_status_kernel, dim3(1), dim3(1), 0, stream, status,
                     comp_bytes != 0 ? kStatusCorrupt : 0);
  return hipGetLastError();
}


uint32_t decode_groups(uint64_t raw_bytes) {
  const uint64_t nchunks = (raw_bytes + kChunkBytes - 1) / kChunkBytes;
  return (uint32_t)((nchunks + kDecodeChunks - 1) / kDecodeChunks);
}

// Per tensor: chunk offsets (8 bytes per chunk), then block offsets (64 bytes
// per chunk), each 16-byte aligned.
size_t decompress_extra(uint64_t raw_bytes) {
  const uint64_t nchunks = (raw_bytes + kChunkBytes - 1) / kChunkBytes;
  return (size_t)(((nchunks + 1) & ~1ull) * 8 + nchunks * kBlocksPerChunk * 2);
}

// Launches of fewer tiles take two kernels: there every decode group of the
// launch would be resident from the start, waiting beside the walks, and
// the walks measured 4-28% slower for it (73-400 tiles); from 768 tiles on
// the single launch was 10-12% faster.
constexpr uint32_t kFusedMinTiles = 512;

// The form is chosen on the launch's count of 64-chunk tiles; outside the
// single kernel, 32-bit symbols walk with 8 lanes per chunk, in tiles of 32.
void plan_decompress(int w, DBatch &b) {
  uint64_t tiles = 0;
  for (uint32_t k = 0; k < b.n; ++k) tiles += (b.t[k].nchunks + kLocateChunks - 1) / kLocateChunks;
  b.fused = tiles >= kFusedMinTiles ? 1u : 0u;
  b.locate_lanes = !b.fused && w == 32 ? kLocateLanesWide : kLocateLanes;
  const uint64_t per_tile = (uint64_t)kLocateThreads / b.locate_lanes;
  b.total_tiles = 0;
  for (uint32_t k = 0; k < b.n; ++k) {
    DTensor &x = b.t[k];
    x.tile_begin = b.total_tiles;
    x.ntiles = (uint32_t)((x.nchunks + per_tile - 1) / per_tile);
    b.total_tiles += x.ntiles;
  }
}

ScratchNeed decompress_need(const DBatch &b, size_t extra) {
  if (b.fused)
    return ScratchNeed{b.total_tiles * kLookbackStride, extra, (1 + kDecodeTickets) * b.total_tiles, b.total_tiles};
  return ScratchNeed{b.total_tiles * kLookbackStride, extra, b.total_tiles, 0};
}

hipError_t launch_decompress(int w, DBatch &batch, uint32_t codec_mask, int tagged,
                             const Scratch &scratch, hipStream_t stream) {
  const DMode mode = make_dmode(w, codec_mask, tagged);
  uint8_t *extra = scratch.extra;
  for (uint32_t k = 0; k < batch.n; ++k) {
    DTensor &x = batch.t[k];
    x.chunk_off = reinterpret_cast<uint64_t *>(extra);
    x.block_off = reinterpret_cast<uint16_t *>(extra + ((x.nchunks + 1) & ~1ull) * 8);
    extra += decompress_extra(x.raw_bytes);
  }
  if (batch.fused) {
    const dim3 grid((1 + kDecodeTickets) * batch.total_tiles);  // T locate tiles, then the decode tickets
    if (w == 16)
      hipLaunchKernelGGL((decompress_kernel<16, kLocateLanes>), grid, dim3(kDecThreads), 0, stream, batch, scratch.err,
                         scratch.epoch, scratch.words, scratch.counter, scratch.counter_base, scratch.done,
                         scratch.done_base, mode);
    else
      hipLaunchKernelGGL((decompress_kernel<32, kLocateLanes>), grid, dim3(kDecThreads), 0, stream, batch, scratch.err,
                         scratch.epoch, scratch.words, scratch.counter, scratch.counter_base, scratch.done,
                         scratch.done_base, mode);
    return hipGetLastError();
  }
  const dim3 grid_a(batch.total_tiles);
  if (w == 16 && batch.locate_lanes == kLocateLanes)
    hipLaunchKernelGGL((locate_kernel<16, kLocateLanes>), grid_a, dim3(kLocateThreads), 0, stream, batch,
                       scratch.err, scratch.epoch, scratch.words, scratch.counter, scratch.counter_base, mode);
  else if (w == 32 && batch.locate_lanes == kLocateLanesWide)
    hipLaunchKernelGGL((locate_kernel<32, kLocateLanesWide>), grid_a, dim3(kLocateThreads), 0, stream, batch,
                       scratch.err, scratch.epoch, scratch.words, scratch.counter, scratch.counter_base, mode);
  else
    return hipErrorInvalidValue;  // a batch that plan_decompress did not number
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid_b(batch.total_groups);
  if (w == 16)
    hipLaunchKernelGGL(decode_kernel<16>, grid_b, dim3(kDecThreads), 0, stream, batch, scratch.err,
                       scratch.epoch, mode);
  else
    hipLaunchKernelGGL(decode_kernel<32>, grid_b, dim3(kDecThreads), 0, stream, batch, scratch.err,
                       scratch.epoch, mode);
  return hipGetLastError();
}

}  // namespace pz
