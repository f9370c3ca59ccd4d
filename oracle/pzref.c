/*
 * pzref.c — plain CPU oracle of the PlaneZip block codec.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
 * baseline of the benchmark, never by the product path. It shares no code,
 * header, table or helper with the HIP library.
 *
 * Everything here is written for obviousness, not speed: bits are moved one
 * at a time, planes are built one bit at a time, and a block is encoded in all
 * five ways before the smallest is kept, exactly as the paper describes the
 * engine (PlaneZip paper, §III-A and Fig. 2: the engine tries all four
 * encodings on every 128-byte block at once and keeps the shortest, or the
 * block itself).
 * The bit layout is FORMAT.md version 1.
 */
#include "pzref.h"

#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define BLOCK_BYTES 128
#define CHUNK_BYTES 4096
#define BLOCKS_PER_CHUNK 32
/* Largest candidate payload is DBX/ZBX at 16 + 17*65 bits; round up. */
#define CAND_BUF_BYTES 256
/* A chunk is coded in full before the raw decision (a chunk that does not
 * shrink is kept raw, §III-A), so the buffer holds 32 blocks of the largest
 * candidate plus its tag: with RAW allowed a block is at most 3 + 1024 bits,
 * but a mode without RAW (a single-codec variant) can reach
 * 3 + CAND_BUF_BYTES * 8 bits. */
#define CHUNK_BUF_BYTES (BLOCKS_PER_CHUNK * (CAND_BUF_BYTES + 1))

/* ------------------------------------------------------------------------ */
/* Bit I/O. Stream bit t is bit (t % 8) of byte (t / 8); a field is written  */
/* least-significant bit first (FORMAT.md §2).                               */
/* ------------------------------------------------------------------------ */

typedef struct {
    uint8_t *buf;
    int64_t cap_bits;
    int64_t pos;
    int overflow;
} bitwriter;

static void put_bits(bitwriter *bw, uint64_t value, int nbits)
{
    for (int i = 0; i < nbits; i++) {
        if (bw->pos >= bw->cap_bits) {
            bw->overflow = 1;
        } else if ((value >> i) & 1u) {
            bw->buf[bw->pos >> 3] |= (uint8_t)(1u << (bw->pos & 7));
        }
        bw->pos++;
    }
}

typedef struct {
    const uint8_t *buf;
    int64_t end_bits;
    int64_t pos;
    int overrun;
} bitreader;

static uint64_t get_bits(bitreader *br, int nbits)
{
    uint64_t value = 0;
    for (int i = 0; i < nbits; i++) {
        if (br->pos >= br->end_bits) {
            br->overrun = 1;
            return 0;
        }
        if ((br->buf[br->pos >> 3] >> (br->pos & 7)) & 1u)
            value |= (uint64_t)1 << i;
        br->pos++;
    }
    return value;
}

/* ------------------------------------------------------------------------ */
/* Small helpers                                                             */
/* ------------------------------------------------------------------------ */

int pzref_width(int dtype, int elem_bits)
{
    /* §III-A: w is the element width: 16 for BF16, 32 for FP32, and 32 for
     * every other type. BF16 may also be coded with 32-bit symbols (§V-A). */
    if (dtype == 0 && (elem_bits == 16 || elem_bits == 32)) return elem_bits;
    if (dtype == 1 && elem_bits == 32) return 32;
    if (dtype == 2 && elem_bits == 32) return 32;
    return -1;
}

size_t pzref_num_chunks(size_t raw_bytes)
{
    return (raw_bytes + CHUNK_BYTES - 1) / CHUNK_BYTES;
}

size_t pzref_max_compressed(size_t raw_bytes)
{
    return 2 * pzref_num_chunks(raw_bytes) + raw_bytes;
}

static int valid_width(int w) { return w == 16 || w == 32; }

/* Zero-run length field width R = log2(w). */
static int run_field_bits(int w) { return w == 16 ? 4 : 5; }

/* Position field width: ceil(log2 L) for L >= 2, else 0. */
static int position_bits(int L)
{
    int pw = 0;
    while (L >= 2 && (1 << pw) < L) pw++;
    return pw;
}

static uint64_t all_ones(int L)
{
    if (L <= 0) return 0;
    if (L >= 64) return ~(uint64_t)0;
    return ((uint64_t)1 << L) - 1;
}

static int count_ones(uint64_t x)
{
    int c = 0;
    for (int i = 0; i < 64; i++) c += (int)((x >> i) & 1u);
    return c;
}

static int lowest_one(uint64_t x)
{
    for (int i = 0; i < 64; i++)
        if ((x >> i) & 1u) return i;
    return -1;
}

/* Symbol i = little-endian unsigned integer of w bits at byte i*w/8. */
static void read_symbols(const uint8_t *block, int w, uint32_t *sym)
{
    int bytes = w / 8;
    int n = 1024 / w;
    for (int i = 0; i < n; i++) {
        uint32_t v = 0;
        for (int b = 0; b < bytes; b++)
            v |= (uint32_t)block[i * bytes + b] << (8 * b);
        sym[i] = v;
    }
}

static void write_symbols(const uint32_t *sym, int w, uint8_t *block)
{
    int bytes = w / 8;
    int n = 1024 / w;
    for (int i = 0; i < n; i++)
        for (int b = 0; b < bytes; b++)
            block[i * bytes + b] = (uint8_t)(sym[i] >> (8 * b));
}

/* ------------------------------------------------------------------------ */
/* The plane coder: BPC's prefix code as sized in §III-A.                    */
/* ------------------------------------------------------------------------ */

/* Codes as stream-order bit strings, stored as LSB-first field values:
 *   "1" -> 1 (1 bit)         verbatim plane follows
 *   "01" -> 2 (2 bits)       zero run of k >= 2 planes, k-2 follows
 *   "001" -> 4 (3 bits)      one zero plane
 *   "00000" -> 0 (5 bits)    all-ones plane
 *   "00001" -> 16 (5 bits)   plane whose pre-XOR value is zero
 *   "00010" -> 8 (5 bits)    two adjacent ones, position follows
 *   "00011" -> 24 (5 bits)   a single one, position follows            */
static void code_planes(bitwriter *bw, const uint64_t *P, int K, int L, int R)
{
    uint64_t X[33];
    int pw = position_bits(L);

    /* XOR adjacent planes; the top plane is kept as is. */
    for (int j = 0; j < K; j++)
        X[j] = P[j] ^ (j + 1 < K ? P[j + 1] : 0);

    int j = K - 1;
    while (j >= 0) {
        if (X[j] == 0) {
            int k = 0;
            while (j - k >= 0 && X[j - k] == 0) k++;
            if (k == 1) {
                put_bits(bw, 4, 3);
            } else {
                put_bits(bw, 2, 2);
                put_bits(bw, (uint64_t)(k - 2), R);
            }
            j -= k;
            continue;
        }
        uint64_t x = X[j];
        int ones = count_ones(x);
        int low = lowest_one(x);
        if (x == all_ones(L)) {
            put_bits(bw, 0, 5);
        } else if (P[j] == 0) {
            put_bits(bw, 16, 5);
        } else if (ones == 2 && x == ((uint64_t)3 << low)) {
            put_bits(bw, 8, 5);
            put_bits(bw, (uint64_t)low, pw);
        } else if (ones == 1) {
            put_bits(bw, 24, 5);
            put_bits(bw, (uint64_t)low, pw);
        } else {
            put_bits(bw, 1, 1);
            put_bits(bw, x, L);
        }
        j--;
    }
}

/* Inverse of code_planes. Returns PZREF_OK or PZREF_ECORRUPT. */
static int decode_planes(bitreader *br, uint64_t *P, int K, int L, int R)
{
    int pw = position_bits(L);
    uint64_t above = 0; /* P[j+1]; P[K] is zero */
    int j = K - 1;
    while (j >= 0) {
        uint64_t x;
        if (get_bits(br, 1)) {                 /* "1": verbatim */
            x = get_bits(br, L);
            P[j] = x ^ above;
        } else if (get_bits(br, 1)) {          /* "01": zero run */
            int k = (int)get_bits(br, R) + 2;
            if (br->overrun) return PZREF_ECORRUPT;
            if (k > j + 1) return PZREF_ECORRUPT;
            for (int i = 0; i < k; i++) P[j - i] = above;
            j -= k;
            continue;
        } else if (get_bits(br, 1)) {          /* "001": one zero plane */
            P[j] = above;
        } else {
            int low2 = (int)get_bits(br, 2);   /* fourth and fifth code bits */
            if (low2 == 0) {                   /* "00000": all ones */
                P[j] = all_ones(L) ^ above;
            } else if (low2 == 2) {            /* "00001": pre-XOR zero */
                P[j] = 0;
            } else {                           /* "00010" pair / "00011" one */
                int p = (int)get_bits(br, pw);
                if (low2 == 1) {
                    if (p > L - 2) return PZREF_ECORRUPT;
                    x = (uint64_t)3 << p;
                } else {
                    if (p > L - 1) return PZREF_ECORRUPT;
                    x = (uint64_t)1 << p;
                }
                P[j] = x ^ above;
            }
        }
        if (br->overrun) return PZREF_ECORRUPT;
        above = P[j];
        j--;
    }
    return br->overrun ? PZREF_ECORRUPT : PZREF_OK;
}

/* ------------------------------------------------------------------------ */
/* The five candidates of §III-A.                                            */
/* ------------------------------------------------------------------------ */

/* ZVC: an N-bit mask marking the symbols that are not zero, then those
 * symbols in order. */
static void encode_zvc(bitwriter *bw, const uint32_t *s, int w)
{
    int n = 1024 / w;
    for (int i = 0; i < n; i++) put_bits(bw, s[i] != 0, 1);
    for (int i = 0; i < n; i++)
        if (s[i] != 0) put_bits(bw, s[i], w);
}

/* DBX: base symbol, then w+1 planes of the N-1 neighbour deltas. */
static void encode_dbx(bitwriter *bw, const uint32_t *s, int w)
{
    int n = 1024 / w;
    int K = w + 1;
    int L = n - 1;
    uint64_t P[33];
    memset(P, 0, sizeof P);
    uint64_t mask = ((uint64_t)1 << (w + 1)) - 1;
    for (int k = 0; k < L; k++) {
        int64_t d = (int64_t)s[k + 1] - (int64_t)s[k];
        uint64_t D = (uint64_t)d & mask; /* (w+1)-bit two's complement */
        for (int j = 0; j < K; j++)
            if ((D >> j) & 1u) P[j] |= (uint64_t)1 << k;
    }
    put_bits(bw, s[0], w);
    code_planes(bw, P, K, L, run_field_bits(w));
}

/* BX: the w planes of the symbols themselves. */
static void encode_bx(bitwriter *bw, const uint32_t *s, int w)
{
    int n = 1024 / w;
    uint64_t P[33];
    memset(P, 0, sizeof P);
    for (int k = 0; k < n; k++)
        for (int j = 0; j < w; j++)
            if ((s[k] >> j) & 1u) P[j] |= (uint64_t)1 << k;
    code_planes(bw, P, w, n, run_field_bits(w));
}

/* ZBX: the same N-bit mask, then BX applied to the n non-zero symbols
 * packed together, so every plane is n bits wide. */
static void encode_zbx(bitwriter *bw, const uint32_t *s, int w)
{
    int n = 1024 / w;
    uint32_t c[64];
    int cnt = 0;
    for (int i = 0; i < n; i++) {
        put_bits(bw, s[i] != 0, 1);
        if (s[i] != 0) c[cnt++] = s[i];
    }
    uint64_t P[33];
    memset(P, 0, sizeof P);
    for (int k = 0; k < cnt; k++)
        for (int j = 0; j < w; j++)
            if ((c[k] >> j) & 1u) P[j] |= (uint64_t)1 << k;
    code_planes(bw, P, w, cnt, run_field_bits(w));
}

static void encode_raw(bitwriter *bw, const uint8_t *block)
{
    for (int i = 0; i < BLOCK_BYTES; i++) put_bits(bw, block[i], 8);
}

static void encode_one(bitwriter *bw, const uint8_t *block, const uint32_t *s,
                       int w, int cand)
{
    switch (cand) {
    case PZREF_ZVC: encode_zvc(bw, s, w); break;
    case PZREF_DBX: encode_dbx(bw, s, w); break;
    case PZREF_BX: encode_bx(bw, s, w); break;
    case PZREF_ZBX: encode_zbx(bw, s, w); break;
    default: encode_raw(bw, block); break;
    }
}

static int decode_one(bitreader *br, int w, int cand, uint8_t *block)
{
    int n = 1024 / w;
    int R = run_field_bits(w);
    uint32_t s[64];
    uint64_t P[33];
    memset(s, 0, sizeof s);
    memset(P, 0, sizeof P);

    if (cand == PZREF_RAW) {
        for (int i = 0; i < BLOCK_BYTES; i++) block[i] = (uint8_t)get_bits(br, 8);
        return br->overrun ? PZREF_ECORRUPT : PZREF_OK;
    }
    if (cand == PZREF_ZVC) {
        int nz[64];
        for (int i = 0; i < n; i++) nz[i] = (int)get_bits(br, 1);
        for (int i = 0; i < n; i++) s[i] = nz[i] ? (uint32_t)get_bits(br, w) : 0;
    } else if (cand == PZREF_DBX) {
        uint32_t base = (uint32_t)get_bits(br, w);
        int rc = decode_planes(br, P, w + 1, n - 1, R);
        if (rc != PZREF_OK) return rc;
        uint64_t wmask = ((uint64_t)1 << w) - 1;
        s[0] = base;
        for (int k = 0; k < n - 1; k++) {
            uint64_t D = 0;
            for (int j = 0; j <= w; j++)
                if ((P[j] >> k) & 1u) D |= (uint64_t)1 << j;
            s[k + 1] = (uint32_t)(((uint64_t)s[k] + D) & wmask);
        }
    } else if (cand == PZREF_BX) {
        int rc = decode_planes(br, P, w, n, R);
        if (rc != PZREF_OK) return rc;
        for (int k = 0; k < n; k++)
            for (int j = 0; j < w; j++)
                if ((P[j] >> k) & 1u) s[k] |= (uint32_t)1 << j;
    } else if (cand == PZREF_ZBX) {
        int nz[64];
        int cnt = 0;
        for (int i = 0; i < n; i++) {
            nz[i] = (int)get_bits(br, 1);
            cnt += nz[i];
        }
        if (br->overrun) return PZREF_ECORRUPT;
        int rc = decode_planes(br, P, w, cnt, R);
        if (rc != PZREF_OK) return rc;
        int k = 0;
        for (int i = 0; i < n; i++) {
            if (!nz[i]) continue;
            for (int j = 0; j < w; j++)
                if ((P[j] >> k) & 1u) s[i] |= (uint32_t)1 << j;
            k++;
        }
    } else {
        return PZREF_ECORRUPT;
    }
    if (br->overrun) return PZREF_ECORRUPT;
    write_symbols(s, w, block);
    return PZREF_OK;
}

/* ------------------------------------------------------------------------ */
/* Public single-block entry points                                          */
/* ------------------------------------------------------------------------ */

int pzref_encode_candidate(const uint8_t *block, int w, int cand, uint8_t *out,
                           size_t cap_bytes, int64_t *nbits)
{
    if (!valid_width(w) || cand < 0 || cand > 4) return PZREF_EINVAL;
    uint32_t s[64];
    read_symbols(block, w, s);
    memset(out, 0, cap_bytes);
    bitwriter bw = {out, (int64_t)cap_bytes * 8, 0, 0};
    encode_one(&bw, block, s, w, cand);
    *nbits = bw.pos;
    return bw.overflow ? PZREF_ENOSPC : PZREF_OK;
}

int pzref_decode_candidate(const uint8_t *in, int64_t in_bits, int w, int cand,
                           uint8_t *block, int64_t *consumed)
{
    if (!valid_width(w) || cand < 0 || cand > 4) return PZREF_EINVAL;
    bitreader br = {in, in_bits, 0, 0};
    int rc = decode_one(&br, w, cand, block);
    *consumed = br.pos;
    return rc;
}

int pzref_block_sizes(const uint8_t *block, int w, int32_t sizes[5])
{
    if (!valid_width(w)) return PZREF_EINVAL;
    uint8_t scratch[CAND_BUF_BYTES];
    for (int cand = 0; cand < 5; cand++) {
        int64_t nbits = 0;
        int rc = pzref_encode_candidate(block, w, cand, scratch, sizeof scratch, &nbits);
        if (rc != PZREF_OK) return rc;
        sizes[cand] = (int32_t)nbits;
    }
    return PZREF_OK;
}

int pzref_code_planes(const uint64_t *P, int K, int L, int R, uint8_t *out,
                      size_t cap_bytes, int64_t *nbits)
{
    if (K < 1 || K > 33 || L < 0 || L > 64 || R < 1 || R > 8) return PZREF_EINVAL;
    memset(out, 0, cap_bytes);
    bitwriter bw = {out, (int64_t)cap_bytes * 8, 0, 0};
    code_planes(&bw, P, K, L, R);
    *nbits = bw.pos;
    return bw.overflow ? PZREF_ENOSPC : PZREF_OK;
}

int pzref_decode_planes(const uint8_t *in, int64_t in_bits, int K, int L, int R,
                        uint64_t *P, int64_t *consumed)
{
    if (K < 1 || K > 33 || L < 0 || L > 64 || R < 1 || R > 8) return PZREF_EINVAL;
    bitreader br = {in, in_bits, 0, 0};
    int rc = decode_planes(&br, P, K, L, R);
    *consumed = br.pos;
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Chunks and streams (§III-A "Stream format")                               */
/* ------------------------------------------------------------------------ */

static int single_codec(uint32_t codec_mask)
{
    for (int t = 0; t < 5; t++)
        if (codec_mask == (1u << t)) return t;
    return -1;
}

static int check_mode(int w, uint32_t codec_mask, int tagged)
{
    if (!valid_width(w)) return PZREF_EINVAL;
    if (codec_mask == 0 || (codec_mask & ~PZREF_ALL_CODECS)) return PZREF_EINVAL;
    if (!tagged && single_codec(codec_mask) < 0) return PZREF_EINVAL;
    return PZREF_OK;
}

int64_t pzref_compress_chunk(const uint8_t *src, size_t raw_len, int w,
                             uint32_t codec_mask, int tagged, uint8_t *payload,
                             uint8_t *tags, int32_t *block_bits)
{
    int rc = check_mode(w, codec_mask, tagged);
    if (rc != PZREF_OK) return -rc;
    if (raw_len == 0 || raw_len > CHUNK_BYTES) return -PZREF_EINVAL;

    uint8_t buf[CHUNK_BUF_BYTES];
    memset(buf, 0, sizeof buf);
    bitwriter chunk = {buf, (int64_t)sizeof buf * 8, 0, 0};
    int nblocks = (int)((raw_len + BLOCK_BYTES - 1) / BLOCK_BYTES);

    for (int b = 0; b < nblocks; b++) {
        /* The last block is padded with zero bytes for encoding. */
        uint8_t block[BLOCK_BYTES];
        memset(block, 0, sizeof block);
        size_t off = (size_t)b * BLOCK_BYTES;
        size_t len = raw_len - off < BLOCK_BYTES ? raw_len - off : BLOCK_BYTES;
        memcpy(block, src + off, len);

        /* Size every allowed candidate and keep the smallest; ties go to the
         * lowest tag. */
        int32_t sizes[5];
        rc = pzref_block_sizes(block, w, sizes);
        if (rc != PZREF_OK) return -rc;
        int best = -1;
        for (int t = 0; t < 5; t++) {
            if (!(codec_mask & (1u << t))) continue;
            if (best < 0 || sizes[t] < sizes[best]) best = t;
        }

        int64_t start = chunk.pos;
        if (tagged) put_bits(&chunk, (uint64_t)best, 3);
        uint32_t s[64];
        read_symbols(block, w, s);
        encode_one(&chunk, block, s, w, best);
        if (tags) tags[b] = (uint8_t)best;
        if (block_bits) block_bits[b] = (int32_t)(chunk.pos - start);
    }
    if (chunk.overflow) return -PZREF_ENOSPC;

    /* Pad to a byte. A chunk that does not shrink is kept raw. */
    size_t coded = (size_t)((chunk.pos + 7) / 8);
    if (coded >= raw_len) {
        memcpy(payload, src, raw_len);
        return (int64_t)raw_len;
    }
    memcpy(payload, buf, coded);
    return (int64_t)coded;
}

int64_t pzref_compress(const uint8_t *src, size_t raw_bytes, int w,
                       uint32_t codec_mask, int tagged, uint8_t *dst,
                       size_t dst_capacity, uint8_t *tags, int32_t *block_bits)
{
    int rc = check_mode(w, codec_mask, tagged);
    if (rc != PZREF_OK) return -rc;
    size_t C = pzref_num_chunks(raw_bytes);
    if (dst_capacity < pzref_max_compressed(raw_bytes)) return -PZREF_ENOSPC;

    size_t out = 2 * C;
    for (size_t c = 0; c < C; c++) {
        size_t off = c * CHUNK_BYTES;
        size_t len = raw_bytes - off < CHUNK_BYTES ? raw_bytes - off : CHUNK_BYTES;
        int64_t H = pzref_compress_chunk(src + off, len, w, codec_mask, tagged,
                                         dst + out,
                                         tags ? tags + c * BLOCKS_PER_CHUNK : NULL,
                                         block_bits ? block_bits + c * BLOCKS_PER_CHUNK : NULL);
        if (H < 0) return H;
        dst[2 * c] = (uint8_t)(H & 0xFF);
        dst[2 * c + 1] = (uint8_t)(H >> 8);
        out += (size_t)H;
    }
    return (int64_t)out;
}

/* Decode one chunk payload of H bytes into raw_len bytes. */
static int decode_chunk(const uint8_t *payload, size_t H, size_t raw_len, int w,
                        uint32_t codec_mask, int tagged, uint8_t *dst)
{
    if (H > raw_len) return PZREF_ECORRUPT;
    if (H == raw_len) {
        memcpy(dst, payload, raw_len);
        return PZREF_OK;
    }
    bitreader br = {payload, (int64_t)H * 8, 0, 0};
    int nblocks = (int)((raw_len + BLOCK_BYTES - 1) / BLOCK_BYTES);
    int fixed = tagged ? -1 : single_codec(codec_mask);
    for (int b = 0; b < nblocks; b++) {
        int cand = fixed;
        if (tagged) {
            cand = (int)get_bits(&br, 3);
            if (br.overrun || cand > 4) return PZREF_ECORRUPT;
        }
        uint8_t block[BLOCK_BYTES];
        int rc = decode_one(&br, w, cand, block);
        if (rc != PZREF_OK) return rc;
        size_t off = (size_t)b * BLOCK_BYTES;
        size_t len = raw_len - off < BLOCK_BYTES ? raw_len - off : BLOCK_BYTES;
        memcpy(dst + off, block, len);
    }
    /* The blocks must end in the last payload byte, followed by zero bits. */
    if ((size_t)((br.pos + 7) / 8) != H) return PZREF_ECORRUPT;
    while (br.pos < (int64_t)H * 8)
        if (get_bits(&br, 1)) return PZREF_ECORRUPT;
    return PZREF_OK;
}

/* Reads the header table; fills offs[c] with payload offsets. */
static int locate_chunks(const uint8_t *src, size_t comp_bytes, size_t raw_bytes,
                         size_t *offs)
{
    size_t C = pzref_num_chunks(raw_bytes);
    if (comp_bytes < 2 * C) return PZREF_ECORRUPT;
    size_t pos = 2 * C;
    for (size_t c = 0; c < C; c++) {
        size_t H = (size_t)src[2 * c] | ((size_t)src[2 * c + 1] << 8);
        offs[c] = pos;
        pos += H;
    }
    return pos == comp_bytes ? PZREF_OK : PZREF_ECORRUPT;
}

int pzref_decompress(const uint8_t *src, size_t comp_bytes, int w,
                     uint32_t codec_mask, int tagged, uint8_t *dst,
                     size_t raw_bytes)
{
    int rc = check_mode(w, codec_mask, tagged);
    if (rc != PZREF_OK) return rc;
    size_t C = pzref_num_chunks(raw_bytes);
    size_t *offs = (size_t *)malloc((C ? C : 1) * sizeof(size_t));
    if (!offs) return PZREF_ENOSPC;
    rc = locate_chunks(src, comp_bytes, raw_bytes, offs);
    for (size_t c = 0; rc == PZREF_OK && c < C; c++) {
        size_t H = (size_t)src[2 * c] | ((size_t)src[2 * c + 1] << 8);
        size_t off = c * CHUNK_BYTES;
        size_t len = raw_bytes - off < CHUNK_BYTES ? raw_bytes - off : CHUNK_BYTES;
        rc = decode_chunk(src + offs[c], H, len, w, codec_mask, tagged, dst + off);
    }
    free(offs);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Chunk-parallel drivers over POSIX threads (same results, more cores).     */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint8_t *src;
    size_t raw_bytes;
    int w;
    uint32_t codec_mask;
    int tagged;
    uint8_t *tmp;      /* compress: chunk c payload at tmp + 4096c */
    int64_t *H;        /* compress: header values */
    uint8_t *dst;
    const size_t *offs;
    size_t c_begin, c_end;
    int rc;
} mt_job;

static void *compress_job(void *arg)
{
    mt_job *job = (mt_job *)arg;
    for (size_t c = job->c_begin; c < job->c_end; c++) {
        size_t off = c * CHUNK_BYTES;
        size_t len = job->raw_bytes - off < CHUNK_BYTES ? job->raw_bytes - off : CHUNK_BYTES;
        job->H[c] = pzref_compress_chunk(job->src + off, len, job->w, job->codec_mask,
                                         job->tagged, job->tmp + off, NULL, NULL);
        if (job->H[c] < 0) job->rc = (int)-job->H[c];
    }
    return NULL;
}

static void *decompress_job(void *arg)
{
    mt_job *job = (mt_job *)arg;
    for (size_t c = job->c_begin; c < job->c_end && job->rc == PZREF_OK; c++) {
        size_t H = (size_t)job->src[2 * c] | ((size_t)job->src[2 * c + 1] << 8);
        size_t off = c * CHUNK_BYTES;
        size_t len = job->raw_bytes - off < CHUNK_BYTES ? job->raw_bytes - off : CHUNK_BYTES;
        job->rc = decode_chunk(job->src + job->offs[c], H, len, job->w, job->codec_mask,
                               job->tagged, job->dst + off);
    }
    return NULL;
}

static void run_jobs(void *(*fn)(void *), mt_job *jobs, int threads, size_t C)
{
    pthread_t tid[256];
    for (int t = 0; t < threads; t++) {
        jobs[t].c_begin = C * (size_t)t / (size_t)threads;
        jobs[t].c_end = C * (size_t)(t + 1) / (size_t)threads;
        jobs[t].rc = PZREF_OK;
        pthread_create(&tid[t], NULL, fn, &jobs[t]);
    }
    for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
}

int64_t pzref_compress_mt(const uint8_t *src, size_t raw_bytes, int w,
                          uint32_t codec_mask, int tagged, uint8_t *dst,
                          size_t dst_capacity, int threads)
{
    int rc = check_mode(w, codec_mask, tagged);
    if (rc != PZREF_OK) return -rc;
    if (threads < 1 || threads > 256) return -PZREF_EINVAL;
    size_t C = pzref_num_chunks(raw_bytes);
    if (dst_capacity < pzref_max_compressed(raw_bytes)) return -PZREF_ENOSPC;
    uint8_t *tmp = (uint8_t *)malloc(raw_bytes ? raw_bytes : 1);
    int64_t *H = (int64_t *)malloc((C ? C : 1) * sizeof(int64_t));
    mt_job jobs[256];
    if (!tmp || !H) {
        free(tmp);
        free(H);
        return -PZREF_ENOSPC;
    }
    for (int t = 0; t < threads; t++) {
        mt_job j = {src, raw_bytes, w, codec_mask, tagged, tmp, H, dst, NULL, 0, 0, 0};
        jobs[t] = j;
    }
    run_jobs(compress_job, jobs, threads, C);
    int64_t result = 0;
    for (int t = 0; t < threads; t++)
        if (jobs[t].rc != PZREF_OK) result = -jobs[t].rc;
    if (result == 0) {
        size_t out = 2 * C;
        for (size_t c = 0; c < C; c++) {
            dst[2 * c] = (uint8_t)(H[c] & 0xFF);
            dst[2 * c + 1] = (uint8_t)(H[c] >> 8);
            memcpy(dst + out, tmp + c * CHUNK_BYTES, (size_t)H[c]);
            out += (size_t)H[c];
        }
        result = (int64_t)out;
    }
    free(tmp);
    free(H);
    return result;
}

int pzref_decompress_mt(const uint8_t *src, size_t comp_bytes, int w,
                        uint32_t codec_mask, int tagged, uint8_t *dst,
                        size_t raw_bytes, int threads)
{
    int rc = check_mode(w, codec_mask, tagged);
    if (rc != PZREF_OK) return rc;
    if (threads < 1 || threads > 256) return PZREF_EINVAL;
    size_t C = pzref_num_chunks(raw_bytes);
    size_t *offs = (size_t *)malloc((C ? C : 1) * sizeof(size_t));
    if (!offs) return PZREF_ENOSPC;
    rc = locate_chunks(src, comp_bytes, raw_bytes, offs);
    if (rc == PZREF_OK) {
        mt_job jobs[256];
        for (int t = 0; t < threads; t++) {
            mt_job j = {src, raw_bytes, w, codec_mask, tagged, NULL, NULL, dst, offs, 0, 0, 0};
            jobs[t] = j;
        }
        run_jobs(decompress_job, jobs, threads, C);
        for (int t = 0; t < threads; t++)
            if (jobs[t].rc != PZREF_OK) rc = jobs[t].rc;
    }
    free(offs);
    return rc;
}
