/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the Unweight weight format
 * and for Y = X * W^T.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or calls this
 * file; only the test suite, the smoke check and the bench's CPU-baseline leg do. It
 * shares no code, header, table or constant with the HIP library: the blob layout below
 * is restated here from the format definition, not included.
 *
 * Source of the method: Cloudflare's blog post "Unweight: how we compressed an LLM 22%
 * without sacrificing quality" (Chinese translation, sections "How weights compress",
 * "Exponents are predictable", "Four ways to use compressed weights" and "How the
 * reconstructive matmul works"). Where the post is silent (code-length limit, tie
 * order, bit order, chunking), the readings are the ones listed in the design notes.
 *
 * Everything is scalar C, one element or one bit at a time. Integer results are exact;
 * the GEMM accumulates in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- blob layout (format version 1), restated from the format definition ---------- */
#define OR_MAGIC 0x31545755u /* bytes 'U','W','T','1' */
#define OR_VERSION 1u
#define OR_HDR_BYTES 256u
#define OR_SECTION_ALIGN 256u
#define OR_STREAM_SLACK 64u

/* header byte offsets */
#define H_MAGIC 0
#define H_VERSION 4
#define H_N 8
#define H_K 16
#define H_CHUNK 24
#define H_LMAX 28
#define H_NPAL 32
#define H_NCHUNKS 36
#define H_PALETTE 40
#define H_CODELEN 56
#define H_NRAW 72
#define H_TOTALBITS 80
#define H_OFF_SM 88
#define H_OFF_BITMAP 96
#define H_OFF_ROWBASE 104
#define H_OFF_RAW 112
#define H_OFF_CHUNK 120
#define H_OFF_STREAM 128
#define H_BYTES_STREAM 136
#define H_TOTAL_BYTES 144
#define H_BITMAP_WORDS 152

enum { OR_OK = 0, OR_EINVAL = 1, OR_ESHAPE = 2, OR_EFORMAT = 3, OR_ERANGE = 4, OR_ENOSPACE = 5 };

static void put_u32(uint8_t* b, size_t off, uint32_t v) { memcpy(b + off, &v, 4); }
static void put_u64(uint8_t* b, size_t off, uint64_t v) { memcpy(b + off, &v, 8); }
static uint32_t get_u32(const uint8_t* b, size_t off) { uint32_t v; memcpy(&v, b + off, 4); return v; }
static uint64_t get_u64(const uint8_t* b, size_t off) { uint64_t v; memcpy(&v, b + off, 8); return v; }
static uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

/* ---- step 1: field split (sign 1 bit, exponent 8 bits, mantissa 7 bits) ----------- */
/* "How weights compress": a bf16 value is sign | exponent | mantissa. The sign and
 * mantissa are kept verbatim, packed into one byte sign<<7 | mantissa. */
void or_split(const uint16_t* w, int64_t n, uint8_t* sm, uint8_t* e)
{
    for (int64_t i = 0; i < n; i++) {
        uint16_t v = w[i];
        uint8_t sign = (uint8_t)(v >> 15);
        uint8_t expo = (uint8_t)((v >> 7) & 0xFF);
        uint8_t mant = (uint8_t)(v & 0x7F);
        if (sm) sm[i] = (uint8_t)((sign << 7) | mant);
        if (e) e[i] = expo;
    }
}

/* inverse of or_split */
void or_join(const uint8_t* sm, const uint8_t* e, int64_t n, uint16_t* w)
{
    for (int64_t i = 0; i < n; i++) {
        uint16_t sign = (uint16_t)(sm[i] >> 7);
        uint16_t mant = (uint16_t)(sm[i] & 0x7F);
        w[i] = (uint16_t)((sign << 15) | ((uint16_t)e[i] << 7) | mant);
    }
}

/* ---- step 2: exponent palette ("Exponents are predictable": the 16 most common
 * exponents of a layer cover almost all weights) ---------------------------------- */
/* Palette = the min(16, #distinct) most frequent exponents, ordered by count
 * descending, ties by exponent value ascending. Returns n_pal. */
int or_palette(const uint8_t* e, int64_t n, uint8_t* palette, uint64_t* hist_out)
{
    uint64_t hist[256];
    memset(hist, 0, sizeof hist);
    for (int64_t i = 0; i < n; i++) hist[e[i]]++;
    if (hist_out) memcpy(hist_out, hist, sizeof hist);
    int taken[256];
    memset(taken, 0, sizeof taken);
    int n_pal = 0;
    for (int r = 0; r < 16; r++) {
        int best = -1;
        for (int v = 0; v < 256; v++) {
            if (taken[v] || hist[v] == 0) continue;
            if (best < 0 || hist[v] > hist[best]) best = v; /* strict '>' keeps the lower value on ties */
        }
        if (best < 0) break;
        taken[best] = 1;
        palette[n_pal++] = (uint8_t)best;
    }
    return n_pal;
}

static int palette_index(const uint8_t* palette, int n_pal, uint8_t e)
{
    for (int i = 0; i < n_pal; i++)
        if (palette[i] == e) return i;
    return -1;
}

/* ---- step 3: 64-weight row fallback ("Exponents are predictable": if any weight of a
 * 64-weight row has an exponent outside the top-16 palette, the whole row is stored
 * as-is). Group (r, j) = elements W[r][64j .. 64j+63]. Outputs, all optional:
 *   bitmap[r * words + j/32] bit (j % 32) = group raw,  words = ceil(K / 2048)
 *   row_base[r] = raw groups in rows before r (N + 1 entries)
 *   raw_exp = the 64 exponent bytes of every raw group, in (r, j) order.
 * Returns the number of raw groups. */
int64_t or_raw_groups(const uint8_t* e, int64_t N, int64_t K, const uint8_t* palette, int n_pal,
                      uint32_t* bitmap, uint32_t* row_base, uint8_t* raw_exp)
{
    int64_t words = (K + 2047) / 2048;
    int64_t n_raw = 0;
    if (bitmap) memset(bitmap, 0, (size_t)(N * words) * 4);
    for (int64_t r = 0; r < N; r++) {
        if (row_base) row_base[r] = (uint32_t)n_raw;
        for (int64_t j = 0; j < K / 64; j++) {
            int raw = 0;
            for (int t = 0; t < 64; t++)
                if (palette_index(palette, n_pal, e[r * K + j * 64 + t]) < 0) raw = 1;
            if (!raw) continue;
            if (bitmap) bitmap[r * words + j / 32] |= 1u << (j % 32);
            if (raw_exp) memcpy(raw_exp + n_raw * 64, e + r * K + j * 64, 64);
            n_raw++;
        }
    }
    if (row_base) row_base[N] = (uint32_t)n_raw;
    return n_raw;
}

/* ---- step 4: length-limited optimal code lengths by package-merge --------------
 * (Larmore & Hirschberg, "A fast algorithm for optimal length-restricted Huffman
 * codes", 1990). Items of the coin-collector problem carry the multiset of symbols
 * they contain; a symbol's code length is how many of the 2m-2 cheapest items at the
 * top denomination contain it. Symbols with f = 0 get length 0; one used symbol gets
 * length 1; none gives all zeros. Returns 0, or -1 if 2^lmax < #used. */
typedef struct {
    uint64_t w;
    uint8_t cnt[16];
} pm_item;

static void item_sort(pm_item* a, int n)
{ /* insertion sort: ascending weight, stable */
    for (int i = 1; i < n; i++) {
        pm_item t = a[i];
        int j = i - 1;
        while (j >= 0 && a[j].w > t.w) { a[j + 1] = a[j]; j--; }
        a[j + 1] = t;
    }
}

int or_code_lengths(const uint64_t* f, int n, int lmax, uint8_t* len)
{
    if (n < 0 || n > 16 || lmax < 1 || lmax > 15) return -1;
    memset(len, 0, (size_t)n);
    pm_item sym[16];
    int m = 0;
    for (int i = 0; i < n; i++) {
        if (f[i] == 0) continue;
        memset(&sym[m], 0, sizeof(pm_item));
        sym[m].w = f[i];
        sym[m].cnt[i] = 1;
        m++;
    }
    if (m == 0) return 0;
    if (m == 1) {
        for (int i = 0; i < n; i++)
            if (f[i]) len[i] = 1;
        return 0;
    }
    if ((1 << lmax) < m) return -1;
    item_sort(sym, m);
    pm_item list[64], next[64];
    int nl = m;
    memcpy(list, sym, sizeof(pm_item) * (size_t)m);
    for (int level = 1; level < lmax; level++) {
        pm_item pack[32];
        int np = nl / 2;
        for (int j = 0; j < np; j++) {
            pack[j].w = list[2 * j].w + list[2 * j + 1].w;
            for (int s = 0; s < 16; s++) pack[j].cnt[s] = (uint8_t)(list[2 * j].cnt[s] + list[2 * j + 1].cnt[s]);
        }
        int a = 0, b = 0, k = 0;
        while (a < m || b < np) {
            if (b >= np || (a < m && sym[a].w <= pack[b].w)) next[k++] = sym[a++];
            else next[k++] = pack[b++];
        }
        nl = k;
        memcpy(list, next, sizeof(pm_item) * (size_t)nl);
    }
    for (int j = 0; j < 2 * m - 2; j++)
        for (int s = 0; s < n; s++) len[s] = (uint8_t)(len[s] + list[j].cnt[s]);
    return 0;
}

/* ---- step 5: canonical code assignment (the DEFLATE rule, RFC 1951 section 3.2.2):
 * used symbols sorted by (length, symbol); the first gets code 0, each next one gets
 * (previous + 1) shifted left by the length increase. */
void or_canonical_codes(const uint8_t* len, int n, uint32_t* code)
{
    int order[16], m = 0;
    for (int l = 1; l <= 15; l++)
        for (int s = 0; s < n; s++)
            if (len[s] == l) order[m++] = s;
    for (int s = 0; s < n; s++) code[s] = 0;
    uint32_t c = 0;
    for (int i = 0; i < m; i++) {
        if (i > 0) c = (c + 1) << (len[order[i]] - len[order[i - 1]]);
        code[order[i]] = c;
    }
}

/* ---- sizes ------------------------------------------------------------------------ */
typedef struct {
    uint64_t off_sm, off_bitmap, off_rowbase, off_raw, off_chunk, off_stream, bytes_stream, total;
} or_layout;

static or_layout layout_of(int64_t N, int64_t K, int64_t n_raw, int64_t n_chunks, uint64_t total_bits)
{
    or_layout L;
    uint64_t words = (uint64_t)((K + 2047) / 2048);
    L.off_sm = OR_HDR_BYTES;
    L.off_bitmap = round_up(L.off_sm + (uint64_t)(N * K), OR_SECTION_ALIGN);
    L.off_rowbase = round_up(L.off_bitmap + 4 * (uint64_t)N * words, OR_SECTION_ALIGN);
    L.off_raw = round_up(L.off_rowbase + 4 * (uint64_t)(N + 1), OR_SECTION_ALIGN);
    L.off_chunk = round_up(L.off_raw + 64 * (uint64_t)n_raw, OR_SECTION_ALIGN);
    L.off_stream = round_up(L.off_chunk + 4 * (uint64_t)(n_chunks + 1), OR_SECTION_ALIGN);
    L.bytes_stream = round_up((total_bits + 7) / 8, 16) + OR_STREAM_SLACK;
    L.total = L.off_stream + L.bytes_stream;
    return L;
}

/* ---- steps 1-6 together: encode a matrix into a blob -------------------------------
 * Symbols are the palette indices of the elements of non-raw groups, in row-major
 * order. Their codes are written MSB first; stream bit b is bit 31 - (b % 32) of the
 * little-endian 32-bit word b / 32. Chunk c covers flattened elements
 * [c*chunk, (c+1)*chunk); off[c] = number of stream bits written before chunk c.
 * Two-call size query: blob == NULL or *blob_bytes too small -> OR_ENOSPACE with
 * *blob_bytes set to the required size. */
int or_encode(const uint16_t* w, int64_t N, int64_t K, uint32_t chunk, uint32_t lmax, uint8_t* blob,
              uint64_t* blob_bytes)
{
    if (N < 1 || K < 1 || K % 64 != 0) return OR_ESHAPE;
    if (chunk == 0 || chunk % 64 != 0) return OR_EINVAL;
    if (lmax < 1 || lmax > 15) return OR_EINVAL;
    int64_t n = N * K;
    uint8_t* sm = (uint8_t*)malloc((size_t)n);
    uint8_t* e = (uint8_t*)malloc((size_t)n);
    or_split(w, n, sm, e);
    uint8_t palette[16] = {0};
    int n_pal = or_palette(e, n, palette, NULL);
    int64_t words = (K + 2047) / 2048;
    uint32_t* bitmap = (uint32_t*)calloc((size_t)(N * words), 4);
    uint32_t* row_base = (uint32_t*)calloc((size_t)(N + 1), 4);
    int64_t n_raw = or_raw_groups(e, N, K, palette, n_pal, bitmap, row_base, NULL);
    uint8_t* raw_exp = (uint8_t*)malloc((size_t)(n_raw * 64 + 1));
    or_raw_groups(e, N, K, palette, n_pal, NULL, NULL, raw_exp);

    /* symbol frequencies over non-raw groups */
    uint64_t f[16] = {0};
    for (int64_t i = 0; i < n; i++) {
        int64_t r = i / K, j = (i % K) / 64;
        if (bitmap[r * words + j / 32] >> (j % 32) & 1) continue;
        f[palette_index(palette, n_pal, e[i])]++;
    }
    uint8_t len[16] = {0};
    if (or_code_lengths(f, n_pal, (int)lmax, len) != 0) {
        free(sm); free(e); free(bitmap); free(row_base); free(raw_exp);
        return OR_EINVAL;
    }
    uint32_t code[16] = {0};
    or_canonical_codes(len, n_pal, code);
    uint64_t total_bits = 0;
    for (int s = 0; s < n_pal; s++) total_bits += f[s] * len[s];
    if (total_bits >= (1ull << 32)) {
        free(sm); free(e); free(bitmap); free(row_base); free(raw_exp);
        return OR_ERANGE;
    }
    int64_t n_chunks = (n + chunk - 1) / chunk;
    or_layout L = layout_of(N, K, n_raw, n_chunks, total_bits);
    if (blob == NULL || *blob_bytes < L.total) {
        *blob_bytes = L.total;
        free(sm); free(e); free(bitmap); free(row_base); free(raw_exp);
        return OR_ENOSPACE;
    }
    *blob_bytes = L.total;
    memset(blob, 0, L.total);
    put_u32(blob, H_MAGIC, OR_MAGIC);
    put_u32(blob, H_VERSION, OR_VERSION);
    put_u64(blob, H_N, (uint64_t)N);
    put_u64(blob, H_K, (uint64_t)K);
    put_u32(blob, H_CHUNK, chunk);
    put_u32(blob, H_LMAX, lmax);
    put_u32(blob, H_NPAL, (uint32_t)n_pal);
    put_u32(blob, H_NCHUNKS, (uint32_t)n_chunks);
    memcpy(blob + H_PALETTE, palette, 16);
    memcpy(blob + H_CODELEN, len, 16);
    put_u64(blob, H_NRAW, (uint64_t)n_raw);
    put_u64(blob, H_TOTALBITS, total_bits);
    put_u64(blob, H_OFF_SM, L.off_sm);
    put_u64(blob, H_OFF_BITMAP, L.off_bitmap);
    put_u64(blob, H_OFF_ROWBASE, L.off_rowbase);
    put_u64(blob, H_OFF_RAW, L.off_raw);
    put_u64(blob, H_OFF_CHUNK, L.off_chunk);
    put_u64(blob, H_OFF_STREAM, L.off_stream);
    put_u64(blob, H_BYTES_STREAM, L.bytes_stream);
    put_u64(blob, H_TOTAL_BYTES, L.total);
    put_u32(blob, H_BITMAP_WORDS, (uint32_t)words);
    memcpy(blob + L.off_sm, sm, (size_t)n);
    memcpy(blob + L.off_bitmap, bitmap, (size_t)(N * words) * 4);
    memcpy(blob + L.off_rowbase, row_base, (size_t)(N + 1) * 4);
    memcpy(blob + L.off_raw, raw_exp, (size_t)n_raw * 64);

    uint32_t* offs = (uint32_t*)(blob + L.off_chunk);
    uint32_t* stream = (uint32_t*)(blob + L.off_stream);
    uint64_t pos = 0;
    for (int64_t i = 0; i < n; i++) {
        if (i % chunk == 0) offs[i / chunk] = (uint32_t)pos;
        int64_t r = i / K, j = (i % K) / 64;
        if (bitmap[r * words + j / 32] >> (j % 32) & 1) continue;
        int s = palette_index(palette, n_pal, e[i]);
        for (int b = len[s] - 1; b >= 0; b--) {
            uint32_t bit = (code[s] >> b) & 1u;
            stream[pos / 32] |= bit << (31 - pos % 32);
            pos++;
        }
    }
    offs[n_chunks] = (uint32_t)pos;
    free(sm); free(e); free(bitmap); free(row_base); free(raw_exp);
    return OR_OK;
}

/* ---- header reader (for blobs written by either side) ------------------------------ */
typedef struct {
    int64_t N, K, n_raw, n_chunks, words;
    uint32_t chunk, lmax, n_pal;
    uint64_t total_bits;
    uint8_t palette[16], len[16];
    or_layout L;
} or_hdr;

static int read_header(const uint8_t* blob, uint64_t bytes, or_hdr* h)
{
    if (bytes < OR_HDR_BYTES) return OR_EFORMAT;
    if (get_u32(blob, H_MAGIC) != OR_MAGIC || get_u32(blob, H_VERSION) != OR_VERSION) return OR_EFORMAT;
    h->N = (int64_t)get_u64(blob, H_N);
    h->K = (int64_t)get_u64(blob, H_K);
    if (h->N < 1 || h->K < 1 || h->K % 64) return OR_EFORMAT;
    h->chunk = get_u32(blob, H_CHUNK);
    h->lmax = get_u32(blob, H_LMAX);
    h->n_pal = get_u32(blob, H_NPAL);
    h->n_chunks = get_u32(blob, H_NCHUNKS);
    h->n_raw = (int64_t)get_u64(blob, H_NRAW);
    h->total_bits = get_u64(blob, H_TOTALBITS);
    h->words = (h->K + 2047) / 2048;
    memcpy(h->palette, blob + H_PALETTE, 16);
    memcpy(h->len, blob + H_CODELEN, 16);
    if (h->chunk == 0 || h->chunk % 64 || h->n_pal > 16 || h->lmax < 1 || h->lmax > 15) return OR_EFORMAT;
    if (h->n_chunks != (h->N * h->K + h->chunk - 1) / h->chunk) return OR_EFORMAT;
    h->L = layout_of(h->N, h->K, h->n_raw, h->n_chunks, h->total_bits);
    if (get_u64(blob, H_OFF_SM) != h->L.off_sm || get_u64(blob, H_OFF_BITMAP) != h->L.off_bitmap ||
        get_u64(blob, H_OFF_ROWBASE) != h->L.off_rowbase || get_u64(blob, H_OFF_RAW) != h->L.off_raw ||
        get_u64(blob, H_OFF_CHUNK) != h->L.off_chunk || get_u64(blob, H_OFF_STREAM) != h->L.off_stream ||
        get_u64(blob, H_BYTES_STREAM) != h->L.bytes_stream || get_u64(blob, H_TOTAL_BYTES) != h->L.total)
        return OR_EFORMAT;
    if (bytes < h->L.total) return OR_EFORMAT;
    return OR_OK;
}

/* ---- step 7: decode, bit by bit, with the textbook canonical decoder: extend the
 * code one bit at a time and accept it once it falls inside the range of codes of the
 * current length. Outputs (each optional): the bf16 weights, the exponent plane (raw
 * groups included) and the 4-bit palette-index plane (low nibble = even element, raw
 * groups 0), i.e. the results of the full-decode, exponent-only and palette-transcode
 * pipelines ("Four ways to use compressed weights"). Returns OR_EFORMAT on a bad code,
 * on a chunk whose symbols do not end exactly at the next chunk offset, or on a
 * palette index >= n_pal. */
int or_decode(const uint8_t* blob, uint64_t bytes, uint16_t* w_out, uint8_t* exp_out, uint8_t* idx_out)
{
    or_hdr h;
    int st = read_header(blob, bytes, &h);
    if (st) return st;
    const uint8_t* sm = blob + h.L.off_sm;
    const uint32_t* bitmap = (const uint32_t*)(blob + h.L.off_bitmap);
    const uint32_t* row_base = (const uint32_t*)(blob + h.L.off_rowbase);
    const uint8_t* raw_exp = blob + h.L.off_raw;
    const uint32_t* offs = (const uint32_t*)(blob + h.L.off_chunk);
    const uint32_t* stream = (const uint32_t*)(blob + h.L.off_stream);

    /* canonical decoding tables */
    int count[17] = {0};
    for (uint32_t s = 0; s < h.n_pal; s++)
        if (h.len[s]) count[h.len[s]]++;
    int sorted[16], ns = 0;
    for (int l = 1; l <= 15; l++)
        for (uint32_t s = 0; s < h.n_pal; s++)
            if (h.len[s] == l) sorted[ns++] = (int)s;
    uint32_t first_code[17] = {0};
    int first_index[17] = {0};
    uint32_t c = 0;
    int idx = 0;
    for (int l = 1; l <= 15; l++) {
        c = (c + (uint32_t)count[l - 1]) << 1;
        first_code[l] = c;
        first_index[l] = idx;
        idx += count[l];
    }

    int64_t n = h.N * h.K;
    if (idx_out) memset(idx_out, 0, (size_t)(n / 2));
    uint64_t pos = 0;
    for (int64_t i = 0; i < n; i++) {
        if (i % h.chunk == 0) {
            if (offs[i / h.chunk] != pos) return OR_EFORMAT;
        }
        int64_t r = i / h.K, j = (i % h.K) / 64;
        uint8_t e;
        int sym = 0;
        if (bitmap[r * h.words + j / 32] >> (j % 32) & 1) {
            /* rank of this group among the raw groups of its row */
            uint32_t before = 0;
            for (int64_t jj = 0; jj < j; jj++) before += bitmap[r * h.words + jj / 32] >> (jj % 32) & 1;
            e = raw_exp[((int64_t)row_base[r] + before) * 64 + (i % 64)];
        } else {
            uint32_t code = 0;
            int l = 0;
            for (;;) {
                if (pos >= h.total_bits) return OR_EFORMAT;
                uint32_t bit = (stream[pos / 32] >> (31 - pos % 32)) & 1u;
                pos++;
                code = (code << 1) | bit;
                l++;
                if (l > (int)h.lmax) return OR_EFORMAT;
                if (count[l] && code >= first_code[l] && code - first_code[l] < (uint32_t)count[l]) {
                    sym = sorted[first_index[l] + (int)(code - first_code[l])];
                    break;
                }
            }
            if ((uint32_t)sym >= h.n_pal) return OR_EFORMAT;
            e = h.palette[sym];
        }
        if (exp_out) exp_out[i] = e;
        if (idx_out && sym) idx_out[i / 2] |= (uint8_t)(sym << (4 * (i % 2)));
        if (w_out) {
            uint16_t sign = (uint16_t)(sm[i] >> 7), mant = (uint16_t)(sm[i] & 0x7F);
            w_out[i] = (uint16_t)((sign << 15) | ((uint16_t)e << 7) | mant);
        }
    }
    if (offs[h.n_chunks] != pos || pos != h.total_bits) return OR_EFORMAT;
    return OR_OK;
}

/* ---- GEMM: Y[m][n] = sum_k x[m][k] * w[n][k], in double, on the original bf16 values;
 * A[m][n] = sum_k |x[m][k] * w[n][k]| is the scale the tolerance is stated against. */
static double bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

void or_gemm_pairs(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, int64_t K,
                   const int64_t* m_idx, const int64_t* n_idx, int64_t cnt, double* y, double* a)
{
    for (int64_t t = 0; t < cnt; t++) {
        double s = 0.0, sa = 0.0;
        const uint16_t* xr = x + m_idx[t] * ldx;
        const uint16_t* wr = w + n_idx[t] * ldw;
        for (int64_t k = 0; k < K; k++) {
            double p = bf16_to_f64(xr[k]) * bf16_to_f64(wr[k]);
            s += p;
            sa += fabs(p);
        }
        y[t] = s;
        if (a) a[t] = sa;
    }
}

void or_gemm(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N, int64_t K, double* y, double* a)
{
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = bf16_to_f64(x[m * K + k]) * bf16_to_f64(w[n * K + k]);
                s += p;
                sa += fabs(p);
            }
            y[m * N + n] = s;
            if (a) a[m * N + n] = sa;
        }
}

/* ---- SwiGLU glue between the MLP projections: h = bf16(silu(g) * u), silu(z) =
 * z / (1 + exp(-z)), evaluated in double and rounded once to bf16, nearest-even. ----- */
static uint16_t f64_to_bf16(double x)
{
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    int ex;
    frexp(a, &ex);        /* a = f * 2^ex, f in [0.5, 1) */
    int E = ex - 1;       /* a in [2^E, 2^(E+1)) */
    if (E < -126) E = -126; /* subnormal range shares the quantum of the lowest binade */
    int q = E - 7;        /* 8 significant bits */
    double r = nearbyint(ldexp(a, -q)); /* default rounding mode: nearest, ties to even */
    double v = ldexp(r, q);
    if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float fv = (float)v; /* exact: v has <= 8 significant bits inside float range */
    uint32_t u;
    memcpy(&u, &fv, 4);
    return (uint16_t)(sign | (u >> 16));
}

void or_swiglu(const float* g, const float* u, int64_t n, uint16_t* h)
{
    for (int64_t i = 0; i < n; i++) {
        double z = (double)g[i];
        double silu = z / (1.0 + exp(-z));
        h[i] = f64_to_bf16(silu * (double)u[i]);
    }
}

uint16_t or_f64_to_bf16(double x) { return f64_to_bf16(x); }
