// Host side of libuw: status strings, the encoder and blob validation.
//
// The format follows the Unweight blog post ("How weights compress", "Exponents are
// predictable"): sign and mantissa verbatim, the exponent byte replaced by its rank in
// the matrix's top-16 exponent palette and Huffman-coded, and any 64-weight row group
// holding an exponent outside the palette stored as-is. Code lengths are optimal under
// a length limit (the limit keeps the decoder's lookup table small enough for LDS; the
// post's decoder keeps a ~16 KB table in on-chip memory, "Sharing the GPU between decode
// and compute").
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "uw_internal.h"

namespace uw {

static thread_local std::string g_err;

void clear_error() { g_err.clear(); }

uw_status fail(uw_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

Layout layout_for(int64_t N, int64_t K, int64_t n_raw, int64_t n_chunks, uint64_t total_bits)
{
    Layout L;
    const uint64_t words = static_cast<uint64_t>((K + 2047) / 2048);
    L.off_sm = sizeof(uw_header);
    L.off_bitmap = round_up(L.off_sm + static_cast<uint64_t>(N) * static_cast<uint64_t>(K), kSectionAlign);
    L.off_rowbase = round_up(L.off_bitmap + 4ull * static_cast<uint64_t>(N) * words, kSectionAlign);
    L.off_raw = round_up(L.off_rowbase + 4ull * static_cast<uint64_t>(N + 1), kSectionAlign);
    L.off_chunk = round_up(L.off_raw + 64ull * static_cast<uint64_t>(n_raw), kSectionAlign);
    L.off_stream = round_up(L.off_chunk + 4ull * static_cast<uint64_t>(n_chunks + 1), kSectionAlign);
    L.bytes_stream = round_up((total_bits + 7) / 8, 16) + kStreamSlack;
    L.total = L.off_stream + L.bytes_stream;
    return L;
}

// Optimal code lengths under a length limit, by dynamic programming over the levels of
// the code tree. With the used symbols sorted by frequency (descending), an optimal
// code assigns non-decreasing lengths, so a tree is described level by level by how
// many of the open nodes at depth d become leaves (taking the next most frequent
// symbols) while the rest split into two nodes at depth d+1. best(d, i, a) is the least
// cost sum f*len of finishing the tree from depth d with symbols i.. unassigned and a
// open nodes; open nodes beyond the unassigned count are useless and are capped.
static bool limited_code_lengths(const uint64_t* f, int n, int lmax, uint8_t* len)
{
    int sym[16];
    int m = 0;
    for (int i = 0; i < n; i++)
        if (f[i]) sym[m++] = i;
    std::stable_sort(sym, sym + m, [&](int a, int b) { return f[a] > f[b]; });
    std::memset(len, 0, static_cast<size_t>(n));
    if (m == 0) return true;
    if (m == 1) {
        len[sym[0]] = 1;
        return true;
    }
    if ((1 << lmax) < m) return false;
    uint64_t pre[17] = {0};  // pre[i] = sum of the i largest frequencies
    for (int i = 0; i < m; i++) pre[i + 1] = pre[i] + f[sym[i]];
    const uint64_t INF = ~0ull;
    // best[d][i][a], choice[d][i][a] for d in 1..lmax, i in 0..m, a in 0..m
    std::vector<uint64_t> best(static_cast<size_t>(17 * 17 * 17), INF);
    std::vector<int8_t> choice(static_cast<size_t>(17 * 17 * 17), -1);
    auto at = [](int d, int i, int a) { return (static_cast<size_t>(d) * 17 + i) * 17 + a; };
    for (int d = lmax; d >= 1; d--) {
        for (int i = 0; i < m; i++) {
            for (int a = 1; a <= m - i; a++) {
                uint64_t b = INF;
                int bk = -1;
                for (int k = 0; k <= a && i + k <= m; k++) {
                    uint64_t here = (pre[i + k] - pre[i]) * static_cast<uint64_t>(d);
                    uint64_t rest;
                    if (i + k == m) {
                        rest = 0;
                    } else {
                        if (a - k < 1 || d == lmax) continue;
                        int a2 = std::min(2 * (a - k), m - i - k);
                        rest = best[at(d + 1, i + k, a2)];
                        if (rest == INF) continue;
                    }
                    if (here + rest < b) {
                        b = here + rest;
                        bk = k;
                    }
                }
                best[at(d, i, a)] = b;
                choice[at(d, i, a)] = static_cast<int8_t>(bk);
            }
        }
    }
    int i = 0, a = std::min(2, m);
    if (best[at(1, 0, a)] == INF) return false;
    for (int d = 1; d <= lmax && i < m; d++) {
        int k = choice[at(d, i, a)];
        if (k < 0) return false;
        for (int t = 0; t < k; t++) len[sym[i + t]] = static_cast<uint8_t>(d);
        i += k;
        a = std::min(2 * (a - k), m - i);
    }
    return i == m;
}

// Canonical codes by the counting construction of RFC 1951 section 3.2.2: the first
// code of each length follows the last code of the previous length, doubled.
static void canonical_codes(const uint8_t* len, int n, uint32_t* code)
{
    uint32_t bl_count[17] = {0};
    for (int s = 0; s < n; s++) bl_count[len[s]]++;
    bl_count[0] = 0;
    uint32_t next[17] = {0};
    uint32_t c = 0;
    for (int l = 1; l <= 16; l++) {
        c = (c + bl_count[l - 1]) << 1;
        next[l] = c;
    }
    for (int s = 0; s < n; s++) code[s] = len[s] ? next[len[s]]++ : 0;
}

void canon_tables(const uw_header* h, CanonTables* t)
{
    std::memset(t, 0, sizeof *t);
    const int n = static_cast<int>(std::min<uint32_t>(h->n_pal, 16));
    uint32_t cnt[17] = {0};
    for (int s = 0; s < n; s++)
        if (h->code_len[s]) cnt[h->code_len[s]]++;
    uint32_t c = 0, idx = 0;
    for (int l = 1; l <= 15; l++) {
        c = (c + cnt[l - 1]) << 1;
        t->first_code[l] = c;
        t->count[l] = cnt[l];
        t->first_index[l] = idx;
        for (int s = 0; s < n; s++)
            if (h->code_len[s] == l) t->sorted[idx++] = static_cast<uint8_t>(s);
    }
    t->n_used = idx;
}

void value_order(const uw_header* h, ValueOrder* v)
{
    const int n = static_cast<int>(std::min<uint32_t>(h->n_pal, 16));
    std::memset(v, 0, sizeof *v);
    for (int i = 0; i < n; i++) {
        int below = 0;
        for (int k = 0; k < n; k++) below += h->palette[k] < h->palette[i];
        v->order[i] = static_cast<uint8_t>(below);
        v->sorted[below] = h->palette[i];
    }
    v->contiguous = true;
    for (int k = 1; k < n; k++) v->contiguous &= v->sorted[k] == v->sorted[0] + k;
}

uw_status check_header(const uw_header* h, size_t blob_bytes)
{
    if (h->magic != kMagic) return fail(UW_EFORMAT, "bad magic 0x%08x", h->magic);
    if (h->version != UW_VERSION) return fail(UW_EFORMAT, "unsupported format version %u", h->version);
    if (h->N < 1 || h->K < 1 || h->K % 64) return fail(UW_EFORMAT, "bad shape %lld x %lld", (long long)h->N, (long long)h->K);
    if (h->N > (1ll << 31) || h->K > (1ll << 31) || h->N * h->K > (1ll << 40))
        return fail(UW_EFORMAT, "shape too large");
    if (h->chunk == 0 || h->chunk % 64) return fail(UW_EFORMAT, "chunk %u not a positive multiple of 64", h->chunk);
    if (h->lmax < 1 || h->lmax > 15) return fail(UW_EFORMAT, "lmax %u outside 1..15", h->lmax);
    if (h->n_pal > 16) return fail(UW_EFORMAT, "palette size %u > 16", h->n_pal);
    const int64_t n = h->N * h->K;
    if (static_cast<int64_t>(h->n_chunks) != (n + h->chunk - 1) / h->chunk)
        return fail(UW_EFORMAT, "n_chunks %u does not match N*K/chunk", h->n_chunks);
    if (h->n_raw < 0 || h->n_raw > n / 64) return fail(UW_EFORMAT, "n_raw %lld out of range", (long long)h->n_raw);
    if (h->total_bits >= (1ull << 32)) return fail(UW_EFORMAT, "total_bits >= 2^32");
    if (h->bitmap_words != static_cast<uint32_t>((h->K + 2047) / 2048)) return fail(UW_EFORMAT, "bad bitmap_words");
    for (uint32_t i = 0; i < h->n_pal; i++)
        for (uint32_t j = i + 1; j < h->n_pal; j++)
            if (h->palette[i] == h->palette[j]) return fail(UW_EFORMAT, "duplicate palette entry");
    double kraft = 0.0;
    uint32_t used = 0;
    for (int s = 0; s < 16; s++) {
        const uint32_t l = h->code_len[s];
        if (l == 0) continue;
        if (static_cast<uint32_t>(s) >= h->n_pal || l > h->lmax) return fail(UW_EFORMAT, "bad code length for index %d", s);
        kraft += 1.0 / static_cast<double>(1u << l);
        used++;
    }
    if (kraft > 1.0) return fail(UW_EFORMAT, "code lengths violate the Kraft inequality");
    const int64_t n_sym = n - 64 * h->n_raw;
    if (n_sym > 0 && used == 0) return fail(UW_EFORMAT, "symbols present but no code");
    if (h->total_bits > static_cast<uint64_t>(n_sym) * h->lmax) return fail(UW_EFORMAT, "total_bits too large");
    const Layout L = layout_for(h->N, h->K, h->n_raw, h->n_chunks, h->total_bits);
    if (h->off_sm != L.off_sm || h->off_bitmap != L.off_bitmap || h->off_rowbase != L.off_rowbase ||
        h->off_raw != L.off_raw || h->off_chunk != L.off_chunk || h->off_stream != L.off_stream ||
        h->bytes_stream != L.bytes_stream || h->total_bytes != L.total)
        return fail(UW_EFORMAT, "section offsets do not follow the layout");
    if (blob_bytes < L.total) return fail(UW_EFORMAT, "blob has %zu bytes, header needs %llu", blob_bytes, (unsigned long long)L.total);
    return UW_OK;
}

}  // namespace uw

using namespace uw;

extern "C" {

const char* uw_status_string(int status)
{
    switch (status) {
    case UW_OK: return "UW_OK";
    case UW_EINVAL: return "UW_EINVAL: invalid argument";
    case UW_ESHAPE: return "UW_ESHAPE: invalid shape";
    case UW_EFORMAT: return "UW_EFORMAT: malformed blob";
    case UW_ERANGE: return "UW_ERANGE: value out of range";
    case UW_ENOSPACE: return "UW_ENOSPACE: buffer too small";
    case UW_EHIP: return "UW_EHIP: HIP runtime error";
    case UW_EUNSUPPORTED: return "UW_EUNSUPPORTED: unsupported combination";
    case UW_EINTERNAL: return "UW_EINTERNAL: internal error";
    default: return "unknown uw_status";
    }
}

const char* uw_last_error(void) { return g_err.c_str(); }

int uw_version(void) { return UW_VERSION; }

uw_status uw_encode(const uint16_t* w, int64_t N, int64_t K, const uw_encode_opts* opts, void* blob,
                    size_t* blob_bytes)
{
    try {
        clear_error();
        if (!w || !blob_bytes) return fail(UW_EINVAL, "w and blob_bytes must not be NULL");
        if (N < 1 || K < 1 || K % 64) return fail(UW_ESHAPE, "need N >= 1, K >= 1, K %% 64 == 0 (got %lld x %lld)", (long long)N, (long long)K);
        if (N > (1ll << 31) || K > (1ll << 31) || N * K > (1ll << 40)) return fail(UW_ESHAPE, "shape too large");
        const uint32_t chunk = (opts && opts->chunk) ? opts->chunk : kDefaultChunk;
        const uint32_t lmax = (opts && opts->lmax) ? opts->lmax : kDefaultLmax;
        if (chunk % 64) return fail(UW_EINVAL, "chunk %u is not a multiple of 64", chunk);
        if (lmax > 15) return fail(UW_EINVAL, "lmax %u outside 1..15", lmax);
        const int64_t n = N * K;
        const int64_t groups_per_row = K / 64;
        const int64_t words = (K + 2047) / 2048;

        // 1. exponent histogram over the whole matrix
        uint64_t hist[256] = {0};
        for (int64_t i = 0; i < n; i++) hist[(w[i] >> 7) & 0xFF]++;

        // 2. palette: count descending, value ascending
        int order[256];
        for (int v = 0; v < 256; v++) order[v] = v;
        std::stable_sort(order, order + 256, [&](int a, int b) { return hist[a] > hist[b]; });
        uint8_t palette[16] = {0};
        int n_pal = 0;
        for (int t = 0; t < 256 && n_pal < 16; t++)
            if (hist[order[t]]) palette[n_pal++] = static_cast<uint8_t>(order[t]);
        int8_t pidx[256];
        std::memset(pidx, -1, sizeof pidx);
        for (int i = 0; i < n_pal; i++) pidx[palette[i]] = static_cast<int8_t>(i);

        // 3. raw 64-weight groups, symbol frequencies
        std::vector<uint32_t> bitmap(static_cast<size_t>(N * words), 0);
        std::vector<uint32_t> row_base(static_cast<size_t>(N + 1), 0);
        std::vector<uint8_t> raw;
        uint64_t freq[16] = {0};
        int64_t n_raw = 0;
        for (int64_t r = 0; r < N; r++) {
            row_base[r] = static_cast<uint32_t>(n_raw);
            for (int64_t j = 0; j < groups_per_row; j++) {
                const uint16_t* g = w + r * K + j * 64;
                bool is_raw = false;
                for (int t = 0; t < 64; t++) is_raw |= pidx[(g[t] >> 7) & 0xFF] < 0;
                if (is_raw) {
                    bitmap[r * words + j / 32] |= 1u << (j % 32);
                    for (int t = 0; t < 64; t++) raw.push_back(static_cast<uint8_t>((g[t] >> 7) & 0xFF));
                    n_raw++;
                } else {
                    for (int t = 0; t < 64; t++) freq[pidx[(g[t] >> 7) & 0xFF]]++;
                }
            }
        }
        if (n_raw >= (1ll << 32)) return fail(UW_ERANGE, "too many raw groups");
        row_base[N] = static_cast<uint32_t>(n_raw);

        // 4. code lengths and canonical codes
        uint8_t len[16] = {0};
        if (!limited_code_lengths(freq, n_pal, static_cast<int>(lmax), len))
            return fail(UW_EINVAL, "lmax %u cannot code the %d used palette indices", lmax, n_pal);
        uint32_t code[16] = {0};
        canonical_codes(len, n_pal, code);
        uint64_t total_bits = 0;
        for (int s = 0; s < n_pal; s++) total_bits += freq[s] * len[s];
        if (total_bits >= (1ull << 32)) return fail(UW_ERANGE, "stream needs %llu bits (>= 2^32)", (unsigned long long)total_bits);

        const int64_t n_chunks = (n + chunk - 1) / chunk;
        const Layout L = layout_for(N, K, n_raw, n_chunks, total_bits);
        if (!blob || *blob_bytes < L.total) {
            *blob_bytes = L.total;
            return fail(UW_ENOSPACE, "blob needs %llu bytes", (unsigned long long)L.total);
        }
        uint8_t* out = static_cast<uint8_t*>(blob);
        std::memset(out, 0, L.total);

        uw_header h;
        std::memset(&h, 0, sizeof h);
        h.magic = kMagic;
        h.version = UW_VERSION;
        h.N = N;
        h.K = K;
        h.chunk = chunk;
        h.lmax = lmax;
        h.n_pal = static_cast<uint32_t>(n_pal);
        h.n_chunks = static_cast<uint32_t>(n_chunks);
        std::memcpy(h.palette, palette, 16);
        std::memcpy(h.code_len, len, 16);
        h.n_raw = n_raw;
        h.total_bits = total_bits;
        h.off_sm = L.off_sm;
        h.off_bitmap = L.off_bitmap;
        h.off_rowbase = L.off_rowbase;
        h.off_raw = L.off_raw;
        h.off_chunk = L.off_chunk;
        h.off_stream = L.off_stream;
        h.bytes_stream = L.bytes_stream;
        h.total_bytes = L.total;
        h.bitmap_words = static_cast<uint32_t>(words);
        std::memcpy(out, &h, sizeof h);

        // sign/mantissa plane
        uint8_t* sm = out + L.off_sm;
        for (int64_t i = 0; i < n; i++) sm[i] = static_cast<uint8_t>(((w[i] >> 8) & 0x80) | (w[i] & 0x7F));
        std::memcpy(out + L.off_bitmap, bitmap.data(), bitmap.size() * 4);
        std::memcpy(out + L.off_rowbase, row_base.data(), row_base.size() * 4);
        if (n_raw) std::memcpy(out + L.off_raw, raw.data(), raw.size());

        // 5. bitstream: MSB-first codes packed into little-endian 32-bit words
        uint32_t* offs = reinterpret_cast<uint32_t*>(out + L.off_chunk);
        uint32_t* stream = reinterpret_cast<uint32_t*>(out + L.off_stream);
        uint64_t acc = 0;  // pending bits, right-aligned
        int nacc = 0;
        uint64_t pos = 0, word = 0;
        uint32_t sym_code[256];
        uint8_t sym_len[256];
        for (int v = 0; v < 256; v++) {
            sym_code[v] = pidx[v] >= 0 ? code[pidx[v]] : 0;
            sym_len[v] = pidx[v] >= 0 ? len[pidx[v]] : 0;
        }
        for (int64_t r = 0; r < N; r++) {
            for (int64_t j = 0; j < groups_per_row; j++) {
                const int64_t flat = r * K + j * 64;
                if (flat % chunk == 0) offs[flat / chunk] = static_cast<uint32_t>(pos);
                if (bitmap[r * words + j / 32] >> (j % 32) & 1u) continue;
                const uint16_t* g = w + flat;
                for (int t = 0; t < 64; t++) {
                    const int e = (g[t] >> 7) & 0xFF;
                    acc = (acc << sym_len[e]) | sym_code[e];
                    nacc += sym_len[e];
                    pos += sym_len[e];
                    if (nacc >= 32) {
                        stream[word++] = static_cast<uint32_t>(acc >> (nacc - 32));
                        nacc -= 32;
                        acc &= (1ull << nacc) - 1;
                    }
                }
            }
        }
        if (nacc > 0) stream[word++] = static_cast<uint32_t>(acc << (32 - nacc));
        offs[n_chunks] = static_cast<uint32_t>(pos);
        *blob_bytes = L.total;
        return UW_OK;
    } catch (const std::bad_alloc&) {
        return fail(UW_EINTERNAL, "out of host memory");
    } catch (...) {
        return fail(UW_EINTERNAL, "unexpected exception in uw_encode");
    }
}

uw_status uw_validate_header(const uw_header* h, size_t blob_bytes)
{
    clear_error();
    if (!h) return fail(UW_EINVAL, "NULL header");
    return check_header(h, blob_bytes);
}

uw_status uw_inspect(const void* blob, size_t blob_bytes, uw_header* out)
{
    try {
        clear_error();
        if (!blob || !out) return fail(UW_EINVAL, "NULL argument");
        if (blob_bytes < sizeof(uw_header)) return fail(UW_EFORMAT, "blob shorter than its header");
        uw_header h;
        std::memcpy(&h, blob, sizeof h);
        uw_status st = check_header(&h, blob_bytes);
        if (st != UW_OK) return st;
        const uint8_t* b = static_cast<const uint8_t*>(blob);
        const int64_t words = h.bitmap_words, gpr = h.K / 64;
        std::vector<uint32_t> bm(static_cast<size_t>(h.N * words)), rb(static_cast<size_t>(h.N + 1));
        std::memcpy(bm.data(), b + h.off_bitmap, bm.size() * 4);
        std::memcpy(rb.data(), b + h.off_rowbase, rb.size() * 4);
        if (rb[0] != 0) return fail(UW_EFORMAT, "row_base[0] != 0");
        for (int64_t r = 0; r < h.N; r++) {
            uint32_t cnt = 0;
            for (int64_t t = 0; t < words; t++) {
                uint32_t v = bm[r * words + t];
                const int64_t valid = std::min<int64_t>(32, gpr - 32 * t);
                if (valid < 32 && (v >> valid) != 0) return fail(UW_EFORMAT, "bitmap bits set beyond the row's groups");
                cnt += static_cast<uint32_t>(__builtin_popcount(v));
            }
            if (rb[r + 1] != rb[r] + cnt) return fail(UW_EFORMAT, "row_base inconsistent with the bitmap at row %lld", (long long)r);
        }
        if (static_cast<int64_t>(rb[h.N]) != h.n_raw) return fail(UW_EFORMAT, "row_base[N] != n_raw");
        std::vector<uint32_t> offs(static_cast<size_t>(h.n_chunks) + 1);
        std::memcpy(offs.data(), b + h.off_chunk, offs.size() * 4);
        if (offs[0] != 0 || offs[h.n_chunks] != h.total_bits) return fail(UW_EFORMAT, "chunk offsets do not span the stream");
        for (uint32_t c = 0; c < h.n_chunks; c++) {
            if (offs[c + 1] < offs[c]) return fail(UW_EFORMAT, "chunk offsets not monotone at chunk %u", c);
            if (static_cast<uint64_t>(offs[c + 1] - offs[c]) > static_cast<uint64_t>(h.chunk) * h.lmax)
                return fail(UW_EFORMAT, "chunk %u longer than chunk*lmax bits", c);
        }
        *out = h;
        return UW_OK;
    } catch (const std::bad_alloc&) {
        return fail(UW_EINTERNAL, "out of host memory");
    } catch (...) {
        return fail(UW_EINTERNAL, "unexpected exception in uw_inspect");
    }
}

uw_status uw_workspace_bytes(const uw_header* h, int32_t pipeline, size_t* out)
{
    clear_error();
    if (!h || !out) return fail(UW_EINVAL, "NULL argument");
    const uint64_t n = static_cast<uint64_t>(h->N) * static_cast<uint64_t>(h->K);
    switch (pipeline) {
    case UW_PIPE_FULL: *out = 2 * n; return UW_OK;
    case UW_PIPE_EXP: *out = n; return UW_OK;
    case UW_PIPE_TRANSCODE: *out = n / 2; return UW_OK;
    case UW_PIPE_DIRECT: *out = 0; return UW_OK;
    case UW_PIPE_EXPAND: *out = 2 * n; return UW_OK;
    default: return fail(UW_EINVAL, "unknown pipeline %d", pipeline);
    }
}

}  // extern "C"
