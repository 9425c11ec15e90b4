// Model bundle: one file that holds every compressed projection of a model and the plans
// measured for it, for both distribution and inference.
//
// The Unweight post ("Bundles and results") ships one Huffman-coded package: it is the
// smallest form to distribute, and at load the runtime transcodes each projection to the
// form its execution pipeline reads (here: uw_prepare_direct into the direct-palette
// plane). Beside the weights it keeps the per-model profile ("Sharing the GPU between
// decode and compute": pipeline, matmul variant and K split per projection shape and
// batch size, chosen by measurement). Everything here is host code on caller buffers.
//
// Layout (little-endian; every offset a multiple of 256 bytes):
//   header  64 bytes: magic "UWB1", version, n_items, n_plans, off_items, off_plans,
//           off_data, total_bytes, checksum of the item and plan tables
//   items   n_items records of 128 bytes: name (64 bytes, NUL-padded), blob offset, blob
//           bytes, checksum of the blob
//   plans   n_plans records of 96 bytes: N, K, M, pipeline, split_k, t_ms, variant name
//           (48 bytes, NUL-padded; "" = the library's default)
//   data    the blobs (uw_encode output, verbatim), each at a 256-byte boundary
#include <cstring>
#include <set>
#include <string>
#include <vector>

#include "uw_internal.h"

namespace uw {
namespace {

constexpr uint32_t kBundleMagic = 0x31425755u;  // "UWB1"
constexpr uint32_t kBundleVersion = 1;
constexpr uint64_t kHdr = 64, kItemRec = 128, kPlanRec = 96, kAlign = 256;

uint64_t up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

void put32(uint8_t* b, uint64_t o, uint32_t v) { std::memcpy(b + o, &v, 4); }
void put64(uint8_t* b, uint64_t o, uint64_t v) { std::memcpy(b + o, &v, 8); }
uint32_t get32(const uint8_t* b, uint64_t o)
{
    uint32_t v;
    std::memcpy(&v, b + o, 4);
    return v;
}
uint64_t get64(const uint8_t* b, uint64_t o)
{
    uint64_t v;
    std::memcpy(&v, b + o, 8);
    return v;
}

// 64-bit checksum over 8-byte words (the tail zero-padded): h = (h ^ w) * an odd
// constant, rotated; fast enough to check gigabytes at load, and a changed or moved
// word changes it.
uint64_t checksum(const uint8_t* p, uint64_t n)
{
    uint64_t h = 0x9E3779B97F4A7C15ull ^ n;
    uint64_t i = 0;
    for (; i + 8 <= n; i += 8) {
        uint64_t w;
        std::memcpy(&w, p + i, 8);
        h = (h ^ w) * 0xFF51AFD7ED558CCDull;
        h = (h << 31) | (h >> 33);
    }
    if (i < n) {
        uint64_t w = 0;
        std::memcpy(&w, p + i, n - i);
        h = (h ^ w) * 0xFF51AFD7ED558CCDull;
        h = (h << 31) | (h >> 33);
    }
    return h ^ (h >> 29);
}

struct Parsed {
    uint32_t n_items, n_plans;
    uint64_t off_items, off_plans, off_data, total;
};

// Header and table bounds of a bundle held in memory.
uw_status parse(const void* bundle, size_t bytes, Parsed* o)
{
    if (!bundle) return fail(UW_EINVAL, "NULL bundle");
    if (bytes < kHdr) return fail(UW_EFORMAT, "bundle shorter than its header");
    const uint8_t* b = static_cast<const uint8_t*>(bundle);
    if (get32(b, 0) != kBundleMagic) return fail(UW_EFORMAT, "not a bundle (bad magic)");
    if (get32(b, 4) != kBundleVersion) return fail(UW_EFORMAT, "bundle version %u not supported", get32(b, 4));
    o->n_items = get32(b, 8);
    o->n_plans = get32(b, 12);
    o->off_items = get64(b, 16);
    o->off_plans = get64(b, 24);
    o->off_data = get64(b, 32);
    o->total = get64(b, 40);
    if (o->total > bytes) return fail(UW_EFORMAT, "bundle truncated: %llu of %llu bytes", (unsigned long long)bytes,
                                      (unsigned long long)o->total);
    if (o->off_items != kAlign || o->off_plans != up(o->off_items + kItemRec * o->n_items, kAlign) ||
        o->off_data != up(o->off_plans + kPlanRec * o->n_plans, kAlign) || o->off_data > o->total)
        return fail(UW_EFORMAT, "bundle tables out of place");
    if (checksum(b + o->off_items, o->off_data - o->off_items) != get64(b, 48))
        return fail(UW_EFORMAT, "bundle tables fail their checksum");
    return UW_OK;
}

bool name_ok(const char* s, size_t cap)
{
    if (!s) return false;
    const size_t n = strnlen(s, cap);
    return n > 0 && n < cap;
}

}  // namespace
}  // namespace uw

using namespace uw;

extern "C" {

int uw_variant_by_name(const char* name)
{
    if (!name) return -1;
    for (int v = 0; v < uw_variant_count(); v++)
        if (std::strcmp(uw_variant_name(v), name) == 0) return v;
    return -1;
}

uw_status uw_bundle_write(const uw_bundle_item* items, int n_items, const uw_bundle_plan* plans, int n_plans, void* out,
                          size_t* out_bytes)
{
    try {
        clear_error();
        if (!out_bytes || n_items < 0 || n_plans < 0 || (n_items > 0 && !items) || (n_plans > 0 && !plans))
            return fail(UW_EINVAL, "NULL argument or negative count");
        std::set<std::string> names;
        std::vector<uw_header> hs(static_cast<size_t>(n_items));
        uint64_t off = up(up(kAlign + kItemRec * n_items, kAlign) + kPlanRec * n_plans, kAlign);
        const uint64_t off_plans = up(kAlign + kItemRec * n_items, kAlign), off_data = off;
        for (int i = 0; i < n_items; i++) {
            if (!name_ok(items[i].name, UW_BUNDLE_NAME_MAX)) return fail(UW_EINVAL, "item %d: name empty or too long", i);
            if (!names.insert(items[i].name).second) return fail(UW_EINVAL, "item %d: name '%s' repeated", i, items[i].name);
            uw_status st = uw_inspect(items[i].blob, items[i].blob_bytes, &hs[i]);
            if (st != UW_OK) {
                const std::string why = uw_last_error();
                return fail(st, "item %d ('%s'): %s", i, items[i].name, why.c_str());
            }
            off = up(off + hs[i].total_bytes, kAlign);
        }
        for (int i = 0; i < n_plans; i++) {
            const uw_bundle_plan& p = plans[i];
            if (p.N < 1 || p.K < 64 || p.K % 64 || p.M < 1) return fail(UW_EINVAL, "plan %d: bad shape", i);
            if (p.pipeline < 0 || p.pipeline >= kPipelines) return fail(UW_EINVAL, "plan %d: bad pipeline", i);
            if (p.split_k < 0 || p.split_k > p.K / 64) return fail(UW_EINVAL, "plan %d: bad split_k", i);
            if (strnlen(p.variant, sizeof p.variant) >= sizeof p.variant) return fail(UW_EINVAL, "plan %d: variant name not terminated", i);
        }
        const uint64_t total = off;
        if (!out || *out_bytes < total) {
            *out_bytes = total;
            return fail(UW_ENOSPACE, "the bundle needs %llu bytes", (unsigned long long)total);
        }
        uint8_t* b = static_cast<uint8_t*>(out);
        std::memset(b, 0, off_data);
        uint64_t at = off_data;
        for (int i = 0; i < n_items; i++) {
            const uw_header& h = hs[i];
            uint8_t* rec = b + kAlign + kItemRec * i;
            std::memcpy(rec, items[i].name, strnlen(items[i].name, UW_BUNDLE_NAME_MAX));
            put64(rec, 64, at);
            put64(rec, 72, h.total_bytes);
            std::memcpy(b + at, items[i].blob, h.total_bytes);
            put64(rec, 80, checksum(b + at, h.total_bytes));
            const uint64_t next = up(at + h.total_bytes, kAlign);
            std::memset(b + at + h.total_bytes, 0, next - at - h.total_bytes);
            at = next;
        }
        for (int i = 0; i < n_plans; i++) {
            const uw_bundle_plan& p = plans[i];
            uint8_t* rec = b + off_plans + kPlanRec * i;
            put64(rec, 0, static_cast<uint64_t>(p.N));
            put64(rec, 8, static_cast<uint64_t>(p.K));
            put64(rec, 16, static_cast<uint64_t>(p.M));
            put32(rec, 24, static_cast<uint32_t>(p.pipeline));
            put32(rec, 28, static_cast<uint32_t>(p.split_k));
            std::memcpy(rec + 32, &p.t_ms, 4);
            std::memcpy(rec + 40, p.variant, strnlen(p.variant, sizeof p.variant));
        }
        put32(b, 0, kBundleMagic);
        put32(b, 4, kBundleVersion);
        put32(b, 8, static_cast<uint32_t>(n_items));
        put32(b, 12, static_cast<uint32_t>(n_plans));
        put64(b, 16, kAlign);
        put64(b, 24, off_plans);
        put64(b, 32, off_data);
        put64(b, 40, total);
        put64(b, 48, checksum(b + kAlign, off_data - kAlign));
        *out_bytes = total;
        return UW_OK;
    } catch (...) {
        return fail(UW_EINTERNAL, "unexpected exception in uw_bundle_write");
    }
}

uw_status uw_bundle_open(const void* bundle, size_t bytes, int verify, uw_bundle_info* info)
{
    try {
        clear_error();
        Parsed p;
        uw_status st = parse(bundle, bytes, &p);
        if (st != UW_OK) return st;
        const uint8_t* b = static_cast<const uint8_t*>(bundle);
        std::set<std::string> names;
        uint64_t expect = p.off_data;
        for (uint32_t i = 0; i < p.n_items; i++) {
            const uint8_t* rec = b + p.off_items + kItemRec * i;
            const char* name = reinterpret_cast<const char*>(rec);
            if (!name_ok(name, UW_BUNDLE_NAME_MAX)) return fail(UW_EFORMAT, "item %u: bad name", i);
            if (!names.insert(std::string(name, strnlen(name, UW_BUNDLE_NAME_MAX))).second)
                return fail(UW_EFORMAT, "item %u: name repeated", i);
            const uint64_t off = get64(rec, 64), n = get64(rec, 72);
            if (off != expect || n > p.total - off || n < sizeof(uw_header))
                return fail(UW_EFORMAT, "item %u: blob out of place", i);
            uw_header h;
            st = verify ? uw_inspect(b + off, n, &h) : uw_validate_header(reinterpret_cast<const uw_header*>(b + off), n);
            if (st != UW_OK) {
                const std::string why = uw_last_error();
                return fail(UW_EFORMAT, "item %u: %s", i, why.c_str());
            }
            if (reinterpret_cast<const uw_header*>(b + off)->total_bytes != n) return fail(UW_EFORMAT, "item %u: size", i);
            if (verify && checksum(b + off, n) != get64(rec, 80)) return fail(UW_EFORMAT, "item %u: blob fails its checksum", i);
            expect = up(off + n, kAlign);
        }
        if (expect != p.total) return fail(UW_EFORMAT, "bundle size does not match its items");
        for (uint32_t i = 0; i < p.n_plans; i++) {
            const uint8_t* rec = b + p.off_plans + kPlanRec * i;
            const int64_t K = static_cast<int64_t>(get64(rec, 8));
            const int32_t pipe = static_cast<int32_t>(get32(rec, 24)), ks = static_cast<int32_t>(get32(rec, 28));
            if (static_cast<int64_t>(get64(rec, 0)) < 1 || K < 64 || K % 64 || static_cast<int64_t>(get64(rec, 16)) < 1 ||
                pipe < 0 || pipe >= kPipelines || ks < 0 || ks > K / 64 || strnlen(reinterpret_cast<const char*>(rec + 40), 48) >= 48)
                return fail(UW_EFORMAT, "plan %u: bad record", i);
        }
        if (info) {
            info->n_items = p.n_items;
            info->n_plans = p.n_plans;
            info->total_bytes = p.total;
        }
        return UW_OK;
    } catch (...) {
        return fail(UW_EINTERNAL, "unexpected exception in uw_bundle_open");
    }
}

uw_status uw_bundle_item_at(const void* bundle, size_t bytes, uint32_t i, uw_bundle_entry* out)
{
    clear_error();
    if (!out) return fail(UW_EINVAL, "NULL argument");
    Parsed p;
    uw_status st = parse(bundle, bytes, &p);
    if (st != UW_OK) return st;
    if (i >= p.n_items) return fail(UW_EINVAL, "item %u of %u", i, p.n_items);
    const uint8_t* b = static_cast<const uint8_t*>(bundle);
    const uint8_t* rec = b + p.off_items + kItemRec * i;
    std::memset(out, 0, sizeof *out);
    std::memcpy(out->name, rec, UW_BUNDLE_NAME_MAX - 1);
    out->offset = get64(rec, 64);
    out->blob_bytes = get64(rec, 72);
    if (out->offset < p.off_data || out->blob_bytes > p.total - out->offset || out->blob_bytes < sizeof(uw_header))
        return fail(UW_EFORMAT, "item %u: blob out of place", i);
    std::memcpy(&out->header, b + out->offset, sizeof(uw_header));
    return uw_validate_header(&out->header, out->blob_bytes);
}

uw_status uw_bundle_plan_at(const void* bundle, size_t bytes, uint32_t i, uw_bundle_plan* out)
{
    clear_error();
    if (!out) return fail(UW_EINVAL, "NULL argument");
    Parsed p;
    uw_status st = parse(bundle, bytes, &p);
    if (st != UW_OK) return st;
    if (i >= p.n_plans) return fail(UW_EINVAL, "plan %u of %u", i, p.n_plans);
    const uint8_t* rec = static_cast<const uint8_t*>(bundle) + p.off_plans + kPlanRec * i;
    std::memset(out, 0, sizeof *out);
    out->N = static_cast<int64_t>(get64(rec, 0));
    out->K = static_cast<int64_t>(get64(rec, 8));
    out->M = static_cast<int64_t>(get64(rec, 16));
    out->pipeline = static_cast<int32_t>(get32(rec, 24));
    out->split_k = static_cast<int32_t>(get32(rec, 28));
    std::memcpy(&out->t_ms, rec + 32, 4);
    std::memcpy(out->variant, rec + 40, sizeof out->variant - 1);
    return UW_OK;
}

}  // extern "C"
