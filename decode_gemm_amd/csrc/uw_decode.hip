// Huffman decoder and palette transcoder for gfx950 (the preprocessing kernels of the
// full-decode, exponent-only and palette-transcode pipelines in the Unweight blog post,
// "Four ways to use compressed weights" and "Sharing the GPU between decode and
// compute").
//
// Work split: one lane per chunk. The stream carries the bit offset of every chunk, so
// the 64 lanes of a wave decode 64 consecutive chunks independently. A lane walks its
// chunk one 64-weight group at a time: a raw group copies its 64 verbatim exponents, any
// other group decodes 64 codes. Codes are resolved with a 2^lmax-entry table in LDS
// (entry = code length | decoded value << 8) built by each workgroup from the canonical
// code lengths in the header, so one table read resolves one code.
//
// After every group the wave's 64 groups (64 x 64 exponents or indices) sit in an LDS
// staging tile; the wave then writes them out cooperatively so that each store
// instruction covers whole 64..128-byte segments instead of 64 scattered bytes.
#include <hip/hip_runtime.h>

#include <cstring>

#include "uw_internal.h"

namespace uw {

namespace {

constexpr int kWaves = 4;        // waves per workgroup
constexpr int kPitch = 17;       // dwords per lane row of the staging tile (16 + 1 pad)
constexpr int kStageDwords = kWaves * 64 * kPitch;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DecodeArgs {
    const uint8_t* sm;
    const uint32_t* bitmap;
    const uint32_t* row_base;
    const uint8_t* raw;
    const uint32_t* offs;
    const uint32_t* stream;
    void* out;
    uint32_t* err;
    int64_t K;
    int64_t n_elems;
    uint32_t chunk, n_chunks, lmax, words;
    uint32_t max_word;  // index of the last readable stream word
    uint32_t raw_max;   // n_raw - 1 (0 when there is no raw group)
    uint32_t first_code[16], count[16], first_index[16];
    uint32_t sorted_lo, sorted_hi, sorted_lo2, sorted_hi2;  // sorted[16] as 4 dwords
    uint32_t pal[4];                                        // palette[16] as 4 dwords
};

__device__ inline uint32_t byte_of(const uint32_t* v4, uint32_t i) { return (v4[i >> 2] >> (8 * (i & 3))) & 0xFF; }

__device__ inline uint32_t ld_word(const DecodeArgs& a, uint32_t i) { return a.stream[i < a.max_word ? i : a.max_word]; }

// Two bf16 weights (elements 2t and 2t+1 of a 4-element group) from a dword of four
// exponent bytes and a dword of four sign/mantissa bytes. half = 0 takes bytes 0, 1;
// half = 1 takes bytes 2, 3.
__device__ inline uint32_t bf16_pair(uint32_t exps, uint32_t sms, int half)
{
    const uint32_t esel = half ? 0x0C030C02u : 0x0C010C00u;  // [e_a, 0, e_b, 0]
    const uint32_t ssel = half ? 0x03030202u : 0x01010000u;  // [s_a, s_a, s_b, s_b]
    const uint32_t ex = __builtin_amdgcn_perm(exps, exps, esel);
    const uint32_t sx = __builtin_amdgcn_perm(sms, sms, ssel) & 0x807F807Fu;
    return (ex << 7) | sx;
}

template <int MODE>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a)
{
    extern __shared__ uint32_t smem[];
    uint32_t* stage = smem + (threadIdx.x >> 6) * 64 * kPitch;
    uint16_t* lut = reinterpret_cast<uint16_t*>(smem + kStageDwords);
    __shared__ uint32_t tab[16 * 3 + 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < 16) {
        tab[tid] = a.first_code[tid];
        tab[16 + tid] = a.count[tid];
        tab[32 + tid] = a.first_index[tid];
    }
    if (tid < 4) {
        tab[48 + tid] = tid == 0 ? a.sorted_lo : tid == 1 ? a.sorted_hi : tid == 2 ? a.sorted_lo2 : a.sorted_hi2;
        tab[52 + tid] = a.pal[tid];
    }
    __syncthreads();
    // Decoding table: entry i answers "which code starts with the lmax bits i".
    const uint32_t lsize = 1u << a.lmax;
    for (uint32_t i = tid; i < lsize; i += 256) {
        uint32_t ent = 0;
        for (uint32_t l = 1; l <= a.lmax; l++) {
            const uint32_t code = i >> (a.lmax - l);
            const uint32_t fc = tab[l], cnt = tab[16 + l];
            if (code >= fc && code - fc < cnt) {
                const uint32_t s = byte_of(&tab[48], tab[32 + l] + (code - fc));
                // tab[52..55]: palette (full / exponent modes) or value-order positions (direct)
                const uint32_t v = MODE == DEC_IDX ? s : byte_of(&tab[52], s);
                ent = l | (v << 8);
                break;
            }
        }
        lut[i] = static_cast<uint16_t>(ent);
    }
    __syncthreads();

    const uint32_t wave_c0 = (blockIdx.x * kWaves + wave) * 64u;
    const uint32_t c = wave_c0 + lane;
    const bool active = c < a.n_chunks;
    const int64_t e0 = static_cast<int64_t>(c) * a.chunk;
    const int64_t left = active ? a.n_elems - e0 : 0;
    const uint32_t ngroups = static_cast<uint32_t>((left < a.chunk ? left : a.chunk) >> 6);

    // bit reader: valid bits MSB-aligned in buf, nb of them
    const uint32_t pos0 = active ? a.offs[c] : 0;
    uint32_t wp = pos0 >> 5;
    uint64_t buf = ((static_cast<uint64_t>(ld_word(a, wp)) << 32) | ld_word(a, wp + 1)) << (pos0 & 31);
    int nb = 64 - static_cast<int>(pos0 & 31);
    wp += 2;
    uint32_t consumed = 0, errbits = 0;
    const uint32_t lmax = a.lmax;

    const uint32_t rounds = a.chunk >> 6;
    for (uint32_t gi = 0; gi < rounds; gi++) {
        if (gi < ngroups) {
            const int64_t flat = e0 + 64 * static_cast<int64_t>(gi);
            const int64_t r = flat / a.K;
            const uint32_t j = static_cast<uint32_t>((flat - r * a.K) >> 6);
            const uint32_t bw = a.bitmap[r * a.words + (j >> 5)];
            uint32_t* row = stage + lane * kPitch;
            if ((bw >> (j & 31)) & 1u) {
                if (MODE == DEC_IDX || MODE == DEC_DIRECT) {
                    for (int t = 0; t < 8; t++) row[t] = 0;  // raw groups carry index 0
                } else {
                    uint32_t before = __popc(bw & ((1u << (j & 31)) - 1u));
                    for (uint32_t t = 0; t < (j >> 5); t++) before += __popc(a.bitmap[r * a.words + t]);
                    uint32_t ri = a.row_base[r] + before;
                    ri = ri < a.raw_max ? ri : a.raw_max;
                    const u32x4* src = reinterpret_cast<const u32x4*>(a.raw + static_cast<uint64_t>(ri) * 64);
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const u32x4 v = src[q];
                        row[4 * q + 0] = v.x;
                        row[4 * q + 1] = v.y;
                        row[4 * q + 2] = v.z;
                        row[4 * q + 3] = v.w;
                    }
                }
            } else {
                constexpr bool NIB = MODE == DEC_IDX || MODE == DEC_DIRECT;
                constexpr int PER = NIB ? 8 : 4;  // values per dword
#pragma unroll
                for (int d = 0; d < 64 / PER; d++) {
                    uint32_t packed = 0;
#pragma unroll
                    for (int t = 0; t < PER; t++) {
                        // index plane: weight t of the dword in nibble t; direct plane:
                        // weights t and t+4 share byte t % 4 (low, high nibble)
                        const int sh = MODE == DEC_IDX ? 4 * t : MODE == DEC_DIRECT ? (t < 4 ? 8 * t : 8 * (t - 4) + 4) : 8 * t;
                        const uint32_t peek = static_cast<uint32_t>(buf >> (64 - lmax));
                        const uint32_t ent = lut[peek];
                        uint32_t len = ent & 15u;
                        errbits |= len == 0 ? UW_DERR_BADCODE : 0u;
                        len = len ? len : lmax;
                        packed |= (ent >> 8) << sh;
                        buf <<= len;
                        nb -= static_cast<int>(len);
                        consumed += len;
                        if (nb < 32) {
                            buf |= static_cast<uint64_t>(ld_word(a, wp)) << (32 - nb);
                            wp++;
                            nb += 32;
                        }
                    }
                    row[d] = packed;
                }
            }
        }
        __syncthreads();
        // cooperative write-out of the wave's 64 staged groups
        if (MODE == DEC_EXP) {
            uint8_t* out = static_cast<uint8_t*>(a.out);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint32_t s = q * 16 + (lane >> 2), p = lane & 3;
                const int64_t fs = static_cast<int64_t>(wave_c0 + s) * a.chunk + 64 * static_cast<int64_t>(gi);
                if (wave_c0 + s < a.n_chunks && fs < a.n_elems) {
                    const uint32_t* src = stage + s * kPitch + 4 * p;
                    u32x4 v = {src[0], src[1], src[2], src[3]};
                    *reinterpret_cast<u32x4*>(out + fs + 16 * p) = v;
                }
            }
        } else if (MODE == DEC_FULL) {
            uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const uint32_t s = q * 8 + (lane >> 3), p = lane & 7;
                const int64_t fs = static_cast<int64_t>(wave_c0 + s) * a.chunk + 64 * static_cast<int64_t>(gi);
                if (wave_c0 + s < a.n_chunks && fs < a.n_elems) {
                    const uint32_t* src = stage + s * kPitch + 2 * p;
                    const uint32_t e_lo = src[0], e_hi = src[1];
                    const u32x2 smv = *reinterpret_cast<const u32x2*>(a.sm + fs + 8 * p);
                    u32x4 v = {bf16_pair(e_lo, smv.x, 0), bf16_pair(e_lo, smv.x, 1), bf16_pair(e_hi, smv.y, 0),
                               bf16_pair(e_hi, smv.y, 1)};
                    *reinterpret_cast<u32x4*>(out + fs + 8 * p) = v;
                }
            }
        } else if (MODE == DEC_IDX) {
            uint8_t* out = static_cast<uint8_t*>(a.out);
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const uint32_t s = q * 32 + (lane >> 1), p = lane & 1;
                const int64_t fs = static_cast<int64_t>(wave_c0 + s) * a.chunk + 64 * static_cast<int64_t>(gi);
                if (wave_c0 + s < a.n_chunks && fs < a.n_elems) {
                    const uint32_t* src = stage + s * kPitch + 4 * p;
                    u32x4 v = {src[0], src[1], src[2], src[3]};
                    *reinterpret_cast<u32x4*>(out + fs / 2 + 16 * p) = v;
                }
            }
        } else {
            // direct plane: tile-major blocks. Item (segment s, lane group g): the 16
            // sign/mantissa bytes of weights 16g..16g+15 of the segment's group, rearranged
            // as (mantissa << 1) | sign of the pair partner, and the two staged index
            // dwords of those weights, stored where MFMA lane 16g + r of the row's tile
            // reads them (raw groups keep their bytes; their staged indices are zero).
            uint8_t* out = static_cast<uint8_t*>(a.out);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint32_t item = q * 64 + lane, s = item >> 2, g = item & 3;
                const int64_t fs = static_cast<int64_t>(wave_c0 + s) * a.chunk + 64 * static_cast<int64_t>(gi);
                if (wave_c0 + s < a.n_chunks && fs < a.n_elems) {
                    const int64_t n = fs / a.K, j = (fs - n * a.K) >> 6;
                    const int64_t blk = 1536 * ((n >> 4) * (a.K >> 6) + j);
                    const uint32_t l = 16 * g + static_cast<uint32_t>(n & 15);
                    u32x4 v = *reinterpret_cast<const u32x4*>(a.sm + fs + 16 * g);
                    v = (v & 0x7F7F7F7Fu) << 1 | ((v << 1) & 0x01000100u) | ((v >> 15) & 0x00010001u);
                    *reinterpret_cast<u32x4*>(out + blk + 16 * l) = v;
                    const uint32_t* src = stage + s * kPitch + 2 * g;
                    *reinterpret_cast<u32x2*>(out + blk + 1024 + 8 * l) = u32x2{src[0], src[1]};
                }
            }
        }
        __syncthreads();
    }
    if (active) {
        const uint32_t want = a.offs[c + 1] - pos0;
        if (consumed != want) errbits |= UW_DERR_CHUNKLEN;
        if (errbits && a.err) atomicOr(a.err, errbits);
    }
}

// Direct plane, second part: one thread per 16-row tile walks the tile's groups in
// order and writes, per (tile, group), the mask of raw rows and the side-table index of
// its first raw row, copies those rows' verbatim exponents from the blob's raw table into
// the side table (ordered by tile, group, row), and zeroes the block bytes of rows past N.
struct MetaArgs {
    const uint32_t* bitmap;
    const uint32_t* row_base;
    const uint8_t* raw;
    uint8_t* blocks;
    uint32_t* meta;
    uint8_t* side;
    int64_t N, G;
    uint32_t T, words, raw_max;
};

__global__ void __launch_bounds__(256) direct_meta_kernel(MetaArgs a)
{
    const uint32_t t = blockIdx.x * 256 + threadIdx.x;
    if (t >= a.T) return;
    if (t == 0) {  // zero the padding between the meta entries and the side table
        uint8_t* pad = reinterpret_cast<uint8_t*>(a.meta + 2 * static_cast<int64_t>(a.T) * a.G);
        for (uint8_t* q = pad; q < a.side; q++) *q = 0;
    }
    const int64_t row0 = 16 * static_cast<int64_t>(t);
    uint32_t running = a.row_base[row0 < a.N ? row0 : a.N];
    uint32_t rb[16], cnt[16];
#pragma unroll
    for (int r = 0; r < 16; r++) {
        rb[r] = row0 + r < a.N ? a.row_base[row0 + r] : 0;
        cnt[r] = 0;
    }
    for (uint32_t wd = 0; wd < a.words; wd++) {
        uint32_t bw[16];
#pragma unroll
        for (int r = 0; r < 16; r++) bw[r] = row0 + r < a.N ? a.bitmap[(row0 + r) * a.words + wd] : 0;
        const int64_t jend = (32 * static_cast<int64_t>(wd) + 32) < a.G ? 32 * static_cast<int64_t>(wd) + 32 : a.G;
        for (int64_t j = 32 * static_cast<int64_t>(wd); j < jend; j++) {
            uint32_t mask = 0;
#pragma unroll
            for (int r = 0; r < 16; r++) mask |= ((bw[r] >> (j & 31)) & 1u) << r;
            uint32_t* m = a.meta + 2 * (static_cast<int64_t>(t) * a.G + j);
            m[0] = mask;
            m[1] = running;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                if ((mask >> r) & 1u) {
                    uint32_t ri = rb[r] + cnt[r];
                    ri = ri < a.raw_max ? ri : a.raw_max;
                    const u32x4* src = reinterpret_cast<const u32x4*>(a.raw + static_cast<uint64_t>(ri) * 64);
                    u32x4* dst = reinterpret_cast<u32x4*>(a.side + static_cast<uint64_t>(running) * 64);
                    dst[0] = src[0];
                    dst[1] = src[1];
                    dst[2] = src[2];
                    dst[3] = src[3];
                    running++;
                    cnt[r]++;
                }
            }
            if (row0 + 16 > a.N) {  // last tile: rows past N are zero
                uint8_t* blk = a.blocks + 1536 * (static_cast<int64_t>(t) * a.G + j);
                for (int r = static_cast<int>(a.N - row0); r < 16; r++)
                    for (int g = 0; g < 4; g++) {
                        *reinterpret_cast<u32x4*>(blk + 16 * (16 * g + r)) = u32x4{0, 0, 0, 0};
                        *reinterpret_cast<u32x2*>(blk + 1024 + 8 * (16 * g + r)) = u32x2{0, 0};
                    }
            }
        }
    }
}

}  // namespace

uint64_t direct_plane_bytes(const uw_header* h)
{
    const uint64_t T = static_cast<uint64_t>((h->N + 15) / 16), G = static_cast<uint64_t>(h->K / 64);
    return 1536 * T * G + (8 * T * G + 63) / 64 * 64 + 64 * static_cast<uint64_t>(h->n_raw);
}

uw_status launch_decode(const uw_header* h, const void* d_blob, void* d_out, int mode, uint32_t* d_err, void* stream)
{
    clear_error();
    if (!h || !d_blob || !d_out) return fail(UW_EINVAL, "NULL argument");
    uw_status st = check_header(h, h->total_bytes);
    if (st != UW_OK) return st;
    if (!aligned(d_blob, 256)) return fail(UW_EINVAL, "d_blob must be 256-byte aligned");
    if (!aligned(d_out, 16)) return fail(UW_EINVAL, "output must be 16-byte aligned");
    if (h->lmax > 14) return fail(UW_EUNSUPPORTED, "device decoder supports lmax <= 14 (got %u)", h->lmax);
    if (h->n_chunks == 0) return UW_OK;
    const uint8_t* b = static_cast<const uint8_t*>(d_blob);
    DecodeArgs a;
    std::memset(&a, 0, sizeof a);
    a.sm = b + h->off_sm;
    a.bitmap = reinterpret_cast<const uint32_t*>(b + h->off_bitmap);
    a.row_base = reinterpret_cast<const uint32_t*>(b + h->off_rowbase);
    a.raw = b + h->off_raw;
    a.offs = reinterpret_cast<const uint32_t*>(b + h->off_chunk);
    a.stream = reinterpret_cast<const uint32_t*>(b + h->off_stream);
    a.out = d_out;
    a.err = d_err;
    a.K = h->K;
    a.n_elems = h->N * h->K;
    a.chunk = h->chunk;
    a.n_chunks = h->n_chunks;
    a.lmax = h->lmax;
    a.words = h->bitmap_words;
    a.max_word = static_cast<uint32_t>(h->bytes_stream / 4 - 1);
    a.raw_max = h->n_raw > 0 ? static_cast<uint32_t>(h->n_raw - 1) : 0;
    CanonTables t;
    canon_tables(h, &t);
    for (int i = 0; i < 16; i++) {
        a.first_code[i] = t.first_code[i];
        a.count[i] = t.count[i];
        a.first_index[i] = t.first_index[i];
    }
    std::memcpy(&a.sorted_lo, t.sorted, 16);
    if (mode == DEC_DIRECT) {
        ValueOrder vo;
        value_order(h, &vo);
        std::memcpy(a.pal, vo.order, 16);
    } else {
        std::memcpy(a.pal, h->palette, 16);
    }
    const size_t lds = kStageDwords * 4 + (2u << h->lmax);
    const dim3 grid((h->n_chunks + 64 * kWaves - 1) / (64 * kWaves));
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (mode) {
    case DEC_FULL: hipLaunchKernelGGL(decode_kernel<DEC_FULL>, grid, dim3(256), lds, s, a); break;
    case DEC_EXP: hipLaunchKernelGGL(decode_kernel<DEC_EXP>, grid, dim3(256), lds, s, a); break;
    case DEC_IDX: hipLaunchKernelGGL(decode_kernel<DEC_IDX>, grid, dim3(256), lds, s, a); break;
    case DEC_DIRECT: hipLaunchKernelGGL(decode_kernel<DEC_DIRECT>, grid, dim3(256), lds, s, a); break;
    default: return fail(UW_EINVAL, "bad decode mode");
    }
    if (mode == DEC_DIRECT) {
        MetaArgs m;
        m.bitmap = a.bitmap;
        m.row_base = a.row_base;
        m.raw = a.raw;
        m.blocks = static_cast<uint8_t*>(d_out);
        const uint64_t T = static_cast<uint64_t>((h->N + 15) / 16), G = static_cast<uint64_t>(h->K / 64);
        m.meta = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(d_out) + 1536 * T * G);
        m.side = static_cast<uint8_t*>(d_out) + 1536 * T * G + (8 * T * G + 63) / 64 * 64;
        m.N = h->N;
        m.G = static_cast<int64_t>(G);
        m.T = static_cast<uint32_t>(T);
        m.words = h->bitmap_words;
        m.raw_max = a.raw_max;
        hipLaunchKernelGGL(direct_meta_kernel, dim3((m.T + 255) / 256), dim3(256), 0, s, m);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(UW_EHIP, "decode launch failed: %s", hipGetErrorString(e));
    return UW_OK;
}

}  // namespace uw

extern "C" {

uw_status uw_decode_full(const uw_header* h, const void* d_blob, uint16_t* d_w, uint32_t* d_err, void* stream)
{
    return uw::launch_decode(h, d_blob, d_w, uw::DEC_FULL, d_err, stream);
}

uw_status uw_decode_exponent(const uw_header* h, const void* d_blob, uint8_t* d_exp, uint32_t* d_err, void* stream)
{
    return uw::launch_decode(h, d_blob, d_exp, uw::DEC_EXP, d_err, stream);
}

uw_status uw_transcode_palette(const uw_header* h, const void* d_blob, uint8_t* d_idx, uint32_t* d_err, void* stream)
{
    return uw::launch_decode(h, d_blob, d_idx, uw::DEC_IDX, d_err, stream);
}

uw_status uw_prepare_direct(const uw_header* h, const void* d_blob, uint8_t* d_direct, uint32_t* d_err, void* stream)
{
    return uw::launch_decode(h, d_blob, d_direct, uw::DEC_DIRECT, d_err, stream);
}

uw_status uw_direct_plane_bytes(const uw_header* h, size_t* out)
{
    uw::clear_error();
    if (!h || !out) return uw::fail(UW_EINVAL, "NULL argument");
    *out = static_cast<size_t>(uw::direct_plane_bytes(h));
    return UW_OK;
}

}  // extern "C"
