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

#include <algorithm>
#include <cstring>
#include <type_traits>

#include "uw_internal.h"
#include "uw_recon.h"

namespace uw {

namespace {

constexpr int kWaves = 4;        // waves per workgroup
constexpr int kPitch = 17;       // dwords per lane row of the staging tile (16 + 1 pad)
constexpr int kStageDwords = kWaves * 64 * kPitch;

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
    int64_t tiles;  // direct plane: 16-row tiles (blocks are group-major)
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
            // direct plane: group-major blocks. Item (segment s, lane group g): the 16
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
                    const int64_t blk = 1536 * (j * a.tiles + (n >> 4));
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

// Direct plane, second part: one wave per 16-row tile, lane j per 64-weight group. Per
// (tile, group) it writes the mask of raw rows and the side-table index of the first raw
// row, copies those rows' verbatim exponents from the blob's raw table into the side
// table (ordered by tile, group, row), and zeroes the block bytes of rows past N.
// The side table has n_raw entries (the header's count). A blob whose bitmap / row_base
// place a raw group at or past that count is corrupt: such a row is left out of its
// block's mask (nothing is written for it) and UW_DERR_RAWINDEX is reported, so no write
// leaves the plane whatever the blob holds.
struct MetaArgs {
    const uint32_t* bitmap;
    const uint32_t* row_base;
    const uint8_t* raw;
    uint8_t* blocks;
    uint32_t* meta;
    uint8_t* side;
    uint32_t* err;
    int64_t N, G;
    uint32_t T, words, raw_max, n_raw;
};

__device__ inline uint32_t lanes_below(uint64_t ballot, uint32_t lane)
{
    return __popcll(ballot & ((1ull << lane) - 1ull));
}

__global__ void __launch_bounds__(256) direct_meta_kernel(MetaArgs a)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (t >= a.T) return;
    if (t == 0 && lane == 0) {  // zero the padding between the meta entries and the side table
        uint8_t* pad = reinterpret_cast<uint8_t*>(a.meta + 2 * static_cast<int64_t>(a.T) * a.G);
        for (uint8_t* q = pad; q < a.side; q++) *q = 0;
    }
    const int64_t row0 = 16 * static_cast<int64_t>(t);
    const int nrows = static_cast<int>(a.N - row0 < 16 ? a.N - row0 : 16);
    uint32_t running = a.row_base[row0];  // raw groups in rows before the tile
    uint32_t rb[16], carry[16];
#pragma unroll
    for (int r = 0; r < 16; r++) {
        rb[r] = r < nrows ? a.row_base[row0 + r] : 0;
        carry[r] = 0;
    }
    for (int64_t jb = 0; jb < a.G; jb += 64) {
        const int64_t j = jb + lane;
        const bool valid = j < a.G;
        uint32_t mask = 0;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            if (valid && r < nrows) mask |= ((a.bitmap[(row0 + r) * a.words + (j >> 5)] >> (j & 31)) & 1u) << r;
        }
        // exclusive prefix of the per-lane raw counts (<= 16, five bits) over the wave
        const uint32_t cnt = __popc(mask);
        uint32_t prefix = 0, total = 0;
#pragma unroll
        for (int b = 0; b < 5; b++) {
            const uint64_t bal = __ballot((cnt >> b) & 1u);
            prefix += lanes_below(bal, lane) << b;
            total += static_cast<uint32_t>(__popcll(bal)) << b;
        }
        const uint32_t first = running + prefix;
        uint32_t kept = mask;  // the mask less the rows whose slot lies past the side table
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const bool bit = (mask >> r) & 1u;
            const uint64_t bal = __ballot(bit);
            if (bit) {
                uint32_t ri = rb[r] + carry[r] + lanes_below(bal, lane);
                ri = ri < a.raw_max ? ri : a.raw_max;
                // slots grow with r, so dropping the rows past the end leaves the base +
                // popcount addressing of the rows below them unchanged
                const uint32_t dst = first + __popc(mask & ((1u << r) - 1u));
                if (dst < a.n_raw) {
                    const u32x4* src = reinterpret_cast<const u32x4*>(a.raw + static_cast<uint64_t>(ri) * 64);
                    u32x4* out = reinterpret_cast<u32x4*>(a.side + static_cast<uint64_t>(dst) * 64);
                    out[0] = src[0];
                    out[1] = src[1];
                    out[2] = src[2];
                    out[3] = src[3];
                } else {
                    kept &= ~(1u << r);
                }
            }
            carry[r] += static_cast<uint32_t>(__popcll(bal));
        }
        if (valid) {
            uint32_t* m = a.meta + 2 * (static_cast<int64_t>(t) * a.G + j);
            m[0] = kept;
            m[1] = first;
            if (kept != mask && a.err) atomicOr(a.err, UW_DERR_RAWINDEX);
        }
        running += total;
        if (valid && nrows < 16) {  // last tile: rows past N are zero
            uint8_t* blk = a.blocks + 1536 * (j * a.T + t);
            for (int r = nrows; r < 16; r++)
                for (int g = 0; g < 4; g++) {
                    *reinterpret_cast<u32x4*>(blk + 16 * (16 * g + r)) = u32x4{0, 0, 0, 0};
                    *reinterpret_cast<u32x2*>(blk + 1024 + 8 * (16 * g + r)) = u32x2{0, 0};
                }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Table-driven decoder for lmax <= 12 and chunks of at most 2048 elements.
//
// Workgroups are persistent (one per CU). Each owns two tables in LDS, indexed by the
// next lmax stream bits: a single-code table (length | value) and a multi-code table
// whose entry holds every whole code that starts those bits, up to six: their values
// (4 bits each), their count and their total length. One table read then advances a
// lane by ~4 symbols on these exponent statistics instead of one.
//
// A wave takes 64 consecutive chunks (one per lane) as a task. It copies the stream
// words those chunks span (their bit offsets bound the span) into an LDS window with
// coalesced 16-byte loads, so the bit reader refills from LDS; a span larger than the
// window is read from global memory instead (the same code instantiated twice, chosen per
// wave). Everything a task reads before decoding (bit offsets, bitmap words, the window)
// is loaded during the previous task. Each lane decodes the symbols of its chunk's
// non-raw groups, up to 256 weights per segment, into a nibble buffer in LDS: multi-code
// steps while six more symbols fit, then single codes. The wave then writes the segment's
// outputs cooperatively, taking raw groups from the blob's raw table.
//
// The workgroup size is chosen per launch so that every wave gets the same number of
// tasks (the last round would otherwise run on a fraction of the waves).
namespace lut {

#ifndef KSM_EARLY
#define KSM_EARLY 16
#endif

constexpr uint32_t kMaxWaves = 8;          // waves per workgroup at most
constexpr int kWinWords = 1792;            // stream window per wave (7 KB)
constexpr int kWinLoads = kWinWords / 256; // 16-byte loads per lane to fill it
constexpr int kInfo = 128;                 // per-wave lane info: raw mask, raw-table base
constexpr int kLutEntries = 4096;          // multi-code table, u32 entries
constexpr int kT1Dwords = 1024;            // single-code table, u8 entries
constexpr uint32_t kMaxSyms = 6;
constexpr uint32_t kMaxChunk = 2048;

// Weights per lane per segment (a segment is decoded into the wave's symbol buffer, then written
// out). The direct plane's write-out, the longest, is fastest in shorter alternations with the
// decode (96 against 117 us on the gate shape); the other outputs in longer ones.
template <int MODE>
constexpr int seg_elems() { return MODE == DEC_DIRECT ? 128 : 256; }
template <int MODE>
constexpr int wave_dwords() { return kWinWords + 64 * (seg_elems<MODE>() / 8 + 1) + kInfo; }
template <int MODE>
constexpr size_t lds_bytes(uint32_t waves) { return 4u * (kLutEntries + kT1Dwords + waves * wave_dwords<MODE>()); }

struct Args {
    const uint8_t* sm;
    const uint32_t* bitmap;
    const uint32_t* row_base;
    const uint8_t* raw;
    const uint32_t* offs;
    const uint32_t* stream;
    uint8_t* out;
    uint32_t* err;
    uint32_t K, Gr, words, chunk, n_chunks, n_tasks, n_elems;
    uint32_t tiles;       // direct plane: 16-row tiles (blocks are group-major)
    uint32_t lmax, n_words, raw_max;
    uint32_t simple;     // chunk is a power of two dividing K: a chunk's groups share one bitmap word
    uint32_t ranges[16];  // canonical rank r: first entry | length << 16 | value << 20 (length 0: unused)
    uint32_t pal[4];      // palette exponents (byte i = exponent of index i)
    uint32_t contig;      // full / exponent: indices in value order and pal[i] = pal[0] + i, so
    uint32_t base4;       //   an exponent is base4 + index per byte (base4 = pal[0] in every byte)
};

// Multi-code entry: values in bits 0..23, total length 24..27, count 28..30, bit 31 set
// when the bits start no code (then count 1, length lmax, value 0).
__device__ __forceinline__ uint32_t ent_len(uint32_t e) { return (e >> 24) & 15u; }
__device__ __forceinline__ uint32_t ent_n(uint32_t e) { return (e >> 28) & 7u; }
constexpr uint32_t kEntErr = 0x80000000u;


// Exponent bytes of four palette indices held one per byte (values 0..15).
__device__ __forceinline__ uint32_t pal4(uint32_t idx4, const uint32_t* pal)
{
    return palette_lookup(idx4 & 0x07070707u, byte_mask_bit7(idx4 << 4), pal);
}

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Sum over the wave of v (< 64).
__device__ __forceinline__ uint32_t wave_sum6(uint32_t v)
{
    uint32_t s = 0;
#pragma unroll
    for (int b = 0; b < 6; b++) s += static_cast<uint32_t>(__popcll(__ballot((v >> b) & 1u))) << b;
    return s;
}

// Sum of v (< 64) over the lanes below this one.
__device__ __forceinline__ uint32_t wave_prefix6(uint32_t v, uint32_t lane)
{
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t s = 0;
#pragma unroll
    for (int b = 0; b < 6; b++) s += static_cast<uint32_t>(__popcll(__ballot((v >> b) & 1u) & below)) << b;
    return s;
}

// Stream word i, from the wave's LDS window (words from wa on) or from global memory.
template <bool IN_LDS>
__device__ __forceinline__ uint32_t read_word(const Args& a, const uint32_t* win, uint32_t wa, uint32_t i)
{
    if (IN_LDS) return win[min(i - wa, static_cast<uint32_t>(kWinWords - 1))];
    return a.stream[min(i, a.n_words - 1)];
}

// Global inputs of one task, loaded a task ahead.
struct TaskIn {
    uint32_t pos0, pos1;  // this lane's chunk: first bit, first bit of the next chunk
    uint32_t wlo, whi;    // first bit of the wave's first chunk / of the chunk after its last
    uint32_t bw;          // bitmap word with this lane's groups (simple layout)
    uint32_t rb;          // row_base of the row holding the wave's first group
    uint32_t pre;         // lane i <= word of that group: bitmap word i of that row
};

template <int MODE>
__global__ void __launch_bounds__(64 * kMaxWaves) decode_lut_kernel(Args a)
{
    extern __shared__ uint32_t smem[];
    constexpr int kSegElems = seg_elems<MODE>();  // weights per lane per segment
    constexpr int kSG = kSegElems / 64;           // groups per segment
    constexpr int kSymPitch = kSegElems / 8 + 1;
    constexpr int kWaveDwords = wave_dwords<MODE>();
    uint32_t* lut = smem;
    uint8_t* t1 = reinterpret_cast<uint8_t*>(smem + kLutEntries);
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const uint32_t nthreads = blockDim.x, waves = nthreads >> 6;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t* win = smem + kLutEntries + kT1Dwords + wave * kWaveDwords;
    uint32_t* sym = win + kWinWords;
    uint32_t* info = sym + 64 * kSymPitch;
    uint32_t* mysym = sym + lane * kSymPitch;

    // ---- tables
    const uint32_t L = a.lmax, lsize = 1u << L;
    // t1: zero (no code), then each canonical code fills the 2^(L - len) entries that
    // start with it
    for (uint32_t d = tid; d < kT1Dwords; d += nthreads) reinterpret_cast<uint32_t*>(t1)[d] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const uint32_t g = a.ranges[r], len = (g >> 16) & 15u;
        if (len == 0) continue;
        const uint32_t lo = g & 0xFFFFu, cnt = 1u << (L - len);
        const uint8_t ent = static_cast<uint8_t>(len | (((g >> 20) & 0xFu) << 4));
        for (uint32_t i = tid; i < cnt; i += nthreads) t1[lo + i] = ent;
    }
    __syncthreads();
    // Multi-code table, one code position at a time for kPer entries per thread so their
    // t1 reads overlap: the code after the first ones is read from t1 at the bits after
    // them (valid while it fits in lmax bits). Entries are visited in a scattered order
    // (an odd multiplier permutes 0..lsize-1): entries with a common prefix read t1 at
    // strides of 2^length and would otherwise pile onto one LDS bank.
    // (10 per thread: one pass over 4096 entries with the usual 7 or 8 waves per workgroup)
    constexpr int kPer = 10;
    for (uint32_t base = 0; base < lsize; base += kPer * nthreads) {
        uint32_t idx[kPer], vals[kPer], used[kPer], n[kPer];
#pragma unroll
        for (int u = 0; u < kPer; u++) {
            idx[u] = (min(base + u * nthreads + tid, lsize - 1) * 0x9E5u) & (lsize - 1);
            const uint32_t e1 = t1[idx[u]];
            used[u] = e1 & 15u;
            vals[u] = e1 >> 4;
            n[u] = used[u] ? 1u : 0u;
        }
#pragma unroll
        for (uint32_t step = 1; step < kMaxSyms; step++) {
            uint32_t e2[kPer];
#pragma unroll
            for (int u = 0; u < kPer; u++) e2[u] = t1[(idx[u] << used[u]) & (lsize - 1)];
#pragma unroll
            for (int u = 0; u < kPer; u++) {
                const uint32_t l2 = e2[u] & 15u;
                const bool ok = n[u] == step && l2 != 0 && used[u] + l2 <= L;
                vals[u] |= ok ? (e2[u] >> 4) << (4 * step) : 0u;
                used[u] += ok ? l2 : 0u;
                n[u] += ok ? 1u : 0u;
            }
        }
#pragma unroll
        for (int u = 0; u < kPer; u++) {
            if (base + u * nthreads + tid < lsize)
                lut[idx[u]] = n[u] ? vals[u] | (used[u] << 24) | (n[u] << 28) : kEntErr | (1u << 28) | (L << 24);
        }
    }
    __syncthreads();

    // ---- tasks
    const uint32_t stride = gridDim.x * waves;
    auto load_in = [&](uint32_t task, TaskIn& t) {
        const uint32_t c0 = task * 64, c = c0 + lane;
        const uint32_t cl = min(c, a.n_chunks - 1);
        t.pos0 = a.offs[cl];
        t.pos1 = a.offs[cl + 1];
        t.wlo = a.offs[c0];
        t.whi = a.offs[min(c0 + 64, a.n_chunks)];
        const uint32_t fg0 = c0 * (a.chunk >> 6);  // the wave's first group (flat)
        const uint32_t row0 = fg0 / a.Gr, j0 = fg0 - row0 * a.Gr;
        t.rb = a.row_base[row0];
        t.pre = lane <= (j0 >> 5) ? a.bitmap[row0 * a.words + lane] : 0u;
        t.bw = 0;
        if (a.simple) {
            const uint32_t fg = cl * (a.chunk >> 6), row = fg / a.Gr, j = fg - row * a.Gr;
            t.bw = a.bitmap[row * a.words + (j >> 5)];
        }
    };
    auto window_of = [&](const TaskIn& t, uint32_t& wa, uint32_t& pieces) {
        const uint32_t w0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(t.wlo)) >> 5;
        const uint32_t w1 = min((static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(t.whi)) >> 5) + 2u, a.n_words);
        wa = w0 & ~3u;
        pieces = (w1 - wa + 3) >> 2;
    };
    // every lane loads all kWinLoads pieces (clamped to the stream) so the loads are
    // straight-line code; pieces past the window's end are not stored
    auto load_window = [&](const TaskIn& t, u32x4* pw) {
        uint32_t wa, pieces;
        window_of(t, wa, pieces);
        const uint32_t last = a.n_words / 4 - 1;
#pragma unroll
        for (int q = 0; q < kWinLoads; q++)
            pw[q] = reinterpret_cast<const u32x4*>(a.stream)[min(wa / 4 + q * 64 + lane, last)];
    };

    uint32_t task = blockIdx.x * waves + wave;
    if (task >= a.n_tasks) return;
    TaskIn cur;
    u32x4 pw[kWinLoads];
    load_in(task, cur);
    load_window(cur, pw);
    for (; task < a.n_tasks; task += stride) {
        const uint32_t c0 = task * 64, c = c0 + lane;
        const bool active = c < a.n_chunks;
        const uint32_t e0 = active ? c * a.chunk : 0;
        const uint32_t len = active ? min(a.chunk, a.n_elems - e0) : 0;
        const uint32_t ng = len >> 6;

        // stream window into LDS
        uint32_t wa, pieces;
        window_of(cur, wa, pieces);
        const bool in_lds = pieces <= static_cast<uint32_t>(kWinWords / 4);
        if (in_lds) {
#pragma unroll
            for (int q = 0; q < kWinLoads; q++) {
                const uint32_t p = q * 64 + lane;
                if (p < pieces) *reinterpret_cast<u32x4*>(win + 4 * p) = pw[q];
            }
        }

        // raw groups of this lane's chunk (bit q = group q)
        uint32_t rawmask = 0;
        if (ng) {
            const uint32_t fg = e0 >> 6;
            uint32_t row = fg / a.Gr, j = fg - row * a.Gr;
            if (a.simple) {
                rawmask = ng >= 32 ? cur.bw : (cur.bw >> (j & 31)) & ((1u << ng) - 1u);
            } else {
                for (uint32_t q = 0; q < ng; q++) {
                    rawmask |= ((a.bitmap[row * a.words + (j >> 5)] >> (j & 31)) & 1u) << q;
                    if (++j == a.Gr) {
                        j = 0;
                        row++;
                    }
                }
            }
        }
        // raw-table index of this lane's first raw group: raw groups before the wave's
        // first group (its row's base plus the set bits before it in that row) plus those
        // of the lanes below (the wave's chunks are consecutive in the raw table's order)
        uint32_t rawbase = 0;
        if (MODE == DEC_EXP || MODE == DEC_FULL) {
            const uint32_t fg0 = c0 * (a.chunk >> 6);
            const uint32_t j0 = fg0 % a.Gr, wj = j0 >> 5;
            const uint32_t before = lane < wj ? __popc(cur.pre) : lane == wj ? __popc(cur.pre & ((1u << (j0 & 31)) - 1u)) : 0u;
            rawbase = __builtin_amdgcn_readfirstlane(cur.rb) + wave_sum6(before) + wave_prefix6(__popc(rawmask), lane);
        }
        info[lane] = rawmask;
        info[64 + lane] = rawbase;
        const uint32_t pos0 = active ? cur.pos0 : 0, pos1 = cur.pos1;

        // the next task's inputs are in flight while this one decodes
        const uint32_t next = task + stride;
        TaskIn nx;
        if (next < a.n_tasks) load_in(next, nx);
        wave_sync();

        // bit reader: nb valid bits MSB-aligned in buf; wp = next word to load
        uint32_t wp = pos0 >> 5;
        uint64_t buf = 0;
        int nb = 64 - static_cast<int>(pos0 & 31);
        uint32_t err = 0;
        auto start = [&](auto lds_tag) {
            constexpr bool IN_LDS = decltype(lds_tag)::value;
            buf = ((static_cast<uint64_t>(read_word<IN_LDS>(a, win, wa, wp)) << 32) | read_word<IN_LDS>(a, win, wa, wp + 1))
                  << (pos0 & 31);
            wp += 2;
        };
        // Decode S symbols into mysym. Lanes that are done step with a null entry (no
        // bits, no symbols). A refill before every two steps keeps >= lmax bits in buf.
        auto decode = [&](auto lds_tag, uint32_t S) {
            constexpr bool IN_LDS = decltype(lds_tag)::value;
            uint32_t k = 0;
            // the symbol word being filled (nibbles below bit bp), stored after every entry
            uint32_t w = 0, bp = 0;
            uint32_t* wq = mysym;
            const int last6 = static_cast<int>(S) - static_cast<int>(kMaxSyms);  // k <= last6: room for a whole entry
            uint32_t wn = read_word<IN_LDS>(a, win, wa, wp);  // word wp, read a refill ahead
            auto refill = [&]() {
                const bool take = nb < 32;
                buf |= take ? static_cast<uint64_t>(wn) << (32 - nb) : 0ull;
                wp += take ? 1u : 0u;
                nb += take ? 32 : 0;
                wn = read_word<IN_LDS>(a, win, wa, wp);
            };
            // the next L stream bits (L <= 12: all in the buffer's high word)
            auto peek = [&]() { return static_cast<uint32_t>(buf >> 32) >> (32 - L); };
            auto put = [&](uint32_t vals, uint32_t n) {
                const uint64_t t = static_cast<uint64_t>(vals) << bp;
                w |= static_cast<uint32_t>(t);
                *wq = w;
                bp += 4 * n;
                const bool cross = bp >= 32;  // the entry ran into the next word: its rest starts it
                w = cross ? static_cast<uint32_t>(t >> 32) : w;
                wq += cross ? 1 : 0;
                bp &= 31;
                k += n;
            };
            // (loops test at the bottom: with the test at the top the compiler copies every
            // loop-carried register once per iteration)
            if (__any(static_cast<int>(k) <= last6)) {
                do {
                    refill();
#pragma unroll
                    for (int u = 0; u < 2; u++) {
                        uint32_t e = lut[peek()];
                        e = static_cast<int>(k) <= last6 ? e : 0u;
                        const uint32_t lt = ent_len(e);
                        buf <<= lt;
                        nb -= static_cast<int>(lt);
                        err |= e;
                        put(e & 0xFFFFFFu, ent_n(e));
                    }
                } while (__any(static_cast<int>(k) <= last6));
            }
            if (__any(k < S)) {
                do {
                    refill();
#pragma unroll
                    for (int u = 0; u < 2; u++) {
                        const uint32_t e1 = t1[peek()];
                        const bool go = k < S;
                        const uint32_t l1 = e1 & 15u;
                        const uint32_t lt = go ? (l1 ? l1 : L) : 0u;
                        buf <<= lt;
                        nb -= static_cast<int>(lt);
                        err |= go && l1 == 0 ? kEntErr : 0u;
                        put(go ? e1 >> 4 : 0u, go ? 1u : 0u);
                    }
                } while (__any(k < S));
            }
        };
        // the task body, instantiated for each word source so that the LDS one never
        // shares a path with pending global reads
        auto run_task = [&](auto lds_tag, auto contig_tag) {
            constexpr bool CONTIG = decltype(contig_tag)::value;
            // exponent bytes of four palette indices held one per byte
            auto exps4 = [&](uint32_t x) __attribute__((always_inline)) { return CONTIG ? x + a.base4 : pal4(x, a.pal); };
            start(lds_tag);
            const uint32_t segs = (a.chunk + kSegElems - 1) / kSegElems;
            for (uint32_t s = 0; s < segs; s++) {
                const uint32_t gq = kSG * s;
                const uint32_t nseg = ng > gq ? min(ng - gq, static_cast<uint32_t>(kSG)) : 0u;
                const uint32_t nonraw = ~(rawmask >> gq) & ((1u << nseg) - 1u);
                const uint32_t S = 64u * __popc(nonraw);
                // sign/mantissa bytes of this lane's write-out items, in flight during the decode
                // (items of 16 weights, item = 64 it + lane: chunk item / (4 kSG), group
                // (item / 4) % kSG, piece item % 4)
                constexpr int kSmItems = MODE == DEC_FULL || MODE == DEC_DIRECT ? 4 * kSG : 1;
                constexpr int kSmEarly = kSmItems > 1 ? (KSM_EARLY < kSmItems ? KSM_EARLY : kSmItems) : 1;  // before the decode
                u32x4 smv[kSmItems];
                auto load_sm = [&](int it) {
                    const uint32_t item = it * 64 + lane, l = item / (4 * kSG), g = (item >> 2) % kSG;
                    const uint32_t cl = min(c0 + l, a.n_chunks - 1);
                    const uint32_t el = cl * a.chunk, q = min(gq + g, (min(a.chunk, a.n_elems - el) >> 6) - 1);
                    smv[it] = *reinterpret_cast<const u32x4*>(a.sm + el + 64 * q + 16 * (lane & 3));
                };
                if (MODE == DEC_FULL || MODE == DEC_DIRECT) {
    #pragma unroll
                    for (int it = 0; it < kSmEarly; it++) load_sm(it);
                }
                decode(lds_tag, S);
                if (MODE == DEC_FULL || MODE == DEC_DIRECT) {
    #pragma unroll
                    for (int it = kSmEarly; it < kSmItems; it++) load_sm(it);
                }
                // the next task's stream window: right away, or (full and direct outputs) halfway
                // through the write-out, once half of the prefetched sign/mantissa registers are
                // free (holding both sets across the write-out made these modes spill)
                constexpr bool kLateWindow = MODE == DEC_FULL || MODE == DEC_DIRECT;
                constexpr int kWindowAt = 0;
                auto prefetch_window = [&]() {
                    if (s == 0 && next < a.n_tasks) load_window(nx, pw);
                };
                if (!kLateWindow) prefetch_window();
                wave_sync();

                // the lane index as an opaque value: the per-item lane constants below are then
                // computed here, not hoisted out of every loop and held (spilled) for the whole task
                uint32_t lw = lane;
                asm volatile("" : "+v"(lw));
                // ---- cooperative write-out of segment s of the wave's 64 chunks. Item
                // (chunk l, group g of the segment, piece p); consecutive lanes cover
                // consecutive output bytes of one chunk.
                auto item_ok = [&](uint32_t l, uint32_t q, uint32_t& el) {
                    const uint32_t cl = c0 + l;
                    if (cl >= a.n_chunks) return false;
                    el = cl * a.chunk;
                    return q < (min(a.chunk, a.n_elems - el) >> 6);
                };
                // symbols of group q (of this segment) start at nibble 64 * (non-raw groups before it)
                auto sym_of = [&](uint32_t l, uint32_t rm, uint32_t g) {
                    return sym + l * kSymPitch + 8u * __popc((~rm >> gq) & ((1u << g) - 1u));
                };
                if (MODE == DEC_EXP) {
    #pragma unroll 4
                    for (int it = 0; it < 4 * kSG; it++) {
                        const uint32_t item = it * 64 + lw, l = item / (4 * kSG), g = (item >> 2) % kSG, p = item & 3, q = gq + g;
                        uint32_t el;
                        if (!item_ok(l, q, el)) continue;
                        const uint32_t rm = info[l];
                        u32x4 v;
                        if ((rm >> q) & 1u) {
                            const uint32_t rb = info[64 + l];
                            const uint32_t ri = min(rb + __popc(rm & ((1u << q) - 1u)), a.raw_max);
                            v = *reinterpret_cast<const u32x4*>(a.raw + static_cast<uint64_t>(ri) * 64 + 16 * p);
                        } else {
                            const uint32_t* sp = sym_of(l, rm, g) + 2 * p;
                            const uint32_t n0 = sp[0], n1 = sp[1];
                            const uint32_t a0 = exps4(n0 & 0x0F0F0F0Fu), b0 = exps4((n0 >> 4) & 0x0F0F0F0Fu);
                            const uint32_t a1 = exps4(n1 & 0x0F0F0F0Fu), b1 = exps4((n1 >> 4) & 0x0F0F0F0Fu);
                            v = u32x4{__builtin_amdgcn_perm(b0, a0, 0x05010400u), __builtin_amdgcn_perm(b0, a0, 0x07030602u),
                                      __builtin_amdgcn_perm(b1, a1, 0x05010400u), __builtin_amdgcn_perm(b1, a1, 0x07030602u)};
                        }
                        *reinterpret_cast<u32x4*>(a.out + el + 64 * q + 16 * p) = v;
                    }
                } else if (MODE == DEC_FULL) {
    #pragma unroll
                    for (int it = 0; it < 4 * kSG; it++) {
                        if (it && (it & 3) == 0) __builtin_amdgcn_sched_barrier(0);  // bound register pressure
                        if (it == kSmItems - 1 + kWindowAt) {
                            prefetch_window();
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        const uint32_t item = it * 64 + lw, l = item / (4 * kSG), g = (item >> 2) % kSG, p = item & 3, q = gq + g;
                        uint32_t el;
                        if (!item_ok(l, q, el)) continue;
                        const uint32_t e = el + 64 * q + 16 * p;
                        const uint32_t rm = info[l];
                        uint32_t ea0, eb0, ea1, eb1;
                        if ((rm >> q) & 1u) {
                            const uint32_t rb = info[64 + l];
                            const uint32_t ri = min(rb + __popc(rm & ((1u << q) - 1u)), a.raw_max);
                            const u32x4 r = *reinterpret_cast<const u32x4*>(a.raw + static_cast<uint64_t>(ri) * 64 + 16 * p);
                            split_exps(r.x, r.y, ea0, eb0);
                            split_exps(r.z, r.w, ea1, eb1);
                        } else {
                            const uint32_t* sp = sym_of(l, rm, g) + 2 * p;
                            const uint32_t n0 = sp[0], n1 = sp[1];
                            ea0 = exps4(n0 & 0x0F0F0F0Fu);
                            eb0 = exps4((n0 >> 4) & 0x0F0F0F0Fu);
                            ea1 = exps4(n1 & 0x0F0F0F0Fu);
                            eb1 = exps4((n1 >> 4) & 0x0F0F0F0Fu);
                        }
                        u32x4* o = reinterpret_cast<u32x4*>(a.out + 2 * static_cast<uint64_t>(e));
                        o[0] = piece_from_split(ea0, eb0, smv[it].x, smv[it].y);
                        o[1] = piece_from_split(ea1, eb1, smv[it].z, smv[it].w);
                    }
                } else if (MODE == DEC_IDX) {
    #pragma unroll
                    for (int it = 0; it < 2 * kSG; it++) {
                        const uint32_t item = it * 64 + lw, l = item / (2 * kSG), g = (item >> 1) % kSG, p = item & 1, q = gq + g;
                        uint32_t el;
                        if (!item_ok(l, q, el)) continue;
                        const uint32_t rm = info[l];
                        u32x4 v = {0, 0, 0, 0};
                        if (!((rm >> q) & 1u)) {
                            const uint32_t* sp = sym_of(l, rm, g) + 4 * p;
                            v = u32x4{sp[0], sp[1], sp[2], sp[3]};
                        }
                        *reinterpret_cast<u32x4*>(a.out + (el + 64 * q) / 2 + 16 * p) = v;
                    }
                } else {
                    // direct plane: the 16 weights of lane group p of a group, at MFMA lane
                    // 16p + (row & 15) of the row tile's block
    #pragma unroll
                    for (int it = 0; it < 4 * kSG; it++) {
                        if (it && (it & 3) == 0) __builtin_amdgcn_sched_barrier(0);  // bound register pressure
                        if (it == kSmItems - 1 + kWindowAt) {
                            prefetch_window();
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        const uint32_t item = it * 64 + lw, l = item / (4 * kSG), g = (item >> 2) % kSG, p = item & 3, q = gq + g;
                        uint32_t el;
                        if (!item_ok(l, q, el)) continue;
                        const uint32_t fs = el + 64 * q;
                        const uint32_t fg = fs >> 6, n = fg / a.Gr, j = fg - n * a.Gr;
                        uint8_t* blk = a.out + 1536ull * (static_cast<uint64_t>(j) * a.tiles + (n >> 4));
                        const uint32_t ll = 16 * p + (n & 15);
                        u32x4 v = smv[it];
                        v = (v & 0x7F7F7F7Fu) << 1 | ((v << 1) & 0x01000100u) | ((v >> 15) & 0x00010001u);
                        *reinterpret_cast<u32x4*>(blk + 16 * ll) = v;
                        const uint32_t rm = info[l];
                        u32x2 d = {0, 0};
                        if (!((rm >> q) & 1u)) {
                            const uint32_t* sp = sym_of(l, rm, g) + 2 * p;
    #pragma unroll
                            for (int h = 0; h < 2; h++) {
                                const uint32_t nat = sp[h], lo = nat & 0x0F0F0F0Fu, hi = (nat >> 4) & 0x0F0F0F0Fu;
                                d[h] = __builtin_amdgcn_perm(hi, lo, 0x05010400u) | (__builtin_amdgcn_perm(hi, lo, 0x07030602u) << 4);
                            }
                        }
                        *reinterpret_cast<u32x2*>(blk + 1024 + 8 * ll) = d;
                    }
                }
                wave_sync();
            }
        };
        // (full and exponent outputs: the exponents of a palette of consecutive values are
        // one byte-wise add, so the write-out comes in a second form for it)
        if (in_lds) {
            if ((MODE == DEC_FULL || MODE == DEC_EXP) && a.contig)
                run_task(std::true_type{}, std::true_type{});
            else
                run_task(std::true_type{}, std::false_type{});
        } else {
            if ((MODE == DEC_FULL || MODE == DEC_EXP) && a.contig)
                run_task(std::false_type{}, std::true_type{});
            else
                run_task(std::false_type{}, std::false_type{});
        }
        if (active) {
            const uint32_t consumed = (wp - (pos0 >> 5)) * 32 - (pos0 & 31) - static_cast<uint32_t>(nb);
            uint32_t bits = (err & kEntErr) ? UW_DERR_BADCODE : 0u;
            if (consumed != pos1 - pos0) bits |= UW_DERR_CHUNKLEN;
            if (bits && a.err) atomicOr(a.err, bits);
        }
        if (next < a.n_tasks) cur = nx;
    }
}

}  // namespace lut

}  // namespace

// Compute units of the current device (the persistent decoder runs one workgroup per CU).
uint32_t cu_count()
{
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;  // benign race: every writer stores the same value
    }
    return static_cast<uint32_t>(cached[dev]);
}

// Compute units a stream's work may run on: its CU mask's population (all of the device
// for the null stream or when the mask cannot be read).
uint32_t stream_cu_count(void* stream)
{
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t cus = cu_count();
    if (!s) return cus;
    uint32_t mask[32] = {};
    if (hipExtStreamGetCUMask(s, 32, mask) != hipSuccess) {
        (void)hipGetLastError();
        return cus;
    }
    uint32_t n = 0;
    for (uint32_t w : mask) n += static_cast<uint32_t>(__builtin_popcount(w));
    return n == 0 || n > cus ? cus : n;
}

template <int MODE>
hipError_t launch_lut(const lut::Args& f, uint32_t blocks, uint32_t waves, hipStream_t s)
{
    static uint64_t attr_done = 0;  // devices the LDS limit was raised on (bit per device; a
                                    // lost update between racing threads only repeats the call)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!((attr_done >> dev) & 1u)) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lut::decode_lut_kernel<MODE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lut::lds_bytes<MODE>(lut::kMaxWaves)));
        if (e != hipSuccess) return e;
        attr_done |= uint64_t{1} << dev;
    }
    hipLaunchKernelGGL(lut::decode_lut_kernel<MODE>, dim3(blocks), dim3(64 * waves), lut::lds_bytes<MODE>(waves), s, f);
    return hipGetLastError();
}

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
    a.tiles = (h->N + 15) / 16;
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
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint64_t n_elems = static_cast<uint64_t>(h->N) * static_cast<uint64_t>(h->K);
    if (h->lmax <= 12 && h->chunk <= lut::kMaxChunk && n_elems + h->chunk < (1ull << 32) &&
        h->K <= 131072) {
        lut::Args f;
        std::memset(&f, 0, sizeof f);
        f.sm = a.sm;
        f.bitmap = a.bitmap;
        f.row_base = a.row_base;
        f.raw = a.raw;
        f.offs = a.offs;
        f.stream = a.stream;
        f.out = static_cast<uint8_t*>(d_out);
        f.err = d_err;
        f.K = static_cast<uint32_t>(h->K);
        f.Gr = static_cast<uint32_t>(h->K / 64);
        f.tiles = static_cast<uint32_t>((h->N + 15) / 16);
        f.words = h->bitmap_words;
        f.chunk = h->chunk;
        f.n_chunks = h->n_chunks;
        f.n_tasks = (h->n_chunks + 63) / 64;
        f.n_elems = static_cast<uint32_t>(n_elems);
        f.lmax = h->lmax;
        f.n_words = static_cast<uint32_t>(h->bytes_stream / 4);
        f.raw_max = a.raw_max;
        // symbol values: the direct plane takes value-ordered indices; full and exponent
        // decode too when the palette's exponents are consecutive (then an exponent is
        // base + index); the index plane keeps the header's order
        uint8_t vmap[16];
        for (int i = 0; i < 16; i++) vmap[i] = static_cast<uint8_t>(i);
        ValueOrder vo;
        value_order(h, &vo);
        const bool contig = (mode == DEC_FULL || mode == DEC_EXP) && vo.contiguous;
        if (mode == DEC_DIRECT || contig) std::memcpy(vmap, vo.order, 16);
        f.contig = contig ? 1u : 0u;
        f.base4 = vo.sorted[0] * 0x01010101u;
        // the canonical codes in rank order: code of rank first_index[l] + k is first_code[l] + k
        for (uint32_t l = 1, r = 0; l <= h->lmax; l++)
            for (uint32_t k = 0; k < t.count[l] && r < 16; k++, r++)
                f.ranges[r] = ((t.first_code[l] + k) << (h->lmax - l)) | (l << 16) |
                              (static_cast<uint32_t>(vmap[t.sorted[r] & 15]) << 20);
        std::memcpy(f.pal, h->palette, 16);
        f.simple = (h->chunk & (h->chunk - 1)) == 0 && h->K % h->chunk == 0;
        // equal rounds: every wave of the persistent grid gets the same number of tasks; the
        // grid is one workgroup per compute unit the stream may use (a CU-masked stream of
        // uw_stream_pair_create runs the decoder on a slice of the device)
        const uint32_t cus = stream_cu_count(s);
        const uint32_t rounds = (f.n_tasks + cus * lut::kMaxWaves - 1) / (cus * lut::kMaxWaves);
        const uint32_t waves = (f.n_tasks + cus * rounds - 1) / (cus * rounds);
        const uint32_t blocks = (f.n_tasks + waves * rounds - 1) / (waves * rounds);
        hipError_t e = hipSuccess;
        switch (mode) {
        case DEC_FULL: e = launch_lut<DEC_FULL>(f, blocks, waves, s); break;
        case DEC_EXP: e = launch_lut<DEC_EXP>(f, blocks, waves, s); break;
        case DEC_IDX: e = launch_lut<DEC_IDX>(f, blocks, waves, s); break;
        case DEC_DIRECT: e = launch_lut<DEC_DIRECT>(f, blocks, waves, s); break;
        default: return fail(UW_EINVAL, "bad decode mode");
        }
        if (e != hipSuccess) return fail(UW_EHIP, "decode launch failed: %s", hipGetErrorString(e));
    } else {
        const size_t lds = kStageDwords * 4 + (2u << h->lmax);
        const dim3 grid((h->n_chunks + 64 * kWaves - 1) / (64 * kWaves));
        switch (mode) {
        case DEC_FULL: hipLaunchKernelGGL(decode_kernel<DEC_FULL>, grid, dim3(256), lds, s, a); break;
        case DEC_EXP: hipLaunchKernelGGL(decode_kernel<DEC_EXP>, grid, dim3(256), lds, s, a); break;
        case DEC_IDX: hipLaunchKernelGGL(decode_kernel<DEC_IDX>, grid, dim3(256), lds, s, a); break;
        case DEC_DIRECT: hipLaunchKernelGGL(decode_kernel<DEC_DIRECT>, grid, dim3(256), lds, s, a); break;
        default: return fail(UW_EINVAL, "bad decode mode");
        }
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
        m.n_raw = static_cast<uint32_t>(h->n_raw);
        m.err = d_err;
        hipLaunchKernelGGL(direct_meta_kernel, dim3((m.T + 3) / 4), dim3(256), 0, s, m);
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
